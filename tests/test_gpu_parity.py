"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several work items (64 tokens and up) and a ragged tail."""
import math

import numpy as np
import pytest
import torch

from attention_reuse_amd import mac
from attention_reuse_amd import workload as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mac_harness import (DEV, Layer, lockstep_compare, params_for, run_steps,
                             to_dev, tolerance_check)


def _cfg(**kw):
    base = dict(name="t", batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
                dtype="bf16", ctx=3000, steps=40, ring_k=256, band_r=64, tau=0.6,
                rope_base=5e5, n_protos=16, switch_p=0.1, sigma=(0.05, 0.05), seed=0)
    base.update(kw)
    return wl.Workload(**base)


def _inputs(cfg):
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    return K, V, qt, q


@pytest.mark.parametrize("shape", [
    dict(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, dtype="f32", ctx=2048, steps=64),
    dict(batch=3, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", ctx=1000, steps=8),
    dict(batch=2, n_q_heads=4, n_kv_heads=4, head_dim=64, dtype="bf16", ctx=700, steps=4),
    dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128, dtype="f32", ctx=500, steps=4),
    dict(batch=2, n_q_heads=8, n_kv_heads=4, head_dim=128, dtype="bf16", ctx=300, steps=4),
])
def test_full_decode_matches_oracle(oracle_lib, shape):
    cfg = _cfg(**shape)
    print("full decode", shape, flush=True)
    K, V, qt, q = _inputs(cfg)
    p = params_for(cfg)
    ws_b = mac.mac_workspace_bytes(p)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=DEV)
    Kd, Vd = to_dev(K), to_dev(V)
    # Ragged positions per request, including m = 0, a chunk boundary and a
    # chunk tail.
    choices = [[0, 127, 128, 129, cfg.capacity - 1], [cfg.capacity - 1, 5, 255, 256, 1000 % cfg.capacity]]
    for pos_list in choices:
        m = np.array([pos_list[b % len(pos_list)] for b in range(cfg.batch)], np.int32)
        qq = q[:, :, cfg.n_warm]
        out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), device=DEV)
        lse = torch.empty((cfg.batch, cfg.n_q_heads), device=DEV)
        mac.mac_full_decode(p, to_dev(qq), Kd, Vd, to_dev(m), out, lse, ws, ws_b,
                            torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_lib.full_decode(qq, K, V, m)
        ok, err = tolerance_check(cfg, out.cpu().numpy(), ref_o)
        assert ok, err
        np.testing.assert_allclose(lse.cpu().numpy(), ref_l, atol=1e-4)
        assert mac.mac_read_device_status(p, ws) == 0


def test_full_decode_any_workspace_contents():
    """mac_full_decode needs no initialised workspace: filled with 0xff bytes
    (every counter and control word maximal) or with zeros, the output is the
    same bit for bit, also on a second call reusing the workspace."""
    cfg = _cfg(batch=4, ctx=3000, steps=4)
    K, V, qt, q = _inputs(cfg)
    p = params_for(cfg)
    ws_b = mac.mac_workspace_bytes(p)
    Kd, Vd = to_dev(K), to_dev(V)
    m = to_dev(np.array([2999, 1500, 64, 777], np.int32))
    qd = to_dev(q[:, :, cfg.n_warm])
    outs = []
    for fill in (0, 255):
        ws = torch.full((ws_b,), fill, dtype=torch.uint8, device=DEV)
        for _ in range(2):
            out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), device=DEV)
            mac.mac_full_decode(p, qd, Kd, Vd, m, out, None, ws, ws_b,
                                torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def _lockstep(oracle_lib, cfg, layer=None, heads=None, n_warm=None, want_ring=True,
              thresh_mode=0, min_context=0, flags=0):
    K, V, qt, q = _inputs(cfg)
    layer = layer or Layer(cfg, K, V, qt, q, n_warm=n_warm,
                           params=params_for(cfg, thresh_mode=thresh_mode,
                                             min_context=min_context, flags=flags))
    layer.init()
    aux = torch.cuda.Stream()
    gpu = run_steps(layer, cfg.steps, aux=aux)
    heads = heads or [(b, h) for b in range(cfg.batch) for h in range(cfg.n_q_heads)]
    W = layer.n_warm
    nw = cfg.n_warm
    t2 = oracle_lib.threshold2(cfg.head_dim, cfg.tau, mode=thresh_mode)
    res = {}
    for (b, h) in heads:
        g = h // cfg.group
        res[(b, h)] = oracle_lib.run_stream(
            K[b, g], V[b, g], qt[b, h, nw - W:nw], q[b, h, nw - W:nw], qt[b, h, nw:],
            q[b, h, nw:], ctx_len=cfg.ctx, ring_k=cfg.ring_k, band_r=cfg.band_r,
            thresh2=t2, want_ring=want_ring, min_context=min_context)
    stats = dict(hits=0, steps=0, exempt=0, diverged=0)
    qr = layer.q_ring.cpu().float().numpy() if want_ring else None
    orr = layer.o_ring.cpu().numpy() if want_ring else None
    lr = layer.lse_ring.cpu().numpy() if want_ring else None
    pr = layer.pos_ring.cpu().numpy() if want_ring else None
    for (b, h), o in res.items():
        n, ex, div = lockstep_compare(cfg, gpu, o, b, h, cfg.steps)
        stats["steps"] += n
        stats["exempt"] += ex
        stats["hits"] += int(o["hit"][:n].sum())
        if div is not None:
            stats["diverged"] += 1
            continue
        if want_ring:
            assert np.array_equal(pr[b, h // cfg.group], o["ring_pos"]), (b, h)
            np.testing.assert_array_equal(qr[b, h], o["ring_q"])
            fin = np.isfinite(o["ring_lse"])
            assert np.array_equal(np.isfinite(lr[b, h]), fin)
            np.testing.assert_allclose(lr[b, h][fin], o["ring_lse"][fin], atol=1e-3)
            ok, err = tolerance_check(cfg, orr[b, h], o["ring_o"])
            assert ok, err
    print(cfg.name, stats, flush=True)
    return gpu, res, stats, layer


def test_lockstep_tiny_f32_config(oracle_lib):
    """The tiny CPU-checkable configuration at full size: 1 request, 4 query
    heads on 1 KV head, d=64 fp32, 2048 context, 64 steps, K=64, r=32."""
    cfg = wl.WORKLOADS[1]
    _, _, st, _ = _lockstep(oracle_lib, cfg)
    assert st["diverged"] == 0 and st["hits"] > 0.8 * st["steps"]


def test_lockstep_gqa_bf16(oracle_lib):
    cfg = _cfg()
    _, _, st, _ = _lockstep(oracle_lib, cfg)
    assert st["hits"] > 0.9 * st["steps"]


def test_lockstep_mixed_hit_miss(oracle_lib):
    """Per-head noise U[0.02, 0.5]: hits and misses mix inside GQA groups."""
    cfg = _cfg(batch=2, ctx=2000, steps=40, ring_k=128, band_r=64, sigma=(0.02, 0.5), seed=3)
    gpu, res, st, _ = _lockstep(oracle_lib, cfg)
    rate = st["hits"] / st["steps"]
    assert 0.3 < rate < 0.97, rate


def test_lockstep_cold_ring_and_edges(oracle_lib):
    # Cold ring: the first step has no candidate.
    cfg = _cfg(batch=1, n_q_heads=8, n_kv_heads=2, ctx=600, steps=30, ring_k=16, band_r=8)
    gpu, res, st, _ = _lockstep(oracle_lib, cfg, n_warm=0)
    assert (gpu["p"][0] == -1).all()
    # r = 0 (nothing recomputed before the match), K = 1 (only m-1 is a candidate),
    # r larger than the context (hits are full attention).
    for kw in (dict(band_r=0), dict(ring_k=1, band_r=3), dict(band_r=5000, ctx=200)):
        _lockstep(oracle_lib, cfg.replace(**kw))


def test_forced_miss_is_bitwise_full_decode():
    """tau = 1 makes the threshold 0: every step misses and must equal the
    full decode bit for bit (same partition, same fold order)."""
    cfg = _cfg(steps=6)
    K, V, qt, q = _inputs(cfg)
    p = params_for(cfg, tau=1.0)
    layer = Layer(cfg, K, V, qt, q, params=p).init()
    gpu = run_steps(layer, cfg.steps, aux=torch.cuda.Stream())
    assert (gpu["p"] == -1).all()
    ws_b = mac.mac_workspace_bytes(p)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=DEV)
    pos = wl.decode_positions(cfg)
    for s in range(cfg.steps):
        out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), device=DEV)
        mac.mac_full_decode(p, layer.dec_q[s], layer.K, layer.V, to_dev(pos[s]), out, None,
                            ws, ws_b, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), gpu["out"][s]), s


def test_run_to_run_deterministic_and_launch_and_append_mode_invariant():
    """Outputs and rings are bitwise identical run to run, as one launch, two
    kernels or three, with the rectify-append on an auxiliary stream, on the
    main stream, or fused into the merge."""
    cfg = _cfg(steps=12, sigma=(0.02, 0.5))
    K, V, qt, q = _inputs(cfg)
    runs = []
    split, fused = mac.MAC_FLAG_SPLIT_STAGES, mac.MAC_FLAG_FUSED_APPEND
    single, two = mac.MAC_FLAG_SINGLE_LAUNCH, mac.MAC_FLAG_TWO_STAGES
    for flags, aux in ((single, torch.cuda.Stream()), (single, None),
                       (single | fused, torch.cuda.Stream()), (0, torch.cuda.Stream()),
                       (split, torch.cuda.Stream()), (split | fused, None), (split, None),
                       (two, torch.cuda.Stream()), (two | fused, None)):
        print("  flags %d, aux stream %s" % (flags, aux is not None), flush=True)
        layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=flags))
        res = run_steps(layer.init(), cfg.steps, aux=aux)
        res["rings"] = [t.cpu().float().numpy() for t in
                        (layer.q_ring, layer.o_ring, layer.lse_ring, layer.pos_ring)]
        runs.append(res)
        layer.release()
    for r in runs[1:]:
        for k in ("out", "lse", "p", "d2"):
            assert np.array_equal(runs[0][k], r[k]), k
        for x, y in zip(runs[0]["rings"], r["rings"]):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("batch", [8, 16])
def test_forms_bitwise_equal_many_groups(batch):
    """Above 16 KV groups (64 and 128: the coarser 128-token grid, the
    two-kernel default and, with missed heads' long ranges, the cross-group
    pool) the one-launch, two-kernel and three-kernel forms give the same
    outputs, matches and rings bit for bit."""
    cfg = _cfg(batch=batch, ctx=6000, steps=10, ring_k=256, band_r=64, sigma=(0.02, 0.5),
               seed=11)
    K, V, qt, q = _inputs(cfg)
    single, two = mac.MAC_FLAG_SINGLE_LAUNCH, mac.MAC_FLAG_TWO_STAGES
    split, fused = mac.MAC_FLAG_SPLIT_STAGES, mac.MAC_FLAG_FUSED_APPEND
    runs = []
    for flags in (split | fused, two | fused, single | fused, 0):
        print("  batch %d, flags %d" % (batch, flags), flush=True)
        layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=flags))
        res = run_steps(layer.init(), cfg.steps)
        res["rings"] = [t.cpu().float().numpy() for t in
                        (layer.q_ring, layer.o_ring, layer.lse_ring, layer.pos_ring)]
        runs.append(res)
        layer.release()
    assert (runs[0]["p"] < 0).any() and (runs[0]["p"] >= 0).any()
    for r in runs[1:]:
        for k in ("out", "lse", "p", "d2"):
            assert np.array_equal(runs[0][k], r[k]), k
        for x, y in zip(runs[0]["rings"], r["rings"]):
            assert np.array_equal(x, y)


def test_lockstep_split_stages(oracle_lib):
    """The three-kernel form of the step against the oracle (the other
    lockstep tests have at most 16 KV groups, so they run one launch)."""
    cfg = _cfg(batch=2, ctx=1800, steps=24, ring_k=128, band_r=48, sigma=(0.02, 0.5), seed=7)
    K, V, qt, q = _inputs(cfg)
    layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=mac.MAC_FLAG_SPLIT_STAGES))
    _lockstep(oracle_lib, cfg, layer=layer)


def test_lockstep_two_stages(oracle_lib):
    """The two-kernel form (match kernel, then one launch for plan,
    attention and merge) against the oracle, over enough steps that both
    sets of per-head keys are used many times."""
    cfg = _cfg(batch=2, ctx=1800, steps=24, ring_k=128, band_r=48, sigma=(0.02, 0.5), seed=9)
    K, V, qt, q = _inputs(cfg)
    layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=mac.MAC_FLAG_TWO_STAGES))
    _lockstep(oracle_lib, cfg, layer=layer)


def test_interleaved_handles_one_stream():
    """Several layers' single-launch steps interleaved on one stream (as in
    a model): each layer's results equal those of that layer run alone."""
    cfg = _cfg(batch=1, steps=8, sigma=(0.02, 0.5))
    K, V, qt, q = _inputs(cfg)
    alone = run_steps(Layer(cfg, K, V, qt, q).init(), cfg.steps)
    layers = [Layer(cfg, K, V, qt, q).init() for _ in range(3)]
    B, H, d = cfg.batch, cfg.n_q_heads, cfg.head_dim
    outs = [torch.empty((cfg.steps, B, H, d), device=DEV) for _ in layers]
    pos = torch.from_numpy(wl.decode_positions(cfg)).to(DEV)
    ms = torch.cuda.current_stream().cuda_stream
    for s in range(cfg.steps):
        for L, o in zip(layers, outs):
            mac.mac_decode_step(L.handle, L.dec_qt[s], L.dec_q[s], L.K, L.V, pos[s], o[s],
                                None, None, None, ms, None)
    torch.cuda.synchronize()
    for L, o in zip(layers, outs):
        assert np.array_equal(o.cpu().numpy(), alone["out"])
        assert mac.mac_read_device_status(L.p, L.ws) == 0
        L.release()


def test_lockstep_fused_append(oracle_lib):
    cfg = _cfg(batch=2, ctx=1500, steps=24, ring_k=128, band_r=32, sigma=(0.02, 0.5), seed=5)
    K, V, qt, q = _inputs(cfg)
    layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=mac.MAC_FLAG_FUSED_APPEND))
    _lockstep(oracle_lib, cfg, layer=layer)


def test_exact_reuse_on_gpu():
    """Identity RoPE, no noise, one prototype: every step hits p = m - 1 (the
    tie goes to the most recent position) and equals full attention."""
    cfg = _cfg(batch=1, n_protos=1, sigma=(0.0, 0.0), switch_p=0.0, steps=20)
    K, V, qt, _ = _inputs(cfg)
    q = wl.from_storage(qt).astype(np.float32)
    layer = Layer(cfg, K, V, qt, q).init()
    gpu = run_steps(layer, cfg.steps)
    m = wl.decode_positions(cfg)[:, 0]
    assert (gpu["p"] == (m - 1)[:, None, None]).all()
    p = params_for(cfg)
    ws_b = mac.mac_workspace_bytes(p)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=DEV)
    for s in (0, 10, 19):
        out = torch.empty((1, cfg.n_q_heads, cfg.head_dim), device=DEV)
        mac.mac_full_decode(p, layer.dec_q[s], layer.K, layer.V, to_dev(np.array([m[s]], np.int32)),
                            out, None, ws, ws_b, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert np.abs(out.cpu().numpy() - gpu["out"][s]).max() < 1e-4


def test_nan_ring_slot_never_selected():
    cfg = _cfg(batch=1, n_protos=1, sigma=(0.0, 0.0), switch_p=0.0, steps=1)
    K, V, qt, _ = _inputs(cfg)
    q = wl.from_storage(qt).astype(np.float32)
    layer = Layer(cfg, K, V, qt, q).init()
    torch.cuda.synchronize()
    slot = (cfg.ctx - 1) % cfg.ring_k
    layer.q_ring[0, :, slot, 5] = float("nan")        # poison position m-1
    gpu = run_steps(layer, 1)
    assert (gpu["p"][0] == cfg.ctx - 2).all()
    layer.init()
    torch.cuda.synchronize()
    layer.q_ring[0, 3, :, 0] = float("nan")           # every candidate of head 3
    gpu = run_steps(layer, 1)
    assert gpu["p"][0, 0, 3] == -1 and np.isinf(gpu["d2"][0, 0, 3])
    assert (gpu["p"][0, 0, :3] >= 0).all()


def test_bad_position_is_flagged_not_faulted():
    cfg = _cfg(batch=2, steps=1)
    K, V, qt, q = _inputs(cfg)
    layer = Layer(cfg, K, V, qt, q).init()
    torch.cuda.synchronize()
    before = layer.pos_ring.cpu().numpy().copy()
    pos = torch.tensor([[cfg.ctx, cfg.capacity]], dtype=torch.int32, device=DEV)
    gpu = run_steps(layer, 1, pos=pos)
    assert mac.mac_read_device_status(layer.p, layer.ws) == mac.MAC_DEV_BAD_POSITION
    assert np.isnan(gpu["out"][0, 1]).all() and np.isfinite(gpu["out"][0, 0]).all()
    after = layer.pos_ring.cpu().numpy()
    assert np.array_equal(after[1], before[1])          # no append for request 1
    assert mac.mac_read_device_status(layer.p, layer.ws) == 0


@pytest.mark.parametrize("flags", [0, mac.MAC_FLAG_SPLIT_STAGES, mac.MAC_FLAG_TWO_STAGES])
def test_lockstep_tau_threshold_rule(oracle_lib, flags):
    """The acceptance rule distance < tau * sqrt(2d) (MAC_THRESH_TAU; the
    paper summary's "Core method" form) against the oracle's threshold in
    the same mode, with per-head noise chosen so that both hits and misses
    occur under it, one launch and three kernels."""
    cfg = _cfg(batch=2, ctx=1500, steps=24, ring_k=128, band_r=48, sigma=(0.3, 0.9), seed=11)
    _, _, st, _ = _lockstep(oracle_lib, cfg, thresh_mode=mac.MAC_THRESH_TAU, flags=flags)
    rate = st["hits"] / st["steps"]
    assert st["diverged"] == 0 and 0.2 < rate < 0.95, rate


@pytest.mark.parametrize("flags", [0, mac.MAC_FLAG_SPLIT_STAGES | mac.MAC_FLAG_FUSED_APPEND])
def test_lockstep_min_context(oracle_lib, flags):
    """Reuse off below the minimum context, decided on the device per
    request: positions cross the limit during the run (requests at
    different positions too), and the blocked steps still fill the rings."""
    cfg = _cfg(batch=2, ctx=1200, steps=24, ring_k=64, band_r=16, sigma=(0.02, 0.2), seed=2)
    lim = cfg.ctx + 10
    gpu, res, st, _ = _lockstep(oracle_lib, cfg, min_context=lim, flags=flags)
    s0 = lim - cfg.ctx
    assert (gpu["p"][:s0] == -1).all() and np.isinf(gpu["d2"][:s0]).all()
    assert (gpu["p"][s0:] >= 0).mean() > 0.5
    assert st["diverged"] == 0


def test_aux_append_ignores_pos_overwritten_after_the_call():
    """The rectify-append on the auxiliary stream appends at the position
    the step's merge recorded, not at whatever the caller's position array
    holds when the append runs: here main_stream overwrites the array right
    after every call while the auxiliary stream is held back by other work,
    and the rings and outputs still equal the fused append's."""
    cfg = _cfg(batch=2, steps=10, sigma=(0.02, 0.5))
    K, V, qt, q = _inputs(cfg)
    ref_layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=mac.MAC_FLAG_FUSED_APPEND))
    ref = run_steps(ref_layer.init(), cfg.steps)
    ref_rings = [t.cpu().float().numpy() for t in
                 (ref_layer.q_ring, ref_layer.o_ring, ref_layer.lse_ring, ref_layer.pos_ring)]
    ref_layer.release()
    for flags in (0, mac.MAC_FLAG_SPLIT_STAGES, mac.MAC_FLAG_TWO_STAGES):
        layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=flags)).init()
        aux = torch.cuda.Stream()
        ms = torch.cuda.current_stream()
        pos_all = torch.from_numpy(wl.decode_positions(cfg)).to(DEV)
        pos = torch.empty(cfg.batch, dtype=torch.int32, device=DEV)
        out = torch.empty((cfg.steps, cfg.batch, cfg.n_q_heads, cfg.head_dim), device=DEV)
        busy = torch.empty(1 << 24, device=DEV)
        for s in range(cfg.steps):
            with torch.cuda.stream(aux):
                for _ in range(4):  # keeps the auxiliary stream busy
                    busy.mul_(1.0001)
            pos.copy_(pos_all[s])
            mac.mac_decode_step(layer.handle, layer.dec_qt[s], layer.dec_q[s], layer.K,
                                layer.V, pos, out[s], None, None, None, ms.cuda_stream,
                                aux.cuda_stream)
            pos.add_(1)  # a valid but different position, before the append runs
        mac.mac_join_aux(layer.handle, ms.cuda_stream)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref["out"]), flags
        rings = [t.cpu().float().numpy() for t in
                 (layer.q_ring, layer.o_ring, layer.lse_ring, layer.pos_ring)]
        for x, y in zip(rings, ref_rings):
            assert np.array_equal(x, y), flags
        layer.release()


def test_full_decode_long_range_matches_oracle(oracle_lib):
    """One request at a 128K-token range (131001 tokens): the split-KV grid
    is 1024 tokens (128 cells), checked against the oracle head by head."""
    cfg = _cfg(batch=1, ctx=131000, steps=2, ring_k=64, band_r=16)
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    assert mac.mac_chunk_tokens(0, cfg.ctx) == 1024 and mac.mac_chunk_tokens(0, 131072) == 2048
    p = params_for(cfg)
    ws_b = mac.mac_workspace_bytes(p)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=DEV)
    m = np.array([cfg.ctx], np.int32)
    qq = q[:, :, cfg.n_warm]
    out = torch.empty((1, cfg.n_q_heads, cfg.head_dim), device=DEV)
    lse = torch.empty((1, cfg.n_q_heads), device=DEV)
    mac.mac_full_decode(p, to_dev(qq), to_dev(K), to_dev(V), to_dev(m), out, lse, ws, ws_b,
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_lib.full_decode(qq, K, V, m)
    ok, err = tolerance_check(cfg, out.cpu().numpy(), ref_o)
    assert ok, err
    np.testing.assert_allclose(lse.cpu().numpy(), ref_l, atol=1e-4)
