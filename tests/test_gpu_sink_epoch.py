"""GPU parity of attention-sink isolation and ready/epoch gating (MAC-Attention
blog, "Production version: one fused persistent BF16 kernel"): the HIP path
through the C ABI against the CPU oracle in lock step, the kernel forms
against each other bit for bit, and the gating inside a captured graph."""
import numpy as np
import pytest
import torch

from attention_reuse_amd import mac
from attention_reuse_amd import workload as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mac_harness import (DEV, Layer, lockstep_compare, params_for, to_dev,
                             tolerance_check)

SPLIT, FUSED, SINGLE, TWO = 2, 1, 4, 16


def _cfg(**kw):
    base = dict(name="t", batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
                dtype="bf16", ctx=1800, steps=24, ring_k=128, band_r=48, tau=0.6,
                rope_base=5e5, n_protos=16, switch_p=0.1, sigma=(0.02, 0.5), seed=7)
    base.update(kw)
    return wl.Workload(**base)


def _restarts(epochs):
    """Oracle restart flags [B, S] for per-step request epochs [S, B]: a
    ring is ready when the epoch is non-negative and equals the one its
    rings were built for (0 after the reset); a step that is not ready
    restarts the ring and adopts the epoch."""
    S, B = epochs.shape
    ring = np.zeros(B, np.int64)
    out = np.zeros((B, S), np.int32)
    for s in range(S):
        for b in range(B):
            e = int(epochs[s, b])
            if not (e >= 0 and e == ring[b]):
                out[b, s] = 1
                ring[b] = e
    return out


def _run(layer, n_steps, epochs=None, aux=None):
    """Decode steps; the bound epoch array is rewritten on the main stream
    before each step, as a caller would do on the device."""
    cfg = layer.cfg
    B, H, d = cfg.batch, cfg.n_q_heads, cfg.head_dim
    out = torch.empty((n_steps, B, H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((n_steps, B, H), dtype=torch.float32, device=DEV)
    mp = torch.empty((n_steps, B, H), dtype=torch.int32, device=DEV)
    md = torch.empty((n_steps, B, H), dtype=torch.float32, device=DEV)
    pos = torch.from_numpy(wl.decode_positions(cfg)[:n_steps]).to(DEV)
    ms = torch.cuda.current_stream().cuda_stream
    aux_s = aux.cuda_stream if aux is not None else None
    ep = None
    if epochs is not None:
        ep = torch.zeros(B, dtype=torch.int32, device=DEV)
        eps = torch.from_numpy(np.ascontiguousarray(epochs, np.int32)).to(DEV)
        mac.mac_bind_epochs(layer.handle, ep)
    for s in range(n_steps):
        if ep is not None:
            ep.copy_(eps[s])
        mac.mac_decode_step(layer.handle, layer.dec_qt[s], layer.dec_q[s], layer.K, layer.V,
                            pos[s], out[s], lse[s], mp[s], md[s], ms, aux_s)
    if aux is not None:
        mac.mac_join_aux(layer.handle, ms)
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), p=mp.cpu().numpy(),
                d2=md.cpu().numpy())


def _lockstep(oracle_lib, cfg, F, flags=0, epochs=None, n_warm=None, aux=True):
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    layer = Layer(cfg, K, V, qt, q, n_warm=n_warm,
                  params=params_for(cfg, flags=flags, front_sink=F)).init()
    gpu = _run(layer, cfg.steps, epochs, aux=torch.cuda.Stream() if aux else None)
    rst = _restarts(epochs) if epochs is not None else None
    W, nw = layer.n_warm, cfg.n_warm
    t2 = oracle_lib.threshold2(cfg.head_dim, cfg.tau)
    pr = layer.pos_ring.cpu().numpy()
    lr = layer.lse_ring.cpu().numpy()
    orr = layer.o_ring.cpu().numpy()
    stats = dict(hits=0, steps=0, exempt=0, diverged=0)
    for b in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            g = h // cfg.group
            o = oracle_lib.run_stream(
                K[b, g], V[b, g], qt[b, h, nw - W:nw], q[b, h, nw - W:nw], qt[b, h, nw:],
                q[b, h, nw:], ctx_len=cfg.ctx, ring_k=cfg.ring_k, band_r=cfg.band_r,
                thresh2=t2, want_ring=True, front_sink=F,
                restart=None if rst is None else rst[b])
            n, ex, div = lockstep_compare(cfg, gpu, o, b, h, cfg.steps)
            stats["steps"] += n
            stats["exempt"] += ex
            stats["hits"] += int(o["hit"][:n].sum())
            if div is not None:
                stats["diverged"] += 1
                continue
            assert np.array_equal(pr[b, g], o["ring_pos"]), (b, h)
            # Slots a restart emptied keep stale contents on the device;
            # only occupied slots are compared.
            occ = o["ring_pos"] >= 0
            fin = np.isfinite(o["ring_lse"]) & occ
            assert np.array_equal(np.isfinite(lr[b, h]) & occ, fin), (b, h)
            np.testing.assert_allclose(lr[b, h][fin], o["ring_lse"][fin], atol=1e-3)
            ok, err = tolerance_check(cfg, orr[b, h][occ], o["ring_o"][occ])
            assert ok, err
    print(cfg.name, "F", F, "flags", flags, stats, flush=True)
    layer.release()
    return gpu, stats


@pytest.mark.parametrize("F,flags", [(64, 0), (128, SPLIT), (128, FUSED), (64, SPLIT | FUSED)])
def test_lockstep_front_sink(oracle_lib, F, flags):
    """Front sinks of 64 and 128 tokens, one launch and three kernels,
    separate and fused append: decisions, outputs and rings as the oracle."""
    cfg = _cfg()
    gpu, st = _lockstep(oracle_lib, cfg, F, flags)
    assert st["diverged"] == 0 and 0.3 < st["hits"] / st["steps"] < 0.97


@pytest.mark.parametrize("n_warm", [0, None])
def test_front_sink_longer_than_context(oracle_lib, n_warm):
    """Positions cross F during the run (m from 100 to 139, F = 128): the
    whole context is sink at first, and ring summaries stay empty until
    m - r reaches F; r larger than the context too."""
    cfg = _cfg(batch=1, n_q_heads=8, n_kv_heads=2, ctx=100, steps=40, ring_k=16, band_r=8,
               sigma=(0.05, 0.05))
    _lockstep(oracle_lib, cfg, 128, 0, n_warm=n_warm)
    _lockstep(oracle_lib, cfg.replace(band_r=300), 64, SPLIT, n_warm=n_warm)


@pytest.mark.parametrize("flags", [0, SPLIT])
def test_front_sink_forced_miss_is_bitwise_full_decode(flags):
    """tau = 1: every step misses; with a front sink the decode step and the
    full decode split the range the same way, so they agree bit for bit."""
    cfg = _cfg(steps=4)
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    p = params_for(cfg, tau=1.0, front_sink=100, flags=flags)
    layer = Layer(cfg, K, V, qt, q, params=p).init()
    gpu = _run(layer, cfg.steps)
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
    layer.release()


def _epoch_schedule(S, B):
    """Request 0: bumped at steps 5 and 6 and again at 15.  Request 1:
    negative (never ready) at steps 9..11, then a new epoch from 12."""
    ep = np.zeros((S, B), np.int32)
    ep[5:, 0] = 1
    ep[6:, 0] = 2
    ep[15:, 0] = 3
    if B > 1:
        ep[9:12, 1] = -1
        ep[12:, 1] = 7
    return ep


@pytest.mark.parametrize("F,flags", [(0, 0), (64, SPLIT), (0, FUSED), (128, SINGLE | FUSED)])
def test_lockstep_epoch_gating(oracle_lib, F, flags):
    cfg = _cfg(sigma=(0.02, 0.1))
    ep = _epoch_schedule(cfg.steps, cfg.batch)
    gpu, st = _lockstep(oracle_lib, cfg, F, flags, epochs=ep)
    assert st["diverged"] == 0
    rst = _restarts(ep)
    for b in range(cfg.batch):
        for s in np.nonzero(rst[b])[0]:
            assert (gpu["p"][s, b] == -1).all() and np.isinf(gpu["d2"][s, b]).all(), (b, s)
    # Requests reuse again after their restarts.
    assert (gpu["p"][7:15, 0] >= 0).any() and (gpu["p"][13:, 1] >= 0).any()


def test_forms_bitwise_with_sink_and_epochs():
    """One launch and three kernels, append separate or fused: identical
    outputs and rings, with a front sink and epoch restarts."""
    cfg = _cfg(steps=18)
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    ep = _epoch_schedule(cfg.steps, cfg.batch)
    runs = []
    for flags, aux in ((SINGLE, torch.cuda.Stream()), (SINGLE | FUSED, None),
                       (SPLIT, torch.cuda.Stream()), (SPLIT | FUSED, None)):
        layer = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=flags, front_sink=64)).init()
        r = _run(layer, cfg.steps, ep, aux=aux)
        r["rings"] = [t.cpu().float().numpy() for t in
                      (layer.q_ring, layer.o_ring, layer.lse_ring, layer.pos_ring)]
        runs.append(r)
        layer.release()
    for r in runs[1:]:
        for k in ("out", "lse", "p", "d2"):
            assert np.array_equal(runs[0][k], r[k]), k
        for x, y in zip(runs[0]["rings"], r["rings"]):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("flags", [FUSED, FUSED | SPLIT, FUSED | TWO])
def test_epoch_gating_inside_captured_graph(flags):
    """A decode step captured once in a HIP graph and replayed (one launch,
    two kernels or three): epochs bumped on the device between replays take
    effect in the graph, and every replay equals the same step run eagerly
    on a second layer.  The two-kernel form alternates its key sets and
    pool sets by the launch epoch counted on the device, so replays of one
    captured launch stay correct."""
    cfg = _cfg(batch=2, steps=12, sigma=(0.02, 0.1))
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    p = params_for(cfg, flags=flags, front_sink=64)
    ep_sched = _epoch_schedule(cfg.steps, cfg.batch)
    ref_layer = Layer(cfg, K, V, qt, q, params=p).init()
    eager = _run(ref_layer, cfg.steps, ep_sched)
    ref_layer.release()

    layer = Layer(cfg, K, V, qt, q, params=p).init()
    B, H, d = cfg.batch, cfg.n_q_heads, cfg.head_dim
    s_qt = torch.empty_like(layer.dec_qt[0])
    s_q = torch.empty_like(layer.dec_q[0])
    s_pos = torch.empty(B, dtype=torch.int32, device=DEV)
    s_out = torch.empty((B, H, d), device=DEV)
    s_mp = torch.empty((B, H), dtype=torch.int32, device=DEV)
    ep = torch.zeros(B, dtype=torch.int32, device=DEV)
    mac.mac_bind_epochs(layer.handle, ep)
    pos = torch.from_numpy(wl.decode_positions(cfg)).to(DEV)
    eps = torch.from_numpy(ep_sched).to(DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        g.capture_begin()
        mac.mac_decode_step(layer.handle, s_qt, s_q, layer.K, layer.V, s_pos, s_out, None,
                            s_mp, None, cs.cuda_stream, None)
        g.capture_end()
    torch.cuda.synchronize()
    for s in range(cfg.steps):
        s_qt.copy_(layer.dec_qt[s])
        s_q.copy_(layer.dec_q[s])
        s_pos.copy_(pos[s])
        ep.copy_(eps[s])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(s_mp.cpu().numpy(), eager["p"][s]), s
        assert np.array_equal(s_out.cpu().numpy(), eager["out"][s]), s
    assert mac.mac_read_device_status(p, layer.ws) == 0
    layer.release()
