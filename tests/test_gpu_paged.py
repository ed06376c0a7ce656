"""GPU tests of the paged K/V input and the fused KV-RoPE append (MAC-Attention
blog, "Production version: one fused persistent BF16 kernel": the production
kernel reads the serving engine's paged BF16 KV, with RoPE fused into the KV
write).  Paged runs must equal dense runs on the same data bit for bit; the
append is checked against the oracle's RoPE (fp64), rounded once."""
import math

import numpy as np
import pytest
import torch

from attention_reuse_amd import mac
from attention_reuse_amd import workload as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mac_harness import DEV, Layer, params_for, run_steps, to_dev


def _cfg(**kw):
    base = dict(name="t", batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
                dtype="bf16", ctx=1800, steps=12, ring_k=128, band_r=48, tau=0.6,
                rope_base=5e5, n_protos=16, switch_p=0.1, sigma=(0.02, 0.5), seed=5)
    base.update(kw)
    return wl.Workload(**base)


def _paged(K, P, layout, rng, spare=3):
    """Scatter dense [B, Hkv, T, d] storage into a shuffled page pool.
    Returns (pool, table [B, pages] int32, strides in elements)."""
    B, Hkv, T, d = K.shape
    npg = -(-T // P)
    total = B * npg + spare
    table = rng.permutation(total)[:B * npg].reshape(B, npg).astype(np.int32)
    if layout == "HND":
        pool = np.zeros((total, Hkv, P, d), K.dtype)
        strides = (Hkv * P * d, P * d, d)
    else:
        pool = np.zeros((total, P, Hkv, d), K.dtype)
        strides = (P * Hkv * d, d, Hkv * d)
    for b in range(B):
        for j in range(npg):
            n = min(P, T - j * P)
            blk = K[b, :, j * P:j * P + n]
            if layout == "HND":
                pool[table[b, j], :, :n] = blk
            else:
                pool[table[b, j], :n] = np.swapaxes(blk, 0, 1)
    return pool, table, strides


def _layers(cfg, P, layout, flags=0, front_sink=0):
    rng = np.random.default_rng(123)
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    dense = Layer(cfg, K, V, qt, q, params=params_for(cfg, flags=flags, front_sink=front_sink))
    kp, table, strides = _paged(K, P, layout, rng)
    vp, table2, _ = _paged(V, P, layout, np.random.default_rng(123))
    assert np.array_equal(table, table2)
    tdev = to_dev(table)
    pp = params_for(cfg, flags=flags, front_sink=front_sink, page_size=P,
                    max_pages=table.shape[1], page_table=tdev, strides=strides)
    paged = Layer(cfg, K, V, qt, q, params=pp, kv_dev=(to_dev(kp), to_dev(vp)))
    paged.table = tdev  # keeps the table alive
    return dense, paged


def _rings(layer):
    return [t.cpu().float().numpy() for t in
            (layer.q_ring, layer.o_ring, layer.lse_ring, layer.pos_ring)]


@pytest.mark.parametrize("P,layout,flags,F", [
    (16, "HND", mac.MAC_FLAG_SINGLE_LAUNCH, 0), (64, "NHD", mac.MAC_FLAG_SPLIT_STAGES, 0),
    (32, "NHD", mac.MAC_FLAG_SINGLE_LAUNCH | mac.MAC_FLAG_FUSED_APPEND, 64),
    (128, "HND", mac.MAC_FLAG_SPLIT_STAGES | mac.MAC_FLAG_FUSED_APPEND, 128)])
def test_paged_decode_equals_dense(P, layout, flags, F):
    cfg = _cfg()
    print("paged", P, layout, flags, F, flush=True)
    dense, paged = _layers(cfg, P, layout, flags, F)
    a = run_steps(dense.init(), cfg.steps, aux=torch.cuda.Stream())
    b = run_steps(paged.init(), cfg.steps, aux=torch.cuda.Stream())
    assert 0.2 < (a["p"] >= 0).mean() < 0.98
    for k in ("out", "lse", "p", "d2"):
        assert np.array_equal(a[k], b[k]), k
    for x, y in zip(_rings(dense), _rings(paged)):
        assert np.array_equal(x, y)
    dense.release()
    paged.release()


@pytest.mark.parametrize("dtype,d,P", [("bf16", 128, 16), ("f32", 64, 64), ("bf16", 64, 32),
                                       ("f32", 128, 256)])
def test_paged_full_decode_equals_dense(dtype, d, P):
    cfg = _cfg(dtype=dtype, head_dim=d, n_q_heads=8, n_kv_heads=2, ctx=1000, steps=2)
    dense, paged = _layers(cfg, P, "HND")
    m = np.array([0, cfg.capacity - 1], np.int32)
    outs = []
    for L in (dense, paged):
        ws_b = mac.mac_workspace_bytes(L.p)
        ws = torch.empty(ws_b, dtype=torch.uint8, device=DEV)
        out = torch.empty((cfg.batch, cfg.n_q_heads, d), device=DEV)
        for mm in (m, np.array([517, 63], np.int32)):
            mac.mac_full_decode(L.p, L.dec_q[0], L.K, L.V, to_dev(mm), out, None, ws, ws_b,
                                torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])


def _rope_expect(oracle_lib, x, pos, base, dtype, to_fp32=False):
    """The oracle's rotation (fp64), then one rounding (bf16 via
    round-to-odd fp32)."""
    y = np.stack([oracle_lib.rope(r, int(pos), base) for r in wl.from_storage(x)])
    if to_fp32:
        return y.astype(np.float32)
    if dtype == "f32":
        return y.astype(np.float32)
    f = y.astype(np.float32)
    # round to odd: truncate toward zero, set the last bit if inexact
    trunc = np.where(np.abs(f.astype(np.float64)) > np.abs(y),
                     np.nextafter(f, np.float32(0)), f).astype(np.float32)
    bits = trunc.view(np.uint32) | (trunc.astype(np.float64) != y).astype(np.uint32)
    return wl.f32_to_bf16_bits(bits.view(np.float32))


@pytest.mark.parametrize("dtype,d,P", [("bf16", 128, 0), ("bf16", 128, 16), ("f32", 64, 64)])
def test_append_kv_fuses_rope(oracle_lib, dtype, d, P):
    cfg = _cfg(dtype=dtype, head_dim=d, n_q_heads=8, n_kv_heads=2, ctx=300, steps=4)
    rng = np.random.default_rng(9)
    B, Hkv, Hq, T = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.capacity
    base = 5e5
    kn = wl.to_storage(rng.standard_normal((B, Hkv, d)), dtype)
    vn = wl.to_storage(rng.standard_normal((B, Hkv, d)), dtype)
    qn = wl.to_storage(rng.standard_normal((B, Hq, d)), dtype)
    pos = np.array([T - 1, 17], np.int32)
    K0 = wl.to_storage(np.full((B, Hkv, T, d), 7.0), dtype)
    if P:
        kp, table, strides = _paged(K0, P, "NHD", rng)
        tdev = to_dev(table)
        p = params_for(cfg, page_size=P, max_pages=table.shape[1], page_table=tdev,
                       strides=strides)
        kc, vc = to_dev(kp), to_dev(kp.copy())
    else:
        p = params_for(cfg)
        kc, vc = to_dev(K0), to_dev(K0.copy())
    qo = torch.empty((B, Hq, d), device=DEV)
    mac.mac_append_kv(p, to_dev(kn), to_dev(vn), to_dev(pos), base, kc, vc, to_dev(qn), qo,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    def view(c):
        a = c.cpu()
        a = (a.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else a.numpy())
        if not P:
            return a
        out = np.empty((B, Hkv, T, d), a.dtype)
        for b in range(B):
            for j in range(table.shape[1]):
                n = min(P, T - j * P)
                out[b, :, j * P:j * P + n] = np.swapaxes(a[table[b, j], :n], 0, 1)
        return out

    Kc, Vc = view(kc), view(vc)
    mask = np.zeros((B, Hkv, T), bool)
    for b in range(B):
        mask[b, :, pos[b]] = True
        for g in range(Hkv):
            want = _rope_expect(oracle_lib, kn[b, g][None], pos[b], base, dtype)[0]
            got = Kc[b, g, pos[b]]
            if dtype == "f32":
                np.testing.assert_array_max_ulp(got, want, maxulp=1)
            else:
                assert np.abs(got.astype(np.int32) - want.astype(np.int32)).max() <= 1
                assert (got == want).mean() > 0.99
            assert np.array_equal(Vc[b, g, pos[b]], vn[b, g])
        for h in range(Hq):
            want = _rope_expect(oracle_lib, qn[b, h][None], pos[b], base, dtype, to_fp32=True)[0]
            np.testing.assert_array_max_ulp(qo[b, h].cpu().numpy(), want, maxulp=1)
    # Every other row is untouched.
    assert np.array_equal(Kc[~mask], K0[~mask]) and np.array_equal(Vc[~mask], K0[~mask])


@pytest.mark.parametrize("flags", [mac.MAC_FLAG_SINGLE_LAUNCH, mac.MAC_FLAG_SPLIT_STAGES | mac.MAC_FLAG_FUSED_APPEND])
def test_features_together_equal_plain_run(flags):
    """Paged K/V, the match filter, a front sink and epoch restarts at once:
    outputs, decisions and rings equal those of a dense, unfiltered run with
    the same sink and epochs, bit for bit (match_d2 on hits)."""
    from test_gpu_sink_epoch import _epoch_schedule, _run
    cfg = _cfg(steps=18)
    ep = _epoch_schedule(cfg.steps, cfg.batch)
    dense, paged = _layers(cfg, 32, "NHD", flags, 64)
    paged.p.flags |= mac.MAC_FLAG_MATCH_FILTER
    a = _run(dense.init(), cfg.steps, ep, aux=torch.cuda.Stream())
    b = _run(paged.init(), cfg.steps, ep, aux=torch.cuda.Stream())
    hit = a["p"] >= 0
    assert 0.2 < hit.mean() < 0.98
    for k in ("out", "lse", "p"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["d2"][hit], b["d2"][hit])
    for x, y in zip(_rings(dense), _rings(paged)):
        assert np.array_equal(x, y)
    dense.release()
    paged.release()
