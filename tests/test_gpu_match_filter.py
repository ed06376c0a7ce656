"""GPU tests of the match's exact lower-bound filter (MAC-Attention blog,
"Production version: one fused persistent BF16 kernel", match-scan item):
with the filter the step's decisions, outputs and rings are those of the
full scan bit for bit, in both kernel forms."""
import math

import numpy as np
import pytest
import torch

from attention_reuse_amd import mac
from attention_reuse_amd import workload as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mac_harness import Layer, params_for, run_steps

FILTER = mac.MAC_FLAG_MATCH_FILTER


def _cfg(**kw):
    base = dict(name="t", batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
                dtype="bf16", ctx=2500, steps=20, ring_k=256, band_r=64, tau=0.6,
                rope_base=5e5, n_protos=16, switch_p=0.1, sigma=(0.02, 0.5), seed=11)
    base.update(kw)
    return wl.Workload(**base)


def _run(cfg, flags, n_warm=None):
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    layer = Layer(cfg, K, V, qt, q, n_warm=n_warm, params=params_for(cfg, flags=flags)).init()
    r = run_steps(layer, cfg.steps, aux=torch.cuda.Stream())
    r["rings"] = [t.cpu().float().numpy() for t in
                  (layer.q_ring, layer.o_ring, layer.lse_ring, layer.pos_ring)]
    layer.release()
    return r


def _t2(cfg):
    return np.float32(2.0 * cfg.head_dim * (1.0 - float(np.float32(cfg.tau))) ** 2)


@pytest.mark.parametrize("kw", [dict(), dict(dtype="f32", head_dim=64, n_q_heads=8, n_kv_heads=2),
                                dict(head_dim=64), dict(dtype="f32", n_q_heads=8, n_kv_heads=2),
                                # ring sizes that end inside a match unit: a multiple of 4
                                # (positions in 16-byte loads) and one that is not
                                dict(ring_k=252), dict(ring_k=250)])
@pytest.mark.parametrize("form", [mac.MAC_FLAG_SPLIT_STAGES, mac.MAC_FLAG_SINGLE_LAUNCH])
def test_filter_keeps_results_bitwise(kw, form):
    """Mixed hits and misses, every head dim and dtype: the filtered step
    equals the full scan bit for bit; match_d2 agrees on hits and stays at
    or above the threshold on misses."""
    cfg = _cfg(**kw)
    print("filter", kw, "form", form, flush=True)
    ref = _run(cfg, form)
    got = _run(cfg, form | FILTER)
    hit = ref["p"] >= 0
    assert 0.2 < hit.mean() < 0.98, hit.mean()
    for k in ("out", "lse", "p"):
        assert np.array_equal(ref[k], got[k]), k
    for x, y in zip(ref["rings"], got["rings"]):
        assert np.array_equal(x, y)
    assert np.array_equal(ref["d2"][hit], got["d2"][hit])
    assert (got["d2"][~hit] >= _t2(cfg)).all()
    assert (got["d2"][~hit] >= ref["d2"][~hit]).all()


def test_filter_cold_ring_and_forms_agree():
    """Cold ring (empty window first): the two forms with the filter agree
    bit for bit, match_d2 included."""
    cfg = _cfg(batch=1, ctx=900, steps=30, ring_k=64, band_r=16)
    a = _run(cfg, mac.MAC_FLAG_SPLIT_STAGES | FILTER, n_warm=0)
    b = _run(cfg, mac.MAC_FLAG_SINGLE_LAUNCH | FILTER, n_warm=0)
    for k in ("out", "lse", "p", "d2"):
        assert np.array_equal(a[k], b[k]), k
    assert (a["p"][0] == -1).all() and np.isinf(a["d2"][0]).all()


def test_filter_lockstep_against_oracle(oracle_lib):
    """With the filter, decisions and outputs against the oracle directly
    (match_d2 is compared on hits only: on a miss the filter may report a
    farther row, always at or above the threshold)."""
    from mac_harness import tolerance_check
    cfg = _cfg(batch=1, ctx=1500, steps=24, ring_k=128, band_r=32)
    gpu = _run(cfg, mac.MAC_FLAG_SPLIT_STAGES | FILTER)
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    W = cfg.n_warm
    t2 = oracle_lib.threshold2(cfg.head_dim, cfg.tau)
    n_hit = n_cmp = 0
    for h in range(cfg.n_q_heads):
        o = oracle_lib.run_stream(K[0, h // cfg.group], V[0, h // cfg.group], qt[0, h, :W],
                                  q[0, h, :W], qt[0, h, W:], q[0, h, W:], ctx_len=cfg.ctx,
                                  ring_k=cfg.ring_k, band_r=cfg.band_r, thresh2=t2)
        for s in range(cfg.steps):
            g_p, o_p = int(gpu["p"][s, 0, h]), int(o["p"][s])
            # Exempt points (ties, the threshold) must agree too: a
            # disagreement there fails with its distances.
            assert g_p == o_p, (h, s, bool(o["exempt"][s]), o["dist"][s], o["dist2"][s])
            ok, err = tolerance_check(cfg, gpu["out"][s, 0, h], o["out"][s])
            assert ok, (h, s, err)
            if o["hit"][s]:
                n_hit += 1
                assert abs(math.sqrt(gpu["d2"][s, 0, h]) - o["dist"][s]) < 1e-3
            else:
                assert gpu["d2"][s, 0, h] >= _t2(cfg)
            n_cmp += 1
    assert n_cmp == cfg.n_q_heads * cfg.steps and 0.2 * n_cmp < n_hit < n_cmp
