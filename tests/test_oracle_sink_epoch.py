"""Pins of the oracle's attention-sink isolation and ring restarts.

MAC-Attention blog, "Production version: one fused persistent BF16 kernel":
the first F positions (the attention sink) stay out of every reusable
summary and are recomputed exactly on each hit; a ring that is not ready or
was invalidated makes the step exact full attention.  Each test checks the
oracle against brute force (piecewise-logit softmax, nearest-neighbour
search) or the library softmax, never against itself.
"""
import math

import numpy as np
import pytest
import torch

from attention_reuse_amd import workload as wl

from test_oracle_pins import _small, _softmax_attend, _stream


def _owner_closed_form(cfg, res, q, K, V, F, restart=None):
    """Expected outputs as one softmax over piecewise logits per step.

    Summaries of disjoint token sets add, so the output at m is exact
    attention in which position u's logit uses the query of the step that
    computed u's contribution.  A ring entry of step t owns [F, t-r]; a hit
    at p takes those positions from p's entry and computes every other
    position of [0, m] (the sink [0, F) among them) with q_m; a miss computes
    [0, m] with q_m.  Returns [S, d] outputs.
    """
    L, r, W = cfg.ctx, cfg.band_r, cfg.n_warm
    qpos = {L - W + j: q[j].astype(np.float64) for j in range(q.shape[0])}
    rect = {t: {u: t for u in range(F, t - r + 1)} for t in range(L - W, L)}
    outs = []
    for s in range(res["out"].shape[0]):
        m = L + s
        if res["hit"][s]:
            own = dict(rect[int(res["p"][s])])
            for u in range(m + 1):
                own.setdefault(u, m)
        else:
            own = {u: m for u in range(m + 1)}
        rect[m] = {u: own[u] for u in range(F, m - r + 1)}
        Qo = np.stack([qpos[own[u]] for u in range(m + 1)])
        Kf, Vf = wl.from_storage(K[:m + 1]), wl.from_storage(V[:m + 1])
        logits = torch.as_tensor((Qo * Kf).sum(1) / math.sqrt(cfg.head_dim))
        outs.append((torch.softmax(logits, 0) @ torch.as_tensor(Vf)).numpy())
    return np.stack(outs)


def _check_decisions(oracle_lib, cfg, res, qt, restart=None):
    """Nearest pre-RoPE query among the last K positions that the ring still
    holds (positions appended since the latest restart), ties to the larger
    position, accepted below the threshold."""
    t2 = oracle_lib.threshold2(cfg.head_dim, cfg.tau)
    qv = wl.from_storage(qt)
    W, L = cfg.n_warm, cfg.ctx
    first = L - W
    for s in range(res["out"].shape[0]):
        m = L + s
        if restart is not None and restart[s]:
            first = m
        cand = list(range(max(first, m - cfg.ring_k), m))
        if not cand:
            assert not res["hit"][s] and res["dist"][s] == math.inf
            continue
        D = {t: float(((qv[W + s] - qv[t - (L - W)]) ** 2).sum()) for t in cand}
        best = min(cand, key=lambda t: (D[t], -t))
        hit = D[best] < t2
        assert bool(res["hit"][s]) == hit, s
        assert res["p"][s] == (best if hit else -1), s


@pytest.mark.parametrize("F", [1, 5, 13, 38, 80])
@pytest.mark.parametrize("kw", [dict(), dict(dtype="bf16", band_r=3, ring_k=5),
                                dict(switch_p=0.5, n_protos=4, ring_k=16, band_r=8)])
def test_sink_piecewise_closed_form(oracle_lib, F, kw):
    cfg = _small(**kw)
    for h in range(cfg.n_q_heads):
        res, K, V, qt, q = _stream(oracle_lib, cfg, h=h, front_sink=F)
        _check_decisions(oracle_lib, cfg, res, qt)
        assert res["hit"].any()
        ref = _owner_closed_form(cfg, res, q, K, V, F)
        np.testing.assert_allclose(res["out"], ref, atol=2e-6, rtol=0)


@pytest.mark.parametrize("F", [0, 3, 7])
def test_sink_ring_summaries_cover_front_to_band(oracle_lib, F):
    """Threshold 0 (every step misses): outputs are full attention, and the
    entry each step leaves in the ring is attention over [F, m-r] alone,
    empty when m - r < F."""
    cfg = _small(ctx=6, ring_k=8, band_r=4, steps=8)
    res, K, V, qt, q = _stream(oracle_lib, cfg, thresh2=0.0, want_ring=True, front_sink=F)
    d, r = cfg.head_dim, cfg.band_r
    for s in range(cfg.steps):
        m = cfg.ctx + s
        ref, ref_l = _softmax_attend(q[cfg.n_warm + s], K[:m + 1], V[:m + 1], 1 / math.sqrt(d))
        np.testing.assert_allclose(res["out"][s], ref, atol=1e-12)
        assert abs(res["lse"][s] - ref_l) < 1e-12
    for k in range(cfg.ring_k):
        m = int(res["ring_pos"][k])
        s = m - cfg.ctx
        if m - r < F:
            assert res["ring_lse"][k] == -math.inf
            assert (res["ring_o"][k] == 0).all()
            continue
        ref, ref_l = _softmax_attend(q[cfg.n_warm + s], K[F:m - r + 1], V[F:m - r + 1],
                                     1 / math.sqrt(d))
        np.testing.assert_allclose(res["ring_o"][k], ref, atol=1e-6)
        assert abs(res["ring_lse"][k] - ref_l) < 1e-5


@pytest.mark.parametrize("F", [0, 4, 9])
def test_sink_warm_summaries(oracle_lib, F):
    """Warm entries for prompt positions t cover [F, t-r] with q_t."""
    cfg = _small(ctx=20, ring_k=8, band_r=4)
    res, K, V, qt, q = _stream(oracle_lib, cfg, n_steps=0, want_ring=True, front_sink=F)
    L, W, r = cfg.ctx, cfg.n_warm, cfg.band_r
    for k in range(cfg.ring_k):
        t = int(res["ring_pos"][k])
        assert L - W <= t < L
        if t - r < F:
            assert res["ring_lse"][k] == -math.inf
            continue
        ref, ref_l = _softmax_attend(q[t - (L - W)], K[F:t - r + 1], V[F:t - r + 1],
                                     1 / math.sqrt(cfg.head_dim))
        np.testing.assert_allclose(res["ring_o"][k], ref, atol=1e-6)
        assert abs(res["ring_lse"][k] - ref_l) < 1e-5


@pytest.mark.parametrize("F", [2, 16])
def test_sink_exact_reuse_invariant(oracle_lib, F):
    """Identity RoPE and one noiseless prototype: every reuse is exact, so
    sink + cached + fresh must tile [0, m] and the output equals full
    attention."""
    cfg = _small(n_protos=1, sigma=(0.0, 0.0), steps=40, switch_p=0.0)
    res, K, V, qt, q = _stream(
        oracle_lib, cfg, front_sink=F,
        q_override=lambda qt, q: wl.from_storage(qt).astype(np.float32))
    assert res["hit"].all()
    m = cfg.ctx + np.arange(cfg.steps)
    qv = wl.from_storage(qt)
    for s in range(cfg.steps):
        ref, ref_l = _softmax_attend(qv[cfg.n_warm + s], K[:m[s] + 1], V[:m[s] + 1],
                                     1 / math.sqrt(cfg.head_dim))
        np.testing.assert_allclose(res["out"][s], ref, atol=2e-6)
        assert abs(res["lse"][s] - ref_l) < 1e-6


@pytest.mark.parametrize("F", [0, 6])
def test_restart_makes_step_exact_and_drops_ring(oracle_lib, F):
    """A restart before step s: no candidate at s (exact attention), and the
    later steps see only positions appended since."""
    cfg = _small(steps=30, switch_p=0.3)
    restart = np.zeros(cfg.steps, np.int32)
    restart[[0, 7, 8, 19]] = 1
    for h in range(cfg.n_q_heads):
        res, K, V, qt, q = _stream(oracle_lib, cfg, h=h, front_sink=F, restart=restart)
        _check_decisions(oracle_lib, cfg, res, qt, restart)
        for s in np.nonzero(restart)[0]:
            m = cfg.ctx + s
            ref, ref_l = _softmax_attend(q[cfg.n_warm + s], K[:m + 1], V[:m + 1],
                                         1 / math.sqrt(cfg.head_dim))
            np.testing.assert_allclose(res["out"][s], ref, atol=1e-12)
        assert res["hit"][1:7].any() and res["hit"][9:19].any()
        ref = _owner_closed_form(cfg, res, q, K, V, F, restart)
        np.testing.assert_allclose(res["out"], ref, atol=2e-6, rtol=0)


def test_restart_every_step_never_hits(oracle_lib):
    cfg = _small(steps=12)
    res, K, V, qt, q = _stream(oracle_lib, cfg, restart=np.ones(cfg.steps, np.int32))
    assert not res["hit"].any() and (res["dist"] == math.inf).all()
