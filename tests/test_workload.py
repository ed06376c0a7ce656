"""Statistics and identities of the synthetic workload generator."""
import math

import numpy as np
import torch

from attention_reuse_amd import workload as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties to even
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_rope_norm_and_composition():
    rng = np.random.default_rng(1)
    d = 128
    x = rng.standard_normal((5, d))
    t = np.array([0, 1, 1000, 262143, 7])
    y = wl.rope(x, t, 5e5)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(y[0], x[0], atol=0)          # position 0 is the identity
    # R(a) R(b) = R(a + b)
    a, b = 1234, 56789
    ab = wl.rope(wl.rope(x[:1], np.array([a]), 5e5), np.array([b]), 5e5)
    np.testing.assert_allclose(ab, wl.rope(x[:1], np.array([a + b]), 5e5), atol=1e-9)


def test_rope_distance_avgcos_identity():
    """|x - R(D)x|^2 = 2|x|^2 (1 - avgcos(D)) with avgcos the energy-weighted
    mean cosine over the rotation frequencies (MAC-Attention blog, "Match
    (1): why match in pre-RoPE space")."""
    rng = np.random.default_rng(2)
    d, base = 64, 1e4
    x = rng.standard_normal(d)
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    energy = x[0::2] ** 2 + x[1::2] ** 2
    for delta in (1, 5, 100, 4096):
        lhs = float(((x - wl.rope(x[None], np.array([delta]), base)[0]) ** 2).sum())
        avgcos = float((energy * np.cos(delta * theta)).sum() / energy.sum())
        assert abs(lhs - 2 * (x @ x) * (1 - avgcos)) < 1e-9
    # Dephasing: far apart, the distance approaches 2|x|^2.
    far = [float(((x - wl.rope(x[None], np.array([D]), base)[0]) ** 2).sum())
           for D in range(10000, 10400)]
    assert abs(np.mean(far) / (2 * (x @ x)) - 1) < 0.15


def test_query_stream_statistics():
    cfg = wl.WORKLOADS[2].replace(batch=1, n_q_heads=4, n_kv_heads=1, ctx=4096,
                                  steps=2048, ring_k=1024)
    sig = 0.05
    switches, same, diff = [], [], []
    for h in range(cfg.n_q_heads):
        qt, q, pick = wl.gen_query_stream(cfg, 0, h, sig)
        switches.append(np.mean(pick[1:] != pick[:-1]))
        x = wl.from_storage(qt)
        D = ((x[1:] - x[:-1]) ** 2).sum(1)
        same.append(D[pick[1:] == pick[:-1]].mean())
        diff.append(D[pick[1:] != pick[:-1]].mean())
        # Post-RoPE query is the rotation of the stored pre-RoPE query.
        pos = wl.stream_positions(cfg)
        np.testing.assert_allclose(q, wl.rope(x, pos, cfg.rope_base).astype(np.float32), atol=0)
    assert abs(np.mean(switches) - cfg.switch_p) < 0.02
    # Same prototype: D ~ 2 sigma^2 chi^2_d, mean 2 d sigma^2.
    assert abs(np.mean(same) / (2 * cfg.head_dim * sig ** 2) - 1) < 0.1
    # Different prototypes: the chance baseline, mean 2 d (1 + sigma^2)
    # (the Gaussian null of the blog's "Match (2)" section).
    assert abs(np.mean(diff) / (2 * cfg.head_dim * (1 + sig ** 2)) - 1) < 0.1


def test_head_sigmas_range_and_determinism():
    cfg = wl.WORKLOADS[5]
    s = wl.head_sigmas(cfg)
    assert s.shape == (16, 32) and s.min() >= 0.02 and s.max() <= 0.5
    assert np.array_equal(s, wl.head_sigmas(cfg))
    assert (wl.head_sigmas(wl.WORKLOADS[2]) == 0.05).all()


def test_kv_deterministic_and_normal():
    cfg = wl.WORKLOADS[1]
    K1, V1 = wl.gen_kv(cfg)
    K2, V2 = wl.gen_kv(cfg, threads=1)
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2)
    assert K1.shape == (1, 1, 2048 + 64, 64) and K1.dtype == np.float32
    assert abs(K1.mean()) < 0.01 and abs(K1.std() - 1) < 0.01
    cfgb = cfg.replace(dtype="bf16")
    Kb, _ = wl.gen_kv(cfgb)
    assert Kb.dtype == np.uint16
    assert np.array_equal(Kb, wl.f32_to_bf16_bits(K1))


def test_workload_table():
    w = wl.WORKLOADS
    assert [w[i].capacity for i in range(1, 6)] == [2112, 33024, 131328, 262656, 65792]
    assert all(w[i].group == 4 for i in range(1, 6))
    assert w[4].switch_p == 0.02 and w[5].sigma == (0.02, 0.5) and w[5].ring_k == 512
    assert math.isclose(w[1].tau, 0.6)
