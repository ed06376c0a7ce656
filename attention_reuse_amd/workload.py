"""Seeded synthetic decode workloads for the MAC-Attention decode step.

This module only draws inputs.  It holds none of the method's arithmetic
(no attention, no summary merge, no distance or threshold); both the GPU
path and the CPU oracle consume what it produces.

Workload recipe (per configuration):
  * K and V caches: N(0, 1) in fp32, rounded to nearest-even bf16 where the
    configuration is bf16.  All ctx + steps positions are pre-filled (the
    caller appends K_m, V_m before the attention step).  Block (b, g) of K
    is drawn from ``default_rng([seed, 1, b, g])``, of V from
    ``default_rng([seed, 2, b, g])``.
  * Pre-RoPE query stream per (b, h), from ``default_rng([seed, 3, b, h])``:
    P prototype vectors ~ N(0, I_d); an initial prototype drawn uniformly;
    at every later position the stream switches, with probability
    ``switch_p``, to a prototype drawn uniformly among the *other* ones;
    qt = prototype + sigma * N(0, I_d), rounded to the K/V dtype.  Draw
    order inside the generator: prototypes, initial pick, switch uniforms,
    replacement picks, noise.  A per-head sigma range draws sigma_h ~
    U[lo, hi] from ``default_rng([seed, 4])`` once for all heads.
    The stream covers W = min(ring_k, ctx) warm prompt positions
    [ctx - W, ctx - 1] followed by the decode positions ctx .. ctx+steps-1.
  * Post-RoPE query q = RoPE(qt, t): interleaved pairs (x[2j], x[2j+1])
    rotated by angle t * base^(-2j/d), evaluated in fp64 from the stored
    qt and rounded once to fp32 (the caller applies RoPE; angles reach
    ~2.6e5 rad at 262K context, beyond what fp32 sin/cos resolve).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str          # "f32" or "bf16": K/V, pre-RoPE queries, query ring
    ctx: int            # L: prompt length = first decode position
    steps: int          # S: decode steps
    ring_k: int         # K: ring capacity / match window
    band_r: int         # r: rectification band
    tau: float
    rope_base: float
    n_protos: int
    switch_p: float
    sigma: tuple        # (lo, hi); lo == hi for a fixed noise level
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def capacity(self) -> int:
        return self.ctx + self.steps

    @property
    def n_warm(self) -> int:
        return min(self.ring_k, self.ctx)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five decode workloads: a tiny CPU-checkable case and four
# Llama-3-8B-shaped single attention layers (32 query / 8 KV heads, d=128).
WORKLOADS = {
    1: Workload("tiny-4q1kv-d64-f32-2k", 1, 4, 1, 64, "f32", 2048, 64, 64, 32,
                0.6, 1e4, 8, 0.1, (0.05, 0.05)),
    2: Workload("llama3-8b-layer-b1-32k", 1, 32, 8, 128, "bf16", 32768, 256,
                1024, 256, 0.6, 5e5, 16, 0.1, (0.05, 0.05)),
    3: Workload("llama3-8b-layer-b8-128k", 8, 32, 8, 128, "bf16", 131072, 256,
                1024, 256, 0.6, 5e5, 16, 0.1, (0.05, 0.05)),
    4: Workload("llama3-8b-layer-b1-256k", 1, 32, 8, 128, "bf16", 262144, 512,
                1024, 256, 0.6, 5e5, 16, 0.02, (0.05, 0.05)),
    5: Workload("llama3-8b-layer-b16-64k-mixed", 16, 32, 8, 128, "bf16", 65536,
                256, 512, 256, 0.6, 5e5, 16, 0.1, (0.02, 0.5)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32/fp64 values -> storage array (float32, or uint16 bf16 bits)."""
    x32 = np.asarray(x, dtype=np.float32)
    return x32.copy() if dtype == "f32" else f32_to_bf16_bits(x32)


def from_storage(a: np.ndarray) -> np.ndarray:
    """Storage array -> float64 values (exact)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def rope(x: np.ndarray, t: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding in fp64 on the last axis.

    x: [..., n, d] float64, t: [n] positions.  Interleaved pairs
    (x[2j], x[2j+1]) rotate by t * base^(-2j/d) -- a direct product of 2x2
    rotations as the MAC-Attention blog's "Match (1)" section describes.
    """
    d = x.shape[-1]
    j = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / d)
    ang = np.asarray(t, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x, dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _kv_block(cfg: Workload, tag: int, b: int, g: int) -> np.ndarray:
    rng = np.random.default_rng([cfg.seed, tag, b, g])
    x = rng.standard_normal((cfg.capacity, cfg.head_dim), dtype=np.float32)
    return to_storage(x, cfg.dtype)


def gen_kv(cfg: Workload, threads: int | None = None):
    """K, V caches [B, Hkv, ctx+steps, d] (float32 or uint16 bf16 bits)."""
    st = np.float32 if cfg.dtype == "f32" else np.uint16
    shape = (cfg.batch, cfg.n_kv_heads, cfg.capacity, cfg.head_dim)
    K = np.empty(shape, st)
    V = np.empty(shape, st)
    jobs = [(A, tag, b, g) for (A, tag) in ((K, 1), (V, 2))
            for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]

    def one(job):
        A, tag, b, g = job
        A[b, g] = _kv_block(cfg, tag, b, g)

    nt = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(one, jobs))
    return K, V


def head_sigmas(cfg: Workload) -> np.ndarray:
    lo, hi = cfg.sigma
    if lo == hi:
        return np.full((cfg.batch, cfg.n_q_heads), lo, np.float64)
    rng = np.random.default_rng([cfg.seed, 4])
    return rng.uniform(lo, hi, size=(cfg.batch, cfg.n_q_heads))


def stream_positions(cfg: Workload) -> np.ndarray:
    """Absolute positions of the query stream: warm part, then decode."""
    return np.arange(cfg.ctx - cfg.n_warm, cfg.ctx + cfg.steps, dtype=np.int64)


def gen_query_stream(cfg: Workload, b: int, h: int, sigma: float):
    """(qt storage [W+S, d], q float32 [W+S, d], prototype index [W+S])."""
    n = cfg.n_warm + cfg.steps
    P, d = cfg.n_protos, cfg.head_dim
    rng = np.random.default_rng([cfg.seed, 3, b, h])
    protos = rng.standard_normal((P, d))
    first = int(rng.integers(P))
    u = rng.random(n)
    alt = rng.integers(max(P - 1, 1), size=n)
    noise = rng.standard_normal((n, d))
    pick = np.empty(n, np.int64)
    cur = first
    for j in range(n):
        if j > 0 and P > 1 and u[j] < cfg.switch_p:
            cur = (cur + 1 + int(alt[j])) % P
        pick[j] = cur
    qt = to_storage(protos[pick] + sigma * noise, cfg.dtype)
    q = rope(from_storage(qt), stream_positions(cfg), cfg.rope_base)
    return qt, q.astype(np.float32), pick


def gen_queries(cfg: Workload):
    """Query streams for every (b, h).

    Returns qt [B, Hq, W+S, d] (storage dtype), q [B, Hq, W+S, d] float32,
    picks [B, Hq, W+S] (prototype index), sigma [B, Hq].
    """
    B, H, d = cfg.batch, cfg.n_q_heads, cfg.head_dim
    n = cfg.n_warm + cfg.steps
    st = np.float32 if cfg.dtype == "f32" else np.uint16
    qt = np.empty((B, H, n, d), st)
    q = np.empty((B, H, n, d), np.float32)
    picks = np.empty((B, H, n), np.int64)
    sig = head_sigmas(cfg)
    for b in range(B):
        for h in range(H):
            qt[b, h], q[b, h], picks[b, h] = gen_query_stream(cfg, b, h, sig[b, h])
    return qt, q, picks, sig


def decode_positions(cfg: Workload) -> np.ndarray:
    """m for every decode step and request: [S, B] int32."""
    m = cfg.ctx + np.arange(cfg.steps, dtype=np.int32)
    return np.repeat(m[:, None], cfg.batch, axis=1).astype(np.int32)
