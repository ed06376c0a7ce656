"""Per-workgroup timeline of the decode step's step kernel (diagnostics).

Runs a synthetic workload through ``libmac_attention_timeline.so`` (the
library built with ``python -m attention_reuse_amd.build --timeline``, in
which the step kernel writes the device's 100 MHz real-time counter at
fixed points of every workgroup; see ``mac_timeline_read`` in
``include/mac_attention.h``) and prints, for the last step kernel launched,
the distribution over workgroups of each point, in microseconds from the
launch's first workgroup start.  The instrumented build writes a few words
per workgroup more than the default one, so its times are close to, not
equal to, those of the default build.

    python -m attention_reuse_amd.timeline --config 3
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

from . import build as hip_build
from . import mac
from . import workload as wl

MARKS = [(0, "workgroup start"), (1, "keys stored / queries staged"),
         (2, "speculative K/V requested"), (3, "group planned"),
         (4, "items published"), (24, "own items: queries in regs"),
         (25, "first item's bounds"), (26, "first item's rows requested"),
         (5, "first item begins"), (27, "item blocks done (latest)"),
         (28, "item rows in LDS (latest)"), (29, "item weights and sums (latest)"),
         (6, "first item computed"),
         (7, "first partial stored"), (8, "first item counted"), (9, "own items done"),
         (20, "merge begins"), (21, "merge: weights / list A"),
         (22, "merge: lists summed"), (23, "merge: outputs written"),
         (10, "merge done (mergers)"), (13, "first pool item"),
         (11, "end (ran items)"), (12, "end (no own item)")]
NOTES = [(16, "items of the group"), (17, "items of its own workgroups"),
         (19, "pool items run")]
TICK_US = 0.01  # 100 MHz


def percentiles(x):
    x = np.sort(np.asarray(x, dtype=np.float64))
    if len(x) == 0:
        return "-"
    q = lambda f: x[min(len(x) - 1, int(f * (len(x) - 1) + 0.5))]
    return "%7.2f %7.2f %7.2f %7.2f %7.2f" % (x[0], q(0.1), q(0.5), q(0.9), x[-1])


def summarize(words):
    """Table lines for the latest launch in the timeline words."""
    w = np.asarray(words, dtype=np.uint64).astype(np.int64)
    entry = w[:, 0]
    live = entry > 0
    if not live.any():
        return ["no step kernel launch recorded"]
    # The latest launch: workgroups that started within 20 us of the last start.
    last = entry[live].max()
    sel = live & (entry >= last - 2000)
    wg = w[sel]
    t0 = wg[:, 0].min()
    lines = ["workgroups of the latest launch: %d" % len(wg),
             "%-30s %5s %7s %7s %7s %7s %7s" % ("point (us from first start)", "n", "min",
                                                 "p10", "p50", "p90", "max")]
    for slot, name in MARKS:
        v = wg[:, slot]
        ok = v >= wg[:, 0]  # written by this launch
        lines.append("%-30s %5d %s" % (name, int(ok.sum()), percentiles((v[ok] - t0) * TICK_US)))
    lines.append("%-30s %5s %7s %7s %7s %7s %7s" % ("count", "n", "min", "p10", "p50", "p90",
                                                     "max"))
    published = wg[:, 4] >= wg[:, 0]
    for slot, name in NOTES:
        ok = published if slot != 19 else (wg[:, 11] >= wg[:, 0])
        lines.append("%-30s %5d %s" % (name, int(ok.sum()), percentiles(wg[ok, slot])))
    began = wg[:, 5] >= wg[:, 0]
    spec = wg[began, 18]
    lines.append("first item from speculative rows: %d, re-requested: %d, none: %d" % (
        int((spec == 1).sum()), int((spec == 2).sum()), int((spec == 0).sum())))
    return lines


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", type=int, default=3, help="workload index (workload.py)")
    ap.add_argument("--launch", choices=("auto", "single", "two"), default="auto")
    ap.add_argument("--layers", type=int, default=8, help="layer copies stepped in turn")
    ap.add_argument("--steps", type=int, default=12, help="decode steps before the read")
    ap.add_argument("--match-filter", choices=("auto", "on", "off"), default="auto")
    args = ap.parse_args(argv)
    if not os.path.exists(hip_build.TIMELINE_LIB):
        sys.exit("%s is missing: build it with python -m attention_reuse_amd.build --timeline"
                 % hip_build.TIMELINE_LIB)
    mac.LIB_PATH = hip_build.TIMELINE_LIB
    import torch

    mac.load()
    dev = "cuda:0"
    cfg = wl.WORKLOADS[args.config]
    B, H, Hkv, d, R, W = (cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                          cfg.ring_k, cfg.n_warm)
    filt = (args.match_filter == "on" or (args.match_filter == "auto" and (
        args.launch == "two" or (args.launch == "auto" and B * Hkv > 16))))
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    K0, V0 = to_dev(K), to_dev(V)
    del K, V
    dec_qt = to_dev(np.moveaxis(qt[:, :, W:], 2, 0))
    dec_q = to_dev(np.moveaxis(q[:, :, W:], 2, 0))
    pos = to_dev(wl.decode_positions(cfg))
    flags = (mac.MAC_FLAG_FUSED_APPEND | (mac.MAC_FLAG_MATCH_FILTER if filt else 0)
             | {"auto": 0, "single": mac.MAC_FLAG_SINGLE_LAUNCH,
                "two": mac.MAC_FLAG_TWO_STAGES}[args.launch])
    p = mac.make_params(B, H, Hkv, d, mac.MAC_DTYPE_F32 if cfg.dtype == "f32"
                        else mac.MAC_DTYPE_BF16, R, cfg.band_r, cfg.capacity, cfg.tau,
                        flags=flags)
    wsb = mac.mac_workspace_bytes(p)
    st = torch.cuda.current_stream().cuda_stream
    layers = []
    for li in range(args.layers):
        layers.append(dict(
            K=K0 if li == 0 else K0.clone(), V=V0 if li == 0 else V0.clone(),
            q_ring=torch.zeros((B, H, R, d), dtype=K0.dtype, device=dev),
            o_ring=torch.zeros((B, H, R, d), device=dev),
            lse_ring=torch.zeros((B, H, R), device=dev),
            pos_ring=torch.zeros((B, Hkv, R), dtype=torch.int32, device=dev),
            ws=torch.empty(wsb, dtype=torch.uint8, device=dev),
            out=torch.empty((B, H, d), device=dev)))
    L0 = layers[0]
    h0 = mac.mac_init_rings(p, L0["q_ring"], L0["o_ring"], L0["lse_ring"], L0["pos_ring"],
                            L0["ws"], wsb, to_dev(qt[:, :, :W]), to_dev(q[:, :, :W]), W,
                            [cfg.ctx] * B, L0["K"], L0["V"], st)
    torch.cuda.synchronize()
    warm = [L0[k].clone() for k in ("q_ring", "o_ring", "lse_ring", "pos_ring")]
    mac.mac_release(h0)
    for L in layers:
        L["h"] = mac.mac_init_rings(p, L["q_ring"], L["o_ring"], L["lse_ring"], L["pos_ring"],
                                    L["ws"], wsb, None, None, 0, [cfg.ctx] * B, L["K"],
                                    L["V"], st)
        for k, src in zip(("q_ring", "o_ring", "lse_ring", "pos_ring"), warm):
            L[k].copy_(src)
    torch.cuda.synchronize()
    n = min(args.steps, cfg.steps)
    for s in range(n):
        for L in layers:
            mac.mac_decode_step(L["h"], dec_qt[s], dec_q[s], L["K"], L["V"], pos[s], L["out"],
                                None, None, None, st, None)
    torch.cuda.synchronize()
    words = mac.mac_timeline_read(layers[-1]["h"])
    print("%s, launch %s, match filter %s, %d layers, %d steps" % (
        cfg.name, args.launch, "on" if filt else "off", args.layers, n))
    for line in summarize(words):
        print(line)
    for L in layers:
        mac.mac_release(L["h"])


if __name__ == "__main__":
    main()
