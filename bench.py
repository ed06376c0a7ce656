"""Decode-attention throughput of the MAC-Attention step on one MI355X.

One step = one MAC decode step (match, plan, attention, merge,
rectify-append) at one position m over NL independent copies of the
attention layer (the layers of a model), each with its own K/V cache and
rings, so the per-step working set is far larger than the 256 MB Infinity
Cache.  Inputs are seeded synthetic data resident in HBM before timing.

Prints one JSON line:  value = B * Hq * NL / t_step  (heads*layers per s).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from attention_reuse_amd import workload as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
STAGES = ("match", "attend", "merge", "append", "step")
KERNEL_NAMES = {"match": "match_kernel", "attend": "attend_kernel",
                "merge": "merge_kernel", "append": "append_kernel", "step": "step_kernel"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=8)
    # Default: the largest workload on one GPU (8 requests x 128K context,
    # 4 GiB of K/V per layer).
    ap.add_argument("--config", type=int, default=3, choices=sorted(wl.WORKLOADS))
    ap.add_argument("--layers", type=int, default=0,
                    help="layer copies per step (0 = enough to overflow the Infinity Cache)")
    ap.add_argument("--mode", choices=("mac", "full"), default="mac")
    ap.add_argument("--append", choices=("aux", "fused"), default="fused",
                    help="rectify-append on the auxiliary stream or fused into the merge")
    ap.add_argument("--launch", choices=("auto", "single", "two", "split"), default="auto",
                    help="decode step as one launch, as a match kernel and one launch for "
                         "plan / attention / merge, as match / attend / merge kernels, "
                         "or the library's choice for the shape")
    ap.add_argument("--match-filter", choices=("auto", "on", "off"), default="auto",
                    help="exact lower-bound filter of the match (second halves of ring "
                         "rows read only where a hit is still possible); auto: on where "
                         "the step runs the match kernel (more than 16 KV groups per "
                         "layer, or --launch two / split), where the match is bound by "
                         "bandwidth, off in the one-launch step, where it is bound by "
                         "latency")
    ap.add_argument("--page-size", type=int, default=0,
                    help="read K/V from a paged pool with pages of this many tokens, "
                         "shuffled through a page table (0 = dense cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--no-full", action="store_true",
                    help="skip the same-run full-decode comparison")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the steps (one graph per step, all "
                         "layers; needs --append fused) instead of eager launches")
    ap.add_argument("--thresh", choices=("one-minus-tau", "tau"), default="one-minus-tau",
                    help="acceptance threshold: distance < (1 - tau) sqrt(2d) (default), or "
                         "< tau sqrt(2d), the other reading of the pages")
    ap.add_argument("--alloc", choices=("pool", "layer"), default="pool",
                    help="K/V, rings and workspaces of all layers as slices of one "
                         "allocation each (as a serving engine's KV pool), or one "
                         "allocation per layer and tensor")
    ap.add_argument("--json-out", default="")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def default_layers(cfg):
    """Enough layer copies that one step touches >= 3x the 256 MB Infinity
    Cache (rings plus a band+tail estimate per layer), so a layer's data is
    evicted before the next step returns to it."""
    e = cfg.elem_bytes
    est = (cfg.batch * cfg.n_q_heads * cfg.ring_k * cfg.head_dim * e
           + cfg.batch * cfg.n_kv_heads * (2 * cfg.band_r + 512) * cfg.head_dim * e * 2)
    return int(max(1, min(64, math.ceil(768 * 2 ** 20 / est))))


DEVICE_SOURCES = ("mac_device.h", "mac_internal.h", "mac_kernels.hip", "mac_step_impl.h",
                  "mac_step_bf16_128.hip", "mac_step_bf16_64.hip", "mac_step_f32_128.hip",
                  "mac_step_f32_64.hip")


def source_hash():
    """Hash of the device-code sources the PMC counters were taken on."""
    h = hashlib.sha256()
    for f in DEVICE_SOURCES:
        h.update(open(os.path.join(ROOT, "attention_reuse_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def thresh_mode(args):
    from attention_reuse_amd import mac
    return mac.MAC_THRESH_TAU if args.thresh == "tau" else mac.MAC_THRESH_ONE_MINUS_TAU


def read_traffic(workload_name, kernel):
    """HBM traffic per launch from committed rocprofv3 PMC summaries, if they
    were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    want = source_hash()
    for ln in open(path):
        f = ln.split()
        if len(f) >= 4 and not ln.startswith("#") and f[0] == workload_name and f[1] == kernel:
            return float(f[2]) if f[-1] == want else None
    return None


def filter_second_halves(cfg, qt, s):
    """Ring rows whose second half the match filter reads at decode step s:
    candidates whose first-half squared distance (fp32) is below the
    threshold times the filter margin.  qt: [B, Hq, W+S, d] storage."""
    W, K, d = cfg.n_warm, min(cfg.ring_k, cfg.ctx), cfg.head_dim
    cur = wl.from_storage(qt[:, :, W + s, : d // 2]).astype(np.float32)
    ring = wl.from_storage(qt[:, :, W + s - K:W + s, : d // 2]).astype(np.float32)
    lb = ((ring - cur[:, :, None, :]) ** 2).sum(-1, dtype=np.float32)
    t2 = np.float32(2.0 * d * (1.0 - float(np.float32(cfg.tau))) ** 2)
    return int((lb < t2 * np.float32(1.0 + 1.0 / 1024.0)).sum())


def algorithmic_bytes(cfg, match_p, m, second_halves=None):
    """Bytes the method must move per layer-step, by stage.

    match_p: [B, Hq] matched position (-1 miss); m: [B] positions;
    second_halves: with the match filter, the ring rows read in full."""
    B, H, Hkv, G, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.group, cfg.head_dim
    e = cfg.elem_bytes
    K_valid = min(cfg.ring_k, cfg.ctx)
    rows = B * H * K_valid * d * e
    if second_halves is not None:
        rows = rows // 2 + second_halves * (d * e // 2)
    match = rows + B * Hkv * K_valid * 4 + B * H * d * e
    start = np.where(match_p >= 0, np.maximum(0, match_p - cfg.band_r + 1), 0)
    s_g = start.reshape(B, Hkv, G).min(axis=2)
    span = (m[:, None] - s_g + 1).astype(np.int64)
    kv = int(span.sum()) * d * e * 2
    attend = kv + B * H * d * 4
    hits = int((match_p >= 0).sum())
    # The merge reads the cached summary of every hit head and writes the
    # output and its lse (split-KV partials are overhead, not credited).
    merge = hits * (d + 1) * 4 + B * H * (d + 1) * 4
    append = B * H * (d * e + (d + 1) * 4) + B * Hkv * 4
    full_kv = int((m + 1).sum()) * Hkv * d * e * 2
    return dict(match=match, plan=0, attend=attend, merge=merge, append=append, kv=kv,
                full_kv=full_kv,
                hits=hits, group_miss=int((match_p.reshape(B, Hkv, G) < 0).any(axis=2).sum()))


def cpu_baseline(cfg, K, V, qt, q, budget_s, mode=0):
    """The CPU oracle, as is, on a bounded sample of the same workload: at
    most one (request, head) stream per thread, spread over the requests and
    heads, for as many decode steps as the time budget allows."""
    from oracle import oracle as orc

    orc.build()
    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = nproc
    threads = max(1, min(16, avail))
    t2 = orc.threshold2(cfg.head_dim, cfg.tau, mode=mode)
    W = cfg.n_warm
    all_heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_q_heads)]
    stride = max(1, len(all_heads) // threads)
    heads = all_heads[::stride][:threads]

    def run(n_steps):
        res = orc.run_streams(K, V, qt, q, heads, ctx_len=cfg.ctx, n_warm=W,
                              ring_k=cfg.ring_k, band_r=cfg.band_r, thresh2=t2,
                              n_steps=n_steps, threads=threads)
        return sum(r["warm_seconds"] for r in res.values())

    # Calibrate on a few steps, then size the sample to the budget.
    probe = min(4, cfg.steps)
    t0 = time.perf_counter()
    warm = run(probe)
    per_step = max(1e-6, (time.perf_counter() - t0 - warm / threads) / probe)
    n_steps = int(min(cfg.steps, max(probe, budget_s / per_step)))
    t0 = time.perf_counter()
    warm = run(n_steps)
    wall = time.perf_counter() - t0
    # Warm-summary evaluation (lazy, off the per-step path) is excluded,
    # spread over the threads that ran it.
    step_time = max(1e-9, wall - warm / threads)
    value = len(heads) * n_steps / step_time
    return dict(value=value, unit="heads*layers/s", cores=threads, nproc=nproc,
                kind="oracle",
                sample="%d (request, head) streams x %d decode steps of %s, fp64 C "
                       "oracle, %d threads on %d host cores, lazy warm summaries "
                       "(%.1f CPU-s) excluded" % (len(heads), n_steps, cfg.name, threads,
                                                   avail, warm))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy}))
        return

    from attention_reuse_amd import mac

    mac.load()
    dev = "cuda:0"
    cfg = wl.WORKLOADS[args.config]
    NL = args.layers or default_layers(cfg)
    if args.warmup + args.steps > cfg.steps:
        sys.exit("warmup + steps exceeds the %d decode steps of the workload" % cfg.steps)
    B, H, Hkv, d, R, W = (cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                          cfg.ring_k, cfg.n_warm)
    if args.match_filter == "auto":
        args.match_filter = args.launch in ("two", "split") or (
            args.launch == "auto" and B * Hkv > 16)
    else:
        args.match_filter = args.match_filter == "on"
    t_gen = time.perf_counter()
    K, V = wl.gen_kv(cfg)
    qt, q, _, _ = wl.gen_queries(cfg)
    print("[bench] %s: inputs generated in %.1fs, %d layers" % (
        cfg.name, time.perf_counter() - t_gen, NL), file=sys.stderr, flush=True)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    K0, V0 = to_dev(K), to_dev(V)
    dec_qt = to_dev(np.moveaxis(qt[:, :, W:], 2, 0))   # [S, B, H, d]
    dec_q = to_dev(np.moveaxis(q[:, :, W:], 2, 0))
    pos_np = wl.decode_positions(cfg)
    pos = to_dev(pos_np)
    paging = {}
    if args.page_size:
        # Pages of [Hkv, P, d], each request's pages scattered over the pool
        # by a seeded shuffle.
        P = args.page_size
        npg = -(-cfg.capacity // P)
        g = torch.Generator().manual_seed(0)
        table = torch.randperm(B * npg, generator=g).reshape(B, npg).to(torch.int32).to(dev)

        def to_pool(X):
            pad = npg * P - cfg.capacity
            Xp = torch.nn.functional.pad(X, (0, 0, 0, pad)) if pad else X
            Xp = Xp.reshape(B, Hkv, npg, P, d).permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, P, d)
            # (with one request the reshape is a strided view: the pool must be dense)
            pool = torch.empty(Xp.shape, dtype=Xp.dtype, device=Xp.device)
            pool[table.reshape(-1).long()] = Xp
            return pool

        K0, V0 = to_pool(K0), to_pool(V0)
        torch.cuda.synchronize()
        paging = dict(page_size=P, max_pages=npg, page_table=table,
                      strides=(Hkv * P * d, P * d, d))
    p = mac.make_params(B, H, Hkv, d, mac.MAC_DTYPE_F32 if cfg.dtype == "f32" else mac.MAC_DTYPE_BF16,
                        R, cfg.band_r, cfg.capacity, cfg.tau, thresh_mode=thresh_mode(args),
                        **paging,
                        flags=(mac.MAC_FLAG_FUSED_APPEND if args.append == "fused" else 0)
                        | (mac.MAC_FLAG_MATCH_FILTER if args.match_filter else 0)
                        | {"auto": 0, "single": mac.MAC_FLAG_SINGLE_LAUNCH,
                           "two": mac.MAC_FLAG_TWO_STAGES,
                           "split": mac.MAC_FLAG_SPLIT_STAGES}[args.launch])
    wsb = mac.mac_workspace_bytes(p)
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    aux = torch.cuda.Stream()

    layers = []
    if args.alloc == "pool":
        # One allocation per kind for all layers; layer li uses slice li.
        wsb_al = -(-wsb // 256) * 256
        pools = dict(K=torch.empty((NL,) + tuple(K0.shape), dtype=K0.dtype, device=dev),
                     V=torch.empty((NL,) + tuple(V0.shape), dtype=V0.dtype, device=dev),
                     q_ring=torch.zeros((NL, B, H, R, d), dtype=K0.dtype, device=dev),
                     o_ring=torch.zeros((NL, B, H, R, d), device=dev),
                     lse_ring=torch.zeros((NL, B, H, R), device=dev),
                     pos_ring=torch.zeros((NL, B, cfg.n_kv_heads, R), dtype=torch.int32,
                                          device=dev),
                     ws=torch.empty((NL, wsb_al), dtype=torch.uint8, device=dev),
                     out=torch.empty((NL, B, H, d), device=dev))
        pools["K"][:] = K0
        pools["V"][:] = V0
        del K0, V0
        for li in range(NL):
            layers.append({k: v[li] for k, v in pools.items()})
        K0, V0 = layers[0]["K"], layers[0]["V"]
    else:
        for li in range(NL):
            L = dict(K=K0 if li == 0 else K0.clone(), V=V0 if li == 0 else V0.clone(),
                     q_ring=torch.zeros((B, H, R, d), dtype=K0.dtype, device=dev),
                     o_ring=torch.zeros((B, H, R, d), device=dev),
                     lse_ring=torch.zeros((B, H, R), device=dev),
                     pos_ring=torch.zeros((B, cfg.n_kv_heads, R), dtype=torch.int32, device=dev),
                     ws=torch.empty(wsb, dtype=torch.uint8, device=dev),
                     out=torch.empty((B, H, d), device=dev))
            layers.append(L)
    # Warm the rings of layer 0 from the prompt tail; the other layers copy them.
    L0 = layers[0]
    h0 = mac.mac_init_rings(p, L0["q_ring"], L0["o_ring"], L0["lse_ring"], L0["pos_ring"],
                            L0["ws"], wsb, to_dev(qt[:, :, :W]), to_dev(q[:, :, :W]), W,
                            [cfg.ctx] * B, L0["K"], L0["V"], st)
    torch.cuda.synchronize()
    warm_state = [L0[k].clone() for k in ("q_ring", "o_ring", "lse_ring", "pos_ring")]
    mac.mac_release(h0)

    def reset_rings():
        for L in layers:
            if L.get("h"):
                mac.mac_release(L["h"])
            L["h"] = mac.mac_init_rings(p, L["q_ring"], L["o_ring"], L["lse_ring"],
                                        L["pos_ring"], L["ws"], wsb, None, None, 0,
                                        [cfg.ctx] * B, L["K"], L["V"], st)
            for k, src in zip(("q_ring", "o_ring", "lse_ring", "pos_ring"), warm_state):
                L[k].copy_(src)
        torch.cuda.synchronize()

    match_rec = torch.full((cfg.steps, NL, B, H), -1, dtype=torch.int32, device=dev)

    def step_on(s, sid, record=True):
        for li, L in enumerate(layers):
            if args.mode == "mac":
                mac.mac_decode_step(L["h"], dec_qt[s], dec_q[s], L["K"], L["V"], pos[s],
                                    L["out"], None, match_rec[s, li] if record else None,
                                    None, sid, aux.cuda_stream)
            else:
                mac.mac_full_decode(p, dec_q[s], L["K"], L["V"], pos[s], L["out"], None,
                                    L["ws"], wsb, sid)

    def step(s, record=True):
        step_on(s, st, record)

    reset_rings()
    graphs = None
    if args.graph:
        # One graph per timed step, captured before anything runs (capture
        # does not execute), replayed in order after the eager warm-up.
        if args.append != "fused" and args.mode == "mac":
            sys.exit("--graph needs --append fused")
        graphs = []
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            for s in range(args.warmup, args.warmup + args.steps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    step_on(s, cap.cuda_stream)
                graphs.append(g)
        torch.cuda.synchronize()
    for s in range(args.warmup):
        step(s)
    for L in layers:
        mac.mac_join_aux(L["h"], st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i, s in enumerate(range(args.warmup, args.warmup + args.steps)):
        if graphs:
            graphs[i].replay()
        else:
            step(s)
    for L in layers:
        mac.mac_join_aux(L["h"], st)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    print("[bench] timed %d steps: %.3f ms/step" % (args.steps, ms_per_step),
          file=sys.stderr, flush=True)

    # Algorithmic bytes of the timed steps (from the recorded decisions).
    mrec = match_rec.cpu().numpy()
    per = {k: 0.0 for k in ("match", "plan", "attend", "merge", "append", "kv", "full_kv",
                            "hits", "group_miss")}
    timed = range(args.warmup, args.warmup + args.steps)
    for s in timed:
        halves = (filter_second_halves(cfg, qt, s)
                  if args.mode == "mac" and args.match_filter else None)
        for li in range(NL):
            mp = mrec[s, li] if args.mode == "mac" else np.full((B, H), -1, np.int32)
            ab = algorithmic_bytes(cfg, mp, pos_np[s].astype(np.int64), halves)
            for k in per:
                per[k] += ab[k]
    n_ls = args.steps * NL
    per_launch = {k: v / n_ls for k, v in per.items()}

    # Per-kernel durations: HIP events recorded by the library around each
    # kernel, on the stream it runs on, in a second pass over the same steps
    # from the same ring state.  (Recorded inside the timed pass, the events
    # would add about 2 us of gap per record to the timed step: 20% at the
    # default workload.)
    stage_ms = None
    if not args.no_profile and args.mode == "mac":
        reset_rings()
        for s in range(args.warmup):
            step(s, record=False)
        for L in layers:
            mac.mac_join_aux(L["h"], st)
            mac.mac_profile_start(L["h"], args.steps)
        for s in timed:
            step(s, record=False)
        tot = {k: 0.0 for k in STAGES}
        cnt = 0
        for L in layers:
            mac.mac_join_aux(L["h"], st)
            ms, n = mac.mac_profile_read(L["h"])
            cnt += n
            for k in STAGES:
                tot[k] += ms[k]
        stage_ms = {k: tot[k] / max(cnt, 1) for k in STAGES}

    roofline = None
    launched = None
    if stage_ms:
        launched = ("split" if stage_ms["step"] == 0 else
                    "two" if stage_ms["match"] > 0 else "single")
    if stage_ms and launched in ("single", "two"):
        # One kernel moves the attention and merge bytes (and the ring append
        # when fused), and the match bytes unless the match kernel ran first.
        dom = "step"
        per_launch["step"] = sum(per_launch[k] for k in ("attend", "merge")) + (
            per_launch["match"] if launched == "single" else 0.0) + (
            per_launch["append"] if args.append == "fused" else 0.0)
    elif stage_ms:
        dom = max(("match", "attend"), key=lambda k: stage_ms[k])
    if stage_ms:
        ach = per_launch[dom] / (stage_ms[dom] * 1e-3) / 1e9
        roofline = dict(bound="hbm", kernel=KERNEL_NAMES[dom], achieved=round(ach, 1),
                        peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4),
                        traffic=read_traffic(cfg.name, KERNEL_NAMES[dom]),
                        alg_bytes_per_launch=int(per_launch[dom]),
                        avg_launch_us=round(stage_ms[dom] * 1e3, 2))
    elif args.mode == "full":
        ach = per_launch["attend"] / (ms_per_step / NL * 1e-3) / 1e9
        roofline = dict(bound="hbm", kernel="full decode step", achieved=round(ach, 1),
                        peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4),
                        traffic=None)

    # Same run: exact full decode of the same layers and positions (the
    # baseline MAC is measured against), and the achievable streaming-read
    # bandwidth of the device (a read-only kernel over a buffer far larger
    # than the Infinity Cache).
    full_ms = None
    if args.mode == "mac" and not args.no_full:
        fws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        nf = min(args.steps, 8)
        for s in range(args.warmup, args.warmup + 2):
            for L in layers:
                mac.mac_full_decode(p, dec_q[s], L["K"], L["V"], pos[s], L["out"], None,
                                    fws, wsb, st)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for s in range(args.warmup, args.warmup + nf):
            for L in layers:
                mac.mac_full_decode(p, dec_q[s], L["K"], L["V"], pos[s], L["out"], None,
                                    fws, wsb, st)
        f1.record(stream)
        torch.cuda.synchronize()
        full_ms = f0.elapsed_time(f1) / nf
        del fws
    read_gbs = None
    if not args.no_full:
        nbytes = 4 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        grid = 8 * torch.cuda.get_device_properties(0).multi_processor_count
        sink = torch.empty(grid, device=dev)
        times = []
        for it in range(6):
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            r0.record(stream)
            mac.mac_stream_read(buf, nbytes, sink, grid, st)
            r1.record(stream)
            torch.cuda.synchronize()
            if it:
                times.append(r0.elapsed_time(r1))
        read_gbs = nbytes / (sorted(times)[len(times) // 2] * 1e-3) / 1e9
        del buf

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(cfg, K, V, qt, q, args.cpu_seconds, mode=thresh_mode(args))

    alg_step = sum(per[k] for k in ("match", "attend", "merge", "append")) / args.steps
    value = B * H * NL / (ms_per_step * 1e-3)
    line = {
        "metric": "decode attention steps/sec (heads*layers) + KV GB read/step + % HBM roofline",
        "value": round(value, 1),
        "unit": "heads*layers/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # K/V, queries and the logits' MFMA operands in the workload's type;
        # accumulation, softmax and summaries in fp32.
        "dtype": cfg.dtype,
        "accum_dtype": "f32",
        "data": "synthetic (seeded N(0,1) K/V, prototype+noise query stream)",
        "config": {"workload": cfg.name, "mode": args.mode,
                   "launch": launched or args.launch,
                   "append": args.append,
                   "match_filter": bool(args.match_filter),
                   "page_size": args.page_size,
                   "layers": NL, "kv_dtype": cfg.dtype,
                   "batch": B, "q_heads": H, "kv_heads": Hkv, "head_dim": d,
                   "context": cfg.ctx, "ring_k": R, "band_r": cfg.band_r, "tau": cfg.tau,
                   "threshold": ("tau*sqrt(2d)" if args.thresh == "tau"
                                 else "(1-tau)*sqrt(2d)"),
                   "parallelism": "1 GPU"},
        "kv_gb_per_step": round(per["kv"] / args.steps / 1e9, 4),
        "full_kv_gb_per_step": round(per["full_kv"] / args.steps / 1e9, 4),
        "alg_gb_per_step": round(alg_step / 1e9, 4),
        "step_hbm_frac": round(alg_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "hit_rate": round(per["hits"] / (n_ls * B * H), 4),
        "group_miss_rate": round(per["group_miss"] / (n_ls * B * Hkv), 4),
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()} if stage_ms else None,
        "timing": ("graph replay" if graphs else "eager launches") + (
            "; per-kernel HIP events from a second eager pass of the same steps"
            if stage_ms else ""),
        "full_decode_ms_per_step": round(full_ms, 4) if full_ms else None,
        "speedup_vs_full_decode": round(full_ms / ms_per_step, 3) if full_ms else None,
        "achievable_read_gbs": round(read_gbs, 1) if read_gbs else None,
        "step_frac_of_achievable": (round(alg_step / (ms_per_step * 1e-3) / 1e9 / read_gbs, 4)
                                    if read_gbs else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")
    for L in layers:
        mac.mac_release(L["h"])


if __name__ == "__main__":
    main()
