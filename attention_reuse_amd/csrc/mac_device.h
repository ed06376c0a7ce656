// Device code of the MAC-Attention decode step for gfx950 (MI355X), shared
// by the launcher sources (mac_kernels.hip, mac_step_*.hip): every kernel
// and device function sits in an anonymous namespace, so each source that
// launches a kernel compiles its own instances.
//
// The step of the MAC-Attention blog ("MAC-Attention: Match-Amend-Complete
// attention reuse ... (MLSys 2026)", section "Paper version: the K1/K2/K3
// micro-pipeline") has four stages:
//
//   match  -- L2 nearest neighbour of the pre-RoPE query among the last K
//       ring entries ("Match (1)-(3)"), one 64-slot split per unit of work,
//       folded into a per-head (distance, position) key by an atomic min.
//   plan + attend -- every workgroup plans from the match keys (final
//       decision per head, threshold, token range [s_g, m] per (request, KV
//       group); every range is cut into items on an absolute 64-token grid
//       (coarser for long ranges) plus the rectify split m-r+1: the
//       span-proportional allocator of "K2"), takes an equal contiguous share
//       of the items' work and streams its split-KV attention.  A K/V
//       row is loaded once (16 B per lane, one 16-lane DPP row per row) and
//       serves the G query heads of the group from registers; each item
//       leaves one partial (o, lse) per head.
//   merge  -- per KV group, the partials are folded in a fixed order with the
//       cached summary ("Complete"), giving the output and the rectified
//       summary of [0, m-r]; with append_fused the ring slot m mod K is
//       written here too.
//   append -- otherwise the rectify-append ("K3") runs as its own kernel on
//       an auxiliary stream.
//
// The stages run either as one launch (step_kernel) or as one kernel each.
// The separate kernels hand over at kernel boundaries.  The single launch
// gives each KV group its own run of workgroups, all resident at once:
// match -> plan is a hand-off of tagged match keys that every workgroup of
// the group polls (the wait is bounded), and attention -> merge a hand-off to
// the workgroup that completes the group's last item.  The eight XCDs of MI355X
// have private L2 caches that are not coherent with each other, and a
// device-scope release fence writes a whole L2 back, which costs tens of
// microseconds under load.  Data that crosses workgroups inside the launch
// therefore travels with device-coherent loads and stores (agent-scope
// atomic accesses, issued with the sc1 bit, which bypass the L2); a
// producer waits for its stores to complete before it signals with an
// atomic counter, and a consumer reads only after the counter says so.
// Both forms run the same device functions in the same order, so their
// results are bitwise identical.
//
// The path is HBM-bound (about 4 flop per KV byte for G = 4).  The match,
// the softmax and P*V run on VALU; for bf16 K with d = 128 and G = 4 the
// logits come from MFMAs (the queries' bf16 high and low parts as 8 of the
// 16 columns), which removes most of the VALU work per token.
#pragma once

#include <math.h>

#include <mutex>
#include <utility>

#include "mac_attention.h"
#include "mac_internal.h"

namespace mac {
namespace {

// Opt-in timeline of the step kernel, in a separate build of the library
// (MAC_TIMELINE defined; the default build compiles the marks to nothing).
// Thread 0 of workgroup w writes the 100 MHz real-time counter (a mark) or
// a count (a note) to word w * kTimelineSlots + slot of its source file's
// array; a launch overwrites the words its workgroups reach.  Slot meanings
// are listed with mac_timeline_read in the public header.
constexpr int kTimelineSlots = 32, kTimelineWgs = 4096;
enum TimelineSlot : int {
    kTlEntry = 0,         // workgroup start
    kTlKeys = 1,          // match keys stored (one launch) / queries staged (group kernel)
    kTlSpec = 2,          // speculative K/V requested
    kTlPlanned = 3,       // group planned (head decisions in LDS)
    kTlPublished = 4,     // items counted, pool entries published
    kTlItem = 5,          // first own item begins (rows requested)
    kTlItemComputed = 6,  // first own item's blocks computed
    kTlItemStored = 7,    // its partial stored (write-through complete)
    kTlItemCounted = 8,   // its count on the group counter done
    kTlOwnDone = 9,       // all own items done
    kTlMergeEnd = 10,     // merge of the own group done (its merger only)
    kTlExit = 11,         // end of a workgroup that ran items
    kTlExitIdle = 12,     // end of a workgroup without own items
    kTlPoolFirst = 13,    // first pool item claimed
    kTlMergeBegin = 20,   // merge of a group begins (its merger)
    kTlMergeWeights = 21, // item weights formed (few items) / list A folded
    kTlMergeSummed = 22,  // both lists' partials summed
    kTlMergeWritten = 23, // outputs and ring entries written (stores issued)
    kTlOwnQueries = 24,   // own-items block: queries read from LDS
    kTlOwnBounds = 25,    // first item's bounds computed
    kTlOwnRows = 26,      // its rows requested (or found speculated)
    kTlBlocksDone = 27,   // an item's blocks done, before the cross-row combine (latest item)
    kTlCombineRows = 28,  // the workgroup's rows of that item in LDS (latest item)
    kTlCombineSums = 29,  // that item's per-head weights and sums formed (latest item)
    kTlNoteItems = 16,    // note: the group's item count
    kTlNoteOwn = 17,      // note: items its own workgroups run
    kTlNoteSpec = 18,     // note: first item from the speculative rows (1), re-requested (2), none (0)
    kTlNotePool = 19,     // note: pool items this workgroup ran
};
#ifdef MAC_TIMELINE
__device__ unsigned long long timeline_words[kTimelineWgs * kTimelineSlots];
#define MAC_NOTE(slot, v)                                                                  \
    do {                                                                                   \
        if (threadIdx.x == 0 && blockIdx.x < kTimelineWgs)                                 \
            timeline_words[blockIdx.x * kTimelineSlots + (slot)] = (unsigned long long)(v); \
    } while (0)
#define MAC_MARK(slot) MAC_NOTE(slot, __builtin_amdgcn_s_memrealtime())
#else
#define MAC_NOTE(slot, v) ((void)0)
#define MAC_MARK(slot) ((void)0)
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

struct F32 {
    using S = float;
    static constexpr int EPL = 4;  // elements per 16-byte lane load
};
struct BF16 {
    using S = uint16_t;
    static constexpr int EPL = 8;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ inline uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// x * scale rounded to bf16 (hi) and the remainder rounded to bf16 (lo).
// No contraction: every caller rounds the product and the difference alike.
__device__ inline void split_bf16(float x, float scale, uint32_t &hi, uint32_t &lo)
{
#pragma clang fp contract(off)
    const float xs = x * scale;
    hi = bf16_bits(xs);
    lo = bf16_bits(xs - __uint_as_float(hi << 16));
}

template <class T>
__device__ inline void unpack(const uint4 &v, float *f);

template <>
__device__ inline void unpack<F32>(const uint4 &v, float *f)
{
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
}

template <>
__device__ inline void unpack<BF16>(const uint4 &v, float *f)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ inline uint4 load16(const void *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}
// The same with the non-temporal hint (nt): the line is not kept in the
// caches for reuse.
__device__ inline uint4 load16_nt(const void *p)
{
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v x = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}
template <bool kNt>
__device__ inline uint4 load16_kv(const void *p)
{
    if constexpr (kNt)
        return load16_nt(p);
    else
        return load16(p);
}

// v_exp_f32 / v_log_f32 (base 2) without library range wrappers; the
// arguments here are <= 0 (exp) or >= 1 (log).
__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float lg2(float x) { return __builtin_amdgcn_logf(x); }

// DPP lane permutations inside a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7-i within 8 lanes
constexpr int kDppRowMirror = 0x140;   // lane i <- 15-i within 16 lanes

template <int CTRL>
__device__ inline float dpp(float v)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over W consecutive lanes (W = 8, 16 or 32); every lane of the group
// receives the same bits (each step adds a symmetric pair).
template <int W>
__device__ inline float row_sum(float v)
{
    static_assert(W == 4 || W == 8 || W == 16 || W == 32, "row width");
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    if (W >= 8)
        v += dpp<kDppHalfMirror>(v);
    if (W >= 16)
        v += dpp<kDppRowMirror>(v);
    if (W == 32)
        v += __shfl_xor(v, 16, 64);
    return v;
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [0, N).
template <class F, int... Is>
__device__ inline void static_for_impl(F &&f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ inline void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kDppRowRor = 0x120;       // + n: lane i <- lane (i - n) mod 16
constexpr int kDppRowShr = 0x110;       // + n: lane i <- lane i - n (0 below n)
constexpr int kDppRowNewBcast = 0x150;  // + n: every lane <- lane n of its row

// Reduce-scatter of 16 values over the 16 lanes of a row: lane L returns
// the row sum of v[L].  Four exchange steps halve the values a lane holds
// (partners: lane ^ 8, the mirror within 8 lanes, lane ^ 2, lane ^ 1).
__device__ inline float row_reduce_scatter16(const float (&v)[16], int lane)
{
    const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
    float a[8], c[4], d[2];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float keep = b3 ? v[8 + m] : v[m];
        const float send = b3 ? v[m] : v[8 + m];
        a[m] = keep + dpp<kDppRowRor + 8>(send);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float keep = b2 ? a[4 + m] : a[m];
        const float send = b2 ? a[m] : a[4 + m];
        c[m] = keep + dpp<kDppHalfMirror>(send);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const float keep = b1 ? c[2 + m] : c[m];
        const float send = b1 ? c[m] : c[2 + m];
        d[m] = keep + dpp<kDppQuadXor2>(send);
    }
    const float keep = b0 ? d[1] : d[0];
    const float send = b0 ? d[0] : d[1];
    return keep + dpp<kDppQuadXor1>(send);
}

// All-reduce (max or sum) over the lanes of a 16-lane row that are equal
// modulo G, by rotations of G, 2G, ... 8 lanes.
template <int G, bool kMax>
__device__ inline float row_mod_reduce(float x)
{
    static_for<4>([&](auto S) {
        constexpr int sh = 1 << S;
        if constexpr (sh >= G) {
            const float y = dpp<kDppRowRor + sh>(x);
            x = kMax ? fmaxf(x, y) : x + y;
        }
    });
    return x;
}

__device__ inline unsigned long long shfl_xor_u64(unsigned long long v, int off)
{
    int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    lo = __shfl_xor(lo, off, 64);
    hi = __shfl_xor(hi, off, 64);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ inline unsigned long long umin64(unsigned long long a, unsigned long long b)
{
    return a < b ? a : b;
}

// (l, o[N]) <- (l, o) (+) (lb, ob) for log2-domain summaries of disjoint
// token sets; the empty summary (l = -inf) is an exact identity.
template <int N>
__device__ inline void merge_into(float &l, float *o, float lb, const float *ob)
{
    if (lb == -INFINITY)
        return;
    if (l == -INFINITY) {
        l = lb;
#pragma unroll
        for (int i = 0; i < N; ++i)
            o[i] = ob[i];
        return;
    }
    const float M = fmaxf(l, lb);
    const float ln = M + lg2(ex2(l - M) + ex2(lb - M));
    const float wa = ex2(l - ln), wb = ex2(lb - ln);
    // One explicit contraction, so every inlining of the merge rounds alike
    // (the kernel forms must agree bit for bit).
#pragma unroll
    for (int i = 0; i < N; ++i)
        o[i] = fmaf(wa, o[i], wb * ob[i]);
    l = ln;
}

__device__ inline int32_t end_of(const StepArgs &a, int b)
{
    return a.pos[b] + (a.mode == kPlanInit ? a.end_offset : 0);
}

__device__ inline bool end_ok(const StepArgs &a, int e)
{
    return e < a.s.T && (a.mode == kPlanInit || e >= 0);
}

// Load of a word that is the same for the whole workgroup and was written
// before the launch began, as a scalar load: such loads are issued back to
// back and waited for together, where plain loads of memory that the kernel
// also writes become vector loads, each waited for before the branch that
// uses it.  The scalar cache is invalidated at launch, so the value is the
// one of the launch's start or a later one.
template <class V>
__device__ inline V ld_uniform(const V *p)
{
    return *(const __attribute__((address_space(4))) V *)p;
}

// Whether KV group grp (of request b) may reuse its rings: always when the
// caller binds no epochs, else when the request's epoch is non-negative and
// equals the one the group's rings were built for.  A group that is not
// ready matches nothing, so every head of it is exact attention; its merge
// adopts the request's epoch, and its append restarts the position ring
// (see ring_append_pos).
__device__ inline bool group_ready(const StepArgs &a, int b, int grp)
{
    if (!a.epoch)
        return true;
    // Both words requested together (the second does not wait for the first).
    const int32_t ep = ld_uniform(a.epoch + b);
    const int32_t built = ld_uniform(a.w.ring_epoch + grp);
    return ep >= 0 && built == ep;
}

// Position-ring update of the rectify-append of KV group grp at position e,
// run by n threads (thread index i): slot e mod K receives e; on a restart
// every other slot is emptied.
__device__ inline void ring_append_pos(const StepArgs &a, int grp, int e, bool restart, int i,
                                       int n)
{
    int32_t *row = a.pos_ring + (int64_t)grp * a.s.K;
    const int slot = e % a.s.K;
    if (!restart) {
        if (i == 0)
            row[slot] = e;
        return;
    }
    for (int k = i; k < a.s.K; k += n)
        row[k] = k == slot ? e : -1;
}

// Device-coherent accesses for data handed between workgroups of one
// launch: relaxed agent-scope atomics, which gfx950 issues with the sc1
// bit (write-through on stores, L2 bypass on loads).
__device__ inline void st_wt(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_wt(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_wt(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_wt(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t ld_wt_u32(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned long long ld_wt(const unsigned long long *p)
{
    return __hip_atomic_load(const_cast<unsigned long long *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-wide AND / OR of a predicate over the kBlock threads: a wave
// vote, then the kBlock / 64 votes through LDS.  The library's
// __syncthreads_and/_or obtain the workgroup size from the dispatch packet,
// which lives in host memory: one uncached read per workgroup, serialised
// across the grid (measured: microseconds per launch).
__device__ inline bool block_and(bool p)
{
    __shared__ int votes[kBlock / 64];
    const bool w = __all(p);
    __syncthreads();  // the previous call's readers are done
    if ((threadIdx.x & 63) == 0)
        votes[threadIdx.x >> 6] = w;
    __syncthreads();
    bool r = true;
#pragma unroll
    for (int i = 0; i < kBlock / 64; ++i)
        r = r && votes[i] != 0;
    return r;
}
__device__ inline bool block_or(bool p) { return !block_and(!p); }

// Cache-policy operand of the buffer-load builtins selecting sc1 (device
// coherence, as the agent-scope atomic accesses above use).
constexpr int kCacheSc1 = 16;
// ... and the non-temporal hint (nt): lines not kept for reuse.
constexpr int kCacheNt = 2;

// s_waitcnt vmcnt(0): this wave's loads and stores have completed (a
// write-through store is then visible to every XCD).  Encoding (gfx9):
// vmcnt bits [3:0] and [15:14] = 0, expcnt [6:4] = 7, lgkmcnt [11:8] = 15.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The per-head match keys of a launch of epoch E (see StepArgs::key_parity).
__device__ inline unsigned long long *key_set(const StepArgs &a, unsigned long long E)
{
    return a.w.keys + (a.key_parity ? (int64_t)(E & 1) * a.s.B * a.s.Hq * kKeyStride : 0);
}

// Decision of one head from its match key: hit iff a candidate exists, the
// position is valid and D < threshold ("Match (2)"); a hit attends from
// max(0, p - r + 1) and reuses the summary in slot p mod K.
struct Decision {
    int start, slot, p;
    float d2;
    bool hit;
};

__device__ inline Decision decide(const StepArgs &a, unsigned long long key, bool ok)
{
    Decision d;
    const bool any = key != ~0ull;
    d.d2 = any ? __uint_as_float((uint32_t)(key >> 32)) : INFINITY;
    d.p = any ? (int)(0xffffffffu - (uint32_t)key) : -1;
    d.hit = ok && any && d.d2 < a.s.thresh2;
    d.start = d.hit ? (d.p - a.s.r + 1 > 0 ? d.p - a.s.r + 1 : 0) : 0;
    d.slot = d.hit ? d.p % a.s.K : -1;
    return d;
}

// Per-head code kept by the planner: p - r + 1 for a hit (may be negative),
// kMissCode otherwise.  The head attends from max(0, code); a hit reuses
// slot (code + r - 1) mod K = p mod K.
constexpr int32_t kMissCode = INT32_MIN;
__device__ inline int code_start(int32_t c) { return c > 0 ? c : 0; }
__device__ inline int code_slot(int32_t c, int r, int K)
{
    return c == kMissCode ? -1 : (c + r - 1) % K;
}

// ---------------------------------------------------------------------------
// Planner, run redundantly by every attention workgroup from the match keys
// (a few KiB, L2-resident): decision per (b, h), token range [s_g, e] and
// item count per (b, g), and exclusive scans of the counts and of the
// groups' work (tokens plus kItemCost per item), all in LDS.  Workgroup 0
// also publishes what the merge kernel and the caller need.
// LDS: ints [BH + 5*NG + 2 + 2*nt/64].
struct PlanTables {
    const int32_t *code, *gstart, *gend, *gcount, *gbegin, *gwork;
    int total, work;
};

__device__ PlanTables plan_tables(const StepArgs &a, int32_t *lds, bool publish)
{
    const Shape &s = a.s;
    const int tid = threadIdx.x, nt = kBlock;
    const int lane = tid & 63, wave = tid >> 6;
    const int BH = s.B * s.Hq, NG = s.B * s.Hkv;
    const int r_split = (a.mode == kPlanInit) ? 0 : s.r;
    int32_t *s_code = lds;
    int32_t *s_gstart = s_code + BH;
    int32_t *s_gend = s_gstart + NG;
    int32_t *s_gcount = s_gend + NG;
    int32_t *s_gbegin = s_gcount + NG;  // NG + 1
    int32_t *s_gwork = s_gbegin + NG + 1;  // NG + 1
    int32_t *s_wave = s_gwork + NG + 1;  // two per wave

    // Decisions per (b, h).
    int bad = 0;
    for (int bh = tid; bh < BH; bh += nt) {
        const int b = bh / s.Hq;
        const int e = end_of(a, b);
        const bool ok = end_ok(a, e);
        bad |= !ok;
        int32_t code = kMissCode, slot = -1;
        if (a.mode == kPlanMatch) {
            const Decision dc = decide(a, a.w.keys[bh * kKeyStride], ok);
            code = dc.hit ? dc.p - s.r + 1 : kMissCode;
            slot = dc.slot;
            if (publish && a.match_p)
                a.match_p[bh] = dc.hit ? dc.p : -1;
            if (publish && a.match_d2)
                a.match_d2[bh] = dc.d2;
        }
        s_code[bh] = code;
        if (publish)
            a.w.dec_slot[bh] = slot;
    }
    bad = block_or(bad);

    // Token range and item count per (b, g): a contiguous run of groups per
    // thread, so the scan below needs one pass over the runs.
    const int per = (NG + nt - 1) / nt;
    const int lo = tid * per, hi = lo + per < NG ? lo + per : NG;
    int run = 0, runw = 0;
    for (int grp = lo; grp < hi; ++grp) {
        const int b = grp / s.Hkv, g = grp - b * s.Hkv;
        const int e = end_of(a, b);
        int st = 0, cnt = 0, wk = 0;
        if (e >= 0 && e < s.T) {
            st = e;
            for (int j = 0; j < s.G; ++j) {
                const int v = code_start(s_code[b * s.Hq + g * s.G + j]);
                st = v < st ? v : st;
            }
            const GroupItems gi(st, e, r_split, s.F, a.mode != kPlanInit, s.cmin);
            cnt = gi.n;
            wk = gi.work();
        }
        s_gstart[grp] = st;
        s_gend[grp] = e;
        s_gcount[grp] = cnt;
        s_gwork[grp] = wk;  // the group's own work until the scan below
        run += cnt;
        runw += wk;
    }
    // Exclusive scans of the counts and the work: inclusive scans of the run
    // totals within each wave, then across the waves.
    int x = run, xw = runw;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64), yw = __shfl_up(xw, o, 64);
        if (lane >= o) {
            x += y;
            xw += yw;
        }
    }
    if (lane == 63) {
        s_wave[wave] = x;
        s_wave[(nt >> 6) + wave] = xw;
    }
    __syncthreads();
    int before = 0, total = 0, beforew = 0, totalw = 0;
    for (int w = 0; w < (nt >> 6); ++w) {
        const int v = s_wave[w], vw = s_wave[(nt >> 6) + w];
        before += w < wave ? v : 0;
        total += v;
        beforew += w < wave ? vw : 0;
        totalw += vw;
    }
    int acc = before + x - run, accw = beforew + xw - runw;
    for (int grp = lo; grp < hi; ++grp) {
        s_gbegin[grp] = acc;
        acc += s_gcount[grp];
        const int wk = s_gwork[grp];
        s_gwork[grp] = accw;
        accw += wk;
    }
    if (tid == 0) {
        s_gbegin[NG] = total;
        s_gwork[NG] = totalw;
    }
    __syncthreads();
    if (total > a.max_items)
        total = (int)a.max_items;

    if (publish) {
        for (int grp = tid; grp < NG; grp += nt) {
            a.w.grp_begin[grp] = s_gbegin[grp];
            a.w.grp_count[grp] = s_gcount[grp];
            a.w.grp_start[grp] = s_gstart[grp];
            if (s_gcount[grp] == 0) {
                a.w.app_pos[grp] = -1;  // nothing to append
                // No item, so no merge will run: the outputs are written here.
                const int b = grp / s.Hkv, g = grp - b * s.Hkv;
                const bool bad = !end_ok(a, s_gend[grp]);
                for (int j = 0; j < s.G; ++j) {
                    const int bh = b * s.Hq + g * s.G + j;
                    for (int d = 0; d < s.D; ++d) {
                        if (a.out)
                            a.out[(int64_t)bh * s.D + d] = bad ? NAN : 0.f;
                        a.w.rect_o[(int64_t)bh * s.D + d] = 0.f;
                    }
                    if (a.out_lse)
                        a.out_lse[bh] = bad ? NAN : -INFINITY;
                    a.w.rect_l[bh] = -INFINITY;
                }
            }
        }
        if (tid == 0) {
            a.w.ctrl[kCtrlItems] = total;
            a.w.ctrl[kCtrlStatus] = bad ? MAC_DEV_BAD_POSITION : 0;
        }
    }
    PlanTables t;
    t.code = s_code;
    t.gstart = s_gstart;
    t.gend = s_gend;
    t.gcount = s_gcount;
    t.gbegin = s_gbegin;
    t.gwork = s_gwork;
    t.total = total;
    t.work = totalw;
    return t;
}

// ---------------------------------------------------------------------------
// Match of one unit: U ring rows per lane of head bh, starting at slot
// `first`; each LPR-lane row of a wave computes the squared distance of one
// slot, and the workgroup keeps the smallest
//   key = float_bits(D) << 32 | (0xffffffff - p)
// (non-negative floats order like their bits; equal D prefers larger p).
// The loads are issued unconditionally: rows past the ring repeat its last
// slot, and rows past the unit belong to the head's next unit.  Either way
// they are slots of the same head, so the minimum is unchanged.  Splitting
// issue from finish lets the caller request other data before the rows are
// needed.
template <class T, int D, int U>
struct MatchLoads {
    uint4 q, raw[U];
    int p[U];
    // The head's query ring as a buffer: a load at offset `oob` (its size)
    // returns zeros without touching memory, so reads are skipped per lane
    // without a branch.
    __amdgpu_buffer_rsrc_t ring;
    uint32_t oob;
    int first;
};

// Ring slot of load u of this lane's row.
template <int U>
__device__ inline int match_slot(const StepArgs &a, int first, int u, int rpb, int row)
{
    const int k = first + u * rpb + row;
    return k < a.s.K ? k : a.s.K - 1;
}

template <class T, int D, int U>
__device__ inline void match_issue(const StepArgs &a, int first, int bh, MatchLoads<T, D, U> &ml)
{
    constexpr int EPL = T::EPL, LPR = D / EPL, RPB = kBlock / LPR;
    using S = typename T::S;
    const Shape &s = a.s;
    const int b = bh / s.Hq, h = bh - b * s.Hq;
    const int lane = threadIdx.x % LPR, row = threadIdx.x / LPR;
    ml.q = load16((const S *)a.qtilde + b * a.qt_sb + h * a.qt_sh + lane * EPL);
    ml.oob = (uint32_t)s.K * D * sizeof(S);
    ml.ring = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<S *>((const S *)a.q_ring + (int64_t)bh * s.K * D), (short)0, (int)ml.oob,
        0x00020000);
    ml.first = first;
    const int32_t *pr = a.pos_ring + ((int64_t)b * s.Hkv + h / s.G) * s.K;
    // With the match filter only the first half of each row is read here.
    const bool first_half = !a.match_filter || lane < LPR / 2;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = match_slot<U>(a, first, u, RPB, row);
        const uint32_t off = first_half ? (uint32_t)(k * D + lane * EPL) * sizeof(S) : ml.oob;
        ml.raw[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ml.ring, off, 0, 0));
        ml.p[u] = pr[k];
    }
}

// Lower bound of the filter: a row whose first-half squared distance is at
// least thresh2 * kFilterMargin has a full distance above the threshold
// whatever the fp32 rounding of either sum (both are sums of the same
// non-negative per-lane terms, so they differ by far less than the margin).
constexpr float kFilterMargin = 1.0f + 1.0f / 1024.0f;

// Key of the unit issued by match_issue at position m; valid in thread 0.
// A group that is not ready has no candidate.  sm holds kBlock/64 words of
// LDS.
template <class T, int D, int U>
__device__ inline unsigned long long match_finish(const StepArgs &a, int m, bool ready,
                                                  const MatchLoads<T, D, U> &ml,
                                                  unsigned long long *sm)
{
    constexpr int EPL = T::EPL, LPR = D / EPL, RPB = kBlock / LPR;
    const Shape &s = a.s;
    // Below the minimum context a request does not reuse: no candidate.
    const bool m_ok = ready && m >= 0 && m < s.T && m >= s.min_ctx;
    float qv[EPL];
    unpack<T>(ml.q, qv);
    // This lane's share of each row's squared distance.
    auto lane_d2 = [&](const uint4 &raw) {
        float rv[EPL];
        unpack<T>(raw, rv);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float df = qv[e] - rv[e];
            acc = fmaf(df, df, acc);
        }
        return acc;
    };
    float part[U];
    bool keep[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        part[u] = lane_d2(ml.raw[u]);
        keep[u] = true;
    }
    if (a.match_filter) {
        // Exact lower-bound filter: the second half of a row is read only
        // when its first half leaves the row able to hit.  The full sum of
        // a kept row is formed below exactly as without the filter.
        const int lane = threadIdx.x % LPR, row = threadIdx.x / LPR;
        const bool upper = lane >= LPR / 2;
        const float lb_max = s.thresh2 * kFilterMargin;
        uint4 raw2[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float lb = row_sum<LPR>(upper ? 0.f : part[u]);
            const int pu = ml.p[u];
            keep[u] = lb < lb_max && m_ok && pu >= 0 && pu >= m - s.K && pu <= m - 1;
            const int k = match_slot<U>(a, ml.first, u, RPB, row);
            const uint32_t off =
                upper && keep[u] ? (uint32_t)(k * D + lane * EPL) * sizeof(typename T::S) : ml.oob;
            raw2[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ml.ring, off, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (upper)
                part[u] = lane_d2(raw2[u]);
    }
    unsigned long long best = ~0ull;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float acc = row_sum<LPR>(part[u]);
        const int pu = ml.p[u];
        const bool valid = keep[u] && m_ok && pu >= 0 && pu >= m - s.K && pu <= m - 1;
        uint32_t bits = __float_as_uint(acc);
        if (acc != acc)
            bits = 0x7f800000u;  // NaN distance counts as +inf
        const unsigned long long key =
            ((unsigned long long)bits << 32) | (0xffffffffu - (uint32_t)pu);
        best = umin64(best, valid ? key : ~0ull);
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
        best = umin64(best, shfl_xor_u64(best, off));
    if ((threadIdx.x & 63) == 0)
        sm[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 1; i < kBlock / 64; ++i)
            best = umin64(best, sm[i]);
    }
    return best;
}

// Filtered match of one unit in half rows (match kernel, filter on).  A
// row's D dims are two halves of H = LPR / 2 lanes; a pass gives each H-lane
// group one row's half, so every lane of a load carries data (the row
// geometry of match_issue leaves half the lanes of the first pass idle) and
// the unit takes half the row load instructions; the time of this kernel
// follows its load instructions, each of which costs address processing for
// the whole wave whether or not a lane reads memory.  A workgroup takes
// kSlotsPerHalvesSplit slots (128: measured 10.1 us against 10.6 us with 64
// and 10.2 us with 256 at the 128K batch-8 workload).  The sums are those of the
// full-row scan bit for bit: row_sum<LPR> is row_sum<H> over each half
// followed by one addition of the two halves, so the first half's
// row_sum<H> is the filter's lower bound and first + second is the row's
// distance, with each lane's products over the same 8 (or 4) dims in the
// same order.  Key and validity as match_finish.  The scalar words (the
// position, readiness and the done counter, returned in *done) are read
// after the rows are requested.  The ring rows are loaded with the
// non-temporal hint: a ring this kernel serves (more than 16 KV groups)
// outgrows the caches before its next step reads it (measured: 0.3 us less
// match, and 0.45 us less in the group kernel that follows, per launch at
// the 128K batch-8 workload).
template <class T, int D>
__device__ inline unsigned long long match_halves(const StepArgs &a, int first, int bh,
                                                  unsigned long long *done, unsigned long long *sm)
{
    using S = typename T::S;
    constexpr int EPL = T::EPL, LPR = D / EPL, H = LPR / 2, RPH = kBlock / H;
    constexpr int UH = kSlotsPerHalvesSplit / RPH;
    static_assert(UH >= 1 && UH * RPH == kSlotsPerHalvesSplit, "half-row unit shape");
    const Shape &s = a.s;
    const int b = bh / s.Hq, h = bh - b * s.Hq;
    const int lane = threadIdx.x % H, row = threadIdx.x / H;
    const S *qp = (const S *)a.qtilde + b * a.qt_sb + h * a.qt_sh + lane * EPL;
    const uint4 q0 = load16(qp), q1 = load16(qp + D / 2);
    const uint32_t oob = (uint32_t)s.K * D * sizeof(S);
    const __amdgpu_buffer_rsrc_t ring = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<S *>((const S *)a.q_ring + (int64_t)bh * s.K * D), (short)0, (int)oob,
        0x00020000);
    const int32_t *pr = a.pos_ring + ((int64_t)b * s.Hkv + h / s.G) * s.K;
    uint4 raw[UH];
    int pos[UH];
#pragma unroll
    for (int u = 0; u < UH; ++u) {
        const int k = match_slot<UH>(a, first, u, RPH, row);
        raw[u] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(ring, (uint32_t)(k * D + lane * EPL) * sizeof(S), 0,
                                                         kCacheNt));
    }
    // The row group's UH positions in one load instruction (lane u of the
    // group reads row u's), handed to the other lanes when the bound is
    // formed: one instruction instead of UH (each costs address processing
    // for the whole wave).
    static_assert(UH <= H, "one position per lane of a half row");
    int pv = 0;
    if (lane < UH)
        pv = pr[match_slot<UH>(a, first, lane, RPH, row)];
    *done = ld_uniform(a.w.sync + kSyncDone);
    const int m = ld_uniform(a.pos + b);
    const bool ready = group_ready(a, b, b * s.Hkv + h / s.G);
    __asm__ volatile("" ::"s"(*done));
    const bool m_ok = ready && m >= 0 && m < s.T && m >= s.min_ctx;
    auto lane_d2 = [&](const uint4 &qv4, const uint4 &rv4) {
        float qv[EPL], rv[EPL];
        unpack<T>(qv4, qv);
        unpack<T>(rv4, rv);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float df = qv[e] - rv[e];
            acc = fmaf(df, df, acc);
        }
        return acc;
    };
    const float lb_max = s.thresh2 * kFilterMargin;
    float h0[UH];
    bool keep[UH], any[UH];
    uint4 raw2[UH];
#pragma unroll
    for (int u = 0; u < UH; ++u) {
        h0[u] = row_sum<H>(lane_d2(q0, raw[u]));
        pos[u] = __shfl(pv, ((int)(threadIdx.x & 63) & ~(H - 1)) + u, 64);
        const int pu = pos[u];
        keep[u] = h0[u] < lb_max && m_ok && pu >= 0 && pu >= m - s.K && pu <= m - 1;
        const int k = match_slot<UH>(a, first, u, RPH, row);
        const uint32_t off = keep[u] ? (uint32_t)(k * D + D / 2 + lane * EPL) * sizeof(S) : oob;
        // A wave none of whose rows can still hit skips the second half:
        // no load instruction (an out-of-range one still costs address
        // processing) and no distance.
        any[u] = __builtin_amdgcn_ballot_w64(keep[u]) != 0;
        raw2[u] = make_uint4(0u, 0u, 0u, 0u);
        if (any[u])
            raw2[u] = __builtin_bit_cast(uint4,
                                         __builtin_amdgcn_raw_buffer_load_b128(ring, off, 0, kCacheNt));
    }
    unsigned long long best = ~0ull;
#pragma unroll
    for (int u = 0; u < UH; ++u) {
        if (!any[u])
            continue;
        const float acc = h0[u] + row_sum<H>(lane_d2(q1, raw2[u]));
        uint32_t bits = __float_as_uint(acc);
        if (acc != acc)
            bits = 0x7f800000u;  // NaN distance counts as +inf
        const unsigned long long key =
            ((unsigned long long)bits << 32) | (0xffffffffu - (uint32_t)pos[u]);
        best = umin64(best, keep[u] ? key : ~0ull);
    }
#pragma unroll
    for (int off = H; off < 64; off <<= 1)
        best = umin64(best, shfl_xor_u64(best, off));
    if ((threadIdx.x & 63) == 0)
        sm[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 1; i < kBlock / 64; ++i)
            best = umin64(best, sm[i]);
    }
    return best;
}

// Match kernel.  Grid (nsplit, B*Hq) of kSlotsPerSplit-slot full-row splits,
// or, with the filter (kHalves), (ceil(K / kSlotsPerHalvesSplit), B*Hq) of
// half-row splits.  The head's key is the minimum over its splits (exact
// and order-independent), folded with a 64-bit atomic minimum; read by the
// next kernel, reset to ~0 by the merge of the step.
template <class T, int D, bool kHalves>
__global__ __launch_bounds__(kBlock) void match_kernel(StepArgs a)
{
    __shared__ unsigned long long sm[kBlock / 64];
    constexpr int U = kSlotsPerSplit / (kBlock / (D / T::EPL));
    const int bh = blockIdx.y, b = bh / a.s.Hq;
    if constexpr (kHalves) {
        // Filter on: half rows (the same keys as the full-row scan).
        unsigned long long done;
        const unsigned long long best = match_halves<T, D>(a, blockIdx.x * kSlotsPerHalvesSplit, bh, &done, sm);
        if (threadIdx.x == 0 && best != ~0ull)
            atomicMin(&key_set(a, done >> a.done_shift)[bh * kKeyStride], best);
        return;
    }
    MatchLoads<T, D, U> ml;
    match_issue<T, D, U>(a, blockIdx.x * kSlotsPerSplit, bh, ml);
    // Scalar words after the rows are requested (a wait for any scalar load
    // waits for all of them).  The done counter selects the key set; read
    // here, in flight with the rows, rather than after the reduction, where
    // it was a further round trip of every workgroup.
    const unsigned long long done = ld_uniform(a.w.sync + kSyncDone);
    const bool ready = group_ready(a, b, b * a.s.Hkv + (bh - b * a.s.Hq) / a.s.G);
    __asm__ volatile("" ::"s"(done));
    const unsigned long long best = match_finish<T, D, U>(a, ld_uniform(a.pos + b), ready, ml, sm);
    if (threadIdx.x == 0 && best != ~0ull)
        atomicMin(&key_set(a, done >> a.done_shift)[bh * kKeyStride], best);
}

// ---------------------------------------------------------------------------
// Merge of one KV group.  The fold has a fixed shape, so a head's result
// depends only on its own item list (not on the thread count that runs it):
// the list is cut into A = items before the rectify split and Bt = the
// rest; with more than MergeDirect<G>::N items each list is cut into at most
// P equal segments folded left to right, then the segments in order.
// R = C (+) A with C the cached summary of the matched slot (empty on a
// miss); out = R (+) Bt.
constexpr int kMergeBlock = 1024;
// Groups with at most N items take the merge's direct path (all of a
// wave's loads in registers at once).
template <int G>
struct MergeDirect {
    static constexpr int N = G >= 8 ? 12 : 24;
};
// Bounded spin of a wait on another workgroup (polls of about a
// microsecond each).
constexpr int kSpinLimit = 1 << 18;

template <class T, int D, int G>
struct MergeShape {
    static constexpr int P = 64 / G;                   // segments per list
    static constexpr int DPT = D / 16;                 // dims per task
    static constexpr int TPS = 16;                     // tasks per (head, segment)
    static constexpr int SEG = D + 1;                  // floats per segment record
    // direct path: weights, list results, and the four waves' sums per list
    static constexpr int kDirect = 2 * G * MergeDirect<G>::N + 4 * G + 8 * G * D;
    static constexpr int kFloats = G * P * SEG > kDirect ? G * P * SEG : kDirect;
    static constexpr int NTASK = G * P * TPS;
    static_assert(NTASK == 1024, "merge shape");
};

// The log2-lse of item tid % MD, head tid / MD (threads below G * MD; -inf
// past cnt), requested by fold_lse before the partial vectors so that the
// weights need not wait for them.
template <int MD, int G, class Src>
__device__ inline float fold_lse(const Src &src, int cnt)
{
    const int tid = threadIdx.x;
    float v = -INFINITY;
    if (tid < G * MD) {
        const int j = tid / MD, i = tid - j * MD;
        if (i < cnt)
            src.lse(i, j, v);
    }
    return v;
}

// Direct fold of a group's items [0, cnt), cnt <= MD, list A = items
// [0, nA), list Bt = the rest.  Per head and list, one lane sums the item
// weights w_i = 2^(l_i - M) in item order against the list maximum M and
// leaves them in LDS with the list's log2-lse M + log2(S) and 1 / S; every
// pair of output dims is then sum_i w_i o_i (item order) times 1 / S.  An
// empty list gives the empty summary.  lv: this thread's fold_lse.  lds:
// 2 * G * MD + 4 * G floats.
template <int MD, int G>
__device__ inline void fold_weights(float lv, int cnt, int nA, float *lds)
{
    float *s_l = lds, *s_w = lds + G * MD, *s_hl = s_w + G * MD, *s_inv = s_hl + 2 * G;
    const int tid = threadIdx.x;
    if (tid < G * MD) {
        s_l[tid] = lv;
        s_w[tid] = 0.f;
    }
    __syncthreads();
    if (tid < 2 * G) {
        const int j = tid >> 1, L = tid & 1;
        const int i0 = L ? nA : 0, i1 = L ? cnt : nA;
        const float *l = s_l + j * MD;
        float M = -INFINITY;
        for (int i = i0; i < i1; ++i)
            M = fmaxf(M, l[i]);
        float S = 0.f;
        if (M != -INFINITY)
            for (int i = i0; i < i1; ++i) {
                const float w = l[i] == -INFINITY ? 0.f : ex2(l[i] - M);
                s_w[j * MD + i] = w;
                S += w;
            }
        s_hl[tid] = M != -INFINITY ? M + lg2(S) : -INFINITY;
        s_inv[tid] = M != -INFINITY ? 1.f / S : 0.f;
    }
    __syncthreads();
}

// Partials of one KV group as the merge reads them.
// PlainParts: the three-kernel arrays, item i of the group at global index
// begin + i; every load is valid.
template <int D, int G>
struct PlainParts {
    const float *o, *l;
    int64_t begin;
    // N floats (a multiple of 4) of item i from float f of its G * D.
    template <int N>
    __device__ void span(int i, int f, float *v) const
    {
        const float *src = o + (begin + i) * G * D + f;
#pragma unroll
        for (int k = 0; k < N; k += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(src + k);
            v[k] = x.x;
            v[k + 1] = x.y;
            v[k + 2] = x.z;
            v[k + 3] = x.w;
        }
    }
    __device__ bool lse(int i, int j, float &v) const
    {
        v = l[(begin + i) * G + j];
        return true;
    }
    // N consecutive dims from d0 (N = 2 or a multiple of 4)
    template <int N>
    __device__ bool vec(int i, int j, int d0, float *v) const
    {
        const float *src = o + ((begin + i) * G + j) * D + d0;
        if constexpr (N == 2) {
            const float2 x = *reinterpret_cast<const float2 *>(src);
            v[0] = x.x;
            v[1] = x.y;
        } else {
#pragma unroll
            for (int k = 0; k < N; k += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(src + k);
                v[k] = x.x;
                v[k + 1] = x.y;
                v[k + 2] = x.z;
                v[k + 3] = x.w;
            }
        }
        return true;
    }
};

// CoherentParts: the single launch's partials of the group (item i at
// index i), written by other workgroups of the same launch and therefore
// read device-coherently.
template <int D, int G>
struct CoherentParts {
    const float *o, *l;
    // As PlainParts::span, with 16-byte loads that carry the same
    // device-coherence bit (sc1) as the agent-scope atomic loads.
    template <int N>
    __device__ void span(int i, int f, float *v) const
    {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(o), (short)0, kItemsPerGroupMax * G * D * 4, 0x00020000);
#pragma unroll
        for (int k = 0; k < N; k += 4) {
            const float4 x = __builtin_bit_cast(
                float4, __builtin_amdgcn_raw_buffer_load_b128(r, (i * G * D + f + k) * 4, 0, kCacheSc1));
            v[k] = x.x;
            v[k + 1] = x.y;
            v[k + 2] = x.z;
            v[k + 3] = x.w;
        }
    }
    __device__ bool lse(int i, int j, float &v) const
    {
        v = ld_wt(l + (int64_t)i * G + j);
        return true;
    }
    template <int N>
    __device__ bool vec(int i, int j, int d0, float *v) const
    {
        const unsigned long long *src =
            reinterpret_cast<const unsigned long long *>(o + ((int64_t)i * G + j) * D + d0);
#pragma unroll
        for (int k = 0; k < N; k += 2) {
            const unsigned long long w = ld_wt(src + k / 2);
            v[k] = __uint_as_float((uint32_t)w);
            v[k + 1] = __uint_as_float((uint32_t)(w >> 32));
        }
        return true;
    }
};

// Fold items [i0, i1) of head j into (l, o) for dims [d0, d0 + DPT), with
// the loads of the next batch of four items in flight during each merge.
template <int D, int G, int DPT, class Src>
__device__ inline void fold_items(const Src &src, int i0, int i1, int j, int d0, float &l,
                                  float *o)
{
    constexpr int NBUF = 4;
    // Two register buffers with compile-time indices (no scratch).
    float lb0[NBUF], ob0[NBUF][DPT], lb1[NBUF], ob1[NBUF][DPT];
    auto fetch = [&](float(&lb)[NBUF], float(&ob)[NBUF][DPT], int base) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            const int i = base + u;
            lb[u] = -INFINITY;
            if (i < i1) {
                src.lse(i, j, lb[u]);
                src.template vec<DPT>(i, j, d0, ob[u]);
            }
        }
    };
    auto consume = [&](const float(&lb)[NBUF], const float(&ob)[NBUF][DPT], int base) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u)
            if (base + u < i1)
                merge_into<DPT>(l, o, lb[u], ob[u]);
    };
    fetch(lb0, ob0, i0);
    for (int base = i0; base < i1; base += 2 * NBUF) {
        if (base + NBUF < i1)
            fetch(lb1, ob1, base + NBUF);
        consume(lb0, ob0, base);
        if (base + NBUF < i1) {
            if (base + 2 * NBUF < i1)
                fetch(lb0, ob0, base + 2 * NBUF);
            consume(lb1, ob1, base + NBUF);
        }
    }
}

// Pair tasks of the merge: two adjacent dims of one head, the same split for
// every thread count NT.
template <int D, int G, int NT>
struct MergePairs {
    static constexpr int NPAIR = G * D / 2;            // pair tasks
    static constexpr int NPK = (NPAIR + NT - 1) / NT;  // pair tasks per thread
};

// Cached summary C of each of this thread's pairs of group grp (empty on a
// miss); slot_of(jj) is the matched ring slot of the group's head jj, or -1.
// The lse is kept as loaded (natural log) so that no instruction waits for
// these loads before the merge uses them.
template <class T, int D, int G, int NT, class SlotOf>
__device__ inline void load_cached(const StepArgs &a, int grp, SlotOf &&slot_of,
                                   float (&c_l)[MergePairs<D, G, NT>::NPK],
                                   float (&c_o)[MergePairs<D, G, NT>::NPK][2])
{
    using MP = MergePairs<D, G, NT>;
    const Shape &s = a.s;
    const int b = grp / s.Hkv, g = grp - b * s.Hkv;
    // Branch-free: the group's G heads' rings as buffers, and a thread with
    // nothing to load reads at the buffers' size, which returns zeros
    // without a memory access (so do all reads where there are no rings:
    // full decode, every head missed).  A plain load whose value is selected
    // afterwards was turned into a conditional load, and the merge's rescale
    // of the lse moved next to it, where it waited for every load requested
    // before it (the first item's K/V rows among them).
    const int64_t h0 = (int64_t)b * s.Hq + g * G;
    const uint32_t n_l = a.lse_ring ? (uint32_t)(G * s.K) * 4u : 0u;
    const uint32_t n_o = a.o_ring ? (uint32_t)(G * s.K * D) * 4u : 0u;
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        a.lse_ring ? a.lse_ring + h0 * s.K : nullptr, (short)0, (int)n_l, 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        a.o_ring ? a.o_ring + h0 * s.K * D : nullptr, (short)0, (int)n_o, 0x00020000);
#pragma unroll
    for (int k = 0; k < MP::NPK; ++k) {
        const int pt = threadIdx.x + k * NT;
        const bool pair = pt < MP::NPAIR;
        const int pp = pair ? pt : 0;
        const int jj = 2 * pp / D, dim = 2 * pp - jj * D;
        const int slot = slot_of(jj);
        const bool use = pair && slot >= 0;
        const uint32_t ri = (uint32_t)(jj * s.K + slot);
        const uint32_t l = __builtin_amdgcn_raw_buffer_load_b32(rl, use ? ri * 4u : n_l, 0, 0);
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(ro, use ? (ri * D + dim) * 4u : n_o, 0, 0);
        c_l[k] = use ? __uint_as_float(l) : -INFINITY;
        c_o[k][0] = __uint_as_float(v[0]);
        c_o[k][1] = __uint_as_float(v[1]);
    }
}

// Merge of group grp by the NT threads of the calling workgroup: cnt items
// read from src, the group's range [gstart, e], with the cached summaries
// (c_l, c_o) from load_cached; ready is group_ready of the group as every
// thread read it before this call.  The caller passes e and ready so that
// the merge does not wait for loads of its own.  Outputs are handled in pair tasks,
// so the fold is the same for every NT and every source.  lds holds
// MergeShape::kFloats floats.
template <class T, int D, int G, int NT, class Src>
__device__ void merge_group(const StepArgs &a, int grp, int cnt, int gstart, int e, bool ready,
                            const Src &src, float *lds,
                            const float (&c_l)[MergePairs<D, G, NT>::NPK],
                            const float (&c_o)[MergePairs<D, G, NT>::NPK][2])
{
    using M = MergeShape<T, D, G>;
    constexpr int P = M::P, DPT = M::DPT, TPS = M::TPS, SEG = M::SEG, NTASK = M::NTASK;
    constexpr int NPAIR = MergePairs<D, G, NT>::NPAIR;
    constexpr int NPK = MergePairs<D, G, NT>::NPK;
    constexpr int MD = MergeDirect<G>::N;
    using S = typename T::S;
    const Shape &s = a.s;
    const int tid = threadIdx.x;
    const int b = grp / s.Hkv, g = grp - b * s.Hkv;
    const int r_split = (a.mode == kPlanInit) ? 0 : s.r;
    const int nA = GroupItems(gstart, e, r_split, s.F, a.mode != kPlanInit, s.cmin).n_before_split();
    MAC_MARK(kTlMergeBegin);
    // The pre-RoPE queries of the fused append are requested first.
    S qa[NPK][2];
    if (a.append_fused) {
#pragma unroll
        for (int k = 0; k < NPK; ++k) {
            const int pt = tid + k * NT;
            const int f = pt < NPAIR ? 2 * pt : 0, jj = f / D, dim = f - jj * D;
            const S *qs = (const S *)a.qtilde + b * a.qt_sb + (g * G + jj) * a.qt_sh + dim;
            qa[k][0] = qs[0];
            qa[k][1] = qs[1];
        }
    }

    // list 0 = A (items [0, nA)), list 1 = Bt (items [nA, cnt), the sink item
    // last); each pair folds into res[list][k].
    float res_l[2][NPK], res_o[2][NPK][2];
    if (cnt <= MD) {
        // Few items: waves 0..3 each load every float of items w, w + 4, ...
        // (16-byte loads, issued before the weights are formed), sum them
        // per list with the weights of fold_weights, and the four wave sums
        // are added in wave order.  The result does not depend on NT.
        constexpr int FPL = G * D / 64 < 4 ? 4 : G * D / 64;  // floats per lane
        constexpr int LANES = G * D / FPL;
        constexpr int IPW = (MD + 3) / 4;
        const int wave = tid >> 6, lane = tid & 63;
        const bool loader = wave < 4 && lane < LANES;
        const int f0 = lane * FPL, jl = (loader ? f0 : 0) / D;
        const float lv = fold_lse<MD, G>(src, cnt);
        float ov[IPW][FPL];
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int i = wave + 4 * u;
#pragma unroll
            for (int e = 0; e < FPL; ++e)
                ov[u][e] = 0.f;
            if (loader)
                src.template span<FPL>(i < cnt ? i : cnt - 1, f0, ov[u]);
        }
        fold_weights<MD, G>(lv, cnt, nA, lds);
        MAC_MARK(kTlMergeWeights);
        const float *s_w = lds + G * MD, *s_hl = s_w + G * MD, *s_inv = s_hl + 2 * G;
        float *s_sum = lds + 2 * G * MD + 4 * G;  // [4 waves][2 lists][G * D]
        if (loader) {
            float acc[2][FPL];
#pragma unroll
            for (int e = 0; e < FPL; ++e)
                acc[0][e] = acc[1][e] = 0.f;
#pragma unroll
            for (int u = 0; u < IPW; ++u) {
                const int i = wave + 4 * u;
                const float w = i < cnt ? s_w[jl * MD + i] : 0.f;
                const float wa = i < nA ? w : 0.f, wb = i < nA ? 0.f : w;
#pragma unroll
                for (int e = 0; e < FPL; ++e) {
                    acc[0][e] = fmaf(wa, ov[u][e], acc[0][e]);
                    acc[1][e] = fmaf(wb, ov[u][e], acc[1][e]);
                }
            }
#pragma unroll
            for (int L = 0; L < 2; ++L)
#pragma unroll
                for (int e = 0; e < FPL; e += 4)
                    *reinterpret_cast<float4 *>(s_sum + (wave * 2 + L) * G * D + f0 + e) =
                        make_float4(acc[L][e], acc[L][e + 1], acc[L][e + 2], acc[L][e + 3]);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NPK; ++k) {
            const int pt = tid + k * NT;
            const int f = pt < NPAIR ? 2 * pt : 0, jj = f / D;
#pragma unroll
            for (int L = 0; L < 2; ++L) {
                float o0 = 0.f, o1 = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float2 x =
                        *reinterpret_cast<const float2 *>(s_sum + (w * 2 + L) * G * D + f);
                    o0 += x.x;
                    o1 += x.y;
                }
                res_l[L][k] = s_hl[2 * jj + L];
                res_o[L][k][0] = o0 * s_inv[2 * jj + L];
                res_o[L][k][1] = o1 * s_inv[2 * jj + L];
            }
        }
        __syncthreads();  // lds is reused below
    } else {
#pragma unroll
        for (int list = 0; list < 2; ++list) {
            const int l0 = list == 0 ? 0 : nA;
            const int L = list == 0 ? nA : cnt - nA;
            const int Pe = L < P ? L : P;
            for (int task = tid; task < NTASK; task += NT) {
                const int j = task / (P * TPS), seg = (task / TPS) % P, d0 = (task % TPS) * DPT;
                float l = -INFINITY, o[DPT];
#pragma unroll
                for (int i = 0; i < DPT; ++i)
                    o[i] = 0.f;
                if (seg < Pe)
                    fold_items<D, G, DPT>(src, l0 + seg * L / Pe, l0 + (seg + 1) * L / Pe, j, d0,
                                          l, o);
                float *rec = lds + (j * P + seg) * SEG;
                if ((task % TPS) == 0)
                    rec[D] = l;
#pragma unroll
                for (int i = 0; i < DPT; ++i)
                    rec[d0 + i] = o[i];
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NPK; ++k) {
                const int pt = tid + k * NT;
                float fl = -INFINITY, fo[2] = {0.f, 0.f};
                if (pt < NPAIR) {
                    const int jj = 2 * pt / D, dim = 2 * pt - jj * D;
                    for (int sg = 0; sg < Pe; ++sg) {
                        const float *r = lds + (jj * P + sg) * SEG;
                        merge_into<2>(fl, fo, r[D], r + dim);
                    }
                }
                res_l[list][k] = fl;
                res_o[list][k][0] = fo[0];
                res_o[list][k][1] = fo[1];
            }
            __syncthreads();
            if (list == 0)
                MAC_MARK(kTlMergeWeights);
        }
    }
    MAC_MARK(kTlMergeSummed);

    // R = C (+) A, out = R (+) Bt.  Results are held until every thread has
    // read its cached summary (and the group's epoch), since the fused
    // append may overwrite them.
    float out_l[NPK], out_o[NPK][2], rec_l[NPK], rec_o[NPK][2];
#pragma unroll
    for (int k = 0; k < NPK; ++k) {
        float lr = c_l[k] * kLog2e, orr[2] = {c_o[k][0], c_o[k][1]};
        merge_into<2>(lr, orr, res_l[0][k], res_o[0][k]);
        float lo = lr, oo[2] = {orr[0], orr[1]};
        merge_into<2>(lo, oo, res_l[1][k], res_o[1][k]);
        out_l[k] = lo;
        out_o[k][0] = oo[0];
        out_o[k][1] = oo[1];
        rec_l[k] = lr;
        rec_o[k][0] = orr[0];
        rec_o[k][1] = orr[1];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NPK; ++k) {
        const int pt = tid + k * NT;
        if (pt >= NPAIR)
            continue;
        const int jj = 2 * pt / D, dim = 2 * pt - jj * D;
        const int h = g * G + jj, bh = b * s.Hq + h;
        if (a.out)
            *reinterpret_cast<float2 *>(a.out + (int64_t)bh * D + dim) =
                make_float2(out_o[k][0], out_o[k][1]);
        if (a.out_lse && dim == 0)
            a.out_lse[bh] = out_l[k] * kLn2;
        if (a.append_fused) {
            // Rectify-append into slot m mod K of this head's rings.
            const int slot = e % s.K;
            const int64_t ri = ((int64_t)bh * s.K + slot) * D + dim;
            ((S *)a.q_ring)[ri] = qa[k][0];
            ((S *)a.q_ring)[ri + 1] = qa[k][1];
            *reinterpret_cast<float2 *>(a.o_ring + ri) = make_float2(rec_o[k][0], rec_o[k][1]);
            if (dim == 0)
                a.lse_ring[(int64_t)bh * s.K + slot] = rec_l[k] * kLn2;
        } else {
            *reinterpret_cast<float2 *>(a.w.rect_o + (int64_t)bh * D + dim) =
                make_float2(rec_o[k][0], rec_o[k][1]);
            if (dim == 0)
                a.w.rect_l[bh] = rec_l[k];
        }
    }
    MAC_MARK(kTlMergeWritten);
    // A group that was not ready adopts the request's epoch; its ring
    // restarts with this step's entry, here or in the append kernel.
    if (!ready && tid == 0)
        a.w.ring_epoch[grp] = a.epoch[b];
    if (a.append_fused) {
        ring_append_pos(a, grp, e, !ready, tid, NT);
    } else if (tid == 0) {
        // For the append kernel: the group's restart flag and position (it
        // never reads the caller's arrays, which main_stream may overwrite).
        a.w.restart[grp] = ready ? 0 : 1;
        a.w.app_pos[grp] = e;
    }
}

// Merge kernel: one workgroup of kMergeBlock threads per KV group, from the
// plan that the attention kernel published.
template <class T, int D, int G, bool kWarm>
__global__ __launch_bounds__(kMergeBlock) void merge_kernel(StepArgs a)
{
    __shared__ float lds[MergeShape<T, D, G>::kFloats];
    const int grp = blockIdx.x;
    if (threadIdx.x < G)  // ready for the next step's match
        a.w.keys[((int64_t)grp * G + threadIdx.x) * kKeyStride] = ~0ull;
    if (grp == 0 && threadIdx.x == 0)  // ready for the next attention launch
        a.w.ctrl[kCtrlClaim] = 0;
    const int cnt = a.w.grp_count[grp];
    if (cnt == 0)
        return;  // the planner wrote this group's outputs
    float c_l[MergePairs<D, G, kMergeBlock>::NPK], c_o[MergePairs<D, G, kMergeBlock>::NPK][2];
    const int32_t *dec = a.w.dec_slot + (int64_t)grp * G;
    load_cached<T, D, G, kMergeBlock>(a, grp, [&](int jj) { return dec[jj]; }, c_l, c_o);
    const PlainParts<D, G> src{a.w.part_o, a.w.part_l, (int64_t)a.w.grp_begin[grp]};
    // The group's epoch is read by every thread before merge_group's
    // barriers; thread 0 rewrites it after them.
    const int b = grp / a.s.Hkv;
    merge_group<T, D, G, kMergeBlock>(a, grp, cnt, a.w.grp_start[grp], end_of(a, b),
                                      group_ready(a, b, grp), src, lds, c_l, c_o);
}

// ---------------------------------------------------------------------------
// Attention over the work list.  Each workgroup loops over items; within an
// item, LPR-lane row `row` handles tokens t0 + i*RPB + row, NB tokens per
// block, with the next block's K/V loads in flight while a block computes.
// Per-row online softmax in log2 units; the RPB row states are combined in
// LDS in a fixed order into one partial (o, log2-lse) per head.
template <class T, int D, int G>
struct AttendShape {
    static constexpr int EPL = T::EPL, LPR = D / EPL, RPB = kBlock / LPR;
    // 16-lane rows use the reduce-scatter softmax (NB * G <= 16 values per
    // lane); other row widths all-reduce every logit.
    static constexpr bool kScatter = LPR == 16;
    static constexpr int NB = kScatter ? (16 / G < 4 ? 16 / G : 4) : 4;  // tokens per row per block
    // bf16 K with d = 128 and 4 heads per KV head: the logits of a wave's 16
    // tokens come from 4 MFMAs (16 tokens x 32 dims x 16 columns: the 4
    // heads' queries split into bf16 high and low parts, 8 columns unused)
    // instead of VALU dot products and a row reduce-scatter.
    static constexpr bool kMfma = kScatter && T::EPL == 8 && D == 128 && G == 4;
    // The MFMA path fits two waves per SIMD (256 registers) when the
    // register allocator is told to; the other shapes are left to it.
    static constexpr int kWavesPerEu = kMfma ? 2 : 1;
    // m, l, acc per row; row weights; per-head sum and maximum
    static constexpr int kFloats = RPB * G * (D + 3) + 2 * G;
};

template <class T, int G, int EPL, int NB>
struct KvBlock {
    uint4 k[NB], v[NB];
    int base;  // token of row 0, i = 0
};

// Per-lane element offset into a K row.  On the MFMA path lane l of a wave
// holds dims 8 * (l / 16) + 32 * kk of its token for MFMA kk (the A-operand
// layout of v_mfma_f32_16x16x32_bf16: row l % 16, 8 consecutive k per 16
// lanes); otherwise lane l % 16 of a row holds dims 8 * (l % 16).
template <class T, int D, int G>
__device__ inline int k_lane_offset()
{
    if constexpr (AttendShape<T, D, G>::kMfma)
        return 8 * ((threadIdx.x & 63) >> 4);
    else
        return (threadIdx.x % (D / T::EPL)) * T::EPL;
}

// Where one KV group's rows live, as seen by one lane.  Dense: row t at
// k + t * kv_st (k at the request and group).  Paged: row t of the request
// at k + table[t >> page_shift] * kv_sb + (t mod page size) * kv_st (k at
// the group only; table is the request's row of the page table).
template <class T>
struct KvRows {
    const typename T::S *k, *v;
    const int32_t *table;  // null when dense
};

template <class T, int D, int G, bool kPaged>
__device__ inline KvRows<T> kv_rows(const StepArgs &a, int b, int g)
{
    using S = typename T::S;
    const Shape &s = a.s;
    const int64_t gb = (kPaged ? 0 : b * s.kv_sb) + g * s.kv_sh;
    KvRows<T> r;
    r.k = (const S *)a.k + gb + k_lane_offset<T, D, G>();
    r.v = (const S *)a.v + gb + (threadIdx.x % (D / T::EPL)) * T::EPL;
    r.table = kPaged ? s.page_table + (int64_t)b * s.max_pages : nullptr;
    return r;
}

// Element offsets of the rows of a paged block: the block's page numbers
// come through scalar loads (the table is read-only during the launch, and
// scalar loads do not queue behind the vector loads in flight), then each
// lane picks its token's page.  A block of TPB tokens spans at most
// TPB / kMinPage + 1 pages.
constexpr int kMinPage = 16;
template <int TPB>
struct BlockPages {
    static constexpr int N = TPB / kMinPage + 1;
    int pg[N];
    int p0, shift;
    __device__ BlockPages() {}
    __device__ BlockPages(const Shape &s, const int32_t *table, int base, int t1)
    {
        base = __builtin_amdgcn_readfirstlane(base);
        t1 = __builtin_amdgcn_readfirstlane(t1);
        shift = s.page_shift;
        const int last = (base + TPB < t1 ? base + TPB : t1) - 1;
        p0 = base >> shift;
        const int pl = last >> shift;
        const __attribute__((address_space(4))) int32_t *ct =
            (const __attribute__((address_space(4))) int32_t *)table;
#pragma unroll
        for (int j = 0; j < N; ++j)
            pg[j] = ct[p0 + j < pl ? p0 + j : pl];
    }
    // The page of token t as pg[0] plus the steps pg[k] - pg[k-1] for
    // k <= j: a sum over the few scalars rather than an indexed read, which
    // the compiler would place in scratch memory.
    __device__ int64_t offset(const Shape &s, int t) const
    {
        const int j = (t >> shift) - p0;
        int page = pg[0];
#pragma unroll
        for (int k = 1; k < N; ++k)
            page += (j >= k) ? pg[k] - pg[k - 1] : 0;
        return (int64_t)page * s.kv_sb + (int64_t)(t & ((1 << shift) - 1)) * s.kv_st;
    }
};

// load_block with row t at element offset off(t) from the lane's column;
// kNt: loads with the non-temporal hint.
template <class T, int D, int G, int LPR, int RPB, int NB, bool kNt = false, class Off>
__device__ inline void load_block_at(KvBlock<T, G, T::EPL, NB> &kv, const KvRows<T> &rows,
                                     int base, int t1, int row, Off &&off)
{
    const typename T::S *kb = rows.k, *vb = rows.v;
    kv.base = base;
    if constexpr (AttendShape<T, D, G>::kMfma) {
        // K in the MFMA A layout: lane l (m = l % 16) loads token
        // base + 16 * (m % 4) + 4 * wave + m / 4, i.e. slot m % 4 of row
        // 4 * wave + m / 4, so that logit row 4 * r + v of the product is
        // slot v of the wave's row r; kb carries the lane's dim offset.
        const int m = threadIdx.x & 15;
        int tk = base + 16 * (m & 3) + 4 * (threadIdx.x >> 6) + (m >> 2);
        tk = tk < t1 ? tk : t1 - 1;
        const int64_t ok = off(tk);
#pragma unroll
        for (int kk = 0; kk < NB; ++kk)
            kv.k[kk] = load16_kv<kNt>(kb + ok + 32 * kk);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            int t = base + i * RPB + row;
            t = t < t1 ? t : t1 - 1;
            kv.v[i] = load16_kv<kNt>(vb + off(t));
        }
    } else {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            int t = base + i * RPB + row;
            t = t < t1 ? t : t1 - 1;
            const int64_t o = off(t);
            kv.k[i] = load16_kv<kNt>(kb + o);
            kv.v[i] = load16_kv<kNt>(vb + o);
        }
    }
}

// K/V rows of one block.  Every lane loads: a token at or past t1 reads row
// t1 - 1 of the item instead, which the block computation masks (its logit
// is -inf, its probability exactly 0).  No branch separates the loads, so
// the compiler can wait for each block on its own.
template <class T, int D, int G, int LPR, int RPB, int NB, bool kPaged, bool kNt = false>
__device__ inline void load_block(KvBlock<T, G, T::EPL, NB> &kv, const KvRows<T> &rows,
                                  const Shape &s, int base, int t1, int row)
{
    if constexpr (kPaged) {
        const BlockPages<RPB * NB> bp(s, rows.table, base, t1);
        load_block_at<T, D, G, LPR, RPB, NB, kNt>(kv, rows, base, t1, row,
                                                  [&](int t) { return bp.offset(s, t); });
    } else {
        const int64_t st = s.kv_st;
        load_block_at<T, D, G, LPR, RPB, NB, kNt>(kv, rows, base, t1, row,
                                                  [&](int t) { return (int64_t)t * st; });
    }
}

// The group's post-RoPE queries in the form the logit computation takes,
// scaled by scale * log2 e: this lane's fp32 slices for the VALU dot
// products, or, on the MFMA path, the B operands of the 4 MFMAs.  B operand
// kk of lane l holds column n = l % 16, dims 32 * kk + 8 * ((l / 16) % 4) + e:
// head n's query rounded to bf16 for n < 4, what that rounding lost (again in
// bf16) for 4 <= n < 8 (the sum of the two columns' logits carries the query
// to about 16 significant bits), zero above.
template <class T, int D, int G>
struct QRegs {
    static constexpr bool kMfma = AttendShape<T, D, G>::kMfma;
    float qr[kMfma ? 1 : G][T::EPL];
    uint4 qb[4];
    // src(j, d0, x): the 4 floats of head j's query from dim d0 into x.
    template <class Src>
    __device__ void fill(Src &&src, float qscale)
    {
        if constexpr (kMfma) {
            const int n = threadIdx.x & 15, kg = (threadIdx.x >> 4) & 3;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = 0.f;
                if (n < 8) {
                    src(n & 3, 32 * kk + 8 * kg, x);
                    src(n & 3, 32 * kk + 8 * kg + 4, x + 4);
                }
                uint32_t bb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t hb, lb;
                    split_bf16(x[e], qscale, hb, lb);
                    bb[e] = n < 4 ? hb : n < 8 ? lb : 0u;
                }
                qb[kk] = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16),
                                    bb[4] | (bb[5] << 16), bb[6] | (bb[7] << 16));
            }
        } else {
            const int lane = threadIdx.x % (D / T::EPL);
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int e4 = 0; e4 < T::EPL; e4 += 4) {
                    float x[4];
                    src(j, lane * T::EPL + e4, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        qr[j][e4 + e] = x[e] * qscale;
                }
        }
    }
};

template <class T, int D, int G, int LPR, int RPB, int NB>
__device__ inline void compute_block(const KvBlock<T, G, T::EPL, NB> &kv, int row,
                                     const float (&qr)[G][T::EPL], const int (&st)[G], int t1,
                                     float (&mrun)[G], float (&lrun)[G],
                                     float (&acc)[G][T::EPL])
{
    constexpr int EPL = T::EPL;
    float sc[NB][G];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        float kf[EPL];
        unpack<T>(kv.k[i], kf);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float x = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                x = fmaf(qr[j][e], kf[e], x);
            sc[i][j] = x;
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float v = row_sum<LPR>(sc[i][j]);
            const int t = kv.base + i * RPB + row;
            sc[i][j] = (t < t1 && t >= st[j]) ? v : -INFINITY;
        }
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float bm = sc[0][j];
#pragma unroll
        for (int i = 1; i < NB; ++i)
            bm = fmaxf(bm, sc[i][j]);
        const float mn = fmaxf(mrun[j], bm);
        const bool live = mn != -INFINITY;
        const float alpha = live ? ex2(mrun[j] - mn) : 1.f;
        float lsum = lrun[j] * alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[j][e] *= alpha;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const float pi = live ? ex2(sc[i][j] - mn) : 0.f;
            sc[i][j] = pi;
            lsum += pi;
        }
        lrun[j] = lsum;
        mrun[j] = mn;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        float vf[EPL];
        unpack<T>(kv.v[i], vf);
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[j][e] = fmaf(sc[i][j], vf[e], acc[j][e]);
    }
}

// One block with 16-lane rows: after the partial dot products each lane
// holds NB*G (<= 16) partial logits; a reduce-scatter leaves lane k with
// the logit of token k / G, head k % G, so the softmax of a block costs two
// exponentials per lane.  The per-head running max and sum live in the
// lanes of that head; probabilities and rescale factors reach the P*V
// products through row broadcasts.
template <class T, int D, int G, int RPB, int NB>
__device__ inline void compute_block_rs(const KvBlock<T, G, T::EPL, NB> &kv, int row, int lane,
                                        const QRegs<T, D, G> &q, int my_st, int t1,
                                        float &mrun, float &lrun, float (&acc)[G][T::EPL])
{
    constexpr bool kMfma = QRegs<T, D, G>::kMfma;
    const auto &qr = q.qr;
    const auto &qb = q.qb;
    constexpr int EPL = T::EPL;
    static_assert(NB * G <= 16, "values per row");
    float sv;
    if constexpr (kMfma) {
        // qb[kk]: this lane's B operand of MFMA kk (see ItemCtx).  Product
        // row 4 * r + v, column n sits in lane 16 * r + n, element v: the
        // logit of slot v of row r against column n.  Column n + 4 holds the
        // low part of head n's query.
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv.k[kk]),
                                                        __builtin_bit_cast(bf16x8, qb[kk]), c, 0,
                                                        0, 0);
        float sh[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sh[v] = c[v] + dpp<kDppRowRor + 12>(c[v]);
        // Lane 4 * v + h of the row takes lane h's value v: the layout of
        // the reduce-scatter below (lane k: slot k / 4, head k % 4).
        const float s1 = dpp<kDppRowShr + 4>(sh[1]);
        const float s2 = dpp<kDppRowShr + 8>(sh[2]);
        const float s3 = dpp<kDppRowShr + 12>(sh[3]);
        const int qd = lane >> 2;
        sv = qd == 0 ? sh[0] : qd == 1 ? s1 : qd == 2 ? s2 : s3;
    } else {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            v[k] = 0.f;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            float kf[EPL];
            unpack<T>(kv.k[i], kf);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float x = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    x = fmaf(qr[j][e], kf[e], x);
                v[i * G + j] = x;
            }
        }
        sv = row_reduce_scatter16(v, lane);
    }
    const int t = kv.base + (lane / G) * RPB + row;
    sv = (lane < NB * G && t < t1 && t >= my_st) ? sv : -INFINITY;
    const float bm = row_mod_reduce<G, true>(sv);
    const float mn = fmaxf(mrun, bm);
    const bool live = mn != -INFINITY;
    const float alpha = live ? ex2(mrun - mn) : 1.f;
    const float p = live ? ex2(sv - mn) : 0.f;
    lrun = lrun * alpha + row_mod_reduce<G, false>(p);
    mrun = mn;
    static_for<G>([&](auto J) {
        const float aj = dpp<kDppRowNewBcast + J>(alpha);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[J][e] *= aj;
    });
    static_for<NB>([&](auto I) {
        float vf[EPL];
        unpack<T>(kv.v[I], vf);
        static_for<G>([&](auto J) {
            const float pb = dpp<kDppRowNewBcast + I * G + J>(p);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[J][e] = fmaf(pb, vf[e], acc[J][e]);
        });
    });
}

// Per-(request, KV group) state of the attention items: this lane's K/V
// row pointers and its slice of the group's post-RoPE queries (pre-scaled
// by scale * log2 e).  Built once per group, before the items are known.
template <class T, int D, int G, bool kPaged = false>
struct ItemCtx {
    using S = typename T::S;
    static constexpr int EPL = T::EPL;
    KvRows<T> rows;
    QRegs<T, D, G> q;
    // K/V rows only; the queries come from queries_from_lds.
    __device__ ItemCtx(const StepArgs &a, int b, int g, bool) : rows(kv_rows<T, D, G, kPaged>(a, b, g)) {}
    // This lane's queries from LDS ([G][D] floats, as QueryStage stores
    // them, and on the MFMA path the B operands QueryStage::store_b forms),
    // scaled as the global-memory constructor scales them.
    __device__ void queries_from_lds(const float *s_q, const uint4 *s_qb, float qscale)
    {
        if constexpr (QRegs<T, D, G>::kMfma) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                q.qb[kk] = s_qb[kk * 64 + (threadIdx.x & 63)];
            return;
        }
        q.fill(
            [&](int j, int d0, float *x) {
                const float4 v = *reinterpret_cast<const float4 *>(s_q + j * D + d0);
                x[0] = v.x;
                x[1] = v.y;
                x[2] = v.z;
                x[3] = v.w;
            },
            qscale);
    }
    __device__ ItemCtx(const StepArgs &a, int b, int g) : ItemCtx(a, b, g, true)
    {
        const float *qp = a.q + b * a.q_sb + (int64_t)(g * G) * a.q_sh;
        const int64_t qsh = a.q_sh;
        q.fill(
            [&](int j, int d0, float *x) {
                const float4 v = *reinterpret_cast<const float4 *>(qp + j * qsh + d0);
                x[0] = v.x;
                x[1] = v.y;
                x[2] = v.z;
                x[3] = v.w;
            },
            a.s.qscale);
    }
};

// The group's post-RoPE queries, G * D floats, read once per workgroup (one
// float2 per thread) instead of once per 16-lane row: request, then store
// to LDS (s_q[G][D]) once the values are needed.
template <int D, int G>
struct QueryStage {
    static constexpr int kPairs = G * D / 2;
    static constexpr int kPer = (kPairs + kBlock - 1) / kBlock;
    float2 v[kPer];
    __device__ void request(const StepArgs &a, int b, int g)
    {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            int i = threadIdx.x + k * kBlock;
            i = i < kPairs ? i : kPairs - 1;
            const int j = i / (D / 2), dim = 2 * (i - j * (D / 2));
            v[k] = *reinterpret_cast<const float2 *>(a.q + b * a.q_sb +
                                                     (int64_t)(g * G + j) * a.q_sh + dim);
        }
    }
    __device__ void store(float *s_q) const
    {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = threadIdx.x + k * kBlock;
            if (i < kPairs)
                *reinterpret_cast<float2 *>(s_q + 2 * i) = v[k];
        }
    }
    // The MFMA B operands of QRegs (D = 128, G = 4), formed once per
    // workgroup: s_qb[kk * 64 + l] is lane l's operand of MFMA kk.  Each
    // thread rounds its pair (high and low bf16 parts, as QRegs::fill does)
    // into the two columns of its head; the threads below 128 clear the
    // unused columns 8..15.
    __device__ void store_b(uint4 *s_qb, float qscale) const
    {
        static_assert(D == 128 && G == 4 && kPer == 1, "MFMA operand shape");
        uint32_t *w = reinterpret_cast<uint32_t *>(s_qb);
        const int i = threadIdx.x;  // pair: head j, dims d, d + 1
        const int j = i / (D / 2), d = 2 * (i - j * (D / 2));
        const int kk = d / 32, kg = (d % 32) / 8, e = d % 8;
        uint32_t h0, h1, l0, l1;
        split_bf16(v[0].x, qscale, h0, l0);
        split_bf16(v[0].y, qscale, h1, l1);
        w[(kk * 64 + 16 * kg + j) * 4 + e / 2] = h0 | (h1 << 16);
        w[(kk * 64 + 16 * kg + j + 4) * 4 + e / 2] = l0 | (l1 << 16);
        if (threadIdx.x < 128) {
            const int zk = threadIdx.x / 32, z = threadIdx.x % 32;
            s_qb[zk * 64 + 16 * (z / 8) + 8 + z % 8] = make_uint4(0, 0, 0, 0);
        }
    }
};

// The first two K/V blocks of a work item (tokens [t0, t1) of the group of
// ctx), requested without waiting.  t0 < t1.
template <class T, int D, int G>
struct ItemBufs {
    using L = AttendShape<T, D, G>;
    KvBlock<T, G, T::EPL, L::NB> a, b;
};

template <class T, int D, int G, bool kPaged>
__device__ inline void item_issue(const StepArgs &a, const ItemCtx<T, D, G, kPaged> &ctx, int t0, int t1,
                                  ItemBufs<T, D, G> &bufs, bool both)
{
    using L = AttendShape<T, D, G>;
    constexpr int LPR = L::LPR, RPB = L::RPB, NB = L::NB, TPB = RPB * NB;
    const int row = threadIdx.x / LPR;
    load_block<T, D, G, LPR, RPB, NB, kPaged>(bufs.a, ctx.rows, a.s, t0, t1, row);
    // both: the second block is requested without a branch (all its rows
    // clamp to t1 - 1 when the item has one block).
    if (both || t0 + TPB < t1)
        load_block<T, D, G, LPR, RPB, NB, kPaged>(bufs.b, ctx.rows, a.s, t0 + TPB, t1, row);
}

// Running state of one work item's attention: per-row online softmax in
// log2 units (with 16-lane rows, lane k keeps the running max / sum of head
// k % G in mrun[0], lrun[0], and my_st is that head's token-start bound).
template <class T, int D, int G>
struct ItemAcc {
    float mrun[G], lrun[G], acc[G][T::EPL];
    int my_st;
    __device__ void reset(const int (&st)[G], int lane)
    {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            mrun[j] = -INFINITY;
            lrun[j] = 0.f;
#pragma unroll
            for (int e = 0; e < T::EPL; ++e)
                acc[j][e] = 0.f;
        }
        my_st = __builtin_amdgcn_readfirstlane(st[0]);
#pragma unroll
        for (int j = 1; j < G; ++j)
            my_st = (lane % G == j) ? __builtin_amdgcn_readfirstlane(st[j]) : my_st;
    }
};

// One block of an item (tokens < t1; head j attends from st[j]).
template <class T, int D, int G>
__device__ inline void item_block(const KvBlock<T, G, T::EPL, AttendShape<T, D, G>::NB> &buf,
                                  int row, int lane, const QRegs<T, D, G> &q,
                                  const int (&st)[G], int t1, ItemAcc<T, D, G> &ia)
{
    using L = AttendShape<T, D, G>;
    if constexpr (L::kScatter)
        compute_block_rs<T, D, G, L::RPB, L::NB>(buf, row, lane, q, ia.my_st, t1, ia.mrun[0],
                                                 ia.lrun[0], ia.acc);
    else
        compute_block<T, D, G, L::LPR, L::RPB, L::NB>(buf, row, q.qr, st, t1, ia.mrun,
                                                      ia.lrun, ia.acc);
}

// The RPB row states of an item are combined in LDS in a fixed order into
// one partial (o, log2-lse) per head, handed to sink(j, dim, o, lse) for
// every dim (lse meaningful at dim 0).  lds holds AttendShape::kFloats
// floats; the call starts and ends with the workgroup in step.
template <class T, int D, int G, class Sink>
__device__ inline void item_combine(const ItemAcc<T, D, G> &ia, float *lds, int row, int lane,
                                    Sink &&sink)
{
    using L = AttendShape<T, D, G>;
    constexpr int EPL = L::EPL, RPB = L::RPB;
    float *sm_m = lds;                  // [RPB][G]
    float *sm_l = lds + RPB * G;        // [RPB][G]
    float *sm_acc = lds + 2 * RPB * G;  // [RPB][G][D]
    if constexpr (L::kScatter) {
        if (lane < G) {
            sm_m[row * G + lane] = ia.mrun[0];
            sm_l[row * G + lane] = ia.lrun[0];
        }
    } else {
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                sm_m[row * G + j] = ia.mrun[j];
                sm_l[row * G + j] = ia.lrun[j];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            sm_acc[(row * G + j) * D + lane * EPL + e] = ia.acc[j][e];
    __syncthreads();
    MAC_MARK(kTlCombineRows);
    // Row weights c[rr][j] = 2^(m[rr][j] - M_j), one per thread; then head
    // j's total sum L_j = sum_rr c[rr][j] * l[rr][j] in row order.
    float *sm_c = sm_acc + RPB * G * D;  // [RPB][G]
    float *sm_hd = sm_c + RPB * G;       // [G]: L_j, then [G]: M_j
    const int wr = threadIdx.x / G, wj = threadIdx.x - wr * G;
    if (threadIdx.x < RPB * G) {
        float Mj = -INFINITY;
#pragma unroll
        for (int q = 0; q < RPB; ++q)
            Mj = fmaxf(Mj, sm_m[q * G + wj]);
        sm_c[wr * G + wj] = Mj != -INFINITY ? ex2(sm_m[wr * G + wj] - Mj) : 0.f;
        if (wr == 0)
            sm_hd[G + wj] = Mj;
    }
    __syncthreads();
    if (threadIdx.x < G) {
        float Ls = 0.f;
        if (sm_hd[G + threadIdx.x] != -INFINITY) {
#pragma unroll
            for (int q = 0; q < RPB; ++q)
                Ls = fmaf(sm_c[q * G + threadIdx.x], sm_l[q * G + threadIdx.x], Ls);
        }
        sm_hd[threadIdx.x] = Ls;
    }
    __syncthreads();
    MAC_MARK(kTlCombineSums);
    for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
        const int j = idx / D, dim = idx - j * D;
        const float ls = sm_hd[j];
        float o = 0.f, Lg = -INFINITY;
        if (ls > 0.f) {
            float os = 0.f;
#pragma unroll
            for (int rr = 0; rr < RPB; ++rr)
                os = fmaf(sm_c[rr * G + j], sm_acc[(rr * G + j) * D + dim], os);
            o = os / ls;
            Lg = sm_hd[G + j] + lg2(ls);
        }
        sink(j, dim, o, Lg);
    }
    __syncthreads();  // lds is free again
}

// Attention of one work item whose first two blocks item_issue requested,
// by the whole workgroup; head j of the group attends from st[j].  Each
// block's successor two blocks ahead is requested as soon as the block has
// been consumed.  The partial goes to sink as in item_combine.
template <class T, int D, int G, bool kPaged, class Sink>
__device__ inline void item_finish(const StepArgs &a, const ItemCtx<T, D, G, kPaged> &ctx, int t0, int t1,
                                   const int (&st)[G], float *lds, ItemBufs<T, D, G> &bufs,
                                   Sink &&sink)
{
    using L = AttendShape<T, D, G>;
    constexpr int LPR = L::LPR, RPB = L::RPB, NB = L::NB;
    constexpr int TPB = RPB * NB;  // tokens per block
    const Shape &s = a.s;
    const int lane = threadIdx.x % LPR, row = threadIdx.x / LPR;
    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    auto &bufA = bufs.a;
    auto &bufB = bufs.b;
    ItemAcc<T, D, G> ia;
    ia.reset(st, lane);
    for (int base = t0; base < t1; base += 2 * TPB) {
        item_block<T, D, G>(bufA, row, lane, ctx.q, st, t1, ia);
        if (base + 2 * TPB < t1)
            load_block<T, D, G, LPR, RPB, NB, kPaged>(bufA, ctx.rows, s, base + 2 * TPB, t1, row);
        if (base + TPB < t1) {
            item_block<T, D, G>(bufB, row, lane, ctx.q, st, t1, ia);
            if (base + 3 * TPB < t1)
                load_block<T, D, G, LPR, RPB, NB, kPaged>(bufB, ctx.rows, s, base + 3 * TPB, t1, row);
        }
    }
    MAC_MARK(kTlBlocksDone);
    item_combine<T, D, G>(ia, lds, row, lane, sink);
}

// This workgroup's share of the work list (see attend_kernel): the items
// in order, skipping empty groups; `valid` is false past the share.
struct ShareIter {
    const PlanTables *pt;
    int NG, r_split, F, cmin, hi;
    bool sink;
    int grp, i, t0, t1;
    bool valid;
    GroupItems gi;
    __device__ ShareIter(const PlanTables &p, int ng, int rsplit, int f, int cmin_, bool snk,
                         int lo, int hi_)
        : pt(&p), NG(ng), r_split(rsplit), F(f), cmin(cmin_), hi(hi_), sink(snk), grp(0), i(0),
          t0(0), t1(0), valid(false)
    {
        int l = 0, h = NG;  // last group with work offset <= lo
        while (l < h) {
            const int mid = (l + h) >> 1;
            if (pt->gwork[mid] <= lo)
                l = mid + 1;
            else
                h = mid;
        }
        grp = l - 1 < 0 ? 0 : l - 1;
        gi = items(grp);
        l = 0;
        h = pt->gcount[grp];  // first item with offset >= lo
        while (l < h) {
            const int mid = (l + h) >> 1;
            if (offset(mid) < lo)
                l = mid + 1;
            else
                h = mid;
        }
        i = l;
        settle();
    }
    __device__ GroupItems items(int gr) const
    {
        return GroupItems(pt->gstart[gr], pt->gend[gr], r_split, F, sink, cmin);
    }
    __device__ int offset(int ii) const { return pt->gwork[grp] + gi.offset(ii); }
    __device__ void settle()
    {
        while (grp < NG && i >= pt->gcount[grp]) {
            ++grp;
            i = 0;
            if (grp < NG)
                gi = items(grp);
        }
        valid = grp < NG && offset(i) < hi;
        if (valid)
            gi.item(i, t0, t1);
        grp = __builtin_amdgcn_readfirstlane(grp);
        t0 = __builtin_amdgcn_readfirstlane(t0);
        t1 = __builtin_amdgcn_readfirstlane(t1);
    }
    __device__ void next()
    {
        ++i;
        settle();
    }
    __device__ int item_index() const { return pt->gbegin[grp] + i; }
};

// Pool items of the attention kernel's claimed tail are handed out longest
// first: those of groups cut on a grid coarser than the minimum (long ranges,
// e.g. a missing head's whole context) before the rest, each class in item
// order, so the last claims are short items and workgroups finish close
// together.  s_bp[g] (g <= NG) receives the number of coarse-grid pool
// items in groups below g; returns their total.  Pool items are the items
// from index `first` on.  Called by the whole workgroup.
__device__ int pool_big_prefix(const PlanTables &pt, int NG, int r_split, int F, int cmin,
                               bool sink, int first, int32_t *s_bp)
{
    __shared__ int s_w[kBlock / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto big_items = [&](int g) {
        const int n = pt.gcount[g];
        if (n == 0)
            return 0;
        const int skip = first > pt.gbegin[g] ? first - pt.gbegin[g] : 0;
        if (skip >= n)
            return 0;
        const GroupItems gi(pt.gstart[g], pt.gend[g], r_split, F, sink, cmin);
        return (gi.n_main > 0 && gi.rs.cs > cmin) ? n - skip : 0;
    };
    const int per = (NG + kBlock - 1) / kBlock;
    const int lo = tid * per, hi = lo + per < NG ? lo + per : NG;
    int run = 0;
    for (int g = lo; g < hi; ++g)
        run += big_items(g);
    int x = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        s_w[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kBlock / 64; ++w) {
        before += w < wave ? s_w[w] : 0;
        total += s_w[w];
    }
    int acc = before + x - run;
    for (int g = lo; g < hi; ++g) {
        s_bp[g] = acc;
        acc += big_items(g);
    }
    if (tid == 0)
        s_bp[NG] = total;
    __syncthreads();
    return total;
}

// Plan + attention kernel.  kWarm only renames the instantiation used by
// the ring warm-up, so kernel profiles separate it from decode steps.
template <class T, int D, int G, bool kWarm, bool kPaged>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(AttendShape<T, D, G>::kWavesPerEu))) void attend_kernel(StepArgs a)
{
    __shared__ float lds[AttendShape<T, D, G>::kFloats];
    extern __shared__ int32_t plan_lds[];
    const PlanTables pt = plan_tables(a, plan_lds, blockIdx.x == 0);
    const Shape &s = a.s;
    const int NG = s.B * s.Hkv;
    const int r_split = (a.mode == kPlanInit) ? 0 : s.r;
    using L = AttendShape<T, D, G>;
    constexpr int LPR = L::LPR, RPB = L::RPB, NB = L::NB, TPB = RPB * NB;
    using S = typename T::S;
    const int lane = threadIdx.x % LPR, row = threadIdx.x / LPR;
    // Work split: the items whose work offset (the group's offset + tokens
    // before the item + kItemCost per earlier item of the group) lies below
    // kStaticPct percent of the total are shared statically, workgroup w
    // running those in [w * Ws / grid, (w + 1) * Ws / grid): a contiguous run
    // of near-equal work.  The remaining items form a pool that workgroups
    // claim one at a time, with an atomic counter, once their share is done,
    // so faster workgroups take more of it.  Which workgroup runs an item
    // does not change the results: partials are stored by item index.
    // The pool pays for its claims (an atomic round trip and a barrier each)
    // only when workgroups have several items to run: at least kPoolItems
    // per workgroup on average.
    const bool pooled = a.dyn_pool && pt.total >= kPoolItems * (int)gridDim.x;
    const int Ws = pooled ? (int)((int64_t)pt.work * kStaticPct / 100) : pt.work;
    const int lo = (int)((int64_t)Ws * blockIdx.x / gridDim.x);
    const int hi = (int)((int64_t)Ws * (blockIdx.x + 1) / gridDim.x);
    __shared__ int s_claim[4];
    int dyn_first;
    const bool with_sink = a.mode != kPlanInit;
    {
        const ShareIter pool(pt, NG, r_split, s.F, s.cmin, with_sink, Ws, INT_MAX);
        dyn_first = pool.valid ? pool.item_index() : pt.total;
    }
    // Claim c of the pool maps to the c-th coarse-grid item, or, past
    // those, to the (c - n_big)-th other item (see pool_big_prefix).
    int32_t *s_bp = plan_lds + (s.B * s.Hq + 5 * NG + 2 + 2 * (kBlock / 64));
    const int n_big =
        pooled ? pool_big_prefix(pt, NG, r_split, s.F, s.cmin, with_sink, dyn_first, s_bp) : 0;
    auto pool_index = [&](int c) {
        const bool big = c < n_big;
        const int k = big ? c : c - n_big;
        // items of the class before group g
        auto before = [&](int g) {
            const int pp = pt.gbegin[g] > dyn_first ? pt.gbegin[g] - dyn_first : 0;
            return big ? s_bp[g] : pp - s_bp[g];
        };
        int l = 0, h = NG - 1;  // the first group g with before(g + 1) > k
        while (l < h) {
            const int mid = (l + h) >> 1;
            if (before(mid + 1) > k)
                h = mid;
            else
                l = mid + 1;
        }
        return (pt.gbegin[l] > dyn_first ? pt.gbegin[l] : dyn_first) + (k - before(l));
    };
    // Claims the next pool item for the whole workgroup (one atomic, handed
    // to the other waves through LDS); pt.total when the pool is empty.  A
    // count outside the pool ends the claims.
    int n_claims = 0;
    auto claim = [&]() {
        if (threadIdx.x == 0) {
            const uint32_t pool = (uint32_t)(pt.total - dyn_first);
            const uint32_t c =
                pooled ? atomicAdd((uint32_t *)&a.w.ctrl[kCtrlClaim], 1u) : pool;
            s_claim[n_claims & 3] = c < pool ? pool_index((int)c) : pt.total;
        }
        __syncthreads();
        const int it = s_claim[n_claims & 3];
        ++n_claims;
        return it < pt.total ? it : pt.total;
    };
    ShareIter cur(pt, NG, r_split, s.F, s.cmin, with_sink, lo, hi);
    // The share's blocks stream through two buffers, two blocks ahead of the
    // computation, across item and group boundaries; the loader also makes
    // the claims, and the computation follows its sequence of items.
    ShareIter ld = cur;
    bool ld_valid = cur.valid;
    int ld_base = ld.t0;
    int n_seen = 0;  // pool items the computation has taken over
    auto pool_item = [&](ShareIter &itr, int it) {
        // Position itr on pool item it (< pt.total).
        int l = 0, h = NG;
        while (l < h) {
            const int mid = (l + h) >> 1;
            if (pt.gbegin[mid] <= it)
                l = mid + 1;
            else
                h = mid;
        }
        itr.grp = __builtin_amdgcn_readfirstlane(l - 1);
        itr.i = it - pt.gbegin[itr.grp];
        itr.gi = itr.items(itr.grp);
        itr.gi.item(itr.i, itr.t0, itr.t1);
        itr.t0 = __builtin_amdgcn_readfirstlane(itr.t0);
        itr.t1 = __builtin_amdgcn_readfirstlane(itr.t1);
        itr.valid = true;
    };
    if (!ld_valid) {
        const int it = claim();
        ld_valid = it < pt.total;
        if (ld_valid) {
            pool_item(ld, it);
            cur = ld;
            ++n_seen;
        }
        ld_base = ld.t0;
    }
    if (!ld_valid)
        return;
    // Paged K/V: the page numbers of the block `issue` requests next are
    // fetched (scalar loads) one block ahead, so no request waits for them.
    BlockPages<TPB> pages;
    auto fetch_pages = [&] {
        if constexpr (kPaged) {
            if (ld_valid)
                pages = BlockPages<TPB>(s, s.page_table + (int64_t)(ld.grp / s.Hkv) * s.max_pages,
                                        ld_base, ld.t1);
        }
    };
    auto issue = [&](KvBlock<T, G, T::EPL, NB> &buf) {
        if (!ld_valid)
            return;
        const int lb = ld.grp / s.Hkv, lg = ld.grp - lb * s.Hkv;
        if constexpr (kPaged)
            load_block_at<T, D, G, LPR, RPB, NB, true>(buf, kv_rows<T, D, G, true>(a, lb, lg),
                                                       ld_base, ld.t1, row,
                                                       [&](int t) { return pages.offset(s, t); });
        else
            load_block<T, D, G, LPR, RPB, NB, false, true>(
                buf, kv_rows<T, D, G, false>(a, lb, lg), s, ld_base, ld.t1, row);
        ld_base += TPB;
        if (ld_base >= ld.t1) {
            if (ld.valid && ld.hi != INT_MAX)
                ld.next();  // the static share's next item, if any
            else
                ld.valid = false;
            if (!ld.valid) {
                const int it = claim();
                if (it < pt.total) {
                    pool_item(ld, it);
                    ld.hi = INT_MAX;  // marks a pool item
                }
            }
            ld_valid = ld.valid;
            ld_base = ld.t0;
        }
        fetch_pages();
    };
    fetch_pages();
    KvBlock<T, G, T::EPL, NB> bufA, bufB;
    issue(bufA);
    issue(bufB);

    int qgrp = cur.grp;
    ItemCtx<T, D, G, kPaged> ctx(a, qgrp / s.Hkv, qgrp % s.Hkv);
    int st[G];
    ItemAcc<T, D, G> ia;
    auto begin_item = [&] {
        const int b = cur.grp / s.Hkv, g = cur.grp - b * s.Hkv;
        const bool sink_item = cur.gi.is_sink(cur.i);  // every head attends the sink
#pragma unroll
        for (int j = 0; j < G; ++j)
            st[j] = sink_item ? 0 : code_start(pt.code[b * s.Hq + g * G + j]);
        if (cur.grp != qgrp) {
            qgrp = cur.grp;
            ctx = ItemCtx<T, D, G, kPaged>(a, b, g);
        }
        ia.reset(st, lane);
    };
    begin_item();
    int cb = cur.t0;  // first token of the block being consumed
    // Consumes the block in buf, refills buf two blocks ahead, and closes the
    // item after its last block; false once the work is done.
    auto consume = [&](KvBlock<T, G, T::EPL, NB> &buf) {
        item_block<T, D, G>(buf, row, lane, ctx.q, st, cur.t1, ia);
        issue(buf);
        cb += TPB;
        if (cb < cur.t1)
            return true;
        const int it = cur.item_index();
        float *po = a.w.part_o + (int64_t)it * G * D;
        float *pl = a.w.part_l + (int64_t)it * G;
        item_combine<T, D, G>(ia, lds, row, lane, [&](int j, int dim, float o, float lgv) {
            po[j * D + dim] = o;
            if (dim == 0)
                pl[j] = lgv;
        });
        // The next item: the static share's, else the pool item the loader
        // claimed next (claims complete before their item is consumed).
        if (cur.valid && cur.hi != INT_MAX)
            cur.next();
        else
            cur.valid = false;
        if (!cur.valid) {
            if (n_seen >= n_claims)
                return false;
            const int pit = s_claim[n_seen & 3];
            ++n_seen;
            if (pit >= pt.total)
                return false;
            pool_item(cur, pit);
            cur.hi = INT_MAX;
        }
        cb = cur.t0;
        begin_item();
        return true;
    };
    while (consume(bufA) && consume(bufB)) {
    }
}

// NaN outputs, an empty staged summary and nothing to append for the G
// heads of group grp (query heads bh0 ...), written by the calling
// workgroup: a position out of range, or a single launch that cannot trust
// its counters.
template <int D, int G>
__device__ inline void group_invalid(const StepArgs &a, int grp, int bh0)
{
    for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
        const int bh = bh0 + idx / D;
        if (a.out)
            a.out[(int64_t)bh * D + idx % D] = NAN;
        a.w.rect_o[(int64_t)bh * D + idx % D] = 0.f;
        if (idx % D == 0) {
            if (a.out_lse)
                a.out_lse[bh] = NAN;
            a.w.rect_l[bh] = -INFINITY;
        }
    }
    if (threadIdx.x == 0)
        a.w.app_pos[grp] = -1;
}

// Single-launch key words (see mac_internal.h): bits 31..24 of the low word
// carry the tag's low byte instead of 0xff (positions are below 2^24).
__device__ inline unsigned long long key_tagged(unsigned long long key, uint32_t tag8)
{
    return (key & ~0xff000000ull) | ((unsigned long long)tag8 << 24);
}

// Wave 0 of a workgroup polls the nkw key words of its group until all hold
// tag8, leaving the untagged keys of the match units in s_keys[upg].
// Returns false if the wait gave up.
__device__ inline bool poll_keys(const StepArgs &a, const unsigned long long *kw, uint32_t tag8,
                                 unsigned long long *s_keys)
{
    const int lane = threadIdx.x & 63;
    for (int spin = 0;; ++spin) {
        bool fresh = true;
        for (int u = lane; u < a.nkw; u += 64) {
            const unsigned long long w = ld_wt(kw + u);
            fresh &= ((uint32_t)(w >> 24) & 0xffu) == tag8;
            if (u < a.upg)
                s_keys[u] = w | 0xff000000ull;
        }
        if (__all(fresh))
            return true;
        if (spin >= kSpinLimit)
            return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Single-launch match unit u of a group: head u / nsplit of the group,
// slots from (u mod nsplit) * unit_slots.  Key words u >= upg carry a copy
// of the last unit (only their tag is read).
__device__ inline void single_unit(const StepArgs &a, int u, int &j, int &first)
{
    u = u < a.upg ? u : a.upg - 1;
    j = u / a.nsplit;
    first = (u - j * a.nsplit) * a.unit_slots;
}

// Minimum of a 64-bit key over aligned groups of W lanes (8 <= W <= 64).
template <int CTRL>
__device__ inline unsigned long long dpp64(unsigned long long v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, true);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
template <int W>
__device__ inline unsigned long long lanes_min64(unsigned long long v)
{
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "lane group");
    v = umin64(v, dpp64<kDppQuadXor1>(v));
    v = umin64(v, dpp64<kDppQuadXor2>(v));
    v = umin64(v, dpp64<kDppHalfMirror>(v));
    if constexpr (W >= 16)
        v = umin64(v, dpp64<kDppRowMirror>(v));
    if constexpr (W >= 32)
        v = umin64(v, shfl_xor_u64(v, 16));
    if constexpr (W >= 64)
        v = umin64(v, shfl_xor_u64(v, 32));
    return v;
}

// Speculative item of workgroup loc of a group at position e: the loc-th
// item from the end of the group's items for the range [e - span + 1, e],
// span being the group's span at its previous step (a range keeps its span
// while every head keeps matching the previous position).  A hit range
// spans at most K + r tokens, so its chunk is the shape's minimum; every main item
// but the first is then fixed by e and r alone, and the sink item by e.
// The range's first item depends on the span, which moves whenever a head's
// match does; it is speculated only if `first`.  False if loc has no such
// item.
__device__ inline bool spec_item(const StepArgs &a, int e, int loc, int span, bool first,
                                 int &t0, int &t1)
{
    if (loc >= kSpecMax || e < 0 || e >= a.s.T)
        return false;
    const int hit_span = a.s.K + a.s.r;
    span = (span <= 0 || span > hit_span) ? hit_span : span;
    const int s0 = e - span + 1;
    const GroupItems gi(s0 > 0 ? s0 : 0, e, a.s.r, a.s.F, true, a.s.cmin, a.s.cmin);
    const int it = gi.n - 1 - loc;
    if (it < 0 || (it == 0 && !first))
        return false;
    gi.item(it, t0, t1);
    return true;
}

// Thread 0's key, tagged, to word u of the group's kKeyReps copies; then a
// workgroup barrier (the match's LDS is reused).
__device__ __forceinline__ void store_unit_key(unsigned long long *kw, int64_t rep_stride, int u,
                                               unsigned long long key, uint32_t tag8)
{
    if (threadIdx.x < 64) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)key);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(key >> 32));
        key = ((unsigned long long)hi << 32) | lo;
        if (threadIdx.x < kKeyReps)
            st_wt(kw + threadIdx.x * rep_stride + u, key_tagged(key, tag8));
    }
    __syncthreads();
}

// Pool set used by the launch of epoch E (alternating by parity).
__device__ inline unsigned long long *pool_set(const StepArgs &a, unsigned long long E)
{
    return a.w.pool + (int64_t)(E & 1) * (kPoolLine + (int64_t)a.pool_cap);
}

// Thread 0: counts group grp as complete on the done counter (no one waits
// for the count's return).
__device__ inline void group_complete(const StepArgs &a, int grp, int NG)
{
    const unsigned long long add =
        grp == 0 ? (1ull << a.done_shift) - (unsigned long long)NG + 1ull : 1ull;
    atomicAdd(&a.w.sync[kSyncDone], add);
}

// The next pool entry for the calling workgroup (group << 8 | item); -1 when
// the pool holds nothing more for this launch (every group has planned and
// every published entry is claimed), -2 if the wait gave up.  Thread 0
// claims and polls; pst / phd are the state and head words it read earlier,
// or ~0 to read them now.  A claim is made only while a published entry is
// unclaimed, so a pool that stays empty costs no atomic.  The result
// reaches every thread through *slot.
__device__ inline int pool_take(unsigned long long *ps, uint32_t tag32, int NG,
                                unsigned long long pst, unsigned long long phd, int *slot)
{
    if (threadIdx.x == 0) {
        int res = -1;
        uint32_t c = 0xffffffffu;  // this workgroup's claim, none yet
        for (int spin = 0;; ++spin) {
            if (pst == ~0ull)
                pst = ld_wt(ps + kPoolState);
            const uint32_t planned = (uint32_t)(pst >> 32), tail = (uint32_t)pst;
            if (c == 0xffffffffu) {
                if (phd == ~0ull)
                    phd = ld_wt(ps + kPoolHead);
                if (phd < tail)
                    c = (uint32_t)atomicAdd(ps + kPoolHead, 1ull);
                else if (planned >= (uint32_t)NG)
                    break;  // all published entries are claimed
            }
            if (c != 0xffffffffu) {
                if (c < tail) {
                    // A reserved entry: its producer writes it.
                    const unsigned long long ent = ld_wt(ps + kPoolLine + c);
                    if ((uint32_t)(ent >> 32) == tag32) {
                        res = (int)(uint32_t)ent;
                        break;
                    }
                } else if (planned >= (uint32_t)NG) {
                    break;  // claimed past the final tail
                }
            }
            if (spin >= kSpinLimit) {
                res = -2;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
            pst = ~0ull;
            phd = ~0ull;
        }
        *slot = res;
    }
    __syncthreads();
    const int r = *slot;
    __syncthreads();  // the slot is reused by the next call
    return r;
}

// The whole decode step in one launch of a.wpg workgroups per KV group, all
// resident at once; U ring rows per lane per match unit.  Workgroup `loc`
// of group grp:
//   1. requests the position and the done counter (the launch's epoch and
//      key tag), its first match unit's ring rows and the group's queries;
//   2. finishes its match units (unit loc, loc + wpg, ...: unit u is head
//      u / nsplit, unit_slots ring slots from split u mod nsplit) and stores
//      each key, tagged, in kKeyReps copies; then requests the K/V of its
//      speculative item, if it has one;
//   3. polls the group's key words (copy loc mod kKeyReps) until all carry
//      the tag, and plans the group: decisions, range [s_g, m], items;
//   4. runs the items n-1-loc, n-1-loc-wpg, ... (from the end of the range,
//      so the speculative loads usually are the first item's data): stores
//      the partials, waits for the stores to complete and counts the item on
//      the group's counter; the workgroup that completes the group merges it
//      (with the fused append), resets the counter and counts the group on
//      the done counter.
// Groups with more items than workgroups publish the rest to a pool that
// the workgroups of every group take from once their own items are done.
// With kMatch false (the second kernel of the two-kernel form), steps 1-3
// are replaced by a read of the group's per-head keys, which the match
// kernel has finished before this launch.
template <class T, int D, int G, int U, bool kPaged, bool kMatch>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void step_kernel(StepArgs a)
{
    using AS = AttendShape<T, D, G>;
    using MS = MergeShape<T, D, G>;
    using MP = MergePairs<D, G, kBlock>;
    // The cross-group pool is part of the group kernel of the two-kernel
    // form only.  In the one-launch kernel (the default up to 16 KV groups)
    // its state cost every hit step more than it saved on the missed ones
    // (measured at 8 groups), so there a group runs all its items itself.
    constexpr bool kPool = !kMatch;
    constexpr int kFloats = AS::kFloats > MS::kFloats ? AS::kFloats : MS::kFloats;
    __shared__ float lds[kFloats];
    __shared__ unsigned long long s_keys[kMaxSingleUnits];
    __shared__ int s_code[G];
    __shared__ int s_last, s_base, s_slot;
    __shared__ int s_plan[kPlanWords];
    __shared__ float s_q[G * D];
    __shared__ uint4 s_qb[AS::kMfma ? 4 * 64 : 1];
    const Shape &s = a.s;
    const int NG = s.B * s.Hkv;
    const int grp = blockIdx.x / a.wpg, loc = blockIdx.x - grp * a.wpg;
    const int b = grp / s.Hkv, g = grp - b * s.Hkv;
    const int bh0 = b * s.Hq + g * G;
    MAC_MARK(kTlEntry);
    unsigned long long *sync = a.w.sync;
    // Entry.  The words of the launch's start (position, counters, the
    // group's previous span, readiness) are scalar loads, requested together
    // with the vector loads that need none of them (the first match unit's
    // ring rows, the queries, the group kernel's key words of both sets);
    // the first wait is for the scalar words.  The done counter's value from
    // earlier launches is visible at kernel start, and the increments of
    // this launch's groups leave floor(done / 2^s) unchanged until this
    // workgroup's own group completes.  Readiness is read before this
    // workgroup's keys are stored (they depend on it), so before the group
    // can complete and its merge restart the rings.
    const int e = ld_uniform(a.pos + b);
    const unsigned long long done = ld_uniform(sync + kSyncDone);
    const unsigned long long broken = ld_uniform(sync + kSyncBroken);
    const int span_prev = (int)ld_uniform(a.w.grp_sync + (int64_t)grp * kGrpStride + kGrpSpan);
    const bool ready = group_ready(a, b, grp);
    // The group's queries and K/V row pointers do not depend on the plan.
    QueryStage<D, G> qs;
    ItemCtx<T, D, G, kPaged> ctx(a, b, g, true);
    unsigned long long hkey = ~0ull;  // group kernel: head's key (lanes j * 64 / G)
    unsigned long long hkey1 = ~0ull;
    int uj = 0, ufirst = 0;
    MatchLoads<T, D, U> ml;
    if constexpr (kMatch) {
        single_unit(a, loc, uj, ufirst);
        match_issue<T, D, U>(a, ufirst, bh0 + uj, ml);
        qs.request(a, b, g);
    } else {
        // The match kernel finished every key of set E & 1; the words of
        // both sets (the workspace always holds two) are requested, so that
        // the request does not wait for E.
        qs.request(a, b, g);
        if (threadIdx.x < 64 && threadIdx.x % (64 / G) == 0) {
            const int64_t o = (int64_t)(bh0 + threadIdx.x / (64 / G)) * kKeyStride;
            hkey = a.w.keys[o];
            hkey1 = a.w.keys[(int64_t)s.B * s.Hq * kKeyStride + o];
        }
    }
    // Keeps the done counter's load with the others: without a use here it
    // is moved past the branch below and waited for on its own.
    __asm__ volatile("" ::"s"(done));
    // An earlier launch on this workspace gave up waiting, so the counters
    // may be inconsistent: every launch until the ring reset writes NaN
    // outputs and computes nothing (no workgroup waits, so none can time out).
    if (broken != 0) {
        if (loc == 0)
            group_invalid<D, G>(a, grp, bh0);
        return;
    }
    const unsigned long long E = done >> a.done_shift;
    int sp_t0 = 0, sp_t1 = 0;
    bool spec = false;
    ItemBufs<T, D, G> bufs;
    bool ok = true;
    if constexpr (kMatch) {
        unsigned long long *klds = reinterpret_cast<unsigned long long *>(lds);
        const int64_t rep_stride = (int64_t)NG * a.nkw;
        unsigned long long *kw = a.w.skeys + (int64_t)grp * a.nkw;
        const uint32_t tag8 = (uint32_t)(E + 1) & 0xffu;
        store_unit_key(kw, rep_stride, loc, match_finish<T, D, U>(a, e, ready, ml, klds), tag8);
        qs.store(s_q);  // read after the barriers of the poll and the plan
        if constexpr (AS::kMfma)
            qs.store_b(s_qb, s.qscale);
        for (int u = loc + a.wpg; u < a.nkw; u += a.wpg) {
            single_unit(a, u, uj, ufirst);
            match_issue<T, D, U>(a, ufirst, bh0 + uj, ml);
            store_unit_key(kw, rep_stride, u, match_finish<T, D, U>(a, e, ready, ml, klds), tag8);
        }
        MAC_MARK(kTlKeys);
        // Speculative K/V, requested once the keys are out: loads complete in
        // order, so requests made earlier would hold back the match (and the
        // first poll of the keys).  They are in flight while the other units'
        // keys arrive.  The loc-th item from the end of the range
        // [e - span + 1, e], span being the group's at its previous step:
        // every item but the range's first has bounds fixed by the grid, e
        // and r alone.  The first is speculated too: the plan waits for
        // the whole match, by when a wrong guess's loads have landed.
        spec = spec_item(a, e, loc, span_prev, true, sp_t0, sp_t1);
        if (spec)
            item_issue<T, D, G, kPaged>(a, ctx, sp_t0, sp_t1, bufs, false);
        MAC_MARK(kTlSpec);
        if (threadIdx.x < 64)
            ok = poll_keys(a, kw + (loc % kKeyReps) * rep_stride, tag8, s_keys);
        ok = block_and(ok);
    } else {
        // Group kernel.  The first workgroup clears the other key set for the
        // next launch's match (the launches that used it have ended).
        if (blockIdx.x == 0) {
            unsigned long long *nxt = key_set(a, E + 1);
            for (int i = threadIdx.x; i < s.B * s.Hq; i += kBlock)
                nxt[(int64_t)i * kKeyStride] = ~0ull;
        }
        if (a.key_parity && (E & 1))
            hkey = hkey1;
        // The queries, requested before the scalar words, have arrived by
        // now.  Stored before the speculative K/V is requested: a wait for
        // them after a conditional request was a wait for every load.
        qs.store(s_q);
        if constexpr (AS::kMfma)
            qs.store_b(s_qb, s.qscale);
        MAC_MARK(kTlKeys);
        // Not the range's first item: the plan follows within a few
        // microseconds, and a wrong guess (the span moves whenever a head's
        // match does) costs its bytes, and its re-request into the same
        // registers waits for the wrong loads to land (without it, 0.7 us
        // less per launch at the 128K batch-8 workload, where most groups'
        // spans move).
        spec = spec_item(a, e, loc, span_prev, false, sp_t0, sp_t1);
        if (spec)
            item_issue<T, D, G, kPaged>(a, ctx, sp_t0, sp_t1, bufs, false);
        MAC_MARK(kTlSpec);
    }
    if (!ok) {
        // The group's keys never all arrived: its outputs are invalid, and
        // the workspace is marked broken until the ring reset (this group's
        // counter and the done counter no longer follow the protocol).
        group_invalid<D, G>(a, grp, bh0);
        if (threadIdx.x == 0) {
            atomicOr(&sync[kSyncSticky], (unsigned long long)MAC_DEV_SYNC_TIMEOUT);
            atomicOr(&sync[kSyncBroken], 1ull);
        }
        return;
    }

    // Plan of the group.  Head j's key is the minimum over its units (exact
    // in any order), taken by the 64 / G lanes j * 64 / G, ... of wave 0;
    // the first of them decides head j.  Every thread then reads the codes
    // from LDS.
    const bool e_ok = e >= 0 && e < s.T;
    if (threadIdx.x < 64) {
        constexpr int LPH = 64 / G;
        const int j = threadIdx.x / LPH, sub = threadIdx.x % LPH;
        unsigned long long key = hkey;
        if constexpr (kMatch) {
            for (int u = sub; u < a.nsplit; u += LPH)
                key = umin64(key, s_keys[j * a.nsplit + u]);
            key = lanes_min64<LPH>(key);
        }
        if (sub == 0) {
            const Decision dc = decide(a, key, e_ok);
            s_code[j] = dc.hit ? dc.p - s.r + 1 : kMissCode;
            if (loc == 0) {
                const int bh = bh0 + j;
                if (a.match_p)
                    a.match_p[bh] = dc.hit ? dc.p : -1;
                if (a.match_d2)
                    a.match_d2[bh] = dc.d2;
            }
        }
    }
    __syncthreads();
    MAC_MARK(kTlPlanned);
    int st[G];
    int sg = e;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        st[j] = code_start(s_code[j]);
        sg = st[j] < sg ? st[j] : sg;
    }
    if (grp == 0 && loc == 0 && threadIdx.x == 0) {
        // Scalar loads: a vector load here would wait for every load this
        // workgroup has in flight (its speculative K/V among them).
        int bad = 0;
        for (int bb = 0; bb < s.B; ++bb) {
            const int eb = ld_uniform(a.pos + bb);
            bad |= !(eb >= 0 && eb < s.T);
        }
        a.w.ctrl[kCtrlStatus] = bad ? MAC_DEV_BAD_POSITION : 0;
    }
    const GroupItems gi(e_ok ? sg : 0, e_ok ? e : 0, s.r, s.F, true, s.cmin);
    const int n = e_ok ? gi.n : 0;

    // Items the group's own workgroups run: all of a hit range; with the
    // pool, of a range cut on a grid coarser than the minimum (a head missed:
    // a long range), one per workgroup -- the items nearest the end -- while
    // the rest go to the launch's pool, where any workgroup that has
    // finished its own work claims them.  The group's first workgroup
    // publishes: the plan record (completed before the entries are written),
    // then the entries, and in any case counts the group as planned.
    const uint32_t tag32 = (uint32_t)(E + 1);
    unsigned long long *ps = pool_set(a, E);
    if (kPool && blockIdx.x == 0 && threadIdx.x == 0) {
        // The other pool set, which no workgroup of this launch touches (the
        // previous launch on this workspace, which used it, has ended), is
        // cleared for the next launch.
        unsigned long long *nxt = pool_set(a, E + 1);
        st_wt(nxt + kPoolState, 0ull);
        st_wt(nxt + kPoolHead, 0ull);
    }
    const bool coarse = n > 0 && gi.n_main > 0 && gi.rs.cs > s.cmin;
    const int n_own = kPool && coarse && n > a.wpg ? a.wpg : n;
    if (kPool && loc == 0) {
        const int n_pool = n - n_own;
        if (n_pool > 0) {
            int32_t *rec = a.w.gplan + (int64_t)grp * kPlanWords;
            const int t = threadIdx.x;
            if (t < kPlanCodes + G) {
                const int v = t == kPlanE       ? e
                              : t == kPlanStart ? sg
                              : t == kPlanN     ? n
                              : t == kPlanReady ? (int)ready
                                                : s_code[t - kPlanCodes];
                st_wt(reinterpret_cast<uint32_t *>(rec + t), (uint32_t)v);
            }
            wait_vmem();
            __syncthreads();
        }
        if (n_pool > 0) {
            if (threadIdx.x == 0)
                s_base = (int)(uint32_t)atomicAdd(ps + kPoolState,
                                                  (1ull << 32) | (unsigned long long)n_pool);
            __syncthreads();
            for (int i = threadIdx.x; i < n_pool; i += kBlock)
                st_wt(ps + kPoolLine + s_base + i,
                      ((unsigned long long)tag32 << 32) | ((uint32_t)grp << 8) | (uint32_t)i);
        } else if (threadIdx.x == 0) {
            // Planned, nothing published: no one waits for this count.
            atomicAdd(ps + kPoolState, 1ull << 32);
        }
    }

    // A workgroup without an item of its own leaves at once: the workgroups
    // that ran items take the pool's items (at least one per item of a
    // group's own workgroups), and idle workgroups polling the pool words
    // would only slow the counters of the others.
    MAC_MARK(kTlPublished);
    MAC_NOTE(kTlNoteItems, n);
    MAC_NOTE(kTlNoteOwn, n_own);
    if (n == 0) {
        // Position out of range: NaN outputs, nothing appended.
        if (loc == 0) {
            group_invalid<D, G>(a, grp, bh0);
            if (threadIdx.x == 0)
                group_complete(a, grp, NG);
        }
        return;
    }
    if (loc >= n_own) {
        MAC_MARK(kTlExitIdle);
        return;
    }
    unsigned long long pst = ~0ull, phd = ~0ull;
    // Counts an item of group cg (cn items); true when the count completes
    // the group.
    auto count_item = [&](int cg, int cn) {
        if (threadIdx.x == 0)
            s_last = atomicAdd(a.w.grp_sync + (int64_t)cg * kGrpStride, 1u) == (uint32_t)(cn - 1);
        __syncthreads();
        return s_last != 0;
    };
    // Merge of group mg, whose last count this workgroup made, with its
    // cached summaries (c_l, c_o from load_cached); the pool words are read
    // again meanwhile.  e and the readiness are the values read at the start
    // of the launch (the group's epoch is not rewritten before this merge
    // does it).
    auto merge = [&](int mg, int mn, int msg, int me, bool mready, const float(&c_l)[MP::NPK],
                     const float(&c_o)[MP::NPK][2]) {
        if (kPool && threadIdx.x == 0) {
            pst = ld_wt(ps + kPoolState);
            phd = ld_wt(ps + kPoolHead);
        }
        const CoherentParts<D, G> src{a.w.part_o + (int64_t)mg * kItemsPerGroupMax * G * D,
                                      a.w.part_l + (int64_t)mg * kItemsPerGroupMax * G};
        merge_group<T, D, G, kBlock>(a, mg, mn, msg, me, mready, src, lds, c_l, c_o);
        if (threadIdx.x == 0) {
            uint32_t *counter = a.w.grp_sync + (int64_t)mg * kGrpStride;
            st_wt(counter, 0u);
            st_wt(counter + kGrpSpan, (uint32_t)(me - msg + 1));
            group_complete(a, mg, NG);
        }
    };

    // Own items n-1-loc, n-1-loc-wpg, ...: the first usually finds its rows
    // in the speculative loads, else requests them at once.  Only then are
    // the cached summaries (in case this workgroup merges the group) and the
    // pool words requested: loads complete in order, so the first item's
    // wait for its rows does not wait for them.
    {
        ctx.queries_from_lds(s_q, s_qb, s.qscale);
        MAC_MARK(kTlOwnQueries);
        float *gpo = a.w.part_o + (int64_t)grp * kItemsPerGroupMax * G * D;
        float *gpl = a.w.part_l + (int64_t)grp * kItemsPerGroupMax * G;
        // Attention of own item it, its rows requested; the partial stored
        // device-coherently, then counted.  The count that completes the
        // group is the group's last, so a workgroup merges its own group at
        // most once, after its items.
        auto own_item = [&](int it, int t0, int t1) {
            // Token-start bounds by value (a reference chosen at run time
            // would put both arrays in scratch memory): the sink item is
            // attended by every head in full.
            const bool sink_item = gi.is_sink(it);
            int sti[G];
#pragma unroll
            for (int j = 0; j < G; ++j)
                sti[j] = sink_item ? 0 : st[j];
            float *po = gpo + (int64_t)it * G * D, *pl = gpl + (int64_t)it * G;
            item_finish<T, D, G, kPaged>(a, ctx, t0, t1, sti, lds, bufs, [&](int j, int dim, float o, float lg) {
                st_wt(po + j * D + dim, o);
                if (dim == 0)
                    st_wt(pl + j, lg);
            });
            const bool first = it == n - 1 - loc;
            if (first)
                MAC_MARK(kTlItemComputed);
            wait_vmem();  // this wave's partial stores have completed
            __syncthreads();
            if (first)
                MAC_MARK(kTlItemStored);
            const bool last = count_item(grp, n);
            if (first)
                MAC_MARK(kTlItemCounted);
            return last;
        };
        int t0, t1;
        gi.item(n - 1 - loc, t0, t1);
        MAC_MARK(kTlOwnBounds);
        if (!(spec && t0 == sp_t0 && t1 == sp_t1))
            item_issue<T, D, G, kPaged>(a, ctx, t0, t1, bufs, false);
        MAC_MARK(kTlOwnRows);
        float c_l[MP::NPK], c_o[MP::NPK][2];
        load_cached<T, D, G, kBlock>(
            a, grp, [&](int j) { return code_slot(s_code[j], s.r, s.K); }, c_l, c_o);
        if (kPool && threadIdx.x == 0) {
            pst = ld_wt(ps + kPoolState);
            phd = ld_wt(ps + kPoolHead);
        }
        // The first item is peeled off the loop, so that its wait for the
        // rows is its own (the loop's items wait for their just-requested
        // rows, the newest loads).
        MAC_NOTE(kTlNoteSpec, !spec ? 0 : (t0 == sp_t0 && t1 == sp_t1) ? 1 : 2);
        MAC_MARK(kTlItem);
        bool merger = own_item(n - 1 - loc, t0, t1);
        for (int jj = loc + a.wpg; jj < n_own; jj += a.wpg) {
            const int it = n - 1 - jj;
            gi.item(it, t0, t1);
            item_issue<T, D, G, kPaged>(a, ctx, t0, t1, bufs, false);
            merger = own_item(it, t0, t1) || merger;
        }
        MAC_MARK(kTlOwnDone);
        if (merger) {
            merge(grp, n, sg, e, ready, c_l, c_o);
            MAC_MARK(kTlMergeEnd);
        }
    }

    if constexpr (!kPool) {
        MAC_MARK(kTlExit);
        return;
    }
    // Pool items of any group, until the pool is drained.
    int n_taken = 0;
    for (;;) {
        const int ent = pool_take(ps, tag32, NG, pst, phd, &s_slot);
        pst = phd = ~0ull;
        if (ent < 0) {
            if (ent == -2 && threadIdx.x == 0) {
                atomicOr(&sync[kSyncSticky], (unsigned long long)MAC_DEV_SYNC_TIMEOUT);
                atomicOr(&sync[kSyncBroken], 1ull);
            }
            break;
        }
        if (n_taken++ == 0)
            MAC_MARK(kTlPoolFirst);
        const int wgrp = __builtin_amdgcn_readfirstlane(ent >> 8);
        const int wit = __builtin_amdgcn_readfirstlane(ent & 0xff);
        // The item's group: plan record and queries.
        const int32_t *rec = a.w.gplan + (int64_t)wgrp * kPlanWords;
        if (threadIdx.x < kPlanCodes + G)
            s_plan[threadIdx.x] =
                (int)ld_wt_u32(reinterpret_cast<const uint32_t *>(rec + threadIdx.x));
        const int b2 = wgrp / s.Hkv, g2 = wgrp - b2 * s.Hkv;
        QueryStage<D, G> q2;
        q2.request(a, b2, g2);
        __syncthreads();  // plan words in LDS; s_q and s_qb free
        q2.store(s_q);
        if constexpr (AS::kMfma)
            q2.store_b(s_qb, s.qscale);
        const int ce = __builtin_amdgcn_readfirstlane(s_plan[kPlanE]);
        const int csg = __builtin_amdgcn_readfirstlane(s_plan[kPlanStart]);
        const int cn = __builtin_amdgcn_readfirstlane(s_plan[kPlanN]);
        const bool cready = __builtin_amdgcn_readfirstlane(s_plan[kPlanReady]) != 0;
        int ccode[G], cst[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            ccode[j] = __builtin_amdgcn_readfirstlane(s_plan[kPlanCodes + j]);
            cst[j] = code_start(ccode[j]);
        }
        const GroupItems cgi(csg, ce, s.r, s.F, true, s.cmin);
        __syncthreads();  // queries in LDS
        ItemCtx<T, D, G, kPaged> ictx(a, b2, g2, true);
        ictx.queries_from_lds(s_q, s_qb, s.qscale);
        int t0, t1;
        cgi.item(wit, t0, t1);
        const bool sink_item = cgi.is_sink(wit);
        int sti[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            sti[j] = sink_item ? 0 : cst[j];
        item_issue<T, D, G, kPaged>(a, ictx, t0, t1, bufs, false);
        float *po = a.w.part_o + ((int64_t)wgrp * kItemsPerGroupMax + wit) * G * D;
        float *pl = a.w.part_l + ((int64_t)wgrp * kItemsPerGroupMax + wit) * G;
        item_finish<T, D, G, kPaged>(a, ictx, t0, t1, sti, lds, bufs, [&](int j, int dim, float o, float lg) {
            st_wt(po + j * D + dim, o);
            if (dim == 0)
                st_wt(pl + j, lg);
        });
        wait_vmem();
        __syncthreads();
        if (count_item(wgrp, cn)) {
            float c_l[MP::NPK], c_o[MP::NPK][2];
            load_cached<T, D, G, kBlock>(
                a, wgrp, [&](int j) { return code_slot(ccode[j], s.r, s.K); }, c_l, c_o);
            merge(wgrp, cn, csg, ce, cready, c_l, c_o);
        }
    }
    MAC_MARK(kTlExit);
    MAC_NOTE(kTlNotePool, n_taken);
}

// ---------------------------------------------------------------------------
// Rectify-append: slot t mod K of every (b, h) receives the pre-RoPE query,
// the rectified summary (natural-log lse) and pos t = pos[b] + pos_offset.
template <class T, int D, bool kWarm>
__global__ __launch_bounds__(D) void append_kernel(StepArgs a, int32_t pos_offset)
{
    using S = typename T::S;
    const Shape &s = a.s;
    const int bh = blockIdx.x, b = bh / s.Hq, h = bh - b * s.Hq;
    const int grp = b * s.Hkv + h / s.G;
    const int dim = threadIdx.x;
    // Decode steps append at the position the merge recorded for the group
    // (-1: none); the warm-up at the workspace's prompt positions.
    const int t = kWarm ? a.pos[b] + pos_offset : a.w.app_pos[grp];
    if (t < 0 || t >= s.T)
        return;
    const int slot = t % s.K;
    const int64_t ri = ((int64_t)bh * s.K + slot) * D + dim;
    ((S *)a.q_ring)[ri] = ((const S *)a.qtilde)[b * a.qt_sb + h * a.qt_sh + dim];
    a.o_ring[ri] = a.w.rect_o[(int64_t)bh * D + dim];
    if (dim == 0)
        a.lse_ring[(int64_t)bh * s.K + slot] = a.w.rect_l[bh] * kLn2;
    if (h % s.G == 0) {
        // The merge of the step recorded whether the group restarts.
        ring_append_pos(a, grp, t, !kWarm && a.w.restart[grp] != 0, dim, D);
    }
}

// Rounding of an fp64 value to the K/V element type, once: fp32 directly;
// bf16 through fp32 rounded to odd, which then rounds to nearest even
// exactly as the fp64 value would.
__device__ inline float kv_round(double x, F32) { return (float)x; }
__device__ inline uint16_t kv_round(double x, BF16)
{
    float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if ((double)f != x)
        u |= 1u;  // round to odd
    return (uint16_t)(bf16_bits(__uint_as_float(u)) & 0xffffu);
}
__device__ inline double kv_value(float x) { return (double)x; }
__device__ inline double kv_value(uint16_t x) { return (double)__uint_as_float((uint32_t)x << 16); }

// New token's K and V into the cache with RoPE applied to K on the way,
// and optionally the post-RoPE query: workgroup (b, x) with x < Hkv a KV
// head, x >= Hkv query head x - Hkv; thread j rotates pair (2j, 2j + 1) by
// pos[b] * base^(-2j/d), in fp64, rounded once ("Match (1)" of the blog
// describes the rotation as independent 2x2 rotations of such pairs).
template <class T, int D>
__global__ __launch_bounds__(D / 2) void append_kv_kernel(Shape s, const void *k_new,
                                                          const void *v_new, const void *q_tilde,
                                                          float *q_out, const int32_t *pos,
                                                          double base, void *k_cache,
                                                          void *v_cache)
{
#pragma clang fp contract(off)
    using S = typename T::S;
    const int nh = s.Hkv + (q_out ? s.Hq : 0);
    const int b = blockIdx.x / nh, x = blockIdx.x - b * nh;
    const int j = threadIdx.x;
    const int m = pos[b];
    if (m < 0 || m >= s.T)
        return;
    double c = 1.0, sn = 0.0;
    if (base > 0.0) {
        const double ang = (double)m * pow(base, -2.0 * j / D);
        sincos(ang, &sn, &c);
    }
    const bool kv = x < s.Hkv;
    const int h = kv ? x : x - s.Hkv;
    const S *src = kv ? (const S *)k_new + ((int64_t)b * s.Hkv + h) * D
                      : (const S *)q_tilde + ((int64_t)b * s.Hq + h) * D;
    const double x0 = kv_value(src[2 * j]), x1 = kv_value(src[2 * j + 1]);
    const double y0 = x0 * c - x1 * sn, y1 = x0 * sn + x1 * c;
    if (!kv) {
        float *qo = q_out + ((int64_t)b * s.Hq + h) * D;
        qo[2 * j] = (float)y0;
        qo[2 * j + 1] = (float)y1;
        return;
    }
    int64_t row;
    if (s.page_table) {
        const int page = s.page_table[(int64_t)b * s.max_pages + (m >> s.page_shift)];
        row = (int64_t)page * s.kv_sb + (int64_t)(m & ((1 << s.page_shift) - 1)) * s.kv_st;
    } else {
        row = (int64_t)b * s.kv_sb + (int64_t)m * s.kv_st;
    }
    row += (int64_t)h * s.kv_sh;
    S *kd = (S *)k_cache + row;
    kd[2 * j] = kv_round(y0, T());
    kd[2 * j + 1] = kv_round(y1, T());
    const S *vs = (const S *)v_new + ((int64_t)b * s.Hkv + h) * D;
    S *vd = (S *)v_cache + row;
    vd[2 * j] = vs[2 * j];
    vd[2 * j + 1] = vs[2 * j + 1];
}

template <class S>
__global__ void ring_reset_kernel(int64_t n_q, S *__restrict__ q_ring,
                                  float *__restrict__ o_ring, int64_t n_l,
                                  float *__restrict__ lse_ring, int64_t n_p,
                                  int32_t *__restrict__ pos_ring,
                                  int32_t *__restrict__ ctrl, int64_t n_keys,
                                  unsigned long long *__restrict__ keys, int64_t n_sync,
                                  unsigned long long *__restrict__ sync, int64_t n_tag,
                                  unsigned long long *__restrict__ skeys, int64_t n_gs,
                                  uint32_t *__restrict__ grp_sync, int64_t n_ep,
                                  int32_t *__restrict__ ring_epoch, int64_t n_pool,
                                  unsigned long long *__restrict__ pool)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = i0; i < n_q; i += stride) {
        q_ring[i] = S(0);
        o_ring[i] = 0.f;
    }
    for (int64_t i = i0; i < n_l; i += stride)
        lse_ring[i] = -INFINITY;
    for (int64_t i = i0; i < n_p; i += stride)
        pos_ring[i] = -1;
    for (int64_t i = i0; i < n_keys; i += stride)
        keys[i * kKeyStride] = ~0ull;
    for (int64_t i = i0; i < n_sync; i += stride)
        sync[i] = i == kSyncMagicWord ? kSyncMagic : 0ull;
    // Tagged words: no stale word may hold a tag of the restarted epochs.
    for (int64_t i = i0; i < n_tag; i += stride)
        skeys[i] = 0;
    for (int64_t i = i0; i < n_gs; i += stride)
        grp_sync[i] = 0;
    for (int64_t i = i0; i < n_ep; i += stride)
        ring_epoch[i] = 0;
    // Pool words and entries: no stale entry may carry a restarted epoch's tag.
    for (int64_t i = i0; i < n_pool; i += stride)
        pool[i] = 0;
    if (i0 < 16)
        ctrl[i0] = 0;
}

// Streaming read of n16 16-byte words (a measurement of the achievable read
// bandwidth, the denominator the decode kernels are compared with): each
// thread keeps kReadUnroll loads in flight, folds every word into one value,
// and stores it only when it equals a value the data never produces, so no
// load can be dropped and nothing is written in practice.
constexpr int kReadUnroll = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                              int64_t n16, float *sink)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x7fc00123u)
        sink[blockIdx.x] = __uint_as_float(acc);
}

}  // namespace

// Resident workgroups per CU of a kernel (cached per kernel, LDS size and
// device).
static int resident_per_cu(const void *fn, size_t lds)
{
    struct Entry {
        const void *fn;
        size_t lds;
        int dev, n;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == fn && cache[i].lds == lds && cache[i].dev == dev)
            return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kBlock, lds) != hipSuccess || n < 1)
        n = 1;
    if (used < 64)
        cache[used++] = Entry{fn, lds, dev, n};
    return n;
}

}  // namespace mac
