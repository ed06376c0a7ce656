// HIP kernels of the MAC-Attention decode step for gfx950 (MI355X).
//
// One kernel per stage of the step described in the MAC-Attention blog
// ("MAC-Attention: Match-Amend-Complete attention reuse ... (MLSys 2026)"),
// section "Paper version: the K1/K2/K3 micro-pipeline":
//   match   -- L2 nearest neighbour of the pre-RoPE query in the query ring
//              ("Match (1)-(3)"), one 64-slot split per workgroup;
//   plan    -- final argmin, hit test, per-(request, KV group) token range
//              and the device work list (the span-proportional allocator:
//              every group gets one work item per kChunk tokens of its range);
//   attend  -- split-KV decode attention over the work list: each item
//              loads its K/V rows once for all G query heads of the group;
//   combine -- fixed-order log-domain merge of the partials with the cached
//              summary ("Complete"); also yields the rectified summary;
//   append  -- writes the query and rectified summary into slot m mod K.
//
// The path is HBM-bound (about 4 flop per KV byte for G = 4): attention and
// match use VALU with 16-byte coalesced row loads, a K/V row (256 B for
// d=128 bf16 or d=64 fp32) being spread over one 16-lane DPP row.
#include <math.h>

#include "mac_attention.h"
#include "mac_internal.h"

namespace mac {
namespace {

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

// Sum over the W consecutive lanes of a row (W a power of two <= 64); every
// lane of the row receives the total.
template <int W>
__device__ inline float row_sum(float v)
{
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
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

// Merge (l, o) <- (l, o) (+) (lb, ob) for log2-domain summaries; the empty
// summary (-inf) is an exact identity.
__device__ inline void merge_into(float &l, float &o, float lb, float ob)
{
    if (lb == -INFINITY)
        return;
    if (l == -INFINITY) {
        l = lb;
        o = ob;
        return;
    }
    const float M = fmaxf(l, lb);
    const float ln = M + log2f(exp2f(l - M) + exp2f(lb - M));
    o = exp2f(l - ln) * o + exp2f(lb - ln) * ob;
    l = ln;
}

// ---------------------------------------------------------------------------
// Match.  Grid (nsplit, B*Hq).  Each LPR-lane row of a wave computes the
// squared distance of one ring slot; the workgroup keeps the smallest key
//   key = float_bits(D) << 32 | (0xffffffff - p)
// (non-negative floats order like their bits; equal D prefers larger p).
template <class T, int D>
__global__ __launch_bounds__(kBlock) void match_kernel(
    const typename T::S *__restrict__ qt, int64_t qt_sb, int64_t qt_sh,
    const typename T::S *__restrict__ q_ring, const int32_t *__restrict__ pos_ring,
    const int32_t *__restrict__ pos, int Hq, int K, int T_cap, int nsplit,
    unsigned long long *__restrict__ keys)
{
    constexpr int EPL = T::EPL, LPR = D / EPL, RPB = kBlock / LPR;
    constexpr int U = kSlotsPerSplit / RPB;
    static_assert(U >= 1 && U * RPB == kSlotsPerSplit, "split shape");
    const int bh = blockIdx.y, b = bh / Hq, h = bh - b * Hq;
    const int lane = threadIdx.x % LPR, row = threadIdx.x / LPR;
    const int m = pos[b];
    const bool m_ok = m >= 0 && m < T_cap;

    float qv[EPL];
    unpack<T>(load16(qt + b * qt_sb + h * qt_sh + lane * EPL), qv);
    const typename T::S *ring = q_ring + (int64_t)bh * K * D + lane * EPL;
    const int32_t *pr = pos_ring + (int64_t)b * K;

    uint4 raw[U];
    int p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = blockIdx.x * kSlotsPerSplit + u * RPB + row;
        if (k < K) {
            raw[u] = load16(ring + (int64_t)k * D);
            p[u] = pr[k];
        } else {
            raw[u] = make_uint4(0, 0, 0, 0);
            p[u] = -1;
        }
    }
    unsigned long long best = ~0ull;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float r[EPL];
        unpack<T>(raw[u], r);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float df = qv[e] - r[e];
            acc = fmaf(df, df, acc);
        }
        acc = row_sum<LPR>(acc);
        const int pu = p[u];
        const bool valid = m_ok && pu >= 0 && pu >= m - K && pu <= m - 1;
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
    __shared__ unsigned long long sm[kBlock / 64];
    if ((threadIdx.x & 63) == 0)
        sm[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 1; i < kBlock / 64; ++i)
            best = umin64(best, sm[i]);
        keys[(int64_t)bh * nsplit + blockIdx.x] = best;
    }
}

// ---------------------------------------------------------------------------
// Single workgroup.  Decision per (b, h), token range per (b, g), exclusive
// scan of the per-group item counts, then the work list.
__global__ __launch_bounds__(1024) void plan_kernel(
    const unsigned long long *__restrict__ keys, int nsplit,
    const int32_t *__restrict__ pos, int32_t mode, int32_t end_offset, int B,
    int Hq, int Hkv, int G, int K, int r, int T_cap, float thresh2,
    int32_t *__restrict__ dec_start, int32_t *__restrict__ dec_slot,
    int32_t *__restrict__ grp_begin, int32_t *__restrict__ grp_count,
    int32_t *__restrict__ ctrl, WorkItem *__restrict__ items,
    int64_t max_items, int32_t *__restrict__ match_p, float *__restrict__ match_d2)
{
    __shared__ int32_t s_scan[1024];
    __shared__ int32_t s_bad;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int off = (mode == kPlanInit) ? end_offset : 0;
    if (tid == 0)
        s_bad = 0;
    __syncthreads();

    for (int bh = tid; bh < B * Hq; bh += nt) {
        const int b = bh / Hq;
        const int e = pos[b] + off;
        const bool ok = (mode == kPlanInit) ? (e < T_cap) : (e >= 0 && e < T_cap);
        if (!ok)
            s_bad = 1;
        int start = 0, slot = -1;
        if (mode == kPlanMatch) {
            unsigned long long key = ~0ull;
            for (int s = 0; s < nsplit; ++s)
                key = umin64(key, keys[(int64_t)bh * nsplit + s]);
            const bool any = key != ~0ull;
            const float d2 = any ? __uint_as_float((uint32_t)(key >> 32)) : INFINITY;
            const int p = any ? (int)(0xffffffffu - (uint32_t)key) : -1;
            const bool hit = ok && any && d2 < thresh2;
            if (hit) {
                start = p - r + 1 > 0 ? p - r + 1 : 0;
                slot = p % K;
            }
            if (match_p)
                match_p[bh] = hit ? p : -1;
            if (match_d2)
                match_d2[bh] = d2;
        }
        dec_start[bh] = start;
        dec_slot[bh] = slot;
    }
    __syncthreads();

    int carry = 0;
    const int n_grp = B * Hkv;
    const int r_split = (mode == kPlanInit) ? 0 : r;
    for (int base = 0; base < n_grp; base += nt) {
        const int grp = base + tid;
        int cnt = 0;
        if (grp < n_grp) {
            const int b = grp / Hkv, g = grp - b * Hkv;
            const int e = pos[b] + off;
            if (e >= 0 && e < T_cap) {
                int s = e;
                for (int j = 0; j < G; ++j) {
                    const int st = dec_start[b * Hq + g * G + j];
                    s = st < s ? st : s;
                }
                cnt = RangeSplit(s, e, r_split).n;
            }
        }
        s_scan[tid] = cnt;
        __syncthreads();
        for (int o = 1; o < nt; o <<= 1) {
            const int v = tid >= o ? s_scan[tid - o] : 0;
            __syncthreads();
            s_scan[tid] += v;
            __syncthreads();
        }
        if (grp < n_grp) {
            grp_begin[grp] = carry + s_scan[tid] - cnt;
            grp_count[grp] = cnt;
        }
        carry += s_scan[nt - 1];
        __syncthreads();
    }

    for (int grp = 0; grp < n_grp; ++grp) {
        const int cnt = grp_count[grp];
        if (cnt == 0)
            continue;
        const int begin = grp_begin[grp];
        const int b = grp / Hkv, g = grp - b * Hkv;
        const int e = pos[b] + off;
        int s = e;
        for (int j = 0; j < G; ++j) {
            const int st = dec_start[b * Hq + g * G + j];
            s = st < s ? st : s;
        }
        const RangeSplit rs(s, e, r_split);
        for (int i = tid; i < cnt; i += nt) {
            if (begin + i >= max_items)
                break;
            WorkItem w;
            w.bg = grp;
            rs.item(i, w.t0, w.t1);
            w.pad = 0;
            items[begin + i] = w;
        }
    }
    if (tid == 0) {
        ctrl[0] = carry < max_items ? carry : (int32_t)max_items;
        ctrl[1] = s_bad ? MAC_DEV_BAD_POSITION : 0;
    }
}

// ---------------------------------------------------------------------------
// Attention over the work list.  Each workgroup loops over items; within an
// item, LPR-lane row `row` handles tokens t0 + i*RPB + row.  A K/V row is
// loaded once (16 B per lane) and serves the G query heads of the group from
// registers.  Per-row online softmax in log2 units; the RPB row states are
// combined in LDS in a fixed order into one partial (o, log2-lse) per head.
template <class T, int D, int G>
__global__ __launch_bounds__(kBlock) void attend_kernel(
    const WorkItem *__restrict__ items, const int32_t *__restrict__ ctrl,
    const float *__restrict__ q, int64_t q_sb, int64_t q_sh,
    const typename T::S *__restrict__ Kc, const typename T::S *__restrict__ Vc,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_st,
    const int32_t *__restrict__ dec_start, int Hq, int Hkv, float qscale,
    float *__restrict__ part_o, float *__restrict__ part_l)
{
    constexpr int EPL = T::EPL, LPR = D / EPL, RPB = kBlock / LPR;
    constexpr int NI = kChunk / RPB;
    constexpr int NB = NI < 8 ? NI : 8;
    static_assert(NI % NB == 0, "chunk shape");
    __shared__ float sm_m[RPB][G];
    __shared__ float sm_l[RPB][G];
    __shared__ float sm_acc[RPB][G][D];

    const int lane = threadIdx.x % LPR, row = threadIdx.x / LPR;
    const int n_items = ctrl[0];
    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const WorkItem w = items[it];
        const int b = w.bg / Hkv, g = w.bg - b * Hkv;

        float qr[G][EPL];
        int st[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float *qp = q + b * q_sb + (int64_t)(g * G + j) * q_sh + lane * EPL;
#pragma unroll
            for (int e4 = 0; e4 < EPL; e4 += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(qp + e4);
                qr[j][e4 + 0] = v.x * qscale;
                qr[j][e4 + 1] = v.y * qscale;
                qr[j][e4 + 2] = v.z * qscale;
                qr[j][e4 + 3] = v.w * qscale;
            }
            st[j] = dec_start[b * Hq + g * G + j];
        }
        const typename T::S *kb = Kc + b * kv_sb + g * kv_sh + lane * EPL;
        const typename T::S *vb = Vc + b * kv_sb + g * kv_sh + lane * EPL;

        float mrun[G], lrun[G], acc[G][EPL];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            mrun[j] = -INFINITY;
            lrun[j] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[j][e] = 0.f;
        }

#pragma unroll 1
        for (int blk = 0; blk < NI / NB; ++blk) {
            uint4 kr[NB], vr[NB];
            int tt[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int t = w.t0 + (blk * NB + i) * RPB + row;
                tt[i] = t;
                if (t < w.t1) {
                    kr[i] = load16(kb + (int64_t)t * kv_st);
                    vr[i] = load16(vb + (int64_t)t * kv_st);
                } else {
                    kr[i] = make_uint4(0, 0, 0, 0);
                    vr[i] = make_uint4(0, 0, 0, 0);
                }
            }
            float s[NB][G];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                float kf[EPL];
                unpack<T>(kr[i], kf);
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        a = fmaf(qr[j][e], kf[e], a);
                    s[i][j] = a;
                }
            }
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const float v = row_sum<LPR>(s[i][j]);
                    s[i][j] = (tt[i] < w.t1 && tt[i] >= st[j]) ? v : -INFINITY;
                }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float bm = s[0][j];
#pragma unroll
                for (int i = 1; i < NB; ++i)
                    bm = fmaxf(bm, s[i][j]);
                const float mn = fmaxf(mrun[j], bm);
                const bool live = mn != -INFINITY;
                const float alpha = live ? exp2f(mrun[j] - mn) : 1.f;
                float lsum = lrun[j] * alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[j][e] *= alpha;
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const float pi = live ? exp2f(s[i][j] - mn) : 0.f;
                    s[i][j] = pi;
                    lsum += pi;
                }
                lrun[j] = lsum;
                mrun[j] = mn;
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                float vf[EPL];
                unpack<T>(vr[i], vf);
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[j][e] = fmaf(s[i][j], vf[e], acc[j][e]);
            }
        }

        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                sm_m[row][j] = mrun[j];
                sm_l[row][j] = lrun[j];
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                sm_acc[row][j][lane * EPL + e] = acc[j][e];
        __syncthreads();
        for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
            const int j = idx / D, dim = idx - j * D;
            float M = -INFINITY;
#pragma unroll 8
            for (int rr = 0; rr < RPB; ++rr)
                M = fmaxf(M, sm_m[rr][j]);
            float o = 0.f, L = -INFINITY;
            if (M != -INFINITY) {
                float ls = 0.f, os = 0.f;
#pragma unroll 8
                for (int rr = 0; rr < RPB; ++rr) {
                    const float c = exp2f(sm_m[rr][j] - M);
                    ls = fmaf(c, sm_l[rr][j], ls);
                    os = fmaf(c, sm_acc[rr][j][dim], os);
                }
                o = os / ls;
                L = M + log2f(ls);
            }
            part_o[((int64_t)it * G + j) * D + dim] = o;
            if (dim == 0)
                part_l[(int64_t)it * G + j] = L;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Combine.  One workgroup of D threads per (b, h), thread = output dim.
// Partials of the group's items are folded in item order into
//   A  = items before the rectify split sp = e - r + 1,
//   Bt = items from sp on,
// then R = C (+) A with C the cached summary of the matched slot (empty on a
// miss) and out = R (+) Bt.  R is the rectified summary of [0, e - r].
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(
    const WorkItem *__restrict__ items, const int32_t *__restrict__ grp_begin,
    const int32_t *__restrict__ grp_count, const int32_t *__restrict__ pos,
    int32_t end_offset, int32_t allow_negative, int Hq, int Hkv, int G, int K,
    int r, int T_cap, const float *__restrict__ part_o,
    const float *__restrict__ part_l, const int32_t *__restrict__ dec_slot,
    const float *__restrict__ o_ring, const float *__restrict__ lse_ring,
    float *__restrict__ out, float *__restrict__ out_lse,
    float *__restrict__ rect_o, float *__restrict__ rect_l)
{
    const int bh = blockIdx.x, b = bh / Hq, h = bh - b * Hq;
    const int g = h / G, j = h - g * G, grp = b * Hkv + g;
    const int dim = threadIdx.x;
    const int e = pos[b] + end_offset;
    const bool ok = e < T_cap && (allow_negative || e >= 0);
    if (!ok) {
        if (out)
            out[(int64_t)bh * D + dim] = NAN;
        if (out_lse && dim == 0)
            out_lse[bh] = NAN;
        rect_o[(int64_t)bh * D + dim] = 0.f;
        if (dim == 0)
            rect_l[bh] = -INFINITY;
        return;
    }
    const int sp = e - r + 1;
    const int begin = grp_begin[grp], cnt = grp_count[grp];
    float la = -INFINITY, oa = 0.f, lb = -INFINITY, ob = 0.f;
    int i = 0;
    for (; i + 4 <= cnt; i += 4) {
        int t0[4];
        float li[4], oi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t ix = (int64_t)begin + i + u;
            t0[u] = items[ix].t0;
            li[u] = part_l[ix * G + j];
            oi[u] = part_o[(ix * G + j) * D + dim];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (t0[u] < sp)
                merge_into(la, oa, li[u], oi[u]);
            else
                merge_into(lb, ob, li[u], oi[u]);
        }
    }
    for (; i < cnt; ++i) {
        const int64_t ix = (int64_t)begin + i;
        const float li = part_l[ix * G + j];
        const float oi = part_o[(ix * G + j) * D + dim];
        if (items[ix].t0 < sp)
            merge_into(la, oa, li, oi);
        else
            merge_into(lb, ob, li, oi);
    }
    float lr = -INFINITY, orr = 0.f;
    const int slot = dec_slot[bh];
    if (slot >= 0) {
        lr = lse_ring[(int64_t)bh * K + slot] * kLog2e;
        orr = o_ring[((int64_t)bh * K + slot) * D + dim];
    }
    merge_into(lr, orr, la, oa);
    float lo = lr, oo = orr;
    merge_into(lo, oo, lb, ob);
    if (out)
        out[(int64_t)bh * D + dim] = oo;
    if (out_lse && dim == 0)
        out_lse[bh] = lo * kLn2;
    rect_o[(int64_t)bh * D + dim] = orr;
    if (dim == 0)
        rect_l[bh] = lr;
}

// ---------------------------------------------------------------------------
// Rectify-append: slot t mod K of every (b, h) receives the pre-RoPE query,
// the rectified summary (natural-log lse) and pos t = pos[b] + pos_offset.
template <class T, int D>
__global__ __launch_bounds__(D) void append_kernel(
    const int32_t *__restrict__ pos, int32_t pos_offset, int T_cap,
    const typename T::S *__restrict__ qt, int64_t qt_sb, int64_t qt_sh,
    const float *__restrict__ rect_o, const float *__restrict__ rect_l, int Hq,
    int K, typename T::S *__restrict__ q_ring, float *__restrict__ o_ring,
    float *__restrict__ lse_ring, int32_t *__restrict__ pos_ring)
{
    const int bh = blockIdx.x, b = bh / Hq, h = bh - b * Hq;
    const int dim = threadIdx.x;
    const int t = pos[b] + pos_offset;
    if (t < 0 || t >= T_cap)
        return;
    const int slot = t % K;
    const int64_t ri = ((int64_t)bh * K + slot) * D + dim;
    q_ring[ri] = qt[b * qt_sb + h * qt_sh + dim];
    o_ring[ri] = rect_o[(int64_t)bh * D + dim];
    if (dim == 0)
        lse_ring[(int64_t)bh * K + slot] = rect_l[bh] * kLn2;
    if (h == 0 && dim == 0)
        pos_ring[(int64_t)b * K + slot] = t;
}

template <class S>
__global__ void ring_reset_kernel(int64_t n_q, S *__restrict__ q_ring,
                                  float *__restrict__ o_ring, int64_t n_l,
                                  float *__restrict__ lse_ring, int64_t n_p,
                                  int32_t *__restrict__ pos_ring,
                                  int32_t *__restrict__ ctrl)
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
    if (i0 == 0) {
        ctrl[0] = 0;
        ctrl[1] = 0;
    }
}

int attend_grid(int64_t max_items)
{
    const int64_t cap = 2048;
    return (int)(max_items < cap ? (max_items > 0 ? max_items : 1) : cap);
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers with (dtype, D, G) dispatch.

hipError_t launch_match(const Shape &s, const void *qtilde, int64_t qt_sb,
                        int64_t qt_sh, const void *q_ring,
                        const int32_t *pos_ring, const int32_t *pos,
                        const WsPtrs &w, int nsplit, hipStream_t st)
{
    const dim3 grid(nsplit, s.B * s.Hq), block(kBlock);
#define MAC_MATCH(TT, DD)                                                     \
    hipLaunchKernelGGL((match_kernel<TT, DD>), grid, block, 0, st,            \
                       (const TT::S *)qtilde, qt_sb, qt_sh,                   \
                       (const TT::S *)q_ring, pos_ring, pos, s.Hq, s.K, s.T,  \
                       nsplit, w.keys)
    if (s.dtype == MAC_DTYPE_BF16 && s.D == 128)
        MAC_MATCH(BF16, 128);
    else if (s.dtype == MAC_DTYPE_BF16 && s.D == 64)
        MAC_MATCH(BF16, 64);
    else if (s.dtype == MAC_DTYPE_F32 && s.D == 128)
        MAC_MATCH(F32, 128);
    else
        MAC_MATCH(F32, 64);
#undef MAC_MATCH
    return hipGetLastError();
}

hipError_t launch_plan(const Shape &s, int32_t mode, int32_t end_offset,
                       const int32_t *pos, const WsPtrs &w, int nsplit,
                       int64_t max_items, int32_t *match_p, float *match_d2,
                       hipStream_t st)
{
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, w.keys,
                       nsplit, pos, mode, end_offset, s.B, s.Hq, s.Hkv, s.G,
                       s.K, s.r, s.T, s.thresh2, w.dec_start, w.dec_slot,
                       w.grp_begin, w.grp_count, w.ctrl, w.items, max_items,
                       match_p, match_d2);
    return hipGetLastError();
}

template <class T, int D>
static void attend_g(const Shape &s, const float *q, int64_t q_sb,
                     int64_t q_sh, const void *k, const void *v,
                     const WsPtrs &w, int grid, hipStream_t st)
{
#define MAC_ATT(GG)                                                           \
    hipLaunchKernelGGL((attend_kernel<T, D, GG>), dim3(grid), dim3(kBlock), 0, \
                       st, w.items, w.ctrl, q, q_sb, q_sh,                    \
                       (const typename T::S *)k, (const typename T::S *)v,    \
                       s.kv_sb, s.kv_sh, s.kv_st, w.dec_start, s.Hq, s.Hkv,   \
                       s.qscale, w.part_o, w.part_l)
    switch (s.G) {
    case 1:
        MAC_ATT(1);
        break;
    case 2:
        MAC_ATT(2);
        break;
    case 4:
        MAC_ATT(4);
        break;
    default:
        MAC_ATT(8);
        break;
    }
#undef MAC_ATT
}

hipError_t launch_attend(const Shape &s, const float *q, int64_t q_sb,
                         int64_t q_sh, const void *k, const void *v,
                         const WsPtrs &w, int64_t max_items, hipStream_t st)
{
    const int grid = attend_grid(max_items);
    if (s.dtype == MAC_DTYPE_BF16 && s.D == 128)
        attend_g<BF16, 128>(s, q, q_sb, q_sh, k, v, w, grid, st);
    else if (s.dtype == MAC_DTYPE_BF16 && s.D == 64)
        attend_g<BF16, 64>(s, q, q_sb, q_sh, k, v, w, grid, st);
    else if (s.dtype == MAC_DTYPE_F32 && s.D == 128)
        attend_g<F32, 128>(s, q, q_sb, q_sh, k, v, w, grid, st);
    else
        attend_g<F32, 64>(s, q, q_sb, q_sh, k, v, w, grid, st);
    return hipGetLastError();
}

hipError_t launch_combine(const Shape &s, int32_t end_offset,
                          int32_t allow_neg, const int32_t *pos,
                          const WsPtrs &w, const float *o_ring,
                          const float *lse_ring, float *out, float *out_lse,
                          hipStream_t st)
{
#define MAC_COMB(DD)                                                          \
    hipLaunchKernelGGL((combine_kernel<DD>), dim3(s.B * s.Hq), dim3(DD), 0,   \
                       st, w.items, w.grp_begin, w.grp_count, pos, end_offset, \
                       allow_neg, s.Hq, s.Hkv, s.G, s.K, s.r, s.T, w.part_o,  \
                       w.part_l, w.dec_slot, o_ring, lse_ring, out, out_lse,  \
                       w.rect_o, w.rect_l)
    if (s.D == 128)
        MAC_COMB(128);
    else
        MAC_COMB(64);
#undef MAC_COMB
    return hipGetLastError();
}

hipError_t launch_append(const Shape &s, int32_t pos_offset,
                         const int32_t *pos, const void *qtilde, int64_t qt_sb,
                         int64_t qt_sh, const WsPtrs &w, void *q_ring,
                         float *o_ring, float *lse_ring, int32_t *pos_ring,
                         hipStream_t st)
{
#define MAC_APP(TT, DD)                                                       \
    hipLaunchKernelGGL((append_kernel<TT, DD>), dim3(s.B * s.Hq), dim3(DD), 0, \
                       st, pos, pos_offset, s.T, (const TT::S *)qtilde, qt_sb, \
                       qt_sh, w.rect_o, w.rect_l, s.Hq, s.K, (TT::S *)q_ring, \
                       o_ring, lse_ring, pos_ring)
    if (s.dtype == MAC_DTYPE_BF16 && s.D == 128)
        MAC_APP(BF16, 128);
    else if (s.dtype == MAC_DTYPE_BF16 && s.D == 64)
        MAC_APP(BF16, 64);
    else if (s.dtype == MAC_DTYPE_F32 && s.D == 128)
        MAC_APP(F32, 128);
    else
        MAC_APP(F32, 64);
#undef MAC_APP
    return hipGetLastError();
}

hipError_t launch_ring_reset(const Shape &s, void *q_ring, float *o_ring,
                             float *lse_ring, int32_t *pos_ring,
                             int32_t *ctrl, hipStream_t st)
{
    const int64_t n_q = (int64_t)s.B * s.Hq * s.K * s.D;
    const int64_t n_l = (int64_t)s.B * s.Hq * s.K;
    const int64_t n_p = (int64_t)s.B * s.K;
    int64_t blocks = (n_q + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (s.dtype == MAC_DTYPE_BF16)
        hipLaunchKernelGGL(ring_reset_kernel<uint16_t>, dim3((int)blocks),
                           dim3(256), 0, st, n_q, (uint16_t *)q_ring, o_ring,
                           n_l, lse_ring, n_p, pos_ring, ctrl);
    else
        hipLaunchKernelGGL(ring_reset_kernel<float>, dim3((int)blocks),
                           dim3(256), 0, st, n_q, (float *)q_ring, o_ring, n_l,
                           lse_ring, n_p, pos_ring, ctrl);
    return hipGetLastError();
}

}  // namespace mac
