// C ABI of libmac_attention.so: argument validation, workspace layout,
// stream/event ordering of the decode step.  Declared in mac_attention.h.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "mac_attention.h"
#include "mac_internal.h"

namespace mac {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int elem_bytes(int32_t dtype) { return dtype == MAC_DTYPE_F32 ? 4 : 2; }

// Fewest splits per head of the single launch's match (largest units).
static int single_min_nsplit(int K, int dtype, int D)
{
    const int slots = single_slots(elem_bytes(dtype), D);
    return (K + slots - 1) / slots;
}

// 64-bit words of the single launch's tagged key region (key words per
// group are at most kMaxSingleUnits).
static int64_t single_tag_words(int B, int Hkv)
{
    return (int64_t)kKeyReps * B * Hkv * kMaxSingleUnits;
}

// 64-bit words of the single launch's two pool sets.
static int64_t single_pool_words(int B, int Hkv)
{
    return 2 * ((int64_t)kPoolLine + (int64_t)B * Hkv * kItemsPerGroupMax);
}

WsLayout ws_layout(int B, int Hq, int Hkv, int D, int K, int T, int dtype, bool single)
{
    WsLayout L;
    const int G = Hq / Hkv;
    L.nsplit = (K + kSlotsPerSplit - 1) / kSlotsPerSplit;
    L.max_items = (int64_t)B * Hkv * kItemsPerGroupMax;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t BH = (size_t)B * Hq, BG = (size_t)B * Hkv;
    // Two sets of per-head match keys (the two-kernel form alternates them).
    L.keys = take(2 * BH * kKeyStride * sizeof(unsigned long long));
    L.ctx = take((size_t)B * 4);
    L.dec_slot = take(BH * 4);
    L.grp_begin = take(BG * 4);
    L.grp_count = take(BG * 4);
    L.grp_start = take(BG * 4);
    L.ctrl = take(64);
    L.sync = take((size_t)kSyncWords * sizeof(unsigned long long));
    L.part_o = take((size_t)L.max_items * G * D * 4);
    L.part_l = take((size_t)L.max_items * G * 4);
    L.rect_o = take(BH * D * 4);
    L.rect_l = take(BH * 4);
    L.ring_epoch = take(BG * 4);
    L.restart = take(BG * 4);
    L.app_pos = take(BG * 4);
    // The single-launch regions come last, so the layout without them is a
    // prefix of the layout with them.
    L.skeys = L.grp_sync = L.pool = L.gplan = 0;
    if (single) {
        L.skeys = take(single_tag_words(B, Hkv) * sizeof(unsigned long long));
        L.grp_sync = take(BG * kGrpStride * sizeof(uint32_t));
        L.pool = take(single_pool_words(B, Hkv) * sizeof(unsigned long long));
        L.gplan = take(BG * kPlanWords * sizeof(int32_t));
    }
    L.total = off;
    return L;
}

WsPtrs ws_ptrs(void *base, const WsLayout &L)
{
    char *c = (char *)base;
    WsPtrs w;
    w.keys = (unsigned long long *)(c + L.keys);
    w.ctx = (int32_t *)(c + L.ctx);
    w.dec_slot = (int32_t *)(c + L.dec_slot);
    w.grp_begin = (int32_t *)(c + L.grp_begin);
    w.grp_count = (int32_t *)(c + L.grp_count);
    w.grp_start = (int32_t *)(c + L.grp_start);
    w.ctrl = (int32_t *)(c + L.ctrl);
    w.sync = (unsigned long long *)(c + L.sync);
    w.part_o = (float *)(c + L.part_o);
    w.part_l = (float *)(c + L.part_l);
    w.rect_o = (float *)(c + L.rect_o);
    w.rect_l = (float *)(c + L.rect_l);
    w.ring_epoch = (int32_t *)(c + L.ring_epoch);
    w.restart = (int32_t *)(c + L.restart);
    w.app_pos = (int32_t *)(c + L.app_pos);
    w.skeys = L.skeys ? (unsigned long long *)(c + L.skeys) : nullptr;
    w.grp_sync = L.grp_sync ? (uint32_t *)(c + L.grp_sync) : nullptr;
    w.pool = L.pool ? (unsigned long long *)(c + L.pool) : nullptr;
    w.gplan = L.gplan ? (int32_t *)(c + L.gplan) : nullptr;
    return w;
}

}  // namespace mac

using namespace mac;

// match, attend (+plan), merge, append, single launch
constexpr int kStages = MAC_PROFILE_STAGES;

// Marks a live handle; mac_release clears it before freeing.
constexpr uint64_t kHandleMagic = 0x4d41432d48414e44ull;

struct mac_handle {
    uint64_t magic = kHandleMagic;
    mac_params p;
    Shape s;
    WsLayout L;
    WsPtrs w;
    void *ws;
    mac_rings rings;
    bool fused_append;
    int form;  // kFormThree, kFormOne or kFormTwo
    int32_t wpg, upg, nkw, done_shift, unit_slots, nsplit;  // single-launch geometry
    const int32_t *epoch = nullptr;  // bound by mac_bind_epochs
    hipEvent_t ev_main = nullptr, ev_aux = nullptr;
    // Per-stage timing events: prof[(step * kStages + stage) * 2 + {0,1}].
    std::vector<hipEvent_t> prof;
    int32_t prof_cap = 0, prof_n = 0;
};

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A handle made by mac_init_rings and not yet released.  (A released
// handle's memory is freed; its cleared mark is what a stale pointer most
// likely still shows, but reading it is not guaranteed.)
static bool handle_ok(const mac_handle *h) { return h && h->magic == kHandleMagic; }

// Host-side validation of the parameter block; fills the kernel shape.
static mac_status check_params(const mac_params *p, Shape *s)
{
    if (!p)
        return MAC_ERR_INVALID_ARG;
    if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 ||
        p->n_q_heads % p->n_kv_heads != 0 || p->ring_k < 1 ||
        p->band_r < 0 || p->kv_capacity < 1 ||
        (p->flags & ~(MAC_FLAG_FUSED_APPEND | MAC_FLAG_SPLIT_STAGES |
                      MAC_FLAG_SINGLE_LAUNCH | MAC_FLAG_MATCH_FILTER |
                      MAC_FLAG_TWO_STAGES)) != 0 ||
        __builtin_popcount(p->flags & (MAC_FLAG_SPLIT_STAGES | MAC_FLAG_SINGLE_LAUNCH |
                                       MAC_FLAG_TWO_STAGES)) > 1 ||
        !isfinite(p->tau) || !isfinite(p->sm_scale) || p->sm_scale < 0.f ||
        p->front_sink < 0 || p->front_sink > kMaxFrontSink ||
        (p->thresh_mode != MAC_THRESH_ONE_MINUS_TAU &&
         p->thresh_mode != MAC_THRESH_TAU) ||
        p->max_context < 0 || p->min_context < 0)
        return MAC_ERR_INVALID_ARG;
    const int G = p->n_q_heads / p->n_kv_heads;
    if ((p->head_dim != 64 && p->head_dim != 128) ||
        (p->kv_dtype != MAC_DTYPE_F32 && p->kv_dtype != MAC_DTYPE_BF16) ||
        (G != 1 && G != 2 && G != 4 && G != 8))
        return MAC_ERR_UNSUPPORTED;
    // Sizes are addressed with 32-bit work items and head indices; the
    // planner keeps its per-head and per-group tables in LDS.
    if ((int64_t)p->kv_capacity > (1 << 30) || p->ring_k > (1 << 24))
        return MAC_ERR_INVALID_ARG;
    // One head's query ring is addressed with 32-bit byte offsets.
    if ((int64_t)p->ring_k * p->head_dim * elem_bytes(p->kv_dtype) >= ((int64_t)1 << 31))
        return MAC_ERR_UNSUPPORTED;
    if ((int64_t)p->batch * p->n_q_heads > 8192 ||
        plan_lds_bytes(p->batch, p->n_q_heads, p->n_kv_heads) > 48 * 1024)
        return MAC_ERR_UNSUPPORTED;
    // The planner's work offsets (tokens plus a per-item cost, summed over
    // the KV groups of a step) are 32-bit.
    if ((int64_t)p->batch * p->n_kv_heads * ((int64_t)p->kv_capacity + (int64_t)kItemCost * kItemsPerGroupMax) >=
        ((int64_t)1 << 31))
        return MAC_ERR_UNSUPPORTED;
    // Paged K/V: a power-of-two page size of at least 16 tokens, a page
    // table whose rows cover kv_capacity.
    const bool paged = p->page_size != 0;
    int shift = 0;
    if (paged) {
        while (shift < 30 && (1 << shift) < p->page_size)
            ++shift;
        if (p->page_size < 16 || p->page_size > (1 << 20) || (1 << shift) != p->page_size ||
            p->max_pages < 1 || !p->page_table || ((uintptr_t)p->page_table & 3u) ||
            (int64_t)p->max_pages * p->page_size < p->kv_capacity ||
            (int64_t)p->batch * p->max_pages >= ((int64_t)1 << 31))
            return MAC_ERR_INVALID_ARG;
    } else if (p->max_pages != 0 || p->page_table) {
        return MAC_ERR_INVALID_ARG;
    }
    int64_t st = p->kv_stride_t, sh = p->kv_stride_h, sb = p->kv_stride_b;
    if (st == 0 && sh == 0 && sb == 0) {
        // Dense [B, Hkv, T, d]; paged [pages, Hkv, page_size, d].
        const int64_t rows = paged ? p->page_size : p->kv_capacity;
        st = p->head_dim;
        sh = st * rows;
        sb = sh * p->n_kv_heads;
    }
    if (st < p->head_dim || sh < 0 || sb < 0)
        return MAC_ERR_INVALID_ARG;
    const int eb = elem_bytes(p->kv_dtype);
    if ((st * eb) % 16 || (sh * eb) % 16 || (sb * eb) % 16)
        return MAC_ERR_MISALIGNED;
    // Entry refused above the maximum context (0: no limit).
    if (p->max_context > 0 && p->kv_capacity > p->max_context)
        return MAC_ERR_CONTEXT_TOO_LONG;
    if (s) {
        const int d = p->head_dim;
        const double scale = p->sm_scale != 0.f ? (double)p->sm_scale
                                                : 1.0 / sqrt((double)d);
        const double f = p->thresh_mode == MAC_THRESH_TAU
                             ? (double)p->tau
                             : 1.0 - (double)p->tau;
        s->B = p->batch;
        s->Hq = p->n_q_heads;
        s->Hkv = p->n_kv_heads;
        s->G = G;
        s->D = d;
        s->dtype = p->kv_dtype;
        s->K = p->ring_k;
        s->r = p->band_r;
        s->T = p->kv_capacity;
        s->F = p->front_sink;
        s->min_ctx = p->min_context;
        s->cmin = (int64_t)p->batch * p->n_kv_heads > kSingleLaunchMaxGroups ? kChunkMinShiftWide
                                                                              : kChunkMinShift;
        s->page_shift = paged ? shift : 0;
        s->max_pages = paged ? p->max_pages : 0;
        s->page_table = paged ? p->page_table : nullptr;
        s->kv_sb = sb;
        s->kv_sh = sh;
        s->kv_st = st;
        s->qscale = (float)(scale * 1.4426950408889634);
        s->thresh2 = (float)(2.0 * d * f * f);
    }
    return MAC_OK;
}

// Shapes the single launch handles: positions that the tagged keys encode,
// match units that its LDS holds.
static bool single_launch_supported(const Shape &s)
{
    return s.T <= kSingleMaxPositions &&
           s.G * single_min_nsplit(s.K, s.dtype, s.D) <= kMaxSingleUnits;
}

// The forms of a step: match, plan + attention and merge as three kernels;
// all in one launch; the match kernel, then plan, attention and merge in one.
enum { kFormThree = 0, kFormOne = 1, kFormTwo = 2 };

// The form a handle for p runs, before the residency check of
// mac_init_rings: the one its flags force, else by the number of KV groups
// (kSingleLaunchMaxGroups, kTwoStageMaxGroups), where shapes allow.  The
// one- and two-kernel forms need positions that the tagged keys and pool
// entries encode; the one-launch form also needs the group's match units to
// fit its LDS.
static int step_form(const mac_params *p, const Shape &s)
{
    if (p->flags & MAC_FLAG_SPLIT_STAGES)
        return kFormThree;
    const bool two_ok = s.T <= kSingleMaxPositions;
    if (p->flags & MAC_FLAG_TWO_STAGES)
        return two_ok ? kFormTwo : kFormThree;
    if (p->flags & MAC_FLAG_SINGLE_LAUNCH)
        return kFormOne;  // mac_init_rings rejects shapes it does not handle
    const int NG = s.B * s.Hkv;
    if (NG <= kSingleLaunchMaxGroups && single_launch_supported(s))
        return kFormOne;
    return two_ok && NG <= kTwoStageMaxGroups ? kFormTwo : kFormThree;
}

static WsLayout layout_for(const mac_params *p, const Shape &s)
{
    return ws_layout(s.B, s.Hq, s.Hkv, s.D, s.K, s.T, s.dtype, step_form(p, s) != kFormThree);
}

extern "C" {

size_t mac_workspace_bytes(const mac_params *p)
{
    Shape s;
    if (check_params(p, &s) != MAC_OK)
        return 0;
    return layout_for(p, s).total;
}

mac_status mac_ring_bytes(const mac_params *p, size_t out[4])
{
    Shape s;
    const mac_status st = check_params(p, &s);
    if (st != MAC_OK)
        return st;
    if (!out)
        return MAC_ERR_INVALID_ARG;
    const size_t n = (size_t)s.B * s.Hq * s.K;
    out[0] = n * s.D * elem_bytes(s.dtype);
    out[1] = n * s.D * 4;
    out[2] = n * 4;
    out[3] = (size_t)s.B * s.Hkv * s.K * 4;
    return MAC_OK;
}

const char *mac_status_string(mac_status s)
{
    switch (s) {
    case MAC_OK:
        return "ok";
    case MAC_ERR_INVALID_ARG:
        return "invalid argument";
    case MAC_ERR_UNSUPPORTED:
        return "unsupported head_dim / dtype / GQA group";
    case MAC_ERR_HIP:
        return "HIP runtime error";
    case MAC_ERR_WORKSPACE_TOO_SMALL:
        return "workspace too small";
    case MAC_ERR_MISALIGNED:
        return "buffer or row not 16-byte aligned";
    case MAC_ERR_CONTEXT_TOO_LONG:
        return "kv_capacity exceeds max_context";
    case MAC_ERR_NOT_INITIALIZED:
        return "handle not initialised by mac_init_rings (or released)";
    case MAC_ERR_SCRATCH_TOO_SMALL:
        return "shape needs more than the static scratch (MAC_NOALLOC_SCRATCH_BYTES, 48 MiB)";
    }
    return "unknown status";
}

// log2 of a valid minimum chunk (a power of two in [64, 2^20]), else -1.
static int chunk_shift_of(int32_t min_chunk)
{
    for (int sh = kChunkMinShift; sh <= 20; ++sh)
        if (min_chunk == (1 << sh))
            return sh;
    return -1;
}

int32_t mac_min_chunk_tokens(const mac_params *p)
{
    Shape s;
    return check_params(p, &s) == MAC_OK ? 1 << s.cmin : -1;
}

int32_t mac_chunk_tokens(int32_t s, int32_t e, int32_t min_chunk)
{
    const int cm = chunk_shift_of(min_chunk);
    return (s < 0 || e < s || cm < 0) ? -1 : RangeSplit::chunk_for(s, e, cm);
}

int32_t mac_partition(int32_t s, int32_t e, int32_t r, int32_t min_chunk, int32_t *t0,
                      int32_t *t1, int32_t cap)
{
    const int cm = chunk_shift_of(min_chunk);
    if (s < 0 || e < s || r < 0 || cap < 0 || cm < 0)
        return -1;
    const RangeSplit rs(s, e, r, RangeSplit::chunk_shift_for(s, e, cm));
    for (int i = 0; i < rs.n && i < cap; ++i)
        rs.item(i, t0[i], t1[i]);
    return rs.n;
}

int32_t mac_group_items(int32_t s, int32_t e, int32_t r, int32_t front_sink, int32_t min_chunk,
                        int32_t *t0, int32_t *t1, int32_t *n_before_split, int32_t cap)
{
    const int cm = chunk_shift_of(min_chunk);
    if (s < 0 || e < s || r < 0 || cap < 0 || front_sink < 0 || front_sink > kMaxFrontSink ||
        cm < 0)
        return -1;
    const GroupItems gi(s, e, r, front_sink, true, cm);
    for (int i = 0; i < gi.n && i < cap; ++i)
        gi.item(i, t0[i], t1[i]);
    if (n_before_split)
        *n_before_split = gi.n_before_split();
    return gi.n;
}

#define MAC_HIP(call)                      \
    do {                                   \
        if ((call) != hipSuccess)          \
            return MAC_ERR_HIP;            \
    } while (0)

// Kernel arguments common to every call on a shape and workspace.
static StepArgs base_args(const Shape &s, const WsLayout &L, const WsPtrs &w)
{
    StepArgs a;
    memset(&a, 0, sizeof a);
    a.s = s;
    a.w = w;
    a.max_items = L.max_items;
    a.nsplit = L.nsplit;
    a.dyn_pool = 1;
    return a;
}

// Full decode into the workspace at ws (laid out without the single-launch
// regions): the plan + attention kernel, then the merge.
static mac_status full_decode_on(const Shape &s, void *ws, const float *q, const void *k_cache,
                                 const void *v_cache, const int32_t *pos, float *out,
                                 float *out_lse, hipStream_t st)
{
    const WsLayout L = ws_layout(s.B, s.Hq, s.Hkv, s.D, s.K, s.T, s.dtype, false);
    StepArgs a = base_args(s, L, ws_ptrs(ws, L));
    a.mode = kPlanFull;
    // A caller's workspace may be fresh: full decode splits its (regular)
    // work statically and claims nothing.
    a.dyn_pool = 0;
    a.pos = pos;
    a.q = q;
    a.q_sh = s.D;
    a.q_sb = (int64_t)s.Hq * s.D;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.out_lse = out_lse;
    MAC_HIP(launch_attend(a, st));
    MAC_HIP(launch_merge(a, st));
    return MAC_OK;
}

mac_status mac_full_decode(const mac_params *p, const float *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *pos, float *out, float *out_lse,
                           void *workspace, size_t ws_bytes, void *stream)
{
    Shape s;
    mac_status rc = check_params(p, &s);
    if (rc != MAC_OK)
        return rc;
    if (!q || !k_cache || !v_cache || !pos || !out || !workspace)
        return MAC_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(workspace))
        return MAC_ERR_MISALIGNED;
    // The documented size is required; full decode uses only the regions
    // that precede the single-launch ones.
    if (ws_bytes < layout_for(p, s).total)
        return MAC_ERR_WORKSPACE_TOO_SMALL;
    return full_decode_on(s, workspace, q, k_cache, v_cache, pos, out, out_lse,
                          (hipStream_t)stream);
}

mac_status mac_full_decode_noalloc(const mac_params *p, const float *q,
                                   const void *k_cache, const void *v_cache,
                                   const int32_t *pos, float *out, float *out_lse,
                                   void *stream)
{
    Shape s;
    mac_status rc = check_params(p, &s);
    if (rc != MAC_OK)
        return rc;
    if (!q || !k_cache || !v_cache || !pos || !out)
        return MAC_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return MAC_ERR_MISALIGNED;
    if (ws_layout(s.B, s.Hq, s.Hkv, s.D, s.K, s.T, s.dtype, false).total >
        MAC_NOALLOC_SCRATCH_BYTES)
        return MAC_ERR_SCRATCH_TOO_SMALL;
    void *scr = nullptr;
    MAC_HIP(noalloc_scratch(&scr));
    return full_decode_on(s, scr, q, k_cache, v_cache, pos, out, out_lse, (hipStream_t)stream);
}

mac_status mac_init_rings(const mac_params *p, const mac_rings *rings,
                          void *workspace, size_t ws_bytes,
                          const void *warm_qtilde, const float *warm_q,
                          int32_t n_warm, const int32_t *ctx_len,
                          const void *k_cache, const void *v_cache,
                          void *stream, mac_handle **out)
{
    Shape s;
    mac_status rc = check_params(p, &s);
    if (rc != MAC_OK)
        return rc;
    if (!rings || !out || !workspace || !rings->q_ring || !rings->o_ring ||
        !rings->lse_ring || !rings->pos_ring)
        return MAC_ERR_INVALID_ARG;
    if (!aligned16(rings->q_ring) || !aligned16(rings->o_ring) ||
        !aligned16(workspace))
        return MAC_ERR_MISALIGNED;
    if (((p->flags & MAC_FLAG_SINGLE_LAUNCH) && !single_launch_supported(s)) ||
        ((p->flags & MAC_FLAG_TWO_STAGES) && s.T > kSingleMaxPositions))
        return MAC_ERR_UNSUPPORTED;
    const WsLayout L = layout_for(p, s);
    if (ws_bytes < L.total)
        return MAC_ERR_WORKSPACE_TOO_SMALL;
    if (n_warm < 0 || n_warm > s.K)
        return MAC_ERR_INVALID_ARG;
    if (n_warm > 0) {
        if (!warm_qtilde || !warm_q || !ctx_len || !k_cache || !v_cache)
            return MAC_ERR_INVALID_ARG;
        if (!aligned16(warm_qtilde) || !aligned16(warm_q) ||
            !aligned16(k_cache) || !aligned16(v_cache))
            return MAC_ERR_MISALIGNED;
        for (int b = 0; b < s.B; ++b)
            if (ctx_len[b] < n_warm || ctx_len[b] > s.T)
                return MAC_ERR_INVALID_ARG;
    }
    hipStream_t st = (hipStream_t)stream;
    const WsPtrs w = ws_ptrs(workspace, L);

    mac_handle *h = new (std::nothrow) mac_handle();
    if (!h)
        return MAC_ERR_INVALID_ARG;
    h->p = *p;
    h->s = s;
    h->L = L;
    h->w = w;
    h->ws = workspace;
    h->rings = *rings;
    h->fused_append = (p->flags & MAC_FLAG_FUSED_APPEND) != 0;
    h->form = step_form(p, s);
    if (h->form != kFormThree) {
        // wpg workgroups per KV group, all resident at once, each with at
        // least one key word to store.
        const int NG = s.B * s.Hkv;
        const int resident = step_resident_workgroups(s);
        h->wpg = resident / NG < kGroupWorkgroups ? resident / NG : kGroupWorkgroups;
        // Match units: the small size when one unit per workgroup covers
        // the group's ring rows with it, the large size otherwise.
        const int eb = elem_bytes(s.dtype);
        const int64_t want = h->wpg > 0 ? ((int64_t)s.G * s.K + h->wpg - 1) / h->wpg : 1;
        int size = 0;
        while (size < kUnitSizes - 1 && want > step_unit_slots(eb, s.D, size))
            ++size;
        h->unit_slots = step_unit_slots(eb, s.D, size);
        h->nsplit = (s.K + h->unit_slots - 1) / h->unit_slots;
        h->upg = s.G * h->nsplit;
        h->nkw = h->upg > h->wpg ? h->upg : h->wpg;
        int sh = 0;
        while ((1 << sh) < NG)
            ++sh;
        h->done_shift = sh;
        if (h->wpg < 1) {
            if (p->flags & (MAC_FLAG_SINGLE_LAUNCH | MAC_FLAG_TWO_STAGES)) {
                delete h;
                return MAC_ERR_UNSUPPORTED;
            }
            h->form = kFormThree;
        }
    }
    if (hipEventCreateWithFlags(&h->ev_main, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_aux, hipEventDisableTiming) != hipSuccess) {
        mac_release(h);
        return MAC_ERR_HIP;
    }
    const int64_t n_tag = L.skeys ? single_tag_words(s.B, s.Hkv) : 0;
    const int64_t n_pool = L.pool ? single_pool_words(s.B, s.Hkv) : 0;
    if (launch_ring_reset(s, rings->q_ring, rings->o_ring, rings->lse_ring,
                          rings->pos_ring, w, n_tag, n_pool, st) != hipSuccess) {
        mac_release(h);
        return MAC_ERR_HIP;
    }
    if (n_warm > 0) {
        int32_t *d_ctx = w.ctx;
        if (hipMemcpyAsync(d_ctx, ctx_len, sizeof(int32_t) * s.B,
                           hipMemcpyHostToDevice, st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess) {
            mac_release(h);
            return MAC_ERR_HIP;
        }
        StepArgs a = base_args(s, L, w);
        a.s.r = 0;  // the warm summary covers all of [0, t - r]
        a.mode = kPlanInit;
        a.pos = d_ctx;
        a.k = k_cache;
        a.v = v_cache;
        a.q_sh = (int64_t)n_warm * s.D;
        a.q_sb = (int64_t)s.Hq * a.q_sh;
        a.qt_sh = a.q_sh;
        a.qt_sb = a.q_sb;
        a.q_ring = rings->q_ring;
        a.o_ring = rings->o_ring;
        a.lse_ring = rings->lse_ring;
        a.pos_ring = rings->pos_ring;
        for (int wi = 0; wi < n_warm && rc == MAC_OK; ++wi) {
            // Warm position t = ctx_len - W + wi; its summary covers [0, t - r].
            const int32_t t_off = wi - n_warm;
            a.end_offset = t_off - s.r;
            a.q = warm_q + (int64_t)wi * s.D;
            a.qtilde = (const char *)warm_qtilde +
                       (int64_t)wi * s.D * elem_bytes(s.dtype);
            if (launch_attend(a, st) != hipSuccess ||
                launch_merge(a, st) != hipSuccess ||
                launch_append(a, t_off, st) != hipSuccess)
                rc = MAC_ERR_HIP;
        }
        if (rc != MAC_OK) {
            mac_release(h);
            return rc;
        }
    }
    *out = h;
    return MAC_OK;
}

mac_status mac_decode_step(mac_handle *h, const void *qtilde, const float *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *pos, float *out, float *out_lse,
                           int32_t *match_p, float *match_d2,
                           void *main_stream, void *aux_stream)
{
    if (!handle_ok(h))
        return MAC_ERR_NOT_INITIALIZED;
    if (!qtilde || !q || !k_cache || !v_cache || !pos || !out)
        return MAC_ERR_INVALID_ARG;
    if (!aligned16(qtilde) || !aligned16(q) || !aligned16(k_cache) ||
        !aligned16(v_cache))
        return MAC_ERR_MISALIGNED;
    const Shape &s = h->s;
    hipStream_t ms = (hipStream_t)main_stream;
    hipStream_t as = aux_stream ? (hipStream_t)aux_stream : ms;
    const bool split = as != ms && !h->fused_append;

    StepArgs a = base_args(s, h->L, h->w);
    a.mode = kPlanMatch;
    a.pos = pos;
    a.qtilde = qtilde;
    a.qt_sh = s.D;
    a.qt_sb = (int64_t)s.Hq * s.D;
    a.q = q;
    a.q_sh = s.D;
    a.q_sb = (int64_t)s.Hq * s.D;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.out_lse = out_lse;
    a.match_p = match_p;
    a.match_d2 = match_d2;
    a.q_ring = h->rings.q_ring;
    a.o_ring = h->rings.o_ring;
    a.lse_ring = h->rings.lse_ring;
    a.pos_ring = h->rings.pos_ring;
    a.append_fused = h->fused_append ? 1 : 0;
    a.epoch = h->epoch;
    a.match_filter = (h->p.flags & MAC_FLAG_MATCH_FILTER) ? 1 : 0;
    a.wpg = h->wpg;
    a.upg = h->upg;
    a.nkw = h->nkw;
    a.done_shift = h->done_shift;
    a.nsplit = h->form == kFormOne ? h->nsplit : h->L.nsplit;
    a.key_parity = h->form == kFormTwo ? 1 : 0;
    a.group_only = h->form == kFormTwo ? 1 : 0;
    a.unit_slots = h->unit_slots;
    a.pool_cap = s.B * s.Hkv * kItemsPerGroupMax;

    const bool prof = h->prof_n < h->prof_cap;
    hipEvent_t *pe = prof ? &h->prof[(size_t)h->prof_n * kStages * 2] : nullptr;
#define MAC_STAGE(idx, stream_, launch)                          \
    do {                                                         \
        if (pe)                                                  \
            MAC_HIP(hipEventRecord(pe[2 * (idx)], stream_));     \
        MAC_HIP(launch);                                         \
        if (pe)                                                  \
            MAC_HIP(hipEventRecord(pe[2 * (idx) + 1], stream_)); \
    } while (0)

    // The previous rectify-append of this handle must have finished before
    // the rings are read and the workspace is reused.
    if (split)
        MAC_HIP(hipStreamWaitEvent(ms, h->ev_aux, 0));
    if (h->form == kFormThree) {
        MAC_STAGE(0, ms, launch_match(a, ms));
        MAC_STAGE(1, ms, launch_attend(a, ms));
        MAC_STAGE(2, ms, launch_merge(a, ms));
    } else if (h->form == kFormTwo) {
        MAC_STAGE(0, ms, launch_match(a, ms));
        MAC_STAGE(4, ms, launch_step(a, ms));
    } else {
        MAC_STAGE(4, ms, launch_step(a, ms));
    }
    if (!h->fused_append) {
        if (split) {
            MAC_HIP(hipEventRecord(h->ev_main, ms));
            MAC_HIP(hipStreamWaitEvent(as, h->ev_main, 0));
        }
        MAC_STAGE(3, as, launch_append(a, 0, as));
        if (split)
            MAC_HIP(hipEventRecord(h->ev_aux, as));
    }
#undef MAC_STAGE
    if (prof)
        ++h->prof_n;
    return MAC_OK;
}

mac_status mac_append_kv(const mac_params *p, const void *k_new, const void *v_new,
                         const void *q_tilde, float *q_out, const int32_t *pos, double rope_base,
                         void *k_cache, void *v_cache, void *stream)
{
    Shape s;
    mac_status rc = check_params(p, &s);
    if (rc != MAC_OK)
        return rc;
    if (!k_new || !v_new || !pos || !k_cache || !v_cache || (!q_tilde) != (!q_out) ||
        !(rope_base >= 0.0) || !isfinite(rope_base))
        return MAC_ERR_INVALID_ARG;
    const int eb = elem_bytes(s.dtype);
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)q_tilde | (uintptr_t)k_cache |
         (uintptr_t)v_cache) % eb || ((uintptr_t)q_out & 3u))
        return MAC_ERR_MISALIGNED;
    MAC_HIP(launch_append_kv(s, k_new, v_new, q_tilde, q_out, pos, rope_base, k_cache, v_cache,
                             (hipStream_t)stream));
    return MAC_OK;
}

mac_status mac_bind_epochs(mac_handle *h, const int32_t *epoch)
{
    if (!handle_ok(h))
        return MAC_ERR_NOT_INITIALIZED;
    if (epoch && ((uintptr_t)epoch & 3u))
        return MAC_ERR_INVALID_ARG;
    h->epoch = epoch;
    return MAC_OK;
}

mac_status mac_join_aux(mac_handle *h, void *stream)
{
    if (!handle_ok(h))
        return MAC_ERR_NOT_INITIALIZED;
    MAC_HIP(hipStreamWaitEvent((hipStream_t)stream, h->ev_aux, 0));
    return MAC_OK;
}

mac_status mac_read_device_status(const mac_params *p, void *workspace,
                                  void *stream, int32_t *flags)
{
    Shape s;
    mac_status rc = check_params(p, &s);
    if (rc != MAC_OK)
        return rc;
    if (!workspace || !flags)
        return MAC_ERR_INVALID_ARG;
    const WsLayout L = ws_layout(s.B, s.Hq, s.Hkv, s.D, s.K, s.T, s.dtype, false);
    const WsPtrs w = ws_ptrs(workspace, L);
    hipStream_t st = (hipStream_t)stream;
    int32_t v = 0;
    unsigned long long sy[3] = {0, 0, 0};
    static const int32_t zero = 0;
    static const unsigned long long zero64 = 0;
    MAC_HIP(hipMemcpyAsync(&v, w.ctrl + kCtrlStatus, sizeof v, hipMemcpyDeviceToHost, st));
    MAC_HIP(hipMemcpyAsync(sy, w.sync, sizeof sy, hipMemcpyDeviceToHost, st));
    MAC_HIP(hipStreamSynchronize(st));
    MAC_HIP(hipMemcpyAsync(w.ctrl + kCtrlStatus, &zero, sizeof zero, hipMemcpyHostToDevice, st));
    // The latched time-outs exist only on a workspace whose rings were
    // initialised (a full-decode-only workspace never holds the marker).
    const bool init = sy[kSyncMagicWord] == kSyncMagic;
    if (init)
        MAC_HIP(hipMemcpyAsync(w.sync + kSyncSticky, &zero64, sizeof zero64,
                               hipMemcpyHostToDevice, st));
    MAC_HIP(hipStreamSynchronize(st));
    *flags = v | (init ? (int32_t)sy[kSyncSticky] : 0);
    return MAC_OK;
}

mac_status mac_profile_start(mac_handle *h, int32_t n_steps)
{
    if (!handle_ok(h))
        return MAC_ERR_NOT_INITIALIZED;
    if (n_steps < 0)
        return MAC_ERR_INVALID_ARG;
    for (hipEvent_t e : h->prof)
        (void)hipEventDestroy(e);
    h->prof.assign((size_t)n_steps * kStages * 2, nullptr);
    // Timing-only events: no system-scope fence (cache write-back) at
    // record time, which would otherwise add microseconds to every stage.
    for (auto &e : h->prof)
        MAC_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    h->prof_cap = n_steps;
    h->prof_n = 0;
    return MAC_OK;
}

mac_status mac_profile_read(mac_handle *h, double ms[MAC_PROFILE_STAGES], int32_t *n)
{
    if (!handle_ok(h))
        return MAC_ERR_NOT_INITIALIZED;
    if (!ms || !n)
        return MAC_ERR_INVALID_ARG;
    for (int k = 0; k < kStages; ++k)
        ms[k] = 0.0;
    MAC_HIP(hipDeviceSynchronize());
    // Stages that ran (and recorded their events) on this handle.
    const bool three = h->form == kFormThree;
    bool ran[kStages] = {h->form != kFormOne, three, three, !h->fused_append, !three};
    for (int i = 0; i < h->prof_n; ++i)
        for (int k = 0; k < kStages; ++k) {
            if (!ran[k])
                continue;
            hipEvent_t a = h->prof[((size_t)i * kStages + k) * 2];
            hipEvent_t b = h->prof[((size_t)i * kStages + k) * 2 + 1];
            float t = 0.f;
            MAC_HIP(hipEventElapsedTime(&t, a, b));
            ms[k] += t;
        }
    *n = h->prof_n;
    h->prof_cap = 0;
    h->prof_n = 0;
    return MAC_OK;
}

mac_status mac_timeline_read(mac_handle *h, void *host, size_t bytes)
{
    if (!handle_ok(h))
        return MAC_ERR_NOT_INITIALIZED;
    if (!host)
        return MAC_ERR_INVALID_ARG;
    const Shape &s = h->s;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess)
        e = s.dtype == MAC_DTYPE_BF16 && s.D == 128  ? timeline_read_bf16_128(host, bytes)
            : s.dtype == MAC_DTYPE_BF16              ? timeline_read_bf16_64(host, bytes)
            : s.D == 128                             ? timeline_read_f32_128(host, bytes)
                                                     : timeline_read_f32_64(host, bytes);
    if (e == hipErrorNotSupported)
        return MAC_ERR_UNSUPPORTED;
    return e == hipSuccess ? MAC_OK : MAC_ERR_HIP;
}

mac_status mac_stream_read(const void *buf, size_t bytes, float *sink, int32_t grid,
                           void *stream)
{
    if (!buf || !sink || grid < 1 || bytes < 16)
        return MAC_ERR_INVALID_ARG;
    if (!aligned16(buf) || ((uintptr_t)sink & 3u))
        return MAC_ERR_MISALIGNED;
    MAC_HIP(launch_stream_read(buf, bytes, sink, grid, (hipStream_t)stream));
    return MAC_OK;
}

mac_status mac_release(mac_handle *h)
{
    if (!handle_ok(h))
        return MAC_ERR_NOT_INITIALIZED;
    h->magic = 0;
    if (h->ev_main)
        (void)hipEventDestroy(h->ev_main);
    if (h->ev_aux)
        (void)hipEventDestroy(h->ev_aux);
    for (hipEvent_t e : h->prof)
        if (e)
            (void)hipEventDestroy(e);
    delete h;
    return MAC_OK;
}

}  // extern "C"
