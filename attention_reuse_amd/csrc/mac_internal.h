// Internal declarations shared by the kernel and host translation units of
// libmac_attention.so.  Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mac {

// Work items: a KV group's token range [s, e] is cut on an absolute grid of
// C tokens, C = kChunkMin * 2^k the smallest such that the range spans at
// most kMaxItemsPerGroup grid cells.  C depends only on the group's own
// range, so a head that misses sees exactly the items of a full decode.
constexpr int kChunkMinShift = 7;
constexpr int kChunkMin = 1 << kChunkMinShift;
constexpr int kMaxItemsPerGroup = 128;
// Ring slots scanned by one match workgroup.
constexpr int kSlotsPerSplit = 64;
// Workgroup size of the match and attention kernels.
constexpr int kBlock = 256;

// Single-launch step: cross-workgroup synchronisation words in the
// workspace, 64-bit, one 128-byte line (kLineU64 words) each:
//   line 0: [0] launch epoch, [1] kSyncMagic once the rings were
//           initialised on the workspace, [2] latched time-outs;
//   lines 1..kBarLines: grid-barrier arrival counters;
//   line 1 + kBarLines: count of completed arrival lines;
//   the kRelLines lines after it: the barrier's release word.
// The per-group arrival counters are 32-bit, kGrpStride words apart.
constexpr int kBarLines = 16;
constexpr int kRelLines = 32;
constexpr int kLineU64 = 16;
constexpr int kSyncWords = kLineU64 * (2 + kBarLines + kRelLines);
constexpr int kGrpStride = 16;
// Default form of the decode step: one launch for at most this many KV
// groups per layer (latency-bound steps), three kernels above (measured on
// MI355X: one launch is ahead at 8 groups, behind at 64 and 128).
constexpr int kSingleLaunchMaxGroups = 16;
// Match keys are kKeyStride words apart (one 128-byte line per head): the
// atomic minima of a head's splits serialise per line, so heads must not
// share one.
constexpr int kKeyStride = 16;
constexpr unsigned long long kSyncMagic = 0x4d41432d53594e43ull;
enum { kSyncEpoch = 0, kSyncMagicWord = 1, kSyncSticky = 2 };

// Plan: work-item partition of one group's token range [s, e].
// Boundaries: s, the multiples of C in (s, e], the rectify split
// sp = e - r + 1 when it falls strictly inside (s, e], and e + 1.
struct RangeSplit {
    // C = 1 << cs; divisions by C are shifts.
    int s, e, cs, c_first, n_grid, sp, has_sp, j_sp, n;
    __host__ __device__ static int chunk_shift_for(int s_, int e_)
    {
        const int span = e_ - s_ + 1;
        int cs = 0;
        while ((kChunkMin << cs) < span && (((span - 1) >> cs) >> kChunkMinShift) + 1 > kMaxItemsPerGroup)
            ++cs;
        return cs + kChunkMinShift;
    }
    __host__ __device__ static int chunk_for(int s_, int e_) { return 1 << chunk_shift_for(s_, e_); }
    __host__ __device__ RangeSplit(int s_, int e_, int r)
    {
        s = s_;
        e = e_;
        cs = chunk_shift_for(s_, e_);
        c_first = (s >> cs) + 1;
        const int c_last = e >> cs;
        n_grid = c_last - c_first + 1;
        if (n_grid < 0)
            n_grid = 0;
        sp = e - r + 1;
        has_sp = (sp > s && sp <= e && (sp & ((1 << cs) - 1)) != 0) ? 1 : 0;
        j_sp = 0;
        if (has_sp) {
            j_sp = ((sp - 1) >> cs) - c_first + 1;
            j_sp = j_sp < 0 ? 0 : (j_sp > n_grid ? n_grid : j_sp);
        }
        n = 1 + n_grid + has_sp;
    }
    __host__ __device__ int boundary(int j) const
    {
        if (has_sp) {
            if (j < j_sp)
                return (c_first + j) << cs;
            if (j == j_sp)
                return sp;
            return (c_first + j - 1) << cs;
        }
        return (c_first + j) << cs;
    }
    __host__ __device__ void item(int i, int &t0, int &t1) const
    {
        t0 = (i == 0) ? s : boundary(i - 1);
        t1 = (i == n - 1) ? e + 1 : boundary(i);
    }
    // Number of leading items that lie before the rectify split sp.
    __host__ __device__ int n_before_split() const
    {
        if (sp <= s)
            return 0;
        if (sp > e)
            return n;
        return (has_sp ? j_sp : (sp >> cs) - c_first) + 1;
    }
};

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
    size_t keys, ctx, dec_slot, grp_begin, grp_count, grp_start, ctrl, sync,
        grp_sync, part_o, part_l, rect_o, rect_l, total;
    int64_t max_items;
    int32_t nsplit;
};

// Plan modes.
enum PlanMode : int32_t {
    kPlanMatch = 0,  // decisions from the match keys (decode step)
    kPlanFull = 1,   // every head misses (full decode)
    kPlanInit = 2,   // full, end = pos[b] + end_offset, a negative end is empty
};

// ctrl words: [0] work items of the latest call, [1] its status flags.
enum { kCtrlItems = 0, kCtrlStatus = 1 };

struct Shape {
    int32_t B, Hq, Hkv, G, D, dtype, K, r, T;
    int64_t kv_sb, kv_sh, kv_st;  // elements
    float qscale;                 // sm_scale * log2(e)
    float thresh2;
};

// Device pointers into the workspace.
struct WsPtrs {
    // [2][B*Hq * kKeyStride] per-head match keys; the three-kernel step
    // uses the first half, the single-launch step alternates by epoch.
    unsigned long long *keys;
    int32_t *ctx;  // [B] prompt lengths during the warm-up
    int32_t *dec_slot, *grp_begin, *grp_count, *grp_start, *ctrl;
    unsigned long long *sync;  // epoch + kBarLines arrival lines
    uint32_t *grp_sync;        // [B*Hkv * kGrpStride] per-group arrivals
    float *part_o, *part_l, *rect_o, *rect_l;
};

// Everything the kernels of one call read or write.
struct StepArgs {
    Shape s;
    WsPtrs w;
    int64_t max_items;
    int32_t nsplit;
    int32_t mode;        // PlanMode
    int32_t end_offset;  // kPlanInit: end = pos[b] + end_offset
    const int32_t *pos;  // [B] device
    // queries (element strides per request and head)
    const void *qtilde;
    int64_t qt_sb, qt_sh;
    const float *q;
    int64_t q_sb, q_sh;
    const void *k, *v;
    // outputs (any may be null except where noted)
    float *out, *out_lse;
    int32_t *match_p;
    float *match_d2;
    // rings: read for the cached summary, written when append_fused
    void *q_ring;
    float *o_ring, *lse_ring;
    int32_t *pos_ring;
    int32_t append_fused;
};

// Bytes of dynamic LDS the planner needs.
size_t plan_lds_bytes(int B, int Hq, int Hkv);

WsLayout ws_layout(int B, int Hq, int Hkv, int D, int K, int T);
WsPtrs ws_ptrs(void *base, const WsLayout &L);

// Kernel launchers (mac_kernels.hip); each returns its launch status.
hipError_t launch_match(const StepArgs &a, hipStream_t st);
// Plan (in every workgroup) + split-KV attention: one partial per item and
// head; workgroup 0 publishes the plan for the merge.
hipError_t launch_attend(const StepArgs &a, hipStream_t st);
// Per-group merge of the partials with the cached summaries; appends to
// the rings itself when append_fused.
hipError_t launch_merge(const StepArgs &a, hipStream_t st);
// The whole decode step (match, plan, attention, merge and, with
// append_fused, the ring append) as one launch of a grid that is resident
// at once.
hipError_t launch_step(const StepArgs &a, hipStream_t st);
// Rectify-append from the workspace staging into the rings; the position of
// request b is pos[b] + pos_offset.
hipError_t launch_append(const StepArgs &a, int32_t pos_offset, hipStream_t st);
hipError_t launch_ring_reset(const Shape &s, void *q_ring, float *o_ring,
                             float *lse_ring, int32_t *pos_ring, const WsPtrs &w,
                             hipStream_t st);
int device_cu_count();

}  // namespace mac
