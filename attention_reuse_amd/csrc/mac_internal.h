// Internal declarations shared by the kernel and host translation units of
// libmac_attention.so.  Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mac {

// Tokens per attention work item.  Item boundaries sit at absolute multiples
// of this (plus the rectify split m-r+1), so a head's partition depends only
// on its own range: a miss and a full decode see the same items.
constexpr int kChunk = 128;
// Ring slots scanned by one match workgroup.
constexpr int kSlotsPerSplit = 64;
// Workgroup size of the match and attention kernels.
constexpr int kBlock = 256;

struct WorkItem {
    int32_t bg;  // b * Hkv + g
    int32_t t0;  // first position (inclusive)
    int32_t t1;  // last position (exclusive)
    int32_t pad;
};

// Plan: work-item partition of one group's token range [s, e].
// Boundaries: s, the multiples of kChunk in (s, e], the rectify split
// sp = e - r + 1 when it falls strictly inside (s, e], and e + 1.
struct RangeSplit {
    int s, e, c_first, n_grid, sp, has_sp, j_sp, n;
    __host__ __device__ RangeSplit(int s_, int e_, int r)
    {
        s = s_;
        e = e_;
        c_first = s / kChunk + 1;
        const int c_last = e / kChunk;
        n_grid = c_last - c_first + 1;
        if (n_grid < 0)
            n_grid = 0;
        sp = e - r + 1;
        has_sp = (sp > s && sp <= e && (sp % kChunk) != 0) ? 1 : 0;
        j_sp = 0;
        if (has_sp) {
            j_sp = (sp - 1) / kChunk - c_first + 1;
            j_sp = j_sp < 0 ? 0 : (j_sp > n_grid ? n_grid : j_sp);
        }
        n = 1 + n_grid + has_sp;
    }
    __host__ __device__ int boundary(int j) const
    {
        if (has_sp) {
            if (j < j_sp)
                return (c_first + j) * kChunk;
            if (j == j_sp)
                return sp;
            return (c_first + j - 1) * kChunk;
        }
        return (c_first + j) * kChunk;
    }
    __host__ __device__ void item(int i, int &t0, int &t1) const
    {
        t0 = (i == 0) ? s : boundary(i - 1);
        t1 = (i == n - 1) ? e + 1 : boundary(i);
    }
};

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
    size_t keys, dec_start, dec_slot, grp_begin, grp_count, ctrl, items,
        part_o, part_l, rect_o, rect_l, total;
    int64_t max_items;
    int32_t nsplit;
};

// Plan modes.
enum PlanMode : int32_t {
    kPlanMatch = 0,  // decisions from the match keys (decode step)
    kPlanFull = 1,   // every head misses (full decode)
    kPlanInit = 2,   // full, end = pos[b] + end_offset, a negative end is empty
};

struct Shape {
    int32_t B, Hq, Hkv, G, D, dtype, K, r, T;
    int64_t kv_sb, kv_sh, kv_st;  // elements
    float qscale;                 // sm_scale * log2(e)
    float thresh2;
};

// Device pointers into the workspace.
struct WsPtrs {
    unsigned long long *keys;
    int32_t *dec_start, *dec_slot, *grp_begin, *grp_count, *ctrl;
    WorkItem *items;
    float *part_o, *part_l, *rect_o, *rect_l;
};

WsLayout ws_layout(int B, int Hq, int Hkv, int D, int K, int T);
WsPtrs ws_ptrs(void *base, const WsLayout &L);

// Kernel launchers (mac_kernels.hip).  Each returns the hipError_t of its
// launch.  q pointers carry (batch, head) strides in elements.
hipError_t launch_match(const Shape &s, const void *qtilde, int64_t qt_sb,
                        int64_t qt_sh, const void *q_ring,
                        const int32_t *pos_ring, const int32_t *pos,
                        const WsPtrs &w, int nsplit, hipStream_t st);
hipError_t launch_plan(const Shape &s, int32_t mode, int32_t end_offset,
                       const int32_t *pos, const WsPtrs &w, int nsplit,
                       int64_t max_items, int32_t *match_p, float *match_d2,
                       hipStream_t st);
hipError_t launch_attend(const Shape &s, const float *q, int64_t q_sb,
                         int64_t q_sh, const void *k, const void *v,
                         const WsPtrs &w, int64_t max_items, hipStream_t st);
hipError_t launch_combine(const Shape &s, int32_t end_offset,
                          int32_t allow_negative, const int32_t *pos,
                          const WsPtrs &w,
                          const float *o_ring, const float *lse_ring,
                          float *out, float *out_lse, hipStream_t st);
hipError_t launch_append(const Shape &s, int32_t pos_offset,
                         const int32_t *pos, const void *qtilde, int64_t qt_sb,
                         int64_t qt_sh, const WsPtrs &w, void *q_ring,
                         float *o_ring, float *lse_ring, int32_t *pos_ring,
                         hipStream_t st);
hipError_t launch_ring_reset(const Shape &s, void *q_ring, float *o_ring,
                             float *lse_ring, int32_t *pos_ring,
                             int32_t *ctrl, hipStream_t st);

}  // namespace mac
