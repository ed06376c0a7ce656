// Internal declarations shared by the kernel and host translation units of
// libmac_attention.so.  Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mac {

// Work items: a KV group's token range [s, e] is cut on an absolute grid of
// C tokens, C = Cmin * 2^k the smallest such that the range spans at most
// kMaxItemsPerGroup grid cells.  C depends only on the group's own range
// and on the shape's minimum Cmin, so a head that misses sees exactly the
// items of a full decode of the same shape.  Cmin is 64 tokens for layers
// of at most kSingleLaunchMaxGroups KV groups (parallelism inside a group
// matters) and 256 above (measured at 64 groups, 8 workgroups each: fewer,
// longer items stream within one workgroup instead of running as two
// items one after the other, and the merge folds fewer partials).
constexpr int kChunkMinShift = 6;
constexpr int kChunkMinShiftWide = 8;
// Work of an item in the attention kernel's balanced split: its tokens plus
// this many (the per-item cost of combining rows and storing the partial).
constexpr int kItemCost = 64;
// The attention kernel splits the first kStaticPct percent of the work
// statically; workgroups that finish their share claim the rest item by item.
constexpr int kStaticPct = 40;
// ... when the plan has at least this many items per workgroup.
constexpr int kPoolItems = 4;
constexpr int kMaxItemsPerGroup = 128;
// Ring slots scanned by one match workgroup.
constexpr int kSlotsPerSplit = 64;
// Ring slots per workgroup of the filtered (half-row) match kernel.
constexpr int kSlotsPerHalvesSplit = 128;
// Single launch: workgroups 0 .. kSpecMax-1 of a group may request the K/V
// of their item before the match has decided the group's range: the item
// they would run if the range kept the span it had at the group's previous
// step, so that the data is in flight during the match.
constexpr int kSpecMax = 24;
// Workgroup size of the match and attention kernels.
constexpr int kBlock = 256;

// Items of one KV group never exceed this (grid cells, the two range ends
// around the rectify split, and the attention-sink item).
constexpr int kItemsPerGroupMax = kMaxItemsPerGroup + 3;
// Largest front sink (tokens that stay out of every reusable summary and
// are attended exactly on every step); the sink is one work item.
constexpr int kMaxFrontSink = 4096;

// Single-launch step.  Each KV group has its own run of workgroups, and data
// crosses workgroups only inside a group:
//   split keys [kKeyReps][groups][key words]: per match unit the key
//       d2_bits << 32 | (0xffffffff - p) with bits 31..24 replaced by the
//       low byte of the launch's tag (positions < 2^24); each workgroup
//       polls the words of its group until all carry the tag.  kKeyReps
//       copies spread the pollers of a group over several lines;
//   partials: the split-KV partial arrays, item i of group grp at index
//       grp * kItemsPerGroupMax + i, handed to the workgroup that completes
//       the group's per-group counter.
// The tag of a launch is 1 + its epoch; the epoch is floor(done / 2^s)
// where `done` grows by exactly 2^s per launch (the merger of group 0 adds
// 2^s - groups + 1, every other group's merger 1), so it is constant during
// a launch until its last group completes, and every workgroup reads it
// before its own group can complete.
constexpr int kKeyReps = 4;
// Ring rows one 256-thread workgroup loads per instruction (one row per
// 16-byte lane group).
__host__ __device__ constexpr int match_rows_per_load(int elem_bytes, int D)
{
    return 4096 / (elem_bytes * D);
}
// Match units of the single launch come in two sizes (0, 1): 4 or 16 loads
// per lane, at most 64 or 256 slots.  The host picks the smallest size whose
// unit covers a workgroup's share of its group's ring rows.  (A unit of 32
// loads per lane would request 512 slots at once, but its registers bring
// the bf16 d = 128 kernel to one wave per SIMD, halving the resident grid.)
// Each size is its own kernel instantiation, so every load of a unit is
// issued without a branch.
constexpr int kUnitSizes = 2;
__host__ __device__ constexpr int step_unit_loads(int size) { return size == 0 ? 4 : 16; }
__host__ __device__ constexpr int step_unit_cap(int size) { return size == 0 ? 64 : 256; }
__host__ __device__ constexpr int step_rows(int elem_bytes, int D, int size)
{
    return step_unit_loads(size) * match_rows_per_load(elem_bytes, D) <= step_unit_cap(size)
               ? step_unit_loads(size)
               : step_unit_cap(size) / match_rows_per_load(elem_bytes, D);
}
__host__ __device__ constexpr int step_unit_slots(int elem_bytes, int D, int size)
{
    return step_rows(elem_bytes, D, size) * match_rows_per_load(elem_bytes, D);
}
__host__ __device__ constexpr int single_slots(int elem_bytes, int D)
{
    return step_unit_slots(elem_bytes, D, kUnitSizes - 1);
}
// Match units per group of the single launch are at most this many (the
// host falls back to three kernels beyond).
constexpr int kMaxSingleUnits = 256;
// Workgroups per group of the single launch (fewer when the device does
// not hold that many resident); those without a match unit store a tagged
// dummy word, so that every workgroup's tag read precedes its group's
// completion.
constexpr int kGroupWorkgroups = 64;
// Per-group line of the single launch, kGrpStride words apart: word 0 the
// arrival counter, word kGrpSpan the span of the group's range at its last
// step (0 = none yet).
constexpr int kGrpStride = 16;
constexpr int kGrpSpan = 1;
// Largest position the tagged keys encode.
constexpr int32_t kSingleMaxPositions = 1 << 24;
// Cross-group pool of the single launch.  A group whose range is cut on a
// grid coarser than the shape's minimum (a long range: a head missed) keeps
// one item per workgroup of its own and publishes the rest; every workgroup
// claims pool items of any group once its own work is done.  Two sets of
// pool words, used by launches of alternating parity (the launch whose last
// group completes resets the other set for the next launch).  Per set: a
// header of kPoolLine words -- [kPoolState] = groups planned << 32 |
// entries published (one atomic add per group), [kPoolHead] = entries
// claimed --
// then one 64-bit entry per published item: (1 + launch epoch) << 32 |
// group << 8 | item.
constexpr int kPoolLine = 32;
enum { kPoolState = 0, kPoolHead = 16 };  // on separate 128-byte lines
// Per-group plan record of the single launch, kPlanWords int32 apart:
// position, range start, item count, readiness, then the G per-head codes;
// written by the group's first workgroup before it publishes pool entries.
constexpr int kPlanWords = 16;
enum { kPlanE = 0, kPlanStart = 1, kPlanN = 2, kPlanReady = 3, kPlanCodes = 4 };
// Synchronisation line of the workspace (64-bit words).
constexpr int kLineU64 = 16;
constexpr int kSyncWords = kLineU64;
// Default form of the decode step: one launch for at most
// kSingleLaunchMaxGroups KV groups per layer (latency-bound steps), the
// match kernel and one launch for the rest up to kTwoStageMaxGroups, three
// kernels above (measured on MI355X: one launch is ahead at 8 groups, two
// kernels at 64, three at 128, where long missed ranges dominate and the
// attention kernel's global balanced split wins).
constexpr int kSingleLaunchMaxGroups = 16;
constexpr int kTwoStageMaxGroups = 64;
// Match keys of the three-kernel step are kKeyStride words apart (one
// 128-byte line per head): the atomic minima of a head's splits serialise
// per line, so heads must not share one.
constexpr int kKeyStride = 16;
constexpr unsigned long long kSyncMagic = 0x4d41432d53594e43ull;
// Synchronisation words: the done counter, the initialised marker, the
// latched time-outs (cleared when read), and the broken mark: set with a
// time-out, cleared only by the ring reset; a single launch that finds it
// set computes nothing and writes NaN outputs, so a handle whose counters a
// time-out left inconsistent fails visibly until it is re-initialised.
enum { kSyncDone = 0, kSyncMagicWord = 1, kSyncSticky = 2, kSyncBroken = 3 };

// Key words per group of the single launch: one per match unit, at least
// one per workgroup, never more than kMaxSingleUnits.

// Plan: work-item partition of one group's token range [s, e].
// Boundaries: s, the multiples of C in (s, e], the rectify split
// sp = e - r + 1 when it falls strictly inside (s, e], and e + 1.
struct RangeSplit {
    // C = 1 << cs; divisions by C are shifts.
    int s, e, cs, c_first, n_grid, sp, has_sp, j_sp, n;
    // Shift of the smallest C = 2^cmin * 2^k with at most kMaxItemsPerGroup
    // grid cells over [s_, e_].
    __host__ __device__ static int chunk_shift_for(int s_, int e_, int cmin)
    {
        const int span = e_ - s_ + 1;
        int cs = 0;
        while ((1 << (cmin + cs)) < span && (((span - 1) >> cs) >> cmin) + 1 > kMaxItemsPerGroup)
            ++cs;
        return cs + cmin;
    }
    __host__ __device__ static int chunk_for(int s_, int e_, int cmin)
    {
        return 1 << chunk_shift_for(s_, e_, cmin);
    }
    // The same cuts with the chunk C = 1 << cs_ given.
    __host__ __device__ RangeSplit(int s_, int e_, int r, int cs_) { init(s_, e_, r, cs_); }
    __host__ __device__ void init(int s_, int e_, int r, int cs_)
    {
        s = s_;
        e = e_;
        cs = cs_;
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

// Work items of one KV group at end position e whose heads attend from s
// (the smallest start over the group's heads).  First the main items: the
// range [max(s, F), e] cut by RangeSplit (none when e < F).  Then, when
// `sink` is set and F > 0, one item [0, min(F, e + 1)) that every head of
// the group attends in full whatever its match: the attention sink, kept
// out of every reusable summary.  The sink item comes after the rectify
// split, so it counts in the output but not in the rectified summary.
// With F = 0 the items are exactly RangeSplit(s, e, r)'s.
struct GroupItems {
    RangeSplit rs;
    int ms, n_main, sink_end, n;
    __host__ __device__ GroupItems() : rs(0, 0, 0, kChunkMinShift), ms(0), n_main(0), sink_end(0), n(0) {}
    // cmin: the shape's minimum grid shift; cs >= 0 forces the grid (1 << cs).
    __host__ __device__ GroupItems(int s, int e, int r, int F, bool sink, int cmin, int cs = -1)
        : rs(0, 0, 0, kChunkMinShift)
    {
        ms = s > F ? s : F;
        n_main = 0;
        if (ms <= e) {
            if (cs < 0)
                rs.init(ms, e, r, RangeSplit::chunk_shift_for(ms, e, cmin));
            else
                rs.init(ms, e, r, cs);
            n_main = rs.n;
        }
        sink_end = (sink && F > 0) ? (F < e + 1 ? F : e + 1) : 0;
        n = n_main + (sink_end > 0 ? 1 : 0);
    }
    __host__ __device__ bool is_sink(int i) const { return i >= n_main; }
    __host__ __device__ void item(int i, int &t0, int &t1) const
    {
        if (i < n_main) {
            rs.item(i, t0, t1);
        } else {
            t0 = 0;
            t1 = sink_end;
        }
    }
    // Leading items before the rectify split (the sink is never among them).
    __host__ __device__ int n_before_split() const { return n_main > 0 ? rs.n_before_split() : 0; }
    __host__ __device__ int main_tokens() const { return n_main > 0 ? rs.e - ms + 1 : 0; }
    // Work of the group in the attention kernel's balanced split: tokens plus
    // kItemCost per item.
    __host__ __device__ int work() const { return main_tokens() + sink_end + kItemCost * n; }
    // Work before item i.
    __host__ __device__ int offset(int i) const
    {
        int t0 = 0, t1 = 0;
        if (i < n_main)
            rs.item(i, t0, t1);
        return (i < n_main ? t0 - ms : main_tokens()) + kItemCost * i;
    }
};

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
    size_t keys, ctx, dec_slot, grp_begin, grp_count, grp_start, ctrl, sync,
        part_o, part_l, rect_o, rect_l, ring_epoch, restart, app_pos, skeys, grp_sync, pool,
        gplan, total;
    int64_t max_items;
    int32_t nsplit;
};

// Plan modes.
enum PlanMode : int32_t {
    kPlanMatch = 0,  // decisions from the match keys (decode step)
    kPlanFull = 1,   // every head misses (full decode)
    kPlanInit = 2,   // full, end = pos[b] + end_offset, a negative end is empty
};

// ctrl words: [0] work items of the latest call, [1] its status flags, [2]
// the attention kernel's claim counter of its dynamic items (reset to 0 by
// the merge kernel that follows every attention launch).
enum { kCtrlItems = 0, kCtrlStatus = 1, kCtrlClaim = 2 };

struct Shape {
    int32_t B, Hq, Hkv, G, D, dtype, K, r, T;
    int32_t F;                    // front sink: leading positions never reused
    int32_t min_ctx;              // positions below it find no match candidate
    int32_t cmin;                 // shift of the minimum work-item grid
    // Paged K/V (page_table non-null): row t of request b, KV head g at
    // b's page page_table[b * max_pages + (t >> page_shift)], element
    // offset page * kv_sb + g * kv_sh + (t mod page size) * kv_st.
    int32_t page_shift, max_pages;
    const int32_t *page_table;
    int64_t kv_sb, kv_sh, kv_st;  // elements
    float qscale;                 // sm_scale * log2(e)
    float thresh2;
};

// Device pointers into the workspace.
struct WsPtrs {
    // [B*Hq * kKeyStride] per-head match keys of the three-kernel step
    unsigned long long *keys;
    int32_t *ctx;  // [B] prompt lengths during the warm-up
    int32_t *dec_slot, *grp_begin, *grp_count, *grp_start, *ctrl;
    unsigned long long *sync;  // done counter, magic, latched time-outs
    float *part_o, *part_l, *rect_o, *rect_l;
    // [B * Hkv] the epoch each KV group's rings were built for (see
    // StepArgs::epoch); reset to 0 with the rings
    int32_t *ring_epoch;
    // [B * Hkv] 1 where the latest step's merge found the group not ready:
    // the separate append kernel then restarts the group's position ring
    int32_t *restart;
    // [B * Hkv] the position the latest step's merge appended for each KV
    // group (-1: nothing to append), so that the separate append kernel never
    // reads the caller's position array on the auxiliary stream
    int32_t *app_pos;
    // single launch only (null otherwise): tagged split keys, per-group
    // arrival counters, the two pool sets, per-group plan records
    unsigned long long *skeys;
    uint32_t *grp_sync;
    unsigned long long *pool;
    int32_t *gplan;
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
    // [B] device, or null: the caller's epoch of each request, read by the
    // match, plan and merge of the step only.  A KV group whose ring_epoch
    // differs, or whose request epoch is negative, is not ready: its match
    // sees no candidate (exact attention), its merge records the epoch, and
    // its append empties the group's position ring before adding the
    // step's entry.
    const int32_t *epoch;
    // single launch: workgroups per group, match units per group (G *
    // nsplit), key words per group, log2 of the done increment per launch,
    // ring slots per match unit
    int32_t wpg, upg, nkw, done_shift, unit_slots;
    // single launch: pool entries per set (B * Hkv * kItemsPerGroupMax)
    int32_t pool_cap;
    // per-head match keys: 0 = set 0 (three kernels: the merge kernel resets
    // them); 1 = set (launch epoch & 1) of the two sets (match kernel, then
    // the group kernel, whose first workgroup clears the other set)
    int32_t key_parity;
    // the one-launch kernel without its match phase: the group kernel of
    // the two-kernel form (keys from the match kernel)
    int32_t group_only;
    // attention kernel: 1 = the last (100 - kStaticPct)% of the work is a pool
    // claimed through ctrl[kCtrlClaim], which must then read 0 at the launch
    // (the ring reset and every merge kernel leave it so); 0 = all of the
    // work is split statically and the counter is not touched
    int32_t dyn_pool;
    // match: read the second half of a ring row only when the first half's
    // squared distance is below the threshold (exact lower-bound filter)
    int32_t match_filter;
};

// Bytes of dynamic LDS the planner needs.
size_t plan_lds_bytes(int B, int Hq, int Hkv);

// single: include the single-launch regions.
WsLayout ws_layout(int B, int Hq, int Hkv, int D, int K, int T, int dtype, bool single);
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
// at once: a.wpg workgroups per KV group.
hipError_t launch_step(const StepArgs &a, hipStream_t st);
// Workgroups of the single-launch kernel for this shape that the device
// holds resident at once (0 if unknown).
int step_resident_workgroups(const Shape &s);
// The two above for one (K/V dtype, head dim) each (mac_step_*.hip).
void launch_step_bf16_128(const StepArgs &a, hipStream_t st);
void launch_step_bf16_64(const StepArgs &a, hipStream_t st);
void launch_step_f32_128(const StepArgs &a, hipStream_t st);
void launch_step_f32_64(const StepArgs &a, hipStream_t st);
int step_resident_bf16_128(const Shape &s);
int step_resident_bf16_64(const Shape &s);
int step_resident_f32_128(const Shape &s);
int step_resident_f32_64(const Shape &s);
// Copies of the step kernels' timeline words (library built with
// MAC_TIMELINE; hipErrorNotSupported otherwise), one per source file.
hipError_t timeline_read_bf16_128(void *host, size_t bytes);
hipError_t timeline_read_bf16_64(void *host, size_t bytes);
hipError_t timeline_read_f32_128(void *host, size_t bytes);
hipError_t timeline_read_f32_64(void *host, size_t bytes);
// Rectify-append from the workspace staging into the rings; the position of
// request b is pos[b] + pos_offset.
hipError_t launch_append(const StepArgs &a, int32_t pos_offset, hipStream_t st);
// Empties the rings, resets the synchronisation words and clears the first
// n_tag words of the single-launch tagged keys and the n_pool words of its
// pool sets (when present in w).
hipError_t launch_ring_reset(const Shape &s, void *q_ring, float *o_ring,
                             float *lse_ring, int32_t *pos_ring, const WsPtrs &w,
                             int64_t n_tag, int64_t n_pool, hipStream_t st);
int device_cu_count();
// Address of this device's static scratch (MAC_NOALLOC_SCRATCH_BYTES), looked
// up once per device with that device current.
hipError_t noalloc_scratch(void **ptr);
// Streaming read of a buffer (bandwidth measurement); sink holds grid floats.
hipError_t launch_stream_read(const void *buf, size_t bytes, float *sink, int grid,
                              hipStream_t st);
// K and V of position pos[b] into the cache, K rotated by RoPE (base > 0),
// and q_out = RoPE(q_tilde) when q_out is non-null.
hipError_t launch_append_kv(const Shape &s, const void *k_new, const void *v_new,
                            const void *q_tilde, float *q_out, const int32_t *pos, double base,
                            void *k_cache, void *v_cache, hipStream_t st);

}  // namespace mac
