/*
 * mac_attention.h -- C ABI of the MI355X (gfx950) MAC-Attention decode step.
 *
 * MAC-Attention (Match-Amend-Complete) reuses attention across decode steps
 * of one request: the current pre-RoPE query is matched against a ring of the
 * last K pre-RoPE queries; on a hit at position p the cached, rectified
 * attention summary of [0, p-r] is merged with fresh attention over
 * [p-r+1, m]; on a miss the step is exact full attention; afterwards the new
 * query and its rectified summary of [0, m-r] are appended to the rings.
 *
 * Sources: "MAC-Attention: Match-Amend-Complete attention reuse, up to 99%
 * less KV reading in long-context decoding (MLSys 2026)" (blog post),
 * sections "Decomposable representation of attention", "Reuse", "Match
 * (1)-(3)", "Amend", "Complete" and "Paper version: the K1/K2/K3
 * micro-pipeline", and "Production version: one fused persistent BF16
 * kernel" for the attention-sink isolation and the ready/epoch gating;
 * "Attention Cache and Sequence Parallelism", section "MHA: per-token K/V"
 * for the baseline decode semantics.
 *
 * Conventions for every entry point:
 *  - All buffers are DEVICE pointers owned by the caller, unless noted.  The
 *    library never allocates device memory; mac_init_rings allocates one
 *    small host-side handle holding two HIP events.
 *  - Streams are hipStream_t passed as void* (NULL = the null stream).
 *  - Positions are 0-indexed.  At decode position m the query attends the
 *    cached positions [0, m] (the caller has already written K_m, V_m).
 *  - GQA: query head h reads KV head h / G with G = n_q_heads / n_kv_heads.
 *  - Logits are scale * <q, K_t>, scale = 1/sqrt(d) unless sm_scale != 0.
 *  - Summaries are (o, lse): the normalised output o = S/Z and lse = ln Z.
 *  - Every call validates its arguments on the host first and returns an
 *    error code without launching anything if they are invalid.  Calls
 *    return without a host synchronisation; device-side errors (positions
 *    out of range) of the latest call on a workspace are recorded in it and
 *    read with mac_read_device_status().  No call aborts the process.
 */
#ifndef MAC_ATTENTION_H
#define MAC_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mac_status {
    MAC_OK = 0,
    MAC_ERR_INVALID_ARG = -1,         /* null pointer, bad size or stride   */
    MAC_ERR_UNSUPPORTED = -2,         /* head_dim / dtype / group not built */
    MAC_ERR_HIP = -3,                 /* a HIP runtime call failed          */
    MAC_ERR_WORKSPACE_TOO_SMALL = -4, /* ws_bytes < mac_workspace_bytes()   */
    MAC_ERR_MISALIGNED = -5,          /* a buffer or row not 16-B aligned   */
    MAC_ERR_CONTEXT_TOO_LONG = -6,    /* kv_capacity > max_context          */
    MAC_ERR_NOT_INITIALIZED = -7,     /* handle NULL, released, or not made
                                         by mac_init_rings                  */
    MAC_ERR_SCRATCH_TOO_SMALL = -8    /* the shape needs more than the
                                         library's static scratch
                                         (MAC_NOALLOC_SCRATCH_BYTES)        */
} mac_status;

/* Size of the device scratch that mac_full_decode_noalloc uses instead of a
 * workspace: one static array per GPU, held from the library's first use on
 * that GPU until the process ends. */
#define MAC_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

/* Element type of the K/V cache, of the pre-RoPE queries and of the query
 * ring.  Post-RoPE queries, outputs and summaries are always fp32. */
enum { MAC_DTYPE_F32 = 0, MAC_DTYPE_BF16 = 1 };

/* Acceptance rule of a match with squared L2 distance D (blog, "Match (2)"):
 *   MAC_THRESH_ONE_MINUS_TAU: D < 2d (1-tau)^2   -- the blog's worked
 *       example (d=128, tau=0.45 -> distance 8.8) and its pseudocode;
 *   MAC_THRESH_TAU:           D < 2d tau^2       -- the paper summary's form.
 * The squared threshold is computed in fp64 from the fp32 tau and rounded
 * once to fp32. */
enum { MAC_THRESH_ONE_MINUS_TAU = 0, MAC_THRESH_TAU = 1 };

/* mac_params.flags bits.
 *   MAC_FLAG_FUSED_APPEND: the rectify-append is done by the merge instead
 *   of a separate kernel on the auxiliary stream.
 *   MAC_FLAG_SPLIT_STAGES: mac_decode_step always runs match, plan +
 *   attention and merge as three kernels.
 *   MAC_FLAG_SINGLE_LAUNCH: mac_decode_step always runs the step as one
 *   launch (MAC_ERR_UNSUPPORTED from mac_init_rings when kv_capacity exceeds
 *   2^24, when a KV group's ring match needs more than 256 units of up to
 *   256 slots, or when the device cannot hold one workgroup per KV group
 *   resident).
 *   MAC_FLAG_TWO_STAGES: mac_decode_step runs the match as one kernel and
 *   plan, attention and merge as a second (MAC_ERR_UNSUPPORTED from
 *   mac_init_rings when kv_capacity exceeds 2^24 or the device cannot hold
 *   one workgroup per KV group resident).
 * At most one of these three may be set.  With none, the step is one launch
 * when a layer has at most 16 KV groups (batch * n_kv_heads) and the shape
 * is one the single launch handles (the step is bound by latency), two
 * kernels up to 64 KV groups, and three kernels above (bound by bandwidth:
 * the attention kernel balances all groups' work across the device).
 * All forms give the same results bit for bit.
 *   MAC_FLAG_MATCH_FILTER: exact lower-bound filter of the match (blog,
 *   "Production version: one fused persistent BF16 kernel", the match-scan
 *   item).  The first half of every candidate row is read; the second half
 *   only when the first half's squared distance is below the threshold
 *   (times 1 + 2^-10, a margin that covers fp32 rounding).  A row cut there
 *   cannot hit, so the decisions, matched positions, outputs and rings are
 *   bit for bit those of the full scan; match_d2 is unchanged for hits, and
 *   for a miss is the smallest distance among the rows read in full (+inf
 *   if none), always at least the threshold.  It pays where the match is
 *   bound by bandwidth (many KV groups, three kernels) and ring rows are
 *   128-byte aligned; it adds a dependent read to a latency-bound step. */
enum {
    MAC_FLAG_FUSED_APPEND = 1,
    MAC_FLAG_SPLIT_STAGES = 2,
    MAC_FLAG_SINGLE_LAUNCH = 4,
    MAC_FLAG_MATCH_FILTER = 8,
    MAC_FLAG_TWO_STAGES = 16
};

/* Device status flags latched in the workspace. */
enum {
    MAC_DEV_BAD_POSITION = 1, /* some m outside [0, kv_capacity)            */
    MAC_DEV_SYNC_TIMEOUT = 2  /* a single-launch step gave up waiting for
                                 workgroups that never became resident: the
                                 waiting groups' outputs are NaN, and every
                                 later single-launch step on the workspace
                                 writes NaN outputs and leaves the rings
                                 untouched until mac_init_rings resets it  */
};

typedef struct mac_params {
    int32_t batch;        /* B requests                                      */
    int32_t n_q_heads;    /* Hq                                              */
    int32_t n_kv_heads;   /* Hkv; G = Hq / Hkv must be 1, 2, 4 or 8          */
    int32_t head_dim;     /* d: 64 or 128                                    */
    int32_t kv_dtype;     /* MAC_DTYPE_*                                     */
    int32_t ring_k;       /* K >= 1: ring capacity = match window            */
    int32_t band_r;       /* r >= 0: rectification band                      */
    int32_t kv_capacity;  /* T: positions held per (request, KV head)        */
    float tau;            /* threshold parameter                             */
    int32_t thresh_mode;  /* MAC_THRESH_*                                    */
    float sm_scale;       /* logit scale; 0 means 1/sqrt(d)                  */
    int32_t flags;        /* MAC_FLAG_* bits, 0 for the defaults             */
    /* K/V cache strides in elements; all 0 means dense [B, Hkv, T, d].
     * Row t of (b, g) starts at b*kv_stride_b + g*kv_stride_h + t*kv_stride_t
     * and must be 16-byte aligned. */
    int64_t kv_stride_b, kv_stride_h, kv_stride_t;
    /* F in [0, 4096]: attention-sink isolation (blog, "Production version:
     * one fused persistent BF16 kernel").  The first F positions never enter
     * a reusable summary: ring summaries cover [F, t-r] instead of
     * [0, t-r], and every step attends [0, min(F, m+1)) exactly with its own
     * query, hit or miss.  0 (the default) is the plain method. */
    int32_t front_sink;
    /* Paged K/V cache (blog, "Production version": the production kernel
     * reads the serving engine's BF16 paged KV).  page_size = 0: the dense
     * layout above.  Otherwise page_size is a power of two >= 16, and row t
     * of request b, KV head g starts at element
     *   page_table[b * max_pages + t / page_size] * kv_stride_b
     *   + g * kv_stride_h + (t % page_size) * kv_stride_t
     * of k_cache / v_cache (all strides 0: pages of [Hkv, page_size, d]).
     * page_table is a DEVICE int32 array [B, max_pages] (4-byte aligned),
     * read on the device at every call, so its contents may change between
     * calls (and between replays of a captured graph) but not during one;
     * max_pages * page_size >= kv_capacity; rows must be 16-byte aligned.
     * The entries that cover positions 0..pos[b] of a request must name
     * pages of the pool (the library reads them as given; an entry outside
     * the pool is an out-of-bounds read). */
    int32_t page_size;
    int32_t max_pages;
    const int32_t *page_table;
    /* Context limits (blog, "Production version: one fused persistent BF16
     * kernel": its settings block turns reuse off below a minimum generated
     * context, and its graph-safe readiness item refuses entry above a
     * maximum context).
     * max_context >= 0: 0 means no limit; otherwise every call whose
     * kv_capacity exceeds it returns MAC_ERR_CONTEXT_TOO_LONG on the host,
     * before any launch.
     * min_context >= 0: a request at position m < min_context finds no
     * match candidate (decided on the device per request and step, so it
     * holds inside captured graphs): the step is exact full attention
     * (match_p -1, match_d2 +inf) and its rectify-append still writes slot
     * m mod K, so reuse can start as soon as m reaches the limit.  0 (the
     * default) never blocks. */
    int32_t max_context;
    int32_t min_context;
} mac_params;

/* Ring buffers of one attention layer, caller-allocated device memory:
 *   q_ring   [B, Hq, K, d] kv_dtype  pre-RoPE queries of the last K positions
 *   o_ring   [B, Hq, K, d] fp32      rectified summaries: normalised output
 *   lse_ring [B, Hq, K]    fp32      rectified summaries: ln Z (-inf = empty)
 *   pos_ring [B, Hkv, K]   int32     position held by each slot of the rings
 *                                   of KV group g's query heads (-1 = empty)
 * Slot of position t is t mod K.  The position ring is kept per KV group
 * so that each group's rings are written only by that group's work.
 * Sizes: mac_ring_bytes(). */
typedef struct mac_rings {
    void *q_ring;
    float *o_ring;
    float *lse_ring;
    int32_t *pos_ring;
} mac_rings;

typedef struct mac_handle mac_handle;

/* Bytes of device workspace the decode and full-decode calls need. */
size_t mac_workspace_bytes(const mac_params *p);

/* Bytes of each ring buffer: out[0..3] = q_ring, o_ring, lse_ring, pos_ring. */
mac_status mac_ring_bytes(const mac_params *p, size_t out[4]);

/*
 * mac_init_rings -- reset one layer's rings and bind them to a handle.
 *
 * Every slot is emptied (pos -1, lse -inf) and the rings' epochs are set to
 * 0 (see mac_bind_epochs).  With n_warm = W > 0 the last W prompt positions
 * t = ctx_len[b] - W + w (w = 0..W-1) are pre-filled: slot t mod K receives
 * the pre-RoPE query warm_qtilde[b, h, w, :], the summary of attention of
 * the post-RoPE query warm_q[b, h, w, :] over [F, t-r] (empty when
 * t - r < F; F = front_sink) and pos t.  W must not exceed K, and
 * ctx_len[b] >= W.
 *   warm_qtilde [B, Hq, W, d] kv_dtype   (device; ignored when W = 0)
 *   warm_q      [B, Hq, W, d] fp32       (device; ignored when W = 0)
 *   ctx_len     [B] int32 on the HOST: the prompt length of each request.
 *   k_cache, v_cache: the layer's cache laid out as described in mac_params.
 *   workspace: >= mac_workspace_bytes(p) device bytes, kept by the handle and
 *   used by every later mac_decode_step on it (one workspace per handle).
 * The rings and workspace must stay valid until mac_release().  On success
 * *out receives a new handle; the work is enqueued on `stream`.
 */
mac_status mac_init_rings(const mac_params *p, const mac_rings *rings,
                          void *workspace, size_t ws_bytes,
                          const void *warm_qtilde, const float *warm_q,
                          int32_t n_warm, const int32_t *ctx_len,
                          const void *k_cache, const void *v_cache,
                          void *stream, mac_handle **out);

/*
 * mac_decode_step -- one Match-Amend-Complete decode step of one layer.
 *   qtilde  [B, Hq, d] kv_dtype  pre-RoPE query at position m
 *   q       [B, Hq, d] fp32      post-RoPE query at position m
 *   pos     [B] int32 (device)   m per request, 0 <= m < kv_capacity
 *   out     [B, Hq, d] fp32      attention output
 *   out_lse [B, Hq] fp32 or NULL ln Z of the output
 *   match_p [B, Hq] int32 or NULL  matched position, -1 on a miss
 *   match_d2[B, Hq] fp32 or NULL   squared distance of the nearest candidate
 *                                  (+inf when the window is empty)
 * With front_sink F > 0 a hit at p merges the cached summary of [F, p-r],
 * the sink [0, min(F, m+1)) and fresh attention over [max(F, p-r+1), m],
 * and the appended summary covers [F, m-r].  Requests whose rings are not
 * ready (mac_bind_epochs) are computed as misses.
 * Match, amend and complete run on main_stream as one kernel launch whose
 * workgroups are all resident at once (the workgroups of each KV group hand
 * match keys and partial summaries to each other inside the launch), as
 * three kernels (match, plan + attention, merge), or as two (the match
 * kernel, then plan, attention and merge in one launch whose workgroups are
 * all resident at once); see MAC_FLAG_SPLIT_STAGES for the choice.  The one-
 * and two-kernel forms need kv_capacity <= 2^24.  Other work
 * that holds compute units while the launch waits for residency only delays
 * it; a launch that cannot get all its workgroups resident within about a
 * second stops waiting and latches MAC_DEV_SYNC_TIMEOUT.  The rectify-append of the rings runs as another
 * kernel on aux_stream (main_stream if NULL or equal), ordered after the
 * merge by an event; the next call on the same handle waits for it.  With
 * MAC_FLAG_FUSED_APPEND the merge writes the rings itself and aux_stream is
 * unused.  The append reads qtilde: when it runs on aux_stream, work that
 * overwrites qtilde must be ordered after mac_join_aux (or after a later
 * mac_decode_step on the handle) on the stream that does it; the other
 * inputs (pos and epoch included: the merge keeps a copy of each request's
 * position in the workspace for the append) are read on main_stream only,
 * so main_stream may overwrite them as soon as the call returns.  Returns without a host
 * synchronisation, so a steady-state step
 * can be captured into a HIP graph (join aux_stream back with mac_join_aux
 * first).  Calls on one handle must not overlap; handles are independent,
 * and each owns its workspace (the single launch keeps synchronisation
 * counters there between calls).
 */
mac_status mac_decode_step(mac_handle *h, const void *qtilde, const float *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *pos, float *out, float *out_lse,
                           int32_t *match_p, float *match_d2,
                           void *main_stream, void *aux_stream);

/*
 * mac_bind_epochs -- device ready/epoch gating (blog, "Production version:
 * one fused persistent BF16 kernel", the graph-safe readiness item).
 *   epoch [B] int32 (device, 4-byte aligned), or NULL to unbind.
 * Binds the caller's per-request epoch array to the handle; later
 * mac_decode_step calls read it on the device.  The rings of each KV group
 * remember the epoch they were built for (0 after mac_init_rings).  At a
 * step where epoch[b] differs from that, or is negative, request b's rings
 * are not ready: its match finds no candidate, so every head of b is exact
 * full attention (match_p -1, match_d2 +inf), and the step's rectify-append
 * empties b's position ring before adding its own entry and adopts
 * epoch[b] (a negative epoch is never adopted as ready).  Bumping epoch[b]
 * on the device -- inside a captured graph too -- thus invalidates and
 * restarts request b's rings without a host call.  The array is read on
 * main_stream and must stay valid while steps that read it run.
 */
mac_status mac_bind_epochs(mac_handle *h, const int32_t *epoch);

/*
 * mac_append_kv -- write the new token of every request into the K/V cache,
 * with RoPE fused into the K write (blog, "Production version", the fused
 * KV-RoPE setting), and optionally produce the post-RoPE query.
 *   k_new, v_new [B, Hkv, d] kv_dtype   key (pre-RoPE) and value of position
 *                                       pos[b]
 *   q_tilde [B, Hq, d] kv_dtype, q_out [B, Hq, d] fp32: both NULL, or both
 *                                       given: q_out = RoPE(q_tilde, pos[b])
 *   pos [B] int32 (device)              positions outside [0, kv_capacity)
 *                                       are skipped
 *   rope_base                           > 0: pair (x[2j], x[2j+1]) rotates by
 *                                       pos * rope_base^(-2j/d); 0: no
 *                                       rotation (K is copied)
 *   k_cache, v_cache                    dense or paged, as in mac_params
 * The rotation is evaluated in fp64 and rounded once to the K element type
 * (to fp32 for q_out).  Rows are written with plain stores on `stream`; run
 * it before the mac_decode_step that attends position pos[b].
 */
mac_status mac_append_kv(const mac_params *p, const void *k_new, const void *v_new,
                         const void *q_tilde, float *q_out, const int32_t *pos,
                         double rope_base, void *k_cache, void *v_cache, void *stream);

/* Make `stream` wait for the last rectify-append enqueued on the handle. */
mac_status mac_join_aux(mac_handle *h, void *stream);

/*
 * mac_full_decode -- exact split-KV decode attention over [0, pos[b]] for
 * every (request, query head); the miss path of mac_decode_step runs the
 * same kernels on the same partition (with front_sink F > 0 the positions
 * [0, F) are their own item in both), so a forced miss gives bitwise the
 * same output.  Arguments as in mac_decode_step; needs a workspace of
 * mac_workspace_bytes(p) (not shared with a concurrently running handle).
 */
mac_status mac_full_decode(const mac_params *p, const float *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *pos, float *out, float *out_lse,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * mac_full_decode_noalloc -- mac_full_decode without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments and results as mac_full_decode, bit for bit (the same kernels on
 * the same partition).  The partials live in a static device array of
 * MAC_NOALLOC_SCRATCH_BYTES per GPU, inside the library; shapes whose
 * mac_full_decode workspace (without the single-launch regions) exceeds it
 * return MAC_ERR_SCRATCH_TOO_SMALL before any launch.  The call allocates
 * nothing: the first call on a device (with that device current) only looks
 * up the array's address.  Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (concurrent streams, threads) race and must
 * be serialised by the caller; calls on different GPUs are independent.
 * Device-side position errors give NaN outputs and are not reported.
 */
mac_status mac_full_decode_noalloc(const mac_params *p, const float *q,
                                   const void *k_cache, const void *v_cache,
                                   const int32_t *pos, float *out, float *out_lse,
                                   void *stream);

/* Read (with a synchronisation of `stream`) and clear the device status
 * flags (MAC_DEV_*) of a workspace laid out for p: MAC_DEV_BAD_POSITION of
 * the latest call, MAC_DEV_SYNC_TIMEOUT of any call since the last read. */
mac_status mac_read_device_status(const mac_params *p, void *workspace,
                                  void *stream, int32_t *flags);

/* Per-kernel timing with HIP events (diagnostics).  mac_profile_start arms
 * recording for the next `n_steps` decode steps of the handle; stages are
 * 0 match (0 for the single launch), 1 plan + attention and 2 merge (0
 * unless three kernels run), 3 rectify-append (0 when fused), 4 the single
 * launch or, in the two-kernel form, its second kernel (0 when three
 * kernels run).  mac_profile_read synchronises, returns the
 * summed milliseconds per stage in ms[5] and the number of recorded steps
 * in *n, and disarms. */
enum { MAC_PROFILE_STAGES = 5 };
mac_status mac_profile_start(mac_handle *h, int32_t n_steps);
mac_status mac_profile_read(mac_handle *h, double ms[MAC_PROFILE_STAGES], int32_t *n);

/* Per-workgroup timeline of the step kernel (diagnostics).  Only a library
 * built with MAC_TIMELINE defined records it (attention_reuse_amd/build.py
 * --timeline makes libmac_attention_timeline.so); the default build returns
 * MAC_ERR_UNSUPPORTED.  Synchronises the device, then copies up to `bytes`
 * bytes of the timeline words of the step kernels of h's K/V dtype and head
 * dim to host memory `host` (caller-owned): 4096 workgroups x 32 uint64
 * words, word w * 32 + slot, each written by the latest launch whose
 * workgroup w reached it (earlier launches' values remain elsewhere).
 * Marks hold the 100 MHz device real-time counter:
 *   0 workgroup start; 1 match keys stored (one launch) or queries staged
 *   (group kernel of the two-kernel form); 2 speculative K/V requested;
 *   3 group planned; 4 items counted and pool entries published; 5 first
 *   own item begins; 6 its blocks computed; 7 its partial stored; 8 its
 *   count done; 9 all own items done; 10 merge of the own group done (its
 *   merger only); 11 end of a workgroup that ran items; 12 end of a
 *   workgroup without own items; 13 first pool item claimed; in the merge
 *   of a group, by its merger: 20 begins, 21 item weights formed (up to 24
 *   items for G <= 4, 12 otherwise) or the first list folded, 22 both lists
 *   summed, 23 outputs and ring entries written (stores issued); in the
 *   own-items block before the first item: 24 queries read from LDS, 25
 *   the item's bounds computed, 26 its rows requested (or speculated);
 *   27 an item's blocks done, before their cross-row combine, and 28 the
 *   row states of all the workgroup's waves in LDS (both for the latest
 *   item of the workgroup).
 * Notes hold counts: 16 the group's items; 17 items of its own workgroups;
 * 18 first item from the speculative rows (1), re-requested (2), none (0);
 * 19 pool items run by this workgroup. */
mac_status mac_timeline_read(mac_handle *h, void *host, size_t bytes);

/* Streaming read of bytes (rounded down to 16) of the device buffer buf by
 * `grid` workgroups, enqueued on `stream` (measurement of the achievable HBM
 * read bandwidth that the decode kernels are compared with).  sink: device
 * floats [grid], written only in the practically impossible case that the
 * data folds to one particular value (it keeps the loads from being
 * optimised away).  buf 16-byte aligned. */
mac_status mac_stream_read(const void *buf, size_t bytes, float *sink, int32_t grid,
                           void *stream);

/* Free the handle and its events (not the caller's buffers). */
mac_status mac_release(mac_handle *h);

const char *mac_status_string(mac_status s);

/* The minimum grid of the split-KV partition for a shape (host mirror of
 * the device planner): 64 tokens for layers of at most 16 KV groups
 * (batch * n_kv_heads), 256 above; -1 on invalid parameters.  Every entry
 * point on the same parameters (decode step in either form, full decode)
 * cuts ranges on the same grid, so a missing head equals the full decode
 * bit for bit. */
int32_t mac_min_chunk_tokens(const mac_params *p);

/* Grid of the split-KV partition for a KV group attending [s, e]: the
 * smallest C = min_chunk * 2^k with at most 128 grid cells over the range
 * (-1 on bad input; min_chunk a power of two >= 64, as
 * mac_min_chunk_tokens returns). */
int32_t mac_chunk_tokens(int32_t s, int32_t e, int32_t min_chunk);

/* The split-KV partition the kernels use for a KV group whose heads attend
 * [s, e] with band r (host mirror of the device planner): item i covers
 * [t0[i], t1[i]); boundaries are s, the multiples of
 * mac_chunk_tokens(s, e, min_chunk) in (s, e], the rectify split e - r + 1
 * when inside (s, e], and e + 1.  With front_sink F > 0 the planner applies
 * this to [max(s, F), e] and adds the sink [0, min(F, e + 1)) as one more
 * item.  Writes min(n, cap) items (host arrays) and returns n, or -1 on bad
 * input. */
int32_t mac_partition(int32_t s, int32_t e, int32_t r, int32_t min_chunk, int32_t *t0,
                      int32_t *t1, int32_t cap);

/* The work items of one KV group at decode position e whose heads attend
 * from s, with band r, front sink F and minimum grid min_chunk (host mirror
 * of the device planner): first the partition of [max(s, F), e] as
 * mac_partition cuts it (none when e < F), then, when F > 0, the sink item
 * [0, min(F, e + 1)).  Writes min(n, cap) items (host arrays) and, if
 * n_before_split is not NULL, the number of leading items before the
 * rectify split e - r + 1 (the items whose partials enter the rectified
 * summary).  Returns n, or -1 on bad input. */
int32_t mac_group_items(int32_t s, int32_t e, int32_t r, int32_t front_sink, int32_t min_chunk,
                        int32_t *t0, int32_t *t1, int32_t *n_before_split, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* MAC_ATTENTION_H */
