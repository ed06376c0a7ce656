// Launchers of the MAC-Attention decode step's kernels (match, plan +
// attention, merge, rectify-append, K/V append, ring reset, streaming read)
// and the workspace of the entry points that allocate nothing.  The
// one-launch step's kernels are instantiated in mac_step_*.hip, one source
// per (K/V dtype, head dim), so that they compile in parallel.
#include "mac_device.h"

namespace mac {
// Workspace of the entry points that allocate nothing: one array per GPU
// (each device holds its own copy, at its own address).  Host code never
// passes `scratch` itself to a kernel -- on the host the name is only a
// stand-in; kernels get the device address that noalloc_scratch looked up.
static __device__ __align__(256) unsigned char scratch[MAC_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, float *sink, int grid,
                              hipStream_t st)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kBlock), 0, st,
                       (const u32x4 *)buf, (int64_t)(bytes / 16), sink);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launchers with (dtype, D, G) dispatch.

size_t plan_lds_bytes(int B, int Hq, int Hkv)
{
    const size_t BH = (size_t)B * Hq, NG = (size_t)B * Hkv;
    // the planner's tables, then the claimed tail's prefix (NG + 1)
    return 4 * (BH + 6 * NG + 3 + 2 * (kBlock / 64));
}

int device_cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

#define MAC_DISPATCH_TD(FN, ...)                             \
    do {                                                     \
        if (a.s.dtype == MAC_DTYPE_BF16 && a.s.D == 128)     \
            FN<BF16, 128>(__VA_ARGS__);                      \
        else if (a.s.dtype == MAC_DTYPE_BF16 && a.s.D == 64) \
            FN<BF16, 64>(__VA_ARGS__);                       \
        else if (a.s.dtype == MAC_DTYPE_F32 && a.s.D == 128) \
            FN<F32, 128>(__VA_ARGS__);                       \
        else                                                 \
            FN<F32, 64>(__VA_ARGS__);                        \
    } while (0)

template <class T, int D>
static void match_go(const StepArgs &a, hipStream_t st)
{
    if (a.match_filter)
        hipLaunchKernelGGL((match_kernel<T, D, true>),
                           dim3((a.s.K + kSlotsPerHalvesSplit - 1) / kSlotsPerHalvesSplit,
                                a.s.B * a.s.Hq),
                           dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((match_kernel<T, D, false>), dim3(a.nsplit, a.s.B * a.s.Hq),
                           dim3(kBlock), 0, st, a);
}

hipError_t launch_match(const StepArgs &a, hipStream_t st)
{
    MAC_DISPATCH_TD(match_go, a, st);
    return hipGetLastError();
}

template <class T, int D, bool P>
static void attend_go_p(const StepArgs &a, hipStream_t st)
{
    const size_t lds = plan_lds_bytes(a.s.B, a.s.Hq, a.s.Hkv);
    // Persistent grid: exactly the workgroups that are resident at once, so
    // no workgroup waits for a slot only to find no work; never more than
    // the item bound.
    const void *fn = a.s.G == 1   ? (const void *)attend_kernel<T, D, 1, false, P>
                     : a.s.G == 2 ? (const void *)attend_kernel<T, D, 2, false, P>
                     : a.s.G == 4 ? (const void *)attend_kernel<T, D, 4, false, P>
                                  : (const void *)attend_kernel<T, D, 8, false, P>;
    int64_t grid = (int64_t)device_cu_count() * resident_per_cu(fn, lds);
    if (grid > a.max_items)
        grid = a.max_items > 0 ? a.max_items : 1;
#define MAC_ATT(GG)                                                                       \
    do {                                                                                  \
        if (a.mode == kPlanInit)                                                          \
            hipLaunchKernelGGL((attend_kernel<T, D, GG, true, P>), dim3((int)grid),        \
                               dim3(kBlock), lds, st, a);                                 \
        else                                                                              \
            hipLaunchKernelGGL((attend_kernel<T, D, GG, false, P>), dim3((int)grid),       \
                               dim3(kBlock), lds, st, a);                                 \
    } while (0)
    switch (a.s.G) {
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

template <class T, int D>
static void attend_go(const StepArgs &a, hipStream_t st)
{
    if (a.s.page_table)
        attend_go_p<T, D, true>(a, st);
    else
        attend_go_p<T, D, false>(a, st);
}

hipError_t launch_attend(const StepArgs &a, hipStream_t st)
{
    MAC_DISPATCH_TD(attend_go, a, st);
    return hipGetLastError();
}

template <class T, int D, bool W>
static void merge_go_w(const StepArgs &a, hipStream_t st)
{
    const dim3 grid(a.s.B * a.s.Hkv), block(kMergeBlock);
    switch (a.s.G) {
    case 1:
        hipLaunchKernelGGL((merge_kernel<T, D, 1, W>), grid, block, 0, st, a);
        break;
    case 2:
        hipLaunchKernelGGL((merge_kernel<T, D, 2, W>), grid, block, 0, st, a);
        break;
    case 4:
        hipLaunchKernelGGL((merge_kernel<T, D, 4, W>), grid, block, 0, st, a);
        break;
    default:
        hipLaunchKernelGGL((merge_kernel<T, D, 8, W>), grid, block, 0, st, a);
        break;
    }
}

template <class T, int D>
static void merge_go(const StepArgs &a, hipStream_t st)
{
    if (a.mode == kPlanInit)
        merge_go_w<T, D, true>(a, st);
    else
        merge_go_w<T, D, false>(a, st);
}

hipError_t launch_merge(const StepArgs &a, hipStream_t st)
{
    MAC_DISPATCH_TD(merge_go, a, st);
    return hipGetLastError();
}

template <class T, int D>
static void append_go(const StepArgs &a, int32_t pos_offset, hipStream_t st)
{
    if (a.mode == kPlanInit)
        hipLaunchKernelGGL((append_kernel<T, D, true>), dim3(a.s.B * a.s.Hq), dim3(D), 0, st, a,
                           pos_offset);
    else
        hipLaunchKernelGGL((append_kernel<T, D, false>), dim3(a.s.B * a.s.Hq), dim3(D), 0, st,
                           a, pos_offset);
}

int step_resident_workgroups(const Shape &s)
{
    if (s.dtype == MAC_DTYPE_BF16 && s.D == 128)
        return step_resident_bf16_128(s);
    if (s.dtype == MAC_DTYPE_BF16 && s.D == 64)
        return step_resident_bf16_64(s);
    if (s.dtype == MAC_DTYPE_F32 && s.D == 128)
        return step_resident_f32_128(s);
    return step_resident_f32_64(s);
}

hipError_t launch_step(const StepArgs &a, hipStream_t st)
{
    if (a.s.dtype == MAC_DTYPE_BF16 && a.s.D == 128)
        launch_step_bf16_128(a, st);
    else if (a.s.dtype == MAC_DTYPE_BF16 && a.s.D == 64)
        launch_step_bf16_64(a, st);
    else if (a.s.dtype == MAC_DTYPE_F32 && a.s.D == 128)
        launch_step_f32_128(a, st);
    else
        launch_step_f32_64(a, st);
    return hipGetLastError();
}

hipError_t launch_append(const StepArgs &a, int32_t pos_offset, hipStream_t st)
{
    MAC_DISPATCH_TD(append_go, a, pos_offset, st);
    return hipGetLastError();
}

template <class T, int D>
static void append_kv_go(const Shape &s, const void *k_new, const void *v_new,
                         const void *q_tilde, float *q_out, const int32_t *pos, double base,
                         void *k_cache, void *v_cache, hipStream_t st)
{
    const int nh = s.Hkv + (q_out ? s.Hq : 0);
    hipLaunchKernelGGL((append_kv_kernel<T, D>), dim3(s.B * nh), dim3(D / 2), 0, st, s, k_new,
                       v_new, q_tilde, q_out, pos, base, k_cache, v_cache);
}

hipError_t launch_append_kv(const Shape &s, const void *k_new, const void *v_new,
                            const void *q_tilde, float *q_out, const int32_t *pos, double base,
                            void *k_cache, void *v_cache, hipStream_t st)
{
    if (s.dtype == MAC_DTYPE_BF16 && s.D == 128)
        append_kv_go<BF16, 128>(s, k_new, v_new, q_tilde, q_out, pos, base, k_cache, v_cache, st);
    else if (s.dtype == MAC_DTYPE_BF16 && s.D == 64)
        append_kv_go<BF16, 64>(s, k_new, v_new, q_tilde, q_out, pos, base, k_cache, v_cache, st);
    else if (s.dtype == MAC_DTYPE_F32 && s.D == 128)
        append_kv_go<F32, 128>(s, k_new, v_new, q_tilde, q_out, pos, base, k_cache, v_cache, st);
    else
        append_kv_go<F32, 64>(s, k_new, v_new, q_tilde, q_out, pos, base, k_cache, v_cache, st);
    return hipGetLastError();
}

hipError_t launch_ring_reset(const Shape &s, void *q_ring, float *o_ring,
                             float *lse_ring, int32_t *pos_ring, const WsPtrs &w,
                             int64_t n_tag, int64_t n_pool, hipStream_t st)
{
    const int64_t n_keys = 2 * (int64_t)s.B * s.Hq;  // both key sets
    const int64_t n_sync = kSyncWords;
    const int64_t n_q = (int64_t)s.B * s.Hq * s.K * s.D;
    const int64_t n_l = (int64_t)s.B * s.Hq * s.K;
    const int64_t n_p = (int64_t)s.B * s.Hkv * s.K;
    const int64_t n_gs = w.grp_sync ? (int64_t)s.B * s.Hkv * kGrpStride : 0;
    int64_t n_max = n_q > n_tag ? n_q : n_tag;
    n_max = n_max > n_pool ? n_max : n_pool;
    int64_t blocks = (n_max + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (s.dtype == MAC_DTYPE_BF16)
        hipLaunchKernelGGL(ring_reset_kernel<uint16_t>, dim3((int)blocks), dim3(256), 0, st,
                           n_q, (uint16_t *)q_ring, o_ring, n_l, lse_ring, n_p, pos_ring, w.ctrl,
                           n_keys, w.keys, n_sync, w.sync, n_tag, w.skeys, n_gs, w.grp_sync, n_p / s.K,
                           w.ring_epoch, n_pool, w.pool);
    else
        hipLaunchKernelGGL(ring_reset_kernel<float>, dim3((int)blocks), dim3(256), 0, st, n_q,
                           (float *)q_ring, o_ring, n_l, lse_ring, n_p, pos_ring, w.ctrl, n_keys,
                           w.keys, n_sync, w.sync, n_tag, w.skeys, n_gs, w.grp_sync, n_p / s.K,
                           w.ring_epoch, n_pool, w.pool);
    return hipGetLastError();
}

}  // namespace mac
