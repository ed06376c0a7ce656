// Host launchers of the one-launch step kernel for one (K/V dtype, head
// dim): included by mac_step_<dtype>_<dim>.hip, which names the pair with
// MAC_STEP_INSTANCE.
#pragma once

#include "mac_device.h"

namespace mac {
namespace {

// Grid of the single-launch step: a.wpg workgroups per KV group (the host
// sized wpg to what is resident at once).
template <class T, int D, int G, bool P>
static void step_go_gp(const StepArgs &a, hipStream_t st)
{
    const int grid = a.wpg * a.s.B * a.s.Hkv;
    constexpr int eb = sizeof(typename T::S);
    if (a.group_only)
        hipLaunchKernelGGL((step_kernel<T, D, G, step_rows(eb, D, 0), P, false>), dim3(grid),
                           dim3(kBlock), 0, st, a);
    else if (a.unit_slots == step_unit_slots(eb, D, 0))
        hipLaunchKernelGGL((step_kernel<T, D, G, step_rows(eb, D, 0), P, true>), dim3(grid),
                           dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((step_kernel<T, D, G, step_rows(eb, D, 1), P, true>), dim3(grid),
                           dim3(kBlock), 0, st, a);
}
template <class T, int D, int G>
static void step_go_g(const StepArgs &a, hipStream_t st)
{
    if (a.s.page_table)
        step_go_gp<T, D, G, true>(a, st);
    else
        step_go_gp<T, D, G, false>(a, st);
}

template <class T, int D>
static void step_go(const StepArgs &a, hipStream_t st)
{
    switch (a.s.G) {
    case 1:
        step_go_g<T, D, 1>(a, st);
        break;
    case 2:
        step_go_g<T, D, 2>(a, st);
        break;
    case 4:
        step_go_g<T, D, 4>(a, st);
        break;
    default:
        step_go_g<T, D, 8>(a, st);
        break;
    }
}

// Resident workgroups of one instantiation on this device.
template <class T, int D, int U, bool P, bool M>
static int step_resident_upm(const Shape &s)
{
    const void *fn = s.G == 1   ? (const void *)step_kernel<T, D, 1, U, P, M>
                     : s.G == 2 ? (const void *)step_kernel<T, D, 2, U, P, M>
                     : s.G == 4 ? (const void *)step_kernel<T, D, 4, U, P, M>
                                : (const void *)step_kernel<T, D, 8, U, P, M>;
    return device_cu_count() * resident_per_cu(fn, 0);
}
// The group kernel of the two-kernel form has no match units: one
// instantiation (the small unit size's) serves both.
template <class T, int D, int U, bool M>
static int step_resident_um(const Shape &s)
{
    return s.page_table ? step_resident_upm<T, D, U, true, M>(s)
                        : step_resident_upm<T, D, U, false, M>(s);
}
template <class T, int D>
static void step_resident_go(const Shape &s, int *n)
{
    constexpr int eb = sizeof(typename T::S);
    constexpr int U0 = step_rows(eb, D, 0), U1 = step_rows(eb, D, 1);
    const int a = step_resident_um<T, D, U0, true>(s);
    const int b = step_resident_um<T, D, U1, true>(s);
    const int c = step_resident_um<T, D, U0, false>(s);
    *n = a < b ? (a < c ? a : c) : (b < c ? b : c);
}

// This source file's timeline words (the step kernels of its dtype and
// head dim write them); hipErrorNotSupported in the default build.
static hipError_t timeline_copy(void *host, size_t bytes)
{
#ifdef MAC_TIMELINE
    constexpr size_t cap = sizeof(unsigned long long) * kTimelineWgs * kTimelineSlots;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(timeline_words), bytes < cap ? bytes : cap, 0,
                               hipMemcpyDeviceToHost);
#else
    (void)host;
    (void)bytes;
    return hipErrorNotSupported;
#endif
}

}  // namespace
}  // namespace mac

#define MAC_STEP_INSTANCE(T, D, NAME)                                  \
    namespace mac {                                                    \
    void launch_step_##NAME(const StepArgs &a, hipStream_t st)         \
    {                                                                  \
        step_go<T, D>(a, st);                                          \
    }                                                                  \
    int step_resident_##NAME(const Shape &s)                           \
    {                                                                  \
        int n = 0;                                                     \
        step_resident_go<T, D>(s, &n);                                 \
        return n;                                                      \
    }                                                                  \
    hipError_t timeline_read_##NAME(void *host, size_t bytes)          \
    {                                                                  \
        return timeline_copy(host, bytes);                             \
    }                                                                  \
    }
