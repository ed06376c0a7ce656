// One-launch step kernels for f32 K/V with head dim 64.
#include "mac_step_impl.h"

MAC_STEP_INSTANCE(F32, 64, f32_64)
