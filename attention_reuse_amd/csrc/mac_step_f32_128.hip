// One-launch step kernels for f32 K/V with head dim 128.
#include "mac_step_impl.h"

MAC_STEP_INSTANCE(F32, 128, f32_128)
