// One-launch step kernels for bf16 K/V with head dim 64.
#include "mac_step_impl.h"

MAC_STEP_INSTANCE(BF16, 64, bf16_64)
