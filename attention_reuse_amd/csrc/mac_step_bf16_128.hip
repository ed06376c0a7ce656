// One-launch step kernels for bf16 K/V with head dim 128.
#include "mac_step_impl.h"

MAC_STEP_INSTANCE(BF16, 128, bf16_128)
