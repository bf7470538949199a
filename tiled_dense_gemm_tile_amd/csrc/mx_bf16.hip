// Kernel instances: block-scaled e4m3 inputs, bf16 output.
#define TG_OUT_BF16 true
#define TG_MX_INSTANCE
#include "mx_launch.hpp"
