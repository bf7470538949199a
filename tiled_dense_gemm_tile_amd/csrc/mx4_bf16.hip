// Kernel instances: block-scaled e2m1 inputs, bf16 output.
#define TG_OUT_BF16 true
#define TG_MX4_INSTANCE
#include "mx4_launch.hpp"
