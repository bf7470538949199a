// Kernel instances: block-scaled e2m1 inputs, f32 output.
#define TG_OUT_BF16 false
#define TG_MX4_INSTANCE
#include "mx4_launch.hpp"
