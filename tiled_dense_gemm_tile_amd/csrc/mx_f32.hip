// Kernel instances: block-scaled e4m3 inputs, f32 output.
#define TG_OUT_BF16 false
#define TG_MX_INSTANCE
#include "mx_launch.hpp"
