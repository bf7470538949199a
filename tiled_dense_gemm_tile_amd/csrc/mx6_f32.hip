// Kernel instances: block-scaled fp6 inputs (e2m3, e3m2), f32 output.
#define TG_OUT_BF16 false
#define TG_MX6_INSTANCE
#include "mx6_launch.hpp"
