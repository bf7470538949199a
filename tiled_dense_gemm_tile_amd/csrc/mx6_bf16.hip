// Kernel instances: block-scaled fp6 inputs (e2m3, e3m2), bf16 output.
#define TG_OUT_BF16 true
#define TG_MX6_INSTANCE
#include "mx6_launch.hpp"
