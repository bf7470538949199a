// Kernel instances: fp16 inputs, f32 output.
#define TG_FP16 true
#define TG_OUT_BF16 false
#define TG_F16_INSTANCE
#include "f16_launch.hpp"
