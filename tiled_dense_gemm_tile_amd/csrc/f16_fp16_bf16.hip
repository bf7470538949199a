// Kernel instances: fp16 inputs, bf16 output.
#define TG_FP16 true
#define TG_OUT_BF16 true
#define TG_F16_INSTANCE
#include "f16_launch.hpp"
