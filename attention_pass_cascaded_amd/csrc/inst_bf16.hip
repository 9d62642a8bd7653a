// Kernel instances for bfloat16 inputs.
#include "instances.hpp"
RF_DEFINE_LAUNCHERS(bf16, __bf16)
