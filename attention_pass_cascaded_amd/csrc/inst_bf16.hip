// Kernel instances for bfloat16 inputs.
#include "instances.hpp"
RF_DEFINE_LAUNCHERS(bf16, __bf16)
RF_DEFINE_BWD_LAUNCHERS(bf16, __bf16)
