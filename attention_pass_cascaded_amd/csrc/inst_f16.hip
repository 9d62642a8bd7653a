// Kernel instances for float16 inputs.
#include "instances.hpp"
RF_DEFINE_LAUNCHERS(f16, _Float16)
RF_DEFINE_BWD_LAUNCHERS(f16, _Float16)
