// Kernel instances for float32 inputs.
#include "instances.hpp"
RF_DEFINE_LAUNCHERS(f32, float)
