// Internal launchers, one translation unit per input dtype (built in parallel).
#pragma once

#include "common.hpp"

namespace rf {

// Fused forward, or split-KV partials when p.split_mode != 0 (MFMA path).
hipError_t launch_fwd_f32(const AttnParams& p, hipStream_t s);
hipError_t launch_fwd_f16(const AttnParams& p, hipStream_t s);
hipError_t launch_fwd_bf16(const AttnParams& p, hipStream_t s);

// Split-KV partials on the streaming decode kernels; they serve all
// (Hq/Hkv)*Nq query rows of a KV head at once, up to this many.
constexpr int DEC_MAX_ROWS_F32 = 8;
constexpr int DEC_MAX_ROWS_16 = 16;
hipError_t launch_decode_f32(const AttnParams& p, hipStream_t s);
hipError_t launch_decode_f16(const AttnParams& p, hipStream_t s);
hipError_t launch_decode_bf16(const AttnParams& p, hipStream_t s);

// Backward (16-bit inputs): row terms, dk/dv and dq kernels.
struct BwdParams;
hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s);

hipError_t launch_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                        int rows, int S, int D, int dtype, hipStream_t s);

}  // namespace rf
