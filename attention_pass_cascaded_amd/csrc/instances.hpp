// Template instantiation and dispatch on (D, RoPE, rows) for one dtype.
#pragma once

#include "decode_kernel.hpp"
#include "decode_mfma_kernel.hpp"
#include "fwd_kernel.hpp"
#include "launch.hpp"

namespace rf {

template <typename T, int D, bool ROPE, bool ALIBI>
hipError_t fwd_launch_one(const AttnParams& p, hipStream_t s) {
    dim3 grid((unsigned)(p.B * p.Hq * p.num_splits * ((p.Nq + FWD_BM - 1) / FWD_BM)));
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, ROPE, ALIBI>), grid, dim3(FWD_THREADS), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t fwd_dispatch_d(const AttnParams& p, hipStream_t s) {
    const bool rope = p.rope_base > 0.f;
    if (p.alibi) return rope ? fwd_launch_one<T, D, true, true>(p, s) : fwd_launch_one<T, D, false, true>(p, s);
    return rope ? fwd_launch_one<T, D, true, false>(p, s) : fwd_launch_one<T, D, false, false>(p, s);
}

template <typename T>
hipError_t fwd_dispatch(const AttnParams& p, hipStream_t s) {
    return p.D == 64 ? fwd_dispatch_d<T, 64>(p, s) : fwd_dispatch_d<T, 128>(p, s);
}

template <typename T, int D, int R>
hipError_t dec_launch_rows(const AttnParams& p, hipStream_t s) {
    dim3 grid((unsigned)p.num_splits, (unsigned)p.Hkv, (unsigned)p.B);
    const bool rope = p.rope_base > 0.f;
    if (p.alibi) {
        if (rope) hipLaunchKernelGGL((attn_decode_kernel<T, D, R, true, true>), grid, dim3(DEC_THREADS), 0, s, p);
        else hipLaunchKernelGGL((attn_decode_kernel<T, D, R, false, true>), grid, dim3(DEC_THREADS), 0, s, p);
    } else {
        if (rope) hipLaunchKernelGGL((attn_decode_kernel<T, D, R, true, false>), grid, dim3(DEC_THREADS), 0, s, p);
        else hipLaunchKernelGGL((attn_decode_kernel<T, D, R, false, false>), grid, dim3(DEC_THREADS), 0, s, p);
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t dec_launch_d(const AttnParams& p, hipStream_t s) {
    const int rows = (p.Hq / p.Hkv) * p.Nq;
    if (rows <= 1) return dec_launch_rows<T, D, 1>(p, s);
    if (rows <= 4) return dec_launch_rows<T, D, 4>(p, s);
    return dec_launch_rows<T, D, 8>(p, s);
}

template <typename T, int D>
hipError_t dec_mfma_launch_d(const AttnParams& p, hipStream_t s) {
    dim3 grid((unsigned)p.num_splits, (unsigned)p.Hkv, (unsigned)p.B);
    const bool rope = p.rope_base > 0.f;
    if (p.alibi) {
        if (rope) hipLaunchKernelGGL((attn_decode_mfma_kernel<T, D, true, true>), grid, dim3(DM_THREADS), 0, s, p);
        else hipLaunchKernelGGL((attn_decode_mfma_kernel<T, D, false, true>), grid, dim3(DM_THREADS), 0, s, p);
    } else {
        if (rope) hipLaunchKernelGGL((attn_decode_mfma_kernel<T, D, true, false>), grid, dim3(DM_THREADS), 0, s, p);
        else hipLaunchKernelGGL((attn_decode_mfma_kernel<T, D, false, false>), grid, dim3(DM_THREADS), 0, s, p);
    }
    return hipGetLastError();
}

// 16-bit inputs: matrix-core streaming kernel (<= 16 rows per KV head);
// float32 inputs: vector-ALU streaming kernel (<= 8 rows per KV head).
template <typename T>
hipError_t dec_dispatch(const AttnParams& p, hipStream_t s) {
    if constexpr (sizeof(T) == 2)
        return p.D == 64 ? dec_mfma_launch_d<T, 64>(p, s) : dec_mfma_launch_d<T, 128>(p, s);
    else
        return p.D == 64 ? dec_launch_d<T, 64>(p, s) : dec_launch_d<T, 128>(p, s);
}

}  // namespace rf

#define RF_DEFINE_LAUNCHERS(SUFFIX, TYPE)                                                          \
    namespace rf {                                                                                 \
    hipError_t launch_fwd_##SUFFIX(const AttnParams& p, hipStream_t s) { return fwd_dispatch<TYPE>(p, s); } \
    hipError_t launch_decode_##SUFFIX(const AttnParams& p, hipStream_t s) { return dec_dispatch<TYPE>(p, s); } \
    }
