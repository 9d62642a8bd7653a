// Template instantiation and dispatch on (D, RoPE, rows) for one dtype.
#pragma once

#include <atomic>
#include <cstdlib>

#include "bwd_kernel.hpp"
#include "decode_kernel.hpp"
#include "decode_mfma_kernel.hpp"
#include "fwd_kernel.hpp"
#include "launch.hpp"

namespace rf {

// work-groups of an instance that fit on one CU (cached per instance; the
// same for every gfx950 device); 0 if the query fails
template <typename T, int D, bool ROPE, bool ALIBI, int KH>
int fwd_resident() {
    static std::atomic<int> resident{0};
    int r = resident.load(std::memory_order_relaxed);
    if (r == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, attn_fwd_kernel<T, D, ROPE, ALIBI, KH>,
                                                         FwdLayout<KH>::THREADS, 0) != hipSuccess) {
            r = 0;
            (void)hipGetLastError();  // a failed query only turns the snake order off
        }
        if (r > 0) resident.store(r, std::memory_order_relaxed);
        else r = 0;
    }
    return r;
}

template <typename T, int D, bool ROPE, bool ALIBI, int KH>
hipError_t fwd_launch_one(const AttnParams& p, hipStream_t s) {
    constexpr int BM = FwdLayout<KH>::BM;
    AttnParams q = p;
    q.launch_runs = fwd_resident<T, D, ROPE, ALIBI, KH>();
    dim3 grid((unsigned)(p.B * p.Hq * p.num_splits * ((p.Nq + BM - 1) / BM)));
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, ROPE, ALIBI, KH>), grid, dim3(FwdLayout<KH>::THREADS), 0, s, q);
    return hipGetLastError();
}

// Work-group layout of the 16-bit D = 64 forward (not split mode), from
// same-box timings of the three layouts over grid sizes (g = 128-row query
// blocks, P = CU count, R_k = work-groups of layout k one CU holds):
//  * unmasked and P <= g <= P * R_2 (every 8-wave group resident at launch):
//    layout 2, the 8-wave key halves (B1 H8 N8192: 171 vs 181 us for layout
//    0 and 198 for layout 1; B2 H16 N2048: 47.6 / 49.1 / 53.8; with RoPE, one
//    group per CU, B1 H8 N4096: 63 / 78 / 82);
//  * otherwise layout 1, the 64-row key halves, when 2g <= P * R_1 (causal
//    and windowed masks; unmasked RoPE or ALiBi grids only below one block
//    per CU): it halves the longest chain of tile steps (B1 H8 N4096 causal
//    46 vs 60 us), but its 32-key steps cost more per key once the grid fills
//    the GPU;
//  * else layout 0.
// The environment variable RF_ATTN_KEY_HALVES=0, 1 or 2 forces a layout (read
// at every call).
template <typename T, int D, bool ROPE, bool ALIBI>
hipError_t fwd_launch_pick(const AttnParams& p, hipStream_t s) {
    if constexpr (D == 64 && sizeof(T) == 2) {
        if (!p.split_mode) {
            const char* env = std::getenv("RF_ATTN_KEY_HALVES");
            int kh = 0;
            if (env && env[0] >= '0' && env[0] <= '2' && env[1] == 0) {
                kh = env[0] - '0';
            } else {
                const long long g = (long long)p.B * p.Hq * p.num_splits * ((p.Nq + FWD_BM - 1) / FWD_BM);
                const long long P = p.cu_count;
                const bool uniform = p.mask == RF_MASK_NONE;
                if (uniform && g >= P && g <= P * fwd_resident<T, D, ROPE, ALIBI, 2>())
                    kh = 2;
                else if (g > 0 && 2 * g <= P * fwd_resident<T, D, ROPE, ALIBI, 1>() &&
                         (!uniform || (!ROPE && !ALIBI) || g < P))
                    kh = 1;
            }
            if (kh == 1) return fwd_launch_one<T, D, ROPE, ALIBI, 1>(p, s);
            if (kh == 2) return fwd_launch_one<T, D, ROPE, ALIBI, 2>(p, s);
        }
    }
    return fwd_launch_one<T, D, ROPE, ALIBI, 0>(p, s);
}

template <typename T, int D>
hipError_t fwd_dispatch_d(const AttnParams& p, hipStream_t s) {
    const bool rope = p.rope_base > 0.f;
    if (p.alibi) return rope ? fwd_launch_pick<T, D, true, true>(p, s) : fwd_launch_pick<T, D, false, true>(p, s);
    return rope ? fwd_launch_pick<T, D, true, false>(p, s) : fwd_launch_pick<T, D, false, false>(p, s);
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

// Backward: row terms, then the key-parallel dk/dv kernel and the
// query-parallel dq kernel (independent of each other).
template <typename T, int D, bool ROPE, bool ALIBI>
hipError_t bwd_launch_one(const BwdParams& p, hipStream_t s) {
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    if (rows > 0) {
        const long long threads = rows * (D / 8);
        hipLaunchKernelGGL((bwd_rowterm_kernel<T, D>), dim3((unsigned)((threads + BWD_THREADS - 1) / BWD_THREADS)),
                           dim3(BWD_THREADS), 0, s, (const T*)p.o, (const T*)p.dout, p.drow, rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((long long)p.B * p.Nk > 0) {
        dim3 grid((unsigned)(p.B * p.Hkv * ((p.Nk + BWD_BK - 1) / BWD_BK)));
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, ROPE, ALIBI>), grid, dim3(BWD_THREADS), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (rows > 0) {
        dim3 grid((unsigned)(p.B * p.Hq * ((p.Nq + FWD_BM - 1) / FWD_BM)));
        hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, ROPE, ALIBI>), grid, dim3(FWD_THREADS), 0, s, p);
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_dispatch_d(const BwdParams& p, hipStream_t s) {
    const bool rope = p.rope_base > 0.f;
    if (p.alibi) return rope ? bwd_launch_one<T, D, true, true>(p, s) : bwd_launch_one<T, D, false, true>(p, s);
    return rope ? bwd_launch_one<T, D, true, false>(p, s) : bwd_launch_one<T, D, false, false>(p, s);
}

template <typename T>
hipError_t bwd_dispatch(const BwdParams& p, hipStream_t s) {
    return p.D == 64 ? bwd_dispatch_d<T, 64>(p, s) : bwd_dispatch_d<T, 128>(p, s);
}

}  // namespace rf

#define RF_DEFINE_BWD_LAUNCHERS(SUFFIX, TYPE)                                                      \
    namespace rf {                                                                                 \
    hipError_t launch_bwd_##SUFFIX(const BwdParams& p, hipStream_t s) { return bwd_dispatch<TYPE>(p, s); } \
    }

#define RF_DEFINE_LAUNCHERS(SUFFIX, TYPE)                                                          \
    namespace rf {                                                                                 \
    hipError_t launch_fwd_##SUFFIX(const AttnParams& p, hipStream_t s) { return fwd_dispatch<TYPE>(p, s); } \
    hipError_t launch_decode_##SUFFIX(const AttnParams& p, hipStream_t s) { return dec_dispatch<TYPE>(p, s); } \
    }
