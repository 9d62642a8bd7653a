// Log-sum-exp merge of split-KV partials (RedFuser Fig. 13; the level-1 max
// and level-2 sum of the cascade applied over chunks, RedFuser Fig. 4):
//   M = max_c lse_c,  lse = M + ln sum_c exp(lse_c - M),
//   O = sum_c exp(lse_c - lse) O_c,  rounded once to the output dtype.
// One work-group per row.  Each wavefront reduces the row's chunk lse values
// (max, then the sum of 2^(lse_c - max)) across its lanes; the threads split
// the chunks into NSL slices, each thread taking 4 consecutive d of its chunks
// with 16-byte loads (its first chunks issued together with the reduction's
// loads), and the slices are summed through LDS.
#pragma once

#include "common.hpp"

namespace rf {

constexpr int MRG_THREADS = 256;

// Wavefront-wide max and sum with DPP moves inside 16-lane rows (quad xor 1,
// quad xor 2, half-row mirror, row mirror), then the exchanges 16 and 32 lanes
// away; each step combines the same two values in both lanes of a pair, so
// every lane ends with identical bits.
template <int CTRL>
__device__ __forceinline__ float merge_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float merge_wave_max(float v) {
    v = fmaxf(v, merge_dpp<0xB1>(v));
    v = fmaxf(v, merge_dpp<0x4E>(v));
    v = fmaxf(v, merge_dpp<0x141>(v));
    v = fmaxf(v, merge_dpp<0x140>(v));
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, swap_halves(v));
}
__device__ __forceinline__ float merge_wave_sum(float v) {
    v += merge_dpp<0xB1>(v);
    v += merge_dpp<0x4E>(v);
    v += merge_dpp<0x141>(v);
    v += merge_dpp<0x140>(v);
    v += __shfl_xor(v, 16, 64);
    return v + swap_halves(v);
}

template <typename T, int D>
__global__ __launch_bounds__(MRG_THREADS) void lse_merge_kernel(const float* __restrict__ o_part,
                                                                const float* __restrict__ lse_part,
                                                                T* __restrict__ o, float* __restrict__ lse,
                                                                int rows, int S) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.6931471805599453f;
    constexpr int TPS = D / 4;               // threads per slice (4 d each)
    constexpr int NSL = MRG_THREADS / TPS;   // chunk slices
    __shared__ float4 part[NSL][TPS];

    const size_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int slice = tid / TPS;
    const int d4 = tid % TPS;
    const float* lp = lse_part + row * S;

    // The first PB chunks of this thread's slice (O partial and chunk lse) are
    // loaded before the row's lse reduction, so their latency overlaps the
    // reduction's own loads: a row of at most 64 chunks (PB * NSL >= 64) is
    // merged after one round trip to memory.
    // (Buffer loads: a chunk past S reads zeros without a branch, so no wait
    // separates these loads; its weight is zeroed below.)
    constexpr int PB = 8;
    const int lane = tid & 63;
    float4 xo[PB];
    float xl[PB], l0;
    const float4* op = (const float4*)(o_part + row * (size_t)S * D) + d4;
    {
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(o_part + row * (size_t)S * D, S * D * (int)sizeof(float));
        const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lp, S * (int)sizeof(float));
#pragma unroll
        for (int k = 0; k < PB; ++k) {
            const unsigned c = (unsigned)(slice + NSL * k);
            xo[k] = __builtin_bit_cast(float4, buf_load16(ors, (c * D + 4u * d4) * (unsigned)sizeof(float)));
            xl[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, (int)(c * sizeof(float)), 0, 0));
        }
        l0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, (int)(lane * sizeof(float)), 0, 0));
    }

    // level 1 and level 2 over the chunks (log2 units): every wavefront takes
    // the row's chunk lse values one per lane (chunks c, c + 64, ...) and
    // reduces them with lane butterflies, so all lanes hold the same bits
    float m = lane < S ? l0 * LOG2E : -INFINITY;
    for (int c = lane + 64; c < S; c += 64) m = fmaxf(m, lp[c] * LOG2E);
    m = merge_wave_max(m);
    const bool live = m != -INFINITY;
    float tot = 0.f;
    if (live) {
        tot = lane < S ? fast_exp2(fmaf(l0, LOG2E, -m)) : 0.f;
        for (int c = lane + 64; c < S; c += 64) tot += fast_exp2(fmaf(lp[c], LOG2E, -m));
    }
    tot = merge_wave_sum(tot);
    const float lse2 = live ? m + fast_log2(tot) : 0.f;

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
#pragma unroll
        for (int k = 0; k < PB; ++k) {
            // empty chunk: 2^-inf = 0; a chunk past S (read as zeros) gets weight 0
            const float w = slice + NSL * k < S ? fast_exp2(fmaf(xl[k], LOG2E, -lse2)) : 0.f;
            acc.x = fmaf(w, xo[k].x, acc.x);
            acc.y = fmaf(w, xo[k].y, acc.y);
            acc.z = fmaf(w, xo[k].z, acc.z);
            acc.w = fmaf(w, xo[k].w, acc.w);
        }
#pragma unroll 8
        for (int c = slice + NSL * PB; c < S; c += NSL) {
            const float w = fast_exp2(fmaf(lp[c], LOG2E, -lse2));
            const float4 x = op[(size_t)c * TPS];
            acc.x = fmaf(w, x.x, acc.x);
            acc.y = fmaf(w, x.y, acc.y);
            acc.z = fmaf(w, x.z, acc.z);
            acc.w = fmaf(w, x.w, acc.w);
        }
    }
    part[slice][d4] = acc;
    __syncthreads();
    if (slice == 0) {
        float4 s = part[0][d4];
#pragma unroll
        for (int k = 1; k < NSL; ++k) {
            const float4 y = part[k][d4];
            s.x += y.x;
            s.y += y.y;
            s.z += y.z;
            s.w += y.w;
        }
        typedef T T4 __attribute__((ext_vector_type(4)));
        T4 w;
        w[0] = from_f32<T>(s.x);
        w[1] = from_f32<T>(s.y);
        w[2] = from_f32<T>(s.z);
        w[3] = from_f32<T>(s.w);
        *(T4*)(o + row * D + 4 * d4) = w;
        if (d4 == 0) lse[row] = live ? lse2 * LN2 : -INFINITY;
    }
}

}  // namespace rf
