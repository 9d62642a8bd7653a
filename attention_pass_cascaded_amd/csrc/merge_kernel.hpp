// Log-sum-exp merge of split-KV partials (RedFuser Fig. 13; the level-1 max
// and level-2 sum of the cascade applied over chunks, RedFuser Fig. 4):
//   M = max_c lse_c,  lse = M + ln sum_c exp(lse_c - M),
//   O = sum_c exp(lse_c - lse) O_c,  rounded once to the output dtype.
// One wavefront per row: the chunk loop reads each chunk's D floats with
// consecutive lanes on consecutive d (coalesced).
#pragma once

#include "common.hpp"

namespace rf {

constexpr int MRG_THREADS = 256;
constexpr int MRG_ROWS = MRG_THREADS / 64;

template <typename T, int D>
__global__ __launch_bounds__(MRG_THREADS) void lse_merge_kernel(const float* __restrict__ o_part,
                                                                const float* __restrict__ lse_part,
                                                                T* __restrict__ o, float* __restrict__ lse,
                                                                int rows, int S) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.6931471805599453f;
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const size_t row = (size_t)blockIdx.x * MRG_ROWS + (threadIdx.x >> 6);
    if (row >= (size_t)rows) return;
    const float* lp = lse_part + row * S;

    float M = -INFINITY;
    for (int cidx = lane; cidx < S; cidx += 64) M = fmaxf(M, lp[cidx]);
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w, 64));
    const bool live = M != -INFINITY;
    const float Mu = live ? M : 0.f;

    float tot = 0.f;
    for (int cidx = lane; cidx < S; cidx += 64) tot += fast_exp2((lp[cidx] - Mu) * LOG2E);
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) tot += __shfl_xor(tot, w, 64);
    const float lse_row = live ? Mu + fast_log2(tot) * LN2 : -INFINITY;

    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    if (live) {
        const float* op = o_part + row * S * D;
        for (int cidx = 0; cidx < S; ++cidx) {
            const float w = fast_exp2((lp[cidx] - lse_row) * LOG2E);  // empty chunk: exp2(-inf) = 0
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, op[(size_t)cidx * D + lane + 64 * i], acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) o[row * D + lane + 64 * i] = from_f32<T>(acc[i]);
    if (lane == 0) lse[row] = lse_row;
}

}  // namespace rf
