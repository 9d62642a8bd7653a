// Standalone rotary embedding (the "pre-rotate" side of AttnFuse's Rotation
// Calculus: abstract and Table 4 compare fusing RoPE into attention against
// rotating Q and K in a separate pass first).
//
// y[r, n, i]       = x[r, n, i] cos a - x[r, n, i + D/2] sin a
// y[r, n, i + D/2] = x[r, n, i] sin a + x[r, n, i + D/2] cos a
// with a = (pos_offset + n) * base^(-2i/D), i < D/2, for every row r of
// [rows, N, D].  A pass over HBM: each thread reads one 16-byte chunk of the
// first half and its partner chunk of the second half and writes both back,
// so y may alias x.  The angle arithmetic matches the fused kernels (period in
// fp64, sin/cos of the fraction of a revolution), so for 16-bit outputs the
// rotated values are the ones the fused kernels feed to the matrix cores.
#pragma once

#include "common.hpp"

namespace rf {

constexpr int ROPE_THREADS = 256;

template <typename T, int D>
__global__ __launch_bounds__(ROPE_THREADS) void rope_rotate_kernel(const T* x, T* y, long long rows_n, int N,
                                                                   RopeTable rope, int pos_offset) {
    typedef typename Vec16<T>::type VecT;
    constexpr int EPC = Vec16<T>::n;
    constexpr int HALF_CH = D / 2 / EPC;  // chunks per half row

    const long long idx = (long long)blockIdx.x * ROPE_THREADS + threadIdx.x;
    const long long row = idx / HALF_CH;  // row of [rows * N, D]
    if (row >= rows_n) return;
    const int c = (int)(idx % HALF_CH);
    const int pos = pos_offset + (int)(row % N);
    const T* xr = x + row * D + c * EPC;
    T* yr = y + row * D + c * EPC;
    const VecT lo = *(const VecT*)xr;
    const VecT hi = *(const VecT*)(xr + D / 2);
    VecT olo, ohi;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        float cs, sn;
        rope_cos_sin(rope.inv_period[c * EPC + e], pos, cs, sn);
        const float a = to_f32(lo[e]), b = to_f32(hi[e]);
        olo[e] = from_f32<T>(a * cs - b * sn);
        ohi[e] = from_f32<T>(a * sn + b * cs);
    }
    *(VecT*)yr = olo;
    *(VecT*)(yr + D / 2) = ohi;
}

}  // namespace rf
