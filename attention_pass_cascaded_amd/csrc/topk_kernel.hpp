// Softmax followed by TopK for gfx950: a cascade on the max/+ row of RedFuser
// Table 1 (TopK combines with max and shifts with +, like Max and ArgMax).
//
// Per row x of E logits:
//   level 1 (max)   m = max_e x_e
//   level 2 (+)     l = sum_e 2^((x_e - m) log2 e)                 (reads m)
//   level 3 (TopK)  the k largest p_e = 2^((x_e - m) log2 e) / l with indices
//                                                                  (reads m, l)
// A group of LPR lanes per row (16 when E <= 256 and k <= 16, else 64), the
// row held in registers (lane l of the group owns elements l, l + LPR, ...):
// the row is read from HBM once and every level runs on it in place.  The k
// largest p are the k largest x (exp is increasing), so the selection
// compares the exact input values; ties go to the lower index, which makes
// the result unique.  Each of the k rounds takes the group's best untaken
// element by a butterfly over (value, index) pairs inside the
// row's lane group; lane j keeps the j-th winner and lanes 0..k-1 write.
#pragma once

#include "common.hpp"

namespace rf {

constexpr int TOPK_THREADS = 256;
constexpr int TOPK_MAX_VPL = 16;    // values per lane: E <= 1024
constexpr int TOPK_MAX_K = 64;

// (v, i) beats (w, j): larger value, then lower index
__device__ __forceinline__ bool topk_better(float v, int i, float w, int j) {
    return v > w || (v == w && i < j);
}

// LPR lanes per row (16 or 64): with 16, a wavefront serves 4 rows and every
// butterfly step stays inside a 16-lane row group.
template <typename T, int VPL, int LPR>
__global__ __launch_bounds__(TOPK_THREADS) void softmax_topk_kernel(const T* __restrict__ x, float* __restrict__ values,
                                                                    int* __restrict__ indices, int rows, int E,
                                                                    int k) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int RPW = 64 / LPR;  // rows per wavefront
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;    // lane within the row group
    const long long row = ((long long)blockIdx.x * (TOPK_THREADS / 64) + (threadIdx.x >> 6)) * RPW + lane / LPR;
    const bool row_ok = row < rows;
    const T* xr = x + (row_ok ? row : 0) * (long long)E;

    float xv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = sub + LPR * i;
        xv[i] = e < E ? to_f32(xr[e]) : -INFINITY;
    }
    // level 1: row max
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i) m = fmaxf(m, xv[i]);
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const float msub = m == -INFINITY ? 0.f : m;
    // level 2: sum of exponentials relative to m
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) l += fast_exp2((xv[i] - msub) * LOG2E);
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
    const float inv_l = 1.f / l;

    // level 3: k rounds of a row-group argmax over the untaken elements
    unsigned taken = 0;
    float my_v = 0.f;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = sub + LPR * i;
            if (e < E && !((taken >> i) & 1u) && topk_better(xv[i], e, bv, bi)) {
                bv = xv[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (topk_better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (bi % LPR == sub) taken |= 1u << (bi / LPR);
        if (sub == j) {
            my_v = bv;
            my_i = bi;
        }
    }
    if (row_ok && sub < k) {
        values[row * k + sub] = fast_exp2((my_v - msub) * LOG2E) * inv_l;
        indices[row * k + sub] = my_i;
    }
}

}  // namespace rf
