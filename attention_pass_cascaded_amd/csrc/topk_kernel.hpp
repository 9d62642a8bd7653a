// Softmax followed by TopK for gfx950: a cascade on the max/+ row of RedFuser
// Table 1 (TopK combines with max and shifts with +, like Max and ArgMax).
//
// Per row x of E logits:
//   level 1 (max)   m = max_e x_e
//   level 2 (+)     l = sum_e 2^((x_e - m) log2 e)                 (reads m)
//   level 3 (TopK)  the k largest p_e = 2^((x_e - m) log2 e) / l with indices
//                                                                  (reads m, l)
// A group of LPR lanes per row (16 when E <= 256 and k <= 16, else 64), the
// row held in registers (float32: lane l of the group owns elements l,
// l + LPR, ...; 16-bit: VPL consecutive elements per lane): the row is read
// from HBM once and every level runs on it in place.  The k
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
                                                                    int k, int /*vec*/) {
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

// ---------------------------------------------------------------------------
// 16-bit inputs: every element becomes one 32-bit key
//   key = (order-preserving bits of x) << 16 | (0xFFFF - e),
// so "larger value, then lower index" is plain unsigned order and each
// comparison of the selection is a single v_max_u32.  The row-group
// reductions use DPP lane moves inside a 16-lane row (quad xor 1, quad xor 2,
// half-row mirror, row mirror: after the four steps every lane of the row
// holds the row's result) instead of LDS permutes; a 64-lane group adds two
// exchanges across rows.  The first winner is the row max m, so level 1 needs
// no pass of its own.

// x's bits mapped so that unsigned order is the order of the values; -0 and
// +0 share a key.  Finite inputs only (NaN has no place in the order).
__device__ __forceinline__ unsigned topk_mono16(unsigned b) {
    b = (b == 0x8000u) ? 0u : b;
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
__device__ __forceinline__ unsigned topk_unmono16(unsigned m) {
    return (m & 0x8000u) ? (m & 0x7FFFu) : (~m & 0xFFFFu);
}

template <int CTRL>
__device__ __forceinline__ unsigned topk_dpp(unsigned x) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// max over the row group of LPR lanes (16 or 64), in every lane of the group
template <int LPR>
__device__ __forceinline__ unsigned topk_group_max(unsigned v) {
    v = max(v, topk_dpp<DPP_QUAD_XOR1>(v));
    v = max(v, topk_dpp<DPP_QUAD_XOR2>(v));
    v = max(v, topk_dpp<DPP_ROW_HALF_MIRROR>(v));
    v = max(v, topk_dpp<DPP_ROW_MIRROR>(v));
    if constexpr (LPR == 64) {
        v = max(v, (unsigned)__shfl_xor((int)v, 16, 64));
        v = max(v, (unsigned)__shfl_xor((int)v, 32, 64));
    }
    return v;
}
// sum over the row group; every lane gets the same bits (each step adds the
// same two partial sums in every lane)
template <int LPR>
__device__ __forceinline__ float topk_group_sum(float v) {
    v += __uint_as_float(topk_dpp<DPP_QUAD_XOR1>(__float_as_uint(v)));
    v += __uint_as_float(topk_dpp<DPP_QUAD_XOR2>(__float_as_uint(v)));
    v += __uint_as_float(topk_dpp<DPP_ROW_HALF_MIRROR>(__float_as_uint(v)));
    v += __uint_as_float(topk_dpp<DPP_ROW_MIRROR>(__float_as_uint(v)));
    if constexpr (LPR == 64) {
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
    }
    return v;
}

// vec: E is a multiple of 8 and x is 16-byte aligned, so with VPL a
// multiple of 8 each lane reads its elements as whole 16-byte chunks.
template <typename T, int VPL, int LPR>
__global__ __launch_bounds__(TOPK_THREADS) void softmax_topk16_kernel(const T* __restrict__ x, float* __restrict__ values,
                                                                      int* __restrict__ indices, int rows, int E,
                                                                      int k, int vec) {
    static_assert(sizeof(T) == 2, "16-bit inputs");
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int RPW = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;
    const long long row = ((long long)blockIdx.x * (TOPK_THREADS / 64) + (threadIdx.x >> 6)) * RPW + lane / LPR;
    const bool row_ok = row < rows;
    const unsigned short* xr = (const unsigned short*)x + (row_ok ? row : 0) * (long long)E;

    // lane `sub` of the group owns the VPL consecutive elements from
    // sub * VPL (the selection below does not depend on which lane holds an
    // element: keys carry the index); absent ones get key 0 (below every
    // present key) and x = -inf
    const int e0 = sub * VPL;
    unsigned short raw[VPL];
    if (VPL % 8 == 0 && vec) {
#pragma unroll
        for (int c = 0; c < VPL / 8; ++c) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (e0 + 8 * c < E) u = *(const uint4*)(xr + e0 + 8 * c);  // E % 8 == 0: whole chunk in the row
            const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 8; ++h) raw[8 * c + h] = (unsigned short)(w[h / 2] >> (16 * (h % 2)));
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) raw[i] = xr[min(e0 + i, E - 1)];  // in-row address for every lane
    }
    unsigned key[VPL];
    float xv[VPL];
    unsigned best = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = e0 + i;
        const unsigned b = raw[i];
        xv[i] = e < E ? to_f32(__builtin_bit_cast(T, (unsigned short)b)) : -INFINITY;
        key[i] = e < E ? (topk_mono16(b) << 16) | (0xFFFFu - (unsigned)e) : 0u;
        best = max(best, key[i]);
    }
    // level 1: the first winner is the row max
    unsigned win = topk_group_max<LPR>(best);
    const float m = to_f32(__builtin_bit_cast(T, (unsigned short)topk_unmono16(win >> 16)));
    const float msub = m == -INFINITY ? 0.f : m;
    // level 2: sum of exponentials relative to m
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) l += fast_exp2((xv[i] - msub) * LOG2E);
    l = topk_group_sum<LPR>(l);
    const float inv_l = 1.f / l;

    // level 3: k - 1 more rounds.  Keys are unique and the winners come in
    // decreasing order, so the untaken keys are exactly those below the last
    // winner: each lane's candidate is its largest key below win, found as
    // w1 - min(w1, min(w1 - key)) with w1 = win - 1 in wrapping unsigned
    // arithmetic.  A taken key (>= win) wraps above w1, so a lane with no
    // untaken key keeps t = w1 and offers 0.  win > 0 in every round since
    // k <= E and every present key is nonzero.
    unsigned mine = sub == 0 ? win : 0u;
    for (int j = 1; j < k; ++j) {
        const unsigned w1 = win - 1u;
        unsigned t = w1;
#pragma unroll
        for (int i = 0; i < VPL; ++i) t = min(t, w1 - key[i]);
        win = topk_group_max<LPR>(w1 - t);
        mine = sub == j ? win : mine;
    }
    if (row_ok && sub < k) {
        const float v = to_f32(__builtin_bit_cast(T, (unsigned short)topk_unmono16(mine >> 16)));
        values[row * k + sub] = fast_exp2((v - msub) * LOG2E) * inv_l;
        indices[row * k + sub] = (int)(0xFFFFu - (mine & 0xFFFFu));
    }
}

}  // namespace rf
