// LayerNorm forward for gfx950: a second cascaded reduction on the same
// incremental machinery as the attention kernels.
//
// Level 1 is the mean (combine +), level 2 the sum of squared deviations from
// that mean (combine +, reading level 1): the reduction + element-wise
// pattern of the "Operator Fusion" guide (section 2, Pattern 2), a cascade
// in the sense of RedFuser (abstract, Table 1).  As in RedFuser Fig. 4b each
// 16-byte chunk updates a running state (n, mean, M2) in registers: a chunk
// with its own (n_b, mean_b, M2_b) moves the mean by delta = mean_b - mean,
// and M2 gets the correction delta^2 n_a n_b / n, the counterpart of the
// softmax's rescale by 2^(m_old - m_new).  Lanes then merge their states
// with the same rule (butterfly over the wavefront, then across the 4
// wavefronts through LDS), and the row is normalised from the registers it
// was loaded into: x is read from HBM once and y written once.
//
// One work-group of 256 threads per row; thread t owns the 16-byte chunks
// t, t + 256, ... (NCH of them), so H <= 256 * NCH * (16 / sizeof(T)).
#pragma once

#include "common.hpp"

namespace rf {

constexpr int LN_THREADS = 256;
constexpr int LN_MAX_CHUNKS = 8;

struct LnState {
    float n, mean, m2;
};

// Merge of two partial states of one row.  Deterministic for a given
// argument order; callers always pass the lower-indexed part first.
__device__ __forceinline__ LnState ln_combine(const LnState& a, const LnState& b) {
    const float n = a.n + b.n;
    if (n == 0.f) return a;
    const float delta = b.mean - a.mean;
    const float wb = b.n / n;
    return {n, fmaf(delta, wb, a.mean), a.m2 + b.m2 + delta * delta * a.n * wb};
}

template <typename T, int NCH>
__global__ __launch_bounds__(LN_THREADS) void layernorm_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                                                               const T* __restrict__ beta, T* __restrict__ y,
                                                               float* __restrict__ mean_out,
                                                               float* __restrict__ rstd_out, int H, float eps) {
    typedef typename Vec16<T>::type VecT;
    constexpr int EPC = Vec16<T>::n;
    __shared__ LnState part[LN_THREADS / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t row = blockIdx.x;
    const T* xr = x + row * (size_t)H;
    const int nchunks = H / EPC;

    VecT v[NCH];
    LnState st = {0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * LN_THREADS;
        if (c < nchunks) {
            v[i] = *(const VecT*)(xr + c * EPC);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) s += to_f32(v[i][e]);
            const float mb = s * (1.f / EPC);
            float m2 = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const float d = to_f32(v[i][e]) - mb;
                m2 = fmaf(d, d, m2);
            }
            st = ln_combine(st, LnState{(float)EPC, mb, m2});
        }
    }
    // butterfly over the wavefront, lower lane's state first on both sides
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const LnState o = {__shfl_xor(st.n, off, 64), __shfl_xor(st.mean, off, 64), __shfl_xor(st.m2, off, 64)};
        st = (lane & off) ? ln_combine(o, st) : ln_combine(st, o);
    }
    if (lane == 0) part[wave] = st;
    __syncthreads();
    st = part[0];
#pragma unroll
    for (int w = 1; w < LN_THREADS / 64; ++w) st = ln_combine(st, part[w]);

    const float mean = st.mean;
    const float rstd = 1.f / sqrtf(st.m2 / (float)H + eps);
    T* yr = y + row * (size_t)H;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + i * LN_THREADS;
        if (c < nchunks) {
            const VecT g = *(const VecT*)(gamma + c * EPC);
            const VecT b = *(const VecT*)(beta + c * EPC);
            VecT o;
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                o[e] = from_f32<T>(fmaf((to_f32(v[i][e]) - mean) * rstd, to_f32(g[e]), to_f32(b[e])));
            *(VecT*)(yr + c * EPC) = o;
        }
    }
    if (tid == 0) {
        mean_out[row] = mean;
        rstd_out[row] = rstd;
    }
}

}  // namespace rf
