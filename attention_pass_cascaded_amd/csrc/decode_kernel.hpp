// Split-KV decode partials for gfx950 (FlashDecoding: RedFuser Fig. 13;
// AttnFuse Table 8, Q.N = 1 over a large KV cache).
//
// Decode reads every K/V byte once and does 4 flops per byte, so it is bound
// by HBM, not by matrix math: this kernel streams K and V with 16-byte
// coalesced loads and does the arithmetic on the vector ALUs.  One work-group
// handles one (batch, KV head, key chunk) and ALL query rows that read that KV
// head (the G = Hq/Hkv heads of a GQA group times the Nq query positions), so
// every K/V byte is fetched exactly once.
//
// Lanes are grouped LPR to a key row; each group owns a strided subset of the
// chunk's keys and keeps its own incremental (m, l, O) state per query row
// (RedFuser Fig. 4b).  At the end the per-group states are combined with the
// same rescale-and-add rule (RedFuser Table 1: max/+ for m, +/* for l and O),
// first across the groups of a wave with lane swaps, then across waves through
// LDS, and the chunk's normalised O and natural-log lse are written.
#pragma once

#include "common.hpp"

namespace rf {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int DEC_NB = 4;  // keys per group processed between rescales

template <typename T, int D>
struct DecCfg {
    static constexpr int EPL = 32 / sizeof(T);         // elements per lane per key row (32 B)
    static constexpr int LPR = D / EPL;                // lanes per key row
    static constexpr int GPW = 64 / LPR;               // key groups per wave
    static constexpr int NG = DEC_THREADS / LPR;       // key groups per work-group
};

template <typename T, int D, int R, bool ROPE, bool ALIBI>
__global__ __launch_bounds__(DEC_THREADS) void attn_decode_kernel(AttnParams p) {
    using C = DecCfg<T, D>;
    constexpr int EPL = C::EPL;
    constexpr int LPR = C::LPR;
    constexpr int NG = C::NG;
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.6931471805599453f;
    typedef typename Vec16<T>::type VecT;
    constexpr int EV = Vec16<T>::n;  // elements per 16-byte load

    __shared__ float red_m[DEC_WAVES][R];
    __shared__ float red_l[DEC_WAVES][R];
    __shared__ __attribute__((aligned(16))) float red_o[DEC_WAVES][R][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane % LPR;          // d slice index
    const int grp = tid / LPR;           // key group in the work-group
    const int d0 = sub * EPL;

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int G = p.Hq / p.Hkv;
    const int rows = G * p.Nq;           // <= R, checked on the host
    const int pos_off = p.Nk - p.Nq;

    int klo = split * p.split_len;
    int khi = min(p.Nk, klo + p.split_len);

    const float c = p.scale * LOG2E;
    const size_t kv_base = ((size_t)b * p.Hkv + g) * (size_t)p.Nk * D;
    const T* __restrict__ kg = (const T*)p.k + kv_base;
    const T* __restrict__ vg = (const T*)p.v + kv_base;

    // ---- query rows r = gi * Nq + qi (head g*G + gi, query qi), this lane's d slice
    float q[R][EPL];
    int qpos[R];
    float slope2[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int gi = r / max(p.Nq, 1), qi = r % max(p.Nq, 1);
        qpos[r] = qi + pos_off;
        slope2[r] = (ALIBI && r < rows) ? p.alibi[g * G + gi] * LOG2E : 0.f;
        if (r < rows) {
            const T* qrow = (const T*)p.q + (((size_t)b * p.Hq + g * G + gi) * p.Nq + qi) * D + d0;
#pragma unroll
            for (int e = 0; e < EPL; e += EV) {
                VecT x = *(const VecT*)(qrow + e);
#pragma unroll
                for (int i = 0; i < EV; ++i) q[r][e + i] = to_f32(x[i]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) q[r][e] = 0.f;
        }
    }

    // RoPE: the partner of element d is d +- D/2, held by lane sub ^ (LPR/2).
    const bool lower = sub < LPR / 2;
    double ipd[ROPE ? EPL : 1];
    if (ROPE) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) ipd[e] = p.rope.inv_period[(d0 + e) % (D / 2)];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float other = __shfl_xor(q[r][e], LPR / 2, 64);
                float cs, sn;
                rope_cos_sin(ipd[e], qpos[r], cs, sn);
                // lower half: x cos - y sin; upper half: y sin + x cos (y = partner)
                q[r][e] = lower ? q[r][e] * cs - other * sn : other * sn + q[r][e] * cs;
            }
    }

    float m_run[R], l_run[R], acc[R][EPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
    }

    // keys visible to some row: tighten the chunk with the mask
    if (p.mask != RF_MASK_NONE) khi = min(khi, (p.Nq - 1) + pos_off + 1);
    if (p.mask == RF_MASK_SLIDING) klo = max(klo, pos_off - p.window + 1);

    for (int base = klo + grp; base < khi; base += DEC_NB * NG) {
        float kx[DEC_NB][EPL], vx[DEC_NB][EPL];
        bool kin[DEC_NB];
#pragma unroll
        for (int u = 0; u < DEC_NB; ++u) {
            const int key = base + u * NG;
            kin[u] = key < khi;
#pragma unroll
            for (int e = 0; e < EPL; e += EV) {
                VecT xk, xv;
                if (kin[u]) {
                    xk = *(const VecT*)(kg + (size_t)key * D + d0 + e);
                    xv = *(const VecT*)(vg + (size_t)key * D + d0 + e);
                } else {
                    xk = VecT{};
                    xv = VecT{};
                }
#pragma unroll
                for (int i = 0; i < EV; ++i) {
                    kx[u][e + i] = to_f32(xk[i]);
                    vx[u][e + i] = to_f32(xv[i]);
                }
            }
            if (ROPE) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const float other = __shfl_xor(kx[u][e], LPR / 2, 64);
                    float cs, sn;
                    rope_cos_sin(ipd[e], key, cs, sn);
                    kx[u][e] = lower ? kx[u][e] * cs - other * sn : other * sn + kx[u][e] * cs;
                }
            }
        }

        // scores for the block, reduced over the LPR lanes of the key row
        float s[R][DEC_NB];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < DEC_NB; ++u) {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) a = fmaf(q[r][e], kx[u][e], a);
#pragma unroll
                for (int w = LPR / 2; w >= 1; w >>= 1) a += __shfl_xor(a, w, 64);
                const int key = base + u * NG;
                bool vis = kin[u];
                if (p.mask != RF_MASK_NONE) vis &= key <= qpos[r];
                if (p.mask == RF_MASK_SLIDING) vis &= key > qpos[r] - p.window;
                if constexpr (ALIBI) a = fmaf(a, c, -slope2[r] * fabsf((float)(key - qpos[r])));
                s[r][u] = vis ? a : -INFINITY;
            }

#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < DEC_NB; ++u) mx = fmaxf(mx, s[r][u]);
            const float m_blk = (mx == -INFINITY) ? -INFINITY : (ALIBI ? mx : mx * c);
            const float m_new = fmaxf(m_run[r], m_blk);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[r] - m_use);
            m_run[r] = m_new;
            float pu[DEC_NB];
            float ls = 0.f;
#pragma unroll
            for (int u = 0; u < DEC_NB; ++u) {
                pu[u] = (s[r][u] == -INFINITY) ? 0.f : fast_exp2(ALIBI ? s[r][u] - m_use : fmaf(s[r][u], c, -m_use));
                ls += pu[u];
            }
            l_run[r] = fmaf(l_run[r], alpha, ls);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float a = acc[r][e] * alpha;
#pragma unroll
                for (int u = 0; u < DEC_NB; ++u) a = fmaf(pu[u], vx[u][e], a);
                acc[r][e] = a;
            }
        }
    }

    // ---- combine the key groups of this wave (same d slice: lanes sub + LPR*k)
#pragma unroll
    for (int w = LPR; w < 64; w <<= 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float mo = __shfl_xor(m_run[r], w, 64);
            const float lo = __shfl_xor(l_run[r], w, 64);
            const float M = fmaxf(m_run[r], mo);
            const float Mu = (M == -INFINITY) ? 0.f : M;
            const float a = fast_exp2(m_run[r] - Mu), ao = fast_exp2(mo - Mu);
            l_run[r] = l_run[r] * a + lo * ao;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float oo = __shfl_xor(acc[r][e], w, 64);
                acc[r][e] = acc[r][e] * a + oo * ao;
            }
            m_run[r] = M;
        }
    }
    if (lane < LPR) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (lane == 0) {
                red_m[wave][r] = m_run[r];
                red_l[wave][r] = l_run[r];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) red_o[wave][r][d0 + e] = acc[r][e];
        }
    }
    __syncthreads();

    // ---- combine the waves and write the chunk's partial
    for (int idx = tid; idx < rows * D; idx += DEC_THREADS) {
        const int r = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, red_m[w][r]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float l = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) {
            const float a = fast_exp2(red_m[w][r] - Mu);
            l = fmaf(red_l[w][r], a, l);
            o = fmaf(red_o[w][r][d], a, o);
        }
        const int gi = r / p.Nq, qi = r % p.Nq;
        const size_t row_id = ((size_t)b * p.Hq + g * G + gi) * p.Nq + qi;
        const bool live = l > 0.f;
        p.o_part[(row_id * p.num_splits + split) * D + d] = live ? o / l : 0.f;
        if (d == 0) p.lse_part[row_id * p.num_splits + split] = live ? (M + fast_log2(l)) * LN2 : -INFINITY;
    }
}

}  // namespace rf
