// Split-KV decode partials for 16-bit inputs on gfx950 (FlashDecoding:
// RedFuser Fig. 13; AttnFuse Table 8, Q.N = 1 over a large KV cache).
//
// Decode reads every K/V byte once and does 4 flops per byte, so HBM bounds
// it; the matrix cores are used here only to keep the vector ALUs free, so
// that the kernel is a pure stream.  One work-group handles one (key chunk,
// KV head, batch) and ALL query rows that read that KV head (the G = Hq/Hkv
// heads of a GQA group times the Nq query positions, at most 16), so every
// K/V byte is fetched from HBM exactly once.
//
// Each wavefront streams its own 32-key sub-blocks of the chunk and keeps an
// incremental (m, l, O) per query row (RedFuser Fig. 4b):
//   S^T = K . Q^T on MFMA 16x16x32 with A = K loaded straight from HBM into
//   registers (lane: key l%16, 8 consecutive d) and B = Q^T (lane: query row
//   l%16), so every lane owns one query row (the MFMA's 16 columns);
//   O^T += V^T . P^T on the same MFMA: V is written row-major into a
//   wave-private LDS buffer and read back transposed (ds_read_b64_tr_b16),
//   P^T comes straight from the score registers.
// No work-group barrier is needed in the loop.  At the end the four waves'
// states are combined with the rescale-and-add rule of RedFuser Table 1
// (max/+ for m, +/* for l and O) through LDS, and the chunk's normalised O and
// natural-log lse are written.
#pragma once

#include "common.hpp"

namespace rf {

constexpr int DM_THREADS = 256;
constexpr int DM_WAVES = DM_THREADS / 64;
constexpr int DM_SUB = 32;        // keys per wave per step
constexpr int DM_MAX_ROWS = 16;   // query rows per KV head served at once

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T, int D, bool ROPE, bool ALIBI>
__global__ __launch_bounds__(DM_THREADS) void attn_decode_mfma_kernel(AttnParams p) {
    static_assert(sizeof(T) == 2, "16-bit inputs only");
    constexpr bool SPLITK = ROPE && !__is_same(T, _Float16);
    constexpr int NKS = D / 32;             // contraction steps over d
    constexpr int NDB = D / 16;             // 16-wide d blocks of O^T
    constexpr int VS = D + 8;               // LDS row pitch of V (elements)
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int VLD = DM_SUB * CPR / 64;  // V chunks per lane per step
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.6931471805599453f;
    constexpr float RESCALE_SLACK = 8.0f;
    typedef typename Vec16<T>::type VecT;
    static_assert(DM_SUB * VS * sizeof(T) >= DM_MAX_ROWS * D * sizeof(float), "V buffer must hold a wave's O at the end");

    __shared__ __attribute__((aligned(16))) T vbuf[DM_WAVES][DM_SUB * VS];
    __shared__ float red_m[DM_WAVES][DM_MAX_ROWS];
    __shared__ float red_l[DM_WAVES][DM_MAX_ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;   // MFMA column: query row of this lane
    const int q = lane >> 4;   // lane group: contraction slots 8q..8q+7

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int G = p.Hq / p.Hkv;
    const int rows = G * p.Nq;  // <= DM_MAX_ROWS, checked on the host
    const int pos_off = p.Nk - p.Nq;

    int klo = split * p.split_len;
    int khi = min(p.Nk, klo + p.split_len);
    if (p.mask != RF_MASK_NONE) khi = min(khi, (p.Nq - 1) + pos_off + 1);
    if (p.mask == RF_MASK_SLIDING) klo = max(klo, pos_off - p.window + 1);

    const float c = fmaxf(p.scale * LOG2E, 1e-30f);
    const size_t kv_base = ((size_t)b * p.Hkv + g) * (size_t)p.Nk * D;
    // K and V of this (batch, KV head); rows past Nk read as zeros.  Rows in
    // [khi, Nk) belong to the next chunk: they are loaded but masked out.
    const int kv_bytes = p.Nk * D * (int)sizeof(T);

    // ---- this lane's query row: head g*G + n/Nq, query n%Nq
    const bool row_ok = n < rows;
    const int gi = row_ok ? n / p.Nq : 0, qi = row_ok ? n % p.Nq : 0;
    const int my_pos = qi + pos_off;
    const int lim_hi = p.mask != RF_MASK_NONE ? min(khi - 1, my_pos) : khi - 1;
    const int lim_lo = p.mask == RF_MASK_SLIDING ? my_pos - p.window + 1 : -(1 << 30);
    const float slope2 = ALIBI ? p.alibi[g * G + gi] * LOG2E : 0.f;  // log2 units

    // Q is loaded first and converted after the first K/V loads are issued
    VecT qraw[NKS];
    {
        const T* qrow = (const T*)p.q + (((size_t)b * p.Hq + g * G + gi) * p.Nq + qi) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qraw[ks] = *(const VecT*)(qrow + 32 * ks + 8 * q);
    }

    // K into A-operand registers, V into registers bound for LDS.  Each set is
    // reloaded for the wave's next sub-block as soon as this one has consumed
    // it, so the loads stay in flight under the softmax and P.V of this step.
    // The loads are issued unconditionally (no branch for the compiler's wait
    // counting to merge); past the wave's last sub-block they go through a
    // zero-size descriptor, which returns zeros without touching memory.
    VecT ka[2][NKS];
    uint4 vr[VLD];
    auto load_k = [&](int k0, bool live) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((const T*)p.k + kv_base, live ? kv_bytes : 0);
#pragma unroll
        for (int kgp = 0; kgp < 2; ++kgp) {
            const int key = k0 + 16 * kgp + n;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                ka[kgp][ks] = __builtin_bit_cast(VecT, buf_load16(rs, ((unsigned)key * D + 32 * ks + 8 * q) * (unsigned)sizeof(T)));
        }
    };
    auto load_v = [&](int k0, bool live) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((const T*)p.v + kv_base, live ? kv_bytes : 0);
#pragma unroll
        for (int it = 0; it < VLD; ++it) {
            const int u = it * 64 + lane;
            vr[it] = buf_load16(rs, ((unsigned)(k0 + u / CPR) * D + (u % CPR) * 8) * (unsigned)sizeof(T));
        }
    };
    constexpr int STRIDE = DM_SUB * DM_WAVES;
    const int k_first = klo + DM_SUB * wave;
    load_k(k_first, k_first < khi);
    load_v(k_first, k_first < khi);
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the wait on Q

    // Q^T operand: lane holds q[row][32*ks + 8*q + i]; RoPE partner is ks +- NKS/2.
    VecT qv[NKS], qlo[SPLITK ? NKS : 1];
    {
        float qf[NKS][8];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) qf[ks][i] = row_ok ? to_f32(qraw[ks][i]) : 0.f;
        if (ROPE) {
#pragma unroll
            for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float cs, sn;
                    rope_cos_sin(p.rope.inv_period[32 * ks + 8 * q + i], my_pos, cs, sn);
                    const float x = qf[ks][i], y = qf[ks + NKS / 2][i];
                    qf[ks][i] = x * cs - y * sn;
                    qf[ks + NKS / 2][i] = x * sn + y * cs;
                }
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qv[ks][i] = from_f32<T>(qf[ks][i]);
                if constexpr (SPLITK) qlo[ks][i] = from_f32<T>(qf[ks][i] - to_f32(qv[ks][i]));
            }
    }
    double ipd[ROPE ? NKS / 2 * 8 : 1];
    if (ROPE) {
#pragma unroll
        for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) ipd[8 * ks + i] = p.rope.inv_period[32 * ks + 8 * q + i];
    }

    f32x4 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};
    float m_ref = -INFINITY, l_run = 0.f;

    T* vb = vbuf[wave];
    // transpose-read addressing: lane j = lane%16 of group q names
    // V[32s + 16h + 4q + j/4][16db + 4(j%4)] and receives V[32s + 16h + 4q + k][16db + n]
    const int tr_row = 4 * q + (n >> 2);
    const int tr_col = 4 * (n & 3);


    for (int k0 = k_first; k0 < khi; k0 += STRIDE) {
        const bool more = k0 + STRIDE < khi;

        // ---- RoPE on K (pairs are in-lane: ks and ks + NKS/2)
        VecT kalo[SPLITK ? 2 : 1][SPLITK ? NKS : 1];
        if (ROPE) {
#pragma unroll
            for (int kgp = 0; kgp < 2; ++kgp) {
                const int key = k0 + 16 * kgp + n;
#pragma unroll
                for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        float cs, sn;
                        rope_cos_sin(ipd[8 * ks + i], key, cs, sn);
                        const float x = to_f32(ka[kgp][ks][i]), y = to_f32(ka[kgp][ks + NKS / 2][i]);
                        const float xr = x * cs - y * sn, yr = x * sn + y * cs;
                        ka[kgp][ks][i] = from_f32<T>(xr);
                        ka[kgp][ks + NKS / 2][i] = from_f32<T>(yr);
                        if constexpr (SPLITK) {
                            kalo[kgp][ks][i] = from_f32<T>(xr - to_f32(ka[kgp][ks][i]));
                            kalo[kgp][ks + NKS / 2][i] = from_f32<T>(yr - to_f32(ka[kgp][ks + NKS / 2][i]));
                        }
                    }
            }
        }

        // ---- S^T = K . Q^T: register i of group kgp is key k0 + 16*kgp + 4*q + i, row n
        f32x4 sacc[2];
#pragma unroll
        for (int kgp = 0; kgp < 2; ++kgp) {
            sacc[kgp] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                sacc[kgp] = mfma16(ka[kgp][ks], qv[ks], sacc[kgp]);
                if constexpr (SPLITK) {
                    sacc[kgp] = mfma16(ka[kgp][ks], qlo[ks], sacc[kgp]);
                    sacc[kgp] = mfma16(kalo[kgp][ks], qv[ks], sacc[kgp]);
                }
            }
        }

        load_k(k0 + STRIDE, more);

        // ---- V tile into this wave's LDS buffer (row-major, padded rows)
#pragma unroll
        for (int it = 0; it < VLD; ++it) {
            const int u = it * 64 + lane;
            *(uint4*)(vb + (u / CPR) * VS + (u % CPR) * 8) = vr[it];
        }
        load_v(k0 + STRIDE, more);

        // ---- mask (ragged chunk end and causal / window bounds), tile max
        const int rel_hi = lim_hi - k0 - 4 * q;
        const int rel_lo = lim_lo - k0 - 4 * q;
        float mx = -INFINITY;
        const float kd = (float)(k0 + 4 * q - my_pos);
#pragma unroll
        for (int kgp = 0; kgp < 2; ++kgp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = 16 * kgp + i;
                float sv = sacc[kgp][i];
                if constexpr (ALIBI) sv = fmaf(sv, c, -slope2 * fabsf(kd + (float)off));
                sacc[kgp][i] = ((off <= rel_hi) & (off >= rel_lo)) ? sv : -INFINITY;
                mx = fmaxf(mx, sacc[kgp][i]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_tile = ALIBI ? mx : mx * c;

        const bool bump = m_tile > m_ref + RESCALE_SLACK;
        if (__builtin_amdgcn_ballot_w64(bump)) {
            const float m_new = bump ? m_tile : m_ref;
            const float alpha = bump ? fast_exp2(m_ref - m_new) : 1.f;
            m_ref = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
        const float m_sub = (m_ref == -INFINITY) ? 0.f : m_ref;

        // P^T operand: slot (q, i) holds key 16*(i/4) + 4*q + i%4 of this step
        VecT pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sv = sacc[i / 4][i % 4];
            pb[i] = from_f32<T>(fast_exp2(ALIBI ? sv - m_sub : fmaf(sv, c, -m_sub)));
        }
        l_run = row_sum8(pb, l_run);

        // the V stores above must land before the transposed reads below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        const T* vrow = vb + tr_row * VS + tr_col;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const i16x4 lo4 = lds_read_tr16(vrow + 16 * db);
            const i16x4 hi4 = lds_read_tr16(vrow + 16 * VS + 16 * db);
            const i16x8 ab = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = mfma16(__builtin_bit_cast(VecT, ab), pb, oacc[db]);
        }
        // the next step overwrites vb: its reads above must be done first
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }

    // ---- combine the four waves: row sums across the lane groups, then LDS
    float l_wave = l_run + __shfl_xor(l_run, 16, 64);
    l_wave += __shfl_xor(l_wave, 32, 64);
    __syncthreads();  // every wave is done with its V buffer
    float* ob = (float*)vb;  // this wave's O^T as [row][d] float32
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[n * D + 16 * db + 4 * q + i] = oacc[db][i];
    if (q == 0) {
        red_m[wave][n] = m_ref;
        red_l[wave][n] = l_wave;
    }
    __syncthreads();
    for (int idx = tid; idx < rows * D; idx += DM_THREADS) {
        const int r = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < DM_WAVES; ++w) M = fmaxf(M, red_m[w][r]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float l = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < DM_WAVES; ++w) {
            const float a = fast_exp2(red_m[w][r] - Mu);
            l = fmaf(red_l[w][r], a, l);
            o = fmaf(((const float*)vbuf[w])[r * D + d], a, o);
        }
        const int rgi = r / p.Nq, rqi = r % p.Nq;
        const size_t row_id = ((size_t)b * p.Hq + g * G + rgi) * p.Nq + rqi;
        const bool live = l > 0.f;
        p.o_part[(row_id * p.num_splits + split) * D + d] = live ? o / l : 0.f;
        if (d == 0) p.lse_part[row_id * p.num_splits + split] = live ? (M + fast_log2(l)) * LN2 : -INFINITY;
    }
}

}  // namespace rf
