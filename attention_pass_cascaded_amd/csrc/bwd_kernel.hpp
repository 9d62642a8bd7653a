// Attention backward for gfx950: dq, dk, dv of the fused forward, from the
// saved log-sum-exp (AttnFuse abstract and Table 9 run these variants inside
// a forward + backward + optimiser training step).
//
// The gradient is the chain rule through the forward (softmax Jacobian):
//   P = exp(s - lse) (recomputed from the saved lse, never stored),
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D_i),  D_i = dO_i . O_i,
//   dq = R^T scale dS k',  dk = R^T scale dS^T q'   (R: the RoPE rotation).
// Three kernels, no atomics, deterministic:
//   bwd_rowterm_kernel  D_i = dO_i . O_i for every query row;
//   attn_bwd_dq_kernel  one work-group per 128 query rows of a head (lane =
//       query, like the forward): S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T;
//   attn_bwd_dkdv_kernel one work-group per 128 keys of a KV head (lane =
//       key) over every query of every head in its GQA group: S = Q K^T,
//       dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
// All products run on the matrix cores with 16-bit operands (P and dS are
// rounded to the input type for the product) and float32 accumulation.
#pragma once

#include "common.hpp"
#include "fwd_kernel.hpp"

namespace rf {

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;      // forward output
    const void* dout;   // gradient of the loss with respect to o
    const float* lse;   // forward log-sum-exp, natural log
    float* drow;        // workspace [B, Hq, Nq]: D_i = dO_i . O_i
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv, Nq, Nk, D;
    float scale;
    int mask;
    int window;
    float rope_base;
    const float* alibi;
    RopeTable rope;
};

constexpr int BWD_THREADS = 256;

// Waves per SIMD the D = 64 dq and dk/dv kernels are compiled for, and the
// query tile of the dk/dv kernel at D = 64: RF_BWD_DQ_WAVES, RF_BWD_KV_WAVES
// and RF_BWD_BQ64 in tuned.hpp.

// ---------------------------------------------------------------- D_i
template <typename T, int D>
__global__ __launch_bounds__(BWD_THREADS) void bwd_rowterm_kernel(const T* o, const T* dout, float* drow, long long rows) {
    typedef typename Vec16<T>::type VecT;
    constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
    const long long idx = (long long)blockIdx.x * BWD_THREADS + threadIdx.x;
    const long long row = idx / LPR;
    const int c = (int)(idx % LPR);
    float acc = 0.f;
    if (row < rows) {
        const VecT a = *(const VecT*)(o + row * D + 8 * c);
        const VecT b = *(const VecT*)(dout + row * D + 8 * c);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(to_f32(a[i]), to_f32(b[i]), acc);
    }
#pragma unroll
    for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, 64);
    if (row < rows && c == 0) drow[row] = acc;
}

// log2-domain lse; a row with no visible key (lse = -inf) gets +inf so that
// every 2^(s - lse2) of it is 0.
__device__ __forceinline__ float lse_log2(float lse) {
    return lse == -INFINITY ? INFINITY : lse * 1.4426950408889634f;
}

// Rotation by -angle of a gradient pair (the transpose of the RoPE rotation).
__device__ __forceinline__ void rope_unrotate(double inv_period, int pos, float& x, float& y) {
    float cs, sn;
    rope_cos_sin(inv_period, pos, cs, sn);
    const float a = x, b = y;
    x = a * cs + b * sn;
    y = b * cs - a * sn;
}

// ---------------------------------------------------------------- dq
// Query-parallel, the forward's layout: S^T = K . Q^T (lane = query row), so
// P^T, dP^T and dS^T sit in the lane's registers and feed dQ^T += K^T . dS^T
// as the B operand, with K^T read from the K tile by the LDS transpose read.
template <typename T, int D, bool ROPE, bool ALIBI>
__global__ __launch_bounds__(FWD_THREADS, D == 64 ? RF_BWD_DQ_WAVES : 1) void attn_bwd_dq_kernel(BwdParams p) {
    using C = FwdCfg<T, D, false>;
    constexpr int BN = C::BN;
    constexpr int EPC = C::EPC;
    constexpr int CPR = C::CPR;
    constexpr int KS = C::KSTRIDE;
    constexpr int NKB = BN / 32;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;
    constexpr float LOG2E = 1.4426950408889634f;
    typedef typename Vec16<T>::type VecT;
    static_assert(sizeof(T) == 2, "16-bit inputs");

    __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // work order: the causal mask makes late query blocks heaviest, start with them
    const int nqb = (p.Nq + FWD_BM - 1) / FWD_BM;
    const int heads = p.B * p.Hq;
    const int pid = blockIdx.x;
    const int qb = p.mask == RF_MASK_CAUSAL ? nqb - 1 - pid / heads : pid / heads;
    const int bh = pid % heads;
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int q0 = qb * FWD_BM;
    const int g = h / (p.Hq / p.Hkv);
    const int pos_off = p.Nk - p.Nq;

    const int last_row = min(p.Nq, q0 + FWD_BM) - 1;
    int klo = 0, khi = p.Nk;
    if (p.mask != RF_MASK_NONE) khi = min(khi, last_row + pos_off + 1);
    if (p.mask == RF_MASK_SLIDING) klo = max(klo, q0 + pos_off - p.window + 1);
    const int ntiles = khi > klo ? (khi - klo + BN - 1) / BN : 0;

    const int wrow0 = q0 + 32 * wave;
    const bool wave_live = wrow0 < p.Nq;
    const int pw_min = wrow0 + pos_off;
    const int pw_max = min(p.Nq, wrow0 + 32) - 1 + pos_off;
    const int my_row = wrow0 + l32;
    const int my_pos = my_row + pos_off;
    const int lim_hi = p.mask != RF_MASK_NONE ? min(khi - 1, my_pos) : khi - 1;
    const int lim_lo = p.mask == RF_MASK_SLIDING ? my_pos - p.window + 1 : -(1 << 30);

    const float c = fmaxf(p.scale * LOG2E, 1e-30f);
    const float slope2 = ALIBI ? p.alibi[h] * LOG2E : 0.f;
    const size_t kv_base = ((size_t)b * p.Hkv + g) * (size_t)p.Nk * D;
    const int kv_bytes = p.Nk * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc((const T*)p.k + kv_base, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const T*)p.v + kv_base, kv_bytes);

    // Q^T and dO^T operands (lane = query, element n of step ks is d = 16 ks + 8 hi + n)
    const bool row_ok = my_row < p.Nq;
    const size_t row_id = ((size_t)b * p.Hq + h) * p.Nq + (size_t)min(my_row, max(p.Nq - 1, 0));
    VecT qv[NKS], dov[NKS];
    {
        constexpr int QN = D / 2;
        float qf[QN];
        const T* qrow = (const T*)p.q + row_id * D;
        const T* drw = (const T*)p.dout + row_id * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const VecT x = *(const VecT*)(qrow + 16 * ks + 8 * hi);
            const VecT y = *(const VecT*)(drw + 16 * ks + 8 * hi);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qf[8 * ks + i] = row_ok ? to_f32(x[i]) : 0.f;
                dov[ks][i] = row_ok ? y[i] : from_f32<T>(0.f);
            }
        }
        if (ROPE) {
#pragma unroll
            for (int n = 0; n < QN / 2; ++n) {
                const int d = 16 * (n / 8) + 8 * hi + (n % 8);
                float cs, sn;
                rope_cos_sin(p.rope.inv_period[d], my_pos, cs, sn);
                const float x = qf[n], y = qf[n + QN / 2];
                qf[n] = x * cs - y * sn;
                qf[n + QN / 2] = x * sn + y * cs;
            }
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) qv[ks][i] = from_f32<T>(qf[8 * ks + i]);
    }
    const float lse2 = row_ok ? lse_log2(p.lse[row_id]) : INFINITY;
    const float dr = row_ok ? p.drow[row_id] : 0.f;

    double ipd[ROPE ? EPC : 1];
    if (ROPE) {
        const int cc = tid % (CPR / 2);
#pragma unroll
        for (int e = 0; e < EPC; ++e) ipd[e] = p.rope.inv_period[cc * EPC + e];
    }

    uint4 kreg[C::CH], vreg[C::CH];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int it = 0; it < C::CH; ++it) {
            int row, ch;
            if (ROPE) {
                const int u = (it / 2) * FWD_THREADS + tid;
                row = u / (CPR / 2);
                ch = u % (CPR / 2) + (it % 2) * (CPR / 2);
            } else {
                const int u = it * FWD_THREADS + tid;
                row = u / CPR;
                ch = u % CPR;
            }
            kreg[it] = buf_load16(krs, ((unsigned)(k0 + row) * D + ch * EPC) * (unsigned)sizeof(T));
        }
#pragma unroll
        for (int it = 0; it < C::CH; ++it) {
            const int u = it * FWD_THREADS + tid;
            vreg[it] = buf_load16(vrs, ((unsigned)(k0 + u / CPR) * D + (u % CPR) * EPC) * (unsigned)sizeof(T));
        }
    };
    auto store_tile = [&](int stage, int k0) {
        T* ks_ = smem + stage * C::STAGE;
        T* vs_ = ks_ + C::K_ELEMS;
        if (ROPE) {
#pragma unroll
            for (int it = 0; it < C::CH; it += 2) {
                const int u = (it / 2) * FWD_THREADS + tid;
                const int row = u / (CPR / 2);
                const int cc = u % (CPR / 2);
                const VecT lo = *(const VecT*)&kreg[it];
                const VecT hi_ = *(const VecT*)&kreg[it + 1];
                VecT olo, ohi;
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    float cs, sn;
                    rope_cos_sin(ipd[e], k0 + row, cs, sn);
                    const float x = to_f32(lo[e]), y = to_f32(hi_[e]);
                    olo[e] = from_f32<T>(x * cs - y * sn);
                    ohi[e] = from_f32<T>(x * sn + y * cs);
                }
                *(VecT*)(ks_ + row * KS + cc * EPC) = olo;
                *(VecT*)(ks_ + row * KS + (cc + CPR / 2) * EPC) = ohi;
            }
        } else {
#pragma unroll
            for (int it = 0; it < C::CH; ++it) {
                const int u = it * FWD_THREADS + tid;
                *(uint4*)(ks_ + (u / CPR) * KS + (u % CPR) * EPC) = kreg[it];
            }
        }
#pragma unroll
        for (int it = 0; it < C::CH; ++it) {
            const int u = it * FWD_THREADS + tid;
            *(uint4*)(vs_ + (u / CPR) * KS + (u % CPR) * EPC) = vreg[it];
        }
    };

    // LDS transpose read of a row-major [keys][D] tile: contraction slot (hi, i)
    // holds key 16 t16 + 8 (i/4) + 4 hi + i%4 (score register 8 (t16%2) + i).
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    f32x16 dqacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

    if (ntiles > 0) {
        load_tile(klo);
        store_tile(0, klo);
    }
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = klo + t * BN;
        const int stage = t & 1;
        __syncthreads();
        if (t + 1 < ntiles) load_tile(k0 + BN);

        bool skip = !wave_live;
        bool need_mask = (k0 + BN > khi);
        if (p.mask != RF_MASK_NONE) {
            skip |= k0 > pw_max;
            need_mask |= (k0 + BN - 1 > pw_min);
            if (p.mask == RF_MASK_SLIDING) {
                skip |= (k0 + BN - 1 <= pw_min - p.window);
                need_mask |= (k0 <= pw_max - p.window);
            }
        }
        if (!skip) {
            const T* ks_ = smem + stage * C::STAGE;
            const T* vs_ = ks_ + C::K_ELEMS;
            f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sacc[kb] = f32x16{};
                dpacc[kb] = f32x16{};
                const T* krow = ks_ + (32 * kb + l32) * KS + 8 * hi;
                const T* vrow = vs_ + (32 * kb + l32) * KS + 8 * hi;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    sacc[kb] = mfma32(*(const VecT*)(krow + 16 * ks), qv[ks], sacc[kb]);
                    dpacc[kb] = mfma32(*(const VecT*)(vrow + 16 * ks), dov[ks], dpacc[kb]);
                }
            }
            if (need_mask) {
                // visible iff rel_lo <= offset <= rel_hi; & keeps it branch-free
                const int rel_hi = lim_hi - k0 - 4 * hi;
                const int rel_lo = lim_lo - k0 - 4 * hi;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int off = 32 * kb + 8 * (j / 4) + (j % 4);
                        sacc[kb][j] = ((off <= rel_hi) & (off >= rel_lo)) ? sacc[kb][j] : -INFINITY;
                    }
            }
            if constexpr (ALIBI) {
                const float kd = (float)(k0 + 4 * hi - my_pos);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float dist = fabsf(kd + (float)(32 * kb + 8 * (j / 4) + (j % 4)));
                        sacc[kb][j] = fmaf(sacc[kb][j], c, -slope2 * dist);
                    }
            }
#pragma unroll
            for (int t16 = 0; t16 < BN / 16; ++t16) {
                VecT dsb;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int kb = t16 / 2, j = 8 * (t16 % 2) + i;
                    const float pr = fast_exp2(ALIBI ? sacc[kb][j] - lse2 : fmaf(sacc[kb][j], c, -lse2));
                    dsb[i] = from_f32<T>(pr * (dpacc[kb][j] - dr));
                }
                const T* krow = ks_ + (16 * t16 + tr_row) * KS + tr_col;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i16x4 lo4 = lds_read_tr16(krow + 32 * db);
                    const i16x4 hi4 = lds_read_tr16(krow + 8 * KS + 32 * db);
                    const i16x8 ab = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                    dqacc[db] = mfma32(__builtin_bit_cast(VecT, ab), dsb, dqacc[db]);
                }
            }
        }
        if (t + 1 < ntiles) store_tile(stage ^ 1, k0 + BN);
    }

    if (!wave_live || !row_ok) return;
    // dq' = scale * acc; register j of block db holds d = 32 db + 8 (j/4) + 4 hi + j%4
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqacc[db] *= p.scale;
    if (ROPE) {
#pragma unroll
        for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int d = 32 * db + 8 * (j / 4) + 4 * hi + (j % 4);
                float x = dqacc[db][j], y = dqacc[db + NDB / 2][j];
                rope_unrotate(p.rope.inv_period[d], my_pos, x, y);
                dqacc[db][j] = x;
                dqacc[db + NDB / 2][j] = y;
            }
    }
    T* orow = (T*)p.dq + row_id * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
            T4 w;
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(dqacc[db][4 * jq + r]);
            *(T4*)(orow + 32 * db + 8 * jq + 4 * hi) = w;
        }
}

// ---------------------------------------------------------------- dk, dv
// Key-parallel: 128 keys of one KV head per work-group, 32 per wave (lane =
// key), over every query tile of every query head of the GQA group.  S and
// dP are computed as [queries x keys] (M = queries), so the lane holds its
// key's column and the registers hold queries: that is the B operand of
// dV^T += dO^T . P and dK^T += Q^T . dS, whose A operands are the transposed
// reads of the row-major Q and dO tiles.
constexpr int BWD_BK = 128;  // keys per work-group

template <typename T, int D>
struct BwdKvCfg {
    static constexpr int BQ = D == 64 ? RF_BWD_BQ64 : 32;  // queries per tile
    static constexpr int NQB = BQ / 32;
    static constexpr int EPC = 8;
    static constexpr int CPR = D / EPC;
    static constexpr int KS = D + EPC;                 // padded row pitch
    static constexpr int TILE = BQ * KS;               // elements of one Q or dO tile
    static constexpr int STAGE = 2 * TILE + 2 * BQ * 2;  // Q, dO, lse2 and drow (floats as 2 T each)
    static constexpr int CH = BQ * CPR / BWD_THREADS;  // 16-byte chunks per thread per tile
    static_assert(CH >= 1, "tile too small");
};

template <typename T, int D, bool ROPE, bool ALIBI>
__global__ __launch_bounds__(BWD_THREADS, D == 64 ? RF_BWD_KV_WAVES : 1) void attn_bwd_dkdv_kernel(BwdParams p) {
    using C = BwdKvCfg<T, D>;
    constexpr int BQ = C::BQ;
    constexpr int NQB = C::NQB;
    constexpr int EPC = C::EPC;
    constexpr int CPR = C::CPR;
    constexpr int KS = C::KS;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;
    constexpr float LOG2E = 1.4426950408889634f;
    typedef typename Vec16<T>::type VecT;
    static_assert(sizeof(T) == 2, "16-bit inputs");

    __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // work order: key block 0 sees the most queries under the causal mask
    const int heads = p.B * p.Hkv;
    const int pid = blockIdx.x;
    const int kblk = pid / heads;
    const int bg = pid % heads;
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int kb0 = kblk * BWD_BK;
    const int kb1 = min(p.Nk, kb0 + BWD_BK);
    const int pos_off = p.Nk - p.Nq;

    // queries any key of the block sees: [qlo, qhi)
    int qlo = 0, qhi = p.Nq;
    if (p.mask != RF_MASK_NONE) qlo = max(0, kb0 - pos_off);
    if (p.mask == RF_MASK_SLIDING) qhi = min(p.Nq, max(0, kb1 - 1 + p.window - pos_off));
    const int qt0 = (qlo / BQ) * BQ;
    const int ntq = qhi > qlo ? (qhi - qt0 + BQ - 1) / BQ : 0;
    const int nit = ntq * G;

    // this wave's keys
    const int kw0 = kb0 + 32 * wave;
    const int kw_last = min(kb1, kw0 + 32) - 1;
    const bool wave_live = kw0 < kb1;
    const int my_key = kw0 + l32;
    const bool key_ok = my_key < p.Nk;

    const float c = fmaxf(p.scale * LOG2E, 1e-30f);
    const size_t kv_row = ((size_t)b * p.Hkv + g) * (size_t)p.Nk + (size_t)min(my_key, max(p.Nk - 1, 0));

    // K^T and V^T operands (lane = key, element n of step ks is d = 16 ks + 8 hi + n)
    VecT kv_[NKS], vv[NKS];
    {
        constexpr int KN = D / 2;
        float kf[KN];
        const T* krow = (const T*)p.k + kv_row * D;
        const T* vrow = (const T*)p.v + kv_row * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const VecT x = *(const VecT*)(krow + 16 * ks + 8 * hi);
            const VecT y = *(const VecT*)(vrow + 16 * ks + 8 * hi);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kf[8 * ks + i] = key_ok ? to_f32(x[i]) : 0.f;
                vv[ks][i] = key_ok ? y[i] : from_f32<T>(0.f);
            }
        }
        if (ROPE) {
#pragma unroll
            for (int n = 0; n < KN / 2; ++n) {
                const int d = 16 * (n / 8) + 8 * hi + (n % 8);
                float cs, sn;
                rope_cos_sin(p.rope.inv_period[d], my_key, cs, sn);
                const float x = kf[n], y = kf[n + KN / 2];
                kf[n] = x * cs - y * sn;
                kf[n + KN / 2] = x * sn + y * cs;
            }
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) kv_[ks][i] = from_f32<T>(kf[8 * ks + i]);
    }

    double ipd[ROPE ? EPC : 1];
    if (ROPE) {
        const int cc = tid % (CPR / 2);
#pragma unroll
        for (int e = 0; e < EPC; ++e) ipd[e] = p.rope.inv_period[cc * EPC + e];
    }

    // staging of one (head, query tile): Q rotated at the query positions, dO,
    // lse in log2 units and the row terms; rows past Nq read as zeros.
    uint4 qreg[C::CH], dreg[C::CH];
    float sreg = 0.f;
    auto tile_of = [&](int it, int& hh, int& q0) {
        hh = g * G + it / ntq;
        q0 = qt0 + (it % ntq) * BQ;
    };
    auto load_tile = [&](int it) {
        int hh, q0;
        tile_of(it, hh, q0);
        const size_t base = ((size_t)b * p.Hq + hh) * (size_t)p.Nq;
        const int bytes = p.Nq * D * (int)sizeof(T);
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const T*)p.q + base * D, bytes);
        const __amdgpu_buffer_rsrc_t drs = make_rsrc((const T*)p.dout + base * D, bytes);
#pragma unroll
        for (int i = 0; i < C::CH; ++i) {
            int row, ch;
            if (ROPE) {
                const int u = (i / 2) * BWD_THREADS + tid;
                row = u / (CPR / 2);
                ch = u % (CPR / 2) + (i % 2) * (CPR / 2);
            } else {
                const int u = i * BWD_THREADS + tid;
                row = u / CPR;
                ch = u % CPR;
            }
            qreg[i] = buf_load16(qrs, ((unsigned)(q0 + row) * D + ch * EPC) * (unsigned)sizeof(T));
        }
#pragma unroll
        for (int i = 0; i < C::CH; ++i) {
            const int u = i * BWD_THREADS + tid;
            dreg[i] = buf_load16(drs, ((unsigned)(q0 + u / CPR) * D + (u % CPR) * EPC) * (unsigned)sizeof(T));
        }
        // lse ([0, BQ)) and row terms ([BQ, 2 BQ)) as loaded; the lse's log2
        // form and the values of rows past Nq are set at the LDS store, so no
        // instruction here waits on these loads (or, through the in-order
        // load counter, on the tile loads above)
        if (tid < 2 * BQ) {
            const float* src = tid < BQ ? p.lse : p.drow;
            sreg = src[base + min(q0 + tid % BQ, p.Nq - 1)];
        }
    };
    auto store_tile = [&](int stage, int it) {
        int hh, q0;
        tile_of(it, hh, q0);
        T* qs_ = smem + stage * C::STAGE;
        T* ds_ = qs_ + C::TILE;
        float* fs_ = (float*)(ds_ + C::TILE);
        if (ROPE) {
#pragma unroll
            for (int i = 0; i < C::CH; i += 2) {
                const int u = (i / 2) * BWD_THREADS + tid;
                const int row = u / (CPR / 2);
                const int cc = u % (CPR / 2);
                const VecT lo = *(const VecT*)&qreg[i];
                const VecT hi_ = *(const VecT*)&qreg[i + 1];
                VecT olo, ohi;
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    float cs, sn;
                    rope_cos_sin(ipd[e], q0 + row + pos_off, cs, sn);
                    const float x = to_f32(lo[e]), y = to_f32(hi_[e]);
                    olo[e] = from_f32<T>(x * cs - y * sn);
                    ohi[e] = from_f32<T>(x * sn + y * cs);
                }
                *(VecT*)(qs_ + row * KS + cc * EPC) = olo;
                *(VecT*)(qs_ + row * KS + (cc + CPR / 2) * EPC) = ohi;
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::CH; ++i) {
                const int u = i * BWD_THREADS + tid;
                *(uint4*)(qs_ + (u / CPR) * KS + (u % CPR) * EPC) = qreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::CH; ++i) {
            const int u = i * BWD_THREADS + tid;
            *(uint4*)(ds_ + (u / CPR) * KS + (u % CPR) * EPC) = dreg[i];
        }
        if (tid < 2 * BQ) {  // [0, BQ): lse in log2 units, [BQ, 2 BQ): drow
            const bool in = q0 + tid % BQ < p.Nq;
            fs_[tid] = tid < BQ ? (in ? lse_log2(sreg) : INFINITY) : (in ? sreg : 0.f);
        }
    };

    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    f32x16 dvacc[NDB], dkacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dvacc[db] = f32x16{};
        dkacc[db] = f32x16{};
    }

    if (nit > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    for (int it = 0; it < nit; ++it) {
        const int stage = it & 1;
        int hh, q0;
        tile_of(it, hh, q0);
        __syncthreads();
        if (it + 1 < nit) load_tile(it + 1);

        // positions of the tile's queries: q0 + pos_off .. q0 + BQ - 1 + pos_off
        const int pt_min = q0 + pos_off;
        const int pt_max = min(p.Nq, q0 + BQ) - 1 + pos_off;
        bool skip = !wave_live;
        bool need_mask = q0 + BQ > p.Nq || kw0 + 32 > p.Nk;
        if (p.mask != RF_MASK_NONE) {
            skip |= pt_max < kw0;                          // every query before the wave's keys
            need_mask |= pt_min < kw_last;
            if (p.mask == RF_MASK_SLIDING) {
                skip |= pt_min - p.window >= kw_last;     // every key left the window
                need_mask |= pt_max - p.window >= kw0;
            }
        }
        if (!skip) {
            const T* qs_ = smem + stage * C::STAGE;
            const T* ds_ = qs_ + C::TILE;
            const float* fs_ = (const float*)(ds_ + C::TILE);
            // S = Q K^T and dP = dO V^T, [queries x keys]: register j of block
            // qb is query 32 qb + 8 (j/4) + 4 hi + j%4 of the tile
            f32x16 sacc[NQB], dpacc[NQB];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                sacc[qb] = f32x16{};
                dpacc[qb] = f32x16{};
                const T* qrow = qs_ + (32 * qb + l32) * KS + 8 * hi;
                const T* drw = ds_ + (32 * qb + l32) * KS + 8 * hi;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    sacc[qb] = mfma32(*(const VecT*)(qrow + 16 * ks), kv_[ks], sacc[qb]);
                    dpacc[qb] = mfma32(*(const VecT*)(drw + 16 * ks), vv[ks], dpacc[qb]);
                }
            }
            // query offset in the tile minus what a visible query must reach
            const int rel = my_key - pos_off - q0 - 4 * hi;  // causal: visible iff off >= rel
            const int rows_left = p.Nq - q0 - 4 * hi;        // valid iff off < rows_left
            if (need_mask) {
                // visible iff lo_b <= offset <= hi_b (bounds per lane; & keeps
                // every element branch-free)
                const int lo_b = p.mask != RF_MASK_NONE ? rel : -(1 << 30);
                int hi_b = rows_left - 1;
                if (p.mask == RF_MASK_SLIDING) hi_b = min(hi_b, rel + p.window - 1);
                if (!key_ok) hi_b = -1;
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int off = 32 * qb + 8 * (j / 4) + (j % 4);
                        sacc[qb][j] = ((off >= lo_b) & (off <= hi_b)) ? sacc[qb][j] : -INFINITY;
                    }
            }
            if constexpr (ALIBI) {
                const float slope2 = p.alibi[hh] * LOG2E;
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float dist = fabsf((float)(32 * qb + 8 * (j / 4) + (j % 4) - rel));
                        sacc[qb][j] = fmaf(sacc[qb][j], c, -slope2 * dist);
                    }
            }
#pragma unroll
            for (int t16 = 0; t16 < BQ / 16; ++t16) {
                const int qb = t16 / 2, jb = 8 * (t16 % 2);
                // lse2 and drow of the 8 queries of this group: 32 qb + 8 (i/4) + 4 hi + i%4 + 16 (t16%2)
                const float4 la = *(const float4*)(fs_ + 32 * qb + 16 * (t16 % 2) + 4 * hi);
                const float4 lb = *(const float4*)(fs_ + 32 * qb + 16 * (t16 % 2) + 8 + 4 * hi);
                const float4 da = *(const float4*)(fs_ + BQ + 32 * qb + 16 * (t16 % 2) + 4 * hi);
                const float4 dbv = *(const float4*)(fs_ + BQ + 32 * qb + 16 * (t16 % 2) + 8 + 4 * hi);
                const float l8[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
                const float d8[8] = {da.x, da.y, da.z, da.w, dbv.x, dbv.y, dbv.z, dbv.w};
                VecT pb, dsb;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float s = sacc[qb][jb + i];
                    const float pr = fast_exp2(ALIBI ? s - l8[i] : fmaf(s, c, -l8[i]));
                    pb[i] = from_f32<T>(pr);
                    dsb[i] = from_f32<T>(pr * (dpacc[qb][jb + i] - d8[i]));
                }
                const T* drow_tr = ds_ + (16 * t16 + tr_row) * KS + tr_col;
                const T* qrow_tr = qs_ + (16 * t16 + tr_row) * KS + tr_col;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i16x4 a0 = lds_read_tr16(drow_tr + 32 * db);
                    const i16x4 a1 = lds_read_tr16(drow_tr + 8 * KS + 32 * db);
                    const i16x8 ad = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                    dvacc[db] = mfma32(__builtin_bit_cast(VecT, ad), pb, dvacc[db]);
                    const i16x4 b0 = lds_read_tr16(qrow_tr + 32 * db);
                    const i16x4 b1 = lds_read_tr16(qrow_tr + 8 * KS + 32 * db);
                    const i16x8 aq = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
                    dkacc[db] = mfma32(__builtin_bit_cast(VecT, aq), dsb, dkacc[db]);
                }
            }
        }
        if (it + 1 < nit) store_tile(stage ^ 1, it + 1);
    }

    if (!wave_live || !key_ok) return;
#pragma unroll
    for (int db = 0; db < NDB; ++db) dkacc[db] *= p.scale;
    if (ROPE) {
#pragma unroll
        for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int d = 32 * db + 8 * (j / 4) + 4 * hi + (j % 4);
                float x = dkacc[db][j], y = dkacc[db + NDB / 2][j];
                rope_unrotate(p.rope.inv_period[d], my_key, x, y);
                dkacc[db][j] = x;
                dkacc[db + NDB / 2][j] = y;
            }
    }
    T* krow = (T*)p.dk + kv_row * D;
    T* vrow = (T*)p.dv + kv_row * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
            T4 wk, wv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wk[r] = from_f32<T>(dkacc[db][4 * jq + r]);
                wv[r] = from_f32<T>(dvacc[db][4 * jq + r]);
            }
            *(T4*)(krow + 32 * db + 8 * jq + 4 * hi) = wk;
            *(T4*)(vrow + 32 * db + 8 * jq + 4 * hi) = wv;
        }
}

}  // namespace rf
