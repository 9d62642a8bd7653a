// Fused single-pass attention forward for gfx950 (MFMA).
//
// The cascade max -> exp-sum -> P.V ("RedFuser", abstract and Fig. 3) runs in
// its incremental form (RedFuser Fig. 4b): each key tile updates a running
// (m, l, O) per query row, so on-chip state is constant in the key length.
// The scores use the max/+ pair and the output the +/* pair of RedFuser
// Table 1; rescaling by 2^(m_old - m_new) is what lets max distribute over +.
// Variants: pre-matmul RoPE on Q and K (AttnFuse abstract, Fig. 1), causal and
// sliding-window visibility (AttnFuse Table 6), GQA head sharing and split-KV
// partials (RedFuser Fig. 13, AttnFuse Table 8).
//
// Work-group: 4 wavefronts, 128 query rows (32 per wave), one (batch, head,
// key chunk).  Per key tile of BN keys:
//   S^T = K . Q^T on MFMA 32x32 (A = K tile from LDS, B = Q^T held in
//   registers), so lane l owns query row (l % 32) and 16 keys per 32-key
//   block: the row max and row sum are in-lane plus one swap between the two
//   32-lane halves.
//   O^T += V^T . P^T on MFMA 32x32 (A = V^T, B = P^T straight from the score
//   registers), so the rescale of O by alpha is a per-lane scalar.  V stays
//   row-major in LDS; the transposed operand comes from the gfx950 LDS
//   transpose read (ds_read_b64_tr_b16), 4 keys of one d column per lane.
// K/V tiles are double-buffered: the global loads of tile t+1 are issued
// before the math of tile t and written to LDS after it (one barrier a tile).
// 16-bit D = 128 without RoPE or ALiBi instead loads straight into LDS, with
// two K buffers and one V buffer (two barriers a tile).
//
// The O rescale is lazy: the reference max m_ref only moves when a tile's max
// exceeds it by more than 2^8, so P = 2^(s - m_ref) <= 256 (exact range in
// fp16 and bf16) and l, O stay consistent with m_ref; the final O / l is the
// same quantity.
#pragma once

#include "common.hpp"
#include "tuned.hpp"

namespace rf {

// SPLITK: K (and Q) are kept as a bf16 hi/lo pair, x = hi + lo, so rotated
// operands keep ~16 mantissa bits; S then takes three MFMAs (hi.hi, hi.lo,
// lo.hi).  Used for bf16 with RoPE, where rounding the rotated q and k to a
// single bf16 dominates the output error.
// Work-group layouts (template parameter KH):
//  0: 4 waves, 128 query rows, one key stream;
//  1: key halves, 4 waves, 64 rows: two groups of 2 waves, 32-key tiles;
//  2: key halves, 8 waves, 128 rows: two groups of 4 waves, 64-key tiles.
template <int KH>
struct FwdLayout {
    static constexpr int WAVES = KH == 2 ? 8 : FWD_WAVES;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int GROUPS = KH ? 2 : 1;       // key streams
    static constexpr int GWAVES = WAVES / GROUPS;   // waves (32-row slots) per stream
    static constexpr int BM = 32 * GWAVES;          // query rows per work-group
};

template <typename T, int D, bool SPLITK = false, int KH = 0>
struct FwdCfg {
    static constexpr bool F32 = sizeof(T) == 4;
    static constexpr int BN = (F32 || KH == 1) ? 32 : 64;  // keys per tile
    static constexpr int GT = 64 * FwdLayout<KH>::GWAVES;  // threads staging one tile stream
    static constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;                 // chunks per row
    static constexpr int KSTRIDE = D + EPC;             // row pitch (elements), +16 B
    static constexpr int K_ELEMS = BN * KSTRIDE * (SPLITK ? 2 : 1);  // hi tile, then lo tile
    static constexpr int STAGE = K_ELEMS + BN * KSTRIDE;  // + V tile, row-major
    static constexpr int CH = BN * CPR / GT;            // 16-byte chunks per thread per tile
    static_assert(CH >= 2 && CH % 2 == 0, "tile must give each thread an even chunk count");
};

// Waves per SIMD the non-RoPE D=64 instance is compiled for (register budget
// 512 / waves): RF_FWD_WAVES_D64 in tuned.hpp.  The other instances need more
// registers and get 2.

// Work-group order (one-dimensional grid of B*Hq*S*nqb query blocks of
// FWD_BM rows); returns the query block qb and bx = (b * Hq + h) * S + split.
//  causal: every head's heaviest (latest) query blocks first, then lighter
//    ones, so the uneven blocks balance across the CUs.  The groups that
//    start at launch are placed statically: group pid goes to the CU
//    numbered pid mod P (P CUs), so a CU receives items pid, pid + P,
//    pid + 2P, ...  When the whole grid is resident at launch, every other
//    run of P items is taken in reverse (snake order), which gives each CU
//    a heavy item from one run and a light one from the next instead of
//    items of the same rank.  A larger grid keeps the plain order: its
//    later groups start wherever a slot frees, which balances by itself;
//  no mask / sliding window (every block costs the same): the dispatcher
//    deals work-groups round-robin over the XCDs (each with its own L2), so
//    renumber to give every XCD a contiguous run of one head's query blocks
//    and keep the K/V tiles that neighbouring blocks share in its L2.
__device__ __forceinline__ void fwd_work_item(const AttnParams& p, int nqb, int& qb, int& bx) {
    const int G = gridDim.x;
    const int pid = blockIdx.x;
    if (p.mask == RF_MASK_CAUSAL) {
        const int heads = G / nqb;
        const int P = p.cu_count;
        int item = pid;  // index in heaviest-first order
        if (P > 0 && (long long)P * p.launch_runs >= G) {
            const int run = pid / P;
            if ((run & 1) && run < G / P) item = run * P + (P - 1 - pid % P);
        }
        qb = nqb - 1 - item / heads;
        bx = item % heads;
    } else {
        const int xcd = pid % NUM_XCD, local = pid / NUM_XCD;
        const int per = G / NUM_XCD, rem = G % NUM_XCD;
        const int L = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
        qb = L % nqb;
        bx = L / nqb;
    }
}

// KH (key halves, 16-bit D = 64): the work-group's key range is cut in two:
// the first group of waves takes the first half, the second group the second,
// each with its own tile stream and LDS double buffer; at the end group 1
// hands (O, m, l) to group 0 through LDS and group 0 merges them (the LSE
// merge of two partial states, RedFuser Fig. 13).  The longest chain of tile
// steps a work-group runs is halved, which shortens a launch whose grid fits
// the GPU in about one wave of work-groups.  KH = 1 keeps 4
// waves (64 rows, 32-key tiles); KH = 2 has 8 waves (128 rows, 64-key tiles,
// each group staging its tiles exactly as the 4-wave 128-row kernel does).
template <typename T, int D, bool ROPE, bool ALIBI, int KH = 0>
__global__ __launch_bounds__(FwdLayout<KH>::THREADS, (D == 64 && !ROPE && !ALIBI) ? RF_FWD_WAVES_D64 : 2)
void attn_fwd_kernel(AttnParams p) {
    constexpr bool SPLITK = ROPE && sizeof(T) == 2 && !__is_same(T, _Float16);
    using L = FwdLayout<KH>;
    using C = FwdCfg<T, D, SPLITK, KH>;
    constexpr int GT = C::GT;
    constexpr int BM = L::BM;  // query rows per work-group
    constexpr bool F32 = C::F32;
    constexpr int BN = C::BN;
    constexpr int EPC = C::EPC;
    constexpr int CPR = C::CPR;
    constexpr int KS = C::KSTRIDE;
    constexpr int NKB = BN / 32;      // 32-key blocks per tile
    constexpr int NDB = D / 32;       // 32-wide d blocks of the output
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.6931471805599453f;
    constexpr float RESCALE_SLACK = 8.0f;  // log2 units
    typedef typename Vec16<T>::type VecT;
    // V1 (16-bit, D = 128, no RoPE or ALiBi): two K buffers and one V buffer
    // (52 KB instead of 70), both filled by buffer loads that write LDS
    // directly, so no registers stage the tiles.  Tile t's V and tile t+1's K
    // are issued together once every wave has finished tile t-1's P.V; V(t)
    // lands under tile t's score products and softmax, and a second barrier
    // precedes the P.V.
    constexpr bool V1 = D == 128 && !F32 && !ROPE && !ALIBI;
    static_assert(!KH || (D == 64 && !F32), "key halves: 16-bit D = 64");

    __shared__ __attribute__((aligned(16))) T smem[V1 ? 2 * C::K_ELEMS + BN * KS : (KH ? 4 : 2) * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    // KH: group (key half) of this wave, its row slot, and the thread's index in the group
    const int grp = KH ? wave / L::GWAVES : 0;
    const int rw = KH ? wave % L::GWAVES : wave;
    const int gtid = KH ? tid % GT : tid;
    T* const gsm = KH ? smem + grp * 2 * C::STAGE : smem;  // this group's two stages

    const int nqb = (p.Nq + BM - 1) / BM;
    int qb, bx;  // bx = (b * Hq + h) * S + split
    fwd_work_item(p, nqb, qb, bx);
    const int split = bx % p.num_splits;
    bx /= p.num_splits;
    const int h = bx % p.Hq;
    const int b = bx / p.Hq;
    const int q0 = qb * BM;
    const int g = h / (p.Hq / p.Hkv);
    const int pos_off = p.Nk - p.Nq;

    // Key range the whole work-group visits.
    const int last_row = min(p.Nq, q0 + BM) - 1;
    int klo = split * p.split_len;
    int khi = min(p.Nk, klo + p.split_len);
    if (p.mask != RF_MASK_NONE) khi = min(khi, last_row + pos_off + 1);
    if (p.mask == RF_MASK_SLIDING) klo = max(klo, q0 + pos_off - p.window + 1);
    // Sliding window (one split, direct-to-LDS staging): tiles sit on the
    // global grid of BN keys and a work-group visits them in the cyclic order
    // that puts tile j at step j mod ntiles.  Interior query blocks all have
    // the same tile count, so neighbouring blocks, running side by side on one
    // XCD, read the tiles they share at the same step and the second read hits
    // L2.  Keys below klo are outside every row's window and are masked like
    // any other.  (Other instances keep the plain ascending order and its code.)
    const bool cyc = V1 && p.mask == RF_MASK_SLIDING && !p.split_mode && khi > klo;
    if (cyc) klo -= klo % BN;
    const int ntiles_wg = khi > klo ? (khi - klo + BN - 1) / BN : 0;
    // KH: group 0 takes tiles [0, n0), group 1 tiles [n0, ntiles_wg); both
    // run n0 steps (group 1 idles in a last step it has no tile for).
    const int n0 = KH ? (ntiles_wg + 1) / 2 : ntiles_wg;
    const int ntiles = KH ? (grp ? ntiles_wg - n0 : n0) : ntiles_wg;  // this group's tiles
    const int nsteps = n0;
    const int kbeg = klo + (KH && grp ? n0 * BN : 0);                 // this group's first key
    // tile index at step 0, then +1 per step with wrap-around
    int tcur = cyc ? (ntiles - (klo / BN) % ntiles) % ntiles : 0;

    // This wave's rows and their positions.
    const int wrow0 = q0 + 32 * rw;
    const bool wave_live = wrow0 < p.Nq;
    const int pw_min = wrow0 + pos_off;
    const int pw_max = min(p.Nq, wrow0 + 32) - 1 + pos_off;
    const int my_row = wrow0 + l32;
    const int my_pos = my_row + pos_off;
    // visible keys of this lane's row: lim_lo <= key <= lim_hi
    const int lim_hi = p.mask != RF_MASK_NONE ? min(khi - 1, my_pos) : khi - 1;
    const int lim_lo = p.mask == RF_MASK_SLIDING ? my_pos - p.window + 1 : -(1 << 30);

    // log2-domain scale; kept >= 1e-30 so masked -inf scores stay -inf after
    // the multiply (scale 0 then gives exactly uniform weights).
    const float c = fmaxf(p.scale * LOG2E, 1e-30f);
    // ALiBi: the scaled score gets -slope_h * |p_i - j|, here in log2 units
    const float slope2 = ALIBI ? p.alibi[h] * LOG2E : 0.f;
    const size_t kv_base = ((size_t)b * p.Hkv + g) * (size_t)p.Nk * D;
    // K and V of this (batch, KV head); rows past Nk read as zeros
    const int kv_bytes = p.Nk * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc((const T*)p.k + kv_base, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const T*)p.v + kv_base, kv_bytes);

    // ---------------- Q^T operand (+ RoPE), loaded once
    // lane element n in [0, D/2): d(n) = 16*(n/8) + 8*hi + n%8 (16-bit)
    //                                   = 2*n + hi               (f32)
    // its rotation partner d(n) + D/2 is element n + D/4 of the same lane.
    constexpr int QN = D / 2;
    float qf[QN];
    {
        const bool ok = my_row < p.Nq;
        const T* qrow = (const T*)p.q + (((size_t)b * p.Hq + h) * p.Nq + (size_t)min(my_row, p.Nq - 1)) * D;
        if constexpr (F32) {
#pragma unroll
            for (int n = 0; n < QN; ++n) qf[n] = ok ? qrow[2 * n + hi] : 0.f;
        } else {
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const VecT x = *(const VecT*)(qrow + 16 * ks + 8 * hi);
#pragma unroll
                for (int i = 0; i < 8; ++i) qf[8 * ks + i] = ok ? to_f32(x[i]) : 0.f;
            }
        }
        if (ROPE) {
#pragma unroll
            for (int n = 0; n < QN / 2; ++n) {
                const int d = F32 ? 2 * n + hi : 16 * (n / 8) + 8 * hi + (n % 8);
                float cs, sn;
                rope_cos_sin(p.rope.inv_period[d], my_pos, cs, sn);
                const float x = qf[n], y = qf[n + QN / 2];
                qf[n] = x * cs - y * sn;
                qf[n + QN / 2] = x * sn + y * cs;
            }
        }
    }
    constexpr int NKS = F32 ? D / 2 : D / 16;  // contraction steps over d
    VecT qv[F32 ? 1 : NKS];
    VecT qlo[SPLITK ? NKS : 1];
    float qs[F32 ? NKS : 1];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (F32) {
            qs[ks] = qf[ks];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qv[ks][i] = from_f32<T>(qf[8 * ks + i]);
                if constexpr (SPLITK) qlo[ks][i] = from_f32<T>(qf[8 * ks + i] - to_f32(qv[ks][i]));
            }
        }
    }

    // ---------------- RoPE state for this thread's K chunks
    // With RoPE the thread loads chunk cc and its partner cc + CPR/2 of rows
    // row0 + j * RSTEP (j < CH/2) of each tile, so it rotates by the angles
    // (k0 + row0 + j * RSTEP) * theta_d, d = cc * EPC + e.  Tiles are stored in
    // key order, BN keys apart, so (rc, rs) = (cos, sin) of the j = 0 angle is
    // carried from tile to tile by the angle-addition identity with the
    // per-frequency step (cos, sin)(BN * theta_d), and rows j > 0 follow with
    // (cos, sin)(RSTEP * theta_d); both steps sit in LDS.  Every
    // ROPE_REANCHOR-th tile the angle is taken exactly again (fp64 fraction
    // of revolutions, then v_sin/v_cos), so float rounding of the recurrence
    // cannot build up over long key ranges.
    constexpr int RSTEP = 2 * GT / CPR;  // rows between a thread's pairs
    constexpr int ROPE_REANCHOR = 64;
    float rc[ROPE ? EPC : 1], rs[ROPE ? EPC : 1];
    __shared__ float2 rope_step[ROPE ? D : 1];     // [d]: BN * theta_d; [D/2 + d]: RSTEP * theta_d
    __shared__ double rope_ip[ROPE ? D / 2 : 1];  // theta_d / (2 pi)
    if (ROPE) {
        if (tid < D / 2) {
            const double ip = p.rope.inv_period[tid];
            float c1, s1, c2, s2;
            rope_cos_sin(ip, BN, c1, s1);
            rope_cos_sin(ip, RSTEP, c2, s2);
            rope_step[tid] = make_float2(c1, s1);
            rope_step[D / 2 + tid] = make_float2(c2, s2);
            rope_ip[tid] = ip;
        }
        __syncthreads();
    }

    // ---------------- tile staging
    // V1: one wave load writes 16 bytes per lane, lane-major, i.e. 64
    // consecutive 16-byte slots of the padded row layout; a lane whose slot is
    // a row's pad reads past the buffer end and gets zeros.  Otherwise:
    // global -> registers -> LDS (RoPE rotates K on the way).
    constexpr int SPR = CPR + 1;                  // 16-byte slots per LDS row (pitch KS)
    constexpr int NLW = (SPR + FWD_WAVES - 1) / FWD_WAVES;
    static_assert(!V1 || (BN == 64 && C::K_ELEMS == BN * KS), "one wave load per 64 slots");
    unsigned dma_off[V1 ? NLW : 1];
    if constexpr (V1) {
#pragma unroll
        for (int i = 0; i < NLW; ++i) {
            const int p_ = 64 * ((wave + FWD_WAVES * i) % SPR) + lane;
            const int row = p_ / SPR, ch = p_ % SPR;
            dma_off[i] = ch < CPR ? (unsigned)((row * D + ch * EPC) * (int)sizeof(T)) : 0x80000000u;
        }
    }
    // the BN rows of K or V from key k0 into dst (a K buffer or the V buffer)
    auto issue_rows = [&](__amdgpu_buffer_rsrc_t rs, T* dst, int k0) {
        const unsigned base = (unsigned)k0 * (unsigned)(D * sizeof(T));
#pragma unroll
        for (int i = 0; i < NLW; ++i) {
            const int jj = wave + FWD_WAVES * i;  // wave-uniform
            if (jj < SPR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + jj * 64 * EPC),
                                                         16, (int)(base + dma_off[i]), 0, 0, 0);
        }
    };

    uint4 kreg[V1 ? 1 : C::CH], vreg[V1 ? 1 : C::CH];

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int it = 0; it < C::CH; ++it) {
            int row, ch;
            if (ROPE) {  // pairs (cc, cc + CPR/2)
                const int u = (it / 2) * GT + gtid;
                row = u / (CPR / 2);
                ch = u % (CPR / 2) + (it % 2) * (CPR / 2);
            } else {
                const int u = it * GT + gtid;
                row = u / CPR;
                ch = u % CPR;
            }
            kreg[it] = buf_load16(krs, ((unsigned)(k0 + row) * D + ch * EPC) * (unsigned)sizeof(T));
        }
#pragma unroll
        for (int it = 0; it < C::CH; ++it) {
            const int u = it * GT + gtid;
            vreg[it] = buf_load16(vrs, ((unsigned)(k0 + u / CPR) * D + (u % CPR) * EPC) * (unsigned)sizeof(T));
        }
    };

    auto store_tile = [&](int stage, int k0) {
        T* ks_ = gsm + stage * C::STAGE;
        T* vs_ = ks_ + C::K_ELEMS;
        if (ROPE) {
            const int cc = gtid % (CPR / 2);
            if (((k0 - kbeg) / BN) % ROPE_REANCHOR == 0) {
                const int pos = k0 + gtid / (CPR / 2);
#pragma unroll
                for (int e = 0; e < EPC; ++e) rope_cos_sin(rope_ip[cc * EPC + e], pos, rc[e], rs[e]);
            } else {
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    const float2 st = rope_step[cc * EPC + e];
                    const float c_ = rc[e] * st.x - rs[e] * st.y;
                    rs[e] = rs[e] * st.x + rc[e] * st.y;
                    rc[e] = c_;
                }
            }
            float cj[EPC], sj[EPC];  // angle of pair j, starting at row0
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                cj[e] = rc[e];
                sj[e] = rs[e];
            }
#pragma unroll
            for (int it = 0; it < C::CH; it += 2) {
                const int u = (it / 2) * GT + gtid;
                const int row = u / (CPR / 2);
                if (it > 0) {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        const float2 st = rope_step[D / 2 + cc * EPC + e];
                        const float c_ = cj[e] * st.x - sj[e] * st.y;
                        sj[e] = sj[e] * st.x + cj[e] * st.y;
                        cj[e] = c_;
                    }
                }
                const VecT lo = *(const VecT*)&kreg[it];
                const VecT hi_ = *(const VecT*)&kreg[it + 1];
                VecT olo, ohi, rlo, rhi;
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    const float cs = cj[e], sn = sj[e];
                    const float x = to_f32(lo[e]), y = to_f32(hi_[e]);
                    const float xr = x * cs - y * sn, yr = x * sn + y * cs;
                    olo[e] = from_f32<T>(xr);
                    ohi[e] = from_f32<T>(yr);
                    if constexpr (SPLITK) {
                        rlo[e] = from_f32<T>(xr - to_f32(olo[e]));
                        rhi[e] = from_f32<T>(yr - to_f32(ohi[e]));
                    }
                }
                *(VecT*)(ks_ + row * KS + cc * EPC) = olo;
                *(VecT*)(ks_ + row * KS + (cc + CPR / 2) * EPC) = ohi;
                if constexpr (SPLITK) {
                    T* kl = ks_ + BN * KS;
                    *(VecT*)(kl + row * KS + cc * EPC) = rlo;
                    *(VecT*)(kl + row * KS + (cc + CPR / 2) * EPC) = rhi;
                }
            }
        } else {
#pragma unroll
            for (int it = 0; it < C::CH; ++it) {
                const int u = it * GT + gtid;
                *(uint4*)(ks_ + (u / CPR) * KS + (u % CPR) * EPC) = kreg[it];
            }
        }
#pragma unroll
        for (int it = 0; it < C::CH; ++it) {
            const int u = it * GT + gtid;
            *(uint4*)(vs_ + (u / CPR) * KS + (u % CPR) * EPC) = vreg[it];
        }
    };

    // V^T operand addressing for the transpose read (16-bit types): lane
    // (q = lane/16, j = lane%16) names V[16t + 4*hi + j/4 (+8)][32db + 16(q&1) + 4(j&3)]
    // and receives V[16t + 4*hi + k (+8)][32db + lane%32] in slot k = 0..3, so
    // contraction slot (hi, i) holds key 16t + 8*(i/4) + 4*hi + i%4: the key of
    // score register 8*(t%2) + i in this lane half.
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // ---------------- running state
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_ref = -INFINITY;  // reference max (log2 units of the scaled scores)
    float l_run = 0.f;

    if (ntiles > 0) {
        if constexpr (V1) {
            issue_rows(krs, smem, klo + tcur * BN);
        } else {
            load_tile(kbeg);
            store_tile(0, kbeg);
        }
    }

    for (int t = 0; t < nsteps; ++t) {
        int k0, k0n;  // this step's tile and the next one's
        if constexpr (V1) {
            k0 = klo + tcur * BN;
            tcur = tcur + 1 == ntiles ? 0 : tcur + 1;
            k0n = klo + tcur * BN;
        } else {
            k0 = kbeg + t * BN;
            k0n = k0 + BN;
        }
        const int stage = t & 1;
        if constexpr (V1) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(t) landed
        __syncthreads();
        if constexpr (V1) {
            issue_rows(vrs, smem + 2 * C::K_ELEMS, k0);
            if (t + 1 < ntiles) issue_rows(krs, smem + (stage ^ 1) * C::K_ELEMS, k0n);
        } else if (t + 1 < ntiles) {
            load_tile(k0n);
        }

        // wave-level skip / mask decisions
        bool skip = !wave_live || t >= ntiles;
        bool need_mask = (k0 + BN > khi);
        if (p.mask != RF_MASK_NONE) {
            skip |= k0 > pw_max;
            need_mask |= (k0 + BN - 1 > pw_min);
            if (p.mask == RF_MASK_SLIDING) {
                skip |= (k0 + BN - 1 <= pw_min - p.window);
                need_mask |= (k0 <= pw_max - p.window);
            }
        }

        const T* ks_ = V1 ? smem + stage * C::K_ELEMS : gsm + stage * C::STAGE;
        const T* vs_ = V1 ? smem + 2 * C::K_ELEMS : ks_ + C::K_ELEMS;
        float pr[NKB][16];
        if (!skip) {
            // S^T = K . Q^T
            f32x16 sacc[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sacc[kb] = f32x16{};
                const T* krow = ks_ + (32 * kb + l32) * KS;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if constexpr (F32) {
                        sacc[kb] = mfma32(krow[2 * ks + hi], qs[ks], sacc[kb]);
                    } else {
                        const VecT a = *(const VecT*)(krow + 16 * ks + 8 * hi);
                        sacc[kb] = mfma32(a, qv[ks], sacc[kb]);
                        if constexpr (SPLITK) {
                            const VecT al = *(const VecT*)(krow + BN * KS + 16 * ks + 8 * hi);
                            sacc[kb] = mfma32(a, qlo[ks], sacc[kb]);
                            sacc[kb] = mfma32(al, qv[ks], sacc[kb]);
                        }
                    }
                }
            }

            if (need_mask) {
                // register j of block kb holds key k0 + 4*hi + 32*kb + 8*(j/4) + j%4;
                // visible iff rel_lo <= offset <= rel_hi (rel_lo only binds for
                // the window)
                const int rel_hi = lim_hi - k0 - 4 * hi;
                const int rel_lo = lim_lo - k0 - 4 * hi;
                if constexpr (D == 128) {
                    // every element branch-free (compares combined with &):
                    // measured faster for the window-heavy D = 128 workloads
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int off = 32 * kb + 8 * (j / 4) + (j % 4);
                            sacc[kb][j] = ((off <= rel_hi) & (off >= rel_lo)) ? sacc[kb][j] : -INFINITY;
                        }
                } else {
                    // D = 64: this form keeps the register budget of 4 waves per SIMD
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int off = 32 * kb + 8 * (j / 4) + (j % 4);
                            const bool vis = p.mask == RF_MASK_SLIDING ? (off <= rel_hi && off >= rel_lo) : off <= rel_hi;
                            sacc[kb][j] = vis ? sacc[kb][j] : -INFINITY;
                        }
                }
            }

            if constexpr (ALIBI) {
                // scores to log2 units with the bias; key - position = kd + off
                const float kd = (float)(k0 + 4 * hi - my_pos);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float dist = fabsf(kd + (float)(32 * kb + 8 * (j / 4) + (j % 4)));
                        sacc[kb][j] = fmaf(sacc[kb][j], c, -slope2 * dist);
                    }
            }

            // level 1: tile max (log2 domain of the scaled scores)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
            mx = fmaxf(mx, swap_halves(mx));
            const float m_tile = ALIBI ? mx : mx * c;

            // lazy correction of levels 2 and 3: only when the max moved by > 2^8
            const bool bump = m_tile > m_ref + RESCALE_SLACK;
            if (__builtin_amdgcn_ballot_w64(bump)) {
                const float m_new = bump ? m_tile : m_ref;
                const float alpha = bump ? fast_exp2(m_ref - m_new) : 1.f;  // m_ref = -inf -> 0
                m_ref = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            }
            const float m_sub = (m_ref == -INFINITY) ? 0.f : m_ref;

            // level 2 terms: P = 2^(s*c - m_ref); masked entries give 2^-inf = 0
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    pr[kb][j] = fast_exp2(ALIBI ? sacc[kb][j] - m_sub : fmaf(sacc[kb][j], c, -m_sub));

        }
        if constexpr (V1) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's V(t) (and K(t+1)) landed
            __syncthreads();                     // ... and every other wave's
        }
        if (!skip) {
            // level 3: O^T += V^T . P^T (16-bit: the rounded P also feeds l)
            if constexpr (F32) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        l_run += pr[kb][j];
                        const int key = 32 * kb + 8 * (j / 4) + 4 * hi + (j % 4);
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            oacc[db] = mfma32(vs_[key * KS + 32 * db + l32], pr[kb][j], oacc[db]);
                    }
            } else {
#pragma unroll
                for (int t16 = 0; t16 < BN / 16; ++t16) {
                    VecT pb;
#pragma unroll
                    for (int i = 0; i < 8; ++i) pb[i] = from_f32<T>(pr[t16 / 2][8 * (t16 % 2) + i]);
                    l_run = row_sum8(pb, l_run);
                    const T* vrow = vs_ + (16 * t16 + tr_row) * KS + tr_col;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const i16x4 lo4 = lds_read_tr16(vrow + 32 * db);
                        const i16x4 hi4 = lds_read_tr16(vrow + 8 * KS + 32 * db);
                        const i16x8 ab = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                        oacc[db] = mfma32(__builtin_bit_cast(VecT, ab), pb, oacc[db]);
                    }
                }
            }
        }

        if constexpr (!V1) {
            if (t + 1 < ntiles) store_tile(stage ^ 1, k0n);
        }
    }

    if constexpr (KH) {
        // group 1 hands its state to group 0 through LDS, element-major
        // ([value][row slot][lane]) so the 64 lanes hit 64 banks
        constexpr int NV = NDB * 16 + 2;
        constexpr int RS = L::GWAVES;  // row slots
        float* xs = (float*)smem;
        static_assert(RS * NV * 64 * sizeof(float) <= sizeof(smem), "merge area");
        __syncthreads();  // every wave is done with the tile buffers
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) xs[((db * 16 + j) * RS + rw) * 64 + lane] = oacc[db][j];
            xs[((NV - 2) * RS + rw) * 64 + lane] = m_ref;
            xs[((NV - 1) * RS + rw) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (grp == 1) return;
        const float m1 = xs[((NV - 2) * RS + rw) * 64 + lane];
        const float l1 = xs[((NV - 1) * RS + rw) * 64 + lane];
        const float mm = fmaxf(m_ref, m1);
        const float a0 = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - mm);  // -inf - -inf would be NaN
        const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][j] = a0 * oacc[db][j] + a1 * xs[((db * 16 + j) * RS + rw) * 64 + lane];
        l_run = a0 * l_run + a1 * l1;
        m_ref = mm;
    }

    // ---------------- epilogue: O /= l, lse = ln sum exp
    const float l_tot = l_run + swap_halves(l_run);
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
    const float lse_v = live ? (m_ref + fast_log2(l_tot)) * LN2 : -INFINITY;
    if (!wave_live || my_row >= p.Nq) return;
    const size_t row_id = ((size_t)b * p.Hq + h) * p.Nq + (size_t)my_row;
    if (p.split_mode) {
        float* orow = p.o_part + (row_id * p.num_splits + split) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
                const int d0 = 32 * db + 8 * jq + 4 * hi;
                *(float4*)(orow + d0) = make_float4(oacc[db][4 * jq] * inv, oacc[db][4 * jq + 1] * inv,
                                                    oacc[db][4 * jq + 2] * inv, oacc[db][4 * jq + 3] * inv);
            }
        if (hi == 0) p.lse_part[row_id * p.num_splits + split] = lse_v;
    } else {
        T* orow = (T*)p.o + row_id * D;
        typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
                const int d0 = 32 * db + 8 * jq + 4 * hi;
                T4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(oacc[db][4 * jq + r] * inv);
                *(T4*)(orow + d0) = w;
            }
        if (hi == 0) p.lse[row_id] = lse_v;
    }
}

}  // namespace rf
