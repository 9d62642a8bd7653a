/*
 * rf_attn.h — C ABI of the MI355X (gfx950) single-pass fused cascaded-reduction
 * attention library (librfattn.so).
 *
 * What is computed.  Attention is "safe softmax followed by a GEMM", the
 * cascaded reduction named in the abstract of "RedFuser: An Automatic Operator
 * Fusion Framework for Cascaded Reductions on AI Accelerators" (Tang et al.):
 *     level 1 (max):       m_i = max_j s_ij
 *     level 2 (sum):       l_i = sum_j exp(s_ij - m_i)
 *     level 3 (sum of *):  O_i = sum_j exp(s_ij - m_i) / l_i * v_j
 * with s_ij = scale * q'_i . k'_j over the keys j visible to query i, fused
 * into one pass in the incremental form of RedFuser Fig. 4 (each key tile
 * updates a running (m, l, O) per query row).  q' and k' are q and k after the
 * optional pre-matmul rotary embedding of "AttnFuse: A Composable DSL for
 * Compiling Attentions to Fused GPU Kernels" (Dasoju, Zhao; abstract, Fig. 1);
 * the masks are the causal and sliding-window patterns of AttnFuse Table 6;
 * split-KV decode with a log-sum-exp merge is RedFuser Fig. 13 / AttnFuse
 * Table 8.
 *
 * Conventions shared by every entry point
 *  - Layout: q [B, Hq, Nq, D], k and v [B, Hkv, Nk, D], o [B, Hq, Nq, D], all
 *    contiguous row-major: element (b, h, n, d) is at ((b*H + h)*N + n)*D + d.
 *    lse [B, Hq, Nq] float32 at (b*Hq + h)*Nq + i.
 *  - Query row i sits at position Nk - Nq + i, key row j at position j.
 *    Causal: j visible iff j <= Nk - Nq + i.  Sliding window W: additionally
 *    j > Nk - Nq + i - W (W counts the diagonal).  A row that sees no key gets
 *    o = 0 and lse = -inf.
 *  - GQA: query head h reads KV head h / (Hq / Hkv).
 *  - RoPE (rope_base > 0): pairs (x[i], x[i + D/2]) of q and k, i < D/2, are
 *    rotated by angle pos * rope_base^(-2i/D) before the product; v is not
 *    rotated; rope_base <= 0 disables it.
 *  - lse is the natural-log log-sum-exp of the scaled, masked, rotated scores.
 *  - Arithmetic: 16-bit inputs feed MFMA with float32 accumulation; softmax
 *    state, O accumulation and lse are float32; o is rounded to the input
 *    dtype once, round-to-nearest-even.
 *  - Memory: every pointer is device memory owned by the caller; q, k, v, o
 *    (and o_part) must be 16-byte aligned; outputs must not alias inputs.
 *    The library never allocates device memory.
 *  - Asynchrony: each call validates its arguments on the host, enqueues its
 *    kernels on `stream` (0 = the null stream) and returns; faults during
 *    execution surface at the caller's next synchronisation.
 *  - Errors: validation happens before any launch; a non-OK status launches
 *    nothing.  RF_ERR_INVALID_ARG: null pointer for a non-empty tensor,
 *    negative size, Hq % Hkv != 0, scale negative or not finite, window < 1
 *    with the sliding mask, unknown mask or dtype, misaligned pointer.
 *    RF_ERR_UNSUPPORTED: D not in {64, 128}, or one KV head of 2 GiB or more
 *    (Nk * D * element size >= 2^31: in-head offsets are 32-bit).
 *    RF_ERR_HIP: a launch failed.
 *    rf_last_error() returns a thread-local message for the last non-OK
 *    status of the calling thread.
 *  - All entry points are thread-safe and keep no state between calls.
 */
#ifndef RF_ATTN_H
#define RF_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RF_OK = 0,
    RF_ERR_INVALID_ARG = 1,
    RF_ERR_UNSUPPORTED = 2,
    RF_ERR_HIP = 3
} rf_status;

typedef enum { RF_F32 = 0, RF_F16 = 1, RF_BF16 = 2 } rf_dtype;

typedef enum { RF_MASK_NONE = 0, RF_MASK_CAUSAL = 1, RF_MASK_SLIDING = 2 } rf_mask;

/*
 * rf_attn_fwd — fused forward (RedFuser Fig. 3b / Fig. 4b; AttnFuse Tables 1-7).
 *
 * q, k, v: inputs of `dtype` in the layout above.  o: output, same dtype as q.
 * lse: float32 [B, Hq, Nq], required.  Sizes: B, Nq, Nk >= 0 (zero means an
 * empty problem: nothing is read; with Nk == 0 every row gets o = 0,
 * lse = -inf), Hq, Hkv >= 1, D in {64, 128}.  scale >= 0 multiplies q'.k'.
 * mask_kind: rf_mask.  window: W for RF_MASK_SLIDING, ignored otherwise.
 * rope_base: > 0 enables RoPE with that base.
 * 16-bit D = 64 launches whose grid is small (at most about two 128-row
 * query blocks per compute unit) run each work-group's key range as two
 * halves merged on chip, either in 64-row work-groups of 4 waves (layout 1)
 * or in 128-row work-groups of 8 waves (layout 2, unmasked grids of one to
 * two blocks per compute unit); the environment variable RF_ATTN_KEY_HALVES=0, 1 or 2 forces a
 * layout (read at every call).  All layouts compute the same quantity; the
 * summation order differs.
 */
rf_status rf_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int D,
                      float scale, int mask_kind, int window, float rope_base,
                      int dtype, hipStream_t stream);

/*
 * rf_attn_splitkv_fwd — split-KV partials (RedFuser Fig. 13, FlashDecoding;
 * AttnFuse Table 8).  The keys are cut into num_splits chunks; chunk c covers
 * [c*ceil(Nk/S), min(Nk, (c+1)*ceil(Nk/S))).  For every query row and chunk it
 * writes the chunk's normalised output and its log-sum-exp:
 *   o_part   float32 [B, Hq, Nq, S, D]  at (((b*Hq + h)*Nq + i)*S + c)*D + d
 *   lse_part float32 [B, Hq, Nq, S]     at ((b*Hq + h)*Nq + i)*S + c
 * A chunk with no visible key gets o_part = 0 and lse_part = -inf.  Other
 * arguments as rf_attn_fwd.  1 <= num_splits <= 4096.
 */
rf_status rf_attn_splitkv_fwd(const void* q, const void* k, const void* v,
                              float* o_part, float* lse_part,
                              int B, int Hq, int Hkv, int Nq, int Nk, int D,
                              float scale, int mask_kind, int window, float rope_base,
                              int num_splits, int dtype, hipStream_t stream);

/*
 * rf_attn_fwd_alibi / rf_attn_splitkv_fwd_alibi — the same two calls with an
 * ALiBi bias (AttnFuse Table 6, "Causal+ALiBi"): query head h adds
 * -alibi_slopes[h] * |p_i - j| to the scaled score of every visible pair
 * before the softmax.  alibi_slopes: device float32 [Hq], 4-byte aligned, read
 * by the kernels; NULL means no bias (identical to the calls above).  The
 * slope schedule is the caller's choice (the usual one is 2^(-8h/Hq),
 * h = 1..Hq).  Other arguments, layouts and errors as above.
 */
rf_status rf_attn_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nk, int D,
                            float scale, int mask_kind, int window, float rope_base,
                            const float* alibi_slopes, int dtype, hipStream_t stream);
rf_status rf_attn_splitkv_fwd_alibi(const void* q, const void* k, const void* v,
                                    float* o_part, float* lse_part,
                                    int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                    float scale, int mask_kind, int window, float rope_base,
                                    const float* alibi_slopes, int num_splits, int dtype,
                                    hipStream_t stream);

/*
 * rf_splitkv_num_splits — a chunk count for rf_attn_splitkv_fwd (the split
 * of FlashDecoding, RedFuser Fig. 13; the decode geometries of AttnFuse
 * Table 8).  The pages fix no rule; this one is measured on MI355X.  The
 * partial kernel runs one work-group per (chunk, KV head, batch), so
 *   S = ceil(RF_SPLIT_GROUPS_PER_CU * cu_count / (B * Hkv)),
 * about two work-groups per compute unit, then capped so every chunk keeps
 * at least RF_SPLIT_MIN_KEYS keys (S <= ceil(Nk / RF_SPLIT_MIN_KEYS)), and
 * clamped to [1, 4096].  (More chunks add merge work that batch-1 steps
 * feel: with graph-replayed steps this rule is the fastest chunk count, or
 * within 0.3 %, at batch 1 for AttnFuse Table 8's geometries, and within
 * 1.2 % at batch 16.)  cu_count <= 0 asks the current device (falls back to
 * 256).  Returns 0 for invalid sizes (B < 1, Hkv < 1, Nk < 0).
 */
#define RF_SPLIT_GROUPS_PER_CU 2
#define RF_SPLIT_MIN_KEYS 128
int rf_splitkv_num_splits(int B, int Hkv, int Nk, int cu_count);

/*
 * rf_splitkv_workspace_bytes — bytes of o_part plus lse_part for the given
 * sizes: B*Hq*Nq*num_splits*(D + 1)*4.  Returns 0 for invalid sizes.
 */
size_t rf_splitkv_workspace_bytes(int B, int Hq, int Nq, int D, int num_splits);

/*
 * rf_lse_merge — merge split-KV partials by log-sum-exp (the level-1/level-2
 * cascade applied over chunks, RedFuser Fig. 4 and Fig. 13):
 *   M = max_c lse_c,  lse = M + ln sum_c exp(lse_c - M),
 *   o = sum_c exp(lse_c - lse) * o_c, rounded once to out_dtype.
 * o_part float32 [rows, S, D], lse_part float32 [rows, S]; o [rows, D] of
 * out_dtype, lse float32 [rows].  Rows whose chunks are all empty get o = 0,
 * lse = -inf.  rows >= 0 (< 2^31), 1 <= num_splits <= 4096, D in {64, 128}.
 * o_part must be 16-byte aligned and o aligned to 4 of its elements.
 */
rf_status rf_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                       int rows, int num_splits, int D, int out_dtype, hipStream_t stream);

/*
 * rf_rope_rotate — the rotary embedding alone, as a separate pass over HBM
 * (the "pre-rotate" alternative of AttnFuse's Rotation Calculus: abstract,
 * Table 4).  x, y: [rows, N, D] of dtype (rows = B*H), 16-byte aligned; y may
 * equal x (in place).  Row n of every [N, D] slice is rotated to position
 * pos_offset + n: pairs (x[i], x[i + D/2]), i < D/2, turn by
 * (pos_offset + n) * base^(-2i/D), rounded once to dtype.  Use pos_offset =
 * Nk - Nq for queries and 0 for keys to match rf_attn_fwd's positions.
 * base > 0.  rows, N >= 0; D in {64, 128}.
 */
rf_status rf_rope_rotate(const void* x, void* y, int rows, int N, int D, float base, int pos_offset,
                         int dtype, hipStream_t stream);

/*
 * rf_attn_bwd — gradients of rf_attn_fwd (the backward of a training step:
 * AttnFuse abstract and Table 9, forward + backward + optimiser step).  The
 * pages print no backward formulas; this is the chain rule through the
 * forward's definition, with P recomputed from the saved lse:
 *   P_ij = exp(s_ij - lse_i),   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,
 *   D_i = dO_i . o_i,           dS_ij = P_ij (dP_ij - D_i),
 *   dq_i = R(p_i)^T scale sum_j dS_ij k'_j,   dk_j = R(j)^T scale sum_i dS_ij q'_i
 * (R = the RoPE rotation; ALiBi adds an input-independent bias, its slopes get
 * no gradient).  With GQA, dk and dv sum over the Hq/Hkv query heads of the
 * group.  lse is taken as not feeding the loss (its gradient is zero).
 *
 * q, k, v, o, lse: the forward's inputs and outputs (same mask, window,
 * rope_base, scale and slopes as the forward call).  dout: gradient of the
 * loss with respect to o, layout of o.  dq [B, Hq, Nq, D], dk and dv
 * [B, Hkv, Nk, D]: outputs of `dtype`, every element written (keys no query
 * sees get 0).  workspace: device float32 buffer of at least
 * rf_attn_bwd_workspace_bytes(B, Hq, Nq) bytes, 4-byte aligned, overwritten.
 * dtype: RF_F16 or RF_BF16 (RF_F32 returns RF_ERR_UNSUPPORTED).  P and dS
 * are rounded to dtype for the matrix products, accumulation is float32,
 * each output is rounded once.  Deterministic: no atomics.
 * Errors as the forward, plus RF_ERR_INVALID_ARG for a missing output or
 * workspace.
 */
rf_status rf_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* workspace,
                      int B, int Hq, int Hkv, int Nq, int Nk, int D,
                      float scale, int mask_kind, int window, float rope_base,
                      const float* alibi_slopes, int dtype, hipStream_t stream);

/* rf_attn_bwd_workspace_bytes — B*Hq*Nq*4 (the per-row D_i); 0 for invalid sizes. */
size_t rf_attn_bwd_workspace_bytes(int B, int Hq, int Nq);

/*
 * rf_attn_bwd_noalloc — rf_attn_bwd without the workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The row terms D_i
 * go to a static device array owned by the library, RF_BWD_NOALLOC_MAX_ROWS
 * floats (16 MiB) on each GPU the library runs on, held until the process
 * ends; its address is looked up once per device on the first call made
 * with that device current.  Nothing is allocated and no memset is issued
 * (the array needs no clearing: every row term is written before it is
 * read).  B*Hq*Nq above RF_BWD_NOALLOC_MAX_ROWS returns RF_ERR_UNSUPPORTED
 * before anything is launched.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  Other arguments, results and errors
 * as rf_attn_bwd.
 */
#define RF_BWD_NOALLOC_MAX_ROWS (1 << 22)
rf_status rf_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Nq, int Nk, int D,
                              float scale, int mask_kind, int window, float rope_base,
                              const float* alibi_slopes, int dtype, hipStream_t stream);

/*
 * rf_layernorm_fwd — LayerNorm, a second cascaded reduction run through the
 * same incremental machinery (RedFuser abstract and Table 1: a later
 * reduction that reads an earlier one's result; "Operator Fusion" guide,
 * section 2, Pattern 2: mean, then variance around it, then normalise):
 *   mean_r = sum_h x[r,h] / H,   var_r = sum_h (x[r,h] - mean_r)^2 / H,
 *   rstd_r = 1 / sqrt(var_r + eps),
 *   y[r,h] = (x[r,h] - mean_r) * rstd_r * gamma[h] + beta[h].
 * Each row is read from HBM once: a running (n, mean, M2) per lane is
 * updated chunk by chunk (a chunk that moves the mean by delta adds
 * delta^2 n_a n_b / n to M2), merged across the work-group, then the row is
 * normalised from registers.
 * x, y: [rows, H] of dtype, 16-byte aligned (y must not alias x); gamma,
 * beta: [H] of dtype, 16-byte aligned; mean, rstd: float32 [rows] outputs.
 * Statistics in float32, y rounded once to dtype.  rows >= 0, eps >= 0;
 * H a multiple of 8 (float16/bfloat16) or 4 (float32), at most 16384
 * (16-bit) or 8192 (float32), else RF_ERR_UNSUPPORTED.
 */
rf_status rf_layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y,
                           float* mean, float* rstd, int rows, int H, float eps,
                           int dtype, hipStream_t stream);

/*
 * rf_softmax_topk — softmax followed by TopK, a cascade on the max/+ row of
 * RedFuser Table 1 (TopK combines with max and shifts with +):
 *   m = max_e x_e,  l = sum_e exp(x_e - m),  and for the k largest
 *   p_e = exp(x_e - m) / l: values[r, j] = p and indices[r, j] = e,
 *   j = 0..k-1 in descending order.
 * Selection compares the exact input values (the k largest p are the k
 * largest x); equal values go to the lower index, so the result is unique.
 * A group of 16 lanes (E <= 256, k <= 16) or a whole wavefront per row
 * holds the row in registers: x is read once.
 * x: [rows, E] of dtype (2-byte aligned for 16-bit, 4 for float32); values:
 * float32 [rows, k]; indices: int32 [rows, k].  1 <= E <= 1024,
 * 1 <= k <= min(E, 64) (E above 1024 returns RF_ERR_UNSUPPORTED).  NaN
 * inputs are not supported.  p is float32 (relative error a few times
 * 2^-24 * (E + |x - m| log2 e)).
 */
rf_status rf_softmax_topk(const void* x, float* values, int* indices, int rows, int E, int k,
                          int dtype, hipStream_t stream);

/* rf_status_string — static text for a status code; any int is accepted
 * (codes outside rf_status give "unknown status"). */
const char* rf_status_string(int s);

/* rf_last_error — thread-local detail for the calling thread's last non-OK return. */
const char* rf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RF_ATTN_H */
