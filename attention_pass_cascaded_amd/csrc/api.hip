// Host side of the C ABI declared in include/rf_attn.h: argument validation,
// choice of kernel, launches on the caller's stream, status codes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>
#include <string>

#include "bwd_kernel.hpp"
#include "launch.hpp"
#include "layernorm_kernel.hpp"
#include "merge_kernel.hpp"
#include "rope_kernel.hpp"
#include "topk_kernel.hpp"

namespace {

thread_local std::string g_last_error;

rf_status fail(rf_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

rf_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return RF_OK;
    return fail(RF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Compute units of the current device, cached per device (0 if the query fails).
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev >= 64) {
        int n = 0;
        return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cache[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}

// theta_i / (2 pi) = base^(-2i/D) / (2 pi), i < D/2, in double on the host.
rf::RopeTable rope_table(float base, int D) {
    rf::RopeTable t{};
    const double two_pi = 6.283185307179586476925;
    for (int i = 0; i < D / 2 && i < 64; ++i) t.inv_period[i] = pow((double)base, -2.0 * i / D) / two_pi;
    return t;
}

// Shared validation of the attention arguments.  Fills p on success.
rf_status check_attn(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int Nq,
                     int Nk, int D, float scale, int mask_kind, int window, float rope_base,
                     int dtype, rf::AttnParams& p) {
    if (B < 0 || Nq < 0 || Nk < 0) return fail(RF_ERR_INVALID_ARG, "negative size (B=%d Nq=%d Nk=%d)", B, Nq, Nk);
    if (Hq < 1 || Hkv < 1) return fail(RF_ERR_INVALID_ARG, "Hq and Hkv must be >= 1 (Hq=%d Hkv=%d)", Hq, Hkv);
    if (Hq % Hkv) return fail(RF_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (dtype != RF_F32 && dtype != RF_F16 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (mask_kind != RF_MASK_NONE && mask_kind != RF_MASK_CAUSAL && mask_kind != RF_MASK_SLIDING)
        return fail(RF_ERR_INVALID_ARG, "unknown mask kind %d", mask_kind);
    if (mask_kind == RF_MASK_SLIDING && window < 1)
        return fail(RF_ERR_INVALID_ARG, "sliding window needs window >= 1 (got %d)", window);
    if (!isfinite(scale) || scale < 0.f) return fail(RF_ERR_INVALID_ARG, "scale must be finite and >= 0");
    if (isnan(rope_base) || isinf(rope_base)) return fail(RF_ERR_INVALID_ARG, "rope_base must be finite");
    if (D != 64 && D != 128) return fail(RF_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", D);
    const bool q_nonempty = (size_t)B * Nq > 0;
    const bool kv_nonempty = (size_t)B * Nk > 0;
    if (q_nonempty && !q) return fail(RF_ERR_INVALID_ARG, "q is null");
    if (kv_nonempty && (!k || !v)) return fail(RF_ERR_INVALID_ARG, "k or v is null");
    if ((q && !aligned16(q)) || (k && !aligned16(k)) || (v && !aligned16(v)))
        return fail(RF_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
    if ((size_t)B * Hq > (size_t)1 << 30) return fail(RF_ERR_INVALID_ARG, "B*Hq too large");
    if ((size_t)Nk * D * (dtype == RF_F32 ? 4 : 2) >= ((size_t)1 << 31))
        return fail(RF_ERR_UNSUPPORTED, "one KV head must be < 2 GiB (Nk*D*elem_size)");
    p = rf::AttnParams{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = Nq;
    p.Nk = Nk;
    p.D = D;
    p.scale = scale;
    p.mask = mask_kind;
    p.window = mask_kind == RF_MASK_SLIDING ? window : 0;
    p.rope_base = rope_base > 0.f ? rope_base : 0.f;
    if (p.rope_base > 0.f) p.rope = rope_table(p.rope_base, D);
    p.num_splits = 1;
    p.split_len = Nk;
    p.cu_count = device_cu_count();
    return RF_OK;
}

hipError_t launch_fwd(const rf::AttnParams& p, int dtype, hipStream_t s) {
    switch (dtype) {
        case RF_F32: return rf::launch_fwd_f32(p, s);
        case RF_F16: return rf::launch_fwd_f16(p, s);
        default: return rf::launch_fwd_bf16(p, s);
    }
}

hipError_t launch_decode(const rf::AttnParams& p, int dtype, hipStream_t s) {
    switch (dtype) {
        case RF_F32: return rf::launch_decode_f32(p, s);
        case RF_F16: return rf::launch_decode_f16(p, s);
        default: return rf::launch_decode_bf16(p, s);
    }
}

}  // namespace

extern "C" {

rf_status rf_attn_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                            int Hq, int Hkv, int Nq, int Nk, int D, float scale, int mask_kind, int window,
                            float rope_base, const float* alibi_slopes, int dtype, hipStream_t stream) {
    rf::AttnParams p;
    rf_status st = check_attn(q, k, v, B, Hq, Hkv, Nq, Nk, D, scale, mask_kind, window, rope_base, dtype, p);
    if (st != RF_OK) return st;
    if (alibi_slopes && ((uintptr_t)alibi_slopes & 3u)) return fail(RF_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if ((size_t)B * Nq == 0) return RF_OK;
    if (!o || !lse) return fail(RF_ERR_INVALID_ARG, "o and lse are required");
    if (!aligned16(o) || ((uintptr_t)lse & 3u)) return fail(RF_ERR_INVALID_ARG, "o must be 16-byte aligned, lse 4-byte aligned");
    if ((size_t)B * Hq * ((Nq + rf::FWD_BM - 1) / rf::FWD_BM) > 0x7fffffffu)
        return fail(RF_ERR_INVALID_ARG, "B*Hq*ceil(Nq/128) too large");
    p.o = o;
    p.lse = lse;
    p.alibi = alibi_slopes;
    return hip_status(launch_fwd(p, dtype, stream), "rf_attn_fwd launch");
}

rf_status rf_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                      int Hkv, int Nq, int Nk, int D, float scale, int mask_kind, int window,
                      float rope_base, int dtype, hipStream_t stream) {
    return rf_attn_fwd_alibi(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, D, scale, mask_kind, window, rope_base,
                             nullptr, dtype, stream);
}

int rf_splitkv_num_splits(int B, int Hkv, int Nk, int cu_count) {
    if (B < 1 || Hkv < 1 || Nk < 0) return 0;
    if (cu_count <= 0) cu_count = device_cu_count();
    if (cu_count <= 0) cu_count = 256;
    const long long heads = (long long)B * Hkv;
    long long s = ((long long)RF_SPLIT_GROUPS_PER_CU * cu_count + heads - 1) / heads;
    const long long cap = ((long long)Nk + RF_SPLIT_MIN_KEYS - 1) / RF_SPLIT_MIN_KEYS;
    if (s > cap) s = cap;
    if (s > 4096) s = 4096;
    return s < 1 ? 1 : (int)s;
}

size_t rf_splitkv_workspace_bytes(int B, int Hq, int Nq, int D, int num_splits) {
    if (B < 0 || Hq < 1 || Nq < 0 || D < 1 || num_splits < 1) return 0;
    return (size_t)B * Hq * Nq * num_splits * (size_t)(D + 1) * sizeof(float);
}

rf_status rf_attn_splitkv_fwd_alibi(const void* q, const void* k, const void* v, float* o_part,
                                    float* lse_part, int B, int Hq, int Hkv, int Nq, int Nk, int D, float scale,
                                    int mask_kind, int window, float rope_base, const float* alibi_slopes,
                                    int num_splits, int dtype, hipStream_t stream) {
    rf::AttnParams p;
    rf_status st = check_attn(q, k, v, B, Hq, Hkv, Nq, Nk, D, scale, mask_kind, window, rope_base, dtype, p);
    if (st != RF_OK) return st;
    if (alibi_slopes && ((uintptr_t)alibi_slopes & 3u)) return fail(RF_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (num_splits < 1 || num_splits > 4096) return fail(RF_ERR_INVALID_ARG, "num_splits must be in [1, 4096] (got %d)", num_splits);
    if ((size_t)B * Nq == 0) return RF_OK;
    if (!o_part || !lse_part) return fail(RF_ERR_INVALID_ARG, "o_part and lse_part are required");
    if (!aligned16(o_part) || ((uintptr_t)lse_part & 3u))
        return fail(RF_ERR_INVALID_ARG, "o_part must be 16-byte aligned, lse_part 4-byte aligned");
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.num_splits = num_splits;
    p.split_len = (Nk + num_splits - 1) / num_splits;
    p.split_mode = 1;
    p.alibi = alibi_slopes;
    const int rows = (Hq / Hkv) * Nq;
    const int max_rows = dtype == RF_F32 ? rf::DEC_MAX_ROWS_F32 : rf::DEC_MAX_ROWS_16;
    if (rows <= max_rows && Hkv <= 65535 && B <= 65535)
        return hip_status(launch_decode(p, dtype, stream), "rf_attn_splitkv_fwd decode launch");
    if ((size_t)B * Hq * num_splits * ((Nq + rf::FWD_BM - 1) / rf::FWD_BM) > 0x7fffffffu)
        return fail(RF_ERR_INVALID_ARG, "B*Hq*num_splits*ceil(Nq/128) too large");
    return hip_status(launch_fwd(p, dtype, stream), "rf_attn_splitkv_fwd launch");
}

rf_status rf_attn_splitkv_fwd(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                              int B, int Hq, int Hkv, int Nq, int Nk, int D, float scale, int mask_kind,
                              int window, float rope_base, int num_splits, int dtype, hipStream_t stream) {
    return rf_attn_splitkv_fwd_alibi(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, D, scale, mask_kind, window,
                                     rope_base, nullptr, num_splits, dtype, stream);
}

rf_status rf_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse, int rows,
                       int num_splits, int D, int out_dtype, hipStream_t stream) {
    if (rows < 0) return fail(RF_ERR_INVALID_ARG, "rows must be >= 0");
    if (num_splits < 1 || num_splits > 4096) return fail(RF_ERR_INVALID_ARG, "num_splits must be in [1, 4096]");
    if (out_dtype != RF_F32 && out_dtype != RF_F16 && out_dtype != RF_BF16)
        return fail(RF_ERR_INVALID_ARG, "unknown dtype %d", out_dtype);
    if (D != 64 && D != 128) return fail(RF_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", D);
    if (rows == 0) return RF_OK;
    if (!o_part || !lse_part || !o || !lse) return fail(RF_ERR_INVALID_ARG, "null pointer");
    if (((uintptr_t)o_part & 15u) || ((uintptr_t)lse_part & 3u) || ((uintptr_t)lse & 3u) ||
        ((uintptr_t)o & (out_dtype == RF_F32 ? 15u : 7u)))
        return fail(RF_ERR_INVALID_ARG, "misaligned pointer (o_part 16 B, o 4 elements, lse 4 B)");
    return hip_status(rf::launch_merge(o_part, lse_part, o, lse, rows, num_splits, D, out_dtype, stream),
                      "rf_lse_merge launch");
}

rf_status rf_rope_rotate(const void* x, void* y, int rows, int N, int D, float base, int pos_offset, int dtype,
                         hipStream_t stream) {
    if (rows < 0 || N < 0) return fail(RF_ERR_INVALID_ARG, "negative size (rows=%d N=%d)", rows, N);
    if (dtype != RF_F32 && dtype != RF_F16 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (!isfinite(base) || base <= 0.f) return fail(RF_ERR_INVALID_ARG, "base must be finite and > 0");
    if (D != 64 && D != 128) return fail(RF_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", D);
    const long long rows_n = (long long)rows * N;
    if (rows_n == 0) return RF_OK;
    if (!x || !y) return fail(RF_ERR_INVALID_ARG, "x or y is null");
    if (!aligned16(x) || !aligned16(y)) return fail(RF_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if (pos_offset < 0 || (long long)pos_offset + N > 0x7fffffffLL) return fail(RF_ERR_INVALID_ARG, "positions out of range");
    const int epc = dtype == RF_F32 ? 4 : 8;
    const long long threads = rows_n * (D / 2 / epc);
    if ((threads + rf::ROPE_THREADS - 1) / rf::ROPE_THREADS > 0x7fffffffLL) return fail(RF_ERR_INVALID_ARG, "too large");
    dim3 grid((unsigned)((threads + rf::ROPE_THREADS - 1) / rf::ROPE_THREADS));
    const rf::RopeTable table = rope_table(base, D);
#define RF_ROPE_LAUNCH(TYPE, DD) \
    hipLaunchKernelGGL((rf::rope_rotate_kernel<TYPE, DD>), grid, dim3(rf::ROPE_THREADS), 0, stream, (const TYPE*)x, (TYPE*)y, rows_n, N, table, pos_offset)
    if (dtype == RF_F32) { if (D == 64) RF_ROPE_LAUNCH(float, 64); else RF_ROPE_LAUNCH(float, 128); }
    else if (dtype == RF_F16) { if (D == 64) RF_ROPE_LAUNCH(_Float16, 64); else RF_ROPE_LAUNCH(_Float16, 128); }
    else { if (D == 64) RF_ROPE_LAUNCH(__bf16, 64); else RF_ROPE_LAUNCH(__bf16, 128); }
#undef RF_ROPE_LAUNCH
    return hip_status(hipGetLastError(), "rf_rope_rotate launch");
}

size_t rf_attn_bwd_workspace_bytes(int B, int Hq, int Nq) {
    if (B < 0 || Hq < 1 || Nq < 0) return 0;
    return (size_t)B * Hq * Nq * sizeof(float);
}

}  // extern "C"

namespace {

// Row terms of rf_attn_bwd_noalloc: one library-owned array per GPU, kept
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host it only names the symbol); it uses the device address
// hipGetSymbolAddress returns, fetched once per device with that device
// current and cached here.
static __device__ __align__(256) float scratch[RF_BWD_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];

rf_status scratch_for_current_device(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(RF_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(RF_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
        g_scratch_ptr[dev] = (float*)ptr;
    }
    *out = g_scratch_ptr[dev];
    return RF_OK;
}

// Validation and launch shared by rf_attn_bwd and rf_attn_bwd_noalloc.
// workspace == nullptr with use_scratch: the row terms go to this device's
// scratch array (B*Hq*Nq <= RF_BWD_NOALLOC_MAX_ROWS, checked before the
// array's address is fetched).
rf_status attn_bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, float* workspace, bool use_scratch,
                        int B, int Hq, int Hkv, int Nq, int Nk, int D, float scale, int mask_kind, int window,
                        float rope_base, const float* alibi_slopes, int dtype, hipStream_t stream) {
    rf::AttnParams a;
    rf_status st = check_attn(q, k, v, B, Hq, Hkv, Nq, Nk, D, scale, mask_kind, window, rope_base, dtype, a);
    if (st != RF_OK) return st;
    if (dtype == RF_F32) return fail(RF_ERR_UNSUPPORTED, "rf_attn_bwd supports float16 and bfloat16 inputs");
    if (alibi_slopes && ((uintptr_t)alibi_slopes & 3u)) return fail(RF_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    const bool q_nonempty = (size_t)B * Nq > 0;
    const bool kv_nonempty = (size_t)B * Nk > 0;
    if (use_scratch && (size_t)B * Hq * Nq > (size_t)RF_BWD_NOALLOC_MAX_ROWS)
        return fail(RF_ERR_UNSUPPORTED, "B*Hq*Nq = %zu rows exceed the %d rows of the static row-term array",
                    (size_t)B * Hq * Nq, RF_BWD_NOALLOC_MAX_ROWS);
    if (q_nonempty && (!o || !lse || !dout || !dq || (!workspace && !use_scratch)))
        return fail(RF_ERR_INVALID_ARG, "o, lse, dout, dq and workspace are required");
    if (kv_nonempty && (!dk || !dv)) return fail(RF_ERR_INVALID_ARG, "dk and dv are required");
    if ((o && !aligned16(o)) || (dout && !aligned16(dout)) || (dq && !aligned16(dq)) || (dk && !aligned16(dk)) ||
        (dv && !aligned16(dv)) || (lse && ((uintptr_t)lse & 3u)) || (workspace && ((uintptr_t)workspace & 3u)))
        return fail(RF_ERR_INVALID_ARG, "o, dout, dq, dk, dv must be 16-byte aligned, lse and workspace 4-byte aligned");
    if ((size_t)B * Hq * ((Nq + rf::FWD_BM - 1) / rf::FWD_BM) > 0x7fffffffu ||
        (size_t)B * Hkv * ((Nk + rf::BWD_BK - 1) / rf::BWD_BK) > 0x7fffffffu)
        return fail(RF_ERR_INVALID_ARG, "grid too large");
    if (!q_nonempty && !kv_nonempty) return RF_OK;
    if (use_scratch) {
        st = scratch_for_current_device(&workspace);
        if (st != RF_OK) return st;
    }
    rf::BwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.drow = workspace;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = Nq;
    p.Nk = Nk;
    p.D = D;
    p.scale = scale;
    p.mask = a.mask;
    p.window = a.window;
    p.rope_base = a.rope_base;
    p.alibi = alibi_slopes;
    p.rope = a.rope;
    const hipError_t e = dtype == RF_F16 ? rf::launch_bwd_f16(p, stream) : rf::launch_bwd_bf16(p, stream);
    return hip_status(e, "rf_attn_bwd launch");
}

}  // namespace

extern "C" {

rf_status rf_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv,
                      int Nq, int Nk, int D, float scale, int mask_kind, int window, float rope_base,
                      const float* alibi_slopes, int dtype, hipStream_t stream) {
    return attn_bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, false, B, Hq, Hkv, Nq, Nk, D, scale,
                         mask_kind, window, rope_base, alibi_slopes, dtype, stream);
}

rf_status rf_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                              int Nk, int D, float scale, int mask_kind, int window, float rope_base,
                              const float* alibi_slopes, int dtype, hipStream_t stream) {
    return attn_bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, nullptr, true, B, Hq, Hkv, Nq, Nk, D, scale,
                         mask_kind, window, rope_base, alibi_slopes, dtype, stream);
}

rf_status rf_layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                           int rows, int H, float eps, int dtype, hipStream_t stream) {
    if (rows < 0 || H < 1) return fail(RF_ERR_INVALID_ARG, "rows must be >= 0 and H >= 1 (rows=%d H=%d)", rows, H);
    if (dtype != RF_F32 && dtype != RF_F16 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (!isfinite(eps) || eps < 0.f) return fail(RF_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const int epc = dtype == RF_F32 ? 4 : 8;
    if (H % epc) return fail(RF_ERR_UNSUPPORTED, "H must be a multiple of %d for this dtype (got %d)", epc, H);
    const int nch = (H / epc + rf::LN_THREADS - 1) / rf::LN_THREADS;
    if (nch > rf::LN_MAX_CHUNKS)
        return fail(RF_ERR_UNSUPPORTED, "H = %d too large (at most %d for this dtype)", H, rf::LN_THREADS * rf::LN_MAX_CHUNKS * epc);
    if (rows == 0) return RF_OK;
    if (!x || !gamma || !beta || !y || !mean || !rstd) return fail(RF_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || !aligned16(y) || ((uintptr_t)mean & 3u) ||
        ((uintptr_t)rstd & 3u))
        return fail(RF_ERR_INVALID_ARG, "x, gamma, beta, y must be 16-byte aligned, mean and rstd 4-byte aligned");
    dim3 grid((unsigned)rows);
#define RF_LN(TYPE, N)                                                                                    \
    hipLaunchKernelGGL((rf::layernorm_kernel<TYPE, N>), grid, dim3(rf::LN_THREADS), 0, stream, (const TYPE*)x, \
                       (const TYPE*)gamma, (const TYPE*)beta, (TYPE*)y, mean, rstd, H, eps)
#define RF_LN_T(TYPE)                           \
    if (nch <= 1) RF_LN(TYPE, 1);               \
    else if (nch <= 2) RF_LN(TYPE, 2);          \
    else if (nch <= 4) RF_LN(TYPE, 4);          \
    else RF_LN(TYPE, 8)
    if (dtype == RF_F32) { RF_LN_T(float); }
    else if (dtype == RF_F16) { RF_LN_T(_Float16); }
    else { RF_LN_T(__bf16); }
#undef RF_LN_T
#undef RF_LN
    return hip_status(hipGetLastError(), "rf_layernorm_fwd launch");
}

rf_status rf_softmax_topk(const void* x, float* values, int* indices, int rows, int E, int k, int dtype,
                          hipStream_t stream) {
    if (rows < 0) return fail(RF_ERR_INVALID_ARG, "rows must be >= 0 (got %d)", rows);
    if (dtype != RF_F32 && dtype != RF_F16 && dtype != RF_BF16) return fail(RF_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (E < 1 || E > 64 * rf::TOPK_MAX_VPL)
        return fail(RF_ERR_UNSUPPORTED, "E = %d not supported (1 .. %d)", E, 64 * rf::TOPK_MAX_VPL);
    if (k < 1 || k > E || k > rf::TOPK_MAX_K)
        return fail(RF_ERR_INVALID_ARG, "k must be in [1, min(E, %d)] (got %d)", rf::TOPK_MAX_K, k);
    if (rows == 0) return RF_OK;
    if (!x || !values || !indices) return fail(RF_ERR_INVALID_ARG, "null pointer");
    if (((uintptr_t)x & (dtype == RF_F32 ? 3u : 1u)) || ((uintptr_t)values & 3u) || ((uintptr_t)indices & 3u))
        return fail(RF_ERR_INVALID_ARG, "misaligned pointer");
    // 16 lanes per row when the row fits 16 values per lane and k <= 16
    // (measured: 8 lanes with 32 values each runs fewer instructions per row
    // but half the wavefronts, and was slower)
    const bool narrow = E <= 16 * rf::TOPK_MAX_VPL && k <= 16;
    const int lpr = narrow ? 16 : 64;
    const int rpb = (rf::TOPK_THREADS / 64) * (64 / lpr);
    dim3 grid((unsigned)((rows + rpb - 1) / rpb));
    const int vpl = (E + lpr - 1) / lpr;
    const int vec = dtype != RF_F32 && E % 8 == 0 && ((uintptr_t)x & 15u) == 0;
#define RF_TK(KERNEL, TYPE, N, L)                                                                          \
    hipLaunchKernelGGL((rf::KERNEL<TYPE, N, L>), grid, dim3(rf::TOPK_THREADS), 0, stream, (const TYPE*)x, values, \
                       indices, rows, E, k, vec)
#define RF_TK_V(KERNEL, TYPE, L)                   \
    if (vpl <= 1) RF_TK(KERNEL, TYPE, 1, L);       \
    else if (vpl <= 2) RF_TK(KERNEL, TYPE, 2, L);  \
    else if (vpl <= 4) RF_TK(KERNEL, TYPE, 4, L);  \
    else if (vpl <= 8) RF_TK(KERNEL, TYPE, 8, L);  \
    else RF_TK(KERNEL, TYPE, 16, L)
#define RF_TK_T(KERNEL, TYPE)                  \
    if (narrow) { RF_TK_V(KERNEL, TYPE, 16); } \
    else { RF_TK_V(KERNEL, TYPE, 64); }
    // 16-bit inputs: packed (value, index) keys; float32: (value, index) pairs
    if (dtype == RF_F32) { RF_TK_T(softmax_topk_kernel, float); }
    else if (dtype == RF_F16) { RF_TK_T(softmax_topk16_kernel, _Float16); }
    else { RF_TK_T(softmax_topk16_kernel, __bf16); }
#undef RF_TK_T
#undef RF_TK_V
#undef RF_TK
    return hip_status(hipGetLastError(), "rf_softmax_topk launch");
}

const char* rf_status_string(int s) {
    switch (s) {
        case RF_OK: return "ok";
        case RF_ERR_INVALID_ARG: return "invalid argument";
        case RF_ERR_UNSUPPORTED: return "unsupported";
        case RF_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* rf_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace rf {

template <typename T, int D>
static hipError_t merge_one(const float* op, const float* lp, void* o, float* lse, int rows, int S, hipStream_t s) {
    dim3 grid((unsigned)rows);
    hipLaunchKernelGGL((lse_merge_kernel<T, D>), grid, dim3(MRG_THREADS), 0, s, op, lp, (T*)o, lse, rows, S);
    return hipGetLastError();
}

hipError_t launch_merge(const float* op, const float* lp, void* o, float* lse, int rows, int S, int D, int dtype,
                        hipStream_t s) {
    if (dtype == RF_F32) return D == 64 ? merge_one<float, 64>(op, lp, o, lse, rows, S, s) : merge_one<float, 128>(op, lp, o, lse, rows, S, s);
    if (dtype == RF_F16) return D == 64 ? merge_one<_Float16, 64>(op, lp, o, lse, rows, S, s) : merge_one<_Float16, 128>(op, lp, o, lse, rows, S, s);
    return D == 64 ? merge_one<__bf16, 64>(op, lp, o, lse, rows, S, s) : merge_one<__bf16, 128>(op, lp, o, lse, rows, S, s);
}

}  // namespace rf
