// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, conversions and the per-call launch parameters.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rf_attn.h"

namespace rf {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// MI355X: 8 accelerator complex dies (XCDs) of 32 CUs, each with its own L2.
constexpr int NUM_XCD = 8;

// Fused forward work-group: 4 wavefronts of 32 query rows each.
constexpr int FWD_WAVES = 4;
constexpr int FWD_THREADS = 64 * FWD_WAVES;
constexpr int FWD_BM = 32 * FWD_WAVES;  // query rows per work-group

// theta_i / (2 pi) = base^(-2i/D) / (2 pi) for i < D/2, computed once on the
// host in double precision and passed by value with the launch.
struct RopeTable {
    double inv_period[64];
};

// Everything a launch needs, filled and validated on the host.
struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;           // final output (input dtype), or null in split mode
    float* lse;        // final lse, or null in split mode
    float* o_part;     // split mode: [B, Hq, Nq, S, D] float32
    float* lse_part;   // split mode: [B, Hq, Nq, S] float32
    int B, Hq, Hkv, Nq, Nk, D;
    float scale;
    int mask;          // rf_mask
    int window;
    float rope_base;   // > 0: RoPE on
    const float* alibi;  // [Hq] ALiBi slopes, or null
    RopeTable rope;      // theta_i / (2 pi), filled on the host when RoPE is on
    int num_splits;    // 1 when not splitting
    int split_len;     // keys per chunk, ceil(Nk / num_splits)
    int split_mode;    // 1: write normalised partials + chunk lse
    int cu_count;      // compute units of the device (work-group placement), 0 if unknown
    int launch_runs;   // work-groups per CU resident at launch (set by the forward launcher)
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Elements of T packed into 16 bytes.
template <typename T> struct Vec16;
template <> struct Vec16<_Float16> { typedef f16x8 type; static constexpr int n = 8; };
template <> struct Vec16<__bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };

// 32x32 output tile, float32 accumulate.  16-bit inputs: 16-deep contraction,
// lane l holds row/column (l % 32) and 8 consecutive contraction slots
// 8*(l/32)..+7 of each operand.  float32 inputs: 2-deep, one slot (l/32).
// Output register j of lane l is element [8*(j/4) + 4*(l/32) + j%4][l % 32].
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS transpose read: in each 16-lane group, lane j names 4 consecutive
// 16-bit elements M[j][0..3]; lane i receives M[4k + i/4][i%4] in slot k.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ptr));
}

// acc + sum of 8 packed 16-bit values, float32 accumulation (v_dot2 with ones).
__device__ __forceinline__ float row_sum8(const f16x8& v, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int i = 0; i < 8; i += 2) acc = __builtin_amdgcn_fdot2(f16x2{v[i], v[i + 1]}, one, acc, false);
    return acc;
}
__device__ __forceinline__ float row_sum8(const bf16x8& v, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 8; i += 2) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[i], v[i + 1]}, one, acc, false);
    return acc;
}

// Exchange with the lane 32 away (the other half of the wavefront):
// v_permlane32_swap trades the upper half of its first operand with the lower
// half of its second, so with x in both, lanes 0-31 find x[l+32] in the second
// result and lanes 32-63 find x[l-32] in the first.
__device__ __forceinline__ float swap_halves(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
}

// Raw buffer resource over [base, base + bytes): 16-byte loads at byte
// offsets at or past `bytes` return zeros without touching memory.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// byte_off is the hardware's unsigned 32-bit offset: computed in unsigned
// arithmetic, an offset past the range (up to 2^32 - 1) reads zeros.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// RoPE angle of frequency i at integer position pos, returned as (cos, sin).
// inv_period = theta_i / (2*pi) is kept in double so the product with large
// positions keeps its fraction; v_sin/v_cos take revolutions in [0, 1).
__device__ __forceinline__ void rope_cos_sin(double inv_period, int pos, float& c, float& s) {
    double r = (double)pos * inv_period;
    r = r - floor(r);
    float rf = (float)r;
    c = __builtin_amdgcn_cosf(rf);
    s = __builtin_amdgcn_sinf(rf);
}

}  // namespace rf
