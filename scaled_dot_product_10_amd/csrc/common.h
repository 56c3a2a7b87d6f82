// Device-side helpers shared by libattn's kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // MFMA bf16 operand (8 values per lane)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;   // 32x32 MFMA accumulator (16 per lane)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Two floats -> two bfloat16 in one dword (hardware round-to-nearest-even convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// acc + lo + hi of two bf16 packed in one dword (v_dot2_f32_bf16 against 1.0, 1.0;
// the products are exact).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// 2^x on the transcendental unit; exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_mfma_f32_32x32x16_bf16: acc[32x32] += A[32x16] * B[16x32].
// Lane l supplies A row (l % 32), B column (l % 32), with k-slots 8*(l/32)..+7
// taken from its 8-value operand.  Result: lane l holds column (l % 32) and
// rows 8*(r/4) + 4*(l/32) + (r%4) for accumulator register r = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& x) { return __builtin_bit_cast(bf16x8, x); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Two ds_read_b64_tr_b16 (LDS, bf16 transposed): within each 16-lane group,
// lane j addresses 4 consecutive bf16 of one row (4 rows x 16 columns per
// group) and receives one column of those 4 rows.  p0 gives k-slots 0-3 of
// an MFMA operand, p1 k-slots 4-7.
__device__ __forceinline__ bf16x8 tr_read_pair(const void* p0, const void* p1) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
    const short __attribute__((ext_vector_type(8))) x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, x);
}

// Workgroups are dealt round-robin over the chip's 8 XCDs (each with its own
// L2).  Map the hardware id so that a contiguous range of logical ids runs
// on one XCD: logical neighbours (tiles of one head) then share that L2.
// Bijective on [0, total); ids past the last multiple of 8 map to themselves.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t w, uint32_t total) {
    const uint32_t per = total / 8u;
    if (w >= per * 8u) return w;
    return (w % 8u) * per + w / 8u;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

}  // namespace attn
