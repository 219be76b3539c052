// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, wave64 reductions, MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace lmoe {

// Calls f(std::integral_constant<int, i>) for i = 0..N-1.  Unlike an unrolled
// loop it can never be left rolled, so register arrays indexed by i stay in
// registers whatever the body's size.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector: unlike the HIP uint4 struct it stays in
// registers when kept in small private arrays.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 (the same result as f32_to_bf16_rne for finite
// inputs; a NaN stays a NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// 32x32x16 bf16 MFMA, fp32 accumulate: acc += A(32x16) * B(16x32).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each as 8
// consecutive k values starting at 8 * (l / 32).
__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b, f32x16_t acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// 32x32x64 fp8 (E4M3 x E4M3) MFMA, fp32 accumulate: acc += A(32x64) * B(64x32).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, 32 codes each.
// The unscaled product only needs a lane's A and B codes to cover the same
// k; the hardware's own K order (measured on the device with block scales)
// is k 16 (l/32) + [0, 16) in the first four registers and 32 + 16 (l/32)
// + [0, 16) in the last four.  The block-scale operands are unused here (0
// selects the unscaled form).
typedef int i32x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16_t mfma32x32x64_fp8(const i32x8_t& a, const i32x8_t& b, f32x16_t acc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}

// The same MFMA with MX block scales (OCP microscaling, E8M0: 2^(s - 127)):
// lane l passes the scale byte of the 32-element K block it holds, for its
// A row in sa and for its B column in sb, in byte OPSEL of the register
// (checked on the device with runtime scales, 127 being 1).
template <int OPSEL>
__device__ __forceinline__ f32x16_t mfma32x32x64_mxfp8(const i32x8_t& a, const i32x8_t& b, f32x16_t acc, int sa,
                                                       int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, OPSEL, sa, OPSEL, sb);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        T w = __shfl_xor(v, o, kWave);
        v = v > w ? v : w;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace lmoe
