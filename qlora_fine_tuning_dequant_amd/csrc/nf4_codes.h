// The 16 NF4 code values (QLoRA's 4-bit NormalFloat, ascending), as float32
// bit patterns. QLoRA (Dettmers et al., 2023) builds them from evenly spaced
// normal quantiles and prints them in its NF4 appendix; these are those
// values.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qlx {
__device__ __constant__ static const uint32_t kNf4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24du, 0xbe3d353fu,
    0xbdba7871u, 0x00000000u, 0x3da2faffu, 0x3e24cae3u, 0x3e7c04ddu, 0x3ead033au,
    0x3ee1a4b8u, 0x3f1007abu, 0x3f3913b3u, 0x3f800000u};

__device__ inline float nf4_value(int code) { return __builtin_bit_cast(float, kNf4Bits[code]); }

__device__ inline uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ inline uint16_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
// Two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ inline uint32_t f32x2_to_bf16x2(float lo, float hi) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, b2_t));
}
// Two floats -> packed fp16 pair (lo in bits 0..15), round to nearest even.
__device__ inline uint32_t f32x2_to_f16x2(float lo, float hi) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, h2_t));
}
__device__ inline float bf16_bits_to_f32(uint16_t b) { return __builtin_bit_cast(float, uint32_t(b) << 16); }
__device__ inline float f16_bits_to_f32(uint16_t b) { return float(__builtin_bit_cast(_Float16, b)); }
// A 16-bit activation (bf16 or fp16 bits, by the format flag) <-> fp32.
__device__ inline float act_to_f32(uint16_t b, bool f16) { return f16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b); }
__device__ inline uint16_t f32_to_act(float f, bool f16) { return f16 ? f32_to_f16_bits(f) : f32_to_bf16_bits(f); }
__device__ inline uint32_t f32x2_to_act2(float lo, float hi, bool f16) {
    return f16 ? f32x2_to_f16x2(lo, hi) : f32x2_to_bf16x2(lo, hi);
}
}  // namespace qlx
