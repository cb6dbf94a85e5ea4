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
__device__ inline float bf16_bits_to_f32(uint16_t b) { return __builtin_bit_cast(float, uint32_t(b) << 16); }
__device__ inline float f16_bits_to_f32(uint16_t b) { return float(__builtin_bit_cast(_Float16, b)); }
}  // namespace qlx
