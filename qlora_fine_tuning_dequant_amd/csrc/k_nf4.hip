// NF4 blockwise quantize / dequantize (QLoRA's 4-bit NormalFloat, blocksize
// 64, fp32 absmax). The pages name NF4 as the frozen base's format (rug.gal
// article, "En detalle"; imasters article, "Como cabe um 8B em 4 GB").
//
// quantize: each thread owns 8 consecutive elements (one 16-B load), 8 lanes
// one 64-element block. absmax is the max of |w| over the block (in-thread,
// then 3 lane-xor steps); x = w / absmax with IEEE fp32 division; the code is
// the number of midpoints m_i = (c_i + c_{i+1})/2 below x, found by a 4-step
// binary search over the midpoints held in registers (selects, no memory);
// 2 elements per byte, even element in the high nibble, one 4-B store per
// thread. Memory-bound in principle: 2 B read + 0.5625 B written per element.
// dequant: each thread turns 4 packed bytes (8 codes, one absmax block) into 8
// outputs, coalesced.
#include "nf4_codes.h"
#include "qlx_internal.h"

namespace qlx {

namespace {
// The 15 midpoints m_i = (c_i + c_{i+1})/2, held in registers. Selects go
// through sel(), which takes values: a conditional expression on two lvalues
// is itself an lvalue, and would be compiled as a load from a selected address
// (the midpoints then live in private memory).
struct Mids {
    float m0, m1, m2, m3, m4, m5, m6, m7, m8, m9, m10, m11, m12, m13, m14;
};
__device__ inline float mid(int i) { return (nf4_value(i) + nf4_value(i + 1)) * 0.5f; }
__device__ inline float sel(bool c, float a, float b) { return c ? a : b; }

// number of the sorted midpoints strictly below x: binary search with each
// step's pivot picked by selects
__device__ inline int nf4_code(float x, const Mids& m) {
    const bool t8 = x > m.m7;
    const bool t4 = x > sel(t8, m.m11, m.m3);
    const bool t2 = x > sel(t8, sel(t4, m.m13, m.m9), sel(t4, m.m5, m.m1));
    const float p1 = sel(t8, sel(t4, sel(t2, m.m14, m.m12), sel(t2, m.m10, m.m8)),
                         sel(t4, sel(t2, m.m6, m.m4), sel(t2, m.m2, m.m0)));
    const bool t1 = x > p1;
    return (t8 ? 8 : 0) + (t4 ? 4 : 0) + (t2 ? 2 : 0) + (t1 ? 1 : 0);
}
}  // namespace

template <bool VEC>
__global__ __launch_bounds__(256) void k_nf4_quantize(const uint16_t* __restrict__ w, int64_t n,
                                                      uint8_t* __restrict__ packed, float* __restrict__ absmax) {
    const Mids m = {mid(0), mid(1), mid(2),  mid(3),  mid(4),  mid(5),  mid(6), mid(7),
                    mid(8), mid(9), mid(10), mid(11), mid(12), mid(13), mid(14)};
    const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;  // 8-element group
    const int64_t i0 = g * 8, blk = g >> 3;
    const int64_t nblk = (n + 63) >> 6;
    if (blk >= nblk) return;  // all 8 lanes of a block leave together
    float v[8];
    const bool fast = VEC && i0 + 8 <= n;  // whole group: straight-line path
    if (fast) {
        const uint4 q = *reinterpret_cast<const uint4*>(w + i0);
        const uint32_t words[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            v[2 * b] = __builtin_bit_cast(float, words[b] << 16);
            v[2 * b + 1] = __builtin_bit_cast(float, words[b] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (i0 + e < n) ? bf16_bits_to_f32(w[i0 + e]) : 0.f;
    }
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    // a == 0 only when every element is +-0: dividing by 1 then gives x = +-0
    const float den = (a > 0.f) ? a : 1.f;
    int code[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e] = nf4_code(__fdiv_rn(v[e], den), m);
    if (fast) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) word |= uint32_t((code[2 * b] << 4) | code[2 * b + 1]) << (8 * b);
        *reinterpret_cast<uint32_t*>(packed + (i0 >> 1)) = word;
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (i0 + 2 * b < n)
                packed[(i0 >> 1) + b] = uint8_t((code[2 * b] << 4) | (i0 + 2 * b + 1 < n ? code[2 * b + 1] : 7));
    }
    if ((g & 7) == 0) absmax[blk] = a;
}

template <int OUT_BF16>
__global__ __launch_bounds__(256) void k_nf4_dequant(const uint8_t* __restrict__ packed,
                                                     const float* __restrict__ absmax, int64_t n,
                                                     void* __restrict__ out) {
    const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // group of 8 elements
    const int64_t i0 = g * 8;
    if (i0 >= n) return;
    const float a = absmax[i0 >> 6];
    if (i0 + 8 <= n) {
        const uint32_t word = *reinterpret_cast<const uint32_t*>(packed + (i0 >> 1));
        float v[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (word >> (8 * b)) & 0xFF;
            v[2 * b] = nf4_value(byte >> 4) * a;
            v[2 * b + 1] = nf4_value(byte & 15) * a;
        }
        if (OUT_BF16) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + i0) =
                make_uint4(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]), f32x2_to_bf16x2(v[4], v[5]),
                           f32x2_to_bf16x2(v[6], v[7]));
        } else {
            float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + i0);
            o[0] = make_float4(v[0], v[1], v[2], v[3]);
            o[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    } else {
        for (int64_t i = i0; i < n; ++i) {
            const uint32_t byte = packed[i >> 1];
            const int code = (i & 1) ? (byte & 15) : (byte >> 4);
            const float v = nf4_value(code) * a;
            if (OUT_BF16) static_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(v);
            else static_cast<float*>(out)[i] = v;
        }
    }
}

void launch_nf4_quantize(const uint16_t* w, int64_t n, uint8_t* packed, float* absmax, hipStream_t s) {
    if (n <= 0) return;
    const int64_t groups = (n + 63) / 64 * 8;  // whole blocks, so every lane of a block is launched
    const int64_t grid = (groups + 255) / 256;
    ProfScope prof("nf4_quantize", 8.0 * n, n * (2.0 + 0.5 + 4.0 / 64), s);
    // VEC: 16-B loads of w and 4-B stores of codes for whole 8-element groups
    if (reinterpret_cast<uintptr_t>(w) % 16 == 0 && reinterpret_cast<uintptr_t>(packed) % 4 == 0)
        hipLaunchKernelGGL(k_nf4_quantize<true>, dim3(unsigned(grid)), dim3(256), 0, s, w, n, packed, absmax);
    else
        hipLaunchKernelGGL(k_nf4_quantize<false>, dim3(unsigned(grid)), dim3(256), 0, s, w, n, packed, absmax);
    check_launch("nf4_quantize");
}

void launch_nf4_dequant(const uint8_t* packed, const float* absmax, int64_t n, int out_dtype, void* out,
                        hipStream_t s) {
    if (n <= 0) return;
    const int64_t groups = (n + 7) / 8;
    const int64_t grid = (groups + 255) / 256;
    ProfScope prof("nf4_dequant", double(n), n * (0.5 + 4.0 / 64 + (out_dtype == QLX_BF16 ? 2 : 4)), s);
    if (out_dtype == QLX_BF16)
        hipLaunchKernelGGL(k_nf4_dequant<1>, dim3(unsigned(grid)), dim3(256), 0, s, packed, absmax, n, out);
    else
        hipLaunchKernelGGL(k_nf4_dequant<0>, dim3(unsigned(grid)), dim3(256), 0, s, packed, absmax, n, out);
    check_launch("nf4_dequant");
}

}  // namespace qlx
