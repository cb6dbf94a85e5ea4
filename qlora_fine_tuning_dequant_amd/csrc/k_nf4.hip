// NF4 blockwise quantize / dequantize (QLoRA's 4-bit NormalFloat, blocksize
// 64, fp32 absmax). The pages name NF4 as the frozen base's format (rug.gal
// article, "En detalle"; imasters article, "Como cabe um 8B em 4 GB").
//
// quantize: one wavefront per 64-element block. Lane l owns element l of the
// block: absmax is a wavefront max-reduction of |w|; x = w / absmax with IEEE
// fp32 division; the code is the number of midpoints m_i = (c_i + c_{i+1})/2
// below x (a 4-step binary search); lanes 2j and 2j+1 meet in a byte, even
// element in the high nibble. Memory-bound: 2 B read + 0.5625 B written per
// element.
// dequant: each thread turns 4 packed bytes (8 codes, one absmax block) into 8
// outputs, coalesced.
#include "nf4_codes.h"
#include "qlx_internal.h"

namespace qlx {

__global__ __launch_bounds__(256) void k_nf4_quantize(const uint16_t* __restrict__ w, int64_t n,
                                                      uint8_t* __restrict__ packed, float* __restrict__ absmax) {
    __shared__ float mid[15];
    if (threadIdx.x < 15) mid[threadIdx.x] = (nf4_value(threadIdx.x) + nf4_value(threadIdx.x + 1)) * 0.5f;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t blk = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t nblk = (n + 63) >> 6;
    if (blk >= nblk) return;  // whole wavefront leaves together
    const int64_t i = blk * 64 + lane;
    const bool valid = i < n;
    const float v = valid ? bf16_bits_to_f32(w[i]) : 0.f;
    float a = fabsf(v);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    int code = 7;
    if (valid) {
        const float x = (a > 0.f) ? __fdiv_rn(v, a) : 0.f;
        int c = 0;
#pragma unroll
        for (int step = 8; step > 0; step >>= 1)
            if (x > mid[c + step - 1]) c += step;
        code = c;
    }
    const int partner = __shfl_down(code, 1, 64);
    if ((lane & 1) == 0 && i < n) packed[i >> 1] = uint8_t((code << 4) | partner);
    if (lane == 0) absmax[blk] = a;
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
    const int64_t nblk = (n + 63) / 64;
    const int64_t grid = (nblk + 3) / 4;
    ProfScope prof("nf4_quantize", 8.0 * n, n * (2.0 + 0.5 + 4.0 / 64), s);
    hipLaunchKernelGGL(k_nf4_quantize, dim3(unsigned(grid)), dim3(256), 0, s, w, n, packed, absmax);
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
