// Measured peaks of the device, for the roofline figures: a bf16 MFMA loop
// (v_mfma_f32_16x16x32_bf16 on register operands, eight independent
// accumulator chains per wavefront so the matrix core never waits on a
// result) and an HBM copy (16-byte loads and stores, grid-stride).
#include <algorithm>

#include "nf4_codes.h"
#include "qlx_internal.h"

namespace qlx {
namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_peak_mfma(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = __bf16(float((lane + e) & 7) * 0.125f);
        b[e] = __bf16(float((lane * 3 + e) & 7) * 0.0625f);
    }
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    out[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;  // keeps the loop alive
}

// The same loop on the 32x32x16 shape (32768 flops per instruction, 16
// accumulators a lane per chain).
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void k_peak_mfma32(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = __bf16(float((lane + e) & 7) * 0.125f);
        b[e] = __bf16(float((lane * 3 + e) & 7) * 0.0625f);
    }
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    out[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_peak_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}
}  // namespace
}  // namespace qlx

using namespace qlx;

extern "C" {

int qlx_peak_mfma(int64_t iters, int workgroups, int shape, float* out, void* stream) {
    return guarded([&] {
        REQ_PTR(out, "out");
        QLX_REQUIRE(iters > 0 && workgroups > 0 && workgroups <= 1 << 20 && (shape == 0 || shape == 1), QLX_EINVAL,
                    "peak_mfma: iters > 0, 0 < workgroups <= 2^20, shape 0 or 1");
        if (shape == 0)
            hipLaunchKernelGGL(k_peak_mfma, dim3(unsigned(workgroups)), dim3(256), 0, static_cast<hipStream_t>(stream),
                               iters, out);
        else
            hipLaunchKernelGGL(k_peak_mfma32, dim3(unsigned(workgroups)), dim3(256), 0,
                               static_cast<hipStream_t>(stream), iters, out);
        check_launch("peak_mfma");
    });
}

int qlx_peak_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
    return guarded([&] {
        REQ_PTR(src, "src");
        REQ_PTR(dst, "dst");
        QLX_REQUIRE(bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                        (reinterpret_cast<uintptr_t>(dst) & 15) == 0,
                    QLX_EINVAL, "peak_copy: 16-byte aligned buffers and a multiple of 16 bytes");
        const int64_t n = int64_t(bytes / 16);
        if (n == 0) return;
        hipLaunchKernelGGL(k_peak_copy, dim3(unsigned(std::min<int64_t>((n + 255) / 256, 1 << 16))), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), static_cast<uint4*>(dst),
                           n);
        check_launch("peak_copy");
    });
}

}  // extern "C"
