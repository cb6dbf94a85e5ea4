// Adapter merge: fold a trained LoRA adapter into its frozen NF4 base,
//   W_merged = W' + s * B A,   W' = fl32(c[code] * absmax)  (the GEMM's
// dequantized value before its bf16 rounding), s = alpha / r,
// rounded once to bf16 (the pages' `soup merge`, guillermodelpino.com article,
// command list; imasters article, closing section). The NF4 output
// re-quantizes that bf16 matrix with the ordinary quantizer.
//
// Tile: 32 rows x 256 columns per workgroup; A [r, 256] and B [32, r] staged in
// LDS 64 columns of r at a time; each thread owns one column and accumulates
// the 32 dot products over r in ascending order, fp32.
#include "nf4_codes.h"
#include "qlx_internal.h"

namespace qlx {

namespace {
constexpr int MR = 32, MC = 256, RK = 64;

__global__ __launch_bounds__(256) void k_lora_merge(const uint8_t* __restrict__ packed, const float* __restrict__ absmax,
                                                    int64_t rows, int64_t cols, const float* __restrict__ A,
                                                    const float* __restrict__ B, int r, float scale,
                                                    uint16_t* __restrict__ out) {
    __shared__ float As[RK][MC];
    __shared__ float Bs[MR][RK + 1];
    const int64_t r0 = int64_t(blockIdx.y) * MR, c0 = int64_t(blockIdx.x) * MC;
    const int tid = threadIdx.x;
    const int64_t col = c0 + tid;
    float acc[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < r; k0 += RK) {
        const int kn = min(RK, r - k0);
        for (int k = 0; k < kn; ++k) As[k][tid] = (col < cols) ? A[int64_t(k0 + k) * cols + col] : 0.f;
        for (int e = tid; e < MR * RK; e += 256) {
            const int i = e / RK, k = e % RK;
            Bs[i][k] = (r0 + i < rows && k < kn) ? B[(r0 + i) * r + k0 + k] : 0.f;
        }
        __syncthreads();
        for (int k = 0; k < kn; ++k) {
            const float a = As[k][tid];
#pragma unroll
            for (int i = 0; i < MR; ++i) acc[i] = fmaf(Bs[i][k], a, acc[i]);
        }
        __syncthreads();
    }
    if (col >= cols) return;
#pragma unroll
    for (int i = 0; i < MR; ++i) {
        const int64_t row = r0 + i;
        if (row >= rows) break;
        const int64_t flat = row * cols + col;
        const uint32_t byte = packed[flat >> 1];
        const int code = (flat & 1) ? int(byte & 15) : int(byte >> 4);
        const float w = nf4_value(code) * absmax[flat >> 6];
        out[flat] = f32_to_bf16_bits(w + scale * acc[i]);
    }
}
}  // namespace

void launch_lora_merge(const uint8_t* packed, const float* absmax, int64_t rows, int64_t cols, const float* A,
                       const float* B, int r, float scale, uint16_t* out, hipStream_t s) {
    if (rows == 0 || cols == 0) return;
    QLX_REQUIRE((rows + MR - 1) / MR <= 65535, QLX_EUNSUPPORTED, "merge: too many rows");
    const double n = double(rows) * cols;
    ProfScope prof("lora_merge", 2.0 * n * r, n * (0.5 + 4.0 / 64 + 2) + 4.0 * r * (rows + cols), s);
    hipLaunchKernelGGL(k_lora_merge, dim3(unsigned((cols + MC - 1) / MC), unsigned((rows + MR - 1) / MR)), dim3(256), 0,
                       s, packed, absmax, rows, cols, A, B, r, scale, out);
    check_launch("lora_merge");
}

}  // namespace qlx
