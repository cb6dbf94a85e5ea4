// Adapter merge: fold a trained LoRA adapter into its frozen NF4 base,
//   W_merged = W' + s * B A,   W' = fl32(c[code] * absmax)  (the GEMM's
// dequantized value before its bf16 rounding), s = alpha / r,
// rounded once to bf16 (the pages' `soup merge`, guillermodelpino.com article,
// command list; imasters article, closing section). The NF4 output
// re-quantizes that bf16 matrix with the ordinary quantizer.
//
// Tile: 32 rows x 256 columns per workgroup of 4 wavefronts; A [r, 256] and
// B [32, r] (transposed) staged in LDS 32 values of r at a time, every global
// load of a stage issued before its LDS stores. Wavefront w owns rows
// 8w..8w+7, lane l columns 4l..4l+3: per step of r one 16-B read of A and two
// broadcast 16-B reads of B feed 32 fp32 FMAs. Each output element is one fp32
// FMA chain over r in ascending order. VEC (cols % 4 == 0 and A 16-B aligned)
// moves A, the codes and the output 4 columns at a time.
#include "nf4_codes.h"
#include "qlx_internal.h"

namespace qlx {

namespace {
constexpr int MR = 32, MC = 256, RK = 32, TR = 8, TC = 4, BPAD = MR + 4;
constexpr int A_LOADS = RK * MC / 4 / 256, B_LOADS = RK * MR / 256;

template <bool VEC>
__global__ __launch_bounds__(256) void k_lora_merge(const uint8_t* __restrict__ packed, const float* __restrict__ absmax,
                                                    int64_t rows, int64_t cols, const float* __restrict__ A,
                                                    const float* __restrict__ B, int r, float scale,
                                                    uint16_t* __restrict__ out) {
    __shared__ __align__(16) float As[RK][MC];
    __shared__ __align__(16) float Bs[RK][BPAD];
    const int64_t r0 = int64_t(blockIdx.y) * MR, c0 = int64_t(blockIdx.x) * MC;
    const int tid = threadIdx.x, ty = tid >> 6, tx = tid & 63;
    float acc[TR][TC];
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
        for (int j = 0; j < TC; ++j) acc[i][j] = 0.f;
    for (int k0 = 0; k0 < r; k0 += RK) {
        const int kn = min(RK, r - k0);
        // A: 16-B unit u covers row u / 64, columns 4 (u % 64) .. +3 of the tile
        float4 av[A_LOADS];
#pragma unroll
        for (int it = 0; it < A_LOADS; ++it) {
            const int u = it * 256 + tid, k = u >> 6, c = (u & 63) * 4;
            const int64_t col = c0 + c;
            const float* src = A + int64_t(k0 + k) * cols + col;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < kn) {
                if (VEC) {
                    if (col < cols) v = *reinterpret_cast<const float4*>(src);
                } else {
                    if (col < cols) v.x = src[0];
                    if (col + 1 < cols) v.y = src[1];
                    if (col + 2 < cols) v.z = src[2];
                    if (col + 3 < cols) v.w = src[3];
                }
            }
            av[it] = v;
        }
        float bv[B_LOADS];
#pragma unroll
        for (int it = 0; it < B_LOADS; ++it) {
            const int e = it * 256 + tid, i = e / RK, k = e % RK;
            bv[it] = (r0 + i < rows && k < kn) ? B[(r0 + i) * r + k0 + k] : 0.f;
        }
#pragma unroll
        for (int it = 0; it < A_LOADS; ++it) {
            const int u = it * 256 + tid;
            *reinterpret_cast<float4*>(&As[u >> 6][(u & 63) * 4]) = av[it];
        }
#pragma unroll
        for (int it = 0; it < B_LOADS; ++it) {
            const int e = it * 256 + tid;
            Bs[e % RK][e / RK] = bv[it];
        }
        __syncthreads();
        // zero-filled rows beyond kn are skipped, not added: the chain over r
        // stays exactly r FMAs long
#pragma unroll 8
        for (int k = 0; k < kn; ++k) {
            const float4 a = *reinterpret_cast<const float4*>(&As[k][tx * TC]);
            const float4 b0 = *reinterpret_cast<const float4*>(&Bs[k][ty * TR]);
            const float4 b1 = *reinterpret_cast<const float4*>(&Bs[k][ty * TR + 4]);
            const float a_[TC] = {a.x, a.y, a.z, a.w};
            const float b_[TR] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < TR; ++i)
#pragma unroll
                for (int j = 0; j < TC; ++j) acc[i][j] = fmaf(b_[i], a_[j], acc[i][j]);
        }
        __syncthreads();
    }
    const int64_t col0 = c0 + tx * TC;
#pragma unroll
    for (int i = 0; i < TR; ++i) {
        const int64_t row = r0 + ty * TR + i;
        if (row >= rows || col0 >= cols) break;
        const int64_t flat = row * cols + col0;
        if (VEC) {
            // 4 columns from a multiple of 4: two code bytes, one absmax block
            const uint32_t b2 = *reinterpret_cast<const uint16_t*>(packed + (flat >> 1));
            const float am = absmax[flat >> 6];
            const int codes[TC] = {int((b2 >> 4) & 15), int(b2 & 15), int(b2 >> 12), int((b2 >> 8) & 15)};
            uint16_t o[TC];
#pragma unroll
            for (int j = 0; j < TC; ++j) o[j] = f32_to_bf16_bits(nf4_value(codes[j]) * am + scale * acc[i][j]);
            *reinterpret_cast<uint2*>(out + flat) =
                make_uint2(uint32_t(o[0]) | (uint32_t(o[1]) << 16), uint32_t(o[2]) | (uint32_t(o[3]) << 16));
        } else {
#pragma unroll
            for (int j = 0; j < TC; ++j) {
                if (col0 + j >= cols) break;
                const int64_t f = flat + j;
                const uint32_t byte = packed[f >> 1];
                const int code = (f & 1) ? int(byte & 15) : int(byte >> 4);
                out[f] = f32_to_bf16_bits(nf4_value(code) * absmax[f >> 6] + scale * acc[i][j]);
            }
        }
    }
}
}  // namespace

void launch_lora_merge(const uint8_t* packed, const float* absmax, int64_t rows, int64_t cols, const float* A,
                       const float* B, int r, float scale, uint16_t* out, hipStream_t s) {
    if (rows == 0 || cols == 0) return;
    QLX_REQUIRE((rows + MR - 1) / MR <= 65535, QLX_EUNSUPPORTED, "merge: too many rows");
    const double n = double(rows) * cols;
    ProfScope prof("lora_merge", 2.0 * n * r, n * (0.5 + 4.0 / 64 + 2) + 4.0 * r * (rows + cols), s);
    const dim3 grid(unsigned((cols + MC - 1) / MC), unsigned((rows + MR - 1) / MR));
    // VEC: 16-B loads of A rows, 2-B code loads and 8-B stores at multiples of 4 columns
    const bool vec = cols % 4 == 0 && reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(out) % 8 == 0 && reinterpret_cast<uintptr_t>(packed) % 2 == 0;
    if (vec)
        hipLaunchKernelGGL(k_lora_merge<true>, grid, dim3(256), 0, s, packed, absmax, rows, cols, A, B, r, scale, out);
    else
        hipLaunchKernelGGL(k_lora_merge<false>, grid, dim3(256), 0, s, packed, absmax, rows, cols, A, B, r, scale, out);
    check_launch("lora_merge");
}

}  // namespace qlx
