// Memory-bound kernels of the decoder layer and the loss: RMSNorm fwd/bwd,
// rotate-half RoPE, SwiGLU fwd/bwd, embedding gather, LoRA operand staging,
// causal-softmax fwd/bwd for attention, grouped-query gradient reduction,
// cross-entropy statistics and gradients, SFT and DPO loss reductions.
//
// The layer is the Llama decoder the pages fine-tune (Llama-3.1-8B-Instruct:
// rug.gal article intro; guillermodelpino.com article, "Qué es exactamente").
// Every reduction runs in a fixed order (per-thread strided partial sums,
// xor-shuffle wavefront trees, then the waves in index order), so results
// never depend on scheduling.
#include <algorithm>
#include <cmath>

#include "nf4_codes.h"
#include "partials.h"
#include "qlx_internal.h"

namespace qlx {

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
// Block-wide sum over 256 threads in a fixed order; every thread gets the result.
__device__ inline float block_sum256(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ inline float block_max256(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ------------------------------------------------------------------ RMSNorm
// y = x * rstd * g, rstd = 1 / sqrt(mean(x^2) + eps). One workgroup per row.
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const float* __restrict__ x, const float* __restrict__ g, int H,
                                                     float eps, void* __restrict__ out, int out_f16,
                                                     float* __restrict__ rstd) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * H;
    float ss = 0.f;
    for (int j = threadIdx.x; j < H; j += 256) ss += xr[j] * xr[j];
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / float(H) + eps);
    if (threadIdx.x == 0 && rstd) rstd[row] = r;
    uint16_t* o = static_cast<uint16_t*>(out) + row * H;
    for (int j = threadIdx.x; j < H; j += 256) {
        const float y = xr[j] * r * g[j];
        o[j] = out_f16 ? f32_to_f16_bits(y) : f32_to_bf16_bits(y);
    }
}

// dx = dres + rstd * (dy*g - xhat * mean(dy*g*xhat)), xhat = x*rstd (g frozen).
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const float* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ g, const float* __restrict__ rstd,
                                                     const float* __restrict__ dres, int H, float* __restrict__ dx) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float* dyr = dy + row * H;
    const float* xr = x + row * H;
    const float r = rstd[row];
    float dot = 0.f;
    for (int j = threadIdx.x; j < H; j += 256) dot += (dyr[j] * g[j]) * (xr[j] * r);
    dot = block_sum256(dot, red) / float(H);
    for (int j = threadIdx.x; j < H; j += 256) {
        const float xhat = xr[j] * r;
        float v = r * (dyr[j] * g[j] - xhat * dot);
        if (dres) v += dres[row * H + j];
        dx[row * H + j] = v;
    }
}

// Row kept in registers (NV float4 per thread, H = 1024 NV): one HBM read
// of x, 16-byte loads and 8-byte stores. Same formulas as above.
template <int NV>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd_v(const float* __restrict__ x, const float* __restrict__ g, int H,
                                                       float eps, void* __restrict__ out, int out_f16,
                                                       float* __restrict__ rstd) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float4* xr = reinterpret_cast<const float4*>(x + row * H);
    const float4* gr = reinterpret_cast<const float4*>(g);
    float4 v[NV];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        v[k] = xr[threadIdx.x + 256 * k];
        ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / float(H) + eps);
    if (threadIdx.x == 0 && rstd) rstd[row] = r;
    uint2* o = reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * H);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const float4 gg = gr[threadIdx.x + 256 * k];
        const float y0 = v[k].x * r * gg.x, y1 = v[k].y * r * gg.y, y2 = v[k].z * r * gg.z, y3 = v[k].w * r * gg.w;
        o[threadIdx.x + 256 * k] =
            out_f16 ? make_uint2(uint32_t(f32_to_f16_bits(y0)) | (uint32_t(f32_to_f16_bits(y1)) << 16),
                                 uint32_t(f32_to_f16_bits(y2)) | (uint32_t(f32_to_f16_bits(y3)) << 16))
                    : make_uint2(f32x2_to_bf16x2(y0, y1), f32x2_to_bf16x2(y2, y3));
    }
}
// out16 (optional): also writes 16-bit(dx * sc), 8-byte stores
__device__ inline void store_act4(uint16_t* out16, int64_t i, const float4& v, float sc, int f16) {
    *reinterpret_cast<uint2*>(out16 + i) =
        make_uint2(f32x2_to_act2(v.x * sc, v.y * sc, f16), f32x2_to_act2(v.z * sc, v.w * sc, f16));
}
template <int NV>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd_v(const float* __restrict__ dy, const float* __restrict__ x,
                                                       const float* __restrict__ g, const float* __restrict__ rstd,
                                                       const float* __restrict__ dres, int H, float* __restrict__ dx,
                                                       uint16_t* __restrict__ out16, float sc, int f16) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float4* dyr = reinterpret_cast<const float4*>(dy + row * H);
    const float4* xr = reinterpret_cast<const float4*>(x + row * H);
    const float4* gr = reinterpret_cast<const float4*>(g);
    const float r = rstd[row];
    float4 a[NV], b[NV];  // dy * g, x * r
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const float4 d = dyr[threadIdx.x + 256 * k], xx = xr[threadIdx.x + 256 * k], gg = gr[threadIdx.x + 256 * k];
        a[k] = make_float4(d.x * gg.x, d.y * gg.y, d.z * gg.z, d.w * gg.w);
        b[k] = make_float4(xx.x * r, xx.y * r, xx.z * r, xx.w * r);
        dot += a[k].x * b[k].x + a[k].y * b[k].y + a[k].z * b[k].z + a[k].w * b[k].w;
    }
    dot = block_sum256(dot, red) / float(H);
    float4* o = reinterpret_cast<float4*>(dx + row * H);
    const float4* dr = dres ? reinterpret_cast<const float4*>(dres + row * H) : nullptr;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        float4 v = make_float4(r * (a[k].x - b[k].x * dot), r * (a[k].y - b[k].y * dot), r * (a[k].z - b[k].z * dot),
                               r * (a[k].w - b[k].w * dot));
        if (dr) {
            const float4 q = dr[threadIdx.x + 256 * k];
            v.x += q.x;
            v.y += q.y;
            v.z += q.z;
            v.w += q.w;
        }
        o[threadIdx.x + 256 * k] = v;
        if (out16) store_act4(out16, row * H + 4 * (threadIdx.x + 256 * k), v, sc, f16);
    }
}
// The vector kernels above with the input row summed from split-K partials
// (the GEMM's reduce pass fused in): forward writes the summed row to xout
// (fp32) too.
template <int NV>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd_p(const Partials q, float* __restrict__ xout,
                                                       const float* __restrict__ g, int H, float eps,
                                                       void* __restrict__ out, int out_f16, float* __restrict__ rstd) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float4* gr = reinterpret_cast<const float4*>(g);
    float4* xo = reinterpret_cast<float4*>(xout + row * H);
    float4 v[NV];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int64_t c = 4 * (threadIdx.x + 256 * k);
        v[k] = part_sum4(q, row * H + c, row * q.ldr + c);
        xo[threadIdx.x + 256 * k] = v[k];
        ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / float(H) + eps);
    if (threadIdx.x == 0 && rstd) rstd[row] = r;
    uint2* o = reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * H);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const float4 gg = gr[threadIdx.x + 256 * k];
        const float y0 = v[k].x * r * gg.x, y1 = v[k].y * r * gg.y, y2 = v[k].z * r * gg.z, y3 = v[k].w * r * gg.w;
        o[threadIdx.x + 256 * k] = make_uint2(f32x2_to_act2(y0, y1, out_f16), f32x2_to_act2(y2, y3, out_f16));
    }
}
template <int NV>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd_p(const Partials q, const float* __restrict__ x,
                                                       const float* __restrict__ g, const float* __restrict__ rstd,
                                                       const float* __restrict__ dres, int H, float* __restrict__ dx,
                                                       uint16_t* __restrict__ out16, float sc, int f16) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float4* xr = reinterpret_cast<const float4*>(x + row * H);
    const float4* gr = reinterpret_cast<const float4*>(g);
    const float r = rstd[row];
    float4 a[NV], b[NV];  // dy * g, x * r
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const float4 d = part_sum4(q, row * H + 4 * (threadIdx.x + 256 * k), 0);
        const float4 xx = xr[threadIdx.x + 256 * k], gg = gr[threadIdx.x + 256 * k];
        a[k] = make_float4(d.x * gg.x, d.y * gg.y, d.z * gg.z, d.w * gg.w);
        b[k] = make_float4(xx.x * r, xx.y * r, xx.z * r, xx.w * r);
        dot += a[k].x * b[k].x + a[k].y * b[k].y + a[k].z * b[k].z + a[k].w * b[k].w;
    }
    dot = block_sum256(dot, red) / float(H);
    float4* o = reinterpret_cast<float4*>(dx + row * H);
    const float4* dr = dres ? reinterpret_cast<const float4*>(dres + row * H) : nullptr;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        float4 v = make_float4(r * (a[k].x - b[k].x * dot), r * (a[k].y - b[k].y * dot), r * (a[k].z - b[k].z * dot),
                               r * (a[k].w - b[k].w * dot));
        if (dr) {
            const float4 q4 = dr[threadIdx.x + 256 * k];
            v.x += q4.x;
            v.y += q4.y;
            v.z += q4.z;
            v.w += q4.w;
        }
        o[threadIdx.x + 256 * k] = v;
        if (out16) store_act4(out16, row * H + 4 * (threadIdx.x + 256 * k), v, sc, f16);
    }
}

static bool rms_vec(int H, const void* a, const void* b, const void* c, const void* d) {
    return H % 1024 == 0 && H <= 4096 && al16(a) && al16(b) && al16(c) && (!d || al16(d));
}

void launch_rmsnorm_fwd(const float* x, const float* g, int T, int H, float eps, void* out, int out_f16, float* rstd,
                        hipStream_t s) {
    if (T <= 0) return;
    ProfScope prof("rmsnorm_fwd", 4.0 * T * H, double(T) * H * (4.0 + (out_f16 ? 2 : 2)) + 4.0 * H, s);
    if (rms_vec(H, x, g, out, nullptr) && (reinterpret_cast<uintptr_t>(out) & 7) == 0) {
        switch (H / 1024) {
            case 1: hipLaunchKernelGGL(k_rmsnorm_fwd_v<1>, dim3(T), dim3(256), 0, s, x, g, H, eps, out, out_f16, rstd); break;
            case 2: hipLaunchKernelGGL(k_rmsnorm_fwd_v<2>, dim3(T), dim3(256), 0, s, x, g, H, eps, out, out_f16, rstd); break;
            case 3: hipLaunchKernelGGL(k_rmsnorm_fwd_v<3>, dim3(T), dim3(256), 0, s, x, g, H, eps, out, out_f16, rstd); break;
            default: hipLaunchKernelGGL(k_rmsnorm_fwd_v<4>, dim3(T), dim3(256), 0, s, x, g, H, eps, out, out_f16, rstd);
        }
    } else {
        hipLaunchKernelGGL(k_rmsnorm_fwd, dim3(T), dim3(256), 0, s, x, g, H, eps, out, out_f16, rstd);
    }
    check_launch("rmsnorm_fwd");
}
void launch_rmsnorm_bwd(const float* dy, const float* x, const float* g, const float* rstd, const float* dres, int T,
                        int H, float* dx, hipStream_t s, uint16_t* out16, float sc, int f16) {
    if (T <= 0) return;
    const bool vec = rms_vec(H, dy, x, g, dres) && al16(dx) && (!out16 || (reinterpret_cast<uintptr_t>(out16) & 7) == 0);
    {
        ProfScope prof("rmsnorm_bwd", 8.0 * T * H, double(T) * H * (12.0 + (dres ? 4 : 0) + (out16 && vec ? 2 : 0)), s);
        uint16_t* o16 = vec ? out16 : nullptr;
        if (vec) {
            switch (H / 1024) {
                case 1: hipLaunchKernelGGL(k_rmsnorm_bwd_v<1>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, o16, sc, f16); break;
                case 2: hipLaunchKernelGGL(k_rmsnorm_bwd_v<2>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, o16, sc, f16); break;
                case 3: hipLaunchKernelGGL(k_rmsnorm_bwd_v<3>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, o16, sc, f16); break;
                default: hipLaunchKernelGGL(k_rmsnorm_bwd_v<4>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, o16, sc, f16);
            }
        } else {
            hipLaunchKernelGGL(k_rmsnorm_bwd, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx);
        }
        check_launch("rmsnorm_bwd");
    }
    if (out16 && !vec) launch_f32_to_act(dx, int64_t(T) * H, out16, f16, sc, s);
}

bool rmsnorm_part_ok(int H) { return H % 1024 == 0 && H >= 1024 && H <= 4096; }
static void check_part(const Partials& q, int64_t mn, const char* what) {
    QLX_REQUIRE(q.p && q.splits >= 1 && q.mn == mn && al16(q.p) && (!q.R || (al16(q.R) && q.ldr % 4 == 0)),
                QLX_EINVAL, std::string(what) + ": bad split-K partials");
}
void launch_rmsnorm_fwd_part(const Partials& x, float* xout, const float* g, int T, int H, float eps, void* out,
                             int out_f16, float* rstd, hipStream_t s) {
    if (T <= 0) return;
    QLX_REQUIRE(rmsnorm_part_ok(H) && al16(xout) && al16(g) && (reinterpret_cast<uintptr_t>(out) & 7) == 0,
                QLX_EINVAL, "rmsnorm_fwd (partials): needs H a multiple of 1024 up to 4096 and aligned rows");
    check_part(x, int64_t(T) * H, "rmsnorm_fwd");
    ProfScope prof("reduce_rmsnorm_fwd", (x.splits + 4.0) * T * H,
                   double(T) * H * (4.0 * x.splits + (x.R ? 4 : 0) + 4 + 2) + 4.0 * H, s);
    switch (H / 1024) {
        case 1: hipLaunchKernelGGL(k_rmsnorm_fwd_p<1>, dim3(T), dim3(256), 0, s, x, xout, g, H, eps, out, out_f16, rstd); break;
        case 2: hipLaunchKernelGGL(k_rmsnorm_fwd_p<2>, dim3(T), dim3(256), 0, s, x, xout, g, H, eps, out, out_f16, rstd); break;
        case 3: hipLaunchKernelGGL(k_rmsnorm_fwd_p<3>, dim3(T), dim3(256), 0, s, x, xout, g, H, eps, out, out_f16, rstd); break;
        default: hipLaunchKernelGGL(k_rmsnorm_fwd_p<4>, dim3(T), dim3(256), 0, s, x, xout, g, H, eps, out, out_f16, rstd);
    }
    check_launch("rmsnorm_fwd (partials)");
}
void launch_rmsnorm_bwd_part(const Partials& dy, const float* x, const float* g, const float* rstd, const float* dres,
                             int T, int H, float* dx, hipStream_t s, uint16_t* out16, float sc, int f16) {
    if (T <= 0) return;
    QLX_REQUIRE(rmsnorm_part_ok(H) && al16(x) && al16(g) && al16(dx) && (!dres || al16(dres)) && !dy.R &&
                    (reinterpret_cast<uintptr_t>(out16) & 7) == 0,
                QLX_EINVAL, "rmsnorm_bwd (partials): needs H a multiple of 1024 up to 4096 and aligned rows");
    check_part(dy, int64_t(T) * H, "rmsnorm_bwd");
    ProfScope prof("reduce_rmsnorm_bwd", (dy.splits + 8.0) * T * H,
                   double(T) * H * (4.0 * dy.splits + 8.0 + (dres ? 4 : 0) + (out16 ? 2 : 0)), s);
    switch (H / 1024) {
        case 1: hipLaunchKernelGGL(k_rmsnorm_bwd_p<1>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, out16, sc, f16); break;
        case 2: hipLaunchKernelGGL(k_rmsnorm_bwd_p<2>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, out16, sc, f16); break;
        case 3: hipLaunchKernelGGL(k_rmsnorm_bwd_p<3>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, out16, sc, f16); break;
        default: hipLaunchKernelGGL(k_rmsnorm_bwd_p<4>, dim3(T), dim3(256), 0, s, dy, x, g, rstd, dres, H, dx, out16, sc, f16);
    }
    check_launch("rmsnorm_bwd (partials)");
}

// 16-bit activations (bf16, or fp16 when f16) x8 <-> fp32 x8 for 16-byte accesses.
__device__ inline void unpack8(const uint4& v, float (&f)[8], bool f16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = act_to_f32(uint16_t(w[k]), f16);
        f[2 * k + 1] = act_to_f32(uint16_t(w[k] >> 16), f16);
    }
}
__device__ inline uint4 pack8(const float (&f)[8], bool f16) {
    return make_uint4(f32x2_to_act2(f[0], f[1], f16), f32x2_to_act2(f[2], f[3], f16), f32x2_to_act2(f[4], f[5], f16),
                      f32x2_to_act2(f[6], f[7], f16));
}

// ------------------------------------------------------------------ RoPE
// Table cs[pos][j] = (cos, sin)(pos * theta^(-2j/hd)), angles in fp64.
__global__ void k_rope_table(int seq, int hd, double theta, float2* cs) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int half = hd / 2;
    if (idx >= seq * half) return;
    const int pos = idx / half, j = idx % half;
    const double inv = pow(theta, -2.0 * double(j) / double(hd));
    const double ang = double(pos) * inv;
    cs[idx] = make_float2(float(cos(ang)), float(sin(ang)));
}

// RoPE, forward rotation of each (j, j + hd/2) pair; one thread per pair.
__global__ void k_rope(uint16_t* __restrict__ buf, int64_t ld, int T, int seq, int col0, int nheads, int hd,
                       const float2* __restrict__ cs, int f16) {
    const int half = hd / 2;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = int64_t(T) * nheads * half;
    if (idx >= total) return;
    const int j = int(idx % half);
    const int h = int((idx / half) % nheads);
    const int t = int(idx / (int64_t(half) * nheads));
    const float2 c = cs[(t % seq) * half + j];
    uint16_t* p = buf + int64_t(t) * ld + col0 + h * hd + j;
    const float x1 = act_to_f32(p[0], f16), x2 = act_to_f32(p[half], f16);
    p[0] = f32_to_act(x1 * c.x - x2 * c.y, f16);
    p[half] = f32_to_act(x2 * c.x + x1 * c.y, f16);
}

// Same rotation, eight consecutive pairs per thread (16-byte loads and
// stores of each half; hd/2 a multiple of 8, rows 16-byte aligned).
__global__ void k_rope8(uint16_t* __restrict__ buf, int64_t ld, int T, int seq, int col0, int nheads, int hd,
                        const float2* __restrict__ cs, int f16) {
    const int half = hd / 2, h8 = half / 8;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = int64_t(T) * nheads * h8;
    if (idx >= total) return;
    const int j = int(idx % h8) * 8;
    const int h = int((idx / h8) % nheads);
    const int t = int(idx / (int64_t(h8) * nheads));
    const float4* c4 = reinterpret_cast<const float4*>(cs + (t % seq) * half + j);
    uint16_t* p = buf + int64_t(t) * ld + col0 + h * hd + j;
    float a[8], b[8], ra[8], rb[8];
    unpack8(*reinterpret_cast<const uint4*>(p), a, f16);
    unpack8(*reinterpret_cast<const uint4*>(p + half), b, f16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 c = c4[k];  // (cos, sin) of pairs 2k and 2k+1
        ra[2 * k] = a[2 * k] * c.x - b[2 * k] * c.y;
        rb[2 * k] = b[2 * k] * c.x + a[2 * k] * c.y;
        ra[2 * k + 1] = a[2 * k + 1] * c.z - b[2 * k + 1] * c.w;
        rb[2 * k + 1] = b[2 * k + 1] * c.z + a[2 * k + 1] * c.w;
    }
    *reinterpret_cast<uint4*>(p) = pack8(ra, f16);
    *reinterpret_cast<uint4*>(p + half) = pack8(rb, f16);
}

// The q|k|v projection's split-K partials summed into the 16-bit buffer,
// heads [0, nrot) rotated as k_rope8 does (eight pairs per thread), heads
// [nrot, nall) copied; rows of nall * hd.
__global__ void k_rope8_part(const Partials q, uint16_t* __restrict__ buf, int T, int seq, int nrot, int nall,
                             int hd, const float2* __restrict__ cs, int f16) {
    const int half = hd / 2, h8 = half / 8;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = int64_t(T) * nall * h8;
    if (idx >= total) return;
    const int j = int(idx % h8) * 8;
    const int h = int((idx / h8) % nall);
    const int t = int(idx / (int64_t(h8) * nall));
    const int64_t i0 = int64_t(t) * nall * hd + h * hd + j;  // flat index of the first half's element j
    float a[8], b[8];
    {
        const float4 a0 = part_sum4(q, i0, 0), a1 = part_sum4(q, i0 + 4, 0);
        const float4 b0 = part_sum4(q, i0 + half, 0), b1 = part_sum4(q, i0 + half + 4, 0);
        a[0] = a0.x, a[1] = a0.y, a[2] = a0.z, a[3] = a0.w, a[4] = a1.x, a[5] = a1.y, a[6] = a1.z, a[7] = a1.w;
        b[0] = b0.x, b[1] = b0.y, b[2] = b0.z, b[3] = b0.w, b[4] = b1.x, b[5] = b1.y, b[6] = b1.z, b[7] = b1.w;
    }
    uint16_t* p = buf + i0;
    if (h < nrot) {
        const float4* c4 = reinterpret_cast<const float4*>(cs + (t % seq) * half + j);
        float ra[8], rb[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 c = c4[k];  // (cos, sin) of pairs 2k and 2k+1
            ra[2 * k] = a[2 * k] * c.x - b[2 * k] * c.y;
            rb[2 * k] = b[2 * k] * c.x + a[2 * k] * c.y;
            ra[2 * k + 1] = a[2 * k + 1] * c.z - b[2 * k + 1] * c.w;
            rb[2 * k + 1] = b[2 * k + 1] * c.z + a[2 * k + 1] * c.w;
        }
        *reinterpret_cast<uint4*>(p) = pack8(ra, f16);
        *reinterpret_cast<uint4*>(p + half) = pack8(rb, f16);
    } else {
        *reinterpret_cast<uint4*>(p) = pack8(a, f16);
        *reinterpret_cast<uint4*>(p + half) = pack8(b, f16);
    }
}
bool rope_part_ok(int hd, int nall) { return hd % 16 == 0 && hd >= 16 && nall >= 1; }
void launch_rope_part(const Partials& src, uint16_t* buf, int T, int seq, int nrot, int nall, int hd, const float* cs,
                      int f16, hipStream_t s) {
    const int64_t total = int64_t(T) * nall * (hd / 16);
    if (total <= 0) return;
    QLX_REQUIRE(rope_part_ok(hd, nall) && nrot >= 0 && nrot <= nall && al16(buf) && al16(cs) && !src.R, QLX_EINVAL,
                "rope (partials): needs hd a multiple of 16 and aligned rows");
    check_part(src, int64_t(T) * nall * hd, "rope");
    const double n = double(T) * nall * hd;
    ProfScope prof("reduce_rope", n * (src.splits + 3.0), n * (4.0 * src.splits + 2.0), s);
    hipLaunchKernelGGL(k_rope8_part, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, src, buf, T, seq, nrot, nall,
                       hd, reinterpret_cast<const float2*>(cs), f16);
    check_launch("rope (partials)");
}

void launch_rope_table(int seq, int hd, float theta, float* cs, hipStream_t s) {
    const int n = seq * (hd / 2);
    ProfScope prof("rope_table", 0.0, 8.0 * n, s);
    hipLaunchKernelGGL(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, s, seq, hd, double(theta),
                       reinterpret_cast<float2*>(cs));
    check_launch("rope_table");
}
void launch_rope(uint16_t* buf, int64_t ld, int T, int seq, int col0, int nheads, int hd, const float* cs, int f16,
                 hipStream_t s) {
    const int64_t total = int64_t(T) * nheads * (hd / 2);
    if (total <= 0) return;
    ProfScope prof("rope", 6.0 * total, 8.0 * total, s);
    if ((hd / 2) % 8 == 0 && ld % 8 == 0 && col0 % 8 == 0 && al16(buf) && al16(cs)) {
        const int64_t t8 = total / 8;
        hipLaunchKernelGGL(k_rope8, dim3(unsigned((t8 + 255) / 256)), dim3(256), 0, s, buf, ld, T, seq, col0, nheads,
                           hd, reinterpret_cast<const float2*>(cs), f16);
        check_launch("rope");
        return;
    }
    hipLaunchKernelGGL(k_rope, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, buf, ld, T, seq, col0, nheads,
                       hd, reinterpret_cast<const float2*>(cs), f16);
    check_launch("rope");
}

// ------------------------------------------------------------------ SwiGLU
// gu = [gate | up] 16-bit [T, 2I]; act = silu(gate) * up.
__device__ inline float silu_sig(float g) { return 1.0f / (1.0f + expf(-g)); }
// VEC: 8 consecutive i per thread with 16-byte accesses (I % 8 == 0, 16-byte
// aligned buffers); the arithmetic per element is the same either way.
template <bool VEC>
__global__ void k_swiglu_fwd(const uint16_t* __restrict__ gu, int T, int I, uint16_t* __restrict__ act, int f16) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (VEC) {
        const int I8 = I / 8;
        if (idx >= int64_t(T) * I8) return;
        const int64_t t = idx / I8, i = (idx % I8) * 8;
        float g[8], u[8], y[8];
        unpack8(*reinterpret_cast<const uint4*>(gu + t * 2 * I + i), g, f16);
        unpack8(*reinterpret_cast<const uint4*>(gu + t * 2 * I + I + i), u, f16);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = g[e] * silu_sig(g[e]) * u[e];
        *reinterpret_cast<uint4*>(act + t * I + i) = pack8(y, f16);
        return;
    }
    if (idx >= int64_t(T) * I) return;
    const int64_t t = idx / I, i = idx % I;
    const float g = act_to_f32(gu[t * 2 * I + i], f16);
    const float u = act_to_f32(gu[t * 2 * I + I + i], f16);
    act[idx] = f32_to_act(g * silu_sig(g) * u, f16);
}
// dgate = da * up * silu'(gate), dup = da * silu(gate); silu' = s (1 + g (1 - s)).
template <bool VEC>
__global__ void k_swiglu_bwd(const uint16_t* __restrict__ dact, const uint16_t* __restrict__ gu, int T, int I,
                             uint16_t* __restrict__ dgu, int f16) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (VEC) {
        const int I8 = I / 8;
        if (idx >= int64_t(T) * I8) return;
        const int64_t t = idx / I8, i = (idx % I8) * 8;
        float g[8], u[8], da[8], dg[8], du[8];
        unpack8(*reinterpret_cast<const uint4*>(gu + t * 2 * I + i), g, f16);
        unpack8(*reinterpret_cast<const uint4*>(gu + t * 2 * I + I + i), u, f16);
        unpack8(*reinterpret_cast<const uint4*>(dact + t * I + i), da, f16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sg = silu_sig(g[e]);
            dg[e] = da[e] * u[e] * (sg * (1.0f + g[e] * (1.0f - sg)));
            du[e] = da[e] * g[e] * sg;
        }
        *reinterpret_cast<uint4*>(dgu + t * 2 * I + i) = pack8(dg, f16);
        *reinterpret_cast<uint4*>(dgu + t * 2 * I + I + i) = pack8(du, f16);
        return;
    }
    if (idx >= int64_t(T) * I) return;
    const int64_t t = idx / I, i = idx % I;
    const float g = act_to_f32(gu[t * 2 * I + i], f16);
    const float u = act_to_f32(gu[t * 2 * I + I + i], f16);
    const float da = act_to_f32(dact[idx], f16);
    const float sg = silu_sig(g);
    dgu[t * 2 * I + i] = f32_to_act(da * u * (sg * (1.0f + g * (1.0f - sg))), f16);
    dgu[t * 2 * I + I + i] = f32_to_act(da * g * sg, f16);
}
void launch_swiglu_fwd(const uint16_t* gu, int T, int I, uint16_t* act, int f16, hipStream_t s) {
    const int64_t n = int64_t(T) * I;
    if (n <= 0) return;
    ProfScope prof("swiglu_fwd", 5.0 * n, 6.0 * n, s);
    if (I % 8 == 0 && al16(gu) && al16(act))
        hipLaunchKernelGGL(k_swiglu_fwd<true>, dim3(unsigned((n / 8 + 255) / 256)), dim3(256), 0, s, gu, T, I, act, f16);
    else
        hipLaunchKernelGGL(k_swiglu_fwd<false>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, gu, T, I, act, f16);
    check_launch("swiglu_fwd");
}
void launch_swiglu_bwd(const uint16_t* dact, const uint16_t* gu, int T, int I, uint16_t* dgu, int f16, hipStream_t s) {
    const int64_t n = int64_t(T) * I;
    if (n <= 0) return;
    ProfScope prof("swiglu_bwd", 10.0 * n, 10.0 * n, s);
    if (I % 8 == 0 && al16(gu) && al16(dact) && al16(dgu))
        hipLaunchKernelGGL(k_swiglu_bwd<true>, dim3(unsigned((n / 8 + 255) / 256)), dim3(256), 0, s, dact, gu, T, I,
                           dgu, f16);
    else
        hipLaunchKernelGGL(k_swiglu_bwd<false>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, dact, gu, T, I,
                           dgu, f16);
    check_launch("swiglu_bwd");
}

// ------------------------------------------------------------------ embedding
// h[t] = fp32(E[tok[t]]); an out-of-range id yields NaN (never an out-of-bounds read).
__global__ void k_embed(const int32_t* __restrict__ tok, const uint16_t* __restrict__ E, int T, int H, int V,
                        float* __restrict__ h) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= int64_t(T) * H) return;
    const int64_t t = idx / H, j = idx % H;
    const int id = tok[t];
    h[idx] = (id >= 0 && id < V) ? f16_bits_to_f32(E[int64_t(id) * H + j]) : __int_as_float(0x7fc00000);
}
void launch_embed(const int32_t* tok, const uint16_t* E, int T, int H, int V, float* h, hipStream_t s) {
    const int64_t n = int64_t(T) * H;
    if (n <= 0) return;
    ProfScope prof("embed", 0.0, 6.0 * n, s);
    hipLaunchKernelGGL(k_embed, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, tok, E, T, H, V, h);
    check_launch("embed");
}

// y = 16-bit(x * scale) (bf16, or fp16 when f16; scale a power of two that
// moves gradients into fp16's normal range). 8 elements per thread (two
// 16-byte loads, one 16-byte store) where the buffers allow, else one.
template <bool VEC>
__global__ void k_f32_to_act(const float* __restrict__ x, int64_t n, uint16_t* __restrict__ y, int f16, float sc) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (VEC) {
        if (i >= n / 8) return;
        const float4 a = reinterpret_cast<const float4*>(x)[2 * i], b = reinterpret_cast<const float4*>(x)[2 * i + 1];
        reinterpret_cast<uint4*>(y)[i] =
            make_uint4(f32x2_to_act2(a.x * sc, a.y * sc, f16), f32x2_to_act2(a.z * sc, a.w * sc, f16),
                       f32x2_to_act2(b.x * sc, b.y * sc, f16), f32x2_to_act2(b.z * sc, b.w * sc, f16));
        return;
    }
    if (i < n) y[i] = f32_to_act(x[i] * sc, f16);
}
void launch_f32_to_act(const float* x, int64_t n, uint16_t* y, int f16, float scale, hipStream_t s) {
    if (n <= 0) return;
    ProfScope prof("f32_to_16", 0.0, 6.0 * n, s);
    if (n % 8 == 0 && al16(x) && al16(y))
        hipLaunchKernelGGL(k_f32_to_act<true>, dim3(unsigned((n / 8 + 255) / 256)), dim3(256), 0, s, x, n, y, f16,
                           scale);
    else
        hipLaunchKernelGGL(k_f32_to_act<false>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, x, n, y, f16, scale);
    check_launch("f32_to_16");
}

// ------------------------------------------------------------------ stream debugging
// Fills n 32-bit words with one pattern (the poison of a freed slot, the
// zero gradients of an empty batch).
__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = v;
}
void launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
    if (n <= 0) return;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_fill_u32, dim3(unsigned(blocks)), dim3(256), 0, s, p, n, v);
    check_launch("fill_u32");
}
// Wire form -> full form of a layer blob's tail in device memory: each block
// maximum's bf16 bits become the upper half of its fp32 word (exact: the
// maxima of bf16 weights are bf16 values) and the two RMSNorm gains are
// copied. Threads [0, ceil(nb/4)) take four maxima each, the next H threads
// one element of each gain.
__global__ void k_blob_widen(const uint16_t* __restrict__ m16, int64_t nb, const float* __restrict__ g1s,
                             const float* __restrict__ g2s, int H, uint32_t* __restrict__ m32,
                             float* __restrict__ g1d, float* __restrict__ g2d) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n4 = (nb + 3) / 4;
    if (i < n4) {
        const int64_t j = i * 4;
        if (j + 4 <= nb) {
            const uint2 v = *reinterpret_cast<const uint2*>(m16 + j);
            *reinterpret_cast<uint4*>(m32 + j) = make_uint4(v.x << 16, v.x & 0xFFFF0000u, v.y << 16, v.y & 0xFFFF0000u);
        } else {
            for (int64_t k = j; k < nb; ++k) m32[k] = uint32_t(m16[k]) << 16;
        }
        return;
    }
    const int64_t k = i - n4;
    if (k < H) {
        g1d[k] = g1s[k];
        g2d[k] = g2s[k];
    }
}
void launch_blob_widen(const uint16_t* m16, int64_t nb, const float* g1s, const float* g2s, int H, uint32_t* m32,
                       float* g1d, float* g2d, hipStream_t s) {
    QLX_REQUIRE((reinterpret_cast<uintptr_t>(m16) & 7) == 0 && al16(m32), QLX_EINVAL,
                "blob widen: maxima must be 8-byte (source) and 16-byte (destination) aligned");
    const int64_t threads = (nb + 3) / 4 + H;
    if (threads <= 0) return;
    ProfScope prof("blob_widen", 0.0, 6.0 * double(nb) + 16.0 * H, s);
    hipLaunchKernelGGL(k_blob_widen, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, m16, nb, g1s, g2s, H, m32,
                       g1d, g2d);
    check_launch("blob_widen");
}

// Occupies its stream for about `sleeps` x 8k cycles (a fixed count of
// s_sleep 127, so it always ends): shifts when the next operation starts.
__global__ void k_spin(int sleeps) {
    for (int i = 0; i < sleeps; ++i) __builtin_amdgcn_s_sleep(127);
}
void launch_spin(int delay_us, hipStream_t s) {
    if (delay_us <= 0) return;
    const int sleeps = std::min(1 << 20, delay_us / 3 + 1);  // s_sleep 127 ~ 8128 cycles ~ 3.4 us
    hipLaunchKernelGGL(k_spin, dim3(1), dim3(64), 0, s, sleeps);
    check_launch("spin");
}

// ------------------------------------------------------------------ LoRA staging
// Acat [nseg*r, in] = 16-bit(A_p) stacked; Bbd [sum out_p, nseg*r]
// block-diagonal with block p = 16-bit(scale * B_p), zeros elsewhere (bf16,
// or fp16 when f16). The zeros contribute exact +0 products, so a projection
// only sees its own adapter.
struct LoraSegs {
    const float* A[3];
    const float* B[3];
    int out[3];
    int nseg;
    int f16;
};
__device__ inline void lora_pack_one(const LoraSegs& sg, int r, int in_f, float scale, uint16_t* __restrict__ Acat,
                                     uint16_t* __restrict__ Bbd, int64_t nA, int64_t nB, int64_t idx) {
    if (idx < nA) {
        const int64_t row = idx / in_f, k = idx % in_f;
        const int p = int(row / r), i = int(row % r);
        Acat[idx] = f32_to_act(sg.A[p][int64_t(i) * in_f + k], sg.f16);
        return;
    }
    const int64_t jdx = idx - nA;
    if (jdx >= nB) return;
    const int rr = sg.nseg * r;
    const int n = int(jdx / rr), c = int(jdx % rr);
    const int q = c / r, j = c % r;
    int off = 0, p = 0;
    while (p < sg.nseg - 1 && n >= off + sg.out[p]) off += sg.out[p++];
    Bbd[jdx] = (p == q) ? f32_to_act(scale * sg.B[p][int64_t(n - off) * r + j], sg.f16) : uint16_t(0);
}
// Eight consecutive elements per thread (in_f and r multiples of 8, every
// pointer 16-byte aligned): two float4 loads and one 16-byte store. idx8
// counts groups of eight; a group never straddles an A row or a B block.
__device__ inline void lora_pack_one8(const LoraSegs& sg, int r, int in_f, float scale, uint16_t* __restrict__ Acat,
                                      uint16_t* __restrict__ Bbd, int64_t nA, int64_t nB, int64_t idx8) {
    const int64_t idx = idx8 * 8;
    float f[8];
    if (idx < nA) {
        const int64_t row = idx / in_f, k = idx % in_f;
        const int p = int(row / r), i = int(row % r);
        const float4* src = reinterpret_cast<const float4*>(sg.A[p] + int64_t(i) * in_f + k);
        const float4 u = src[0], v = src[1];
        f[0] = u.x, f[1] = u.y, f[2] = u.z, f[3] = u.w, f[4] = v.x, f[5] = v.y, f[6] = v.z, f[7] = v.w;
        *reinterpret_cast<uint4*>(Acat + idx) = pack8(f, sg.f16);
        return;
    }
    const int64_t jdx = idx - nA;
    if (jdx >= nB) return;
    const int rr = sg.nseg * r;
    const int n = int(jdx / rr), c = int(jdx % rr);
    const int q = c / r, j = c % r;
    int off = 0, p = 0;
    while (p < sg.nseg - 1 && n >= off + sg.out[p]) off += sg.out[p++];
    uint4 o = make_uint4(0, 0, 0, 0);
    if (p == q) {
        const float4* src = reinterpret_cast<const float4*>(sg.B[p] + int64_t(n - off) * r + j);
        const float4 u = src[0], v = src[1];
        f[0] = scale * u.x, f[1] = scale * u.y, f[2] = scale * u.z, f[3] = scale * u.w;
        f[4] = scale * v.x, f[5] = scale * v.y, f[6] = scale * v.z, f[7] = scale * v.w;
        o = pack8(f, sg.f16);
    }
    *reinterpret_cast<uint4*>(Bbd + jdx) = o;
}
__global__ void k_lora_pack(const LoraSegs sg, int r, int in_f, float scale, uint16_t* __restrict__ Acat,
                            uint16_t* __restrict__ Bbd, int64_t nA, int64_t nB, int ntot) {
    lora_pack_one(sg, r, in_f, scale, Acat, Bbd, nA, nB, int64_t(blockIdx.x) * blockDim.x + threadIdx.x);
}
struct LoraPackArgs {
    LoraSegs sg[4];
    int in_f[4];
    uint16_t* Acat[4];
    uint16_t* Bbd[4];
    int64_t nA[4], nB[4];
};
// grid row y packs job y; rows past a job's size return at once
template <bool VEC>
__global__ void k_lora_pack_jobs(const LoraPackArgs a, int r, float scale) {
    const int y = blockIdx.y;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (VEC)
        lora_pack_one8(a.sg[y], r, a.in_f[y], scale, a.Acat[y], a.Bbd[y], a.nA[y], a.nB[y], i);
    else
        lora_pack_one(a.sg[y], r, a.in_f[y], scale, a.Acat[y], a.Bbd[y], a.nA[y], a.nB[y], i);
}
void launch_lora_pack(const LoraSeg* segs, int nseg, int r, int in_f, float scale, uint16_t* Acat, uint16_t* Bbd,
                      int f16, hipStream_t s) {
    LoraSegs sg{};
    sg.f16 = f16;
    int ntot = 0;
    for (int p = 0; p < nseg; ++p) {
        sg.A[p] = segs[p].A;
        sg.B[p] = segs[p].B;
        sg.out[p] = segs[p].out_p;
        ntot += segs[p].out_p;
    }
    sg.nseg = nseg;
    const int64_t nA = int64_t(nseg) * r * in_f, nB = int64_t(ntot) * nseg * r;
    const int64_t n = nA + nB;
    ProfScope prof("lora_pack", double(nB), 4.0 * nA + 2.0 * nA + 2.0 * nB + 4.0 * (nB / nseg), s);
    hipLaunchKernelGGL(k_lora_pack, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, sg, r, in_f, scale, Acat, Bbd,
                       nA, nB, ntot);
    check_launch("lora_pack");
}

void launch_lora_pack_jobs(const LoraPackJob* jobs, int njobs, int r, float scale, int f16, hipStream_t s) {
    QLX_REQUIRE(njobs >= 1 && njobs <= 4, QLX_EINVAL, "lora pack: 1..4 jobs");
    LoraPackArgs a{};
    int64_t nmax = 0;
    double bytes = 0, elems = 0;
    bool vec = r % 8 == 0;
    for (int y = 0; y < njobs; ++y) {
        const LoraPackJob& jb = jobs[y];
        int ntot = 0;
        for (int p = 0; p < jb.nseg; ++p) {
            a.sg[y].A[p] = jb.segs[p].A;
            a.sg[y].B[p] = jb.segs[p].B;
            a.sg[y].out[p] = jb.segs[p].out_p;
            ntot += jb.segs[p].out_p;
            vec = vec && al16(jb.segs[p].A) && al16(jb.segs[p].B);
        }
        vec = vec && jb.in_f % 8 == 0 && al16(jb.Acat) && al16(jb.Bbd);
        a.sg[y].nseg = jb.nseg;
        a.sg[y].f16 = f16;
        a.in_f[y] = jb.in_f;
        a.Acat[y] = jb.Acat;
        a.Bbd[y] = jb.Bbd;
        a.nA[y] = int64_t(jb.nseg) * r * jb.in_f;
        a.nB[y] = int64_t(ntot) * jb.nseg * r;
        nmax = std::max(nmax, a.nA[y] + a.nB[y]);
        bytes += 6.0 * a.nA[y] + 2.0 * a.nB[y] + 4.0 * (a.nB[y] / jb.nseg);
        elems += double(a.nB[y]);
    }
    if (nmax == 0) return;
    ProfScope prof("lora_pack", elems, bytes, s);
    if (vec)
        hipLaunchKernelGGL(k_lora_pack_jobs<true>, dim3(unsigned((nmax / 8 + 255) / 256), unsigned(njobs)), dim3(256), 0,
                           s, a, r, scale);
    else
        hipLaunchKernelGGL(k_lora_pack_jobs<false>, dim3(unsigned((nmax + 255) / 256), unsigned(njobs)), dim3(256), 0,
                           s, a, r, scale);
    check_launch("lora_pack");
}

// Per-query-head gradients dh [B*nH, S, hd] -> per-KV-head sums written as
// 16-bit values (bf16, or fp16 when f16) into out[(b*S + t)*ldo + col0 +
// kvh*hd + d]; group members summed in order.
__global__ void k_gqa_reduce(const float* __restrict__ dh, int B, int nH, int nKV, int S, int hd,
                             uint16_t* __restrict__ out, int64_t ldo, int col0, const float2* __restrict__ rope,
                             int f16) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int half = hd / 2, np = rope ? half : hd;  // a thread: one dim, or one rotated pair
    const int64_t total = int64_t(B) * nKV * S * np;
    if (idx >= total) return;
    const int d = int(idx % np);
    const int t = int((idx / np) % S);
    const int kvh = int((idx / (int64_t(np) * S)) % nKV);
    const int b = int(idx / (int64_t(np) * S * nKV));
    const int grp = nH / nKV;
    float v = 0.f, w = 0.f;
    for (int g = 0; g < grp; ++g) {
        const float* src = dh + ((int64_t(b) * nH + kvh * grp + g) * S + t) * hd;
        v += src[d];
        if (rope) w += src[d + half];
    }
    uint16_t* o = out + (int64_t(b) * S + t) * ldo + col0 + kvh * hd;
    if (!rope) {
        o[d] = f32_to_act(v, f16);
        return;
    }
    const float2 c = rope[int64_t(t) * half + d];  // the rotation's transpose
    o[d] = f32_to_act(v * c.x + w * c.y, f16);
    o[d + half] = f32_to_act(w * c.x - v * c.y, f16);
}
void launch_gqa_reduce(const float* dh, int B, int nH, int nKV, int S, int hd, uint16_t* out, int64_t ldo, int col0,
                       const float* rope, int f16, hipStream_t s) {
    const int64_t total = int64_t(B) * nKV * S * (rope ? hd / 2 : hd);
    if (total <= 0) return;
    ProfScope prof("gqa_reduce", double(B) * nKV * S * hd * (nH / nKV), double(B) * nKV * S * hd * (4.0 * (nH / nKV) + 2.0),
                   s);
    hipLaunchKernelGGL(k_gqa_reduce, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, dh, B, nH, nKV, S, hd, out,
                       ldo, col0, reinterpret_cast<const float2*>(rope), f16);
    check_launch("gqa_reduce");
}

// ------------------------------------------------------------------ cross-entropy
// Row t predicts tokens[t + 1] when its position in the sequence lies in
// [start, seq - 1); otherwise it has no target (-1).
__device__ inline int row_target(const int32_t* tokens, int t, int seq, int start) {
    const int s = t % seq;
    if (s < start || s >= seq - 1) return -1;
    return tokens[t + 1];
}

// lse of each row from the LM-head epilogue's per-64-column partials
// (max m_b, sum s_b of exp(z - m_b)): m = max_b m_b, lse = m + log(sum_b s_b
// exp(m_b - m)), one wavefront per row, blocks split over lanes in a fixed
// pattern and joined in a fixed tree. Rows without a target get lse =
// picked = 0; a target outside the vocabulary gives NaN.
__global__ __launch_bounds__(256) void k_ce_reduce(const float* __restrict__ pm, const float* __restrict__ ps, int nb,
                                                   int T, int V, const int32_t* __restrict__ tokens, int seq, int start,
                                                   float* __restrict__ lse, float* __restrict__ picked) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= T) return;
    const int tgt = row_target(tokens, t, seq, start);
    if (tgt < 0) {
        if (lane == 0) lse[t] = picked[t] = 0.f;
        return;
    }
    const float* m_ = pm + int64_t(t) * nb;
    const float* s_ = ps + int64_t(t) * nb;
    float m = -INFINITY;
    for (int b = lane; b < nb; b += 64) m = fmaxf(m, m_[b]);
    m = wave_max(m);
    float sum = 0.f;
    for (int b = lane; b < nb; b += 64)
        if (m_[b] > -INFINITY) sum += s_[b] * expf(m_[b] - m);
    sum = wave_sum(sum);
    if (lane == 0) {
        const bool ok = tgt < V;
        lse[t] = ok ? m + logf(sum) : __int_as_float(0x7fc00000);
        if (!ok) picked[t] = __int_as_float(0x7fc00000);
    }
}
void launch_ce_reduce(const float* pm, const float* ps, int nb, int T, int V, const int32_t* tokens, int seq, int start,
                      float* lse, float* picked, hipStream_t s) {
    if (T <= 0) return;
    ProfScope prof("ce_reduce", 3.0 * T * nb, 8.0 * T * nb, s);
    hipLaunchKernelGGL(k_ce_reduce, dim3(unsigned((T + 3) / 4)), dim3(256), 0, s, pm, ps, nb, T, V, tokens, seq, start,
                       lse, picked);
    check_launch("ce_reduce");
}

// dz of one vocabulary chunk from the LM head's fp32 logits z (the statistics
// pass keeps them): dz[t, j] = fp16((exp(z[t, col0 + j] - lse[t]) -
// [col0 + j == target]) * scale), scale = sc (times gseq[t / seq] when given),
// 0 on rows without a target. dz = softmax - onehot is the cross-entropy's
// gradient with respect to the logits; sc carries the loss's 1/N and the
// fixed power-of-two range factor. One thread: 8 consecutive columns.
__global__ __launch_bounds__(256) void k_ce_dz(const float* __restrict__ z, int64_t ldz, int T, int cw, int col0,
                                               const int32_t* __restrict__ tokens, int seq, int start,
                                               const float* __restrict__ lse, float sc,
                                               const float* __restrict__ gseq, uint16_t* __restrict__ dz,
                                               int64_t lddz) {
    const int groups = (cw + 7) / 8;
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= int64_t(T) * groups) return;
    const int t = int(i / groups), j0 = int(i % groups) * 8;
    const int tgt = row_target(tokens, t, seq, start);
    const float scale = sc * (gseq ? gseq[t / seq] : 1.f);
    const float l = tgt >= 0 ? lse[t] : 0.f;
    const float* src = z + int64_t(t) * ldz + col0 + j0;
    uint16_t* dst = dz + int64_t(t) * lddz + j0;
    const int v0 = col0 + j0;
    if (j0 + 8 <= cw && (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float v_lo = tgt < 0 ? 0.f : (expf(x[2 * k] - l) - (v0 + 2 * k == tgt ? 1.f : 0.f)) * scale;
            const float v_hi = tgt < 0 ? 0.f : (expf(x[2 * k + 1] - l) - (v0 + 2 * k + 1 == tgt ? 1.f : 0.f)) * scale;
            w[k] = uint32_t(f32_to_f16_bits(v_lo)) | (uint32_t(f32_to_f16_bits(v_hi)) << 16);
        }
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        for (int c = 0; c < 8 && j0 + c < cw; ++c)
            dst[c] = f32_to_f16_bits(tgt < 0 ? 0.f : (expf(src[c] - l) - (v0 + c == tgt ? 1.f : 0.f)) * scale);
    }
}
void launch_ce_dz(const float* z, int64_t ldz, int T, int cw, int col0, const int32_t* tokens, int seq, int start,
                  const float* lse, float sc, const float* gseq, uint16_t* dz, int64_t lddz, hipStream_t s) {
    if (T <= 0 || cw <= 0) return;
    const int64_t n = int64_t(T) * ((cw + 7) / 8);
    ProfScope prof("ce_dz", 4.0 * T * cw, 6.0 * T * cw, s);
    hipLaunchKernelGGL(k_ce_dz, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, z, ldz, T, cw, col0, tokens, seq,
                       start, lse, sc, gseq, dz, lddz);
    check_launch("ce_dz");
}

// SFT loss = sum over target rows of (lse - picked) / (#rows with a target).
__global__ __launch_bounds__(256) void k_sft_loss(const float* __restrict__ lse, const float* __restrict__ picked,
                                                  int T, int seq, float* __restrict__ loss) {
    __shared__ float red[4];
    float acc = 0.f;
    for (int t = threadIdx.x; t < T; t += 256) acc += lse[t] - picked[t];
    acc = block_sum256(acc, red);
    if (threadIdx.x == 0) {
        const int nseq = T / seq;
        loss[0] = acc / float(nseq * (seq - 1));
    }
}
void launch_sft_loss(const float* lse, const float* picked, int T, int seq, float* loss, hipStream_t s) {
    ProfScope prof("loss_reduce", 2.0 * T, 8.0 * T, s);
    hipLaunchKernelGGL(k_sft_loss, dim3(1), dim3(256), 0, s, lse, picked, T, seq, loss);
    check_launch("sft_loss");
}

// Preference losses from per-sequence summed response log-probs. One
// workgroup: per-sequence sums of picked - lse (rows outside the response are
// zero), then one thread evaluates the loss and dL/ds in double:
//  DPO (Rafailov et al. 2023, eq. 7): mean over pairs of -log sigmoid(beta Delta).
//  ORPO (Hong et al. 2024, eqs. 2-7): mean over pairs of -l_c + lambda *
//    -log sigmoid(log odds_c - log odds_r), l = s/n, log odds = l - log(1 - e^l).
//  SimPO (Meng et al. 2024, eq. 6): mean over pairs of
//    -log sigmoid(beta (l_c - l_r) - gamma).
//  KTO (Ethayarajh et al. 2024, eq. 8): r = s_pol - s_ref; z0 = max(0, mean
//    of the mismatched pairs' s_pol - s_ref), constant for the gradient;
//    mean over examples of lambda_y - v, v = lambda_D sigmoid(beta (r - z0))
//    for chosen, lambda_U sigmoid(beta (z0 - r)) for rejected.
// logps: [4P] policy chosen, policy rejected, reference chosen, reference
// rejected (zeros for the reference-free kinds). gseq: dL/ds per sequence.
namespace {
__device__ inline double log_sigmoid(double x) { return (x >= 0.0) ? -log1p(exp(-x)) : x - log1p(exp(x)); }
__device__ inline double sigmoid(double x) { return (x >= 0.0) ? 1.0 / (1.0 + exp(-x)) : exp(x) / (1.0 + exp(x)); }
__device__ inline double log1mexp(double l) { return (l > -0.6931471805599453) ? log(-expm1(l)) : log1p(-exp(l)); }

__device__ float seq_sum(const float* __restrict__ lse, const float* __restrict__ pk, int b, int seq, float* red) {
    float a = 0.f;
    for (int s = threadIdx.x; s < seq; s += 256) {
        const int64_t t = int64_t(b) * seq + s;
        a += pk[t] - lse[t];
    }
    return block_sum256(a, red);
}
}  // namespace

__global__ __launch_bounds__(256) void k_pref_loss(PrefLossArgs a) {
    __shared__ float red[4];
    __shared__ float lp[4][64];  // policy, reference, KL policy, KL reference
    const int nseq = 2 * a.pairs;
    for (int b = 0; b < nseq; ++b) {
        const float p = seq_sum(a.lse_p, a.pk_p, b, a.seq, red);
        const float r = a.lse_r ? seq_sum(a.lse_r, a.pk_r, b, a.seq, red) : 0.f;
        const float kp = a.kl_lse_p ? seq_sum(a.kl_lse_p, a.kl_pk_p, b, a.seq, red) : 0.f;
        const float kr = a.kl_lse_r ? seq_sum(a.kl_lse_r, a.kl_pk_r, b, a.seq, red) : 0.f;
        if (threadIdx.x == 0) {
            lp[0][b] = p;
            lp[1][b] = r;
            lp[2][b] = kp;
            lp[3][b] = kr;
        }
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    const int P = a.pairs;
    const double n = double(a.nresp), beta = a.beta;
    double tot = 0.0;
    if (a.kind == PREF_DPO) {
        for (int i = 0; i < P; ++i) {
            const float delta = (lp[0][i] - lp[1][i]) - (lp[0][P + i] - lp[1][P + i]);
            const double x = beta * double(delta);
            tot += (x >= 0.0) ? log1p(exp(-x)) : (-x + log1p(exp(x)));
            const double g = -beta / (1.0 + exp(x)) / double(P);
            a.gseq[i] = float(g);
            a.gseq[P + i] = float(-g);
        }
        a.loss[0] = float(tot / double(P));
    } else if (a.kind == PREF_ORPO) {
        for (int i = 0; i < P; ++i) {
            const double lc = double(lp[0][i]) / n, lr = double(lp[0][P + i]) / n;
            const double z = (lc - log1mexp(lc)) - (lr - log1mexp(lr));
            tot += -lc - beta * log_sigmoid(z);
            const double sg = sigmoid(-z);
            a.gseq[i] = float((-1.0 - beta * sg / (-expm1(lc))) / (double(P) * n));
            a.gseq[P + i] = float((beta * sg / (-expm1(lr))) / (double(P) * n));
        }
        a.loss[0] = float(tot / double(P));
    } else if (a.kind == PREF_SIMPO) {
        for (int i = 0; i < P; ++i) {
            const double u = beta * (double(lp[0][i]) / n - double(lp[0][P + i]) / n) - double(a.gamma);
            tot += -log_sigmoid(u);
            const double g = -sigmoid(-u) * beta / (double(P) * n);
            a.gseq[i] = float(g);
            a.gseq[P + i] = float(-g);
        }
        a.loss[0] = float(tot / double(P));
    } else {  // KTO
        double kl = 0.0;
        for (int b = 0; b < nseq; ++b) kl += double(lp[2][b]) - double(lp[3][b]);
        const double z0 = fmax(0.0, kl / double(nseq));
        for (int b = 0; b < nseq; ++b) {
            const double r = double(lp[0][b]) - double(lp[1][b]);
            const bool des = b < P;
            const double lam = des ? a.lambda_d : a.lambda_u;
            const double x = des ? beta * (r - z0) : beta * (z0 - r);
            const double sx = sigmoid(x);
            tot += lam - lam * sx;
            const double g = lam * beta * sx * sigmoid(-x) / double(nseq);
            a.gseq[b] = float(des ? -g : g);
        }
        a.loss[0] = float(tot / double(nseq));
    }
    for (int b = 0; b < nseq; ++b) {
        a.logps[b] = lp[0][b];
        a.logps[nseq + b] = lp[1][b];
    }
}

void launch_pref_loss(const PrefLossArgs& a, hipStream_t s) {
    QLX_REQUIRE(a.pairs >= 1 && 2 * a.pairs <= 64, QLX_EINVAL, "pref loss: pairs must be in 1..32");
    const int nstat = 2 + (a.lse_r ? 2 : 0) + (a.kl_lse_p ? 4 : 0);
    ProfScope prof("loss_reduce", 2.0 * a.seq * a.pairs * nstat, 8.0 * a.seq * a.pairs * nstat, s);
    hipLaunchKernelGGL(k_pref_loss, dim3(1), dim3(256), 0, s, a);
    check_launch("pref_loss");
}

// KTO's mismatched pairs: sequence j = its own prompt followed by the
// completion of sequence (j + 1) mod B.
__global__ __launch_bounds__(256) void k_kl_tokens(const int32_t* __restrict__ toks, int B, int seq, int prompt_len,
                                                   int32_t* __restrict__ out) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= int64_t(B) * seq) return;
    const int b = int(i / seq), t = int(i % seq);
    out[i] = (t < prompt_len) ? toks[i] : toks[int64_t((b + 1) % B) * seq + t];
}
void launch_kl_tokens(const int32_t* toks, int B, int seq, int prompt_len, int32_t* out, hipStream_t s) {
    const int64_t n = int64_t(B) * seq;
    ProfScope prof("kl_tokens", 0.0, 8.0 * n, s);
    hipLaunchKernelGGL(k_kl_tokens, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, toks, B, seq, prompt_len, out);
    check_launch("kl_tokens");
}

}  // namespace qlx
