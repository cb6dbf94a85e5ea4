// GEMM family on CDNA4 bf16/fp16 MFMA (v_mfma_f32_16x16x32_{bf16,f16}) with
// the NF4 dequantization fused into the weight-operand load.
//
// What it computes: C = alpha * (A . op(B) + A2 . op(B2)) (+ R) (+ C_old),
// fp32 accumulation. For the QLoRA linear (LoRA, Hu et al. 2021, section 4.1,
// on the frozen NF4 base the pages describe: rug.gal article "En detalle") the
// first K phase runs over the NF4 weight and the second phase ("slab",
// K2 = r or a few r) adds the LoRA term u . (sB)^T, so the adapter costs one
// short extra K stretch instead of a separate pass over the output.
//
// Structure: a workgroup of (BM/WM)*(BN/WN) wavefronts computes a BM x BN tile
// in K chunks of 64. Each chunk: global loads of the NEXT chunk are issued into
// registers, the wavefronts run their MFMAs on the CURRENT chunk from LDS, then
// the prefetched registers are (for NF4: unpacked, looked up in a 16-entry LDS
// table of code values, multiplied by the block absmax, rounded to bf16) and
// written to the other LDS buffer; one barrier per chunk. LDS tiles are stored
// k-contiguous ([rows][64+8]) so every MFMA fragment is one 16-byte LDS read.
// Loaders exist for every operand layout the training step needs (A row-major
// or transposed; B NF4 [N][K] or [K][N], dense [N][K] or [K][N]), so no operand
// is ever transposed in memory. Edges are zero-filled by the loaders and
// masked by the epilogue. The generic kernel and the dense full-tile kernel
// (whose fp16 weight is the large operand) order tiles so the M-tiles sharing
// one weight tile run on the same XCD (one L2) together; the NF4 full-tile
// kernels put the N-tiles sharing one activation row block there instead
// (bf16 activations are 4x the bytes of NF4 weights per element: measured
// 1-4% faster, 12% fewer HBM bytes fetched by the dX product).
// Split-K writes fp32 partials that a second kernel sums in a fixed order:
// results depend only on shapes, never on timing or pointer values.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "nf4_codes.h"
#include "qlx_internal.h"

namespace qlx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64, BKP = BK + 8;

template <int TE>
__device__ inline f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
    if constexpr (TE == TE_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

__device__ inline uint32_t pack2(uint32_t lo, uint32_t hi) { return (lo & 0xFFFFu) | (hi << 16); }

// ---------------------------------------------------------------------------
// Tile addressing: padded rows of BKP elements, or (SWZ) unpadded 64-element
// rows whose 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7).
template <bool SWZ>
__device__ __forceinline__ int tile_off(int r, int c) {
    if constexpr (SWZ) return r * 64 + ((c ^ ((r >> 1) & 7)) << 3);
    else return r * BKP + c * 8;
}

// Row-major operand: tile[r][k] = src[(r0 + r) * ld + k0 + k], r < R, k < 64.
template <int R, int NT, bool SWZ = false>
struct RowLoader {
    static constexpr int U = R * (BK / 8) / NT;
    static_assert(U >= 1 && R * (BK / 8) % NT == 0, "row loader shape");
    uint4 v[U];
    __device__ inline void load(const uint16_t* __restrict__ src, int64_t ld, int r0, int k0, int rows, int K,
                                int vec_ok) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            const int r = idx >> 3, c = (idx & 7) * 8;
            const int gr = r0 + r, gc = k0 + c;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (gr < rows) {
                const uint16_t* p = src + int64_t(gr) * ld + gc;
                if (vec_ok && gc + 8 <= K) {
                    val = *reinterpret_cast<const uint4*>(p);
                } else {
                    uint32_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (gc + j < K) ? p[j] : 0u;
                    val = make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
                }
            }
            v[u] = val;
        }
    }
    __device__ inline void store(uint16_t* __restrict__ tile) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            *reinterpret_cast<uint4*>(tile + tile_off<SWZ>(idx >> 3, idx & 7)) = v[u];
        }
    }
};

// Transposed operand: tile[r][k] = src[(k0 + k) * ld + r0 + r]. A unit is 4
// consecutive r from 8 consecutive k rows, written as 4 k-contiguous vectors.
// With fewer units than threads, the surplus threads load and store nothing.
template <int R, int NT, bool SWZ = false>
struct TransLoader {
    static constexpr int UNITS = (R / 4) * (BK / 8);
    static constexpr int U = UNITS >= NT ? UNITS / NT : 1;
    static_assert(UNITS % NT == 0 || NT % UNITS == 0, "trans loader shape");
    uint2 v[U][8];
    __device__ inline void load(const uint16_t* __restrict__ src, int64_t ld, int r0, int k0, int rows, int K,
                                int vec_ok) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            if (UNITS < NT && idx >= UNITS) break;
            const int rg = (idx % (R / 4)) * 4, kg = (idx / (R / 4)) * 8;
            const int gr = r0 + rg;
#pragma unroll
            for (int kr = 0; kr < 8; ++kr) {
                const int gk = k0 + kg + kr;
                uint2 w = make_uint2(0, 0);
                if (gk < K) {
                    const uint16_t* p = src + int64_t(gk) * ld + gr;
                    if (vec_ok && gr + 4 <= rows) {
                        w = *reinterpret_cast<const uint2*>(p);
                    } else {
                        uint32_t e[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) e[j] = (gr + j < rows) ? p[j] : 0u;
                        w = make_uint2(pack2(e[0], e[1]), pack2(e[2], e[3]));
                    }
                }
                v[u][kr] = w;
            }
        }
    }
    __device__ inline void store(uint16_t* __restrict__ tile) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            if (UNITS < NT && idx >= UNITS) break;
            const int rg = (idx % (R / 4)) * 4, kg = (idx / (R / 4)) * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sh = (j & 1) * 16;
                uint32_t e[8];
#pragma unroll
                for (int kr = 0; kr < 8; ++kr) e[kr] = ((j < 2 ? v[u][kr].x : v[u][kr].y) >> sh) & 0xFFFFu;
                *reinterpret_cast<uint4*>(tile + tile_off<SWZ>(rg + j, kg >> 3)) =
                    make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
            }
        }
    }
};

__device__ inline uint32_t nf4_elem(const uint8_t* __restrict__ packed, const float* __restrict__ absmax,
                                    int64_t flat, const float* lut) {
    const uint32_t byte = packed[flat >> 1];
    const int code = (flat & 1) ? int(byte & 15) : int(byte >> 4);
    return f32_to_bf16_bits(lut[code] * absmax[flat >> 6]);
}

__device__ inline uint32_t deq2(uint32_t byte, float a, const float* lut) {
    // byte -> bf16 pair (high nibble = even element in the low half)
    return f32x2_to_bf16x2(lut[byte >> 4] * a, lut[byte & 15] * a);
}

// NF4 weight stored [N][K] (flat n*cols + k): tile[n][k]. A unit is 32 codes
// (16 bytes) of one row inside one 64-element absmax block.
template <int R, int NT>
struct Nf4NtLoader {
    static constexpr int U = R * 2 / NT;
    static_assert(U >= 1 && R * 2 % NT == 0, "nf4 nt loader shape");
    uint4 w[U];
    float a[U];
    bool fast;
    __device__ inline void load(const uint8_t* __restrict__ packed, const float* __restrict__ absmax, int64_t cols,
                                int n0, int k0, int N, int K, int aligned) {
        fast = aligned && n0 + R <= N && k0 + BK <= K;
        if (!fast) return;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            const int64_t flat = int64_t(n0 + (idx >> 1)) * cols + k0 + (idx & 1) * 32;
            w[u] = *reinterpret_cast<const uint4*>(packed + (flat >> 1));
            a[u] = absmax[flat >> 6];
        }
    }
    __device__ inline void store(uint16_t* __restrict__ tile, const uint8_t* __restrict__ packed,
                                 const float* __restrict__ absmax, int64_t cols, int n0, int k0, int N, int K,
                                 const float* lut) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            const int r = idx >> 1, half = idx & 1;
            uint16_t* dst = tile + r * BKP + half * 32;
            if (fast) {
                const uint32_t words[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t x = words[q];
                    *reinterpret_cast<uint4*>(dst + q * 8) =
                        make_uint4(deq2(x & 0xFF, a[u], lut), deq2((x >> 8) & 0xFF, a[u], lut),
                                   deq2((x >> 16) & 0xFF, a[u], lut), deq2(x >> 24, a[u], lut));
                }
            } else {
                const int gn = n0 + r, gk = k0 + half * 32;
                for (int j = 0; j < 32; ++j) {
                    const int k = gk + j;
                    dst[j] = (gn < N && k < K) ? uint16_t(nf4_elem(packed, absmax, int64_t(gn) * cols + k, lut))
                                               : uint16_t(0);
                }
            }
        }
    }
};

// NF4 weight stored [K][N] (flat k*cols + n): tile[n][k]. A unit is 4
// consecutive n (2 bytes) from each of 8 consecutive k rows.
template <int R, int NT>
struct Nf4NnLoader {
    static constexpr int U = (R / 4) * (BK / 8) / NT;
    static_assert(U >= 1 && (R / 4) * (BK / 8) % NT == 0, "nf4 nn loader shape");
    uint32_t two[U][8];
    float a[U][8];
    bool fast;
    __device__ inline void load(const uint8_t* __restrict__ packed, const float* __restrict__ absmax, int64_t cols,
                                int n0, int k0, int N, int K, int aligned) {
        fast = aligned && n0 + R <= N && k0 + BK <= K;
        if (!fast) return;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            const int ng = (idx % (R / 4)) * 4, kg = (idx / (R / 4)) * 8;
#pragma unroll
            for (int kr = 0; kr < 8; ++kr) {
                const int64_t flat = int64_t(k0 + kg + kr) * cols + n0 + ng;
                two[u][kr] = *reinterpret_cast<const uint16_t*>(packed + (flat >> 1));
                a[u][kr] = absmax[flat >> 6];
            }
        }
    }
    __device__ inline void store(uint16_t* __restrict__ tile, const uint8_t* __restrict__ packed,
                                 const float* __restrict__ absmax, int64_t cols, int n0, int k0, int N, int K,
                                 const float* lut) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            const int ng = (idx % (R / 4)) * 4, kg = (idx / (R / 4)) * 8;
            // e2[kr][h]: bf16 pair (n = ng + 2h, ng + 2h + 1) of k row kr
            uint32_t e2[8][2];
            if (fast) {
#pragma unroll
                for (int kr = 0; kr < 8; ++kr) {
                    const uint32_t t = two[u][kr];
                    const float s = a[u][kr];
                    e2[kr][0] = f32x2_to_bf16x2(lut[(t >> 4) & 15] * s, lut[t & 15] * s);
                    e2[kr][1] = f32x2_to_bf16x2(lut[(t >> 12) & 15] * s, lut[(t >> 8) & 15] * s);
                }
            } else {
#pragma unroll
                for (int kr = 0; kr < 8; ++kr) {
                    const int gk = k0 + kg + kr;
                    uint32_t e[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int gn = n0 + ng + j;
                        e[j] = (gk < K && gn < N) ? nf4_elem(packed, absmax, int64_t(gk) * cols + gn, lut) : 0u;
                    }
                    e2[kr][0] = pack2(e[0], e[1]);
                    e2[kr][1] = pack2(e[2], e[3]);
                }
            }
            // transpose: column j of the 8 x 4 block -> one k-contiguous vector
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = j >> 1, sh = (j & 1) * 16;
                uint32_t c[8];
#pragma unroll
                for (int kr = 0; kr < 8; ++kr) c[kr] = (e2[kr][h] >> sh) & 0xFFFFu;
                *reinterpret_cast<uint4*>(tile + (ng + j) * BKP + kg) =
                    make_uint4(pack2(c[0], c[1]), pack2(c[2], c[3]), pack2(c[4], c[5]), pack2(c[6], c[7]));
            }
        }
    }
};

// One K chunk of MFMAs for wavefront (wm, wn) owning a WM x WN sub-tile.
template <int TE, int WM, int WN>
__device__ inline void mma_chunk(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                 f32x4 (&acc)[WM / 16][WN / 16], int wm, int wn, int lane) {
    const int lr = lane & 15, lk = (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
        uint4 a[WM / 16], b[WN / 16];
#pragma unroll
        for (int i = 0; i < WM / 16; ++i)
            a[i] = *reinterpret_cast<const uint4*>(As + (wm * WM + i * 16 + lr) * BKP + kk + lk);
#pragma unroll
        for (int j = 0; j < WN / 16; ++j)
            b[j] = *reinterpret_cast<const uint4*>(Bs + (wn * WN + j * 16 + lr) * BKP + kk + lk);
#pragma unroll
        for (int i = 0; i < WM / 16; ++i)
#pragma unroll
            for (int j = 0; j < WN / 16; ++j) acc[i][j] = mfma16<TE>(a[i], b[j], acc[i][j]);
    }
}

__device__ inline void store_out(const GemmParams& p, int bo, int bi, int row, int col, float v) {
    v *= p.alpha;
    if (p.R) v += p.R[int64_t(row) * p.ldr + col];
    void* C = p.C;
    int64_t off;
    if (p.seg_rows > 0) {
        C = p.Cseg[row / p.seg_rows];
        off = int64_t(row % p.seg_rows) * p.ldc + col;
    } else {
        off = int64_t(bo) * p.c_so + int64_t(bi) * p.c_si + int64_t(row) * p.ldc + col;
    }
    if (p.c_type == C_F32) {
        float* c = static_cast<float*>(C) + off;
        if (p.accumulate) v += *c;
        *c = v;
    } else if (p.c_type == C_BF16) {
        static_cast<uint16_t*>(C)[off] = f32_to_bf16_bits(v);
    } else {
        static_cast<uint16_t*>(C)[off] = f32_to_f16_bits(v);
    }
}

// Writes n consecutive outputs of one row starting at col (values already
// accumulated, alpha not yet applied). Vector path for plain bf16 and fp32
// (+ residual) rows; store_out element by element otherwise.
__device__ inline void store_row(const GemmParams& p, int bo, int bi, int row, int col, const float* v, int n) {
    if (p.seg_rows == 0 && !p.accumulate && col + n <= p.N && (n & 7) == 0) {
        const int64_t off = int64_t(bo) * p.c_so + int64_t(bi) * p.c_si + int64_t(row) * p.ldc + col;
        if (p.c_type == C_BF16 && (off & 7) == 0 && !p.R) {
            uint16_t* dst = static_cast<uint16_t*>(p.C) + off;
            for (int c = 0; c < n; c += 8) {
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w[k] = f32x2_to_bf16x2(v[c + 2 * k] * p.alpha, v[c + 2 * k + 1] * p.alpha);
                *reinterpret_cast<uint4*>(dst + c) = make_uint4(w[0], w[1], w[2], w[3]);
            }
            return;
        }
        if (p.c_type == C_F32 && (off & 3) == 0 && (!p.R || ((int64_t(row) * p.ldr + col) & 3) == 0)) {
            float* dst = static_cast<float*>(p.C) + off;
            const float* r = p.R ? p.R + int64_t(row) * p.ldr + col : nullptr;
            for (int c = 0; c < n; c += 4) {
                float4 o = make_float4(v[c] * p.alpha, v[c + 1] * p.alpha, v[c + 2] * p.alpha, v[c + 3] * p.alpha);
                if (r) {
                    const float4 q = *reinterpret_cast<const float4*>(r + c);
                    o.x += q.x;
                    o.y += q.y;
                    o.z += q.z;
                    o.w += q.w;
                }
                *reinterpret_cast<float4*>(dst + c) = o;
            }
            return;
        }
    }
    for (int c = 0; c < n; ++c)
        if (col + c < p.N) store_out(p, bo, bi, row, col + c, v[c]);
}

template <int AK, int R, int NT>
using ALoader = typename std::conditional<AK == A_ROW, RowLoader<R, NT>, TransLoader<R, NT>>::type;
template <int BKIND, int R, int NT>
using BLoader = typename std::conditional<
    BKIND == B_NF4_NT, Nf4NtLoader<R, NT>,
    typename std::conditional<BKIND == B_NF4_NN, Nf4NnLoader<R, NT>,
                              typename std::conditional<BKIND == B_DENSE_NT, RowLoader<R, NT>,
                                                        TransLoader<R, NT>>::type>::type>::type;

// LM-head cross-entropy epilogues. The lane holds 16 consecutive columns
// col0.. of one row; the 4 lanes of a row are lanes 4k..4k+3 of the
// wavefront (one 64-column block). Mode 1: the block's max and sum of
// exp(z - max) (joined over the 4 lanes), and the target's logit. Mode 2: fp16
// dz = (exp(z - lse) - onehot) * scale.
__device__ inline int ce_target(const GemmParams& p, int t) {
    const int s = t % p.ce_seq;
    if (s < p.ce_start || s >= p.ce_seq - 1) return -1;
    return p.ce_tokens[t + 1];
}
__device__ void ce_epilogue(const GemmParams& p, int row, int col0, const float* src) {
    const bool rok = row < p.M;
    const int tgt = rok ? ce_target(p, row) : -1;
    const int v0 = p.ce_col0 + col0;  // vocab index of src[0]
    if (p.ce_mode == 1) {
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (col0 + c < p.N) mx = fmaxf(mx, src[c]);
        float sm = 0.f;
        if (mx > -INFINITY) {
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (col0 + c < p.N) sm += expf(src[c] - mx);
        }
#pragma unroll
        for (int off = 1; off <= 2; off <<= 1) {
            const float om = __shfl_xor(mx, off, 64), os = __shfl_xor(sm, off, 64);
            const float nm = fmaxf(mx, om);
            sm = (nm == -INFINITY) ? 0.f : sm * expf(mx - nm) + os * expf(om - nm);
            mx = nm;
        }
        if (rok && (threadIdx.x & 3) == 0 && col0 < p.N) {
            const int64_t o = int64_t(row) * p.ce_pld + v0 / 64;
            p.ce_pm[o] = mx;
            p.ce_ps[o] = sm;
        }
        if (rok && tgt >= v0 && tgt < v0 + 16 && tgt - p.ce_col0 < p.N) p.ce_picked[row] = src[tgt - v0];
        return;
    }
    if (!rok) return;
    const float scale = p.ce_sc * (p.ce_gseq ? p.ce_gseq[row / p.ce_seq] : 1.f);
    const float lse = tgt >= 0 ? p.ce_lse[row] : 0.f;
    float v[16];
#pragma unroll
    for (int c = 0; c < 16; ++c)
        v[c] = tgt < 0 ? 0.f : (expf(src[c] - lse) - (v0 + c == tgt ? 1.f : 0.f)) * scale;
    uint16_t* dst = static_cast<uint16_t*>(p.C) + int64_t(row) * p.ldc + col0;
    if (col0 + 16 <= p.N && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            w[k] = uint32_t(f32_to_f16_bits(v[2 * k])) | (uint32_t(f32_to_f16_bits(v[2 * k + 1])) << 16);
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
        for (int c = 0; c < 16; ++c)
            if (col0 + c < p.N) dst[c] = f32_to_f16_bits(v[c]);
    }
}

template <int AK, int BKIND, int TE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm(const GemmParams p) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    constexpr bool kNf4 = (BKIND == B_NF4_NT || BKIND == B_NF4_NN);
    __shared__ __align__(16) uint16_t As[2][BM * BKP];
    __shared__ __align__(16) uint16_t Bs[2][BN * BKP];
    __shared__ float lut[16];
    const int tid = threadIdx.x;
    if (kNf4 && tid < 16) lut[tid] = nf4_value(tid);

    // tile order: the gy M-tiles of one N-tile are consecutive within an XCD
    const int gx = (p.N + BN - 1) / BN, gy = (p.M + BM - 1) / BM;
    const int ntile = gx * gy;
    int t = blockIdx.x;
    if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
    const int m0 = (t % gy) * BM, n0 = (t / gy) * BN;
    const int split = blockIdx.y % p.splits;
    const int bz = blockIdx.y / p.splits;
    const int bo = bz / p.zdiv, bi = bz % p.zdiv;
    if (p.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;  // tile strictly above the diagonal

    const uint16_t* A = p.A + int64_t(bo) * p.a_so + int64_t(bi / p.a_grp) * p.a_si;
    const uint16_t* Bd =
        static_cast<const uint16_t*>(p.B) + (kNf4 ? 0 : int64_t(bo) * p.b_so + int64_t(bi / p.b_grp) * p.b_si);
    if constexpr (BKIND == B_DENSE_NN)
        if (p.seg_rows > 0) Bd += p.bseg[m0 / p.seg_rows];  // the segment's B columns
    const uint8_t* Bq = static_cast<const uint8_t*>(p.B);

    int kbeg = split * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    if (p.causal == CAUSAL_K_LE_M) kend = min(kend, m0 + BM);
    if (p.causal == CAUSAL_K_GE_M) kbeg = max(kbeg, (m0 / BK) * BK);

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / (BN / WN), wn = wave % (BN / WN);
    f32x4 acc[WM / 16][WN / 16];
#pragma unroll
    for (int i = 0; i < WM / 16; ++i)
#pragma unroll
        for (int j = 0; j < WN / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    {
        ALoader<AK, BM, NT> la;
        BLoader<BKIND, BN, NT> lb;
        __syncthreads();  // lut ready
        if (kbeg < kend) {
            la.load(A, p.lda, m0, kbeg, p.M, p.K, p.a_vec);
            if constexpr (kNf4) {
                lb.load(Bq, p.absmax, p.nf4_cols, n0, kbeg, p.N, p.K, p.b_vec);
                lb.store(Bs[0], Bq, p.absmax, p.nf4_cols, n0, kbeg, p.N, p.K, lut);
            } else {
                lb.load(Bd, p.ldb, n0, kbeg, p.N, p.K, p.b_vec);
                lb.store(Bs[0]);
            }
            la.store(As[0]);
        }
        __syncthreads();
        int buf = 0;
        for (int k0 = kbeg; k0 < kend; k0 += BK) {
            const int kn = k0 + BK;
            const bool more = kn < kend;
            if (more) {
                la.load(A, p.lda, m0, kn, p.M, p.K, p.a_vec);
                if constexpr (kNf4) lb.load(Bq, p.absmax, p.nf4_cols, n0, kn, p.N, p.K, p.b_vec);
                else lb.load(Bd, p.ldb, n0, kn, p.N, p.K, p.b_vec);
            }
            mma_chunk<TE, WM, WN>(As[buf], Bs[buf], acc, wm, wn, lane);
            if (more) {
                la.store(As[buf ^ 1]);
                if constexpr (kNf4) lb.store(Bs[buf ^ 1], Bq, p.absmax, p.nf4_cols, n0, kn, p.N, p.K, lut);
                else lb.store(Bs[buf ^ 1]);
            }
            __syncthreads();
            buf ^= 1;
        }
    }
    if constexpr (kNf4) {
        if (p.K2 > 0 && split == p.splits - 1) {
            RowLoader<BM, NT> la;
            typename std::conditional<BKIND == B_NF4_NT, RowLoader<BN, NT>, TransLoader<BN, NT>>::type lb;
            for (int k0 = 0; k0 < p.K2; k0 += BK) {
                la.load(p.A2, p.lda2, m0, k0, p.M, p.K2, p.a2_vec);
                lb.load(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec);
                la.store(As[0]);
                lb.store(Bs[0]);
                __syncthreads();
                mma_chunk<TE, WM, WN>(As[0], Bs[0], acc, wm, wn, lane);
                __syncthreads();
            }
        }
    }

    // epilogue: each wavefront stages one 16-row band of its sub-tile in LDS
    // (static register indexing), then every lane writes 16 consecutive
    // columns of one row (vector stores where the layout allows).
    __syncthreads();
    float* stage = reinterpret_cast<float*>(&As[0][0]) + wave * (16 * (WN + 4));
    const int srow = lane / (64 / 16) % 16;                 // 0..15
    const int scol = (lane % (64 / 16)) * (WN / 4);          // WN/4 columns per lane
#pragma unroll
    for (int i = 0; i < WM / 16; ++i) {
#pragma unroll
        for (int j = 0; j < WN / 16; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                stage[((lane >> 4) * 4 + e) * (WN + 4) + j * 16 + (lane & 15)] = acc[i][j][e];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row = m0 + wm * WM + i * 16 + srow;
        const int col0 = n0 + wn * WN + scol;
        if (WN == 64 && p.ce_mode) {  // every lane: the row's 4 lanes combine
            ce_epilogue(p, row, col0, stage + srow * (WN + 4) + scol);
        } else if (row < p.M) {
            const float* src = stage + srow * (WN + 4) + scol;
            if (p.splits > 1) {
                float* dst = p.partial + (int64_t(split) * p.M + row) * p.N + col0;
                if (col0 + WN / 4 <= p.N && (p.N & 3) == 0) {
#pragma unroll
                    for (int c = 0; c < WN / 4; c += 4)
                        *reinterpret_cast<float4*>(dst + c) = make_float4(src[c], src[c + 1], src[c + 2], src[c + 3]);
                } else {
                    for (int c = 0; c < WN / 4; ++c)
                        if (col0 + c < p.N) dst[c] = src[c];
                }
            } else {
                store_row(p, bo, bi, row, col0, src, WN / 4);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ---------------------------------------------------------------------------
// Full-tile NF4 kernel (M % 256 == 0, N % 128 == 0, K % 64 == 0, 16-byte
// aligned operands, NF4 rows a whole number of absmax blocks): a 256 x 128
// tile on 8 wavefronts (4 x 2, two per SIMD) of 64 x 64, so one wavefront's
// dequantization and LDS traffic overlaps the other's MFMAs.
//
// Every global read goes straight into LDS (global_load_lds): per 64-wide K
// chunk the A tile (32 KB), the weight tile's packed codes (4 KB) and its
// absmax values (512 B). A runs two chunks ahead and the codes three, in
// three LDS stages each, so a stage has about two chunks of MFMA time to
// arrive; the waits are explicit vmcnt counts that leave the newer stages in
// flight (the compiler's own barrier would wait for everything). Each DMA
// address is a wavefront-uniform base (scalar registers, advanced once per
// chunk) plus a per-lane 32-bit offset computed once, so the loop spends no
// vector instructions on addressing. During chunk t's MFMAs each thread
// dequantizes 16 elements of chunk t+1: one LDS read of the packed codes, one
// 8-byte LDS lookup per code byte in a 256-entry table of value pairs (at LDS
// address 0, so the address is the byte times 8), two fp32 multiplies by the
// block absmax and one paired bf16 conversion, then 16-byte LDS writes into
// the swizzled bf16 tile. LDS tiles are unpadded; the 16-byte chunk c of row
// r is stored at chunk c ^ ((r >> 1) & 7), so fragment reads are
// conflict-free and each fragment address is a per-lane base plus an
// immediate offset.
namespace fast {
constexpr int BM = 256, BN = 128, NTH = 512, NW = 8, WGN = 2, WM = 64, WN = 64, FI = WM / 16, FJ = WN / 16;
constexpr int SA = BM * 64 * 2, SB = BN * 64 * 2, SR = BN * 32, SS = 512;  // bytes per stage
constexpr int OFF_L = 0, OFF_A = 256 * 8, OFF_B = OFF_A + 3 * SA, OFF_R = OFF_B + 3 * SB, OFF_S = OFF_R + 3 * SR;
constexpr int LDS_BYTES = OFF_S + 3 * SS;
static_assert(LDS_BYTES <= 160 * 1024, "fast NF4 tile exceeds LDS");
constexpr int NA = BM / 8 / NW;  // 16-byte A DMAs per thread per chunk
constexpr int NR = 2;            // code + absmax DMAs per thread per chunk

typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

// s_waitcnt vmcnt(VM) lgkmcnt(0), then a workgroup barrier that does not
// drain the DMA queue (the "memory" clobber keeps LDS accesses on their side)
template <int VM>
__device__ __forceinline__ void stage_sync() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (0x7 << 4));
    asm volatile("s_barrier" ::: "memory");
}

// Per-lane DMA offsets (bytes, fixed for the whole K loop) into three buffer
// resources based at the tile's chunk-0 origin; a chunk adds a uniform
// scalar offset, so the DMAs cost no vector instructions.
//  A tile (256 rows x 64 k, bf16): each wavefront moves 4 KB in four 1 KB
//  instructions; lane l of one instruction lands at byte 16 l of its 1 KB
//  block, so it fetches the 16 bytes that belong in that slot of the
//  swizzled layout.
//  Codes, in natural order: NT [128 n][32 B] with one absmax per row; NN
//  [64 k][64 B] with two absmax per row. Every wavefront issues exactly one
//  16-byte DMA (32 lanes) and one 4-byte DMA (16 lanes), so the
//  per-wavefront vmcnt bookkeeping is the same everywhere.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t as_lds(char* p) {
    return reinterpret_cast<lds_ptr_t>(reinterpret_cast<uintptr_t>(p));
}
// raw buffer: stride 0, 2 GiB range (every offset used here is far below),
// the gfx9 default data format word
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
template <int BKIND>
struct DmaPlan {
    uint32_t a[NA];
    uint32_t code, scale;
    int wave;  // wavefront-uniform
    __amdgpu_buffer_rsrc_t ra, rc, rs;
    __device__ __forceinline__ void init(const void* a0, const void* c0, const void* s0, int64_t lda, int64_t cols) {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        ra = rsrc(a0);
        rc = rsrc(c0);
        rs = rsrc(s0);
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int r = (wave * NA + u) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            a[u] = uint32_t((int64_t(r) * lda + c * 8) * 2);
        }
        const int q = wave * 32 + (lane & 31), qs = wave * 16 + (lane & 15);
        if constexpr (BKIND == B_NF4_NN) {
            code = uint32_t(int64_t(q >> 2) * (cols >> 1) + (q & 3) * 16);
            scale = uint32_t((int64_t(qs >> 1) * (cols >> 6) + (qs & 1)) * 4);
        } else {
            code = uint32_t(int64_t(q >> 1) * (cols >> 1) + (q & 1) * 16);
            scale = uint32_t(int64_t(qs) * (cols >> 6) * 4);
        }
    }
    __device__ __forceinline__ void a_dma(uint32_t soff, char* __restrict__ dst) const {
#pragma unroll
        for (int u = 0; u < NA; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, as_lds(dst + (wave * NA + u) * 1024), 16, a[u], soff, 0, 0);
    }
    __device__ __forceinline__ void code_dma(uint32_t coff, uint32_t soff, char* __restrict__ raw,
                                             char* __restrict__ sc) const {
        const int lane = threadIdx.x & 63;
        if (lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, as_lds(raw + wave * 512), 16, code, coff, 0, 0);
        if (lane < 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, as_lds(sc + wave * 64), 4, scale, soff, 0, 0);
    }
};

// Codes of one chunk (LDS) -> bf16 tile [n][k] (LDS). lut2[b] (LDS address
// 8 b) holds the code values of byte b's high nibble (the even element) and
// low nibble.
template <int BKIND>
__device__ __forceinline__ void dequant(const char* __restrict__ raw, const char* __restrict__ sc,
                                        const char* __restrict__ lds0, uint16_t* __restrict__ tile) {
    const int t = threadIdx.x;
    const float* s = reinterpret_cast<const float*>(sc);
    auto lut = [&](uint32_t byte) { return *reinterpret_cast<const f2*>(lds0 + OFF_L + (byte << 3)); };
    if constexpr (BKIND == B_NF4_NT) {
        // thread = 16 consecutive k of row t >> 2
        const int r = t >> 2, q4 = t & 3;
        const uint2 w = *reinterpret_cast<const uint2*>(raw + r * 32 + q4 * 8);
        const float a = s[r];
        uint32_t e[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const f2 v = lut(((b < 4 ? w.x : w.y) >> (8 * (b & 3))) & 0xFF);
            e[b] = f32x2_to_bf16x2(v.x * a, v.y * a);
        }
        *reinterpret_cast<uint4*>(tile + swz(r, 2 * q4)) = make_uint4(e[0], e[1], e[2], e[3]);
        *reinterpret_cast<uint4*>(tile + swz(r, 2 * q4 + 1)) = make_uint4(e[4], e[5], e[6], e[7]);
    } else {
        // thread = 4 consecutive n x 4 consecutive k; pairs along k convert together
        const int ng = (t & 31) * 4, kg = (t >> 5) * 4;
        f2 v[4][2];
        float a[4];
#pragma unroll
        for (int kr = 0; kr < 4; ++kr) {
            const uint32_t two = *reinterpret_cast<const uint16_t*>(raw + (kg + kr) * 64 + (ng >> 1));
            a[kr] = s[(kg + kr) * 2 + (ng >> 6)];
            v[kr][0] = lut(two & 0xFF);
            v[kr][1] = lut(two >> 8);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float x[4];
#pragma unroll
            for (int kr = 0; kr < 4; ++kr) x[kr] = ((j & 1) ? v[kr][j >> 1].y : v[kr][j >> 1].x) * a[kr];
            *reinterpret_cast<uint2*>(tile + swz(ng + j, kg >> 3) + (kg & 4)) =
                make_uint2(f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3]));
        }
    }
}

// One 64-wide chunk of MFMAs for a (16 FI_) x (16 FJ_) wavefront tile. Row
// (base + i*16 + lr) swizzles with (lr >> 1) & 7 only, so each K half has one
// per-lane base.
template <int FI_, int FJ_, int TE_ = TE_BF16>
__device__ __forceinline__ void mma(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                    f32x4 (&acc)[FI_][FJ_], int rm, int rn, int lane) {
    const int lr = lane & 15, lc = lane >> 4, sw = (lr >> 1) & 7;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int ch = ((kk * 4 + lc) ^ sw) << 3;
        const uint16_t* ab = As + (rm + lr) * 64 + ch;
        const uint16_t* bb = Bs + (rn + lr) * 64 + ch;
        uint4 a[FI_], b[FJ_];
#pragma unroll
        for (int i = 0; i < FI_; ++i) a[i] = *reinterpret_cast<const uint4*>(ab + i * 16 * 64);
#pragma unroll
        for (int j = 0; j < FJ_; ++j) b[j] = *reinterpret_cast<const uint4*>(bb + j * 16 * 64);
#pragma unroll
        for (int i = 0; i < FI_; ++i)
#pragma unroll
            for (int j = 0; j < FJ_; ++j) acc[i][j] = mfma16<TE_>(a[i], b[j], acc[i][j]);
    }
}

// LoRA slab of a full tile (last split only): K2 in 64-wide chunks through
// the 64-wide swizzled layout at As (BM_ rows) and Bs (BN_ rows), zero-filled
// past K2. The caller has drained every DMA and barriered.
template <int BKIND, int BM_, int BN_, int FI_, int FJ_>
__device__ __forceinline__ void slab(const GemmParams& p, uint16_t* As, uint16_t* Bs, f32x4 (&acc)[FI_][FJ_], int m0,
                                     int n0, int rm, int rn, int lane) {
    for (int k0 = 0; k0 < p.K2; k0 += 64) {
        RowLoader<BM_, NTH, true> la;
        la.load(p.A2, p.lda2, m0, k0, p.M, p.K2, p.a2_vec);
        if constexpr (BKIND == B_NF4_NT) {
            RowLoader<BN_, NTH, true> lb;
            lb.load(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec);
            lb.store(Bs);
        } else {
            TransLoader<BN_, NTH, true> lb;
            lb.load(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec);
            lb.store(Bs);
        }
        la.store(As);
        __syncthreads();
        mma(As, Bs, acc, rm, rn, lane);
        __syncthreads();
    }
}

// Epilogue of a full tile: each wavefront stages 16-row bands of its
// (16 FI_) x WN_ tile through LDS (stage: 16 x (WN_ + 4) floats of its own),
// then each lane writes WN_/4 consecutive columns of one row: fp32 partials
// when split, the GEMM's output otherwise.
template <int FI_, int WN_, bool CE = false>
__device__ __forceinline__ void epilogue(const GemmParams& p, const f32x4 (&acc)[FI_][WN_ / 16], float* stage, int row0,
                                         int col0, int split, int lane) {
    const int srow = (lane >> 2) & 15;
    const int scol = (lane & 3) * (WN_ / 4);
#pragma unroll
    for (int i = 0; i < FI_; ++i) {
#pragma unroll
        for (int j = 0; j < WN_ / 16; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) stage[((lane >> 4) * 4 + e) * (WN_ + 4) + j * 16 + (lane & 15)] = acc[i][j][e];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row = row0 + i * 16 + srow;
        const int col = col0 + scol;
        const float* src = stage + srow * (WN_ + 4) + scol;
        if constexpr (CE) {
            ce_epilogue(p, row, col, src);
        } else if (p.splits > 1) {
            float* dst = p.partial + (int64_t(split) * p.M + row) * p.N + col;
#pragma unroll
            for (int c = 0; c < WN_ / 4; c += 4)
                *reinterpret_cast<float4*>(dst + c) = make_float4(src[c], src[c + 1], src[c + 2], src[c + 3]);
        } else {
            store_row(p, 0, 0, row, col, src, WN_ / 4);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}
}  // namespace fast

template <int BKIND>
__global__ __launch_bounds__(fast::NTH) void k_nf4_tile(const GemmParams p) {
    using namespace fast;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    if (tid < 256) reinterpret_cast<f2*>(lds + OFF_L)[tid] = f2{nf4_value(tid >> 4), nf4_value(tid & 15)};

    const int gx = p.N / BN, gy = p.M / BM;
    const int ntile = gx * gy;
    int t = blockIdx.x;
    if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
    const int m0 = (t / gx) * BM, n0 = (t % gx) * BN;  // the gx N-tiles of one M-tile together
    const int split = blockIdx.y;
    const int kbeg = split * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    const int nch = (kend - kbeg) / 64;  // >= 1
    const int64_t cols = p.nf4_cols;

    // chunk-0 origins; per chunk A moves 128 bytes, the codes 32 bytes (NT)
    // or 64 rows (NN), the absmax 1 entry (NT) or 64 rows (NN)
    const int64_t flat0 = (BKIND == B_NF4_NN) ? int64_t(kbeg) * cols + n0 : int64_t(n0) * cols + kbeg;
    DmaPlan<BKIND> plan;
    plan.init(p.A + int64_t(m0) * p.lda + kbeg, static_cast<const char*>(p.B) + (flat0 >> 1), p.absmax + (flat0 >> 6),
              p.lda, cols);
    const uint32_t cstep = (BKIND == B_NF4_NN) ? uint32_t(32 * cols) : 32u;
    const uint32_t sstep = (BKIND == B_NF4_NN) ? uint32_t(4 * cols) : 4u;  // bytes

    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk c reads A stage c % 3 and bf16 stage c % 3; loads past the end
    // re-read the last chunk into stages nobody reads again
    auto cl = [&](int c) { return min(c, nch - 1); };
    auto sa = [&](int s) { return lds + OFF_A + s * SA; };
    auto sb = [&](int s) { return reinterpret_cast<uint16_t*>(lds + OFF_B + s * SB); };
    auto sr = [&](int s) { return lds + OFF_R + s * SR; };
    auto ss = [&](int s) { return lds + OFF_S + s * SS; };
    auto a_dma = [&](int c, int s) { plan.a_dma(uint32_t(cl(c)) * 128u, sa(s)); };
    auto code_dma = [&](int c, int s) { plan.code_dma(uint32_t(cl(c)) * cstep, uint32_t(cl(c)) * sstep, sr(s), ss(s)); };
    code_dma(0, 0);
    a_dma(0, 0);
    code_dma(1, 1);
    a_dma(1, 1);
    code_dma(2, 2);
    stage_sync<2 * NA + 2 * NR>();  // codes 0 (and the table) in LDS
    dequant<BKIND>(sr(0), ss(0), lds, sb(0));
    stage_sync<NA + NR>();          // A 0, codes 1, bf16 0
    auto step = [&](int c, auto stage) {
        constexpr int S0 = decltype(stage)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
        a_dma(c + 2, S2);
        code_dma(c + 3, S0);
        mma(reinterpret_cast<const uint16_t*>(sa(S0)), sb(S0), acc, wm * WM, wn * WN, lane);
        dequant<BKIND>(sr(S1), ss(S1), lds, sb(S1));
        stage_sync<NA + NR>();      // A c+1, codes c+2, bf16 c+1
    };
    for (int c = 0; c < nch; c += 3) {
        step(c, std::integral_constant<int, 0>());
        if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
        if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
    }
    stage_sync<0>();

    if (p.K2 > 0 && split == p.splits - 1)  // LoRA slab, any K2 (zero-filled tail)
        slab<BKIND, BM, BN>(p, reinterpret_cast<uint16_t*>(sa(0)), sb(0), acc, m0, n0, wm * WM, wn * WN, lane);
    epilogue<FI, WN>(p, acc, reinterpret_cast<float*>(lds + OFF_A) + wave * (16 * (WN + 4)), m0 + wm * WM,
                     n0 + wn * WN, split, lane);
}

// ---------------------------------------------------------------------------
// Full-tile dense NT kernel for the LM head's fp16 products with the
// cross-entropy epilogues (M % 256 == 0, N % 128 == 0, K % 64 == 0, 16-byte
// aligned rows): the NF4 tile's pipeline with the weight tile fetched like the
// activations. Per 64-wide K chunk each wavefront moves 4 KB of the 256-row A
// tile and 2 KB of the 128-row B tile straight into LDS (global_load_lds, a
// per-lane offset computed once plus a scalar offset per chunk), both two
// chunks ahead in three stages; the same explicit partial waits, the same
// XOR-swizzled unpadded tiles and 8 wavefronts of 64 x 64.
namespace dense {
using fast::BM;
using fast::BN;
using fast::NTH;
using fast::NW;
using fast::WGN;
using fast::WM;
using fast::WN;
using fast::FI;
using fast::FJ;
using fast::SA;
using fast::SB;
constexpr int OFF_A = 0, OFF_B = 3 * SA, LDS_BYTES = OFF_B + 3 * SB;
static_assert(LDS_BYTES <= 160 * 1024, "dense tile exceeds LDS");
constexpr int NA = BM / 8 / NW, NB = BN / 8 / NW;  // 1 KB DMAs per wavefront per chunk
struct Plan {
    uint32_t a[NA], b[NB];
    int wave;
    __amdgpu_buffer_rsrc_t ra, rb;
    // lane l of a 1 KB block lands at byte 16 l: row (block row 0) + (l >> 3),
    // slot l & 7, which holds the row's global chunk (l & 7) ^ ((row >> 1) & 7)
    __device__ __forceinline__ void init(const void* a0, const void* b0, int64_t lda, int64_t ldb) {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        ra = fast::rsrc(a0);
        rb = fast::rsrc(b0);
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int r = (wave * NA + u) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            a[u] = uint32_t((int64_t(r) * lda + c * 8) * 2);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int r = (wave * NB + u) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            b[u] = uint32_t((int64_t(r) * ldb + c * 8) * 2);
        }
    }
    __device__ __forceinline__ void dma(uint32_t soff, char* __restrict__ da, char* __restrict__ db) const {
#pragma unroll
        for (int u = 0; u < NA; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, fast::as_lds(da + (wave * NA + u) * 1024), 16, a[u], soff, 0,
                                                     0);
#pragma unroll
        for (int u = 0; u < NB; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, fast::as_lds(db + (wave * NB + u) * 1024), 16, b[u], soff, 0,
                                                     0);
    }
};
}  // namespace dense

template <int TE>
__global__ __launch_bounds__(dense::NTH) void k_dense_tile(const GemmParams p) {
    using namespace dense;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int gx = p.N / BN, gy = p.M / BM;
    const int ntile = gx * gy;
    int t = blockIdx.x;
    if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
    const int m0 = (t % gy) * BM, n0 = (t / gy) * BN;  // the gy M-tiles of one weight tile together
    const int nch = p.K / 64;  // >= 1
    Plan plan;
    plan.init(p.A + int64_t(m0) * p.lda, static_cast<const uint16_t*>(p.B) + int64_t(n0) * p.ldb, p.lda, p.ldb);

    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk c goes to stage c % 3; DMAs past the end re-read the last chunk
    // into a stage nobody reads again, so every step issues the same count
    auto sa = [&](int st) { return lds + OFF_A + st * SA; };
    auto sb = [&](int st) { return lds + OFF_B + st * SB; };
    auto dma = [&](int c, int st) { plan.dma(uint32_t(min(c, nch - 1)) * 128u, sa(st), sb(st)); };
    dma(0, 0);
    dma(1, 1);
    fast::stage_sync<NA + NB>();  // chunk 0 in LDS
    auto step = [&](int c, auto stage) {
        constexpr int S0 = decltype(stage)::value, S2 = (S0 + 2) % 3;
        dma(c + 2, S2);  // S2 was last read by chunk c - 1, finished before the last barrier
        fast::mma<FI, FJ, TE>(reinterpret_cast<const uint16_t*>(sa(S0)), reinterpret_cast<const uint16_t*>(sb(S0)),
                              acc, wm * WM, wn * WN, lane);
        fast::stage_sync<NA + NB>();  // chunk c + 1 in LDS, c + 2 in flight
    };
    for (int c = 0; c < nch; c += 3) {
        step(c, std::integral_constant<int, 0>());
        if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
        if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
    }
    fast::stage_sync<0>();
    fast::epilogue<FI, WN, true>(p, acc, reinterpret_cast<float*>(lds + OFF_A) + wave * (16 * (WN + 4)),
                                 m0 + wm * WM, n0 + wn * WN, 0, lane);
}

// ---------------------------------------------------------------------------
// Wide NF4 tile (M % 512 == 0, otherwise as the full tile): 512 x 128 on 8
// wavefronts (4 x 2) of 128 x 64, in K chunks of 32. Each dequantized weight
// tile now serves 512 rows and each wavefront's fragment reads feed twice the
// MFMAs, so LDS traffic per MFMA falls by about a third; the price is half as
// many tiles, which pays where the 256 x 128 grid would leave part of a round
// idle (the launcher decides from the shapes). The pipeline is the full
// tile's: A two chunks ahead, codes three, explicit partial waits, scalar DMA
// offsets, table lookups from LDS address 0. Rows are 64 bytes here, with
// 16-byte chunk c of row r at c ^ ((r >> 2) & 3).
namespace wide {
constexpr int BM = 512, BN = 128, BKW = 32, NTH = 512, WGN = 2, WM = 128, WN = 64, FI = WM / 16, FJ = WN / 16;
constexpr int SA = BM * BKW * 2, SB = BN * BKW * 2, SR = BN * BKW / 2, SS = 512;  // bytes per stage
constexpr int OFF_L = 0, OFF_A = 256 * 8, OFF_B = OFF_A + 3 * SA, OFF_R = OFF_B + 3 * SB, OFF_S = OFF_R + 3 * SR;
constexpr int LDS_BYTES = OFF_S + 3 * SS;
static_assert(LDS_BYTES <= 160 * 1024, "wide NF4 tile exceeds LDS");
static_assert(3 * SA >= BM * 64 * 2 && 3 * SB >= BN * 64 * 2, "slab tiles must fit the stage regions");
constexpr int NA = SA / 1024 / 8;  // 1 KB A DMAs per wavefront per chunk
constexpr int NR = 2;
typedef float f2 __attribute__((ext_vector_type(2)));
// 64-byte rows of four 16-byte chunks; chunk c of row r at c ^ ((r >> 2) & 3)
__device__ __forceinline__ int swz(int r, int c) { return r * 32 + ((c ^ ((r >> 2) & 3)) << 3); }
template <int BKIND>
struct Plan {
    uint32_t a[NA];
    uint32_t code, scale;
    int wave;
    __amdgpu_buffer_rsrc_t ra, rc, rs;
    __device__ __forceinline__ void init(const void* a0, const void* c0, const void* s0, int64_t lda, int64_t cols) {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        ra = fast::rsrc(a0); rc = fast::rsrc(c0); rs = fast::rsrc(s0);
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int r = (wave * NA + u) * 16 + (lane >> 2);   // 1 KB = 16 rows x 64 B
            const int c = (lane & 3) ^ ((r >> 2) & 3);
            a[u] = uint32_t((int64_t(r) * lda + c * 8) * 2);
        }
        const int q = wave * 16 + (lane & 15);                  // 128 x 16-byte code pieces
        const int qs = (BKIND == B_NF4_NN) ? wave * 8 + (lane & 7) : wave * 16 + (lane & 15);
        if constexpr (BKIND == B_NF4_NN) {
            code = uint32_t(int64_t(q >> 2) * (cols >> 1) + (q & 3) * 16);       // 32 k-rows x 64 B
            scale = uint32_t((int64_t(qs >> 1) * (cols >> 6) + (qs & 1)) * 4);  // 32 rows x 2 (lanes < 8)
        } else {
            code = uint32_t(int64_t(q) * (cols >> 1));                          // 128 rows x 16 B
            scale = uint32_t(int64_t(qs) * (cols >> 6) * 4);                     // 128 rows x 1
        }
    }
    __device__ __forceinline__ void a_dma(uint32_t soff, char* __restrict__ dst) const {
#pragma unroll
        for (int u = 0; u < NA; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, fast::as_lds(dst + (wave * NA + u) * 1024), 16, a[u], soff, 0, 0);
    }
    __device__ __forceinline__ void code_dma(uint32_t coff, uint32_t soff, char* __restrict__ raw, char* __restrict__ sc) const {
        const int lane = threadIdx.x & 63;
        if (lane < 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, fast::as_lds(raw + wave * 256), 16, code, coff, 0, 0);
        if (lane < (BKIND == B_NF4_NN ? 8 : 16))
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, fast::as_lds(sc + wave * (BKIND == B_NF4_NN ? 32 : 64)), 4, scale, soff, 0, 0);
    }
};
template <int BKIND>
__device__ __forceinline__ void dequant(const char* __restrict__ raw, const char* __restrict__ sc, const char* __restrict__ lds0,
                                        uint16_t* __restrict__ tile) {
    const int t = threadIdx.x;
    const float* s = reinterpret_cast<const float*>(sc);
    auto lut = [&](uint32_t byte) { return *reinterpret_cast<const f2*>(lds0 + OFF_L + (byte << 3)); };
    if constexpr (BKIND == B_NF4_NT) {
        const int r = t >> 2, q4 = t & 3;                        // 8 consecutive k of row r
        const uint32_t w = *reinterpret_cast<const uint32_t*>(raw + r * 16 + q4 * 4);
        const float a = s[r];
        uint32_t e[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f2 v = lut((w >> (8 * b)) & 0xFF);
            e[b] = f32x2_to_bf16x2(v.x * a, v.y * a);
        }
        *reinterpret_cast<uint4*>(tile + swz(r, q4)) = make_uint4(e[0], e[1], e[2], e[3]);
    } else {
        const int ng = (t & 63) * 2, kg = (t >> 6) * 4;            // 2 n x 4 k
        f2 v[4];
        float a[4];
#pragma unroll
        for (int kr = 0; kr < 4; ++kr) {
            const uint32_t byte = *reinterpret_cast<const uint8_t*>(raw + (kg + kr) * 64 + (ng >> 1));
            a[kr] = s[(kg + kr) * 2 + (ng >> 6)];
            v[kr] = lut(byte);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float x[4];
#pragma unroll
            for (int kr = 0; kr < 4; ++kr) x[kr] = (j ? v[kr].y : v[kr].x) * a[kr];
            *reinterpret_cast<uint2*>(tile + swz(ng + j, kg >> 3) + (kg & 4)) =
                make_uint2(f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3]));
        }
    }
}
__device__ __forceinline__ void mma(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs, f32x4 (&acc)[FI][FJ],
                                    int rm, int rn, int lane) {
    const int lr = lane & 15, lc = lane >> 4;
    // rows rm + i*16 + lr: (row >> 2) & 3 == (lr >> 2) & 3 since rm, i*16 are multiples of 16
    const int ch = (lc ^ ((lr >> 2) & 3)) << 3;
    const uint16_t* ab = As + (rm + lr) * 32 + ch;
    const uint16_t* bb = Bs + (rn + lr) * 32 + ch;
    uint4 a[FI], b[FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i) a[i] = *reinterpret_cast<const uint4*>(ab + i * 16 * 32);
#pragma unroll
    for (int j = 0; j < FJ; ++j) b[j] = *reinterpret_cast<const uint4*>(bb + j * 16 * 32);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = mfma16<TE_BF16>(a[i], b[j], acc[i][j]);
}
}  // namespace wide

template <int BKIND>
__global__ __launch_bounds__(wide::NTH) void k_nf4_wide(const GemmParams p) {
    using namespace wide;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    if (tid < 256) reinterpret_cast<f2*>(lds + OFF_L)[tid] = f2{nf4_value(tid >> 4), nf4_value(tid & 15)};
    const int gx = p.N / BN, gy = p.M / BM;
    const int ntile = gx * gy;
    int t = blockIdx.x;
    if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
    const int m0 = (t / gx) * BM, n0 = (t % gx) * BN;  // the gx N-tiles of one M-tile together
    const int split = blockIdx.y;
    const int kbeg = split * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    const int nch = (kend - kbeg) / BKW;
    const int64_t cols = p.nf4_cols;
    const int64_t flat0 = (BKIND == B_NF4_NN) ? int64_t(kbeg) * cols + n0 : int64_t(n0) * cols + kbeg;
    Plan<BKIND> plan;
    plan.init(p.A + int64_t(m0) * p.lda + kbeg, static_cast<const char*>(p.B) + (flat0 >> 1), p.absmax + (flat0 >> 6), p.lda, cols);
    // per 32-wide chunk: A 64 bytes; codes 16 bytes (NT) or 32 rows (NN); absmax: NT advances every
    // other chunk (64-element blocks), NN 32 rows
    const uint32_t cstep = (BKIND == B_NF4_NN) ? uint32_t(16 * cols) : 16u;
    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto cl = [&](int c) { return min(c, nch - 1); };
    auto soff = [&](int c) { return (BKIND == B_NF4_NN) ? uint32_t(cl(c)) * uint32_t(2 * cols) : uint32_t(cl(c) >> 1) * 4u; };
    auto sa = [&](int s) { return lds + OFF_A + s * SA; };
    auto sb = [&](int s) { return reinterpret_cast<uint16_t*>(lds + OFF_B + s * SB); };
    auto sr = [&](int s) { return lds + OFF_R + s * SR; };
    auto ss = [&](int s) { return lds + OFF_S + s * SS; };
    auto a_dma = [&](int c, int s) { plan.a_dma(uint32_t(cl(c)) * 64u, sa(s)); };
    auto code_dma = [&](int c, int s) { plan.code_dma(uint32_t(cl(c)) * cstep, soff(c), sr(s), ss(s)); };
    code_dma(0, 0);
    a_dma(0, 0);
    code_dma(1, 1);
    a_dma(1, 1);
    code_dma(2, 2);
    fast::stage_sync<2 * NA + 2 * NR>();
    dequant<BKIND>(sr(0), ss(0), lds, sb(0));
    fast::stage_sync<NA + NR>();
    auto step = [&](int c, auto stage) {
        constexpr int S0 = decltype(stage)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
        a_dma(c + 2, S2);
        code_dma(c + 3, S0);
        mma(reinterpret_cast<const uint16_t*>(sa(S0)), sb(S0), acc, wm * WM, wn * WN, lane);
        dequant<BKIND>(sr(S1), ss(S1), lds, sb(S1));
        fast::stage_sync<NA + NR>();
    };
    for (int c = 0; c < nch; c += 3) {
        step(c, std::integral_constant<int, 0>());
        if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
        if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
    }
    fast::stage_sync<0>();
    if (p.K2 > 0 && split == p.splits - 1)  // slab tiles are 64 wide: A2 spans two A stages, B2 two B stages
        fast::slab<BKIND, BM, BN>(p, reinterpret_cast<uint16_t*>(sa(0)), sb(0), acc, m0, n0, wm * WM, wn * WN, lane);
    fast::epilogue<FI, WN>(p, acc, reinterpret_cast<float*>(lds + OFF_A) + wave * (16 * (WN + 4)), m0 + wm * WM,
                           n0 + wn * WN, split, lane);
}

// Sums the split-K partials in split order (fixed, so results do not depend
// on timing). Four consecutive outputs per thread when N % 4 == 0.
__global__ __launch_bounds__(256) void k_splitk_reduce(const GemmParams p) {
    const int64_t MN = int64_t(p.M) * p.N;
    if ((p.N & 3) == 0) {
        const int64_t idx = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
        if (idx >= MN) return;
        const float4* src = reinterpret_cast<const float4*>(p.partial + idx);
        const int64_t st = MN / 4;
        auto add = [](float4& a, const float4& b) {
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        };
        float4 v = src[0];
        int s = 1;
        for (; s + 4 <= p.splits; s += 4) {  // four loads in flight, added in split order
            const float4 w0 = src[s * st], w1 = src[(s + 1) * st], w2 = src[(s + 2) * st], w3 = src[(s + 3) * st];
            add(v, w0);
            add(v, w1);
            add(v, w2);
            add(v, w3);
        }
        for (; s < p.splits; ++s) add(v, src[s * st]);
        const int row = int(idx / p.N), col = int(idx % p.N);
        store_out(p, 0, 0, row, col, v.x);
        store_out(p, 0, 0, row, col + 1, v.y);
        store_out(p, 0, 0, row, col + 2, v.z);
        store_out(p, 0, 0, row, col + 3, v.w);
        return;
    }
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= MN) return;
    float v = 0.f;
    for (int s = 0; s < p.splits; ++s) v += p.partial[s * MN + idx];
    store_out(p, 0, 0, int(idx / p.N), int(idx % p.N), v);
}

// ---------------------------------------------------------------------------
struct TileCfg {
    int bm, bn;
};

template <int AK, int BKIND, int TE, int BM, int BN, int WM, int WN>
static void launch_cfg(const GemmParams& p, int batch_splits, hipStream_t s) {
    const int gx = (p.N + BN - 1) / BN, gy = (p.M + BM - 1) / BM;
    hipLaunchKernelGGL((k_gemm<AK, BKIND, TE, BM, BN, WM, WN>), dim3(gx * gy, batch_splits),
                       dim3((BM / WM) * (BN / WN) * 64), 0, s, p);
}

// Tile shapes: NF4 GEMMs with at least 512 rows use 256 x 128 (each weight
// tile is dequantized half as often per MFMA); everything else 128 x 128.
static TileCfg pick_tile(const GemmParams& p, int bkind) {
    const bool nf4 = (bkind == B_NF4_NT || bkind == B_NF4_NN);
    if (nf4 && p.M >= 512) return {256, 128};
    return {128, 128};
}

template <int AK, int BKIND, int TE>
static void launch_kind(const GemmParams& p, TileCfg tc, int batch_splits, hipStream_t s) {
    if (tc.bm == 256) launch_cfg<AK, BKIND, TE, 256, 128, 128, 64>(p, batch_splits, s);
    else launch_cfg<AK, BKIND, TE, 128, 128, 64, 64>(p, batch_splits, s);
}

static bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

// The full-tile kernels take up to 160 KB of dynamic LDS, which each device
// has to allow once per kernel before the first launch. The flags are atomic:
// host threads racing on a first launch at worst repeat the idempotent call.
static void allow_lds(std::atomic<bool> (&allowed)[64], const void* fn, int bytes) {
    int dev = 0;
    QLX_CHECK_HIP(hipGetDevice(&dev));
    QLX_REQUIRE(dev >= 0 && dev < 64, QLX_EUNSUPPORTED, "gemm: device index out of range");
    if (!allowed[dev].load(std::memory_order_acquire)) {
        QLX_CHECK_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes));
        allowed[dev].store(true, std::memory_order_release);
    }
}
template <int BKIND>
static void launch_fast(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_nf4_tile<BKIND>), fast::LDS_BYTES);
    hipExtLaunchKernelGGL(k_nf4_tile<BKIND>, dim3(tiles, p.splits), dim3(fast::NTH), fast::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p);
}
template <int BKIND>
static void launch_wide(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_nf4_wide<BKIND>), wide::LDS_BYTES);
    hipExtLaunchKernelGGL(k_nf4_wide<BKIND>, dim3(tiles, p.splits), dim3(wide::NTH), wide::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p);
}
static void launch_dense(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_dense_tile<TE_F16>), dense::LDS_BYTES);
    hipExtLaunchKernelGGL(k_dense_tile<TE_F16>, dim3(tiles), dim3(dense::NTH), dense::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p);
}
static bool aligned8(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 7) == 0; }

void gemm(GemmParams p, int akind, int bkind, int te, float* partial_ws, hipStream_t s) {
    if (p.M <= 0 || p.N <= 0) return;
    const bool nf4 = (bkind == B_NF4_NT || bkind == B_NF4_NN);
    QLX_REQUIRE(!(p.K2 > 0 && !nf4), QLX_EINVAL, "gemm: the LoRA slab rides only on NF4 GEMMs");
    QLX_REQUIRE(!(te == TE_F16 && nf4), QLX_EINVAL, "gemm: NF4 operands are bf16");
    QLX_REQUIRE(!p.ce_mode || (te == TE_F16 && akind == A_ROW && bkind == B_DENSE_NT && p.batch == 1 &&
                               p.causal == CAUSAL_NONE && p.ce_seq > 0),
                QLX_EINVAL, "gemm: the cross-entropy epilogues take a plain fp16 NT product");
    if (p.ce_mode) partial_ws = nullptr;  // no split: the epilogue needs whole sums
    // vector-load eligibility (uniform per launch; depends on layout, not data)
    if (akind == A_ROW) p.a_vec = aligned16(p.A) && p.lda % 8 == 0 && p.a_so % 8 == 0 && p.a_si % 8 == 0;
    else p.a_vec = aligned8(p.A) && p.lda % 4 == 0 && p.a_so % 4 == 0 && p.a_si % 4 == 0;
    if (bkind == B_NF4_NT) p.b_vec = aligned16(p.B) && p.nf4_cols % 64 == 0;
    else if (bkind == B_NF4_NN) p.b_vec = aligned16(p.B) && p.nf4_cols % 64 == 0;
    else if (bkind == B_DENSE_NT) p.b_vec = aligned16(p.B) && p.ldb % 8 == 0 && p.b_so % 8 == 0 && p.b_si % 8 == 0;
    else p.b_vec = aligned8(p.B) && p.ldb % 4 == 0 && p.b_so % 4 == 0 && p.b_si % 4 == 0;
    if (p.seg_rows > 0)
        QLX_REQUIRE(p.batch == 1 && int64_t(p.M) <= 8 * int64_t(p.seg_rows), QLX_EINVAL,
                    "gemm: at most 8 output segments, no batching");
    for (int i = 0; i < 8; ++i) {
        if (p.bseg[i] == 0) continue;
        QLX_REQUIRE(bkind == B_DENSE_NN && p.seg_rows > 0 && p.seg_rows % 128 == 0 && p.bseg[i] % 4 == 0 &&
                        p.causal == CAUSAL_NONE,
                    QLX_EINVAL, "gemm: per-segment B offsets need a dense NN B and 128-row segments");
    }
    if (p.K2 > 0) {
        p.a2_vec = aligned16(p.A2) && p.lda2 % 8 == 0;
        p.b2_vec = (bkind == B_NF4_NT) ? (aligned16(p.B2) && p.ldb2 % 8 == 0) : (aligned8(p.B2) && p.ldb2 % 4 == 0);
    }
    const bool fast_ok = nf4 && te == TE_BF16 && akind == A_ROW && p.batch == 1 && p.causal == CAUSAL_NONE &&
                         p.M % fast::BM == 0 && p.N % fast::BN == 0 && p.K % 64 == 0 && p.K >= 64 && p.a_vec &&
                         p.b_vec && aligned16(p.absmax) && p.nf4_cols % 64 == 0 &&
                         int64_t(p.M) * p.lda * 2 < (int64_t(1) << 31) &&
                         int64_t(p.N) * p.K / 2 < (int64_t(1) << 31);  // never depends on the slab
    // Skinny dense products (the LoRA terms: one side is r, 2r or 3r) are
    // bound by reading the long operand; 64 x 64 tiles with a K split keep
    // many workgroups streaming it without a large partial buffer.
    const bool skinny = !nf4 && te == TE_BF16 && p.batch == 1 && p.causal == CAUSAL_NONE && std::min(p.M, p.N) <= 256;
    // the LM head's fp16 NT products with a cross-entropy epilogue (never split)
    const bool dense_fast = p.ce_mode && te == TE_F16 && akind == A_ROW && bkind == B_DENSE_NT && p.batch == 1 &&
                            p.M % dense::BM == 0 && p.N % dense::BN == 0 && p.K % 64 == 0 && p.K >= 64 && p.a_vec &&
                            p.b_vec && int64_t(dense::BM) * p.lda * 2 + int64_t(p.K) * 2 < (int64_t(1) << 31) &&
                            int64_t(dense::BN) * p.ldb * 2 + int64_t(p.K) * 2 < (int64_t(1) << 31);
    const TileCfg tc = fast_ok ? TileCfg{fast::BM, fast::BN}
                       : dense_fast ? TileCfg{dense::BM, dense::BN}
                       : skinny     ? TileCfg{64, 64}
                                    : pick_tile(p, bkind);
    const int gx = (p.N + tc.bn - 1) / tc.bn, gy = (p.M + tc.bm - 1) / tc.bm;
    // split-K when the grid would leave CUs idle: shapes decide, nothing else
    p.splits = 1;
    p.kchunk = ((p.K + BK - 1) / BK) * BK;
    int tiles = gx * gy;
    bool wide_tile = false;
    if (fast_ok) {
        // One workgroup fits a CU, so the grid runs in rounds of 256. Pick the
        // tile (256 x 128, or 512 x 128 when M allows) and split count with the
        // least estimated time, in units of one 64-wide chunk of a 256 x 128
        // tile: rounds x (chunks per split + ~3 of pipeline fill and epilogue)
        // x tile cost (1.85 for the wide tile: twice the work at ~8% better
        // throughput, fitted to the 8B-shaped projections; it must also win by
        // 3%) + the reduce pass (fp32 partials at ~4 TB/s, a chunk being
        // ~1.35 us, plus ~2 chunks of launch). Shapes decide, nothing else.
        const int nch = p.K / 64;
        const double mn = double(p.M) * p.N;
        double best = 1e300;
        int best_s = 1;
        for (int wide = 0; wide < 2; ++wide) {
            if (wide && p.M % wide::BM != 0) continue;
            const int bm = wide ? wide::BM : fast::BM;
            const int t = (p.M / bm) * (p.N / fast::BN);
            const double unit = wide ? 1.85 * 1.03 : 1.0;
            for (int sp = 1; sp <= 16 && nch / sp >= 4; ++sp) {
                if (sp > 1 && (!partial_ws || size_t(sp) * p.M * p.N > kGemmPartialFloats)) break;
                const int per = (nch + sp - 1) / sp;
                const double rounds = double((t * sp + 255) / 256);
                double cost = rounds * (per + 3.0) * unit;
                if (sp > 1) cost += mn * 4.0 * (sp + 1) / 4e12 / 1.35e-6 + 2.0;
                if (cost < best - 1e-9) best = cost, best_s = sp, wide_tile = wide;
            }
        }
        if (best_s > 1) {
            const int kc = (nch + best_s - 1) / best_s * 64;
            p.kchunk = kc;
            p.splits = (p.K + kc - 1) / kc;
            p.partial = partial_ws;
        }
        if (wide_tile) tiles = (p.M / wide::BM) * (p.N / fast::BN);
        } else if (skinny) {
        // measured on the 8B-shaped LoRA products: at least 512 workgroups
        // (four fit a CU), at most 2048 of K per split, at least 256
        if (partial_ws) {
            int sp = 1;
            while (sp < 16 && tiles * sp < 512) sp *= 2;
            while (sp < 16 && p.K / sp > 2048) sp *= 2;
            sp = std::min(sp, std::max(1, p.K / 256));
            while (sp > 1 && size_t(sp) * tiles * tc.bm * tc.bn > kGemmPartialFloats) sp /= 2;
            if (sp > 1) {
                const int kc = (((p.K + sp - 1) / sp) + BK - 1) / BK * BK;
                p.kchunk = kc;
                p.splits = (p.K + kc - 1) / kc;
                p.partial = partial_ws;
            }
        }
    } else if (p.batch == 1 && p.causal == CAUSAL_NONE && partial_ws && tiles < 256 && p.K >= 256) {
        // about one workgroup per CU (the NF4 tiles hold one workgroup per CU)
        int want = ((nf4 ? 256 : 512) + tiles - 1) / tiles;
        want = std::min(want, p.K / 128);
        want = std::min(want, 16);
        while (want > 1 && size_t(want) * tiles * tc.bm * tc.bn > kGemmPartialFloats) --want;
        if (want > 1) {
            const int kc = (((p.K + want - 1) / want) + BK - 1) / BK * BK;
            p.kchunk = kc;
            p.splits = (p.K + kc - 1) / kc;
            p.partial = partial_ws;
        }
    }
    QLX_REQUIRE(p.batch >= 1 && p.batch * p.splits <= 65535, QLX_EUNSUPPORTED, "gemm: grid too large");
    const int key = akind * 100 + bkind * 10 + te;
    // algorithmic work: multiply-adds actually needed (causal halves, no zero blocks)
    double pairs_k;
    const double M = p.M, N = p.N, K = p.K;
    if (p.causal == CAUSAL_SKIP_UPPER) pairs_k = (M * (M + 1) / 2) * K;
    else if (p.causal == CAUSAL_K_LE_M || p.causal == CAUSAL_K_GE_M) pairs_k = N * (M * (M + 1) / 2);
    else pairs_k = M * N * K;
    const double k2 = p.K2 > 0 ? (p.slab_alg_k >= 0 ? p.slab_alg_k : p.K2) : 0;
    const double flops = 2.0 * p.batch * (pairs_k + M * N * k2);
    const double belt = (te == TE_F16 || !nf4) ? 2.0 : 0.5 + 4.0 / 64.0;
    const double cb = p.c_type == C_F32 ? 4.0 : 2.0;
    const double bytes = p.batch * (M * K * 2 + N * K * belt + M * N * cb * (p.accumulate ? 2 : 1) +
                                    (p.R ? M * N * 4 : 0) + (p.K2 ? (M + N) * p.K2 * 2.0 : 0));
    static const char* kNames[] = {"gemm_nf4_nt", "gemm_nf4_nn", "gemm_bf16_nt", "gemm_bf16_nn",
                                   "gemm_bf16_tn", "gemm_f16_nt", "gemm_f16_nn", "gemm_other"};
    static const char* kWideNames[] = {"gemm_nf4_nt_wide", "gemm_nf4_nn_wide"};
    const int ni = key == 0 ? 0 : key == 10 ? 1 : key == 20 ? 2 : key == 30 ? 3 : key == 130 ? 4
                 : key == 21 ? 5 : key == 31 ? 6 : 7;
    const int bsz = p.batch * p.splits;
    {
        ProfScope prof(p.tag ? p.tag : (wide_tile ? kWideNames[ni] : kNames[ni]), flops, bytes, s,
                       fast_ok || dense_fast);
        switch (key) {
            case A_ROW * 100 + B_NF4_NT * 10 + TE_BF16:
                if (fast_ok)
                    wide_tile ? launch_wide<B_NF4_NT>(p, tiles, s, prof) : launch_fast<B_NF4_NT>(p, tiles, s, prof);
                else
                    launch_kind<A_ROW, B_NF4_NT, TE_BF16>(p, tc, bsz, s);
                break;
            case A_ROW * 100 + B_NF4_NN * 10 + TE_BF16:
                if (fast_ok)
                    wide_tile ? launch_wide<B_NF4_NN>(p, tiles, s, prof) : launch_fast<B_NF4_NN>(p, tiles, s, prof);
                else
                    launch_kind<A_ROW, B_NF4_NN, TE_BF16>(p, tc, bsz, s);
                break;
            case A_ROW * 100 + B_DENSE_NT * 10 + TE_BF16:
                if (tc.bm == 64) launch_cfg<A_ROW, B_DENSE_NT, TE_BF16, 64, 64, 32, 32>(p, bsz, s);
                else launch_cfg<A_ROW, B_DENSE_NT, TE_BF16, 128, 128, 64, 64>(p, bsz, s);
                break;
            case A_ROW * 100 + B_DENSE_NN * 10 + TE_BF16:
                if (tc.bm == 64) launch_cfg<A_ROW, B_DENSE_NN, TE_BF16, 64, 64, 32, 32>(p, bsz, s);
                else launch_cfg<A_ROW, B_DENSE_NN, TE_BF16, 128, 128, 64, 64>(p, bsz, s);
                break;
            case A_TRANS * 100 + B_DENSE_NN * 10 + TE_BF16:
                if (tc.bm == 64) launch_cfg<A_TRANS, B_DENSE_NN, TE_BF16, 64, 64, 32, 32>(p, bsz, s);
                else launch_cfg<A_TRANS, B_DENSE_NN, TE_BF16, 128, 128, 64, 64>(p, bsz, s);
                break;
            case A_ROW * 100 + B_DENSE_NT * 10 + TE_F16:
                if (dense_fast) launch_dense(p, tiles, s, prof);
                else launch_cfg<A_ROW, B_DENSE_NT, TE_F16, 128, 128, 64, 64>(p, bsz, s);
                break;
            case A_ROW * 100 + B_DENSE_NN * 10 + TE_F16:
                launch_cfg<A_ROW, B_DENSE_NN, TE_F16, 128, 128, 64, 64>(p, bsz, s);
                break;
            default: throw Error{QLX_EUNSUPPORTED, "gemm: operand combination not built"};
        }
        check_launch("gemm");
    }
    if (p.splits > 1) {
        const int64_t MN = int64_t(p.M) * p.N;
        ProfScope prof("splitk_reduce", double(MN) * p.splits, double(MN) * (4.0 * p.splits + cb + (p.R ? 4 : 0)), s);
        const int64_t threads = (p.N & 3) == 0 ? MN / 4 : MN;
        hipLaunchKernelGGL(k_splitk_reduce, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, p);
        check_launch("gemm splitk reduce");
    }
}

}  // namespace qlx
