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
#include <cstdlib>
#include <string>
#include <type_traits>

#include <hip/hip_ext.h>

#include "nf4_codes.h"
#include "qlx_internal.h"

// producer wavefronts of the warp-specialized NF4 kernel (4 or 8), forward
// (NT) and dX (NN): 8 run the forward 4-7% and the dX 3-9% faster than 4 on
// the 8B shapes
#ifndef QLX_WS_NPW_NT
#define QLX_WS_NPW_NT 8
#endif
#ifndef QLX_WS_NPW_NN
#define QLX_WS_NPW_NN 8
#endif

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

// Transposed operand staged as it lies in memory: tile[k][r] =
// src[(k0 + k) * ld + r0 + r], rows of R + 8 elements, 16-byte loads and
// stores of 8 consecutive r (zeros past K or past `rows`). The MFMA fragments
// come out with the transposing LDS read (ktfrag), so no 2-byte transposed
// stores: the tile holds the same values the row-major layout would.
template <int R, int NT>
struct KLoader {
    static constexpr int RP = R + 8;
    static constexpr int U = BK * (R / 8) / NT;
    static_assert(U >= 1 && BK * (R / 8) % NT == 0, "k-major loader shape");
    static_assert(BK * RP <= R * BKP, "k-major tile must fit the row-major buffer");
    uint4 v[U];
    __device__ inline void load(const uint16_t* __restrict__ src, int64_t ld, int r0, int k0, int rows, int K,
                                int /*vec_ok*/) {
        const bool v16 = (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (ld & 7) == 0 && (r0 & 7) == 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
            const int k = idx / (R / 8), rg = (idx % (R / 8)) * 8;
            const int gk = k0 + k, gr = r0 + rg;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (gk < K) {
                const uint16_t* q = src + int64_t(gk) * ld + gr;
                if (v16 && gr + 8 <= rows) {
                    val = *reinterpret_cast<const uint4*>(q);
                } else {
                    uint32_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (gr + j < rows) ? q[j] : 0u;
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
            *reinterpret_cast<uint4*>(tile + (idx / (R / 8)) * RP + (idx % (R / 8)) * 8) = v[u];
        }
    }
};

// gfx950's transposing LDS read (ds_read_b64_tr_b16): within each group of
// 16 lanes, lane i points at row r0 + i / 4, columns c0 + 4 (i % 4) .. + 3
// of a 16-bit tile, and lane j receives column c0 + j of rows r0 .. r0 + 3.
__device__ inline uint2 tr_read(const uint16_t* q) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4* lds_s4_t;
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_s4_t>(uint32_t(reinterpret_cast<uintptr_t>(q))));
    return __builtin_bit_cast(uint2, v);
}
// The MFMA fragment of a k-major tile (rows of RP elements): lane (c = lane &
// 15, g = lane >> 4) gets column cb + c at k = kk + 8 g .. + 7, the same
// eight values the row-major layout gives it.
template <int RP>
__device__ inline uint4 ktfrag(const uint16_t* __restrict__ tile, int kk, int cb, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const uint16_t* q = tile + (kk + 8 * g + (i >> 2)) * RP + cb + 4 * (i & 3);
    const uint2 lo = tr_read(q), hi = tr_read(q + 4 * RP);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// The weight operand is the dequantized value rounded to bf16 (QLoRA's
// computation type). With fp16 activations (TE_F16) that bf16 value is then
// converted to fp16, exactly for every |value| in [2^-17, 65504] (fp16 holds
// bf16's 8-bit significands there), so the product sees the same weights.
// (For fp16, the conversion with a zero low half leaves bf16(x) << 16, the
// fp32 bits of bf16(x) itself: three instructions per pair instead of four.)
template <int TE>
__device__ __forceinline__ uint32_t wpair(float lo, float hi) {
    if constexpr (TE == TE_BF16) {
        return f32x2_to_bf16x2(lo, hi);
    } else {
        const float l = __builtin_bit_cast(float, f32x2_to_bf16x2(0.f, lo));
        const float h = __builtin_bit_cast(float, f32x2_to_bf16x2(0.f, hi));
        return f32x2_to_f16x2(l, h);
    }
}
template <int TE>
__device__ __forceinline__ uint32_t wone(float v) {
    return wpair<TE>(v, 0.f) & 0xFFFFu;
}

template <int TE>
__device__ inline uint32_t nf4_elem(const uint8_t* __restrict__ packed, const float* __restrict__ absmax,
                                    int64_t flat, const float* lut) {
    const uint32_t byte = packed[flat >> 1];
    const int code = (flat & 1) ? int(byte & 15) : int(byte >> 4);
    return wone<TE>(lut[code] * absmax[flat >> 6]);
}

template <int TE>
__device__ inline uint32_t deq2(uint32_t byte, float a, const float* lut) {
    // byte -> 16-bit pair (high nibble = even element in the low half)
    return wpair<TE>(lut[byte >> 4] * a, lut[byte & 15] * a);
}

// NF4 weight stored [N][K] (flat n*cols + k): tile[n][k]. A unit is 32 codes
// (16 bytes) of one row inside one 64-element absmax block.
template <int R, int NT, int TE>
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
                        make_uint4(deq2<TE>(x & 0xFF, a[u], lut), deq2<TE>((x >> 8) & 0xFF, a[u], lut),
                                   deq2<TE>((x >> 16) & 0xFF, a[u], lut), deq2<TE>(x >> 24, a[u], lut));
                }
            } else {
                const int gn = n0 + r, gk = k0 + half * 32;
                for (int j = 0; j < 32; ++j) {
                    const int k = gk + j;
                    dst[j] = (gn < N && k < K) ? uint16_t(nf4_elem<TE>(packed, absmax, int64_t(gn) * cols + k, lut))
                                               : uint16_t(0);
                }
            }
        }
    }
};

// NF4 weight stored [K][N] (flat k*cols + n): tile[n][k]. A unit is 4
// consecutive n (2 bytes) from each of 8 consecutive k rows.
template <int R, int NT, int TE>
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
                    e2[kr][0] = wpair<TE>(lut[(t >> 4) & 15] * s, lut[t & 15] * s);
                    e2[kr][1] = wpair<TE>(lut[(t >> 12) & 15] * s, lut[(t >> 8) & 15] * s);
                }
            } else {
#pragma unroll
                for (int kr = 0; kr < 8; ++kr) {
                    const int gk = k0 + kg + kr;
                    uint32_t e[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int gn = n0 + ng + j;
                        e[j] = (gk < K && gn < N) ? nf4_elem<TE>(packed, absmax, int64_t(gk) * cols + gn, lut) : 0u;
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
// AK_ / BK_: the A / B tile is k-major (KLoader, rows of APR / BPR elements)
// rather than row-major with BKP-element rows.
template <int TE, int WM, int WN, bool AK_ = false, bool BK_ = false, int APR = 0, int BPR = 0>
__device__ inline void mma_chunk(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                 f32x4 (&acc)[WM / 16][WN / 16], int wm, int wn, int lane) {
    const int lr = lane & 15, lk = (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
        uint4 a[WM / 16], b[WN / 16];
#pragma unroll
        for (int i = 0; i < WM / 16; ++i)
            a[i] = AK_ ? ktfrag<APR>(As, kk, wm * WM + i * 16, lane)
                       : *reinterpret_cast<const uint4*>(As + (wm * WM + i * 16 + lr) * BKP + kk + lk);
#pragma unroll
        for (int j = 0; j < WN / 16; ++j)
            b[j] = BK_ ? ktfrag<BPR>(Bs, kk, wn * WN + j * 16, lane)
                       : *reinterpret_cast<const uint4*>(Bs + (wn * WN + j * 16 + lr) * BKP + kk + lk);
#pragma unroll
        for (int i = 0; i < WM / 16; ++i)
#pragma unroll
            for (int j = 0; j < WN / 16; ++j) acc[i][j] = mfma16<TE>(a[i], b[j], acc[i][j]);
    }
}

// SEG = false: the caller guarantees seg_rows == 0 (no indexed access into
// the parameter block, so a kernel's local copy of it stays in registers)
template <bool SEG = true>
__device__ inline void store_out(const GemmParams& p, int bo, int bi, int row, int col, float v) {
    v *= p.alpha;
    if (p.R) v += p.R[int64_t(row) * p.ldr + col];
    void* C = p.C;
    int64_t off;
    if (SEG && p.seg_rows > 0) {
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
template <bool SEG = true>
__device__ inline void store_row(const GemmParams& p, int bo, int bi, int row, int col, const float* v, int n) {
    if ((!SEG || p.seg_rows == 0) && !p.accumulate && col + n <= p.N && (n & 7) == 0) {
        const int64_t off = int64_t(bo) * p.c_so + int64_t(bi) * p.c_si + int64_t(row) * p.ldc + col;
        if ((p.c_type == C_BF16 || p.c_type == C_F16) && (off & 7) == 0 && !p.R) {
            uint16_t* dst = static_cast<uint16_t*>(p.C) + off;
            const bool h = p.c_type == C_F16;
            for (int c = 0; c < n; c += 8) {
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float lo = v[c + 2 * k] * p.alpha, hi = v[c + 2 * k + 1] * p.alpha;
                    w[k] = h ? f32x2_to_f16x2(lo, hi) : f32x2_to_bf16x2(lo, hi);
                }
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
        if (col + c < p.N) store_out<SEG>(p, bo, bi, row, col + c, v[c]);
}

template <int AK, int R, int NT>
using ALoader = typename std::conditional<AK == A_ROW, RowLoader<R, NT>, KLoader<R, NT>>::type;
template <int BKIND, int R, int NT, int TE>
using BLoader = typename std::conditional<
    BKIND == B_NF4_NT, Nf4NtLoader<R, NT, TE>,
    typename std::conditional<BKIND == B_NF4_NN, Nf4NnLoader<R, NT, TE>,
                              typename std::conditional<BKIND == B_DENSE_NT, RowLoader<R, NT>,
                                                        KLoader<R, NT>>::type>::type>::type;

// LM-head cross-entropy statistics epilogue. The lane holds 16 consecutive
// columns col0.. of one row; the 4 lanes of a row are lanes 4k..4k+3 of the
// wavefront (one 64-column block). It writes the block's max and sum of
// exp(z - max) (joined over the 4 lanes) and the target's logit, and, when
// ce_logits is set, the 16 fp32 logits themselves (row stride ce_ldl), from
// which the backward forms dz without running the product again.
__device__ inline int ce_target(const GemmParams& p, int t) {
    const int s = t % p.ce_seq;
    if (s < p.ce_start || s >= p.ce_seq - 1) return -1;
    return p.ce_tokens[t + 1];
}
__device__ void ce_epilogue(const GemmParams& p, int row, int col0, const float* src) {
    const bool rok = row < p.M;
    const int tgt = rok ? ce_target(p, row) : -1;
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
        const int64_t o = int64_t(row) * p.ce_pld + col0 / 64;
        p.ce_pm[o] = mx;
        p.ce_ps[o] = sm;
    }
    if (rok && tgt >= col0 && tgt < col0 + 16 && tgt < p.N) p.ce_picked[row] = src[tgt - col0];
    if (rok && p.ce_logits && col0 < p.N) {
        float* dst = p.ce_logits + int64_t(row) * p.ce_ldl + col0;
        if (col0 + 16 <= p.N && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
#pragma unroll
            for (int c = 0; c < 16; c += 4)
                *reinterpret_cast<float4*>(dst + c) = make_float4(src[c], src[c + 1], src[c + 2], src[c + 3]);
        } else {
            for (int c = 0; c < 16; ++c)
                if (col0 + c < p.N) dst[c] = src[c];
        }
    }
}

// Workgroup b of a full-tile NF4 GEMM's 1-D grid of gx * gy * splits
// workgroups -> (M-tile, N-tile, split): split b / (gx gy), and within a
// split workgroups go to the 8 XCDs in turn (b % 8) with the gx N-tiles of
// one M-tile on one XCD, so they share its activation rows in one L2. (An
// order giving each XCD whole (M-tile, split) groups fetched 40% fewer bytes
// from memory at 512 tokens but ran 1-3% slower.)
struct TileIdx {
    int m, n, split;
};
__device__ __forceinline__ TileIdx tile_of(int b, int gx, int gy, int splits) {
    (void)splits;
    const int ntile = gx * gy;
    const int bt = b % ntile, sp = b / ntile;
    const int t = (ntile % 8 == 0) ? (bt % 8) * (ntile / 8) + bt / 8 : bt;
    return TileIdx{t / gx, t % gx, sp};
}

// One output tile of the generic GEMM: tile t (M-tile t % gy of N-tile
// t / gy), grid row y = batch index * splits + split. GRP: a grouped
// problem (no segments, batching or split), p a local copy.
template <int AK, int BKIND, int TE, int BM, int BN, int WM, int WN, bool GRP = false>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const int t, const int y) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    constexpr bool kNf4 = (BKIND == B_NF4_NT || BKIND == B_NF4_NN);
    __shared__ __align__(16) uint16_t As[2][BM * BKP];
    __shared__ __align__(16) uint16_t Bs[2][BN * BKP];
    __shared__ float lut[16];
    const int tid = threadIdx.x;
    if (kNf4 && tid < 16) lut[tid] = nf4_value(tid);

    const int gy = (p.M + BM - 1) / BM;
    const int m0 = (t % gy) * BM, n0 = (t / gy) * BN;
    const int split = y % p.splits;
    const int bz = y / p.splits;
    const int bo = bz / p.zdiv, bi = bz % p.zdiv;
    if (p.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;  // tile strictly above the diagonal

    const uint16_t* A = p.A + int64_t(bo) * p.a_so + int64_t(bi / p.a_grp) * p.a_si;
    const uint16_t* Bd =
        static_cast<const uint16_t*>(p.B) + (kNf4 ? 0 : int64_t(bo) * p.b_so + int64_t(bi / p.b_grp) * p.b_si);
    if constexpr (BKIND == B_DENSE_NN)
        if (!GRP && p.seg_rows > 0) Bd += p.bseg[m0 / p.seg_rows];  // the segment's B columns
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
        BLoader<BKIND, BN, NT, TE> lb;
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
            mma_chunk<TE, WM, WN, AK == A_TRANS, BKIND == B_DENSE_NN, BM + 8, BN + 8>(As[buf], Bs[buf], acc, wm, wn,
                                                                                     lane);
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
                store_row<!GRP>(p, bo, bi, row, col0, src, WN / 4);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

template <int AK, int BKIND, int TE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm(const GemmParams p) {
    // tile order: the gy M-tiles of one N-tile are consecutive within an XCD
    const int ntile = ((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
    int t = blockIdx.x;
    if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
    gemm_tile<AK, BKIND, TE, BM, BN, WM, WN>(p, t, blockIdx.y);
}

// A group of independent products in one launch (no split, no batching):
// workgroup b runs tile b - prob[i].tile0 of the problem i whose tile range
// holds b; the problems share everything in base but operands, sizes, output
// and alpha.
template <int AK, int BKIND, int TE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_group(const GemmParams base, const GemmGroup g) {
    const int b = blockIdx.x;
    int i = 0;
    while (i + 1 < g.n && b >= g.prob[i + 1].tile0) ++i;
    const GemmProb& q = g.prob[i];
    GemmParams p = base;
    p.A = q.A;
    p.lda = q.lda;
    p.B = q.B;
    p.ldb = q.ldb;
    p.C = q.C;
    p.ldc = q.ldc;
    p.M = q.M;
    p.N = q.N;
    p.alpha = q.alpha;
    gemm_tile<AK, BKIND, TE, BM, BN, WM, WN, true>(p, b - q.tile0, 0);
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
//  [64 k][64 B] with two absmax per row, which land transposed
//  ([2 blocks][64 k]) so a thread reads its 8 rows' maxima as two 16-byte
//  vectors. Every wavefront issues exactly one
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
            scale = uint32_t((int64_t(qs & 63) * (cols >> 6) + (qs >> 6)) * 4);
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

// The table entry of byte B of w. The kernels that dequantize through it
// declare no static LDS, so their dynamic buffer, and the table at its
// offset 0, start at LDS address 0: the entry's address is the byte times 8,
// one byte-select shift (SDWA) and no base to add.
static_assert(OFF_L == 0, "the table lookups address LDS from 0");
template <int B>
__device__ __forceinline__ f2 lut_at(uint32_t w) {
    static_assert(B >= 0 && B < 4, "byte index");
    uint32_t off;
    if constexpr (B == 0)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
            : "=v"(off) : "v"(w));
    else if constexpr (B == 1)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
            : "=v"(off) : "v"(w));
    else if constexpr (B == 2)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
            : "=v"(off) : "v"(w));
    else
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
            : "=v"(off) : "v"(w));
    return *reinterpret_cast<const __attribute__((address_space(3))) f2*>(static_cast<uintptr_t>(off));
}
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>());
        static_for<I + 1, N>(f);
    }
}

// Codes of one chunk (LDS) -> bf16 tile [n][k] (LDS). lut2[b] (LDS address
// 8 b) holds the code values of byte b's high nibble (the even element) and
// low nibble.
// t: the thread's slot, 0..511 (a 512-thread workgroup passes threadIdx.x)
template <int BKIND, int TE>
__device__ __forceinline__ void dequant(const char* __restrict__ raw, const char* __restrict__ sc,
                                        const char* __restrict__ lds0, uint16_t* __restrict__ tile, const int t) {
    const float* s = reinterpret_cast<const float*>(sc);
    (void)lds0;  // the table is read at its absolute LDS address (lut_at)
    if constexpr (BKIND == B_NF4_NT) {
        // thread = 16 consecutive k of row t >> 2
        const int r = t >> 2, q4 = t & 3;
        const uint2 w = *reinterpret_cast<const uint2*>(raw + r * 32 + q4 * 8);
        const float a = s[r];
        uint32_t e[8];
        static_for<0, 8>([&](auto bb) {
            constexpr int b = decltype(bb)::value;
            const f2 v = lut_at<b & 3>(b < 4 ? w.x : w.y);
            e[b] = wpair<TE>(v.x * a, v.y * a);
        });
        *reinterpret_cast<uint4*>(tile + swz(r, 2 * q4)) = make_uint4(e[0], e[1], e[2], e[3]);
        *reinterpret_cast<uint4*>(tile + swz(r, 2 * q4 + 1)) = make_uint4(e[4], e[5], e[6], e[7]);
    } else {
        // thread = one code byte column (n = ng, ng + 1) x 8 consecutive k:
        // per k row one byte, whose high nibble is n = ng; the 8 k of each n
        // are one 16-byte chunk of the tile. The 64 lanes of a wavefront take
        // the 64 byte columns, so a row write's lanes cover all 8 swizzled
        // chunk positions (with 4 n x 4 k per thread they covered 4, in
        // 8-byte halves: a 4-way LDS bank conflict on every write).
        const int i = t & 63, ng = 2 * i, kg = (t >> 6) * 8;
        // maxima of block ng / 64 for rows kg..kg+7 ([block][k] in LDS)
        const float4 a0 = *reinterpret_cast<const float4*>(s + (i >> 5) * 64 + kg);
        const float4 a1 = *reinterpret_cast<const float4*>(s + (i >> 5) * 64 + kg + 4);
        const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        f2 v[8];
#pragma unroll
        for (int kr = 0; kr < 8; ++kr) v[kr] = lut_at<0>(*reinterpret_cast<const uint8_t*>(raw + (kg + kr) * 64 + i));
        uint32_t e[8], o[8];
#pragma unroll
        for (int kr = 0; kr < 8; kr += 2) {
            e[kr >> 1] = wpair<TE>(v[kr].x * a[kr], v[kr + 1].x * a[kr + 1]);
            o[kr >> 1] = wpair<TE>(v[kr].y * a[kr], v[kr + 1].y * a[kr + 1]);
        }
        *reinterpret_cast<uint4*>(tile + swz(ng, kg >> 3)) = make_uint4(e[0], e[1], e[2], e[3]);
        *reinterpret_cast<uint4*>(tile + swz(ng + 1, kg >> 3)) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// One 64-wide chunk of MFMAs for a (16 FI_) x (16 FJ_) wavefront tile. Row
// (base + i*16 + lr) swizzles with (lr >> 1) & 7 only, so each K half has one
// per-lane base.
// TR: each accumulator holds its 16 x 16 block transposed (the MFMA takes the
// B fragment as its first operand), so a lane ends with 4 consecutive
// columns of one row instead of 4 rows of one column.
template <int FI_, int FJ_, int TE_ = TE_BF16, bool TR = false>
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
            for (int j = 0; j < FJ_; ++j)
                acc[i][j] = TR ? mfma16<TE_>(b[j], a[i], acc[i][j]) : mfma16<TE_>(a[i], b[j], acc[i][j]);
    }
}

// LoRA slab of a full tile (last split only): K2 in 64-wide chunks through
// the 64-wide swizzled layout at As (BM_ rows) and Bs (BN_ rows), zero-filled
// past K2. The caller has drained every DMA and barriered.
template <int BKIND, int BM_, int BN_, int TE, int FI_, int FJ_>
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
        mma<FI_, FJ_, TE>(As, Bs, acc, rm, rn, lane);
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

template <int BKIND, int TE>
__global__ __launch_bounds__(fast::NTH) void k_nf4_tile(const GemmParams p) {
    using namespace fast;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    if (tid < 256) reinterpret_cast<f2*>(lds + OFF_L)[tid] = f2{nf4_value(tid >> 4), nf4_value(tid & 15)};

    const TileIdx ti = tile_of(blockIdx.x, p.N / BN, p.M / BM, p.splits);
    const int m0 = ti.m * BM, n0 = ti.n * BN, split = ti.split;
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
    dequant<BKIND, TE>(sr(0), ss(0), lds, sb(0), tid);
    stage_sync<NA + NR>();          // A 0, codes 1, bf16 0
    auto step = [&](int c, auto stage) {
        constexpr int S0 = decltype(stage)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
        a_dma(c + 2, S2);
        code_dma(c + 3, S0);
        mma<FI, FJ, TE>(reinterpret_cast<const uint16_t*>(sa(S0)), sb(S0), acc, wm * WM, wn * WN, lane);
        dequant<BKIND, TE>(sr(S1), ss(S1), lds, sb(S1), tid);
        stage_sync<NA + NR>();      // A c+1, codes c+2, bf16 c+1
    };
    for (int c = 0; c < nch; c += 3) {
        step(c, std::integral_constant<int, 0>());
        if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
        if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
    }
    stage_sync<0>();

    if (p.K2 > 0 && split == p.splits - 1)  // LoRA slab, any K2 (zero-filled tail)
        slab<BKIND, BM, BN, TE>(p, reinterpret_cast<uint16_t*>(sa(0)), sb(0), acc, m0, n0, wm * WM, wn * WN, lane);
    epilogue<FI, WN>(p, acc, reinterpret_cast<float*>(lds + OFF_A) + wave * (16 * (WN + 4)), m0 + wm * WM,
                     n0 + wn * WN, split, lane);
}

// ---------------------------------------------------------------------------
// Warp-specialized full-tile NF4 kernel: the 256 x 128 tile of k_nf4_tile
// with its two kinds of work on different wavefronts. Eight MFMA wavefronts
// (4 x 2, 64 x 64 each, two per SIMD) only read fragments and issue MFMAs;
// NPW producer wavefronts (4 or 8: one or two per SIMD) issue every DMA of
// the tile and dequantize the next chunk's codes into the bf16/fp16 tile.
// Each SIMD so always has a wavefront with MFMAs ready beside one doing LDS
// lookups and conversions, and the MFMA wavefronts never wait on the
// dequantization chain. One workgroup barrier per 64-wide chunk publishes A (two chunks
// ahead), the codes (three ahead) and the converted tile (one ahead, two LDS
// stages). Same operand values, order of MFMAs and epilogue as k_nf4_tile,
// so the results are bit-identical to it.
namespace ws {
constexpr int BM = 256, BN = 128, NMW = 8, WGN = 2, WM = 64, WN = 64;
constexpr int FI = WM / 16, FJ = WN / 16;
constexpr int SA = BM * 64 * 2, SB = BN * 64 * 2, SR = BN * 32, SS = 512;
constexpr int OFF_L = 0, OFF_A = 256 * 8, OFF_B = OFF_A + 3 * SA, OFF_R = OFF_B + 2 * SB, OFF_S = OFF_R + 3 * SR;
constexpr int LDS_BYTES = OFF_S + 3 * SS;
static_assert(LDS_BYTES <= 160 * 1024, "warp-specialized NF4 tile exceeds LDS");
static_assert(OFF_L == fast::OFF_L, "the dequantization reads the table at the fast tile's offset");
// NPW producer wavefronts (4 or 8): per chunk each issues NA 16-byte A DMAs
// and NC code + NC absmax DMAs, and dequantizes 512 / (64 NPW) slots per lane
template <int NPW>
struct Prod {
    static_assert(NPW == 4 || NPW == 8, "4 or 8 producer wavefronts");
    static constexpr int NTH = (NMW + NPW) * 64;
    static constexpr int NA = BM / 8 / NPW;
    static constexpr int NC = 8 / NPW;
    static constexpr int NR = 2 * NC;
    static constexpr int NDQ = 512 / (64 * NPW);
};

// The producers' DMA offsets: the A tile in 1 KB blocks (8 rows x 128 B, the
// swizzled layout of k_nf4_tile), then the codes in 16-byte slots q (256 per
// chunk: NT row q >> 1, NN k-row q >> 2) and the maxima in 4-byte slots qs
// (128 per chunk). pw = producer wavefront 0..NPW-1.
template <int BKIND, int NPW>
struct DmaPlanP {
    static constexpr int NA = Prod<NPW>::NA, NC = Prod<NPW>::NC;
    uint32_t a[NA];
    uint32_t code[NC], scale[NC];
    int pw;
    __amdgpu_buffer_rsrc_t ra, rc, rs;
    __device__ __forceinline__ void init(const void* a0, const void* c0, const void* s0, int64_t lda, int64_t cols,
                                         int pw_) {
        const int lane = threadIdx.x & 63;
        pw = pw_;
        ra = fast::rsrc(a0);
        rc = fast::rsrc(c0);
        rs = fast::rsrc(s0);
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int r = (pw * NA + u) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            a[u] = uint32_t((int64_t(r) * lda + c * 8) * 2);
        }
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int q = (pw * NC + j) * 32 + (lane & 31), qs = (pw * NC + j) * 16 + (lane & 15);
            if constexpr (BKIND == B_NF4_NN) {
                code[j] = uint32_t(int64_t(q >> 2) * (cols >> 1) + (q & 3) * 16);
                scale[j] = uint32_t((int64_t(qs & 63) * (cols >> 6) + (qs >> 6)) * 4);
            } else {
                code[j] = uint32_t(int64_t(q >> 1) * (cols >> 1) + (q & 1) * 16);
                scale[j] = uint32_t(int64_t(qs) * (cols >> 6) * 4);
            }
        }
    }
    __device__ __forceinline__ void a_dma(uint32_t soff, char* __restrict__ dst) const {
#pragma unroll
        for (int u = 0; u < NA; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, fast::as_lds(dst + (pw * NA + u) * 1024), 16, a[u], soff, 0, 0);
    }
    __device__ __forceinline__ void code_dma(uint32_t coff, uint32_t soff, char* __restrict__ raw,
                                             char* __restrict__ sc) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            if (lane < 32)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, fast::as_lds(raw + (pw * NC + j) * 32 * 16), 16, code[j],
                                                         coff, 0, 0);
            if (lane < 16)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, fast::as_lds(sc + (pw * NC + j) * 16 * 4), 4, scale[j],
                                                         soff, 0, 0);
        }
    }
};

// LoRA slab (last split): the MFMA wavefronts stage A2 / B2 and multiply; the
// producers only keep the barriers.
template <int BKIND, int TE>
__device__ __forceinline__ void slab(const GemmParams& p, bool mw, uint16_t* As, uint16_t* Bs,
                                     f32x4 (&acc)[FI][FJ], int m0, int n0, int rm, int rn, int lane) {
    for (int k0 = 0; k0 < p.K2; k0 += 64) {
        if (mw) {
            RowLoader<BM, NMW * 64, true> la;
            la.load(p.A2, p.lda2, m0, k0, p.M, p.K2, p.a2_vec);
            if constexpr (BKIND == B_NF4_NT) {
                RowLoader<BN, NMW * 64, true> lb;
                lb.load(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec);
                lb.store(Bs);
            } else {
                // B2 is [K2][N]: one element at a time into the swizzled
                // [n][k] tile (reads along n coalesce; few registers, so the
                // accumulators need not leave them)
                for (int e = threadIdx.x; e < BN * 64; e += NMW * 64) {
                    const int k = e / BN, n = e % BN, gk = k0 + k, gn = n0 + n;
                    Bs[tile_off<true>(n, k >> 3) + (k & 7)] = (gk < p.K2 && gn < p.N) ? p.B2[int64_t(gk) * p.ldb2 + gn]
                                                                                      : uint16_t(0);
                }
            }
            la.store(As);
        }
        __syncthreads();
        if (mw) fast::mma<FI, FJ, TE>(As, Bs, acc, rm, rn, lane);
        __syncthreads();
    }
}
}  // namespace ws

template <int BKIND, int TE, int NPW>
__global__ __launch_bounds__(ws::Prod<NPW>::NTH) void k_nf4_ws(const GemmParams p) {
    using namespace ws;
    constexpr int NA = Prod<NPW>::NA, NR = Prod<NPW>::NR, NDQ = Prod<NPW>::NDQ;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool mw = wave < NMW;  // MFMA wavefront (else producer)
    const int wm = wave / WGN, wn = wave % WGN;
    if (tid < 256) reinterpret_cast<fast::f2*>(lds + OFF_L)[tid] = fast::f2{nf4_value(tid >> 4), nf4_value(tid & 15)};

    const TileIdx ti = tile_of(blockIdx.x, p.N / BN, p.M / BM, p.splits);
    const int m0 = ti.m * BM, n0 = ti.n * BN, split = ti.split;
    const int kbeg = split * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    const int nch = (kend - kbeg) / 64;
    const int64_t cols = p.nf4_cols;

    auto sa = [&](int s) { return lds + OFF_A + s * SA; };
    auto sb = [&](int s) { return reinterpret_cast<uint16_t*>(lds + OFF_B + s * SB); };
    auto sr = [&](int s) { return lds + OFF_R + s * SR; };
    auto ss = [&](int s) { return lds + OFF_S + s * SS; };
    const bool slab = p.K2 > 0 && split == p.splits - 1;  // LoRA slab, any K2 (zero-filled tail)
    // The two roles run separate code with the same barriers in the same
    // order, so neither keeps the other's registers live.
    if (mw) {
        f32x4 acc[FI][FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        fast::stage_sync<0>();  // codes 0 (and the table) in LDS
        fast::stage_sync<0>();  // A 0, codes 1, converted 0
        auto step = [&](int c, auto stage) {
            constexpr int S0 = decltype(stage)::value;
            fast::mma<FI, FJ, TE>(reinterpret_cast<const uint16_t*>(sa(S0)), sb(c & 1), acc, wm * WM, wn * WN, lane);
            fast::stage_sync<0>();  // A c+1, codes c+2, converted c+1
        };
        for (int c = 0; c < nch; c += 3) {
            step(c, std::integral_constant<int, 0>());
            if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
            if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
        }
        fast::stage_sync<0>();
        if (slab) ws::slab<BKIND, TE>(p, true, reinterpret_cast<uint16_t*>(sa(0)), sb(0), acc, m0, n0, wm * WM, wn * WN, lane);
        fast::epilogue<FI, WN>(p, acc, reinterpret_cast<float*>(lds + OFF_A) + wave * (16 * (WN + 4)), m0 + wm * WM,
                               n0 + wn * WN, split, lane);
    } else {
        const int64_t flat0 = (BKIND == B_NF4_NN) ? int64_t(kbeg) * cols + n0 : int64_t(n0) * cols + kbeg;
        DmaPlanP<BKIND, NPW> plan;
        plan.init(p.A + int64_t(m0) * p.lda + kbeg, static_cast<const char*>(p.B) + (flat0 >> 1),
                  p.absmax + (flat0 >> 6), p.lda, cols, wave - NMW);
        const uint32_t cstep = (BKIND == B_NF4_NN) ? uint32_t(32 * cols) : 32u;
        const uint32_t sstep = (BKIND == B_NF4_NN) ? uint32_t(4 * cols) : 4u;
        auto cl = [&](int c) { return min(c, nch - 1); };
        auto a_dma = [&](int c, int s) { plan.a_dma(uint32_t(cl(c)) * 128u, sa(s)); };
        auto code_dma = [&](int c, int s) {
            plan.code_dma(uint32_t(cl(c)) * cstep, uint32_t(cl(c)) * sstep, sr(s), ss(s));
        };
        // the producers' lanes dequantize as the 512 slots of k_nf4_tile, NDQ each
        const int pt = tid - NMW * 64;
        auto dq = [&](int rs_, uint16_t* tile) {
#pragma unroll
            for (int j = 0; j < NDQ; ++j) fast::dequant<BKIND, TE>(sr(rs_), ss(rs_), lds, tile, pt + j * NPW * 64);
        };
        code_dma(0, 0);
        a_dma(0, 0);
        code_dma(1, 1);
        a_dma(1, 1);
        code_dma(2, 2);
        fast::stage_sync<2 * NA + 2 * NR>();  // codes 0 (and the table) in LDS
        dq(0, sb(0));
        fast::stage_sync<NA + NR>();          // A 0, codes 1, converted 0
        auto step = [&](int c, auto stage) {
            constexpr int S0 = decltype(stage)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
            a_dma(c + 2, S2);
            code_dma(c + 3, S0);
            dq(S1, sb((c + 1) & 1));
            fast::stage_sync<NA + NR>();  // A c+1, codes c+2, converted c+1
        };
        for (int c = 0; c < nch; c += 3) {
            step(c, std::integral_constant<int, 0>());
            if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
            if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
        }
        fast::stage_sync<0>();
        if (slab)  // the producers keep the slab's barriers
            for (int k0 = 0; k0 < p.K2; k0 += 64) {
                __syncthreads();
                __syncthreads();
            }
    }
}

// ---------------------------------------------------------------------------
// Persistent form of k_nf4_ws: the same 256 x 128 tile, roles, LDS stages and
// one barrier per 64-wide chunk, but one workgroup per CU for the whole
// launch. Workgroup b takes tiles b, b + G, b + 2G, ... (G, the grid, is a
// multiple of 8 whenever a workgroup takes more than one tile, so a tile runs
// on the XCD a one-tile-per-workgroup launch gives it) and runs them as one
// stream of chunks: a tile's K chunks, then on the last split its LoRA slab
// chunks, whose A2 rows the producers fetch by DMA like A and whose B2 block
// they load into the converted-tile stage. The producers' DMAs and
// dequantization so run on into the next tile while the MFMA wavefronts
// store the finished one, and the pipeline fills once per launch instead of
// once per tile (fill, epilogue and workgroup turnover measured ~9 us per
// tile of 64 chunks, ~12% of the 2048-row projections). The MFMAs accumulate
// each 16 x 16 block transposed, so a lane holds 4 consecutive columns and
// the epilogue stores 8 or 16 bytes at a time straight from the accumulators
// (LDS staging would collide with the stages already filling). Operands,
// products and output arithmetic are those of k_nf4_ws, and so are the bits. Takes K2 % 64 == 0 with 16-byte
// aligned A2 and B2 rows, no output segments, residual or accumulation.
namespace wsp {
using ws::BM;
using ws::BN;

// A position in a workgroup's chunk stream. Past the last chunk the cursor
// stays on it with done set, so clamped DMAs still read valid memory. The
// tile's operand origins (chunk 0 of A, A2, the codes and the maxima) are
// set when the cursor enters the tile; a chunk adds a scalar byte offset.
template <int BKIND>
struct Cursor {
    int w, c;  // tile index; chunk in the tile: [0, nch) K chunks, then nsl slab chunks
    int m0, n0, nch, nsl, split;
    bool done;
    const char *a0, *a20, *c0, *s0;
    __device__ __forceinline__ void load(const GemmParams& p, int w_) {
        const TileIdx ti = tile_of(w_, p.N / BN, p.M / BM, p.splits);
        w = w_;
        c = 0;
        m0 = ti.m * BM;
        n0 = ti.n * BN;
        split = ti.split;
        const int kbeg = split * p.kchunk;
        nch = (min(p.K, kbeg + p.kchunk) - kbeg) / 64;
        nsl = (p.K2 > 0 && split == p.splits - 1) ? p.K2 / 64 : 0;
        done = false;
        a0 = reinterpret_cast<const char*>(p.A + int64_t(m0) * p.lda + kbeg);
        a20 = reinterpret_cast<const char*>(p.A2 + int64_t(m0) * p.lda2);
        const int64_t flat = (BKIND == B_NF4_NN) ? int64_t(kbeg) * p.nf4_cols + n0 : int64_t(n0) * p.nf4_cols + kbeg;
        c0 = static_cast<const char*>(p.B) + (flat >> 1);
        s0 = reinterpret_cast<const char*>(p.absmax + (flat >> 6));
    }
    __device__ __forceinline__ void advance(const GemmParams& p, int G, int nitems) {
        if (c + 1 < nch + nsl) ++c;
        else if (w + G < nitems) load(p, w + G);
        else done = true;
    }
    __device__ __forceinline__ bool slab() const { return c >= nch; }
};

// The producers' per-lane DMA offsets (bytes, fixed for the launch): the A
// tile and the A2 slab rows in 1 KB blocks of the swizzled layout, the codes
// and maxima as in k_nf4_ws. Each DMA is a buffer resource at the tile's
// origin, a scalar chunk offset and the per-lane offset.
template <int BKIND, int NPW>
struct Plan {
    static constexpr int NA = ws::Prod<NPW>::NA, NC = ws::Prod<NPW>::NC;
    uint32_t a[NA], a2[NA];
    uint32_t code[NC], scale[NC];
    uint32_t cstep, sstep;  // bytes per K chunk of the codes and the maxima
    int pw;
    __device__ __forceinline__ void init(const GemmParams& p, int pw_) {
        const int lane = threadIdx.x & 63;
        pw = pw_;
        const int64_t cols = p.nf4_cols;
        cstep = (BKIND == B_NF4_NN) ? uint32_t(32 * cols) : 32u;
        sstep = (BKIND == B_NF4_NN) ? uint32_t(4 * cols) : 4u;
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int r = (pw * NA + u) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            a[u] = uint32_t((int64_t(r) * p.lda + c * 8) * 2);
            a2[u] = uint32_t((int64_t(r) * p.lda2 + c * 8) * 2);
        }
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int q = (pw * NC + j) * 32 + (lane & 31), qs = (pw * NC + j) * 16 + (lane & 15);
            if constexpr (BKIND == B_NF4_NN) {
                code[j] = uint32_t(int64_t(q >> 2) * (cols >> 1) + (q & 3) * 16);
                scale[j] = uint32_t((int64_t(qs & 63) * (cols >> 6) + (qs >> 6)) * 4);
            } else {
                code[j] = uint32_t(int64_t(q >> 1) * (cols >> 1) + (q & 1) * 16);
                scale[j] = uint32_t(int64_t(qs) * (cols >> 6) * 4);
            }
        }
    }
    // A rows of the cursor's chunk (A2 rows for a slab chunk) -> A stage
    __device__ __forceinline__ void a_dma(const Cursor<BKIND>& u, char* __restrict__ dst) const {
        const bool sl = u.slab();
        const auto r = fast::rsrc(sl ? u.a20 : u.a0);
        const uint32_t soff = uint32_t(sl ? u.c - u.nch : u.c) * 128u;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, fast::as_lds(dst + (pw * NA + i) * 1024), 16, sl ? a2[i] : a[i],
                                                     soff, 0, 0);
    }
    // K chunk c of a tile whose origins the resources hold (the steps whose
    // three chunks of lookahead stay in one tile)
    __device__ __forceinline__ void a_dma_k(__amdgpu_buffer_rsrc_t r, int c, char* __restrict__ dst) const {
#pragma unroll
        for (int i = 0; i < NA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, fast::as_lds(dst + (pw * NA + i) * 1024), 16, a[i],
                                                     uint32_t(c) * 128u, 0, 0);
    }
    __device__ __forceinline__ void code_dma_k(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int c,
                                               char* __restrict__ raw, char* __restrict__ sc) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            if (lane < 32)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, fast::as_lds(raw + (pw * NC + j) * 32 * 16), 16, code[j],
                                                         uint32_t(c) * cstep, 0, 0);
            if (lane < 16)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, fast::as_lds(sc + (pw * NC + j) * 16 * 4), 4, scale[j],
                                                         uint32_t(c) * sstep, 0, 0);
        }
    }
    // codes and maxima of the cursor's K chunk (a slab chunk re-reads the
    // tile's first K chunk: every step issues the same DMAs)
    __device__ __forceinline__ void code_dma(const Cursor<BKIND>& u, char* __restrict__ raw,
                                             char* __restrict__ sc) const {
        const int lane = threadIdx.x & 63;
        const uint32_t kc = uint32_t(u.slab() ? 0 : u.c);
        const auto rc = fast::rsrc(u.c0);
        const auto rs = fast::rsrc(u.s0);
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            if (lane < 32)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, fast::as_lds(raw + (pw * NC + j) * 32 * 16), 16, code[j],
                                                         kc * cstep, 0, 0);
            if (lane < 16)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, fast::as_lds(sc + (pw * NC + j) * 16 * 4), 4, scale[j],
                                                         kc * sstep, 0, 0);
        }
    }
};

// The B2 block of a slab chunk (128 n x 64 k) for the converted-tile stage:
// 1024 16-byte loads over the producer lanes. NT: B2 is [N][K2], lane rows
// along n; NN: B2 is [K2][N], eight n of one k per load, written transposed.
template <int BKIND, int NPW>
struct SlabB {
    static constexpr int NH = 1024 / (NPW * 64);  // 16-byte loads per producer lane
    uint4 v[NH];
    __device__ __forceinline__ void load(const GemmParams& p, const Cursor<BKIND>& u, int pt) {
        const int s = u.c - u.nch;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int idx = pt + h * NPW * 64;
            if constexpr (BKIND == B_NF4_NT)
                v[h] = *reinterpret_cast<const uint4*>(p.B2 + int64_t(u.n0 + (idx >> 3)) * p.ldb2 + s * 64 +
                                                       (idx & 7) * 8);
            else
                v[h] = *reinterpret_cast<const uint4*>(p.B2 + int64_t(s * 64 + (idx >> 4)) * p.ldb2 + u.n0 +
                                                       (idx & 15) * 8);
        }
    }
    __device__ __forceinline__ void store(uint16_t* __restrict__ tile, int pt) const {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int idx = pt + h * NPW * 64;
            if constexpr (BKIND == B_NF4_NT) {
                *reinterpret_cast<uint4*>(tile + tile_off<true>(idx >> 3, idx & 7)) = v[h];
            } else {
                const int k = idx >> 4, n = (idx & 15) * 8;
                const uint32_t w[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    tile[tile_off<true>(n + e, k >> 3) + (k & 7)] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
};

// Output of one 64 x 64 wavefront tile straight from transposed accumulators
// (mma<..., true>): lane (r = lane & 15, q = lane >> 4) holds columns
// 4q..4q+3 of row r of each 16 x 16 block, stored 16 bytes (fp32) or 8 bytes
// (16-bit) at a time. The arithmetic is store_row's: fp32 partials as they
// are; otherwise alpha times the sum, rounded to the output type (no
// residual: its loads would stall the MFMA wavefronts between tiles).
template <int FI_, int FJ_>
__device__ __forceinline__ void epilogue(const GemmParams& p, const f32x4 (&acc)[FI_][FJ_], int row_b, int col_b,
                                         int split) {
    if (p.splits > 1 || p.c_type == C_F32) {
        const bool part = p.splits > 1;
        float* d = part ? p.partial + (int64_t(split) * p.M + row_b) * p.N + col_b
                        : static_cast<float*>(p.C) + int64_t(row_b) * p.ldc + col_b;
        const int64_t ld = part ? int64_t(p.N) : p.ldc;
        const float al = part ? 1.f : p.alpha;
#pragma unroll
        for (int i = 0; i < FI_; ++i)
#pragma unroll
            for (int j = 0; j < FJ_; ++j) {
                const f32x4 v = acc[i][j];
                *reinterpret_cast<float4*>(d + int64_t(i * 16) * ld + j * 16) =
                    part ? make_float4(v[0], v[1], v[2], v[3]) : make_float4(v[0] * al, v[1] * al, v[2] * al, v[3] * al);
            }
        return;
    }
    uint16_t* d = static_cast<uint16_t*>(p.C) + int64_t(row_b) * p.ldc + col_b;
    const bool h = p.c_type == C_F16;
    const float al = p.alpha;
#pragma unroll
    for (int i = 0; i < FI_; ++i)
#pragma unroll
        for (int j = 0; j < FJ_; ++j) {
            const f32x4 v = acc[i][j];
            const float x0 = v[0] * al, x1 = v[1] * al, x2 = v[2] * al, x3 = v[3] * al;
            *reinterpret_cast<uint2*>(d + int64_t(i * 16) * p.ldc + j * 16) =
                h ? make_uint2(f32x2_to_f16x2(x0, x1), f32x2_to_f16x2(x2, x3))
                  : make_uint2(f32x2_to_bf16x2(x0, x1), f32x2_to_bf16x2(x2, x3));
        }
}
}  // namespace wsp

template <int BKIND, int TE, int NPW>
__global__ __launch_bounds__(ws::Prod<NPW>::NTH) void k_nf4_wsp(const GemmParams p, const int nitems) {
    using namespace ws;
    constexpr int NA = Prod<NPW>::NA, NR = Prod<NPW>::NR, NDQ = Prod<NPW>::NDQ;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool mw = wave < NMW;  // MFMA wavefront (else producer)
    const int wm = wave / WGN, wn = wave % WGN;
    const int G = gridDim.x;
    if (tid < 256) reinterpret_cast<fast::f2*>(lds + OFF_L)[tid] = fast::f2{nf4_value(tid >> 4), nf4_value(tid & 15)};

    auto sa = [&](int s) { return lds + OFF_A + s * SA; };
    auto sb = [&](int s) { return reinterpret_cast<uint16_t*>(lds + OFF_B + s * SB); };
    auto sr = [&](int s) { return lds + OFF_R + s * SR; };
    auto ss = [&](int s) { return lds + OFF_S + s * SS; };
    // The two roles run separate code with the same barriers in the same
    // order: two in the prologue, then one per chunk of the stream.
    if (mw) {
        fast::stage_sync<0>();  // codes 0 (and the table) in LDS
        fast::stage_sync<0>();  // A 0, codes 1, converted 0
        int s3 = 0, s2 = 0;     // A and converted-tile stages of the current chunk
        for (int w = blockIdx.x; w < nitems; w += G) {
            const TileIdx ti = tile_of(w, p.N / BN, p.M / BM, p.splits);
            const int kbeg = ti.split * p.kchunk;
            const int n = (min(p.K, kbeg + p.kchunk) - kbeg) / 64 +
                          ((p.K2 > 0 && ti.split == p.splits - 1) ? p.K2 / 64 : 0);
            f32x4 acc[FI][FJ];
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < n; ++c) {
                fast::mma<FI, FJ, TE, true>(reinterpret_cast<const uint16_t*>(sa(s3)), sb(s2), acc, wm * WM, wn * WN,
                                            lane);
                // next chunk's A and converted tile; the barrier does not wait
                // for the previous tile's stores (vmcnt 63: no wait)
                fast::stage_sync<63>();
                s3 = s3 == 2 ? 0 : s3 + 1;
                s2 ^= 1;
            }
            wsp::epilogue<FI, FJ>(p, acc, ti.m * BM + wm * WM + (lane & 15), ti.n * BN + wn * WN + (lane >> 4) * 4,
                                  ti.split);
        }
    } else {
        wsp::Plan<BKIND, NPW> plan;
        plan.init(p, wave - NMW);
        const int pt = tid - NMW * 64;
        // chunk g (this step), g + 1 (converted), g + 2 (A), g + 3 (codes)
        wsp::Cursor<BKIND> cg, cd, ca, cc;
        cg.load(p, blockIdx.x);
        cd = cg;
        ca = cg;
        cc = cg;
        auto adv = [&](wsp::Cursor<BKIND>& u) { u.advance(p, G, nitems); };
        auto dq = [&](int rs_, uint16_t* tile) {
#pragma unroll
            for (int j = 0; j < NDQ; ++j) fast::dequant<BKIND, TE>(sr(rs_), ss(rs_), lds, tile, pt + j * NPW * 64);
        };
        plan.code_dma(cc, sr(0), ss(0));
        adv(cc);
        plan.a_dma(ca, sa(0));
        adv(ca);
        plan.code_dma(cc, sr(1), ss(1));
        adv(cc);
        plan.a_dma(ca, sa(1));
        adv(ca);
        plan.code_dma(cc, sr(2), ss(2));
        adv(cc);
        fast::stage_sync<2 * NA + 2 * NR>();  // codes 0 (and the table) in LDS
        dq(0, sb(0));                         // chunk 0 is always a K chunk
        adv(cd);
        fast::stage_sync<NA + NR>();  // A 0, codes 1, converted 0
        int s0 = 0;                   // chunk g's A stage (= the codes stage of g + 3)
        int par = 1;                  // converted-tile stage of chunk g + 1
        for (;;) {
            if (cg.c + 3 < cg.nch) {
                // chunks g + 1..g + 3 are K chunks of g's tile (so are the
                // other cursors): the plain step, addressed from the tile's
                // origins, with no cursor work
                const int last = cg.nch - 3;
                const auto ra = fast::rsrc(cg.a0), rc = fast::rsrc(cg.c0), rs = fast::rsrc(cg.s0);
                for (int c = cg.c; c < last; ++c) {
                    const int s1 = s0 == 2 ? 0 : s0 + 1, s2 = s1 == 2 ? 0 : s1 + 1;
                    plan.a_dma_k(ra, c + 2, sa(s2));
                    plan.code_dma_k(rc, rs, c + 3, sr(s0), ss(s0));
                    dq(s1, sb(par));
                    fast::stage_sync<NA + NR>();  // A g+1, codes g+2, converted g+1
                    s0 = s1;
                    par ^= 1;
                }
                cg.c = last;
                cd.c = last + 1;
                ca.c = last + 2;
                cc.c = last + 2;
                adv(cc);  // to the tile's end: its slab, the next tile or done
            }
            const int s1 = s0 == 2 ? 0 : s0 + 1, s2 = s1 == 2 ? 0 : s1 + 1;
            plan.a_dma(ca, sa(s2));
            adv(ca);
            plan.code_dma(cc, sr(s0), ss(s0));
            adv(cc);
            uint16_t* const tile = sb(par);
            if (!cd.done) {
                if (!cd.slab()) {
                    dq(s1, tile);
                } else {
                    // loaded, waited for and stored within the branch, so no
                    // load is pending on the registers the K chunks reuse
                    // (the wait also covers this step's DMAs: a slab chunk
                    // costs one load latency)
                    wsp::SlabB<BKIND, NPW> b2;
                    b2.load(p, cd, pt);
                    b2.store(tile, pt);
                }
            }
            adv(cd);
            fast::stage_sync<NA + NR>();  // A g+1, codes g+2, converted g+1
            adv(cg);
            if (cg.done) break;
            s0 = s1;
            par ^= 1;
        }
        __builtin_amdgcn_s_waitcnt(0);  // the clamped DMAs past the stream land before the workgroup ends
    }
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
template <int BKIND, int TE>
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
            e[b] = wpair<TE>(v.x * a, v.y * a);
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
                make_uint2(wpair<TE>(x[0], x[1]), wpair<TE>(x[2], x[3]));
        }
    }
}
template <int TE>
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
        for (int j = 0; j < FJ; ++j) acc[i][j] = mfma16<TE>(a[i], b[j], acc[i][j]);
}
}  // namespace wide

template <int BKIND, int TE>
__global__ __launch_bounds__(wide::NTH) void k_nf4_wide(const GemmParams p) {
    using namespace wide;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    if (tid < 256) reinterpret_cast<f2*>(lds + OFF_L)[tid] = f2{nf4_value(tid >> 4), nf4_value(tid & 15)};
    const TileIdx ti = tile_of(blockIdx.x, p.N / BN, p.M / BM, p.splits);
    const int m0 = ti.m * BM, n0 = ti.n * BN, split = ti.split;
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
    dequant<BKIND, TE>(sr(0), ss(0), lds, sb(0));
    fast::stage_sync<NA + NR>();
    auto step = [&](int c, auto stage) {
        constexpr int S0 = decltype(stage)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
        a_dma(c + 2, S2);
        code_dma(c + 3, S0);
        mma<TE>(reinterpret_cast<const uint16_t*>(sa(S0)), sb(S0), acc, wm * WM, wn * WN, lane);
        dequant<BKIND, TE>(sr(S1), ss(S1), lds, sb(S1));
        fast::stage_sync<NA + NR>();
    };
    for (int c = 0; c < nch; c += 3) {
        step(c, std::integral_constant<int, 0>());
        if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
        if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
    }
    fast::stage_sync<0>();
    if (p.K2 > 0 && split == p.splits - 1)  // slab tiles are 64 wide: A2 spans two A stages, B2 two B stages
        fast::slab<BKIND, BM, BN, TE>(p, reinterpret_cast<uint16_t*>(sa(0)), sb(0), acc, m0, n0, wm * WM, wn * WN, lane);
    fast::epilogue<FI, WN>(p, acc, reinterpret_cast<float*>(lds + OFF_A) + wave * (16 * (WN + 4)), m0 + wm * WM,
                           n0 + wn * WN, split, lane);
}

// ---------------------------------------------------------------------------
// Tall NF4 tile (M % 512 == 0, N % 64 == 0, K % 64 == 0): 512 x 64 on 8
// wavefronts stacked along M, each owning 64 rows x all 64 columns. The
// activation operand never passes through LDS: each wavefront loads its own
// 64 rows straight into registers (raw buffer loads, per-lane offsets fixed
// for the whole K loop plus a scalar offset per chunk), two chunks ahead of
// the MFMAs that read them. LDS holds only the weight side: the packed codes
// and block maxima of each 64-wide K chunk (DMA, three chunks ahead), the 16
// code values (a 64-byte table, so every lookup is conflict-free: lanes that
// read the same code share one bank word), and the dequantized bf16 tile in
// three stages. Each dequantized weight tile serves 512 rows and every
// wavefront reads it once per chunk, so the LDS traffic per MFMA is about
// 40% of the 256 x 128 tile's.
//
// The K index of a chunk is permuted inside the MFMA (a contraction does not
// care which k pairs with which, as long as both operands agree): lane group g
// (lane >> 4) of K step t holds k = 16 g + 8 t + (0..7), so the two 16-byte
// loads a lane makes per row and chunk are adjacent in memory; the weight
// tile is read with the same map.
namespace tall {
constexpr int BM = 512, BN = 64, NTH = 512, NW = 8, WM = 64, WN = 64, FI = WM / 16, FJ = WN / 16;
constexpr int SB = BN * 64 * 2;  // one bf16 weight stage: 8 KB
constexpr int SR = BN * 32;      // packed codes of one chunk: 2 KB
constexpr int SS = 2048;         // block maxima of one chunk: 8 x 64 floats (see CodePlan)
constexpr int OFF_L = 0, OFF_B = 256, OFF_R = OFF_B + 3 * SB, OFF_S = OFF_R + 3 * SR;
constexpr int LDS_MAIN = OFF_S + 3 * SS;
// the LoRA slab reuses LDS from 0 once the main loop has drained: A2 tile
// 512 x 64 bf16, then B2 64 x 64; the epilogue stages 8 x 16 x 68 floats
constexpr int SLAB_B = BM * 64 * 2;
constexpr int LDS_BYTES = (LDS_MAIN > SLAB_B + SB) ? LDS_MAIN : SLAB_B + SB;
static_assert(LDS_BYTES <= 160 * 1024 && NW * 16 * (WN + 4) * 4 <= LDS_BYTES, "tall NF4 tile LDS");
constexpr int NA = FI * 2;  // 16-byte activation loads per lane per chunk
constexpr int NR = 2;       // code + block-maximum DMAs per wavefront per chunk

// Activation loads: lane (r = lane & 15, g = lane >> 4) of wavefront w reads
// row 64 w + 16 i + r, bytes [32 g, 32 g + 32) of the chunk's 128.
struct APlan {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off[FI];
    __device__ __forceinline__ void init(const uint16_t* a0, int64_t lda, int wave, int lane) {
        rs = fast::rsrc(a0);
#pragma unroll
        for (int i = 0; i < FI; ++i)
            off[i] = uint32_t((int64_t(wave * WM + i * 16 + (lane & 15)) * lda + (lane >> 4) * 16) * 2);
    }
    __device__ __forceinline__ void load(uint32_t soff, uint4 (&a)[FI][2]) const {
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            a[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], soff, 0));
            a[i][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i] + 16, soff, 0));
        }
    }
};

// Codes and block maxima of one chunk, DMA'd into LDS, where a row is an
// output column n (NT) or a K row (NN): in both layouts a chunk is 64 rows of
// 32 code bytes and one block maximum per row. Wavefront w moves rows
// [8 w, 8 w + 8) with two 4-byte DMAs over all 64 lanes (no lane masked off,
// so the compiler's count of loads in flight stays exact): the codes as
// [row][32 bytes]; the maxima as 64 floats per wavefront, lane l holding row
// 8 w + (l & 7) (eight copies of each).
struct CodePlan {
    __amdgpu_buffer_rsrc_t rc, rs;
    uint32_t code, scale;
    int wave;
    __device__ __forceinline__ void init(const void* c0, const void* s0, int64_t cols, int lane) {
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rc = fast::rsrc(c0);
        rs = fast::rsrc(s0);
        code = uint32_t(int64_t(wave * 8 + (lane >> 3)) * (cols >> 1) + (lane & 7) * 4);
        scale = uint32_t(int64_t(wave * 8 + (lane & 7)) * (cols >> 6) * 4);
    }
    __device__ __forceinline__ void dma(uint32_t coff, uint32_t soff, char* __restrict__ raw,
                                        char* __restrict__ sc) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, fast::as_lds(raw + wave * 256), 4, code, coff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, fast::as_lds(sc + wave * 256), 4, scale, soff, 0, 0);
    }
};
// block maximum of row r (0..63) in a chunk's maxima stage
__device__ __forceinline__ float row_max(const float* s, int r) { return s[(r >> 3) * 64 + (r & 7)]; }

// Codes of one chunk (LDS) -> bf16 tile [64 n][64 k] (LDS, fast::swz layout):
// each thread produces one 16-byte chunk of one row, 8 consecutive k.
template <int BKIND, int TE>
__device__ __forceinline__ void dequant(const char* __restrict__ raw, const char* __restrict__ sc,
                                        const float* __restrict__ lut, uint16_t* __restrict__ tile) {
    const int t = threadIdx.x;
    const float* s = reinterpret_cast<const float*>(sc);
    uint32_t e[4];
    if constexpr (BKIND == B_NF4_NT) {
        // row n = t >> 3, k = 8 (t & 7) + (0..7): four code bytes, one block maximum
        const int n = t >> 3, q = t & 7;
        const uint32_t w = *reinterpret_cast<const uint32_t*>(raw + n * 32 + q * 4);
        const float a = row_max(s, n);
#pragma unroll
        for (int b = 0; b < 4; ++b)  // byte b: high nibble = even element
            e[b] = wpair<TE>(lut[(w >> (8 * b + 4)) & 15] * a, lut[(w >> (8 * b)) & 15] * a);
        *reinterpret_cast<uint4*>(tile + fast::swz(n, q)) = make_uint4(e[0], e[1], e[2], e[3]);
    } else {
        // column n = t & 63 of K rows 8 kc .. 8 kc + 7 (kc = t >> 6): one nibble
        // of each row's byte n / 2, each row with its own block maximum
        const int n = t & 63, kc = t >> 6, sh = (n & 1) ? 0 : 4;
        float v[8];
#pragma unroll
        for (int kr = 0; kr < 8; ++kr) {
            const uint32_t byte = *reinterpret_cast<const uint8_t*>(raw + (kc * 8 + kr) * 32 + (n >> 1));
            v[kr] = lut[(byte >> sh) & 15] * row_max(s, kc * 8 + kr);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) e[b] = wpair<TE>(v[2 * b], v[2 * b + 1]);
        *reinterpret_cast<uint4*>(tile + fast::swz(n, kc)) = make_uint4(e[0], e[1], e[2], e[3]);
    }
}

// One chunk of MFMAs: activation fragments from registers, weight fragments
// from the bf16 tile (row 16 j + (lane & 15), 16-byte chunk 2 g + t).
template <int TE>
__device__ __forceinline__ void mma(const uint4 (&a)[FI][2], const uint16_t* __restrict__ Bs, f32x4 (&acc)[FI][FJ],
                                    int lane) {
    const int lr = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        uint4 b[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) b[j] = *reinterpret_cast<const uint4*>(Bs + fast::swz(j * 16 + lr, 2 * g + t));
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) acc[i][j] = mfma16<TE>(a[i][t], b[j], acc[i][j]);
    }
}
}  // namespace tall

template <int BKIND, int TE>
__global__ __launch_bounds__(tall::NTH) void k_nf4_tall(const GemmParams p) {
    using namespace tall;
    extern __shared__ __align__(16) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float* lut = reinterpret_cast<float*>(lds + OFF_L);
    if (tid < 16) lut[tid] = nf4_value(tid);

    const TileIdx ti = tile_of(blockIdx.x, p.N / BN, p.M / BM, p.splits);
    const int m0 = ti.m * BM, n0 = ti.n * BN, split = ti.split;
    const int kbeg = split * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    const int nch = (kend - kbeg) / 64;  // >= 1
    const int64_t cols = p.nf4_cols;
    const int64_t flat0 = (BKIND == B_NF4_NN) ? int64_t(kbeg) * cols + n0 : int64_t(n0) * cols + kbeg;

    APlan ap;
    ap.init(p.A + int64_t(m0) * p.lda + kbeg, p.lda, wave, lane);
    CodePlan cp;
    cp.init(static_cast<const char*>(p.B) + (flat0 >> 1), p.absmax + (flat0 >> 6), cols, lane);
    // per chunk: codes 32 bytes on (NT) or 64 rows down (NN); maxima one
    // entry on (NT) or 64 rows down (NN); activations 128 bytes on
    const uint32_t cstep = (BKIND == B_NF4_NN) ? uint32_t(32 * cols) : 32u;
    const uint32_t sstep = (BKIND == B_NF4_NN) ? uint32_t(4 * cols) : 4u;

    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk c: activations in register set c % 3, codes and bf16 weights in
    // LDS stage c % 3; loads past the end re-read the last chunk into a set
    // or stage nobody reads again, so every step issues the same NA + NR
    // vector-memory instructions. The loop body is three whole steps (the
    // register sets rotate with period 3) and the last nch % 3 steps follow
    // it, so the register allocation of the loop is the same on every path.
    auto cl = [&](int c) { return uint32_t(min(c, nch - 1)); };
    auto sb = [&](int s) { return reinterpret_cast<uint16_t*>(lds + OFF_B + s * SB); };
    auto sr = [&](int s) { return lds + OFF_R + s * SR; };
    auto ss = [&](int s) { return lds + OFF_S + s * SS; };
    auto code_dma = [&](int c, int s) { cp.dma(cl(c) * cstep, cl(c) * sstep, sr(s), ss(s)); };
    uint4 ar[3][FI][2];
    code_dma(0, 0);
    code_dma(1, 1);
    ap.load(cl(0) * 128u, ar[0]);
    code_dma(2, 2);
    ap.load(cl(1) * 128u, ar[1]);
    fast::stage_sync<NA + NR + NA>();  // codes 0 and 1 (and the table) in LDS
    dequant<BKIND, TE>(sr(0), ss(0), lut, sb(0));
    fast::stage_sync<NA + NR + NA>();  // bf16 stage 0 complete
    auto step = [&](int c, auto r3) {
        constexpr int S0 = decltype(r3)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
        ap.load(cl(c + 2) * 128u, ar[S2]);
        code_dma(c + 3, S0);  // code stage c % 3 was dequantized last step
        tall::mma<TE>(ar[S0], sb(S0), acc, lane);
        dequant<BKIND, TE>(sr(S1), ss(S1), lut, sb(S1));
        fast::stage_sync<NA + NR>();  // codes c + 2 and activations c + 1 landed; bf16 c + 1 complete
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    const int nfull = nch - nch % 3;
    for (int c = 0; c < nfull; c += 3) {
        step(c, I0());
        step(c + 1, I1());
        step(c + 2, I2());
    }
    if (nfull < nch) step(nfull, I0());
    if (nfull + 1 < nch) step(nfull + 1, I1());
    fast::stage_sync<0>();

    if (p.K2 > 0 && split == p.splits - 1)  // LoRA slab, any K2 (zero-filled tail)
        fast::slab<BKIND, BM, BN, TE>(p, reinterpret_cast<uint16_t*>(lds), reinterpret_cast<uint16_t*>(lds + SLAB_B), acc,
                                  m0, n0, wave * WM, 0, lane);
    fast::epilogue<FI, WN>(p, acc, reinterpret_cast<float*>(lds) + wave * (16 * (WN + 4)), m0 + wave * WM, n0, split,
                           lane);
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
static bool aligned8(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 7) == 0; }

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
template <int BKIND, int TE>
static void launch_fast(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_nf4_tile<BKIND, TE>), fast::LDS_BYTES);
    hipExtLaunchKernelGGL(k_nf4_tile<BKIND, TE>, dim3(tiles * p.splits), dim3(fast::NTH), fast::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p);
}
// every (direction, element type, producer count) instance, named so both
// compiler passes emit it
template __global__ void k_nf4_ws<B_NF4_NT, TE_BF16, 4>(const GemmParams);
template __global__ void k_nf4_ws<B_NF4_NT, TE_F16, 4>(const GemmParams);
template __global__ void k_nf4_ws<B_NF4_NN, TE_BF16, 4>(const GemmParams);
template __global__ void k_nf4_ws<B_NF4_NN, TE_F16, 4>(const GemmParams);
template __global__ void k_nf4_ws<B_NF4_NT, TE_BF16, 8>(const GemmParams);
template __global__ void k_nf4_ws<B_NF4_NT, TE_F16, 8>(const GemmParams);
template __global__ void k_nf4_ws<B_NF4_NN, TE_BF16, 8>(const GemmParams);
template __global__ void k_nf4_ws<B_NF4_NN, TE_F16, 8>(const GemmParams);
// QLX_WS_NPW_NT / QLX_WS_NPW_NN (4 or 8) in the environment override the
// built-in producer counts, read per call
static int ws_npw(int bkind) {
    const char* e = std::getenv(bkind == B_NF4_NT ? "QLX_WS_NPW_NT" : "QLX_WS_NPW_NN");
    if (e && (e[0] == '4' || e[0] == '8') && e[1] == 0) return e[0] - '0';
    return bkind == B_NF4_NT ? QLX_WS_NPW_NT : QLX_WS_NPW_NN;
}
template <int BKIND, int TE, int NPW>
static void launch_ws_n(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_nf4_ws<BKIND, TE, NPW>), ws::LDS_BYTES);
    hipExtLaunchKernelGGL((k_nf4_ws<BKIND, TE, NPW>), dim3(tiles * p.splits), dim3(ws::Prod<NPW>::NTH),
                          ws::LDS_BYTES, s, prof.start(), prof.stop(), 0, p);
}
template <int BKIND, int TE>
static void launch_ws(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    if (ws_npw(BKIND) == 8) launch_ws_n<BKIND, TE, 8>(p, tiles, s, prof);
    else launch_ws_n<BKIND, TE, 4>(p, tiles, s, prof);
}
template __global__ void k_nf4_wsp<B_NF4_NT, TE_BF16, 8>(const GemmParams, const int);
template __global__ void k_nf4_wsp<B_NF4_NT, TE_F16, 8>(const GemmParams, const int);
template __global__ void k_nf4_wsp<B_NF4_NN, TE_BF16, 8>(const GemmParams, const int);
template __global__ void k_nf4_wsp<B_NF4_NN, TE_F16, 8>(const GemmParams, const int);
// compute units of the current device (one persistent workgroup each)
static int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    QLX_CHECK_HIP(hipGetDevice(&dev));
    QLX_REQUIRE(dev >= 0 && dev < 64, QLX_EUNSUPPORTED, "gemm: device index out of range");
    int n = cus[dev].load(std::memory_order_acquire);
    if (n == 0) {
        QLX_CHECK_HIP(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev));
        QLX_REQUIRE(n > 0, QLX_EUNSUPPORTED, "gemm: device reports no compute units");
        cus[dev].store(n, std::memory_order_release);
    }
    return n;
}
// QLX_NF4_PERSIST=0 keeps the one-tile-per-workgroup k_nf4_ws
static bool nf4_persist() {
    const char* e = std::getenv("QLX_NF4_PERSIST");
    return !(e && e[0] == '0');
}
// what k_nf4_wsp takes on top of the full-tile conditions (checked on the
// host: slab rows fetched 16 bytes at a time, plain outputs)
static bool wsp_ok(const GemmParams& p) {
    // (a residual only enters an unsplit output: split-K writes partials)
    if (p.seg_rows > 0 || p.accumulate || (p.R && p.splits == 1)) return false;
    if (p.splits > 1 ? !aligned16(p.partial)
                     : !(p.ldc % 4 == 0 && (p.c_type == C_F32 ? aligned16(p.C) : aligned8(p.C))))
        return false;
    return p.K2 == 0 || (p.K2 % 64 == 0 && p.a2_vec && aligned16(p.B2) && p.ldb2 % 8 == 0);
}
template <int BKIND, int TE>
static void launch_wsp(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_nf4_wsp<BKIND, TE, 8>), ws::LDS_BYTES);
    const int nitems = tiles * p.splits, cus = device_cus();
    // one workgroup per CU; a multiple of 8 whenever a workgroup takes several tiles
    const int G = nitems <= cus ? nitems : std::max(8, cus / 8 * 8);
    hipExtLaunchKernelGGL((k_nf4_wsp<BKIND, TE, 8>), dim3(G), dim3(ws::Prod<8>::NTH), ws::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p, nitems);
}
template <int BKIND, int TE>
static void launch_wide(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_nf4_wide<BKIND, TE>), wide::LDS_BYTES);
    hipExtLaunchKernelGGL(k_nf4_wide<BKIND, TE>, dim3(tiles * p.splits), dim3(wide::NTH), wide::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p);
}
template <int BKIND, int TE>
static void launch_tall(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_nf4_tall<BKIND, TE>), tall::LDS_BYTES);
    hipExtLaunchKernelGGL(k_nf4_tall<BKIND, TE>, dim3(tiles * p.splits), dim3(tall::NTH), tall::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p);
}
static void launch_dense(const GemmParams& p, int tiles, hipStream_t s, const ProfScope& prof) {
    static std::atomic<bool> allowed[64];
    allow_lds(allowed, reinterpret_cast<const void*>(&k_dense_tile<TE_F16>), dense::LDS_BYTES);
    hipExtLaunchKernelGGL(k_dense_tile<TE_F16>, dim3(tiles), dim3(dense::NTH), dense::LDS_BYTES, s, prof.start(),
                          prof.stop(), 0, p);
}

// Relative cost of one 64-wide chunk of the 512 x 64 NF4 tile against one of
// the 256 x 128 tile (same work per chunk): measured 1.4-1.8x on the 8B-shaped
// projections (its activation loads, one 16-byte fragment per lane straight
// from memory, move twice the bytes per MFMA through the vector memory path
// of the LDS-staged tiles), so the cost model never picks it.
constexpr double kTallUnit = 1.6;
// QLX_NF4_TILE = 256x128 | 512x128 | 512x64 pins the full-tile NF4 shape
// wherever it applies (for measurements); unset: chosen by the cost model.
// The 256 x 128 tile runs on the warp-specialized kernel (2-3% faster in the
// 8B-shaped steps, same bits); QLX_NF4_WS=0 selects k_nf4_tile instead
static bool nf4_ws() {
    const char* e = std::getenv("QLX_NF4_WS");
    return !(e && e[0] == '0');
}
static int nf4_shape_override() {
    const char* e = std::getenv("QLX_NF4_TILE");
    if (!e) return -1;
    const std::string v(e);
    return v == "256x128" ? 0 : v == "512x128" ? 1 : v == "512x64" ? 2 : -1;
}

// Kernel choice for one element type (every operand combination the step uses).
template <int TE>
static void dispatch(const GemmParams& p, int akind, int bkind, bool fast_ok, bool dense_fast, int shape, TileCfg tc,
                     int tiles, int bsz, hipStream_t s, const ProfScope& prof) {
    switch (akind * 10 + bkind) {
        case A_ROW * 10 + B_NF4_NT:
            if (fast_ok)
                shape == 2 ? launch_tall<B_NF4_NT, TE>(p, tiles, s, prof)
                : shape == 1 ? launch_wide<B_NF4_NT, TE>(p, tiles, s, prof)
                : nf4_ws()   ? (nf4_persist() && wsp_ok(p) ? launch_wsp<B_NF4_NT, TE>(p, tiles, s, prof)
                                                                : launch_ws<B_NF4_NT, TE>(p, tiles, s, prof))
                             : launch_fast<B_NF4_NT, TE>(p, tiles, s, prof);
            else
                launch_kind<A_ROW, B_NF4_NT, TE>(p, tc, bsz, s);
            break;
        case A_ROW * 10 + B_NF4_NN:
            if (fast_ok)
                shape == 2 ? launch_tall<B_NF4_NN, TE>(p, tiles, s, prof)
                : shape == 1 ? launch_wide<B_NF4_NN, TE>(p, tiles, s, prof)
                : nf4_ws()   ? (nf4_persist() && wsp_ok(p) ? launch_wsp<B_NF4_NN, TE>(p, tiles, s, prof)
                                                                : launch_ws<B_NF4_NN, TE>(p, tiles, s, prof))
                             : launch_fast<B_NF4_NN, TE>(p, tiles, s, prof);
            else
                launch_kind<A_ROW, B_NF4_NN, TE>(p, tc, bsz, s);
            break;
        case A_ROW * 10 + B_DENSE_NT:
            if (dense_fast && TE == TE_F16) launch_dense(p, tiles, s, prof);
            else if (tc.bm == 64 && tc.bn == 128) launch_cfg<A_ROW, B_DENSE_NT, TE, 64, 128, 32, 64>(p, bsz, s);
            else if (tc.bm == 64) launch_cfg<A_ROW, B_DENSE_NT, TE, 64, 64, 32, 32>(p, bsz, s);
            else launch_cfg<A_ROW, B_DENSE_NT, TE, 128, 128, 64, 64>(p, bsz, s);
            break;
        case A_ROW * 10 + B_DENSE_NN:
            if (tc.bm == 64 && tc.bn == 128) launch_cfg<A_ROW, B_DENSE_NN, TE, 64, 128, 32, 64>(p, bsz, s);
            else if (tc.bm == 64) launch_cfg<A_ROW, B_DENSE_NN, TE, 64, 64, 32, 32>(p, bsz, s);
            else launch_cfg<A_ROW, B_DENSE_NN, TE, 128, 128, 64, 64>(p, bsz, s);
            break;
        case A_TRANS * 10 + B_DENSE_NN:
            if (tc.bm == 64) launch_cfg<A_TRANS, B_DENSE_NN, TE, 64, 64, 32, 32>(p, bsz, s);
            else launch_cfg<A_TRANS, B_DENSE_NN, TE, 128, 128, 64, 64>(p, bsz, s);
            break;
        default: throw Error{QLX_EUNSUPPORTED, "gemm: operand combination not built"};
    }
}

void gemm_group_tn(GemmGroup g, int K, int te, const char* tag, hipStream_t s) {
    QLX_REQUIRE(g.n >= 1 && g.n <= kGemmGroupMax && K >= 1, QLX_EINVAL, "gemm group: 1..16 problems, K >= 1");
    constexpr int T = 64;  // 64 x 64 tiles on four 32 x 32 wavefronts
    GemmParams p;
    p.K = K;
    p.kchunk = ((K + BK - 1) / BK) * BK;
    p.splits = 1;
    p.c_type = C_F32;
    p.a_vec = p.b_vec = 1;
    int total = 0;
    double flops = 0, bytes = 0;
    for (int i = 0; i < g.n; ++i) {
        GemmProb& q = g.prob[i];
        QLX_REQUIRE(q.M >= 1 && q.N >= 1 && q.A && q.B && q.C, QLX_EINVAL, "gemm group: empty problem");
        p.a_vec &= aligned8(q.A) && q.lda % 4 == 0;
        p.b_vec &= aligned8(q.B) && q.ldb % 4 == 0;
        q.tile0 = total;
        total += ((q.M + T - 1) / T) * ((q.N + T - 1) / T);
        flops += 2.0 * q.M * q.N * K;
        bytes += (double(q.M) + q.N) * K * 2 + double(q.M) * q.N * 4;
    }
    ProfScope prof(tag, flops, bytes, s);
    if (te == TE_F16)
        hipLaunchKernelGGL((k_gemm_group<A_TRANS, B_DENSE_NN, TE_F16, T, T, 32, 32>), dim3(total), dim3(256), 0, s, p,
                           g);
    else
        hipLaunchKernelGGL((k_gemm_group<A_TRANS, B_DENSE_NN, TE_BF16, T, T, 32, 32>), dim3(total), dim3(256), 0, s,
                           p, g);
    check_launch("gemm group");
}

int gemm(GemmParams p, int akind, int bkind, int te, float* partial_ws, hipStream_t s) {
    if (p.M <= 0 || p.N <= 0) return 1;
    const bool nf4 = (bkind == B_NF4_NT || bkind == B_NF4_NN);
    QLX_REQUIRE(!(p.K2 > 0 && !nf4), QLX_EINVAL, "gemm: the LoRA slab rides only on NF4 GEMMs");
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
    const bool fast_ok = nf4 && akind == A_ROW && p.batch == 1 && p.causal == CAUSAL_NONE &&
                         p.M % fast::BM == 0 && p.N % fast::BN == 0 && p.K % 64 == 0 && p.K >= 64 && p.a_vec &&
                         p.b_vec && aligned16(p.absmax) && p.nf4_cols % 64 == 0 &&
                         int64_t(p.M) * p.lda * 2 < (int64_t(1) << 31) &&
                         int64_t(p.N) * p.K / 2 < (int64_t(1) << 31);  // never depends on the slab
    // Skinny dense products (the LoRA terms: one side is r, 2r or 3r) are
    // bound by reading the long operand; 64 x 64 tiles with a K split keep
    // many workgroups streaming it without a large partial buffer.
    const bool skinny = !nf4 && !p.ce_mode && p.batch == 1 && p.causal == CAUSAL_NONE && std::min(p.M, p.N) <= 256;
    // the LM head's fp16 NT products with a cross-entropy epilogue (never split)
    const bool dense_fast = p.ce_mode && te == TE_F16 && akind == A_ROW && bkind == B_DENSE_NT && p.batch == 1 &&
                            p.M % dense::BM == 0 && p.N % dense::BN == 0 && p.K % 64 == 0 && p.K >= 64 && p.a_vec &&
                            p.b_vec && int64_t(dense::BM) * p.lda * 2 + int64_t(p.K) * 2 < (int64_t(1) << 31) &&
                            int64_t(dense::BN) * p.ldb * 2 + int64_t(p.K) * 2 < (int64_t(1) << 31);
    const TileCfg tc = fast_ok ? TileCfg{fast::BM, fast::BN}
                       : dense_fast ? TileCfg{dense::BM, dense::BN}
                       : skinny     ? TileCfg{64, (akind == A_ROW && p.N % 128 == 0) ? 128 : 64}
                                    : pick_tile(p, bkind);
    const int gx = (p.N + tc.bn - 1) / tc.bn, gy = (p.M + tc.bm - 1) / tc.bm;
    // split-K when the grid would leave CUs idle: shapes decide, nothing else
    p.splits = 1;
    p.kchunk = ((p.K + BK - 1) / BK) * BK;
    int tiles = gx * gy;
    int shape = 0;  // full-tile NF4 kernels: 0 = 256 x 128, 1 = 512 x 128 (wide), 2 = 512 x 64 (tall)
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
        // tile shape: 0 = 256 x 128, 1 = 512 x 128, 2 = 512 x 64 (each chunk
        // of the 512 x 128 shape is two 256 x 128 chunks of work)
        const int forced = nf4_shape_override();
        // the 256 x 128 tile on the persistent kernel: the pipeline fills
        // once per launch, so a tile costs its chunks plus ~half a chunk.
        // Outputs decide, not which kernel runs: QLX_NF4_WS / QLX_NF4_PERSIST
        // swap kernels under the same split, so the bits stay comparable.
        const bool persist = p.seg_rows == 0 && !p.accumulate;
        for (int sh = 0; sh < 3; ++sh) {
            if (sh > 0 && p.M % 512 != 0) continue;
            if (forced >= 0 && sh != forced && !(forced > 0 && p.M % 512 != 0 && sh == 0)) continue;
            // the persistent 256 x 128 kernel measured at least as fast as the
            // 512 x 128 one on every 8B-shaped step (whole steps, one box)
            if (forced < 0 && sh == 1 && persist) continue;
            const int t = (p.M / (sh ? 512 : 256)) * (p.N / (sh == 2 ? 64 : 128));
            const double unit = sh == 1 ? 1.85 * 1.03 : sh == 2 ? kTallUnit : 1.0;
            for (int sp = 1; sp <= 16 && nch / sp >= 4; ++sp) {
                if (sp > 1 && (!partial_ws || size_t(sp) * p.M * p.N > p.partial_cap)) break;
                const int per = (nch + sp - 1) / sp;
                const double rounds = double((t * sp + 255) / 256);
                double cost = (sh == 0 && persist) ? rounds * (per + 0.5) + 3.0 : rounds * (per + 3.0) * unit;
                if (sp > 1) cost += mn * 4.0 * (sp + 1) / 4e12 / 1.35e-6 + 2.0;
                if (cost < best - 1e-9) best = cost, best_s = sp, shape = sh;
            }
        }
        if (best_s > 1) {
            const int kc = (nch + best_s - 1) / best_s * 64;
            p.kchunk = kc;
            p.splits = (p.K + kc - 1) / kc;
            p.partial = partial_ws;
        }
        wide_tile = shape == 1;
        if (shape == 1) tiles = (p.M / wide::BM) * (p.N / fast::BN);
        if (shape == 2) tiles = (p.M / tall::BM) * (p.N / tall::BN);
        } else if (skinny) {
        // measured on the 8B-shaped LoRA products: at least 512 workgroups
        // (four fit a CU), at most 2048 of K per split, at least 256, at most
        // 32 splits (16 left the 512-token products on 128 workgroups: the
        // step 1.4% slower); a product 128 (or a multiple) wide takes 64 x 128
        // tiles, so its long operand is read once rather than once per 64
        // columns
        if (partial_ws) {
            int sp = 1;
            while (sp < 32 && tiles * sp < 512) sp *= 2;
            while (sp < 32 && p.K / sp > 2048) sp *= 2;
            sp = std::min(sp, std::max(1, p.K / 256));
            while (sp > 1 && size_t(sp) * tiles * tc.bm * tc.bn > p.partial_cap) sp /= 2;
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
        while (want > 1 && size_t(want) * tiles * tc.bm * tc.bn > p.partial_cap) --want;
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
    const double belt = !nf4 ? 2.0 : 0.5 + 4.0 / 64.0;
    const double cb = p.c_type == C_F32 ? 4.0 : 2.0;
    // the cross-entropy epilogue writes no C: two floats per row and 64
    // columns, and the fp32 logits when they are kept
    const double out_bytes = p.ce_mode ? M * std::ceil(N / 64.0) * 8.0 + (p.ce_logits ? M * N * 4.0 : 0.0)
                                       : M * N * cb * (p.accumulate ? 2 : 1);
    const double bytes = p.batch * (M * K * 2 + N * K * belt + out_bytes + (p.R ? M * N * 4 : 0) +
                                    (p.K2 ? (M + N) * p.K2 * 2.0 : 0));
    static const char* kNames[] = {"gemm_nf4_nt", "gemm_nf4_nn", "gemm_bf16_nt", "gemm_bf16_nn",
                                   "gemm_bf16_tn", "gemm_f16_nt", "gemm_f16_nn", "gemm_other"};
    static const char* kWideNames[] = {"gemm_nf4_nt_wide", "gemm_nf4_nn_wide"};
    static const char* kTallNames[] = {"gemm_nf4_nt_tall", "gemm_nf4_nn_tall"};
    const int ab = akind * 10 + bkind;  // the NF4 rows keep their names under either activation type
    const int ni = ab == 0 ? 0 : ab == 1 ? 1 : key == 20 ? 2 : key == 30 ? 3 : key == 130 ? 4
                 : key == 21 ? 5 : key == 31 ? 6 : 7;
    const int bsz = p.batch * p.splits;
    {
        ProfScope prof(p.tag ? p.tag : (shape == 2 && fast_ok && ni < 2) ? kTallNames[ni]
                                     : (wide_tile ? kWideNames[ni] : kNames[ni]), flops, bytes, s,
                       fast_ok || dense_fast);
        if (te == TE_BF16) dispatch<TE_BF16>(p, akind, bkind, fast_ok, dense_fast, shape, tc, tiles, bsz, s, prof);
        else dispatch<TE_F16>(p, akind, bkind, fast_ok, dense_fast, shape, tc, tiles, bsz, s, prof);
        check_launch("gemm");
    }
    if (p.splits > 1 && !p.defer_reduce) {
        const int64_t MN = int64_t(p.M) * p.N;
        ProfScope prof("splitk_reduce", double(MN) * p.splits, double(MN) * (4.0 * p.splits + cb + (p.R ? 4 : 0)), s);
        const int64_t threads = (p.N & 3) == 0 ? MN / 4 : MN;
        hipLaunchKernelGGL(k_splitk_reduce, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, p);
        check_launch("gemm splitk reduce");
    }
    return p.splits;
}

}  // namespace qlx
