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
// masked by the epilogue. Tiles are ordered so the M-tiles sharing one weight
// tile run on the same XCD (one L2) together.
// Split-K writes fp32 partials that a second kernel sums in a fixed order:
// results depend only on shapes, never on timing or pointer values.
#include <algorithm>
#include <type_traits>

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
template <int R, int NT, bool SWZ = false>
struct TransLoader {
    static constexpr int U = (R / 4) * (BK / 8) / NT;
    static_assert(U >= 1 && (R / 4) * (BK / 8) % NT == 0, "trans loader shape");
    uint2 v[U][8];
    __device__ inline void load(const uint16_t* __restrict__ src, int64_t ld, int r0, int k0, int rows, int K,
                                int vec_ok) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = threadIdx.x + u * NT;
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
        if (row < p.M) {
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
// Full-tile NF4 kernel (M % 256 == 0, N % 128 == 0, K % 128 == 0, 16-byte
// aligned operands, NF4 rows a whole number of absmax blocks): a 256 x 128
// tile on 4 wavefronts (2 x 2) of 128 x 64. LDS tiles are unpadded, with each
// row's 16-byte chunk c stored at chunk c ^ ((row >> 1) & 7) so fragment reads
// and stores are bank-conflict free. Operands of chunk t+2 are loaded into
// registers while chunk t's MFMAs run and chunk t+1 is dequantized into the
// other LDS buffer; the body is branch-free (loads past the end re-read the
// last chunk) so the scheduler can interleave dequant VALU with the MFMAs.
namespace fast {
constexpr int BM = 256, BN = 128, NT = 256;
__device__ __forceinline__ int swz(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

// A tile (256 rows x 64 k, bf16) straight from global memory into the
// swizzled LDS layout with global_load_lds_dwordx4: each instruction writes
// 1 KB of LDS, lane l at byte 16*l, so every lane fetches the 16 bytes that
// belong at its slot. No registers, no VALU. The caller waits vmcnt(0) and
// barriers before the tile is read.
__device__ __forceinline__ void a_dma(const uint16_t* __restrict__ A, int64_t lda, int m0, int k0,
                                      uint16_t* __restrict__ tile) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int blk = wave * 8 + u;                   // 1 KB block = 8 rows
        const int r = blk * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);      // logical chunk stored at slot lane & 7
        __builtin_amdgcn_global_load_lds(A + int64_t(m0 + r) * lda + k0 + c * 8, tile + blk * 512, 16, 0, 0);
    }
}
// Scheduling hint for one chunk: spread the dequantization VALU and LDS
// traffic between the 64 MFMAs instead of after them.
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x3F70); }

// NF4 [N][K]: thread = half a row's 64-element block (16 bytes, one absmax)
struct Nf4Nt {
    uint4 w;
    float a;
    __device__ __forceinline__ void load(const uint8_t* __restrict__ P, const float* __restrict__ S, int64_t cols, int n0,
                                int k0) {
        const int64_t flat = int64_t(n0 + (threadIdx.x >> 1)) * cols + k0 + (threadIdx.x & 1) * 32;
        w = *reinterpret_cast<const uint4*>(P + (flat >> 1));
        a = S[flat >> 6];
    }
    __device__ __forceinline__ void store(uint16_t* __restrict__ tile, const float* lut) const {
        const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
        uint32_t e2[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t byte = (words[q] >> (8 * b)) & 0xFF;
                e2[q][b] = f32x2_to_bf16x2(lut[byte >> 4] * a, lut[byte & 15] * a);
            }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint4*>(tile + swz(r, half * 4 + q)) = make_uint4(e2[q][0], e2[q][1], e2[q][2], e2[q][3]);
    }
};

// NF4 [K][N]: thread = 4 consecutive n from 8 consecutive k rows
struct Nf4Nn {
    uint32_t two[8];
    float a[8];
    __device__ __forceinline__ void load(const uint8_t* __restrict__ P, const float* __restrict__ S, int64_t cols, int n0,
                                int k0) {
        const int ng = (threadIdx.x & 31) * 4, kg = (threadIdx.x >> 5) * 8;
#pragma unroll
        for (int kr = 0; kr < 8; ++kr) {
            const int64_t flat = int64_t(k0 + kg + kr) * cols + n0 + ng;
            two[kr] = *reinterpret_cast<const uint16_t*>(P + (flat >> 1));
            a[kr] = S[flat >> 6];
        }
    }
    __device__ __forceinline__ void store(uint16_t* __restrict__ tile, const float* lut) const {
        const int ng = (threadIdx.x & 31) * 4, kg = (threadIdx.x >> 5) * 8;
        uint32_t e2[8][2];
#pragma unroll
        for (int kr = 0; kr < 8; ++kr) {
            const uint32_t t = two[kr];
            e2[kr][0] = f32x2_to_bf16x2(lut[(t >> 4) & 15] * a[kr], lut[t & 15] * a[kr]);
            e2[kr][1] = f32x2_to_bf16x2(lut[(t >> 12) & 15] * a[kr], lut[(t >> 8) & 15] * a[kr]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = j >> 1, sh = (j & 1) * 16;
            uint32_t c[8];
#pragma unroll
            for (int kr = 0; kr < 8; ++kr) c[kr] = (e2[kr][h] >> sh) & 0xFFFFu;
            *reinterpret_cast<uint4*>(tile + swz(ng + j, kg >> 3)) =
                make_uint4(pack2(c[0], c[1]), pack2(c[2], c[3]), pack2(c[4], c[5]), pack2(c[6], c[7]));
        }
    }
};

// Fragment reads: row (base + i*16 + lr) swizzles with (lr >> 1) & 7 only, so
// each K half (kk) has one per-lane base and every fragment is base + an
// immediate offset.
__device__ __forceinline__ void mma(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                    f32x4 (&acc)[8][4], int wm, int wn, int lane) {
    const int lr = lane & 15, lc = lane >> 4, sw = (lr >> 1) & 7;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int ch = ((kk * 4 + lc) ^ sw) << 3;
        const uint16_t* ab = As + (wm * 128 + lr) * 64 + ch;
        const uint16_t* bb = Bs + (wn * 64 + lr) * 64 + ch;
        uint4 a[8], b[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const uint4*>(ab + i * 16 * 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const uint4*>(bb + j * 16 * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<TE_BF16>(a[i], b[j], acc[i][j]);
    }
}
}  // namespace fast

template <int BKIND>
__global__ __launch_bounds__(256) void k_nf4_tile(const GemmParams p) {
    using namespace fast;
    using BRegs = typename std::conditional<BKIND == B_NF4_NT, Nf4Nt, Nf4Nn>::type;
    __shared__ __align__(16) uint16_t A0[BM * 64];
    __shared__ __align__(16) uint16_t A1[BM * 64];
    __shared__ __align__(16) uint16_t B0[BN * 64];
    __shared__ __align__(16) uint16_t B1[BN * 64];
    __shared__ float lut[16];
    const int tid = threadIdx.x;
    if (tid < 16) lut[tid] = nf4_value(tid);

    const int gx = p.N / BN, gy = p.M / BM;
    const int ntile = gx * gy;
    int t = blockIdx.x;
    if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
    const int m0 = (t % gy) * BM, n0 = (t / gy) * BN;
    const int split = blockIdx.y;
    const int kbeg = split * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    const int nch = (kend - kbeg) / 64;  // even, >= 2
    const uint16_t* A = p.A;
    const uint8_t* P = static_cast<const uint8_t*>(p.B);
    const float* S = p.absmax;
    const int64_t cols = p.nf4_cols;

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk t+1: A by DMA into the other LDS buffer, B into registers, both
    // issued before chunk t's MFMAs; B is dequantized after them.
    BRegs rb;
    __syncthreads();  // lut
    a_dma(A, p.lda, m0, kbeg, A0);
    rb.load(P, S, cols, n0, kbeg);
    rb.store(B0, lut);
    wait_vmem_all();
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {
        {  // even chunk c in (A0, B0)
            const int kn = kbeg + (c + 1) * 64;
            a_dma(A, p.lda, m0, kn, A1);
            rb.load(P, S, cols, n0, kn);
            mma(A0, B0, acc, wm, wn, lane);
            rb.store(B1, lut);
            interleave_hint();
            wait_vmem_all();
            __syncthreads();
        }
        {  // odd chunk c+1 in (A1, B1)
            const int kn = kbeg + min(c + 2, nch - 1) * 64;
            a_dma(A, p.lda, m0, kn, A0);
            rb.load(P, S, cols, n0, kn);
            mma(A1, B1, acc, wm, wn, lane);
            rb.store(B0, lut);
            interleave_hint();
            wait_vmem_all();
            __syncthreads();
        }
    }
    if (p.K2 > 0 && split == p.splits - 1) {  // LoRA slab, any K2 (zero-filled tail)
        for (int k0 = 0; k0 < p.K2; k0 += 64) {
            RowLoader<BM, NT, true> la;
            la.load(p.A2, p.lda2, m0, k0, p.M, p.K2, p.a2_vec);
            if constexpr (BKIND == B_NF4_NT) {
                RowLoader<BN, NT, true> lb;
                lb.load(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec);
                lb.store(B0);
            } else {
                TransLoader<BN, NT, true> lb;
                lb.load(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec);
                lb.store(B0);
            }
            la.store(A0);
            __syncthreads();
            mma(A0, B0, acc, wm, wn, lane);
            __syncthreads();
        }
    }

    // epilogue (as the generic kernel): 16-row bands staged through LDS
    constexpr int WN = 64;
    float* stage = reinterpret_cast<float*>(A0) + wave * (16 * (WN + 4));
    const int srow = (lane >> 2) & 15;
    const int scol = (lane & 3) * (WN / 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) stage[((lane >> 4) * 4 + e) * (WN + 4) + j * 16 + (lane & 15)] = acc[i][j][e];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row = m0 + wm * 128 + i * 16 + srow;
        const int col0 = n0 + wn * WN + scol;
        const float* src = stage + srow * (WN + 4) + scol;
        if (p.splits > 1) {
            float* dst = p.partial + (int64_t(split) * p.M + row) * p.N + col0;
#pragma unroll
            for (int c = 0; c < WN / 4; c += 4)
                *reinterpret_cast<float4*>(dst + c) = make_float4(src[c], src[c + 1], src[c + 2], src[c + 3]);
        } else {
            store_row(p, 0, 0, row, col0, src, WN / 4);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

__global__ __launch_bounds__(256) void k_splitk_reduce(const GemmParams p) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t MN = int64_t(p.M) * p.N;
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

void gemm(GemmParams p, int akind, int bkind, int te, float* partial_ws, hipStream_t s) {
    if (p.M <= 0 || p.N <= 0) return;
    const bool nf4 = (bkind == B_NF4_NT || bkind == B_NF4_NN);
    QLX_REQUIRE(!(p.K2 > 0 && !nf4), QLX_EINVAL, "gemm: the LoRA slab rides only on NF4 GEMMs");
    QLX_REQUIRE(!(te == TE_F16 && nf4), QLX_EINVAL, "gemm: NF4 operands are bf16");
    // vector-load eligibility (uniform per launch; depends on layout, not data)
    if (akind == A_ROW) p.a_vec = aligned16(p.A) && p.lda % 8 == 0 && p.a_so % 8 == 0 && p.a_si % 8 == 0;
    else p.a_vec = aligned8(p.A) && p.lda % 4 == 0 && p.a_so % 4 == 0 && p.a_si % 4 == 0;
    if (bkind == B_NF4_NT) p.b_vec = aligned16(p.B) && p.nf4_cols % 64 == 0;
    else if (bkind == B_NF4_NN) p.b_vec = aligned16(p.B) && p.nf4_cols % 64 == 0;
    else if (bkind == B_DENSE_NT) p.b_vec = aligned16(p.B) && p.ldb % 8 == 0 && p.b_so % 8 == 0 && p.b_si % 8 == 0;
    else p.b_vec = aligned8(p.B) && p.ldb % 4 == 0 && p.b_so % 4 == 0 && p.b_si % 4 == 0;
    if (p.K2 > 0) {
        p.a2_vec = aligned16(p.A2) && p.lda2 % 8 == 0;
        p.b2_vec = (bkind == B_NF4_NT) ? (aligned16(p.B2) && p.ldb2 % 8 == 0) : (aligned8(p.B2) && p.ldb2 % 4 == 0);
    }
    const bool fast_ok = nf4 && te == TE_BF16 && akind == A_ROW && p.batch == 1 && p.causal == CAUSAL_NONE &&
                         p.M % 256 == 0 && p.N % 128 == 0 && p.K % 128 == 0 && p.K >= 128 && p.a_vec && p.b_vec &&
                         (bkind == B_NF4_NT || p.nf4_cols % 4 == 0);  // never depends on the slab
    const TileCfg tc = fast_ok ? TileCfg{256, 128} : pick_tile(p, bkind);
    const int gx = (p.N + tc.bn - 1) / tc.bn, gy = (p.M + tc.bm - 1) / tc.bm;
    // split-K when the grid would leave CUs idle: shapes decide, nothing else
    p.splits = 1;
    p.kchunk = ((p.K + BK - 1) / BK) * BK;
    const int tiles = gx * gy;
    if (fast_ok) {
        // about one workgroup per CU; every split gets an even number (>= 8) of 64-wide chunks
        if (partial_ws && tiles < 256) {
            int want = std::min((256 + tiles - 1) / tiles, std::min(p.K / 512, 16));
            while (want > 1 && size_t(want) * tiles * tc.bm * tc.bn > kGemmPartialFloats) --want;
            if (want > 1) {
                const int kc = (((p.K + want - 1) / want) + 127) / 128 * 128;
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
    const int ni = key == 0 ? 0 : key == 10 ? 1 : key == 20 ? 2 : key == 30 ? 3 : key == 130 ? 4
                 : key == 21 ? 5 : key == 31 ? 6 : 7;
    const int bsz = p.batch * p.splits;
    {
        ProfScope prof(kNames[ni], flops, bytes, s);
        switch (key) {
            case A_ROW * 100 + B_NF4_NT * 10 + TE_BF16:
                if (fast_ok)
                    hipLaunchKernelGGL(k_nf4_tile<B_NF4_NT>, dim3(tiles, p.splits), dim3(256), 0, s, p);
                else
                    launch_kind<A_ROW, B_NF4_NT, TE_BF16>(p, tc, bsz, s);
                break;
            case A_ROW * 100 + B_NF4_NN * 10 + TE_BF16:
                if (fast_ok)
                    hipLaunchKernelGGL(k_nf4_tile<B_NF4_NN>, dim3(tiles, p.splits), dim3(256), 0, s, p);
                else
                    launch_kind<A_ROW, B_NF4_NN, TE_BF16>(p, tc, bsz, s);
                break;
            case A_ROW * 100 + B_DENSE_NT * 10 + TE_BF16:
                launch_cfg<A_ROW, B_DENSE_NT, TE_BF16, 128, 128, 64, 64>(p, bsz, s);
                break;
            case A_ROW * 100 + B_DENSE_NN * 10 + TE_BF16:
                launch_cfg<A_ROW, B_DENSE_NN, TE_BF16, 128, 128, 64, 64>(p, bsz, s);
                break;
            case A_TRANS * 100 + B_DENSE_NN * 10 + TE_BF16:
                launch_cfg<A_TRANS, B_DENSE_NN, TE_BF16, 128, 128, 64, 64>(p, bsz, s);
                break;
            case A_ROW * 100 + B_DENSE_NT * 10 + TE_F16:
                launch_cfg<A_ROW, B_DENSE_NT, TE_F16, 128, 128, 64, 64>(p, bsz, s);
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
        hipLaunchKernelGGL(k_splitk_reduce, dim3(unsigned((MN + 255) / 256)), dim3(256), 0, s, p);
        check_launch("gemm splitk reduce");
    }
}

}  // namespace qlx
