// GEMM family on CDNA4 bf16/fp16 MFMA (v_mfma_f32_16x16x32_{bf16,f16}) with
// the NF4 dequantization fused into the weight-operand load.
//
// What it computes: C = alpha * (A . op(B) + A2 . op(B2)) (+ R) (+ C_old),
// fp32 accumulation. For the QLoRA linear (LoRA, Hu et al. 2021, section 4.1,
// on the NF4 base that the pages describe: rug.gal article "En detalle") the
// first phase runs over the frozen NF4 weight and the second phase ("slab",
// K2 = r or a few r) adds the LoRA term u . (sB)^T, so the adapter costs one
// short extra K stretch instead of a separate pass over the output.
//
// Structure (one workgroup = 256 threads = 4 wavefronts, tile 128 x 128,
// K chunks of 64):
//   global -> registers -> (NF4: unpack nibble, code value from a 16-entry LDS
//   table, * absmax, round to bf16) -> LDS tiles As[128][64+8], Bs[128][64+8]
//   stored k-contiguous -> each wavefront computes a 64 x 64 sub-tile as 4 x 4
//   MFMA 16x16x32 blocks, reading 16-byte fragments from LDS.
// Loaders exist for every layout the training step needs (A row-major or
// transposed; B NF4 [N][K] or [K][N], dense [N][K] or [K][N]), so no operand
// is ever transposed in memory. Edges (M, N, K not multiples of the tile) are
// zero-filled in the loaders and masked in the epilogue.
// Split-K writes fp32 partials that a second kernel sums in a fixed order:
// results depend only on shapes, never on timing or pointer values.
#include <algorithm>

#include "nf4_codes.h"
#include "qlx_internal.h"

namespace qlx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64, BKP = BK + 8, NTHR = 256;

template <int TE>
__device__ inline f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
    if constexpr (TE == TE_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

__device__ inline uint32_t pack2(uint16_t lo, uint16_t hi) { return uint32_t(lo) | (uint32_t(hi) << 16); }

// ---------------------------------------------------------------------------
// Row-major loader: tile[r][k] = src[(r0 + r) * ld + k0 + k] for r < 128,
// k < 64, zero outside [0, rows) x [0, K). Each thread moves 4 vectors of 8.
__device__ inline void load_rowmajor(const uint16_t* __restrict__ src, int64_t ld, int r0, int k0, int rows, int K,
                                     int vec_ok, uint16_t* __restrict__ tile) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int v = tid + it * NTHR;
        const int r = v >> 3, c = (v & 7) * 8;
        const int gr = r0 + r, gc = k0 + c;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (gr < rows) {
            const uint16_t* p = src + int64_t(gr) * ld + gc;
            if (vec_ok && gc + 8 <= K) {
                val = *reinterpret_cast<const uint4*>(p);
            } else {
                uint16_t e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) e[j] = (gc + j < K) ? p[j] : uint16_t(0);
                val = make_uint4(pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7]));
            }
        }
        *reinterpret_cast<uint4*>(tile + r * BKP + c) = val;
    }
}

// Transposed loader: tile[r][k] = src[(k0 + k) * ld + r0 + r]. Each thread
// reads 4 consecutive r from 8 consecutive k rows and writes 4 k-contiguous
// 16-byte vectors.
__device__ inline void load_transposed(const uint16_t* __restrict__ src, int64_t ld, int r0, int k0, int rows, int K,
                                       int vec_ok, uint16_t* __restrict__ tile) {
    const int tid = threadIdx.x;
    const int rg = (tid & 31) * 4, kg = (tid >> 5) * 8;
    uint16_t e[8][4];
#pragma unroll
    for (int kr = 0; kr < 8; ++kr) {
        const int gk = k0 + kg + kr;
        const int gr = r0 + rg;
        if (gk < K) {
            const uint16_t* p = src + int64_t(gk) * ld + gr;
            if (vec_ok && gr + 4 <= rows) {
                const uint2 w = *reinterpret_cast<const uint2*>(p);
                e[kr][0] = uint16_t(w.x);
                e[kr][1] = uint16_t(w.x >> 16);
                e[kr][2] = uint16_t(w.y);
                e[kr][3] = uint16_t(w.y >> 16);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) e[kr][j] = (gr + j < rows) ? p[j] : uint16_t(0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) e[kr][j] = 0;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 val = make_uint4(pack2(e[0][j], e[1][j]), pack2(e[2][j], e[3][j]), pack2(e[4][j], e[5][j]),
                                     pack2(e[6][j], e[7][j]));
        *reinterpret_cast<uint4*>(tile + (rg + j) * BKP + kg) = val;
    }
}

__device__ inline uint16_t nf4_elem(const uint8_t* __restrict__ packed, const float* __restrict__ absmax,
                                    int64_t flat, const float* lut) {
    const uint32_t byte = packed[flat >> 1];
    const int code = (flat & 1) ? int(byte & 15) : int(byte >> 4);
    return f32_to_bf16_bits(lut[code] * absmax[flat >> 6]);
}

// NF4 weight stored [N][K] (flat n*cols + k): tile[n][k] = bf16(c[code] * absmax).
// Fast path: two threads per row, 32 codes (16 bytes) each, one absmax.
__device__ inline void load_nf4_nt(const uint8_t* __restrict__ packed, const float* __restrict__ absmax, int64_t cols,
                                   int n0, int k0, int N, int K, int aligned, const float* lut,
                                   uint16_t* __restrict__ tile) {
    const int tid = threadIdx.x;
    const int r = tid >> 1, half = tid & 1;
    const int gn = n0 + r, gk = k0 + half * 32;
    uint16_t* dst = tile + r * BKP + half * 32;
    if (gn < N && aligned && gk + 32 <= K) {
        const int64_t flat = int64_t(gn) * cols + gk;
        const uint4 w = *reinterpret_cast<const uint4*>(packed + (flat >> 1));
        const float a = absmax[flat >> 6];
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint16_t o[8];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t byte = (words[q] >> (8 * b)) & 0xFF;
                o[2 * b] = f32_to_bf16_bits(lut[byte >> 4] * a);
                o[2 * b + 1] = f32_to_bf16_bits(lut[byte & 15] * a);
            }
            *reinterpret_cast<uint4*>(dst + q * 8) = *reinterpret_cast<uint4*>(o);
        }
    } else {
        for (int j = 0; j < 32; ++j) {
            const int k = gk + j;
            dst[j] = (gn < N && k < K) ? nf4_elem(packed, absmax, int64_t(gn) * cols + k, lut) : uint16_t(0);
        }
    }
}

// NF4 weight stored [K][N] (flat k*cols + n): tile[n][k]. Each thread dequantizes
// 4 consecutive n (2 bytes) from 8 consecutive k rows and writes 4 vectors.
__device__ inline void load_nf4_nn(const uint8_t* __restrict__ packed, const float* __restrict__ absmax, int64_t cols,
                                   int n0, int k0, int N, int K, int aligned, const float* lut,
                                   uint16_t* __restrict__ tile) {
    const int tid = threadIdx.x;
    const int ng = (tid & 31) * 4, kg = (tid >> 5) * 8;
    const int gn = n0 + ng;
    uint16_t e[8][4];
#pragma unroll
    for (int kr = 0; kr < 8; ++kr) {
        const int gk = k0 + kg + kr;
        if (gk < K && aligned && gn + 4 <= N) {
            const int64_t flat = int64_t(gk) * cols + gn;
            const uint32_t two = *reinterpret_cast<const uint16_t*>(packed + (flat >> 1));
            const float a = absmax[flat >> 6];
            e[kr][0] = f32_to_bf16_bits(lut[(two >> 4) & 15] * a);
            e[kr][1] = f32_to_bf16_bits(lut[two & 15] * a);
            e[kr][2] = f32_to_bf16_bits(lut[(two >> 12) & 15] * a);
            e[kr][3] = f32_to_bf16_bits(lut[(two >> 8) & 15] * a);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                e[kr][j] = (gk < K && gn + j < N) ? nf4_elem(packed, absmax, int64_t(gk) * cols + gn + j, lut)
                                                  : uint16_t(0);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 val = make_uint4(pack2(e[0][j], e[1][j]), pack2(e[2][j], e[3][j]), pack2(e[4][j], e[5][j]),
                                     pack2(e[6][j], e[7][j]));
        *reinterpret_cast<uint4*>(tile + (ng + j) * BKP + kg) = val;
    }
}

// One K chunk of MFMAs: wavefront (wm, wn) owns rows wm*64.. and cols wn*64..
template <int TE>
__device__ inline void mma_chunk(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs, f32x4 (&acc)[4][4],
                                 int wm, int wn, int lane) {
    const int lr = lane & 15, lk = (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
        uint4 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 16 + lr) * BKP + kk + lk);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + j * 16 + lr) * BKP + kk + lk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<TE>(a[i], b[j], acc[i][j]);
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

template <int AK, int BKIND, int TE>
__global__ __launch_bounds__(NTHR) void k_gemm(const GemmParams p) {
    __shared__ __align__(16) uint16_t As[BM * BKP];
    __shared__ __align__(16) uint16_t Bs[BN * BKP];
    __shared__ float lut[16];
    constexpr bool kNf4 = (BKIND == B_NF4_NT || BKIND == B_NF4_NN);
    const int tid = threadIdx.x;
    if (kNf4 && tid < 16) lut[tid] = nf4_value(tid);

    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int split = blockIdx.z % p.splits;
    const int bz = blockIdx.z / p.splits;
    const int bo = bz / p.zdiv, bi = bz % p.zdiv;
    if (p.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;  // tile strictly above the diagonal

    const uint16_t* A = p.A + int64_t(bo) * p.a_so + int64_t(bi / p.a_grp) * p.a_si;
    const uint16_t* Bd = static_cast<const uint16_t*>(p.B) + (kNf4 ? 0 : int64_t(bo) * p.b_so + int64_t(bi / p.b_grp) * p.b_si);
    const uint8_t* Bq = static_cast<const uint8_t*>(p.B);

    int kbeg = split * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    if (p.causal == CAUSAL_K_LE_M) kend = min(kend, m0 + BM);
    if (p.causal == CAUSAL_K_GE_M) kbeg = max(kbeg, (m0 / BK) * BK);

    const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = kbeg; k0 < kend; k0 += BK) {
        __syncthreads();
        if (AK == A_ROW) load_rowmajor(A, p.lda, m0, k0, p.M, p.K, p.a_vec, As);
        else load_transposed(A, p.lda, m0, k0, p.M, p.K, p.a_vec, As);
        if (BKIND == B_NF4_NT) load_nf4_nt(Bq, p.absmax, p.nf4_cols, n0, k0, p.N, p.K, p.b_vec, lut, Bs);
        else if (BKIND == B_NF4_NN) load_nf4_nn(Bq, p.absmax, p.nf4_cols, n0, k0, p.N, p.K, p.b_vec, lut, Bs);
        else if (BKIND == B_DENSE_NT) load_rowmajor(Bd, p.ldb, n0, k0, p.N, p.K, p.b_vec, Bs);
        else load_transposed(Bd, p.ldb, n0, k0, p.N, p.K, p.b_vec, Bs);
        __syncthreads();
        mma_chunk<TE>(As, Bs, acc, wm, wn, lane);
    }
    if (kNf4 && p.K2 > 0 && split == p.splits - 1) {
        for (int k0 = 0; k0 < p.K2; k0 += BK) {
            __syncthreads();
            load_rowmajor(p.A2, p.lda2, m0, k0, p.M, p.K2, p.a2_vec, As);
            if (BKIND == B_NF4_NT) load_rowmajor(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec, Bs);
            else load_transposed(p.B2, p.ldb2, n0, k0, p.N, p.K2, p.b2_vec, Bs);
            __syncthreads();
            mma_chunk<TE>(As, Bs, acc, wm, wn, lane);
        }
    }

    // epilogue: lane holds rows (lane/16)*4 + e of each 16x16 block, column lane%16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + j * 16 + (lane & 15);
            if (col >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
                if (row >= p.M) continue;
                if (p.splits > 1) p.partial[(int64_t(split) * p.M + row) * p.N + col] = acc[i][j][e];
                else store_out(p, bo, bi, row, col, acc[i][j][e]);
            }
        }
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
template <int AK, int BKIND, int TE>
static void launch(const GemmParams& p, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((k_gemm<AK, BKIND, TE>), grid, dim3(NTHR), 0, s, p);
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
    else if (bkind == B_NF4_NN) p.b_vec = aligned16(p.B) && p.nf4_cols % 4 == 0;
    else if (bkind == B_DENSE_NT) p.b_vec = aligned16(p.B) && p.ldb % 8 == 0 && p.b_so % 8 == 0 && p.b_si % 8 == 0;
    else p.b_vec = aligned8(p.B) && p.ldb % 4 == 0 && p.b_so % 4 == 0 && p.b_si % 4 == 0;
    if (p.K2 > 0) {
        p.a2_vec = aligned16(p.A2) && p.lda2 % 8 == 0;
        p.b2_vec = (bkind == B_NF4_NT) ? (aligned16(p.B2) && p.ldb2 % 8 == 0) : (aligned8(p.B2) && p.ldb2 % 4 == 0);
    }
    const int gx = (p.N + BN - 1) / BN, gy = (p.M + BM - 1) / BM;
    // split-K for under-filled grids (256 CUs): shapes decide, nothing else
    p.splits = 1;
    p.kchunk = ((p.K + BK - 1) / BK) * BK;
    if (p.batch == 1 && p.causal == CAUSAL_NONE && partial_ws && p.K >= 1024) {
        const int tiles = gx * gy;
        int want = 512 / tiles;
        want = std::min(want, p.K / 512);
        want = std::min(want, 16);
        while (want > 1 && size_t(want) * tiles * BM * BN > kGemmPartialFloats) --want;
        if (want > 1) {
            const int kc = (((p.K + want - 1) / want) + BK - 1) / BK * BK;
            p.kchunk = kc;
            p.splits = (p.K + kc - 1) / kc;
            p.partial = partial_ws;
        }
    }
    QLX_REQUIRE(p.batch >= 1 && p.batch * p.splits <= 65535, QLX_EUNSUPPORTED, "gemm: grid.z too large");
    dim3 grid(gx, gy, p.batch * p.splits);
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
    {
    ProfScope prof(kNames[ni], flops, bytes, s);
    switch (key) {
        case A_ROW * 100 + B_NF4_NT * 10 + TE_BF16: launch<A_ROW, B_NF4_NT, TE_BF16>(p, grid, s); break;
        case A_ROW * 100 + B_NF4_NN * 10 + TE_BF16: launch<A_ROW, B_NF4_NN, TE_BF16>(p, grid, s); break;
        case A_ROW * 100 + B_DENSE_NT * 10 + TE_BF16: launch<A_ROW, B_DENSE_NT, TE_BF16>(p, grid, s); break;
        case A_ROW * 100 + B_DENSE_NN * 10 + TE_BF16: launch<A_ROW, B_DENSE_NN, TE_BF16>(p, grid, s); break;
        case A_TRANS * 100 + B_DENSE_NN * 10 + TE_BF16: launch<A_TRANS, B_DENSE_NN, TE_BF16>(p, grid, s); break;
        case A_ROW * 100 + B_DENSE_NT * 10 + TE_F16: launch<A_ROW, B_DENSE_NT, TE_F16>(p, grid, s); break;
        case A_ROW * 100 + B_DENSE_NN * 10 + TE_F16: launch<A_ROW, B_DENSE_NN, TE_F16>(p, grid, s); break;
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
