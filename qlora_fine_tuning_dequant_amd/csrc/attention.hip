// Causal grouped-query attention, flash-style (the score matrix is never
// stored): forward with an online softmax that keeps each query's log-sum-exp
// for the backward, and a backward that recomputes the probabilities block by
// block. The method is the Llama decoder's attention (softmax(q k^T / sqrt(d)
// + causal mask) v, grouped-query: nH / nKV query heads share one key/value
// head); the tiling is the FlashAttention scheme (Dao et al., 2022; Dao,
// 2023) written for CDNA4 wave64 MFMA v_mfma_f32_16x16x32_bf16.
//
// Forward, one workgroup per (64 queries, head, sequence), 4 wavefronts of
// 16 queries. It computes S^T = K Q^T rather than S, so each lane holds the
// scores of ONE query (4 keys per 16-key tile): the running max and sum are
// per-lane scalars shared by the 4 lanes of a query, the rescale of the
// output is a per-lane multiply, and the probabilities already sit in the
// layout of the B operand of O^T += V^T P^T (V^T fragments come from the
// row-major V tile through the transposing LDS read).
// P is rounded to the 16-bit operand type for that product; the running sum
// uses the fp32 values.
//
// RoPE (rotate-half, pairs (j, j + hd/2)) is applied to q|k in place by one
// launch before the forward (rotating while loading would redo each key
// block's rotation for every query block that stages it). The backward rotates
// dq back in registers before its store (a lane's dims d and d + hd/2 sit in
// accumulator tiles dt and dt + hd/32) and dk in the GQA reduce, so dq|dk
// come out as gradients of the unrotated q|k.
//
// Backward (deterministic, no atomics): D_q = sum_d dO o; dK/dV per (key block
// of 64, query head), each wavefront owning 16 keys and walking the query
// blocks at or after its own (S = Q K^T here, so each lane holds one KEY and
// P^T, dS^T are A operands in registers); the per-head fp32 dK, dV are then
// summed over the heads of a group in a fixed order by the GQA reduce. dQ in a
// separate pass per (64 queries, head), S^T formulation as in the forward.
#include <cmath>

#include "nf4_codes.h"
#include "partials.h"
#include "qlx_internal.h"

namespace qlx {

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-bit operands are bf16 (TE_BF16) or fp16 (TE_F16): q, k, v, o, dO, and
// the probabilities and score gradients rounded for the products.
template <int TE>
__device__ inline f32x4 mfma(const uint4& a, const uint4& b, f32x4 c) {
    if constexpr (TE == TE_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
}
template <int TE>
__device__ inline uint32_t pack2(float lo, float hi) {
    if constexpr (TE == TE_BF16) return f32x2_to_bf16x2(lo, hi);
    else return f32x2_to_f16x2(lo, hi);
}

constexpr int QB = 64;       // queries (or keys) per workgroup block
constexpr float kLog2e = 1.4426950408889634f;

// A block's rows in two halves, so its global loads can be in flight while
// the previous block computes: load_rows takes rows [r0, r0 + 64) x HD of a
// [T, ld] 16-bit matrix (column offset col) into registers, rows at or past
// `rows` as zeros; store_rows puts them into LDS row-major (stride HD + 8).
// 256 threads: 4 per row, HD/4 columns each.
template <int HD>
__device__ inline void load_rows(const uint16_t* __restrict__ src, int64_t ld, int64_t base_row, int r0, int rows,
                                 int64_t col, uint4 (&v)[HD / 32]) {
    const int tid = threadIdx.x, r = tid >> 2, part = tid & 3;
    const bool ok = r0 + r < rows;
    const uint16_t* s = src + (base_row + r0 + r) * ld + col + part * (HD / 4);
#pragma unroll
    for (int c8 = 0; c8 < HD / 32; ++c8) v[c8] = ok ? *reinterpret_cast<const uint4*>(s + c8 * 8) : make_uint4(0, 0, 0, 0);
}
template <int HD>
__device__ inline void store_rows(const uint4 (&v)[HD / 32], uint16_t* __restrict__ dst_row) {
    const int tid = threadIdx.x, r = tid >> 2, part = tid & 3;
#pragma unroll
    for (int c8 = 0; c8 < HD / 32; ++c8)
        *reinterpret_cast<uint4*>(dst_row + r * (HD + 8) + part * (HD / 4) + c8 * 8) = v[c8];
}

// A-operand fragment of the transposed block (columns = the 64 block rows)
// for a 32-wide slice js, in the order the accumulator layout hands out rows:
// lane (column d = lane & 15 of the 16-column tile dt, group g = lane >> 4)
// takes block rows 32 js + 4 g + {0..3} and 32 js + 16 + 4 g + {0..3}.
// It is read from the row-major tile (HD + 8 elements per row) with gfx950's
// transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i points at row r0 + i / 4, columns c0 + 4 (i % 4) .. + 3, and lane j
// receives column c0 + j of rows r0 .. r0 + 3. So no transposed copy of the
// tile is staged (its 2-byte LDS stores cost more than the products they
// feed).
__device__ inline uint2 tr_read(const uint16_t* p) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4* lds_s4_t;
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_s4_t>(uint32_t(reinterpret_cast<uintptr_t>(p))));
    return __builtin_bit_cast(uint2, v);
}
template <int HD>
__device__ inline uint4 trfrag(const uint16_t* __restrict__ t, int dt, int js, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const uint16_t* p = t + (js * 32 + g * 4 + (i >> 2)) * (HD + 8) + dt * 16 + (i & 3) * 4;
    const uint2 lo = tr_read(p);
    const uint2 hi = tr_read(p + 16 * (HD + 8));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

}  // namespace

// ------------------------------------------------------------------ forward
template <int HD, int TE>
__global__ __launch_bounds__(256) void k_flash_fwd(const AttnArgs a) {
    __shared__ __align__(16) uint16_t Ks[QB * (HD + 8)];
    __shared__ __align__(16) uint16_t Vs[QB * (HD + 8)];
    const int nqb = (a.S + QB - 1) / QB;
    const int qb = nqb - 1 - int(blockIdx.x);  // longest (latest) query blocks first
    const int h = blockIdx.y, b = blockIdx.z, kh = h / (a.nH / a.nKV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
    const int q = qb * QB + wave * 16 + lr;
    const int64_t row0 = int64_t(b) * a.S;
    uint4 qf[HD / 32];
#pragma unroll
    for (int ds = 0; ds < HD / 32; ++ds)
        qf[ds] = q < a.S ? *reinterpret_cast<const uint4*>(a.qkv + (row0 + q) * a.ld + int64_t(h) * HD + ds * 32 + g * 8)
                         : make_uint4(0, 0, 0, 0);
    f32x4 o[HD / 16];
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    const float c = a.scale * kLog2e;
    const int64_t kcol = a.qdim + int64_t(kh) * HD, vcol = kcol + a.kvdim;
    uint4 kr[HD / 32], vr[HD / 32];  // the next key block, in flight during this one's compute
    load_rows<HD>(a.qkv, a.ld, row0, 0, a.S, kcol, kr);
    load_rows<HD>(a.qkv, a.ld, row0, 0, a.S, vcol, vr);
    for (int kb = 0; kb <= qb; ++kb) {
        store_rows<HD>(kr, Ks);
        store_rows<HD>(vr, Vs);
        __syncthreads();
        if (kb < qb) {
            load_rows<HD>(a.qkv, a.ld, row0, (kb + 1) * QB, a.S, kcol, kr);
            load_rows<HD>(a.qkv, a.ld, row0, (kb + 1) * QB, a.S, vcol, vr);
        }
        f32x4 st[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < HD / 32; ++ds)
                st[kt] = mfma<TE>(*reinterpret_cast<const uint4*>(Ks + (kt * 16 + lr) * (HD + 8) + ds * 32 + g * 8), qf[ds],
                              st[kt]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = kb * QB + kt * 16 + g * 4 + e;
                if (key > q || key >= a.S) st[kt][e] = -INFINITY;
                mx = fmaxf(mx, st[kt][e]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m, mx);  // finite: key block 0 holds key 0 <= q
        const float alpha = exp2f((m - mnew) * c);
        m = mnew;
        const float mc = m * c;
        float ps = 0.f;
        uint32_t pk[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2f(fmaf(st[kt][e], c, -mc));
                ps += p[e];
            }
            pk[kt][0] = pack2<TE>(p[0], p[1]);
            pk[kt][1] = pack2<TE>(p[2], p[3]);
        }
        l = l * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            const uint4 pf = make_uint4(pk[2 * js][0], pk[2 * js][1], pk[2 * js + 1][0], pk[2 * js + 1][1]);
#pragma unroll
            for (int dt = 0; dt < HD / 16; ++dt) o[dt] = mfma<TE>(trfrag<HD>(Vs, dt, js, lane), pf, o[dt]);
        }
        __syncthreads();
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (q >= a.S) return;
    const float inv = 1.f / l;
    uint16_t* dst = a.o + (row0 + q) * a.ldo + int64_t(h) * HD + g * 4;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
        *reinterpret_cast<uint2*>(dst + dt * 16) =
            make_uint2(pack2<TE>(o[dt][0] * inv, o[dt][1] * inv), pack2<TE>(o[dt][2] * inv, o[dt][3] * inv));
    if (g == 0) a.lse[(int64_t(b) * a.nH + h) * a.S + q] = m * a.scale + logf(l);
}

// ------------------------------------------------------------------ backward
// D[b, h, q] = sum_d dO[q, h d] o[q, h d]: hd/8 lanes per (query, head),
// each with one 16-byte load of dO and of o (consecutive lanes read
// consecutive bytes of a token row), joined by xor shuffles in a fixed order.
template <int TE, bool PART>
__global__ __launch_bounds__(256) void k_flash_bwd_dot(const AttnArgs a, int hd) {
    const int L = hd / 8;  // 8 or 16 lanes per (query, head)
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t T = int64_t(a.B) * a.S;
    const int64_t pair = idx / L;
    const int part = int(idx % L);
    const bool live = pair < T * a.nH;
    const int64_t pc = live ? pair : 0;
    const int64_t t = pc / a.nH;
    const int h = int(pc % a.nH);
    uint4 u;
    if constexpr (PART) {  // dO from the o projection's split-K partials, rounded as its reduce pass would
        const int64_t i = t * a.qdim + int64_t(h) * hd + part * 8;
        const float4 x0 = part_sum4(a.dO_part, i, 0), x1 = part_sum4(a.dO_part, i + 4, 0);
        const bool f = TE == TE_F16;
        u = make_uint4(f32x2_to_act2(x0.x, x0.y, f), f32x2_to_act2(x0.z, x0.w, f), f32x2_to_act2(x1.x, x1.y, f),
                       f32x2_to_act2(x1.z, x1.w, f));
        if (live) *reinterpret_cast<uint4*>(a.dO_out + t * a.ldo + int64_t(h) * hd + part * 8) = u;
    } else {
        u = *reinterpret_cast<const uint4*>(a.dO + t * a.ldo + int64_t(h) * hd + part * 8);
    }
    const uint4 v = *reinterpret_cast<const uint4*>(a.O + t * a.ldo + int64_t(h) * hd + part * 8);
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w}, vw[4] = {v.x, v.y, v.z, v.w};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (TE == TE_BF16) {
            s = fmaf(__builtin_bit_cast(float, uw[e] << 16), __builtin_bit_cast(float, vw[e] << 16), s);
            s = fmaf(__builtin_bit_cast(float, uw[e] & 0xFFFF0000u), __builtin_bit_cast(float, vw[e] & 0xFFFF0000u), s);
        } else {
            s = fmaf(f16_bits_to_f32(uint16_t(uw[e])), f16_bits_to_f32(uint16_t(vw[e])), s);
            s = fmaf(f16_bits_to_f32(uint16_t(uw[e] >> 16)), f16_bits_to_f32(uint16_t(vw[e] >> 16)), s);
        }
    }
    for (int off = L / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (live && part == 0) {
        const int64_t b = t / a.S, qi = t % a.S;
        a.Dq[(b * a.nH + h) * a.S + qi] = s;
    }
}

// dK_h, dV_h (fp32, per query head) for one block of 64 keys.
template <int HD, int TE>
__global__ __launch_bounds__(256) void k_flash_bwd_kv(const AttnArgs a) {
    __shared__ __align__(16) uint16_t Qs[QB * (HD + 8)];
    __shared__ __align__(16) uint16_t Ds[QB * (HD + 8)];  // dO
    __shared__ float lse_s[QB], dq_s[QB];
    const int nkb = (a.S + QB - 1) / QB;
    const int kb = int(blockIdx.x);  // early key blocks see the most queries
    const int h = blockIdx.y, b = blockIdx.z, kh = h / (a.nH / a.nKV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
    const int key = kb * QB + wave * 16 + lr;  // this lane's key (B-operand column of S and dP)
    const int64_t row0 = int64_t(b) * a.S;
    const int64_t kcol = a.qdim + int64_t(kh) * HD, vcol = kcol + a.kvdim;
    uint4 kf[HD / 32], vf[HD / 32];
#pragma unroll
    for (int ds = 0; ds < HD / 32; ++ds) {
        const bool ok = key < a.S;
        kf[ds] = ok ? *reinterpret_cast<const uint4*>(a.qkv + (row0 + key) * a.ld + kcol + ds * 32 + g * 8)
                    : make_uint4(0, 0, 0, 0);
        vf[ds] = ok ? *reinterpret_cast<const uint4*>(a.qkv + (row0 + key) * a.ld + vcol + ds * 32 + g * 8)
                    : make_uint4(0, 0, 0, 0);
    }
    f32x4 dk[HD / 16], dv[HD / 16];
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float c = a.scale * kLog2e;
    const int64_t zrow = (int64_t(b) * a.nH + h) * a.S;
    uint4 qr[HD / 32], dr[HD / 32];  // the next query block, in flight during this one's compute
    load_rows<HD>(a.qkv, a.ld, row0, kb * QB, a.S, int64_t(h) * HD, qr);
    load_rows<HD>(a.dO, a.ldo, row0, kb * QB, a.S, int64_t(h) * HD, dr);
    for (int qb = kb; qb < nkb; ++qb) {
        store_rows<HD>(qr, Qs);
        store_rows<HD>(dr, Ds);
        if (tid < QB) {
            const int qq = qb * QB + tid;
            lse_s[tid] = qq < a.S ? a.lse[zrow + qq] * kLog2e : 0.f;
            dq_s[tid] = qq < a.S ? a.Dq[zrow + qq] : 0.f;
        }
        __syncthreads();
        if (qb + 1 < nkb) {
            load_rows<HD>(a.qkv, a.ld, row0, (qb + 1) * QB, a.S, int64_t(h) * HD, qr);
            load_rows<HD>(a.dO, a.ldo, row0, (qb + 1) * QB, a.S, int64_t(h) * HD, dr);
        }
        // S = Q K^T and dP = dO V^T for 64 queries x this wavefront's 16 keys
        f32x4 s[4], dp[4];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            s[qt] = dp[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < HD / 32; ++ds) {
                s[qt] = mfma<TE>(*reinterpret_cast<const uint4*>(Qs + (qt * 16 + lr) * (HD + 8) + ds * 32 + g * 8), kf[ds],
                             s[qt]);
                dp[qt] = mfma<TE>(*reinterpret_cast<const uint4*>(Ds + (qt * 16 + lr) * (HD + 8) + ds * 32 + g * 8), vf[ds],
                              dp[qt]);
            }
        }
        // P and dS = P (dP - D), lane = key, 16 queries per lane
        uint32_t pk[4][2], sk[4][2];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            float p[4], d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ql = qt * 16 + g * 4 + e, qq = qb * QB + ql;
                const bool live = qq < a.S && key < a.S && key <= qq;
                p[e] = live ? exp2f(fmaf(s[qt][e], c, -lse_s[ql])) : 0.f;
                d[e] = p[e] * (dp[qt][e] - dq_s[ql]);
            }
            pk[qt][0] = pack2<TE>(p[0], p[1]);
            pk[qt][1] = pack2<TE>(p[2], p[3]);
            sk[qt][0] = pack2<TE>(d[0], d[1]);
            sk[qt][1] = pack2<TE>(d[2], d[3]);
        }
        // dV += P^T dO and dK += dS^T Q over the 64 queries (two slices of 32)
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            const uint4 pa = make_uint4(pk[2 * js][0], pk[2 * js][1], pk[2 * js + 1][0], pk[2 * js + 1][1]);
            const uint4 sa = make_uint4(sk[2 * js][0], sk[2 * js][1], sk[2 * js + 1][0], sk[2 * js + 1][1]);
#pragma unroll
            for (int dt = 0; dt < HD / 16; ++dt) {
                dv[dt] = mfma<TE>(pa, trfrag<HD>(Ds, dt, js, lane), dv[dt]);
                dk[dt] = mfma<TE>(sa, trfrag<HD>(Qs, dt, js, lane), dk[dt]);
            }
        }
        __syncthreads();
    }
    // dk[dt][e], dv[dt][e]: key kb*64 + 16 wave + 4 g + e, dim 16 dt + lr
    const int64_t zk = (int64_t(b) * a.nH + h) * a.S;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int kk = kb * QB + wave * 16 + g * 4 + e;
        if (kk >= a.S) continue;
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt) {
            a.dKh[(zk + kk) * HD + dt * 16 + lr] = dk[dt][e] * a.scale;
            a.dVh[(zk + kk) * HD + dt * 16 + lr] = dv[dt][e];
        }
    }
}

// dQ for 64 queries of one head.
template <int HD, int TE>
__global__ __launch_bounds__(256) void k_flash_bwd_q(const AttnArgs a) {
    __shared__ __align__(16) uint16_t Ks[QB * (HD + 8)];
    __shared__ __align__(16) uint16_t Vs[QB * (HD + 8)];
    const int nqb = (a.S + QB - 1) / QB;
    const int qb = nqb - 1 - int(blockIdx.x);
    const int h = blockIdx.y, b = blockIdx.z, kh = h / (a.nH / a.nKV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
    const int q = qb * QB + wave * 16 + lr;
    const int64_t row0 = int64_t(b) * a.S;
    const bool qok = q < a.S;
    uint4 qf[HD / 32], df[HD / 32];
#pragma unroll
    for (int ds = 0; ds < HD / 32; ++ds) {
        qf[ds] = qok ? *reinterpret_cast<const uint4*>(a.qkv + (row0 + q) * a.ld + int64_t(h) * HD + ds * 32 + g * 8)
                     : make_uint4(0, 0, 0, 0);
        df[ds] = qok ? *reinterpret_cast<const uint4*>(a.dO + (row0 + q) * a.ldo + int64_t(h) * HD + ds * 32 + g * 8)
                     : make_uint4(0, 0, 0, 0);
    }
    const int64_t zq = (int64_t(b) * a.nH + h) * a.S + q;
    const float lse2 = qok ? a.lse[zq] * kLog2e : 0.f, dd = qok ? a.Dq[zq] : 0.f;
    f32x4 dq[HD / 16];
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float c = a.scale * kLog2e;
    const int64_t kcol = a.qdim + int64_t(kh) * HD, vcol = kcol + a.kvdim;
    uint4 kr[HD / 32], vr[HD / 32];
    load_rows<HD>(a.qkv, a.ld, row0, 0, a.S, kcol, kr);
    load_rows<HD>(a.qkv, a.ld, row0, 0, a.S, vcol, vr);
    for (int kb = 0; kb <= qb; ++kb) {
        store_rows<HD>(kr, Ks);
        store_rows<HD>(vr, Vs);
        __syncthreads();
        if (kb < qb) {
            load_rows<HD>(a.qkv, a.ld, row0, (kb + 1) * QB, a.S, kcol, kr);
            load_rows<HD>(a.qkv, a.ld, row0, (kb + 1) * QB, a.S, vcol, vr);
        }
        uint32_t sk[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f}, dpt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < HD / 32; ++ds) {
                st = mfma<TE>(*reinterpret_cast<const uint4*>(Ks + (kt * 16 + lr) * (HD + 8) + ds * 32 + g * 8), qf[ds], st);
                dpt = mfma<TE>(*reinterpret_cast<const uint4*>(Vs + (kt * 16 + lr) * (HD + 8) + ds * 32 + g * 8), df[ds],
                           dpt);
            }
            float d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = kb * QB + kt * 16 + g * 4 + e;
                const bool live = qok && key < a.S && key <= q;
                const float p = live ? exp2f(fmaf(st[e], c, -lse2)) : 0.f;
                d[e] = p * (dpt[e] - dd);
            }
            sk[kt][0] = pack2<TE>(d[0], d[1]);
            sk[kt][1] = pack2<TE>(d[2], d[3]);
        }
        // dQ^T += K^T dS^T over the 64 keys
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            const uint4 sb = make_uint4(sk[2 * js][0], sk[2 * js][1], sk[2 * js + 1][0], sk[2 * js + 1][1]);
#pragma unroll
            for (int dt = 0; dt < HD / 16; ++dt) dq[dt] = mfma<TE>(trfrag<HD>(Ks, dt, js, lane), sb, dq[dt]);
        }
        __syncthreads();
    }
    if (!qok) return;
    // dq of the rotated q, rotated back (the transpose of the rotation):
    // dq[dt][e] is dim dt*16 + 4g + e, its pair dim in tile dt + HD/32
    const float2* cs = a.rope + int64_t(q) * (HD / 2);
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float2 c = cs[dt * 16 + g * 4 + e];
            const float x1 = dq[dt][e] * a.scale, x2 = dq[dt + HD / 32][e] * a.scale;
            dq[dt][e] = x1 * c.x + x2 * c.y;
            dq[dt + HD / 32][e] = x2 * c.x - x1 * c.y;
        }
    uint16_t* dst = a.dqkv + (row0 + q) * a.lddq + int64_t(h) * HD + g * 4;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
        *reinterpret_cast<uint2*>(dst + dt * 16) =
            make_uint2(pack2<TE>(dq[dt][0], dq[dt][1]), pack2<TE>(dq[dt][2], dq[dt][3]));
}

// ------------------------------------------------------------------ launchers
static void check_attn(const AttnArgs& a) {
    QLX_REQUIRE(a.hd == 64 || a.hd == 128, QLX_EUNSUPPORTED, "attention: head_dim must be 64 or 128");
    QLX_REQUIRE(a.nKV > 0 && a.nH % a.nKV == 0, QLX_EINVAL, "attention: n_heads must be a multiple of n_kv_heads");
    QLX_REQUIRE(a.ld % 8 == 0 && a.ldo % 8 == 0 && a.qdim % 8 == 0 && a.kvdim % 8 == 0, QLX_EUNSUPPORTED,
                "attention: row strides must be multiples of 8 elements");
    QLX_REQUIRE(a.nH <= 65535 && a.B <= 65535, QLX_EUNSUPPORTED, "attention: grid too large");
    QLX_REQUIRE(a.rope != nullptr, QLX_EINVAL, "attention: RoPE table is NULL (dq is rotated back)");
}

void launch_flash_fwd(const AttnArgs& a, hipStream_t s) {
    if (a.B == 0 || a.S == 0) return;
    check_attn(a);
    const dim3 grid(unsigned((a.S + QB - 1) / QB), unsigned(a.nH), unsigned(a.B));
    const double Sd = a.S;
    const double flops = 4.0 * a.B * a.nH * a.hd * (Sd * (Sd + 1) / 2);
    ProfScope prof("attn_fwd", flops, double(a.B) * a.S * (a.qdim * 4.0 + a.kvdim * 4.0 + a.nH * 4.0), s);
    if (a.hd == 128) {
        if (a.f16) hipLaunchKernelGGL((k_flash_fwd<128, TE_F16>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_flash_fwd<128, TE_BF16>), grid, dim3(256), 0, s, a);
    } else {
        if (a.f16) hipLaunchKernelGGL((k_flash_fwd<64, TE_F16>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_flash_fwd<64, TE_BF16>), grid, dim3(256), 0, s, a);
    }
    check_launch("attn_fwd");
}

void launch_flash_bwd(const AttnArgs& a, hipStream_t s) {
    if (a.B == 0 || a.S == 0) return;
    check_attn(a);
    const int64_t n = int64_t(a.B) * a.S * a.nH;
    {
        const int64_t threads = n * (a.hd / 8);
        const dim3 g(unsigned((threads + 255) / 256));
        if (a.dO_part.p) {
            const Partials& q = a.dO_part;
            QLX_REQUIRE(a.dO_out && a.dO_out == a.dO && q.splits >= 1 && !q.R && q.mn == int64_t(a.B) * a.S * a.qdim &&
                            (reinterpret_cast<uintptr_t>(q.p) & 15) == 0,
                        QLX_EINVAL, "attention backward: bad dO partials");
            ProfScope prof("reduce_attn_dot", double(n) * a.hd * (q.splits + 2.0),
                           double(n) * (a.hd * (4.0 * q.splits + 4.0) + 4.0), s);
            if (a.f16) hipLaunchKernelGGL((k_flash_bwd_dot<TE_F16, true>), g, dim3(256), 0, s, a, a.hd);
            else hipLaunchKernelGGL((k_flash_bwd_dot<TE_BF16, true>), g, dim3(256), 0, s, a, a.hd);
        } else {
            ProfScope prof("attn_bwd_dot", 2.0 * n * a.hd, double(n) * (a.hd * 4.0 + 4.0), s);
            if (a.f16) hipLaunchKernelGGL((k_flash_bwd_dot<TE_F16, false>), g, dim3(256), 0, s, a, a.hd);
            else hipLaunchKernelGGL((k_flash_bwd_dot<TE_BF16, false>), g, dim3(256), 0, s, a, a.hd);
        }
        check_launch("attn_bwd_dot");
    }
    const dim3 grid(unsigned((a.S + QB - 1) / QB), unsigned(a.nH), unsigned(a.B));
    const double Sd = a.S, causal = Sd * (Sd + 1) / 2;
    {  // recompute S and dP, then dV and dK: 4 products
        ProfScope prof("attn_bwd_kv", 8.0 * a.B * a.nH * a.hd * causal,
                       double(a.B) * a.S * (a.qdim * 4.0 + a.kvdim * 4.0 + a.nH * 2.0 * a.hd * 4.0), s);
        if (a.hd == 128) {
            if (a.f16) hipLaunchKernelGGL((k_flash_bwd_kv<128, TE_F16>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_flash_bwd_kv<128, TE_BF16>), grid, dim3(256), 0, s, a);
        } else {
            if (a.f16) hipLaunchKernelGGL((k_flash_bwd_kv<64, TE_F16>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_flash_bwd_kv<64, TE_BF16>), grid, dim3(256), 0, s, a);
        }
        check_launch("attn_bwd_kv");
    }
    {  // recompute S and dP, then dQ: 3 products
        ProfScope prof("attn_bwd_q", 6.0 * a.B * a.nH * a.hd * causal,
                       double(a.B) * a.S * (a.qdim * 6.0 + a.kvdim * 4.0), s);
        if (a.hd == 128) {
            if (a.f16) hipLaunchKernelGGL((k_flash_bwd_q<128, TE_F16>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_flash_bwd_q<128, TE_BF16>), grid, dim3(256), 0, s, a);
        } else {
            if (a.f16) hipLaunchKernelGGL((k_flash_bwd_q<64, TE_F16>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_flash_bwd_q<64, TE_BF16>), grid, dim3(256), 0, s, a);
        }
        check_launch("attn_bwd_q");
    }
}

}  // namespace qlx
