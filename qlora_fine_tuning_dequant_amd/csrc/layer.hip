// Decoder-layer orchestration on one HIP stream: the Llama decoder layer with
// a frozen NF4 base and LoRA adapters, forward and backward (the backward
// recomputes the forward from the layer's input first).
//
// Pages: the frozen base is fed to the GPU one decoder layer at a time and
// only the LoRA adapters train (rug.gal article, "En detalle";
// guillermodelpino.com article, "El streaming de capas"); the layer is
// Llama-3.1-8B's (all pages' intros), so: RMSNorm, q/k/v projections, RoPE,
// causal grouped-query attention, o projection + residual, RMSNorm, SwiGLU
// MLP + residual.
//
// Fusions: q|k|v is one NF4 GEMM over the concatenated rows (N = (nH+2nKV)hd),
// gate|up likewise (N = 2I); each LoRA term rides in its base GEMM as a short
// second K phase against block-diagonal staged adapters; residual adds happen
// in the o/down GEMM epilogues; the backward dX GEMMs read the NF4 weight in
// its stored [out][in] layout (no transposed copy) and fold the LoRA dX term
// (du . A) in the same way.
#include <algorithm>
#include <cmath>

#include "layer.h"

namespace qlx {

LayerGeom make_geom(const qlx_dims& d, int batch, int seq) {
    LayerGeom g;
    g.H = d.hidden;
    g.nH = d.n_heads;
    g.nKV = d.n_kv_heads;
    g.hd = d.head_dim;
    g.I = d.inter;
    g.r = d.lora_r;
    g.s = d.lora_alpha / float(d.lora_r);
    g.eps = d.rms_eps;
    g.theta = d.rope_theta;
    g.B = batch;
    g.S = seq;
    g.T = batch * seq;
    g.qdim = g.nH * g.hd;
    g.kvdim = g.nKV * g.hd;
    g.nqkv = g.qdim + 2 * g.kvdim;
    const int outs[7] = {g.qdim, g.kvdim, g.kvdim, g.H, g.I, g.I, g.H};
    const int ins[7] = {g.H, g.H, g.H, g.qdim, g.H, g.H, g.I};
    for (int p = 0; p < 7; ++p) {
        g.out[p] = outs[p];
        g.in[p] = ins[p];
        g.nel[p] = int64_t(outs[p]) * ins[p];
    }
    g.f16 = d.act_dtype == QLX_ACT_F16 ? 1 : 0;
    g.te = g.f16 ? TE_F16 : TE_BF16;
    g.ct = g.f16 ? C_F16 : C_BF16;
    return g;
}

void validate_dims(const qlx_dims* d) {
    QLX_REQUIRE(d, QLX_EINVAL, "dims is NULL");
    QLX_REQUIRE(d->hidden > 0 && d->n_heads > 0 && d->n_kv_heads > 0 && d->head_dim > 0 && d->inter > 0 &&
                    d->vocab > 0 && d->n_layers > 0 && d->lora_r > 0,
                QLX_EINVAL, "dims: every size must be positive");
    QLX_REQUIRE(d->n_heads % d->n_kv_heads == 0, QLX_EINVAL, "dims: n_heads must be a multiple of n_kv_heads");
    QLX_REQUIRE(d->head_dim % 2 == 0, QLX_EINVAL, "dims: head_dim must be even (rotate-half RoPE)");
    QLX_REQUIRE(d->act_dtype == QLX_ACT_BF16 || d->act_dtype == QLX_ACT_F16, QLX_EINVAL,
                "dims: act_dtype must be QLX_ACT_BF16 or QLX_ACT_F16");
    QLX_REQUIRE(d->lora_alpha == d->lora_alpha && d->rms_eps > 0 && d->rope_theta > 0, QLX_EINVAL,
                "dims: lora_alpha, rms_eps, rope_theta must be finite and positive");
    const LayerGeom g = make_geom(*d, 1, 1);
    for (int p = 0; p < 7; ++p)
        QLX_REQUIRE(g.nel[p] % 64 == 0, QLX_EUNSUPPORTED,
                    "dims: every projection must hold a multiple of 64 elements (NF4 blocks may not straddle projections)");
    QLX_REQUIRE(g.hidden_ok(), QLX_EUNSUPPORTED, "dims: hidden, heads*head_dim and inter must be multiples of 4");
}

void blob_layout(const qlx_dims& d, uint64_t off[QLX_BLOB_NSEG], uint64_t* total) {
    const LayerGeom g = make_geom(d, 1, 1);
    auto al = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    uint64_t o = 0;
    for (int p = 0; p < 7; ++p) {
        off[p] = o;
        o += uint64_t(g.nel[p] / 2);  // packed regions back to back (each a multiple of 32 bytes)
    }
    o = al(o);
    for (int p = 0; p < 7; ++p) {
        off[7 + p] = o;
        o += uint64_t(g.nel[p] / 64) * 4;
    }
    o = al(o);
    off[14] = o;
    o = al(o + uint64_t(g.H) * 4);
    off[15] = o;
    o = al(o + uint64_t(g.H) * 4);
    *total = o;
}

// Wire form: the packed regions exactly as above, then every block maximum
// as its upper 16 bits (bf16) back to back, then the two gains. Block maxima
// of bf16 weights are bf16 values, so the low 16 bits dropped are zero.
void wire_layout(const qlx_dims& d, uint64_t off[QLX_BLOB_NSEG], uint64_t* total) {
    const LayerGeom g = make_geom(d, 1, 1);
    auto al = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    uint64_t full[QLX_BLOB_NSEG], ftotal;
    blob_layout(d, full, &ftotal);
    uint64_t o = full[7];
    for (int p = 0; p < 7; ++p) {
        off[p] = full[p];
        off[7 + p] = o;
        o += uint64_t(g.nel[p] / 64) * 2;
    }
    o = al(o);
    off[14] = o;
    o = al(o + uint64_t(g.H) * 4);
    off[15] = o;
    o = al(o + uint64_t(g.H) * 4);
    *total = o;
}

uint64_t absmax_blocks(const qlx_dims& d) {
    const LayerGeom g = make_geom(d, 1, 1);
    uint64_t nb = 0;
    for (int p = 0; p < 7; ++p) nb += uint64_t(g.nel[p] / 64);
    return nb;
}

BlobPtrs blob_ptrs(const qlx_dims& d, const void* blob) {
    uint64_t off[QLX_BLOB_NSEG], total;
    blob_layout(d, off, &total);
    const char* b = static_cast<const char*>(blob);
    BlobPtrs w;
    for (int p = 0; p < 7; ++p) {
        w.packed[p] = reinterpret_cast<const uint8_t*>(b + off[p]);
        w.absmax[p] = reinterpret_cast<const float*>(b + off[7 + p]);
    }
    w.g1 = reinterpret_cast<const float*>(b + off[14]);
    w.g2 = reinterpret_cast<const float*>(b + off[15]);
    return w;
}

void point_u(LayerWs& w, uint16_t* base, const LayerGeom& g) {
    const size_t T = size_t(g.T), r = size_t(g.r);
    w.u_qkv = base;
    w.u_o = base + T * 3 * r;
    w.u_gu = base + T * 4 * r;
    w.u_d = base + T * 6 * r;
}

LayerWs carve_layer(Carver& c, const LayerGeom& g) {
    LayerWs w;
    const size_t T = size_t(g.T), H = size_t(g.H), r = size_t(g.r);
    const size_t Z = size_t(g.B) * g.nH;
    w.n1 = c.take<uint16_t>(T * H);
    w.qkv = c.take<uint16_t>(T * g.nqkv);
    w.oattn = c.take<uint16_t>(T * g.qdim);
    w.n2 = c.take<uint16_t>(T * H);
    w.gu = c.take<uint16_t>(T * 2 * g.I);
    w.act = c.take<uint16_t>(T * g.I);
    w.h1 = c.take<float>(T * H);
    w.rstd1 = c.take<float>(T);
    w.rstd2 = c.take<float>(T);
    w.lse = c.take<float>(Z * g.S);
    w.Dq = c.take<float>(Z * g.S);
    w.u_qkv = c.take<uint16_t>(T * 3 * r);
    w.u_o = c.take<uint16_t>(T * r);
    w.u_gu = c.take<uint16_t>(T * 2 * r);
    w.u_d = c.take<uint16_t>(T * r);
    w.A_qkv = c.take<uint16_t>(3 * r * H);
    w.B_qkv = c.take<uint16_t>(size_t(g.nqkv) * 3 * r);
    w.A_o = c.take<uint16_t>(r * g.qdim);
    w.B_o = c.take<uint16_t>(H * r);
    w.A_gu = c.take<uint16_t>(2 * r * H);
    w.B_gu = c.take<uint16_t>(size_t(2) * g.I * 2 * r);
    w.A_d = c.take<uint16_t>(r * g.I);
    w.B_d = c.take<uint16_t>(H * r);
    w.rope_cs = c.take<float>(size_t(g.S) * g.hd);
    w.partial = c.take<float>(kGemmPartialFloats);
    // backward
    w.dy16 = c.take<uint16_t>(T * H);
    w.dy16o = c.take<uint16_t>(T * H);
    w.dact = c.take<uint16_t>(T * g.I);
    w.dgu = c.take<uint16_t>(T * 2 * g.I);
    w.doattn = c.take<uint16_t>(T * g.qdim);
    w.dqkv = c.take<uint16_t>(T * g.nqkv);
    w.du_d = c.take<uint16_t>(T * r);
    w.du_gu = c.take<uint16_t>(T * 2 * r);
    w.du_o = c.take<uint16_t>(T * r);
    w.du_qkv = c.take<uint16_t>(T * 3 * r);
    w.dn2 = c.take<float>(T * H);
    w.dh1 = c.take<float>(T * H);
    w.dKh = c.take<float>(Z * g.S * g.hd);
    w.dVh = c.take<float>(Z * g.S * g.hd);
    w.dn1 = c.take<float>(T * H);
    return w;
}

size_t layer_ws_bytes(const LayerGeom& g) {
    Carver c(nullptr);
    carve_layer(c, g);
    return c.size();
}

// ---------------------------------------------------------------- helpers
static GemmParams nf4_gemm(int M, int N, int K, const uint16_t* A, int64_t lda, const uint8_t* packed,
                           const float* absmax, int64_t cols) {
    GemmParams p;
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = A;
    p.lda = lda;
    p.B = packed;
    p.absmax = absmax;
    p.nf4_cols = cols;
    return p;
}
static GemmParams dense_gemm(int M, int N, int K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb) {
    GemmParams p;
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = A;
    p.lda = lda;
    p.B = B;
    p.ldb = ldb;
    return p;
}
static void out16(GemmParams& p, uint16_t* C, int64_t ldc, const LayerGeom& g) {
    p.C = C;
    p.ldc = ldc;
    p.c_type = g.ct;
}
static void out_f32(GemmParams& p, float* C, int64_t ldc) {
    p.C = C;
    p.ldc = ldc;
    p.c_type = C_F32;
}

static bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
static Partials partials(const float* p, int splits, int64_t mn, float alpha = 1.f, const float* R = nullptr,
                         int64_t ldr = 0) {
    Partials q;
    q.p = p;
    q.splits = splits;
    q.mn = mn;
    q.alpha = alpha;
    q.R = R;
    q.ldr = ldr;
    return q;
}

static AttnArgs attn_args(const LayerGeom& g, LayerWs& w) {
    AttnArgs a;
    a.qkv = w.qkv;
    a.ld = g.nqkv;
    a.B = g.B;
    a.S = g.S;
    a.nH = g.nH;
    a.nKV = g.nKV;
    a.hd = g.hd;
    a.qdim = g.qdim;
    a.kvdim = g.kvdim;
    a.scale = 1.0f / sqrtf(float(g.hd));
    a.o = w.oattn;
    a.ldo = g.qdim;
    a.lse = w.lse;
    a.dO = w.doattn;
    a.O = w.oattn;
    a.Dq = w.Dq;
    a.dKh = w.dKh;
    a.dVh = w.dVh;
    a.dqkv = w.dqkv;
    a.lddq = g.nqkv;
    a.rope = reinterpret_cast<const float2*>(w.rope_cs);
    a.f16 = g.f16;
    return a;
}

void stage_lora(const LayerGeom& g, const qlx_lora* lora, LayerWs& w, hipStream_t s) {
    const int r = g.r;
    // the layer's four packs (q|k|v, o, gate|up, down) in one launch
    LoraSeg qkv[3] = {{lora->A[0], lora->B[0], g.qdim}, {lora->A[1], lora->B[1], g.kvdim},
                      {lora->A[2], lora->B[2], g.kvdim}};
    LoraSeg o[1] = {{lora->A[3], lora->B[3], g.H}};
    LoraSeg gu[2] = {{lora->A[4], lora->B[4], g.I}, {lora->A[5], lora->B[5], g.I}};
    LoraSeg dn[1] = {{lora->A[6], lora->B[6], g.H}};
    const LoraPackJob jobs[4] = {{qkv, 3, g.H, w.A_qkv, w.B_qkv}, {o, 1, g.qdim, w.A_o, w.B_o},
                                 {gu, 2, g.H, w.A_gu, w.B_gu}, {dn, 1, g.I, w.A_d, w.B_d}};
    launch_lora_pack_jobs(jobs, 4, r, g.s, g.f16, s);
}

// Forward. h_out == nullptr skips the down projection (the backward does not
// need the layer output). lora_staged: adapters already staged in w.
void layer_forward(const LayerGeom& g, const BlobPtrs& wt, const qlx_lora* lora, bool lora_staged, const float* h_in,
                   float* h_out, LayerWs& w, hipStream_t s, bool u_given) {
    const int T = g.T, H = g.H, r = g.r;
    const bool L = lora != nullptr;
    const bool U = L && !u_given;  // compute the adapters' u = x A^T here
    if (L && !lora_staged) stage_lora(g, lora, w, s);
    if (!w.rope_ready) {  // once per workspace: every layer pass of a step shares the table
        launch_rope_table(g.S, g.hd, g.theta, w.rope_cs, s);
        w.rope_ready = true;
    }

    // attention block
    launch_rmsnorm_fwd(h_in, wt.g1, T, H, g.eps, w.n1, g.f16, w.rstd1, s);
    if (U) {
        GemmParams pu = dense_gemm(T, 3 * r, H, w.n1, H, w.A_qkv, H);
        out16(pu, w.u_qkv, 3 * r, g);
        pu.tag = "gemm_lora_u";
        gemm(pu, A_ROW, B_DENSE_NT, g.te, w.partial, s);
    }
    {
        GemmParams p = nf4_gemm(T, g.nqkv, H, w.n1, H, wt.packed[0], wt.absmax[0], H);
        if (L) {
            p.K2 = 3 * r;
            p.A2 = w.u_qkv;
            p.lda2 = 3 * r;
            p.B2 = w.B_qkv;
            p.ldb2 = 3 * r;
            p.slab_alg_k = r;  // block-diagonal: each output column sees one adapter
        }
        out16(p, w.qkv, g.nqkv, g);
        const int nall = g.nH + 2 * g.nKV;  // q and k heads are contiguous, then v
        p.defer_reduce = rope_part_ok(g.hd, nall);
        const int sp = gemm(p, A_ROW, B_NF4_NT, g.te, w.partial, s);
        if (p.defer_reduce && sp > 1) launch_rope_part(partials(w.partial, sp, int64_t(T) * g.nqkv), w.qkv, T, g.S, g.nH + g.nKV, nall, g.hd,
                                     w.rope_cs, g.f16, s);
        else launch_rope(w.qkv, g.nqkv, T, g.S, 0, g.nH + g.nKV, g.hd, w.rope_cs, g.f16, s);
    }
    launch_flash_fwd(attn_args(g, w), s);
    if (U) {
        GemmParams pu = dense_gemm(T, r, g.qdim, w.oattn, g.qdim, w.A_o, g.qdim);
        out16(pu, w.u_o, r, g);
        pu.tag = "gemm_lora_u";
        gemm(pu, A_ROW, B_DENSE_NT, g.te, w.partial, s);
    }
    int sp_o;  // > 1: the o projection's partials wait for the norm (deferred)
    {  // h1 = h_in + o_proj(o)
        GemmParams p = nf4_gemm(T, H, g.qdim, w.oattn, g.qdim, wt.packed[3], wt.absmax[3], g.qdim);
        if (L) {
            p.K2 = r;
            p.A2 = w.u_o;
            p.lda2 = r;
            p.B2 = w.B_o;
            p.ldb2 = r;
        }
        out_f32(p, w.h1, H);
        p.R = h_in;
        p.ldr = H;
        p.defer_reduce = rmsnorm_part_ok(H) && a16(h_in) && a16(wt.g2);
        sp_o = gemm(p, A_ROW, B_NF4_NT, g.te, w.partial, s);
        if (!p.defer_reduce) sp_o = 1;
    }
    // MLP block (the o projection's split-K sum, + h_in, written to h1 by the norm when deferred)
    if (sp_o > 1)
        launch_rmsnorm_fwd_part(partials(w.partial, sp_o, int64_t(T) * H, 1.f, h_in, H), w.h1, wt.g2, T, H, g.eps, w.n2,
                                g.f16, w.rstd2, s);
    else
        launch_rmsnorm_fwd(w.h1, wt.g2, T, H, g.eps, w.n2, g.f16, w.rstd2, s);
    if (U) {
        GemmParams pu = dense_gemm(T, 2 * r, H, w.n2, H, w.A_gu, H);
        out16(pu, w.u_gu, 2 * r, g);
        pu.tag = "gemm_lora_u";
        gemm(pu, A_ROW, B_DENSE_NT, g.te, w.partial, s);
    }
    {
        GemmParams p = nf4_gemm(T, 2 * g.I, H, w.n2, H, wt.packed[4], wt.absmax[4], H);
        if (L) {
            p.K2 = 2 * r;
            p.A2 = w.u_gu;
            p.lda2 = 2 * r;
            p.B2 = w.B_gu;
            p.ldb2 = 2 * r;
            p.slab_alg_k = r;
        }
        out16(p, w.gu, 2 * g.I, g);
        gemm(p, A_ROW, B_NF4_NT, g.te, w.partial, s);
    }
    launch_swiglu_fwd(w.gu, T, g.I, w.act, g.f16, s);
    if (U) {
        GemmParams pu = dense_gemm(T, r, g.I, w.act, g.I, w.A_d, g.I);
        out16(pu, w.u_d, r, g);
        pu.tag = "gemm_lora_u";
        gemm(pu, A_ROW, B_DENSE_NT, g.te, w.partial, s);
    }
    if (h_out) {
        GemmParams p = nf4_gemm(T, H, g.I, w.act, g.I, wt.packed[6], wt.absmax[6], g.I);
        if (L) {
            p.K2 = r;
            p.A2 = w.u_d;
            p.lda2 = r;
            p.B2 = w.B_d;
            p.ldb2 = r;
        }
        out_f32(p, h_out, H);
        p.R = w.h1;
        p.ldr = H;
        gemm(p, A_ROW, B_NF4_NT, g.te, w.partial, s);
    }
}

// The 14 LoRA weight gradients of one layer's backward, gathered while it
// runs and computed in one launch at its end (each a product over the T
// tokens: dB = s dy^T u, dA = du^T x, with dy and du holding gsc x the
// gradient).
struct LoraGradGroup {
    GemmGroup g;
    // dB of the projection whose output gradient is dy (column slice of a
    // [T, ld_dy] buffer, out columns), u its r columns of a [T, ld_u] buffer
    void dB(const LayerGeom& L, const uint16_t* dy, int64_t ld_dy, int out, const uint16_t* u, int64_t ld_u,
            float* C) {
        GemmProb& q = g.prob[g.n++];
        q.A = dy, q.lda = ld_dy, q.M = out;
        q.B = u, q.ldb = ld_u, q.N = L.r;
        q.C = C, q.ldc = L.r;
        q.alpha = L.s / L.gsc;
    }
    // dA from du (r columns of a [T, ld_du] buffer) and the projection's input x [T, in]
    void dA(const LayerGeom& L, const uint16_t* du, int64_t ld_du, const uint16_t* x, int in, float* C) {
        GemmProb& q = g.prob[g.n++];
        q.A = du, q.lda = ld_du, q.M = L.r;
        q.B = x, q.ldb = in, q.N = in;
        q.C = C, q.ldc = in;
        q.alpha = 1.0f / L.gsc;
    }
};

void layer_backward(const LayerGeom& g, const BlobPtrs& wt, const qlx_lora* lora, const float* h_in,
                    const float* dh_out, float* dh_in, const qlx_lora_grad* grads, LayerWs& w, hipStream_t s,
                    bool recompute, bool u_given) {
    const int T = g.T, H = g.H, r = g.r, S = g.S;
    if (recompute) layer_forward(g, wt, lora, false, h_in, nullptr, w, s, u_given);
    LoraGradGroup lg;
    int sp_o = 1;

    // ---- down projection: out = h1 + down(act)
    if (w.dy16_src != dh_out)  // gradients scaled by gsc from here
        launch_f32_to_act(dh_out, int64_t(T) * H, w.dy16, g.f16, g.gsc, s);
    w.dy16_src = nullptr;
    {
        GemmParams p = dense_gemm(T, r, H, w.dy16, H, w.B_d, r);
        out16(p, w.du_d, r, g);
        p.tag = "gemm_lora_du";
        gemm(p, A_ROW, B_DENSE_NN, g.te, w.partial, s);
    }
    {
        GemmParams p = nf4_gemm(T, g.I, H, w.dy16, H, wt.packed[6], wt.absmax[6], g.I);
        p.K2 = r;
        p.A2 = w.du_d;
        p.lda2 = r;
        p.B2 = w.A_d;
        p.ldb2 = g.I;
        out16(p, w.dact, g.I, g);
        gemm(p, A_ROW, B_NF4_NN, g.te, w.partial, s);
    }
    lg.dB(g, w.dy16, H, H, w.u_d, r, grads->dB[6]);
    lg.dA(g, w.du_d, r, w.act, g.I, grads->dA[6]);
    // ---- SwiGLU and gate/up
    launch_swiglu_bwd(w.dact, w.gu, T, g.I, w.dgu, g.f16, s);
    {
        GemmParams p = dense_gemm(T, 2 * r, 2 * g.I, w.dgu, 2 * g.I, w.B_gu, 2 * r);
        out16(p, w.du_gu, 2 * r, g);
        p.tag = "gemm_lora_du";
        gemm(p, A_ROW, B_DENSE_NN, g.te, w.partial, s);
    }
    {
        GemmParams p = nf4_gemm(T, H, 2 * g.I, w.dgu, 2 * g.I, wt.packed[4], wt.absmax[4], H);
        p.K2 = 2 * r;
        p.A2 = w.du_gu;
        p.lda2 = 2 * r;
        p.B2 = w.A_gu;
        p.ldb2 = H;
        out_f32(p, w.dn2, H);
        p.alpha = 1.0f / g.gsc;  // back to true gradients on the fp32 residual path
        p.defer_reduce = rmsnorm_part_ok(H) && a16(wt.g2) && a16(dh_out);
        const int sp = gemm(p, A_ROW, B_NF4_NN, g.te, w.partial, s);
        // dh1, and its 16-bit scaled copy: the o projection's output gradient
        if (p.defer_reduce && sp > 1)
            launch_rmsnorm_bwd_part(partials(w.partial, sp, int64_t(T) * H, p.alpha), w.h1, wt.g2, w.rstd2, dh_out, T, H,
                                    w.dh1, s, w.dy16o, g.gsc, g.f16);
        else
            launch_rmsnorm_bwd(w.dn2, w.h1, wt.g2, w.rstd2, dh_out, T, H, w.dh1, s, w.dy16o, g.gsc, g.f16);
    }
    for (int j = 0; j < 2; ++j) {  // gate, up
        lg.dB(g, w.dgu + int64_t(j) * g.I, 2 * g.I, g.I, w.u_gu + j * r, 2 * r, grads->dB[4 + j]);
        lg.dA(g, w.du_gu + j * r, 2 * r, w.n2, H, grads->dA[4 + j]);
    }

    // ---- o projection: h1 = h + o(oattn)
    {
        GemmParams p = dense_gemm(T, r, H, w.dy16o, H, w.B_o, r);
        out16(p, w.du_o, r, g);
        p.tag = "gemm_lora_du";
        gemm(p, A_ROW, B_DENSE_NN, g.te, w.partial, s);
    }
    {
        GemmParams p = nf4_gemm(T, g.qdim, H, w.dy16o, H, wt.packed[3], wt.absmax[3], g.qdim);
        p.K2 = r;
        p.A2 = w.du_o;
        p.lda2 = r;
        p.B2 = w.A_o;
        p.ldb2 = g.qdim;
        out16(p, w.doattn, g.qdim, g);
        p.defer_reduce = 1;  // summed by the attention backward's first kernel
        sp_o = gemm(p, A_ROW, B_NF4_NN, g.te, w.partial, s);
    }
    lg.dB(g, w.dy16o, H, H, w.u_o, r, grads->dB[3]);
    lg.dA(g, w.du_o, r, w.oattn, g.qdim, grads->dA[3]);

    // ---- attention: dq into dqkv, per-head fp32 dK, dV summed over each group below
    {
        AttnArgs a = attn_args(g, w);
        if (sp_o > 1) {
            a.dO_part = partials(w.partial, sp_o, int64_t(T) * g.qdim);
            a.dO_out = w.doattn;
        }
        launch_flash_bwd(a, s);
    }
    launch_gqa_reduce(w.dKh, g.B, g.nH, g.nKV, S, g.hd, w.dqkv, g.nqkv, g.qdim, w.rope_cs, g.f16, s);  // dk, rotated back
    launch_gqa_reduce(w.dVh, g.B, g.nH, g.nKV, S, g.hd, w.dqkv, g.nqkv, g.qdim + g.kvdim, nullptr, g.f16, s);

    // ---- q/k/v projections
    {
        GemmParams p = dense_gemm(T, 3 * r, g.nqkv, w.dqkv, g.nqkv, w.B_qkv, 3 * r);
        out16(p, w.du_qkv, 3 * r, g);
        p.tag = "gemm_lora_du";
        gemm(p, A_ROW, B_DENSE_NN, g.te, w.partial, s);
    }
    // q, k, v: output columns [0, qdim), [qdim, qdim + kvdim), [qdim + kvdim, nqkv) of dqkv
    {
        const int col[3] = {0, g.qdim, g.qdim + g.kvdim}, out[3] = {g.qdim, g.kvdim, g.kvdim};
        for (int j = 0; j < 3; ++j) {
            lg.dB(g, w.dqkv + col[j], g.nqkv, out[j], w.u_qkv + j * r, 3 * r, grads->dB[j]);
            lg.dA(g, w.du_qkv + j * r, 3 * r, w.n1, H, grads->dA[j]);
        }
    }
    gemm_group_tn(lg.g, T, g.te, "gemm_lora_grads", s);
    if (dh_in) {
        GemmParams p = nf4_gemm(T, H, g.nqkv, w.dqkv, g.nqkv, wt.packed[0], wt.absmax[0], H);
        p.K2 = 3 * r;
        p.A2 = w.du_qkv;
        p.lda2 = 3 * r;
        p.B2 = w.A_qkv;
        p.ldb2 = H;
        out_f32(p, w.dn1, H);
        p.alpha = 1.0f / g.gsc;
        p.defer_reduce = rmsnorm_part_ok(H) && a16(h_in) && a16(wt.g1) && a16(dh_in);
        const int sp = gemm(p, A_ROW, B_NF4_NN, g.te, w.partial, s);
        if (p.defer_reduce && sp > 1)
            launch_rmsnorm_bwd_part(partials(w.partial, sp, int64_t(T) * H, p.alpha), h_in, wt.g1, w.rstd1, w.dh1, T, H,
                                    dh_in, s, w.dy16, g.gsc, g.f16);
        else
            launch_rmsnorm_bwd(w.dn1, h_in, wt.g1, w.rstd1, w.dh1, T, H, dh_in, s, w.dy16, g.gsc, g.f16);
        w.dy16_src = dh_in;  // the layer below starts from dy16 as written here
    }
}

}  // namespace qlx
