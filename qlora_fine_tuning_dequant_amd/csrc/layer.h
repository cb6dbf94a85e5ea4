// Decoder-layer geometry, blob addressing, workspace and orchestration.
#pragma once
#include "qlx_internal.h"

namespace qlx {

struct LayerGeom {
    int H, nH, nKV, hd, I, r;
    float s, eps, theta;
    int B, S, T;
    int qdim, kvdim, nqkv;
    int out[7], in[7];
    int64_t nel[7];
    // 16-bit activation type: f16 = 1 for fp16 (MFMA TE_F16, stores C_F16),
    // else bf16; te / ct are the GEMM element and output codes
    int f16 = 0, te = TE_BF16, ct = C_BF16;
    // gradient scale: the backward's 16-bit gradients hold gsc x the true
    // values (a power of two; 1 with bf16), fp32 outputs come out unscaled
    float gsc = 1.f;
    bool hidden_ok() const { return H % 4 == 0 && qdim % 4 == 0 && I % 4 == 0 && kvdim % 4 == 0; }
};

struct BlobPtrs {
    const uint8_t* packed[7];
    const float* absmax[7];
    const float* g1;
    const float* g2;
};

// Every intermediate of one layer's forward and backward (bf16 activations,
// fp32 residual-stream values, attention log-sum-exp, LoRA staging, split-K
// scratch). Carved from the caller's workspace.
struct LayerWs {
    uint16_t *n1, *qkv, *oattn, *n2, *gu, *act;
    float *h1, *rstd1, *rstd2;
    float *lse, *Dq;  // [B, nH, S] attention log-sum-exp and sum_d dO o
    uint16_t *u_qkv, *u_o, *u_gu, *u_d;
    uint16_t *A_qkv, *B_qkv, *A_o, *B_o, *A_gu, *B_gu, *A_d, *B_d;
    float* rope_cs;
    bool rope_ready = false;  // host flag: rope_cs holds this geometry's table
    // host flag: dy16 already holds 16-bit(gsc x this buffer) (written by the
    // backward of the layer above, whose input gradient it is)
    const float* dy16_src = nullptr;
    float* partial;
    uint16_t *dy16, *dy16o, *dact, *dgu, *doattn, *dqkv;  // dy16: down's output gradient, dy16o: o's
    uint16_t *du_d, *du_gu, *du_o, *du_qkv;
    float *dn2, *dh1, *dKh, *dVh, *dn1;
};

LayerGeom make_geom(const qlx_dims& d, int batch, int seq);
void validate_dims(const qlx_dims* d);
void blob_layout(const qlx_dims& d, uint64_t off[QLX_BLOB_NSEG], uint64_t* total);
// Wire form of a layer blob (block maxima as bf16; offsets as in blob_layout,
// [7..13] pointing at bf16 arrays). The packed regions sit at the same offsets
// in both forms and end where the wire form's maxima begin (off[7]).
void wire_layout(const qlx_dims& d, uint64_t off[QLX_BLOB_NSEG], uint64_t* total);
uint64_t absmax_blocks(const qlx_dims& d);  // NF4 blocks in one layer
BlobPtrs blob_ptrs(const qlx_dims& d, const void* blob);
LayerWs carve_layer(Carver& c, const LayerGeom& g);
size_t layer_ws_bytes(const LayerGeom& g);
void stage_lora(const LayerGeom& g, const qlx_lora* lora, LayerWs& w, hipStream_t s);
// u_given: w.u_qkv, u_o, u_gu, u_d already hold this layer's u = x A^T (kept
// from its forward), so those four products are not run again.
void layer_forward(const LayerGeom& g, const BlobPtrs& wt, const qlx_lora* lora, bool lora_staged, const float* h_in,
                   float* h_out, LayerWs& w, hipStream_t s, bool u_given = false);
// Points w's u buffers at a caller area of T * 7r bf16 (u_qkv | u_o | u_gu | u_d).
void point_u(LayerWs& w, uint16_t* base, const LayerGeom& g);
// recompute = false: w still holds this layer's forward activations and
// staged adapters (the last layer_forward on w was this layer's, with
// `lora`, from h_in), so the forward is not run again.
void layer_backward(const LayerGeom& g, const BlobPtrs& wt, const qlx_lora* lora, const float* h_in,
                    const float* dh_out, float* dh_in, const qlx_lora_grad* grads, LayerWs& w, hipStream_t s,
                    bool recompute = true, bool u_given = false);

}  // namespace qlx
