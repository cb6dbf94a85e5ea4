// C ABI of libqlx: argument validation, workspace carving, the layer
// streamer and the SFT / DPO steps.
//
// Layer streaming (rug.gal article, intro and "En detalle"; guillermodelpino.com
// article, "El streaming de capas"; imasters article, "Como cabe um 8B em
// 4 GB"): the frozen NF4 base stays in pinned host RAM; one decoder layer at a
// time is copied to the GPU, computed, and its slot reused. Here the copy runs
// on a side stream into two device slots (double buffering): the copy of layer
// i+1 overlaps compute on layer i, ordered only by events (copy_done[slot] on
// the side stream, compute_done[slot] on the compute stream). The backward
// re-streams the layers in reverse from layer-boundary checkpoints; the two
// layers still in the slots when the forward ends are used directly.
// DPO (same pages, "Do SFT para os métodos de preferência"): the reference
// model is the same layer stream with the adapters off. With
// QLX_DPO_REF_FUSED the reference forward of each layer runs while that layer
// is resident for the policy forward, so DPO reads the stack as often as SFT;
// QLX_DPO_REF_SEPARATE streams a separate reference pass first.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include <chrono>

#include "layer.h"
#include "source.h"

namespace qlx {

static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }
void check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) throw Error{QLX_EHIP, std::string(what) + ": " + hipGetErrorString(e)};
}

static inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
#define REQ_AL(p, name) QLX_REQUIRE(al16(p), QLX_EINVAL, std::string(name) + " must be 16-byte aligned")

static void check_ws(void* ws, size_t ws_bytes, size_t need) {
    QLX_REQUIRE(ws_bytes >= need, QLX_EWORKSPACE,
                "workspace too small: need " + std::to_string(need) + " bytes, got " + std::to_string(ws_bytes));
    QLX_REQUIRE(need == 0 || ws != nullptr, QLX_EINVAL, "workspace is NULL");
    QLX_REQUIRE(al16(ws), QLX_EINVAL, "workspace must be 16-byte aligned");
}

// ------------------------------------------------------------ QLoRA linear
struct LinearWs {
    uint16_t *Ab, *Bb, *u, *du;
    float* partial;
};
static LinearWs carve_linear(Carver& c, int64_t T, int64_t in_f, int64_t out_f, int r) {
    LinearWs w;
    w.Ab = c.take<uint16_t>(size_t(r) * in_f);
    w.Bb = c.take<uint16_t>(size_t(out_f) * r);
    w.u = c.take<uint16_t>(size_t(T) * r);
    w.du = c.take<uint16_t>(size_t(T) * r);
    w.partial = c.take<float>(kGemmPartialFloats);
    return w;
}

static void validate_linear(int64_t T, const qlx_nf4& W, const float* A, const float* B, int r) {
    QLX_REQUIRE(T >= 0 && W.rows > 0 && W.cols > 0, QLX_EINVAL, "linear: T >= 0, W.rows > 0, W.cols > 0");
    QLX_REQUIRE(T <= INT32_MAX && W.rows <= INT32_MAX && W.cols <= INT32_MAX, QLX_EUNSUPPORTED, "linear: sizes exceed int32");
    REQ_PTR(W.packed, "W.packed");
    REQ_PTR(W.absmax, "W.absmax");
    REQ_AL(W.packed, "W.packed");
    QLX_REQUIRE((A == nullptr) == (B == nullptr), QLX_EINVAL, "linear: A and B must both be set or both NULL");
    if (A) QLX_REQUIRE(r > 0, QLX_EINVAL, "linear: r must be positive with LoRA on");
    QLX_REQUIRE(W.cols % 4 == 0, QLX_EUNSUPPORTED, "linear: in_features must be a multiple of 4");
}

}  // namespace qlx

using namespace qlx;

extern "C" {

const char* qlx_last_error(void) { return g_err.c_str(); }
const char* qlx_version(void) { return "qlx 0.1 (gfx950)"; }

int nf4_quantize(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* packed, float* absmax, void* stream) {
    return guarded([&] {
        QLX_REQUIRE(rows >= 0 && cols >= 0, QLX_EINVAL, "nf4_quantize: negative size");
        const int64_t n = rows * cols;
        if (n == 0) return;
        REQ_PTR(w, "w");
        REQ_PTR(packed, "packed");
        REQ_PTR(absmax, "absmax");
        launch_nf4_quantize(w, n, packed, absmax, static_cast<hipStream_t>(stream));
    });
}

int nf4_dequant(const uint8_t* packed, const float* absmax, int64_t rows, int64_t cols, int out_dtype, void* out,
                void* stream) {
    return guarded([&] {
        QLX_REQUIRE(rows >= 0 && cols >= 0, QLX_EINVAL, "nf4_dequant: negative size");
        QLX_REQUIRE(out_dtype == QLX_F32 || out_dtype == QLX_BF16, QLX_EINVAL, "nf4_dequant: out_dtype");
        const int64_t n = rows * cols;
        if (n == 0) return;
        REQ_PTR(packed, "packed");
        REQ_PTR(absmax, "absmax");
        REQ_PTR(out, "out");
        QLX_REQUIRE((reinterpret_cast<uintptr_t>(packed) & 3) == 0, QLX_EINVAL, "packed must be 4-byte aligned");
        REQ_AL(out, "out");
        launch_nf4_dequant(packed, absmax, n, out_dtype, out, static_cast<hipStream_t>(stream));
    });
}

size_t qlx_linear_workspace_bytes(int64_t T, int64_t in_f, int64_t out_f, int r) {
    if (T < 0 || in_f <= 0 || out_f <= 0 || r < 0) return 0;
    Carver c(nullptr);
    carve_linear(c, T, in_f, out_f, std::max(r, 0));
    return c.size();
}

}  // extern "C"

namespace qlx {
// The QLoRA linear forward on a workspace laid out by carve_linear, whose
// split-K partial region holds partial_cap floats.
static void linear_fwd(const uint16_t* x, int64_t T, const qlx_nf4& W, const float* A, const float* B, int r,
                       float scale, uint16_t* y, LinearWs w, size_t partial_cap, hipStream_t s) {
    const int M = int(T), N = int(W.rows), K = int(W.cols);
    GemmParams p;
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = x;
    p.lda = K;
    p.B = W.packed;
    p.absmax = W.absmax;
    p.nf4_cols = K;
    p.partial_cap = partial_cap;
    if (A) {
        LoraSeg seg{A, B, N};
        launch_lora_pack(&seg, 1, r, K, scale, w.Ab, w.Bb, 0, s);  // the linear calls take bf16
        GemmParams pu;
        pu.M = M;
        pu.N = r;
        pu.K = K;
        pu.A = x;
        pu.lda = K;
        pu.B = w.Ab;
        pu.ldb = K;
        pu.C = w.u;
        pu.ldc = r;
        pu.c_type = C_BF16;
        pu.partial_cap = partial_cap;
        gemm(pu, A_ROW, B_DENSE_NT, TE_BF16, w.partial, s);
        p.K2 = r;
        p.A2 = w.u;
        p.lda2 = r;
        p.B2 = w.Bb;
        p.ldb2 = r;
    }
    p.C = y;
    p.ldc = N;
    p.c_type = C_BF16;
    gemm(p, A_ROW, B_NF4_NT, TE_BF16, w.partial, s);
}

// Scratch of the allocation-free forward: one copy per GPU the library runs
// on, held until the process ends. Host code never passes `scratch` itself to
// a kernel (in host code it names a host-side stand-in): it uses the device
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = QLX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64] = {};

static char* scratch_on_current_device() {
    int dev = 0;
    QLX_CHECK_HIP(hipGetDevice(&dev));
    QLX_REQUIRE(dev >= 0 && dev < 64, QLX_EUNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        QLX_CHECK_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        QLX_REQUIRE(ptr != nullptr, QLX_EHIP, "scratch: no device address");
        g_scratch_ptr[dev] = ptr;
    }
    return static_cast<char*>(g_scratch_ptr[dev]);
}
}  // namespace qlx

extern "C" {

int qlora_linear_fwd(const uint16_t* x, int64_t T, qlx_nf4 W, const float* A, const float* B, int r, float scale,
                     uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
    return guarded([&] {
        validate_linear(T, W, A, B, r);
        if (T == 0) return;
        REQ_PTR(x, "x");
        REQ_PTR(y, "y");
        const int rr = A ? r : 0;
        check_ws(ws, ws_bytes, qlx_linear_workspace_bytes(T, W.cols, W.rows, rr));
        Carver c(ws);
        const LinearWs w = carve_linear(c, T, W.cols, W.rows, rr);
        linear_fwd(x, T, W, A, B, r, scale, y, w, kGemmPartialFloats, static_cast<hipStream_t>(stream));
    });
}

int qlora_linear_fwd_noalloc(const uint16_t* x, int64_t T, qlx_nf4 W, const float* A, const float* B, int r,
                             float scale, uint16_t* y, void* stream) {
    return guarded([&] {
        validate_linear(T, W, A, B, r);
        if (T == 0) return;
        REQ_PTR(x, "x");
        REQ_PTR(y, "y");
        const int rr = A ? r : 0;
        // the staging (adapters in bf16, u) first, then whatever is left for split-K partials
        Carver probe(nullptr);
        probe.take<uint16_t>(size_t(rr) * W.cols);
        probe.take<uint16_t>(size_t(W.rows) * rr);
        probe.take<uint16_t>(size_t(T) * rr);
        probe.take<uint16_t>(size_t(T) * rr);
        const size_t staging = probe.size();
        QLX_REQUIRE(staging <= kNoAllocScratchBytes, QLX_EINVAL,
                    "qlora_linear_fwd_noalloc: the adapter staging (" + std::to_string(staging) +
                        " bytes) exceeds the static scratch (" + std::to_string(kNoAllocScratchBytes) + " bytes)");
        char* base = scratch_on_current_device();
        Carver c(base);
        LinearWs w;
        w.Ab = c.take<uint16_t>(size_t(rr) * W.cols);
        w.Bb = c.take<uint16_t>(size_t(W.rows) * rr);
        w.u = c.take<uint16_t>(size_t(T) * rr);
        w.du = c.take<uint16_t>(size_t(T) * rr);
        const size_t used = c.size();
        w.partial = reinterpret_cast<float*>(base + used);
        linear_fwd(x, T, W, A, B, r, scale, y, w, (kNoAllocScratchBytes - used) / sizeof(float),
                   static_cast<hipStream_t>(stream));
    });
}

int qlora_linear_bwd(const uint16_t* dy, const uint16_t* x, int64_t T, qlx_nf4 W, const float* A, const float* B,
                     int r, float scale, uint16_t* dx, float* dA, float* dB, int accumulate, void* ws,
                     size_t ws_bytes, void* stream) {
    return guarded([&] {
        validate_linear(T, W, A, B, r);
        if (A) {
            REQ_PTR(dA, "dA");
            REQ_PTR(dB, "dB");
        }
        if (T == 0) {  // empty sums over the tokens: dA = dB = 0 (or unchanged when accumulating)
            if (A && !accumulate) {
                hipStream_t s = static_cast<hipStream_t>(stream);
                launch_fill_u32(reinterpret_cast<uint32_t*>(dA), int64_t(r) * W.cols, 0u, s);
                launch_fill_u32(reinterpret_cast<uint32_t*>(dB), W.rows * int64_t(r), 0u, s);
            }
            return;
        }
        REQ_PTR(dy, "dy");
        REQ_PTR(x, "x");
        const int rr = A ? r : 0;
        check_ws(ws, ws_bytes, qlx_linear_workspace_bytes(T, W.cols, W.rows, rr));
        hipStream_t s = static_cast<hipStream_t>(stream);
        Carver c(ws);
        LinearWs w = carve_linear(c, T, W.cols, W.rows, rr);
        const int M = int(T), N = int(W.rows), K = int(W.cols);  // forward: y [T, N] = x [T, K] W^T
        if (A) {
            LoraSeg seg{A, B, N};
            launch_lora_pack(&seg, 1, r, K, scale, w.Ab, w.Bb, 0, s);  // the linear calls take bf16
            GemmParams pu;  // u = x A^T
            pu.M = M;
            pu.N = r;
            pu.K = K;
            pu.A = x;
            pu.lda = K;
            pu.B = w.Ab;
            pu.ldb = K;
            pu.C = w.u;
            pu.ldc = r;
            pu.c_type = C_BF16;
            gemm(pu, A_ROW, B_DENSE_NT, TE_BF16, w.partial, s);
            GemmParams pd;  // du = dy (sB)
            pd.M = M;
            pd.N = r;
            pd.K = N;
            pd.A = dy;
            pd.lda = N;
            pd.B = w.Bb;
            pd.ldb = r;
            pd.C = w.du;
            pd.ldc = r;
            pd.c_type = C_BF16;
            gemm(pd, A_ROW, B_DENSE_NN, TE_BF16, w.partial, s);
        }
        if (dx) {
            GemmParams p;
            p.M = M;
            p.N = K;
            p.K = N;
            p.A = dy;
            p.lda = N;
            p.B = W.packed;
            p.absmax = W.absmax;
            p.nf4_cols = K;
            if (A) {
                p.K2 = r;
                p.A2 = w.du;
                p.lda2 = r;
                p.B2 = w.Ab;
                p.ldb2 = K;
            }
            p.C = dx;
            p.ldc = K;
            p.c_type = C_BF16;
            gemm(p, A_ROW, B_NF4_NN, TE_BF16, w.partial, s);
        }
        if (A) {
            GemmParams pb;  // dB = s dy^T u
            pb.M = N;
            pb.N = r;
            pb.K = M;
            pb.A = dy;
            pb.lda = N;
            pb.B = w.u;
            pb.ldb = r;
            pb.C = dB;
            pb.ldc = r;
            pb.c_type = C_F32;
            pb.alpha = scale;
            pb.accumulate = accumulate;
            gemm(pb, A_TRANS, B_DENSE_NN, TE_BF16, w.partial, s);
            GemmParams pa;  // dA = du^T x
            pa.M = r;
            pa.N = K;
            pa.K = M;
            pa.A = w.du;
            pa.lda = r;
            pa.B = x;
            pa.ldb = K;
            pa.C = dA;
            pa.ldc = K;
            pa.c_type = C_F32;
            pa.accumulate = accumulate;
            gemm(pa, A_TRANS, B_DENSE_NN, TE_BF16, w.partial, s);
        }
    });
}

int qlx_layer_blob_layout(const qlx_dims* d, uint64_t offsets[QLX_BLOB_NSEG], uint64_t* total_bytes) {
    return guarded([&] {
        validate_dims(d);
        REQ_PTR(offsets, "offsets");
        REQ_PTR(total_bytes, "total_bytes");
        blob_layout(*d, offsets, total_bytes);
    });
}

int qlx_layer_wire_layout(const qlx_dims* d, uint64_t offsets[QLX_BLOB_NSEG], uint64_t* total_bytes) {
    return guarded([&] {
        validate_dims(d);
        REQ_PTR(offsets, "offsets");
        REQ_PTR(total_bytes, "total_bytes");
        wire_layout(*d, offsets, total_bytes);
    });
}

int qlx_layer_blob_to_wire(const qlx_dims* d, const void* blob, void* wire) {
    return guarded([&] {
        validate_dims(d);
        REQ_PTR(blob, "blob");
        REQ_PTR(wire, "wire");
        uint64_t fo[QLX_BLOB_NSEG], wo[QLX_BLOB_NSEG], ft, wt;
        blob_layout(*d, fo, &ft);
        wire_layout(*d, wo, &wt);
        const char* b = static_cast<const char*>(blob);
        char* w = static_cast<char*>(wire);
        const uint64_t nb = absmax_blocks(*d);
        // check every maximum first, so a refused blob leaves `wire` untouched
        for (uint64_t i = 0; i < nb; ++i) {
            uint32_t v;
            std::memcpy(&v, b + fo[7] + 4 * i, 4);
            QLX_REQUIRE((v & 0xFFFFu) == 0, QLX_EINVAL,
                        "block maximum " + std::to_string(i) +
                            " is not a bf16 value (its low 16 bits are set): the wire form holds blobs quantized "
                            "from bf16 weights");
        }
        std::memset(w, 0, size_t(wt));
        std::memcpy(w, b, size_t(fo[7]));  // packed regions, same offsets
        for (uint64_t i = 0; i < nb; ++i) {
            uint32_t v;
            std::memcpy(&v, b + fo[7] + 4 * i, 4);
            const uint16_t hi = uint16_t(v >> 16);
            std::memcpy(w + wo[7] + 2 * i, &hi, 2);
        }
        std::memcpy(w + wo[14], b + fo[14], size_t(d->hidden) * 4);
        std::memcpy(w + wo[15], b + fo[15], size_t(d->hidden) * 4);
    });
}

size_t qlx_layer_workspace_bytes(const qlx_dims* d, int batch, int seq) {
    if (!d || batch <= 0 || seq <= 0) return 0;
    return layer_ws_bytes(make_geom(*d, batch, seq));
}

static void validate_lora(const qlx_lora* l) {
    for (int p = 0; p < 7; ++p) {
        QLX_REQUIRE(l->A[p] && l->B[p], QLX_EINVAL, "lora: every A[p] and B[p] must be set");
    }
}
static void validate_grads(const qlx_lora_grad* g) {
    REQ_PTR(g, "grads");
    for (int p = 0; p < 7; ++p) QLX_REQUIRE(g->dA[p] && g->dB[p], QLX_EINVAL, "grads: every dA[p], dB[p] must be set");
}
static void validate_bs(int batch, int seq) {
    QLX_REQUIRE(batch > 0 && seq > 0, QLX_EINVAL, "batch and seq must be positive");
    QLX_REQUIRE(int64_t(batch) * seq <= (1 << 24), QLX_EUNSUPPORTED, "batch*seq too large");
}

int layer_fwd(const qlx_dims* d, const void* blob, const qlx_lora* lora, const float* h_in, int batch, int seq,
              float* h_out, void* ws, size_t ws_bytes, void* stream) {
    return guarded([&] {
        validate_dims(d);
        validate_bs(batch, seq);
        REQ_PTR(blob, "blob");
        REQ_AL(blob, "blob");
        REQ_PTR(h_in, "h_in");
        REQ_PTR(h_out, "h_out");
        if (lora) validate_lora(lora);
        const LayerGeom g = make_geom(*d, batch, seq);
        check_ws(ws, ws_bytes, layer_ws_bytes(g));
        Carver c(ws);
        LayerWs w = carve_layer(c, g);
        layer_forward(g, blob_ptrs(*d, blob), lora, false, h_in, h_out, w, static_cast<hipStream_t>(stream));
    });
}

int layer_bwd(const qlx_dims* d, const void* blob, const qlx_lora* lora, const float* h_in, const float* dh_out,
              int batch, int seq, float* dh_in, const qlx_lora_grad* grads, void* ws, size_t ws_bytes, void* stream) {
    return guarded([&] {
        validate_dims(d);
        validate_bs(batch, seq);
        REQ_PTR(blob, "blob");
        REQ_AL(blob, "blob");
        REQ_PTR(lora, "lora");
        validate_lora(lora);
        validate_grads(grads);
        REQ_PTR(h_in, "h_in");
        REQ_PTR(dh_out, "dh_out");
        const LayerGeom g = make_geom(*d, batch, seq);
        check_ws(ws, ws_bytes, layer_ws_bytes(g));
        Carver c(ws);
        LayerWs w = carve_layer(c, g);
        layer_backward(g, blob_ptrs(*d, blob), lora, h_in, dh_out, dh_in, grads, w, static_cast<hipStream_t>(stream));
    });
}

}  // extern "C"

// ===================================================================== streamer
struct qlx_ctx {
    int device = 0;
    hipStream_t side = nullptr;
    hipStream_t side2 = nullptr;      // second copy stream (copy_split == 2)
    hipEvent_t half_done = nullptr;   // side2's half of the current copy
    hipEvent_t copy_start = nullptr;  // side is ready to overwrite the slot
    hipEvent_t join = nullptr;        // end of a step: the copy streams' work joined into the main stream
    int copy_split = 2;
    int debug = 0;                    // QLX_DEBUG_* flags
    int delay_us = 0;
    hipEvent_t copy_done[2] = {nullptr, nullptr};
    hipEvent_t compute_done[2] = {nullptr, nullptr};
    hipEvent_t step_begin = nullptr, step_end = nullptr;
    std::vector<hipEvent_t> copy_ev;  // timing pairs for copies (begin, end)
    size_t copies_used = 0;
    qlx_stats stats{};
    qlx_layer_file* source = nullptr;  // QLX_STREAMED_DISK
    // qlx_ctx_set_keep_layers: what each slot held when the last step ended
    int keep_layers = 0;
    // qlx_ctx_set_adamw: AdamW applied to each layer's adapters inside the
    // backward, as soon as that layer's gradients are final
    struct FusedAdam {
        bool on = false;
        std::vector<qlx_lora_buf> params, m, v;
        qlx_adamw_cfg cfg{};
        int64_t t = 0;  // update count of the next step
    } adam;
    struct Kept {
        int layer = -1;
        const void* src = nullptr;  // the layer's host blob, or the layer file
        const char* slot = nullptr;
        int form = 0;
    } kept[2];
};

namespace qlx {

constexpr int kVocabChunk = 16384;  // LM-head backward: dz columns per chunk

struct StepWs {
    char* slot[2];
    float* ckpt;     // (L+1) x [T, H]
    uint16_t* usave;  // L x [T, 7r] bf16: each layer's u = x A^T from its forward, for its backward
    float* href[2];  // reference stream (DPO)
    int32_t* toks;   // [T]
    LayerWs lw;
    uint16_t* nf;  // fp16 [T, H]
    float* rstd_f;
    float *ce_pm, *ce_ps;  // [T, V/64] LM-head row partials (max, sum exp)
    float* logits;         // [T, V] the LM head's fp32 logits, kept from the statistics pass for dz
    uint16_t* dzc;         // fp16 [T, kVocabChunk] one vocabulary chunk of dz
    float *lse, *picked, *lse_ref, *pk_ref;
    float* dnf;  // [T, H]
    float* dh[2];
    float* gseq;
    int32_t* kl_toks;                  // KTO only
    float* hkl[2];                     // KTO: mismatched pairs, policy stream
    float* hklr[2];                    // KTO: mismatched pairs, reference stream
    float *kl_lse, *kl_pk, *kl_lse_r, *kl_pk_r;
};

static uint64_t wire_tail_bytes(const qlx_dims& d) {
    uint64_t off[QLX_BLOB_NSEG], total;
    wire_layout(d, off, &total);
    return total - off[7];
}

static StepWs carve_step(Carver& c, const qlx_dims& d, int T, int kind, uint64_t blob_bytes) {
    StepWs w{};
    const LayerGeom g = make_geom(d, 1, T);  // only H, V needed here
    const size_t H = size_t(d.hidden), V = size_t(d.vocab), L = size_t(d.n_layers), Tz = size_t(T);
    // a slot: the full-form blob, then room for a wire-form tail (block
    // maxima as bf16 and the gains) that the widen kernel expands in place
    const uint64_t slot_bytes = blob_bytes + wire_tail_bytes(d);
    w.slot[0] = c.take<char>(slot_bytes);
    w.slot[1] = c.take<char>(slot_bytes);
    w.ckpt = c.take<float>((L + 1) * Tz * H);
    w.usave = c.take<uint16_t>(L * Tz * 7 * size_t(d.lora_r));
    if (kind >= 1) {
        w.href[0] = c.take<float>(Tz * H);
        w.href[1] = c.take<float>(Tz * H);
        w.toks = c.take<int32_t>(Tz);
        w.lse_ref = c.take<float>(Tz);
        w.pk_ref = c.take<float>(Tz);
        w.gseq = c.take<float>(64);
    }
    if (kind == 2) {  // KTO: the mismatched pairs' tokens, two forward streams and their CE stats
        w.kl_toks = c.take<int32_t>(Tz);
        for (int i = 0; i < 2; ++i) {
            w.hkl[i] = c.take<float>(Tz * H);
            w.hklr[i] = c.take<float>(Tz * H);
        }
        w.kl_lse = c.take<float>(Tz);
        w.kl_pk = c.take<float>(Tz);
        w.kl_lse_r = c.take<float>(Tz);
        w.kl_pk_r = c.take<float>(Tz);
    }
    w.nf = c.take<uint16_t>(Tz * H);
    w.rstd_f = c.take<float>(Tz);
    w.ce_pm = c.take<float>(Tz * ((V + 63) / 64));
    w.ce_ps = c.take<float>(Tz * ((V + 63) / 64));
    w.logits = c.take<float>(Tz * V);
    w.dzc = c.take<uint16_t>(Tz * kVocabChunk);
    w.lse = c.take<float>(Tz);
    w.picked = c.take<float>(Tz);
    w.dnf = c.take<float>(Tz * H);
    w.dh[0] = c.take<float>(Tz * H);
    w.dh[1] = c.take<float>(Tz * H);
    (void)g;
    return w;
}

static size_t step_ws_bytes(const qlx_dims& d, int kind, int batch, int seq) {
    uint64_t off[QLX_BLOB_NSEG], blob_bytes;
    blob_layout(d, off, &blob_bytes);
    const int T = batch * seq;
    Carver c(nullptr);
    carve_step(c, d, T, kind, blob_bytes);
    carve_layer(c, make_geom(d, batch, seq));
    return c.size();
}

// Streams layers through the two slots and hands each resident layer to `use`.
class Streamer {
   public:
    Streamer(qlx_ctx* ctx, const qlx_model* m, int mode, const StepWs& w, uint64_t blob_bytes, hipStream_t main)
        : ctx_(ctx), m_(m), mode_(mode), w_(w), bytes_(blob_bytes), main_(main) {
        held_[0] = held_[1] = -1;
        form_ = mode == QLX_STREAMED_DISK ? ctx->source->form : mode == QLX_STREAMED ? m->blob_form : QLX_BLOB_FULL;
        blob_layout(m->dims, full_, &bytes_);
        wire_layout(m->dims, wire_, &wire_bytes_);
        nblocks_ = int64_t(absmax_blocks(m->dims));
        // keep-layers: a slot still holds what the last step left in it when
        // it is the same workspace slot and the layer's source and form match
        for (int sl = 0; sl < 2; ++sl) {
            const qlx_ctx::Kept k = ctx->kept[sl];
            ctx->kept[sl] = qlx_ctx::Kept{};  // valid again only once this step completes its enqueue
            if (ctx->keep_layers && mode != QLX_RESIDENT && k.layer >= 0 && k.layer < m->dims.n_layers &&
                k.slot == w_.slot[sl] && k.form == form_ && k.src == source_of(k.layer) && slot_of(k.layer) == sl)
                held_[sl] = k.layer;
        }
    }
    // End of a step: with keep-layers on, remember what the slots hold.
    void keep() {
        if (!ctx_->keep_layers || mode_ == QLX_RESIDENT) return;
        for (int sl = 0; sl < 2; ++sl)  // (a slot whose widen never ran is not kept)
            if (held_[sl] >= 0 && !widen_pending_[sl])
                ctx_->kept[sl] = qlx_ctx::Kept{held_[sl], source_of(held_[sl]), w_.slot[sl], form_};
    }
    // Make layer i resident (if not already), wait for it on the main stream,
    // and return its device pointer. prefetch_next >= 0 also starts the copy
    // of that layer into the other slot once its previous user is done.
    const void* acquire(int i) {
        if (mode_ == QLX_RESIDENT) return m_->layer_blobs[i];
        const int sl = slot_of(i);
        if (held_[sl] != i) issue_copy(i, sl);
        QLX_CHECK_HIP(hipStreamWaitEvent(main_, ctx_->copy_done[sl], 0));
        if (widen_pending_[sl]) {
            // wire form: block maxima bf16 -> fp32 and the gains into their
            // full-form places, on the compute stream, so the copy stream
            // goes straight on to the next layer's bytes
            char* b = w_.slot[sl];
            const char* tail = b + bytes_;  // wire offset wire_[7] landed here
            launch_blob_widen(reinterpret_cast<const uint16_t*>(tail), nblocks_,
                              reinterpret_cast<const float*>(tail + (wire_[14] - wire_[7])),
                              reinterpret_cast<const float*>(tail + (wire_[15] - wire_[7])), m_->dims.hidden,
                              reinterpret_cast<uint32_t*>(b + full_[7]), reinterpret_cast<float*>(b + full_[14]),
                              reinterpret_cast<float*>(b + full_[15]), main_);
            widen_pending_[sl] = false;
            if (ctx_->debug & QLX_DEBUG_POISON_LIVE)  // control: poisons the slot it just filled
                launch_fill_u32(reinterpret_cast<uint32_t*>(b), int64_t(bytes_ / 4), 0xFFFFFFFFu, main_);
        }
        if (ctx_->debug & QLX_DEBUG_DELAY_COMPUTE) launch_spin(ctx_->delay_us, main_);
        return w_.slot[sl];
    }
    void prefetch(int i) {
        if (mode_ == QLX_RESIDENT || i < 0 || i >= m_->dims.n_layers) return;
        const int sl = slot_of(i);
        if (held_[sl] == i) return;
        issue_copy(i, sl);
    }
    void release(int i) {
        if (mode_ == QLX_RESIDENT) return;
        QLX_CHECK_HIP(hipEventRecord(ctx_->compute_done[slot_of(i)], main_));
        if (ctx_->debug & QLX_DEBUG_SERIALIZE) QLX_CHECK_HIP(hipStreamSynchronize(main_));
    }
    void forget() { held_[0] = held_[1] = -1; }

   private:
    int slot_of(int i) const { return i & 1; }
    const void* source_of(int i) const {
        return mode_ == QLX_STREAMED_DISK ? static_cast<const void*>(ctx_->source) : m_->layer_blobs[i];
    }
    void issue_copy(int i, int sl) {
        // the slot's previous contents must be finished with on the main stream
        QLX_CHECK_HIP(hipStreamWaitEvent(ctx_->side, ctx_->compute_done[sl], 0));
        const void* src = nullptr;
        int k = -1;
        qlx_layer_file* f = ctx_->source;
        if (mode_ == QLX_STREAMED_DISK) {
            // disk -> pinned staging buffer k (once the copy that last read it
            // is done) on this thread, then staging -> slot on the side stream
            k = f->next;
            f->next = (k + 1) % kStaging;
            QLX_CHECK_HIP(hipEventSynchronize(f->staging_free[k]));
            const auto t0 = std::chrono::steady_clock::now();
            layer_file_read(f, i, f->staging[k]);
            ctx_->stats.disk_ms +=
                std::chrono::duration<float, std::milli>(std::chrono::steady_clock::now() - t0).count();
            ctx_->stats.disk_bytes += int64_t(f->stride);
            src = f->staging[k];
        } else {
            src = m_->layer_blobs[i];
        }
        // debugging: a freed slot is filled with NaN bytes before it is
        // refilled (a read of it after its release would show as NaN), and a
        // spin shifts the copy against the compute
        const bool wire = form_ == QLX_BLOB_WIRE;
        const uint64_t nbytes = wire ? wire_bytes_ : bytes_;  // bytes that cross the link
        if (ctx_->debug & QLX_DEBUG_POISON)
            launch_fill_u32(reinterpret_cast<uint32_t*>(w_.slot[sl]), int64_t((bytes_ + wire_bytes_ - wire_[7]) / 4),
                            0xFFFFFFFFu, ctx_->side);
        if (ctx_->debug & QLX_DEBUG_DELAY_COPY) launch_spin(ctx_->delay_us, ctx_->side);
        hipEvent_t* ev = next_timing_pair();
        if (ev) QLX_CHECK_HIP(hipEventRecord(ev[0], ctx_->side));
        const char* s8 = static_cast<const char*>(src);
        if (ctx_->copy_split == 2 && nbytes > 8192) {
            // the two halves on two streams, so two copy engines share the link
            const uint64_t h = (nbytes / 2 + 4095) & ~uint64_t(4095);
            if (ctx_->debug & (QLX_DEBUG_POISON | QLX_DEBUG_DELAY_COPY)) {
                // after the poison fill / spin on the first copy stream
                QLX_CHECK_HIP(hipEventRecord(ctx_->copy_start, ctx_->side));
                QLX_CHECK_HIP(hipStreamWaitEvent(ctx_->side2, ctx_->copy_start, 0));
            } else {
                // only after the slot's previous user, as the first half: at a
                // layer boundary neither copy stream waits for the other
                // (a hop between the two streams cost ~30 us of idle link)
                QLX_CHECK_HIP(hipStreamWaitEvent(ctx_->side2, ctx_->compute_done[sl], 0));
            }
            put(s8, h, nbytes, w_.slot[sl], ctx_->side2);
            QLX_CHECK_HIP(hipEventRecord(ctx_->half_done, ctx_->side2));
            put(s8, 0, h, w_.slot[sl], ctx_->side);
            QLX_CHECK_HIP(hipStreamWaitEvent(ctx_->side, ctx_->half_done, 0));
        } else {
            put(s8, 0, nbytes, w_.slot[sl], ctx_->side);
        }
        widen_pending_[sl] = wire;  // the widen runs on the compute stream in acquire()
        if (ev) QLX_CHECK_HIP(hipEventRecord(ev[1], ctx_->side));
        if (k >= 0) QLX_CHECK_HIP(hipEventRecord(f->staging_free[k], ctx_->side));
        if ((ctx_->debug & QLX_DEBUG_POISON_LIVE) && !wire)  // control: poisons the slot it just filled
            launch_fill_u32(reinterpret_cast<uint32_t*>(w_.slot[sl]), int64_t(bytes_ / 4), 0xFFFFFFFFu, ctx_->side);
        QLX_CHECK_HIP(hipEventRecord(ctx_->copy_done[sl], ctx_->side));
        if (ctx_->debug & QLX_DEBUG_SERIALIZE) QLX_CHECK_HIP(hipStreamSynchronize(ctx_->side));
        held_[sl] = i;
        ctx_->stats.layer_reads += 1;
        ctx_->stats.h2d_bytes += int64_t(nbytes);
    }
    // Copies bytes [lo, hi) of a layer's source blob to their place in slot
    // `dst`: the full form is copied as is; in the wire form the packed
    // regions (before wire_[7]) keep their offsets and the tail lands after
    // the full-form blob, where the widen kernel reads it.
    void put(const char* src, uint64_t lo, uint64_t hi, char* dst, hipStream_t st) {
        const uint64_t P = form_ == QLX_BLOB_WIRE ? wire_[7] : hi;
        if (lo < std::min(hi, P))
            QLX_CHECK_HIP(hipMemcpyAsync(dst + lo, src + lo, std::min(hi, P) - lo, hipMemcpyHostToDevice, st));
        const uint64_t a = std::max(lo, P);
        if (a < hi) QLX_CHECK_HIP(hipMemcpyAsync(dst + bytes_ + (a - P), src + a, hi - a, hipMemcpyHostToDevice, st));
    }
    hipEvent_t* next_timing_pair() {
        if (ctx_->copies_used + 2 > ctx_->copy_ev.size()) return nullptr;
        hipEvent_t* e = &ctx_->copy_ev[ctx_->copies_used];
        ctx_->copies_used += 2;
        return e;
    }
    qlx_ctx* ctx_;
    const qlx_model* m_;
    int mode_;
    const StepWs& w_;
    uint64_t bytes_;  // full-form blob
    hipStream_t main_;
    int held_[2];
    bool widen_pending_[2] = {false, false};  // wire-form slot copied, not yet widened
    int form_ = QLX_BLOB_FULL;
    uint64_t full_[QLX_BLOB_NSEG] = {}, wire_[QLX_BLOB_NSEG] = {}, wire_bytes_ = 0;
    int64_t nblocks_ = 0;
};

// A fused AdamW must update exactly the step's adapters.
static void check_fused_adam(const qlx_ctx* ctx, const qlx_model* m) {
    if (!ctx->adam.on) return;
    QLX_REQUIRE(int(ctx->adam.params.size()) == m->dims.n_layers, QLX_EINVAL,
                "fused AdamW: registered for another number of layers");
    for (int l = 0; l < m->dims.n_layers; ++l)
        for (int p = 0; p < 7; ++p)
            QLX_REQUIRE(ctx->adam.params[l].A[p] == m->lora[l].A[p] && ctx->adam.params[l].B[p] == m->lora[l].B[p],
                        QLX_EINVAL, "fused AdamW: its parameters are not the model's adapters");
}

static void validate_model(qlx_ctx* ctx, const qlx_model* m, int mode) {
    REQ_PTR(ctx, "ctx");
    REQ_PTR(m, "model");
    validate_dims(&m->dims);
    QLX_REQUIRE(mode == QLX_STREAMED || mode == QLX_RESIDENT || mode == QLX_STREAMED_DISK, QLX_EINVAL,
                "mode must be QLX_STREAMED, QLX_RESIDENT or QLX_STREAMED_DISK");
    if (mode == QLX_STREAMED_DISK) {
        const qlx_layer_file* f = ctx->source;
        QLX_REQUIRE(f != nullptr, QLX_EINVAL, "QLX_STREAMED_DISK needs a layer file attached to the context");
        uint64_t off[QLX_BLOB_NSEG], blob_bytes = 0;
        if (f->form == QLX_BLOB_WIRE) wire_layout(m->dims, off, &blob_bytes);
        else blob_layout(m->dims, off, &blob_bytes);
        QLX_REQUIRE(f->dims.n_layers == m->dims.n_layers && f->blob_bytes == blob_bytes, QLX_EINVAL,
                    "the context's layer file was opened for other model dims");
    } else {
        REQ_PTR(m->layer_blobs, "model.layer_blobs");
        QLX_REQUIRE(m->blob_form == QLX_BLOB_FULL || (m->blob_form == QLX_BLOB_WIRE && mode == QLX_STREAMED),
                    QLX_EINVAL, "model.blob_form: QLX_BLOB_FULL, or QLX_BLOB_WIRE with QLX_STREAMED");
    }
    REQ_PTR(m->embed_f16, "model.embed_f16");
    REQ_PTR(m->lm_head_f16, "model.lm_head_f16");
    REQ_PTR(m->final_norm, "model.final_norm");
    REQ_PTR(m->lora, "model.lora");
    check_fused_adam(ctx, m);
    REQ_AL(m->lm_head_f16, "model.lm_head_f16");
    for (int i = 0; i < m->dims.n_layers; ++i) {
        validate_lora(&m->lora[i]);
        if (mode == QLX_STREAMED_DISK) continue;
        const void* b = m->layer_blobs[i];
        QLX_REQUIRE(b != nullptr, QLX_EINVAL, "model.layer_blobs[" + std::to_string(i) + "] is NULL");
        REQ_AL(b, "layer blob");
        if (mode == QLX_STREAMED) {
            hipPointerAttribute_t attr;
            const hipError_t e = hipPointerGetAttributes(&attr, b);
            if (e != hipSuccess) (void)hipGetLastError();
            QLX_REQUIRE(e == hipSuccess && attr.type == hipMemoryTypeHost, QLX_ENOTPINNED,
                        "layer blob " + std::to_string(i) + " is not pinned host memory");
        }
    }
}

static void begin_step(qlx_ctx* ctx, hipStream_t main) {
    QLX_CHECK_HIP(hipSetDevice(ctx->device));
    ctx->stats = qlx_stats{};
    ctx->copies_used = 0;
    QLX_CHECK_HIP(hipEventRecord(ctx->step_begin, main));
    // the side stream starts after everything already queued on main
    QLX_CHECK_HIP(hipEventRecord(ctx->compute_done[0], main));
    QLX_CHECK_HIP(hipEventRecord(ctx->compute_done[1], main));
}
static void end_step(qlx_ctx* ctx, hipStream_t main) {
    // (side2's half of every copy is already waited for on side)
    QLX_CHECK_HIP(hipEventRecord(ctx->join, ctx->side));
    QLX_CHECK_HIP(hipStreamWaitEvent(main, ctx->join, 0));
    QLX_CHECK_HIP(hipEventRecord(ctx->step_end, main));
}

// Fused LM head + cross-entropy. Forward: final RMSNorm (fp16 out), then the
// head GEMM whose epilogue reduces each row's logits to per-64-column (max,
// sum exp) partials, picks the target's logit and, for the stream whose
// backward follows (logits non-null), stores the fp32 logits; a row reduce
// gives lse. Backward: per vocabulary chunk of kVocabChunk columns, fp16
// dz = (softmax - onehot) * scale from the stored logits, then dnf +=
// dz_chunk . head_chunk (fp32, chunk order), then RMSNorm backward. (Keeping
// the logits costs 4 T V bytes of workspace and saves a second pass of the
// head product.)
static void head_stats(const qlx_model* m, const float* hL, int T, const int32_t* tokens, int seq, int start,
                       float* lse, float* picked, float* logits, StepWs& w, float* partial, hipStream_t s) {
    const qlx_dims& d = m->dims;
    const int nb = (d.vocab + 63) / 64;
    launch_rmsnorm_fwd(hL, m->final_norm, T, d.hidden, d.rms_eps, w.nf, 1, w.rstd_f, s);
    GemmParams p;
    p.M = T;
    p.N = d.vocab;
    p.K = d.hidden;
    p.A = w.nf;
    p.lda = d.hidden;
    p.B = m->lm_head_f16;
    p.ldb = d.hidden;
    p.c_type = C_F16;
    p.ce_mode = 1;
    p.ce_tokens = tokens;
    p.ce_seq = seq;
    p.ce_start = start;
    p.ce_pm = w.ce_pm;
    p.ce_ps = w.ce_ps;
    p.ce_pld = nb;
    p.ce_picked = picked;
    p.ce_logits = logits;
    p.ce_ldl = d.vocab;
    p.tag = "gemm_head";
    gemm(p, A_ROW, B_DENSE_NT, TE_F16, partial, s);
    launch_ce_reduce(w.ce_pm, w.ce_ps, nb, T, d.vocab, tokens, seq, start, lse, picked, s);
}
// dh = RMSNorm^T( (dz . head) * alpha ), dz = (softmax - onehot) * sc (* gseq per sequence)
static void head_grad(const qlx_model* m, const float* hL, int T, const int32_t* tokens, int seq, int start,
                      const float* lse, float sc, const float* gseq, float alpha, StepWs& w, float* dh_out,
                      float* partial, hipStream_t s) {
    const qlx_dims& d = m->dims;
    for (int c0 = 0; c0 < d.vocab; c0 += kVocabChunk) {
        const int cw = std::min(kVocabChunk, d.vocab - c0);
        const uint16_t* head = m->lm_head_f16 + size_t(c0) * d.hidden;
        launch_ce_dz(w.logits, d.vocab, T, cw, c0, tokens, seq, start, lse, sc, gseq, w.dzc, kVocabChunk, s);
        GemmParams q;
        q.M = T;
        q.N = d.hidden;
        q.K = cw;
        q.A = w.dzc;
        q.lda = kVocabChunk;
        q.B = head;
        q.ldb = d.hidden;
        q.C = w.dnf;
        q.ldc = d.hidden;
        q.c_type = C_F32;
        q.alpha = alpha;
        q.accumulate = c0 > 0;
        q.tag = "gemm_head_dx";
        gemm(q, A_ROW, B_DENSE_NN, TE_F16, partial, s);
    }
    launch_rmsnorm_bwd(w.dnf, hL, m->final_norm, w.rstd_f, nullptr, T, d.hidden, dh_out, s);
}

// dz is stored in fp16 scaled by 2^12 so that softmax values ~1/V stay normal.
constexpr float kDzScale = 4096.f;

// Gradient scale of a step's backward with fp16 activations: the power of two
// that puts the loss's largest possible per-position logit gradient (bound)
// at 2^10. The layers' 16-bit gradients then stay far above fp16's smallest
// normal value (2^-14) and below its largest (65504) as long as they grow at
// most ~60x over the head's bound through the stack. With bf16 (fp32's
// exponent range) no scale is needed: 1.
static float grad_scale(const LayerGeom& g, double bound) {
    if (!g.f16 || !(bound > 0.0)) return 1.f;
    return float(std::exp2(std::floor(std::log2(1024.0 / bound))));
}
// the preference losses' bound on |dL/dz| per position (= |dL/dlp| of a sequence)
static double pref_grad_bound(const qlx_pref_cfg& cfg, int pairs, int nresp) {
    const double P = pairs, n = std::max(1, nresp), b = cfg.beta;
    switch (cfg.kind) {
        case QLX_PREF_ORPO: return (1.0 + b) / (P * n);  // while the mean response probability stays below 1/2
        case QLX_PREF_SIMPO: return b / (P * n);
        case QLX_PREF_KTO: return std::max(cfg.lambda_d, cfg.lambda_u) * b / 4.0 / (2.0 * P);
        default: return b / P;  // DPO
    }
}

static void check_adamw_cfg(const qlx_adamw_cfg* cfg, int64_t t) {
    REQ_PTR(cfg, "cfg");
    QLX_REQUIRE(t >= 1, QLX_EINVAL, "adamw: t (1-based update count) must be >= 1");
    QLX_REQUIRE(std::isfinite(cfg->lr) && cfg->lr >= 0.0, QLX_EINVAL, "adamw: lr must be finite and >= 0");
    QLX_REQUIRE(cfg->beta1 >= 0.0 && cfg->beta1 < 1.0 && cfg->beta2 >= 0.0 && cfg->beta2 < 1.0, QLX_EINVAL,
                "adamw: betas must lie in [0, 1)");
    QLX_REQUIRE(std::isfinite(cfg->eps) && cfg->eps > 0.0, QLX_EINVAL, "adamw: eps must be finite and > 0");
    QLX_REQUIRE(std::isfinite(cfg->weight_decay) && cfg->weight_decay >= 0.0, QLX_EINVAL,
                "adamw: weight_decay must be finite and >= 0");
}
// Update-t constants, formed in double (1 - beta before any rounding).
static AdamScalars adam_scalars(const qlx_adamw_cfg& cfg, int64_t t) {
    AdamScalars c;
    c.decay = float(1.0 - cfg.lr * cfg.weight_decay);
    c.b1 = float(cfg.beta1);
    c.one_m_b1 = float(1.0 - cfg.beta1);
    c.b2 = float(cfg.beta2);
    c.one_m_b2 = float(1.0 - cfg.beta2);
    c.step_size = float(cfg.lr / (1.0 - std::pow(cfg.beta1, double(t))));
    c.inv_bc2_sqrt = float(1.0 / std::sqrt(1.0 - std::pow(cfg.beta2, double(t))));
    c.eps = float(cfg.eps);
    return c;
}
// AdamW on one layer's 14 adapter tensors: one launch.
static void adamw_layer(const LayerGeom& g, int r, const qlx_lora_buf& p, const qlx_lora_grad& gr,
                        const qlx_lora_buf& m, const qlx_lora_buf& v, const AdamScalars& c, hipStream_t s) {
    AdamTensor ts[14];
    for (int q = 0; q < 7; ++q) {
        ts[2 * q] = {p.A[q], gr.dA[q], m.A[q], v.A[q], int64_t(r) * g.in[q]};
        ts[2 * q + 1] = {p.B[q], gr.dB[q], m.B[q], v.B[q], int64_t(g.out[q]) * r};
    }
    launch_adamw(ts, 14, c, s);
}

// Layer i's kept u (u_qkv | u_o | u_gu | u_d, T x 7r bf16).
static uint16_t* u_area(const StepWs& w, const LayerGeom& g, int i) {
    return w.usave + size_t(i) * size_t(g.T) * 7 * size_t(g.r);
}

// The backward over all layers, last to first. The layer workspace still
// holds the last layer's forward activations (its policy forward is the last
// layer pass of every step's forward; the head only uses its own buffers and
// the split-K scratch), so that layer is not recomputed. With a fused AdamW
// on the context, layer i's adapters are updated right after its backward:
// nothing later in the step reads them, and the update overlaps the copies
// and compute of the layers still to come.
static void backward_layers(qlx_ctx* ctx, Streamer& st, const qlx_model* m, const LayerGeom& g, StepWs& w, float* dh,
                            const qlx_lora_grad* grads, hipStream_t s) {
    const int L = m->dims.n_layers;
    const size_t TH = size_t(g.T) * g.H;
    float* cur = dh;
    float* nxt = (dh == w.dh[0]) ? w.dh[1] : w.dh[0];
    const qlx_ctx::FusedAdam& fa = ctx->adam;
    const LayerGeom g1 = make_geom(m->dims, 1, 1);
    const AdamScalars ac = fa.on ? adam_scalars(fa.cfg, fa.t) : AdamScalars{};
    for (int i = L - 1; i >= 0; --i) {
        const void* blob = st.acquire(i);
        st.prefetch(i - 1);
        point_u(w.lw, u_area(w, g, i), g);  // its forward's u: the recompute skips those products
        layer_backward(g, blob_ptrs(m->dims, blob), &m->lora[i], w.ckpt + size_t(i) * TH, cur, i > 0 ? nxt : nullptr,
                       &grads[i], w.lw, s, /*recompute=*/i != L - 1, /*u_given=*/true);
        if (fa.on) adamw_layer(g1, m->dims.lora_r, fa.params[i], grads[i], fa.m[i], fa.v[i], ac, s);
        st.release(i);
        std::swap(cur, nxt);
    }
}


}  // namespace qlx

extern "C" {

int qlx_ctx_create(qlx_ctx** out, int device) {
    return guarded([&] {
        REQ_PTR(out, "out");
        int n = 0;
        QLX_CHECK_HIP(hipGetDeviceCount(&n));
        QLX_REQUIRE(device >= 0 && device < n, QLX_EINVAL, "device out of range");
        QLX_CHECK_HIP(hipSetDevice(device));
        qlx_ctx* c = new qlx_ctx();
        c->device = device;
        QLX_CHECK_HIP(hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking));
        QLX_CHECK_HIP(hipStreamCreateWithFlags(&c->side2, hipStreamNonBlocking));
        QLX_CHECK_HIP(hipEventCreateWithFlags(&c->half_done, hipEventDisableTiming));
        QLX_CHECK_HIP(hipEventCreateWithFlags(&c->copy_start, hipEventDisableTiming));
        QLX_CHECK_HIP(hipEventCreateWithFlags(&c->join, hipEventDisableTiming));
        // QLX_COPY_SPLIT=1: one copy stream (default 2: each layer copy in two halves on two streams)
        if (const char* e = std::getenv("QLX_COPY_SPLIT")) c->copy_split = std::atoi(e) == 1 ? 1 : 2;
        for (int i = 0; i < 2; ++i) {
            QLX_CHECK_HIP(hipEventCreateWithFlags(&c->copy_done[i], hipEventDisableTiming));
            QLX_CHECK_HIP(hipEventCreateWithFlags(&c->compute_done[i], hipEventDisableTiming));
        }
        QLX_CHECK_HIP(hipEventCreate(&c->step_begin));
        QLX_CHECK_HIP(hipEventCreate(&c->step_end));
        c->copy_ev.resize(512);
        for (auto& e : c->copy_ev) QLX_CHECK_HIP(hipEventCreate(&e));
        *out = c;
    });
}

int qlx_ctx_destroy(qlx_ctx* ctx) {
    return guarded([&] {
        if (!ctx) return;
        (void)hipSetDevice(ctx->device);
        (void)hipStreamSynchronize(ctx->side);
        if (ctx->source) ctx->source->attached -= 1;  // the file outlives the context
        for (auto& e : ctx->copy_ev) (void)hipEventDestroy(e);
        for (int i = 0; i < 2; ++i) {
            (void)hipEventDestroy(ctx->copy_done[i]);
            (void)hipEventDestroy(ctx->compute_done[i]);
        }
        (void)hipEventDestroy(ctx->step_begin);
        (void)hipEventDestroy(ctx->step_end);
        (void)hipStreamSynchronize(ctx->side2);
        (void)hipEventDestroy(ctx->half_done);
        (void)hipEventDestroy(ctx->copy_start);
        (void)hipEventDestroy(ctx->join);
        (void)hipStreamDestroy(ctx->side2);
        (void)hipStreamDestroy(ctx->side);
        delete ctx;
    });
}

int qlx_ctx_set_debug(qlx_ctx* ctx, int flags, int delay_us) {
    return guarded([&] {
        REQ_PTR(ctx, "ctx");
        QLX_REQUIRE((flags & ~(QLX_DEBUG_SERIALIZE | QLX_DEBUG_POISON | QLX_DEBUG_DELAY_COPY | QLX_DEBUG_DELAY_COMPUTE |
                               QLX_DEBUG_POISON_LIVE)) == 0,
                    QLX_EINVAL, "unknown debug flags");
        QLX_REQUIRE(delay_us >= 0 && delay_us <= 1000000, QLX_EINVAL, "delay_us must be in 0..1000000");
        ctx->debug = flags;
        ctx->delay_us = delay_us;
    });
}

int qlx_ctx_set_keep_layers(qlx_ctx* ctx, int on) {
    return guarded([&] {
        REQ_PTR(ctx, "ctx");
        QLX_REQUIRE(on == 0 || on == 1, QLX_EINVAL, "keep_layers: 0 or 1");
        ctx->keep_layers = on;
        ctx->kept[0] = ctx->kept[1] = qlx_ctx::Kept{};
    });
}

int qlx_ctx_set_adamw(qlx_ctx* ctx, int n_layers, const qlx_lora_buf* params, const qlx_lora_buf* m,
                      const qlx_lora_buf* v, const qlx_adamw_cfg* cfg, int64_t t_next) {
    return guarded([&] {
        REQ_PTR(ctx, "ctx");
        if (!params) {
            ctx->adam = qlx_ctx::FusedAdam{};
            return;
        }
        REQ_PTR(m, "m");
        REQ_PTR(v, "v");
        QLX_REQUIRE(n_layers >= 1, QLX_EINVAL, "adamw: n_layers must be >= 1");
        check_adamw_cfg(cfg, t_next);
        for (int l = 0; l < n_layers; ++l)
            for (int p = 0; p < 7; ++p)
                QLX_REQUIRE(params[l].A[p] && params[l].B[p] && m[l].A[p] && m[l].B[p] && v[l].A[p] && v[l].B[p],
                            QLX_EINVAL, "adamw: every params/m/v A[p], B[p] must be set");
        qlx_ctx::FusedAdam fa;
        fa.on = true;
        fa.params.assign(params, params + n_layers);
        fa.m.assign(m, m + n_layers);
        fa.v.assign(v, v + n_layers);
        fa.cfg = *cfg;
        fa.t = t_next;
        ctx->adam = std::move(fa);
    });
}

int qlx_ctx_adamw_t(const qlx_ctx* ctx, int64_t* t_next) {
    return guarded([&] {
        REQ_PTR(ctx, "ctx");
        REQ_PTR(t_next, "t_next");
        *t_next = ctx->adam.on ? ctx->adam.t : 0;
    });
}

int qlx_ctx_set_layer_source(qlx_ctx* ctx, qlx_layer_file* f) {
    return guarded([&] {
        REQ_PTR(ctx, "ctx");
        if (f == ctx->source) return;
        // slots filled from another source are never taken for this one's layers
        // (a later file could even reuse the detached one's address)
        ctx->kept[0] = ctx->kept[1] = qlx_ctx::Kept{};
        if (!f) {
            ctx->source->attached -= 1;
            ctx->source = nullptr;
            return;
        }
        QLX_REQUIRE(f->device < 0 || f->device == ctx->device, QLX_EINVAL,
                    "the layer file is bound to device " + std::to_string(f->device));
        QLX_CHECK_HIP(hipSetDevice(ctx->device));
        if (f->device < 0) {
            for (int k = 0; k < kStaging; ++k) {
                QLX_CHECK_HIP(hipHostMalloc(reinterpret_cast<void**>(&f->staging[k]), f->stride, hipHostMallocDefault));
                QLX_CHECK_HIP(hipEventCreateWithFlags(&f->staging_free[k], hipEventDisableTiming));
                QLX_CHECK_HIP(hipEventRecord(f->staging_free[k], ctx->side));  // free from the start
            }
            f->device = ctx->device;
        }
        if (ctx->source) ctx->source->attached -= 1;
        ctx->source = f;
        f->attached += 1;
    });
}

int qlx_ctx_sync(qlx_ctx* ctx, qlx_stats* stats) {
    return guarded([&] {
        REQ_PTR(ctx, "ctx");
        QLX_CHECK_HIP(hipSetDevice(ctx->device));
        QLX_CHECK_HIP(hipStreamSynchronize(ctx->side));
        QLX_CHECK_HIP(hipEventSynchronize(ctx->step_end));
        float ms = 0.f;
        QLX_CHECK_HIP(hipEventElapsedTime(&ms, ctx->step_begin, ctx->step_end));
        ctx->stats.step_ms = ms;
        float h2d = 0.f;
        for (size_t i = 0; i + 1 < ctx->copies_used; i += 2) {
            float t = 0.f;
            QLX_CHECK_HIP(hipEventElapsedTime(&t, ctx->copy_ev[i], ctx->copy_ev[i + 1]));
            h2d += t;
        }
        ctx->stats.h2d_ms = h2d;
        if (stats) *stats = ctx->stats;
    });
}

size_t qlx_step_workspace_bytes(const qlx_dims* d, int kind, int batch, int seq) {
    if (!d || batch <= 0 || seq <= 0 || kind < 0 || kind > 2) return 0;
    return step_ws_bytes(*d, kind, kind >= 1 ? 2 * batch : batch, seq);
}

int stream_step_sft(qlx_ctx* ctx, const qlx_model* m, const int32_t* tokens, int batch, int seq, int mode,
                    float* loss, const qlx_lora_grad* grads, void* ws, size_t ws_bytes, void* stream) {
    return guarded([&] {
        validate_model(ctx, m, mode);
        validate_bs(batch, seq);
        QLX_REQUIRE(seq >= 2, QLX_EINVAL, "seq must be >= 2 for next-token loss");
        REQ_PTR(tokens, "tokens");
        REQ_PTR(loss, "loss");
        REQ_PTR(grads, "grads");
        for (int i = 0; i < m->dims.n_layers; ++i) validate_grads(&grads[i]);
        const qlx_dims& d = m->dims;
        check_ws(ws, ws_bytes, step_ws_bytes(d, 0, batch, seq));
        hipStream_t s = static_cast<hipStream_t>(stream);
        uint64_t off[QLX_BLOB_NSEG], blob_bytes;
        blob_layout(d, off, &blob_bytes);
        const int T = batch * seq;
        Carver c(ws);
        StepWs w = carve_step(c, d, T, 0, blob_bytes);
        LayerGeom g = make_geom(d, batch, seq);
        g.gsc = grad_scale(g, 1.0 / (double(batch) * double(seq - 1)));  // SFT: |dL/dz| <= 1/N
        w.lw = carve_layer(c, g);
        const size_t TH = size_t(T) * d.hidden;
        const int L = d.n_layers;

        begin_step(ctx, s);
        Streamer st(ctx, m, mode, w, blob_bytes, s);
        launch_embed(tokens, m->embed_f16, T, d.hidden, d.vocab, w.ckpt, s);
        st.prefetch(0);
        for (int i = 0; i < L; ++i) {
            const void* blob = st.acquire(i);
            st.prefetch(i + 1);
            point_u(w.lw, u_area(w, g, i), g);  // kept for this layer's backward
            layer_forward(g, blob_ptrs(d, blob), &m->lora[i], false, w.ckpt + size_t(i) * TH,
                          w.ckpt + size_t(i + 1) * TH, w.lw, s);
            st.release(i);
        }
        const float* hL = w.ckpt + size_t(L) * TH;
        head_stats(m, hL, T, tokens, seq, 0, w.lse, w.picked, w.logits, w, w.lw.partial, s);
        launch_sft_loss(w.lse, w.picked, T, seq, loss, s);
        const float alpha = 1.0f / (kDzScale * float(batch) * float(seq - 1));
        head_grad(m, hL, T, tokens, seq, 0, w.lse, kDzScale, nullptr, alpha, w, w.dh[0], w.lw.partial, s);
        ctx->stats.layer_passes = 2 * L;
        backward_layers(ctx, st, m, g, w, w.dh[0], grads, s);
        st.keep();
        if (ctx->adam.on) ctx->adam.t += 1;
        end_step(ctx, s);
    });
}

// One preference step: DPO, ORPO, SimPO or KTO on the same layer stream.
// The reference-free kinds (ORPO, SimPO) skip the reference pass; KTO adds
// forward-only passes over the mismatched pairs (policy and reference) for z0.
static void pref_step(qlx_ctx* ctx, const qlx_model* m, const qlx_pref_cfg& cfg, const int32_t* chosen,
                      const int32_t* rejected, int pairs, int seq, int prompt_len, int mode, float* loss, float* logps,
                      const qlx_lora_grad* grads, void* ws, size_t ws_bytes, hipStream_t s) {
    validate_model(ctx, m, mode);
    QLX_REQUIRE(pairs > 0 && pairs <= 32, QLX_EINVAL, "pairs must be in 1..32");
    validate_bs(2 * pairs, seq);
    QLX_REQUIRE(prompt_len >= 1 && prompt_len < seq, QLX_EINVAL, "prompt_len must be in [1, seq)");
    QLX_REQUIRE(cfg.kind >= QLX_PREF_DPO && cfg.kind <= QLX_PREF_KTO, QLX_EINVAL, "preference kind");
    QLX_REQUIRE(cfg.ref_schedule == QLX_DPO_REF_FUSED || cfg.ref_schedule == QLX_DPO_REF_SEPARATE, QLX_EINVAL,
                "ref_schedule");
    QLX_REQUIRE(std::isfinite(cfg.beta) && std::isfinite(cfg.gamma) && std::isfinite(cfg.lambda_d) &&
                    std::isfinite(cfg.lambda_u),
                QLX_EINVAL, "preference hyperparameters must be finite");
    REQ_PTR(chosen, "chosen");
    REQ_PTR(rejected, "rejected");
    REQ_PTR(loss, "loss");
    REQ_PTR(logps, "logps");
    REQ_PTR(grads, "grads");
    for (int i = 0; i < m->dims.n_layers; ++i) validate_grads(&grads[i]);
    const qlx_dims& d = m->dims;
    const int B = 2 * pairs;
    const bool kto = cfg.kind == QLX_PREF_KTO;
    const bool need_ref = cfg.kind == QLX_PREF_DPO || kto;
    const int wkind = kto ? 2 : 1;
    check_ws(ws, ws_bytes, step_ws_bytes(d, wkind, B, seq));
    uint64_t off[QLX_BLOB_NSEG], blob_bytes;
    blob_layout(d, off, &blob_bytes);
    const int T = B * seq;
    Carver c(ws);
    StepWs w = carve_step(c, d, T, wkind, blob_bytes);
    LayerGeom g = make_geom(d, B, seq);
    g.gsc = grad_scale(g, pref_grad_bound(cfg, pairs, seq - prompt_len));
    w.lw = carve_layer(c, g);
    const size_t TH = size_t(T) * d.hidden;
    const int L = d.n_layers;

    begin_step(ctx, s);
    const size_t half = size_t(pairs) * seq * sizeof(int32_t);
    QLX_CHECK_HIP(hipMemcpyAsync(w.toks, chosen, half, hipMemcpyDeviceToDevice, s));
    QLX_CHECK_HIP(hipMemcpyAsync(w.toks + size_t(pairs) * seq, rejected, half, hipMemcpyDeviceToDevice, s));
    Streamer st(ctx, m, mode, w, blob_bytes, s);
    launch_embed(w.toks, m->embed_f16, T, d.hidden, d.vocab, w.ckpt, s);
    // forward streams besides the policy's checkpoints: (input, ping, pong, lora)
    struct Fwd {
        float* cur;
        float* buf[2];
        const bool lora;
    };
    std::vector<Fwd> extra;
    if (need_ref) extra.push_back(Fwd{w.ckpt, {w.href[0], w.href[1]}, false});  // reference shares h_0
    if (kto) {
        launch_kl_tokens(w.toks, B, seq, prompt_len, w.kl_toks, s);
        launch_embed(w.kl_toks, m->embed_f16, T, d.hidden, d.vocab, w.hklr[0], s);
        QLX_CHECK_HIP(hipMemcpyAsync(w.hkl[0], w.hklr[0], TH * sizeof(float), hipMemcpyDeviceToDevice, s));
        extra.push_back(Fwd{w.hklr[0], {w.hklr[1], w.hklr[0]}, false});  // mismatched pairs, reference
        extra.push_back(Fwd{w.hkl[0], {w.hkl[1], w.hkl[0]}, true});      // mismatched pairs, policy
    }
    uint16_t* const own_u[4] = {w.lw.u_qkv, w.lw.u_o, w.lw.u_gu, w.lw.u_d};
    auto advance = [&](Fwd& f, const BlobPtrs& wt, int i) {
        float* nxt = (f.cur == f.buf[0]) ? f.buf[1] : f.buf[0];
        w.lw.u_qkv = own_u[0];  // forward-only passes: u in the layer workspace's own buffers
        w.lw.u_o = own_u[1];
        w.lw.u_gu = own_u[2];
        w.lw.u_d = own_u[3];
        layer_forward(g, wt, f.lora ? &m->lora[i] : nullptr, false, f.cur, nxt, w.lw, s);
        f.cur = nxt;
    };
    const bool separate = need_ref && cfg.ref_schedule == QLX_DPO_REF_SEPARATE;
    if (separate) {  // the forward-only streams first, then the policy pass streams the stack again
        st.prefetch(0);
        for (int i = 0; i < L; ++i) {
            const void* blob = st.acquire(i);
            st.prefetch(i + 1);
            const BlobPtrs wt = blob_ptrs(d, blob);
            for (Fwd& f : extra) advance(f, wt, i);
            st.release(i);
        }
        st.forget();
    }
    st.prefetch(0);
    for (int i = 0; i < L; ++i) {
        const void* blob = st.acquire(i);
        st.prefetch(i + 1);
        const BlobPtrs wt = blob_ptrs(d, blob);
        if (!separate)
            for (Fwd& f : extra) advance(f, wt, i);
        point_u(w.lw, u_area(w, g, i), g);  // kept for this layer's backward
        layer_forward(g, wt, &m->lora[i], false, w.ckpt + size_t(i) * TH, w.ckpt + size_t(i + 1) * TH, w.lw, s);
        st.release(i);
    }
    const int start = prompt_len - 1;
    if (need_ref) {  // reference log-probs
        head_stats(m, extra[0].cur, T, w.toks, seq, start, w.lse_ref, w.pk_ref, nullptr, w, w.lw.partial, s);
    }
    if (kto) {  // mismatched pairs: reference, then policy
        head_stats(m, extra[1].cur, T, w.kl_toks, seq, start, w.kl_lse_r, w.kl_pk_r, nullptr, w, w.lw.partial, s);
        head_stats(m, extra[2].cur, T, w.kl_toks, seq, start, w.kl_lse, w.kl_pk, nullptr, w, w.lw.partial, s);
    }
    // policy log-probs, loss, and dL/dlp
    const float* hL = w.ckpt + size_t(L) * TH;
    head_stats(m, hL, T, w.toks, seq, start, w.lse, w.picked, w.logits, w, w.lw.partial, s);
    PrefLossArgs la{};
    la.lse_p = w.lse;
    la.pk_p = w.picked;
    la.lse_r = need_ref ? w.lse_ref : nullptr;
    la.pk_r = need_ref ? w.pk_ref : nullptr;
    la.kl_lse_p = kto ? w.kl_lse : nullptr;
    la.kl_pk_p = kto ? w.kl_pk : nullptr;
    la.kl_lse_r = kto ? w.kl_lse_r : nullptr;
    la.kl_pk_r = kto ? w.kl_pk_r : nullptr;
    la.pairs = pairs;
    la.seq = seq;
    la.nresp = seq - prompt_len;
    la.kind = cfg.kind;
    la.beta = cfg.beta;
    la.gamma = cfg.gamma;
    la.lambda_d = cfg.lambda_d;
    la.lambda_u = cfg.lambda_u;
    la.loss = loss;
    la.logps = logps;
    la.gseq = w.gseq;
    launch_pref_loss(la, s);
    // dz = g_seq (onehot - softmax) = (softmax - onehot) * (-g_seq)
    head_grad(m, hL, T, w.toks, seq, start, w.lse, -kDzScale, w.gseq, 1.0f / kDzScale, w, w.dh[0], w.lw.partial, s);
    ctx->stats.layer_passes = int64_t(2 + extra.size()) * L;
    backward_layers(ctx, st, m, g, w, w.dh[0], grads, s);
    st.keep();
    if (ctx->adam.on) ctx->adam.t += 1;
    end_step(ctx, s);
}

int stream_step_dpo(qlx_ctx* ctx, const qlx_model* m, const int32_t* chosen, const int32_t* rejected, int pairs,
                    int seq, int prompt_len, float beta, int mode, int ref_schedule, float* loss, float* logps,
                    const qlx_lora_grad* grads, void* ws, size_t ws_bytes, void* stream) {
    return guarded([&] {
        QLX_REQUIRE(beta == beta, QLX_EINVAL, "beta is NaN");
        qlx_pref_cfg cfg{QLX_PREF_DPO, ref_schedule, beta, 0.f, 1.f, 1.f};
        pref_step(ctx, m, cfg, chosen, rejected, pairs, seq, prompt_len, mode, loss, logps, grads, ws, ws_bytes,
                  static_cast<hipStream_t>(stream));
    });
}

int stream_step_pref(qlx_ctx* ctx, const qlx_model* m, const qlx_pref_cfg* cfg, const int32_t* chosen,
                     const int32_t* rejected, int pairs, int seq, int prompt_len, int mode, float* loss, float* logps,
                     const qlx_lora_grad* grads, void* ws, size_t ws_bytes, void* stream) {
    return guarded([&] {
        REQ_PTR(cfg, "cfg");
        pref_step(ctx, m, *cfg, chosen, rejected, pairs, seq, prompt_len, mode, loss, logps, grads, ws, ws_bytes,
                  static_cast<hipStream_t>(stream));
    });
}

}  // extern "C"

extern "C" int qlx_adamw_lora(const qlx_dims* d, const qlx_lora_buf* params, const qlx_lora_grad* grads,
                              const qlx_lora_buf* m, const qlx_lora_buf* v, int64_t t, const qlx_adamw_cfg* cfg,
                              void* stream) {
    return guarded([&] {
        validate_dims(d);
        REQ_PTR(params, "params");
        REQ_PTR(grads, "grads");
        REQ_PTR(m, "m");
        REQ_PTR(v, "v");
        check_adamw_cfg(cfg, t);
        const int L = d->n_layers, r = d->lora_r;
        for (int l = 0; l < L; ++l) {
            validate_grads(&grads[l]);
            for (int p = 0; p < 7; ++p)
                QLX_REQUIRE(params[l].A[p] && params[l].B[p] && m[l].A[p] && m[l].B[p] && v[l].A[p] && v[l].B[p],
                            QLX_EINVAL, "adamw: every params/m/v A[p], B[p] must be set");
        }
        const LayerGeom g = make_geom(*d, 1, 1);
        const AdamScalars c = adam_scalars(*cfg, t);
        const hipStream_t s = static_cast<hipStream_t>(stream);
        for (int l = 0; l < L; ++l) adamw_layer(g, r, params[l], grads[l], m[l], v[l], c, s);
    });
}

extern "C" size_t qlx_merge_workspace_bytes(int64_t rows, int64_t cols, int out_kind) {
    if (rows < 0 || cols < 0 || (out_kind != QLX_MERGE_BF16 && out_kind != QLX_MERGE_NF4)) return 0;
    return out_kind == QLX_MERGE_NF4 ? size_t(rows) * size_t(cols) * 2 : 0;
}

extern "C" int qlx_lora_merge(qlx_nf4 W, const float* A, const float* B, int r, float scale, int out_kind, void* out,
                              float* out_absmax, void* ws, size_t ws_bytes, void* stream) {
    return guarded([&] {
        QLX_REQUIRE(W.rows >= 0 && W.cols >= 0, QLX_EINVAL, "merge: negative size");
        QLX_REQUIRE(out_kind == QLX_MERGE_BF16 || out_kind == QLX_MERGE_NF4, QLX_EINVAL, "merge: out_kind");
        QLX_REQUIRE(r >= 1, QLX_EINVAL, "merge: r must be >= 1");
        QLX_REQUIRE(std::isfinite(scale), QLX_EINVAL, "merge: scale must be finite");
        const int64_t n = W.rows * W.cols;
        if (n == 0) return;
        REQ_PTR(W.packed, "W.packed");
        REQ_PTR(W.absmax, "W.absmax");
        REQ_PTR(A, "A");
        REQ_PTR(B, "B");
        REQ_PTR(out, "out");
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (out_kind == QLX_MERGE_BF16) {
            launch_lora_merge(W.packed, W.absmax, W.rows, W.cols, A, B, r, scale, static_cast<uint16_t*>(out), s);
            return;
        }
        REQ_PTR(out_absmax, "out_absmax");
        check_ws(ws, ws_bytes, qlx_merge_workspace_bytes(W.rows, W.cols, out_kind));
        uint16_t* merged = static_cast<uint16_t*>(ws);
        launch_lora_merge(W.packed, W.absmax, W.rows, W.cols, A, B, r, scale, merged, s);
        launch_nf4_quantize(merged, n, static_cast<uint8_t*>(out), out_absmax, s);
    });
}

