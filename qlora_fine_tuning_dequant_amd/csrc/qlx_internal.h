// Internal interfaces of libqlx (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <exception>
#include <string>

#include "qlx.h"

namespace qlx {

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
struct Error {
    int code;
    std::string msg;
};
#define QLX_CHECK_HIP(expr)                                                          \
    do {                                                                             \
        hipError_t e_ = (expr);                                                      \
        if (e_ != hipSuccess)                                                        \
            throw ::qlx::Error{QLX_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)}; \
    } while (0)
#define QLX_REQUIRE(cond, code, msg)                                                 \
    do {                                                                             \
        if (!(cond)) throw ::qlx::Error{(code), (msg)};                              \
    } while (0)
void check_launch(const char* what);
#define REQ_PTR(p, name) QLX_REQUIRE((p) != nullptr, QLX_EINVAL, std::string(name) + " is NULL")

// Runs f and turns what it throws into a status (the ABI's error contract).
template <typename F>
inline int guarded(F&& f) {
    try {
        f();
        return QLX_OK;
    } catch (const Error& e) {
        set_error(e.msg);
        return e.code;
    } catch (const std::exception& e) {
        set_error(std::string("internal error: ") + e.what());
        return QLX_EHIP;
    } catch (...) {
        set_error("internal error");
        return QLX_EHIP;
    }
}

// Brackets one kernel launch with timing events when profiling is on.
struct ProfScope {
    // ext: the launcher records the pair itself through hipExtLaunchKernel
    // (start() / stop(), null when this launch is not profiled), which times
    // the kernel's own execution rather than the stream between two markers
    ProfScope(const char* name, double flops, double bytes, hipStream_t s, bool ext = false);
    ~ProfScope();
    hipEvent_t start() const;
    hipEvent_t stop() const;
    hipStream_t s_;
    int64_t idx_ = -1;
    bool ext_ = false;
};

// ---------------------------------------------------------- workspace carving
// Hands out 256-byte aligned sub-buffers of a caller workspace. With a null
// base it only measures (every take() returns nullptr and bumps the size).
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t count) {
        off = (off + 255) & ~size_t(255);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
    size_t size() const { return (off + 255) & ~size_t(255); }
};

// ---------------------------------------------------------------- NF4
void launch_nf4_quantize(const uint16_t* w, int64_t n, uint8_t* packed, float* absmax, hipStream_t s);
void launch_lora_merge(const uint8_t* packed, const float* absmax, int64_t rows, int64_t cols, const float* A,
                       const float* B, int r, float scale, uint16_t* out, hipStream_t s);
void launch_nf4_dequant(const uint8_t* packed, const float* absmax, int64_t n, int out_dtype, void* out,
                        hipStream_t s);

// ---------------------------------------------------------------- GEMM
// C[M,N] = alpha * (A . op(B) [+ A2 . op(B2)]) [+ R] [+ C_old], fp32 accumulation.
// Element types: bf16 (TE_BF16) or fp16 (TE_F16) for A and dense B.
enum AKind { A_ROW = 0, A_TRANS = 1 };  // A_ROW: A[m*lda+k]; A_TRANS: A[k*lda+m]
enum BKind { B_NF4_NT = 0, B_NF4_NN = 1, B_DENSE_NT = 2, B_DENSE_NN = 3 };
// B_*_NT: stored [N][K] (element (n,k) at n*ldb+k, NF4: flat n*nf4_cols+k)
// B_*_NN: stored [K][N] (element (n,k) at k*ldb+n, NF4: flat k*nf4_cols+n)
enum TElem { TE_BF16 = 0, TE_F16 = 1 };
enum CType { C_F32 = 0, C_BF16 = 1, C_F16 = 2 };
enum Causal { CAUSAL_NONE = 0, CAUSAL_SKIP_UPPER = 1, CAUSAL_K_LE_M = 2, CAUSAL_K_GE_M = 3 };

struct GemmParams {
    int M = 0, N = 0, K = 0;
    const uint16_t* A = nullptr;
    int64_t lda = 0;
    const void* B = nullptr;  // dense: uint16 elements; NF4: packed bytes
    int64_t ldb = 0;
    const float* absmax = nullptr;  // NF4 only
    int64_t nf4_cols = 0;           // NF4: row length of the stored matrix
    // second K phase ("slab"): A2 [M, K2] row-major, B2 dense with the
    // orientation of B (NT for B_NF4_NT, NN for B_NF4_NN)
    int K2 = 0;
    const uint16_t* A2 = nullptr;
    int64_t lda2 = 0;
    const uint16_t* B2 = nullptr;
    int64_t ldb2 = 0;
    // batching over grid.z: z -> (bo = z / zdiv, bi = z % zdiv)
    int batch = 1, zdiv = 1, a_grp = 1, b_grp = 1;
    int64_t a_so = 0, a_si = 0, b_so = 0, b_si = 0, c_so = 0, c_si = 0;
    // split-K (chosen by the launcher from the shapes and the room for
    // partials: at most partial_cap floats at partial_ws)
    int splits = 1, kchunk = 0;
    float* partial = nullptr;
    size_t partial_cap = size_t(1024) * 128 * 128;
    // epilogue
    void* C = nullptr;
    int64_t ldc = 0;
    int c_type = C_F32;
    float alpha = 1.f;
    const float* R = nullptr;  // residual added after alpha (fp32, ldr), no batching
    int64_t ldr = 0;
    int accumulate = 0;        // C (fp32) += result
    int seg_rows = 0;          // >0: row m goes to Cseg[m / seg_rows] row m % seg_rows (M <= 8 seg_rows)
    void* Cseg[8] = {};
    // dense NN B with seg_rows > 0: the M-tiles of segment i read B from
    // element offset bseg[i] (a multiple of 4; seg_rows a multiple of 128 when
    // any offset is non-zero, so no tile straddles two segments)
    int64_t bseg[8] = {};
    int causal = CAUSAL_NONE;
    // 1: when the launcher splits K, it leaves the fp32 partials for the
    // caller's next kernel to sum (no reduce pass, C not written); gemm()
    // returns the split count either way
    int defer_reduce = 0;
    int slab_alg_k = -1;  // algorithmic K of the slab for flop accounting (-1: K2)
    // LM-head cross-entropy statistics epilogue (fp16 NT products on 64-wide
    // wavefront tiles, no split; ce_mode 1): per row and per 64 columns, the
    // max and the sum of exp(z - max) (ce_pm, ce_ps, row stride ce_pld), the
    // target's logit (ce_picked) and, when ce_logits is non-null, the fp32
    // logits z (row stride ce_ldl). C is not written. Column j is vocab index
    // j; the target of row t is ce_tokens[t + 1] when t % ce_seq lies in
    // [ce_start, ce_seq - 1).
    int ce_mode = 0;
    const int32_t* ce_tokens = nullptr;
    int ce_seq = 0, ce_start = 0, ce_pld = 0;
    float *ce_pm = nullptr, *ce_ps = nullptr, *ce_picked = nullptr;
    float* ce_logits = nullptr;
    int64_t ce_ldl = 0;
    // set by the launcher
    int a_vec = 0, b_vec = 0, a2_vec = 0, b2_vec = 0;
    const char* tag = nullptr;  // profiling label (host side only; default: the operand kinds)
};

// Floats of split-K scratch the launcher may use for any one GEMM.
constexpr size_t kGemmPartialFloats = size_t(1024) * 128 * 128;
// Returns the number of K splits it ran (1: C written).
int gemm(GemmParams p, int akind, int bkind, int te, float* partial_ws, hipStream_t s);

// Split-K partial sums left for a consumer kernel (GemmParams::defer_reduce):
// element (row, col) of an [M, N] product is alpha * (p[0][i] + p[1][i] + ...
// in split order) [+ R[row * ldr + col]], i = row * N + col, split s at p + s * mn.
struct Partials {
    const float* p = nullptr;
    int splits = 0;
    int64_t mn = 0;
    float alpha = 1.f;
    const float* R = nullptr;
    int64_t ldr = 0;
};

// Independent products C_i[M_i, N_i] (fp32) = alpha_i * A_i^T . B_i over one
// shared K, in one launch without a split: A_i [K][lda_i] and B_i [K][ldb_i]
// 16-bit (the element type te), each problem's columns read from its own
// pointers. tile0 is set by the launcher.
struct GemmProb {
    const uint16_t* A = nullptr;
    const uint16_t* B = nullptr;
    float* C = nullptr;
    int64_t lda = 0, ldb = 0, ldc = 0;
    int M = 0, N = 0;
    float alpha = 1.f;
    int tile0 = 0;
};
constexpr int kGemmGroupMax = 16;
struct GemmGroup {
    int n = 0;
    GemmProb prob[kGemmGroupMax];
};
void gemm_group_tn(GemmGroup g, int K, int te, const char* tag, hipStream_t s);

// ---------------------------------------------------------------- AdamW
struct AdamTensor {
    float* p;
    const float* g;
    float* m;
    float* v;
    int64_t n;
};
// per-step constants, computed on the host in double
struct AdamScalars {
    float decay;         // 1 - lr * weight_decay
    float b1, one_m_b1;  // beta1, 1 - beta1
    float b2, one_m_b2;  // beta2, 1 - beta2
    float step_size;     // lr / (1 - beta1^t)
    float inv_bc2_sqrt;  // 1 / sqrt(1 - beta2^t)
    float eps;
};
constexpr int kAdamMaxTensors = 14;
void launch_adamw(const AdamTensor* ts, int n, const AdamScalars& c, hipStream_t s);

// ---------------------------------------------------------------- elementwise
void launch_rmsnorm_fwd(const float* x, const float* g, int T, int H, float eps, void* out, int out_f16,
                        float* rstd, hipStream_t s);
// out16 (optional): also writes the 16-bit activation type (f16) of dx * sc
void launch_rmsnorm_bwd(const float* dy, const float* x, const float* g, const float* rstd, const float* dres,
                        int T, int H, float* dx, hipStream_t s, uint16_t* out16 = nullptr, float sc = 1.f,
                        int f16 = 0);
// The same two with the input (forward: x, also written to xout in fp32;
// backward: dy) summed from split-K partials of an [T, H] product. Only where
// rmsnorm_part_ok(H) holds (the launchers check it).
bool rmsnorm_part_ok(int H);
void launch_rmsnorm_fwd_part(const Partials& x, float* xout, const float* g, int T, int H, float eps, void* out,
                             int out_f16, float* rstd, hipStream_t s);
void launch_rmsnorm_bwd_part(const Partials& dy, const float* x, const float* g, const float* rstd, const float* dres,
                             int T, int H, float* dx, hipStream_t s, uint16_t* out16 = nullptr, float sc = 1.f,
                             int f16 = 0);
void launch_rope_table(int seq, int hd, float theta, float* cs, hipStream_t s);
// Rotates pairs (j, j + hd/2) of nheads heads in columns [col0, col0 + nheads*hd)
// of a bf16 [T, ld] buffer in place; row t has position t % seq.
// 16-bit activations below are bf16, or fp16 when f16 != 0.
void launch_rope(uint16_t* buf, int64_t ld, int T, int seq, int col0, int nheads, int hd, const float* cs, int f16,
                 hipStream_t s);
// Sums split-K partials of an [T, nall * hd] product into the 16-bit buf
// (row stride nall * hd), rotating heads [0, nrot) as launch_rope does and
// copying the rest. Only where rope_part_ok(hd, nall) holds.
bool rope_part_ok(int hd, int nall);
void launch_rope_part(const Partials& src, uint16_t* buf, int T, int seq, int nrot, int nall, int hd, const float* cs,
                      int f16, hipStream_t s);
void launch_swiglu_fwd(const uint16_t* gu, int T, int I, uint16_t* act, int f16, hipStream_t s);
void launch_swiglu_bwd(const uint16_t* dact, const uint16_t* gu, int T, int I, uint16_t* dgu, int f16, hipStream_t s);
void launch_embed(const int32_t* tok, const uint16_t* E, int T, int H, int V, float* h, hipStream_t s);
// y = 16-bit(x * scale)
void launch_f32_to_act(const float* x, int64_t n, uint16_t* y, int f16, float scale, hipStream_t s);
void launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
// Layer blob wire form -> full form on the device: m32[i] = m16[i] << 16 for
// the nb block maxima; g1d/g2d = g1s/g2s (H floats each).
void launch_blob_widen(const uint16_t* m16, int64_t nb, const float* g1s, const float* g2s, int H, uint32_t* m32,
                       float* g1d, float* g2d, hipStream_t s);

// Flash-style causal GQA attention over q|k|v packed per token row.
struct AttnArgs {
    const uint16_t* qkv = nullptr;  // [B*S, ld]: q at column 0, k at qdim, v at qdim + kvdim (bf16)
    int64_t ld = 0;
    int B = 0, S = 0, nH = 0, nKV = 0, hd = 0;
    int64_t qdim = 0, kvdim = 0;
    float scale = 1.f;
    uint16_t* o = nullptr;  // [B*S, ldo] attention output (forward)
    int64_t ldo = 0;        // also the row stride of dO and O (backward)
    float* lse = nullptr;   // [B, nH, S] natural log-sum-exp of the scaled scores
    const uint16_t* dO = nullptr;
    const uint16_t* O = nullptr;
    float* Dq = nullptr;                      // [B, nH, S] sum_d dO o
    float *dKh = nullptr, *dVh = nullptr;     // [B, nH, S, hd] fp32 per query head
    uint16_t* dqkv = nullptr;                 // dq written at column 0 (bf16)
    int64_t lddq = 0;
    const float2* rope = nullptr;             // [S, hd/2] (cos, sin): dq rotated back before its store
    int f16 = 0;                              // 16-bit operands: 0 bf16, 1 fp16
    // backward: when dO_part.p is set, dO is first formed from these split-K
    // partials of [B*S, qdim] (rounded to 16 bits, written to dO_out, row
    // stride ldo) by the kernel that computes Dq
    Partials dO_part;
    uint16_t* dO_out = nullptr;
};
void launch_flash_fwd(const AttnArgs& a, hipStream_t s);
void launch_flash_bwd(const AttnArgs& a, hipStream_t s);
void launch_spin(int delay_us, hipStream_t s);
struct LoraSeg {
    const float* A;  // [r, in]
    const float* B;  // [out_p, r]
    int out_p;
};
void launch_lora_pack(const LoraSeg* segs, int nseg, int r, int in_f, float scale, uint16_t* Acat,
                      uint16_t* Bbd, int f16, hipStream_t s);
// Several packs in one launch (one per grid row).
struct LoraPackJob {
    const LoraSeg* segs;
    int nseg, in_f;
    uint16_t *Acat, *Bbd;
};
void launch_lora_pack_jobs(const LoraPackJob* jobs, int njobs, int r, float scale, int f16, hipStream_t s);
// rope non-null: each (j, j + hd/2) pair of the sums is rotated back (RoPE
// transpose, table [S, hd/2]) before the bf16 store.
void launch_gqa_reduce(const float* dh, int B, int nH, int nKV, int S, int hd, uint16_t* out, int64_t ldo,
                       int col0, const float* rope, int f16, hipStream_t s);
// Cross-entropy pieces over logits [T, V] (fp32).
// target[t] < 0 marks a row with no loss. lse[t], picked[t] = z[t, target].
void launch_ce_reduce(const float* pm, const float* ps, int nb, int T, int V, const int32_t* tokens, int seq, int start,
                      float* lse, float* picked, hipStream_t s);
// fp16 dz = (softmax - onehot) * sc (* gseq[t / seq]) of vocabulary columns
// col0 .. col0 + cw - 1 from fp32 logits z [T, ldz] into dz [T, lddz].
void launch_ce_dz(const float* z, int64_t ldz, int T, int cw, int col0, const int32_t* tokens, int seq, int start,
                  const float* lse, float sc, const float* gseq, uint16_t* dz, int64_t lddz, hipStream_t s);
void launch_sft_loss(const float* lse, const float* picked, int T, int seq, float* loss, hipStream_t s);
enum PrefKind { PREF_DPO = 0, PREF_ORPO = 1, PREF_SIMPO = 2, PREF_KTO = 3 };
struct PrefLossArgs {
    const float *lse_p, *pk_p;            // policy CE stats [2P*seq]
    const float *lse_r, *pk_r;            // reference (DPO, KTO), else null
    const float *kl_lse_p, *kl_pk_p;      // KTO mismatched pairs, policy, else null
    const float *kl_lse_r, *kl_pk_r;      // KTO mismatched pairs, reference, else null
    int pairs, seq, nresp, kind;
    float beta, gamma, lambda_d, lambda_u;
    float* loss;
    float* logps;  // [4P]
    float* gseq;   // [2P]
};
void launch_pref_loss(const PrefLossArgs& a, hipStream_t s);
void launch_kl_tokens(const int32_t* toks, int B, int seq, int prompt_len, int32_t* out, hipStream_t s);

}  // namespace qlx
