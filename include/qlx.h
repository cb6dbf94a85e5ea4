/*
 * qlx.h — C ABI of libqlx: the hot path of layer-streamed QLoRA fine-tuning
 * (a frozen NF4-quantized Llama-style decoder stack with trainable LoRA
 * adapters; the base weights stay in pinned host RAM and reach the GPU one
 * decoder layer at a time) on AMD Instinct MI355X (gfx950).
 *
 * What the method is (cited by page title and section):
 *  - rug.gal, "Soup: fine-tune an 8B model on a 4 GB laptop GPU (layer
 *    streaming)", intro and "En detalle": the frozen base is kept off the GPU
 *    and fed to it one decoder layer at a time (load, compute, unload); only the
 *    LoRA adapters and the batch stay resident; the result is bit-exact with a
 *    non-streamed run; DPO's reference model is the same layer stream with the
 *    adapters switched off.
 *  - guillermodelpino.com, "Soup: afinar un modelo de 8.000 millones de
 *    parámetros en un portátil con 4 GB de gráfica", "Qué es exactamente"
 *    (LoRA r 64, alpha 16, quantization 4bit) and "El streaming de capas".
 *  - imasters.com.br, "Soup promete fine-tuning de modelo 8B em GPU de notebook
 *    com 4 GB", "Como cabe um 8B em 4 GB" (NF4; base in host RAM) and "Do SFT
 *    para os métodos de preferência" (DPO reference with adapters off).
 *  - NF4 as defined by QLoRA (Dettmers et al., 2023); LoRA (Hu et al., 2021);
 *    the Llama decoder (RMSNorm, rotate-half RoPE, grouped-query causal
 *    attention, SwiGLU); DPO (Rafailov et al., 2023, eq. 7).
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless marked HOST. bf16 and fp16 values
 *    travel as uint16_t bit patterns. Matrices are row-major.
 *  - The caller owns every buffer. No call allocates device memory; scratch
 *    space comes from a caller-provided workspace whose size the matching
 *    qlx_*_workspace_bytes() call reports. Pass ws = NULL with ws_bytes = 0
 *    only when that size is 0.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls are
 *    asynchronous on it: outputs are valid once the stream reaches that
 *    point. Streaming steps fork to the context's side stream and join back
 *    with events before returning.
 *  - Return value: qlx_status. Arguments are validated on the host before
 *    any launch; on a non-OK return nothing was launched (except QLX_EHIP,
 *    which reports a launch or runtime failure). qlx_last_error() gives a
 *    thread-local message. No exception crosses the ABI.
 *  - Results are deterministic: no floating-point atomics anywhere, fixed
 *    reduction orders, and kernel choice depends only on shapes (never on
 *    pointer values), so the same inputs give the same bits whether the
 *    layer bytes sit in a streaming slot or stay resident.
 */
#ifndef QLX_H
#define QLX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QLX_OK = 0,
    QLX_EINVAL = 1,        /* null pointer, negative size, inconsistent shapes */
    QLX_EUNSUPPORTED = 2,  /* valid request the library does not handle */
    QLX_EWORKSPACE = 3,    /* ws_bytes smaller than the reported requirement */
    QLX_ENOTPINNED = 4,    /* a streamed layer blob is not pinned host memory */
    QLX_EHIP = 5,          /* the HIP runtime reported an error */
    QLX_EIO = 6            /* a layer file could not be created, opened or read */
} qlx_status;

enum { QLX_F32 = 0, QLX_BF16 = 1 };                /* nf4_dequant output type */
/* where layer blobs live: pinned host RAM, device memory, or a layer file
 * attached to the context (qlx_ctx_set_layer_source) */
enum { QLX_STREAMED = 0, QLX_RESIDENT = 1, QLX_STREAMED_DISK = 2 };
enum { QLX_DPO_REF_FUSED = 0, QLX_DPO_REF_SEPARATE = 1 };

/* Thread-local text of the last non-OK status (never NULL). */
const char* qlx_last_error(void);
/* Library version string. */
const char* qlx_version(void);

/* Decoder dimensions. rms_eps 1e-5 and rope_theta 5e5 for the Llama-3.1
 * shape; lora_alpha / lora_r is the LoRA scale s.
 * act_dtype: the 16-bit type of the activations and gradients the layer and
 * step calls keep between kernels and feed to the MFMA products.
 *   QLX_ACT_BF16 (0): bf16 activations, bf16 weight operand (QLoRA's
 *     computation type; the frozen weight enters as bf16 of its NF4 value).
 *   QLX_ACT_F16 (1): fp16 activations and gradients; the weight operand is
 *     still bf16 of the NF4 value, carried in fp16 (exact for magnitudes in
 *     [2^-17, 65504]), so only the activation side changes: 10 significand
 *     bits instead of 7 at the same MFMA rate. Gradients travel scaled by a
 *     power of two (chosen per step from the loss's largest per-position
 *     logit gradient) and come out unscaled.
 * fp32 everywhere else (residual stream, reductions, LoRA gradients). */
enum { QLX_ACT_BF16 = 0, QLX_ACT_F16 = 1 };
typedef struct {
    int32_t hidden, n_heads, n_kv_heads, head_dim, inter, vocab, n_layers, lora_r;
    float lora_alpha, rms_eps, rope_theta;
    int32_t act_dtype;
} qlx_dims;

/* ---------------------------------------------------------------------------
 * NF4 (QLoRA's 4-bit NormalFloat), blocksize 64, fp32 absmax.
 * Source: rug.gal article "En detalle" and imasters article "Como cabe um 8B
 * em 4 GB" name NF4; the values and rounding follow QLoRA's NF4 definition.
 * Layout ("canonical NF4 tensor"): the tensor is flattened row-major; block b
 * covers elements [64b, 64b+64) (blocks may straddle rows); absmax[b] =
 * max |w| over the block (fp32); each element's code is the nearest of the 16
 * NF4 values to w / absmax[b] (fp32 division; an exact midpoint goes to the
 * lower code; an all-zero block has absmax 0 and codes 7); packed[j] holds
 * element 2j in its high nibble and 2j+1 in its low nibble (an odd count pads
 * the last low nibble with code 7).
 * ------------------------------------------------------------------------- */

/* Quantize w (bf16, n = rows*cols elements) into packed (ceil(n/2) bytes)
 * and absmax (ceil(n/64) floats). n = 0 is a no-op. */
int nf4_quantize(const uint16_t* w_bf16, int64_t rows, int64_t cols,
                 uint8_t* packed, float* absmax, void* stream);

/* out[i] = fl32(code_value[code_i] * absmax[i/64]) as fp32 (QLX_F32) or that
 * value rounded to nearest-even bf16 (QLX_BF16), for i < rows*cols. */
int nf4_dequant(const uint8_t* packed, const float* absmax, int64_t rows, int64_t cols,
                int out_dtype, void* out, void* stream);

/* A canonical NF4 matrix W [rows = out_features, cols = in_features]. */
typedef struct {
    const uint8_t* packed;
    const float* absmax;
    int64_t rows, cols;
} qlx_nf4;

/* ---------------------------------------------------------------------------
 * QLoRA linear (LoRA, Hu et al. 2021, section 4.1, on an NF4 base).
 *   y = x W'^T + s (x A^T) B^T,  W' = bf16(dequant(W)),  s = scale
 * x bf16 [T, in]; A fp32 [r, in]; B fp32 [out, r]; y bf16 [T, out].
 * A = B = NULL switches LoRA off (y = x W'^T exactly; B = 0 gives the same
 * bits). The base GEMM runs on bf16 MFMA with fp32 accumulation and the
 * dequantization fused into its weight-operand load.
 * ------------------------------------------------------------------------- */
size_t qlx_linear_workspace_bytes(int64_t T, int64_t in_f, int64_t out_f, int r);

int qlora_linear_fwd(const uint16_t* x, int64_t T, qlx_nf4 W, const float* A, const float* B,
                     int r, float scale, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* The same forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the adapter staging and the split-K partials live in a
 * static device array of QLX_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (its device address is looked up
 * once per device on the first call there). Calls no allocating routine.
 * Inputs as qlora_linear_fwd; with LoRA on, the staging (2 r (in + out) +
 * 4 T r bytes, rounded up to 256-byte pieces) must fit the scratch, else
 * QLX_EINVAL before any launch; what is left of the scratch bounds the
 * split-K partials (fewer splits, never a different result than the split
 * count the shapes choose within that room). Calls that overlap on one GPU
 * share the array and race: serialize them (one stream, or events). */
#define QLX_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int qlora_linear_fwd_noalloc(const uint16_t* x, int64_t T, qlx_nf4 W, const float* A, const float* B,
                             int r, float scale, uint16_t* y, void* stream);

/* Backward with W frozen. dy bf16 [T, out], x bf16 [T, in] (the forward input).
 *   du = s dy B;  dx = dy W' + du A (bf16 [T, in], NULL = skip);
 *   dB = s dy^T (x A^T) (fp32 [out, r]);  dA = du^T x (fp32 [r, in]).
 * accumulate = 1 adds into dA/dB instead of overwriting them. With LoRA off
 * (A = B = NULL) only dx is produced. T = 0 writes no dx and leaves dA/dB
 * zero (or unchanged with accumulate = 1); the forward with T = 0 is a no-op. */
int qlora_linear_bwd(const uint16_t* dy, const uint16_t* x, int64_t T, qlx_nf4 W,
                     const float* A, const float* B, int r, float scale,
                     uint16_t* dx, float* dA, float* dB, int accumulate,
                     void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Decoder layer blob: one contiguous region per layer holding
 *   packed q,k,v,o,gate,up,down (back to back, in that order)
 *   absmax q,k,v,o,gate,up,down (back to back, in that order)
 *   g_attn fp32 [hidden], g_mlp fp32 [hidden] (RMSNorm gains)
 * with each region 256-byte aligned. Projection shapes [out, in]:
 *   q [nH*hd, H], k/v [nKV*hd, H], o [H, nH*hd], gate/up [I, H], down [H, I].
 * Every projection must hold a multiple of 64 elements (true for all Llama
 * shapes), so q|k|v and gate|up are each one canonical NF4 matrix.
 * offsets[0..6] = packed q..down, [7..13] = absmax q..down, [14] = g_attn,
 * [15] = g_mlp; *total_bytes = blob size (a multiple of 256).
 * ------------------------------------------------------------------------- */
#define QLX_BLOB_NSEG 16
int qlx_layer_blob_layout(const qlx_dims* d, uint64_t offsets[QLX_BLOB_NSEG], uint64_t* total_bytes);

/* Wire form of a layer blob: what a streamed layer sends over the host link.
 * The NF4 scheme keeps one fp32 maximum per 64-element block (rug.gal
 * article, "En detalle"); for weights quantized from bf16 that maximum is
 * itself a bf16 value, so its low 16 bits are zero and the wire form keeps
 * only the upper 16. Layout: the packed regions at the full form's offsets
 * (offsets[0..6]), then all block maxima as bf16, q..down back to back
 * (offsets[7..13]), then g_attn and g_mlp fp32 (offsets[14], [15]), each
 * region 256-byte aligned; 4.25 instead of 4.5 bits per weight. After the
 * copy the library widens the maxima back to fp32 on the device, so the
 * kernels see the full form bit for bit. */
enum { QLX_BLOB_FULL = 0, QLX_BLOB_WIRE = 1 };
int qlx_layer_wire_layout(const qlx_dims* d, uint64_t offsets[QLX_BLOB_NSEG], uint64_t* total_bytes);
/* Converts a full-form blob to the wire form (both HOST, any alignment;
 * wire holds the wire layout's total_bytes). QLX_EINVAL, with wire left
 * untouched, if a block maximum has any of its low 16 bits set (weights that
 * were not bf16). */
int qlx_layer_blob_to_wire(const qlx_dims* d, const void* blob, void* wire);

/* LoRA adapters of one layer (fp32, device): A[p] [r, in_p], B[p] [out_p, r]
 * for p = q,k,v,o,gate,up,down. */
typedef struct { const float* A[7]; const float* B[7]; } qlx_lora;
typedef struct { float* dA[7]; float* dB[7]; } qlx_lora_grad;

/* One decoder layer (Llama: RMSNorm, q/k/v QLoRA, RoPE, causal GQA attention,
 * o QLoRA + residual, RMSNorm, SwiGLU QLoRA MLP + residual).
 * h_in / h_out: the fp32 residual stream [batch*seq, hidden] (row b*seq + t).
 * blob: DEVICE layer blob (layout above). lora = NULL runs the base only.
 * Positions restart at 0 for every sequence; attention is causal.
 * batch >= 1 and seq >= 1, else QLX_EINVAL. */
size_t qlx_layer_workspace_bytes(const qlx_dims* d, int batch, int seq);
int layer_fwd(const qlx_dims* d, const void* blob, const qlx_lora* lora, const float* h_in,
              int batch, int seq, float* h_out, void* ws, size_t ws_bytes, void* stream);

/* Backward of layer_fwd: recomputes the layer forward from h_in first, then
 * returns dh_in (fp32, NULL = skip the input gradient) and overwrites the 14
 * LoRA gradients in `grads` (fp32). lora must be non-NULL. */
int layer_bwd(const qlx_dims* d, const void* blob, const qlx_lora* lora, const float* h_in,
              const float* dh_out, int batch, int seq, float* dh_in, const qlx_lora_grad* grads,
              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Streaming context: owns a side stream (default priority, non-blocking),
 * the slot events and the step statistics. Nothing else.
 * ------------------------------------------------------------------------- */
typedef struct qlx_ctx qlx_ctx;

typedef struct {
    int64_t layer_reads;   /* layer blobs copied host -> device in the last step */
    int64_t h2d_bytes;     /* bytes those copies moved */
    int64_t layer_passes;  /* layer computations (fwd, recompute+bwd, reference) */
    float step_ms;         /* first to last event of the last step */
    float h2d_ms;          /* sum of the copies' durations (side stream) */
    int64_t disk_bytes;    /* bytes read from the layer file (QLX_STREAMED_DISK) */
    float disk_ms;         /* host wall time of those reads */
} qlx_stats;

int qlx_ctx_create(qlx_ctx** out, int device);
int qlx_ctx_destroy(qlx_ctx* ctx);
/* Waits for all work of the last step and fills *stats (HOST) if non-NULL. */
int qlx_ctx_sync(qlx_ctx* ctx, qlx_stats* stats);

/* Stream debugging (fault injection for the one race the streamer can have:
 * a copy overwriting a slot that a kernel still reads). None changes what a
 * step computes; every mode but QLX_DEBUG_POISON_LIVE must give the same bits
 * as a normal run.
 *   QLX_DEBUG_SERIALIZE: synchronize after every copy and every layer (no
 *     overlap at all).
 *   QLX_DEBUG_POISON: before a slot is refilled, fill it with 0xFF bytes (NaN
 *     absmax and norm gains), so a read after its release turns into NaN.
 *   QLX_DEBUG_DELAY_COPY / _DELAY_COMPUTE: a spin of about delay_us on the
 *     copy stream before each copy / on the compute stream before each layer,
 *     shifting the overlap either way.
 *   QLX_DEBUG_POISON_LIVE: control for the poison: fills each slot right after
 *     its copy, so the step must come out NaN.
 * The copies of one layer run in two halves on two side streams (two copy
 * engines); the environment variable QLX_COPY_SPLIT=1 at context creation
 * keeps them on one. */
enum {
    QLX_DEBUG_SERIALIZE = 1,
    QLX_DEBUG_POISON = 2,
    QLX_DEBUG_DELAY_COPY = 4,
    QLX_DEBUG_DELAY_COMPUTE = 8,
    QLX_DEBUG_POISON_LIVE = 16
};
int qlx_ctx_set_debug(qlx_ctx* ctx, int flags, int delay_us);

/* Keep-layers (on = 1, off = 0; off by default): at the end of a streamed
 * step the two slots hold layers 1 and 0, the first two layers the next
 * step's forward needs. With keep-layers on, the next step on this context
 * uses them without copying them again when its workspace slots are the same
 * memory, the layers' sources are the same (the same host blob pointers, or
 * the same attached layer file) and the blob form is the same: steady-state
 * layer reads per step fall by 2 and the first layer's compute starts at
 * once. The caller promises that neither the workspace nor those host blobs
 * (or the file) are written between the steps; resident-mode steps,
 * qlx_ctx_set_layer_source and qlx_ctx_set_keep_layers itself forget what
 * the slots held. Results are bit-identical to a step that copies every
 * layer. */
int qlx_ctx_set_keep_layers(qlx_ctx* ctx, int on);

/* Disk stream source (rug.gal article, "En detalle": the frozen base sits in
 * CPU memory or on disk; imasters article, "Como cabe um 8B em 4 GB": the
 * `stream_source: auto` setting, RAM when the stack fits and the NVMe disk
 * when it does not).
 * A layer file holds the n_layers blobs of a model, blob i at byte offset
 * i * stride, stride = the blob size (qlx_layer_blob_layout, or
 * qlx_layer_wire_layout for a file of wire-form blobs) rounded up to 4096,
 * zero padded. Reads use O_DIRECT (no page cache) unless the file
 * system refuses it or QLX_FILE_BUFFERED is given; reader threads (16, or
 * the environment variable QLX_FILE_READERS at open, 1..64) keep several
 * 8 MiB reads in flight. A file serves one context at a time. */
typedef struct qlx_layer_file qlx_layer_file;
enum {
    QLX_FILE_BUFFERED = 1, /* qlx_layer_file_open: read through the page cache */
    QLX_FILE_WIRE = 2      /* the file holds wire-form blobs (write and open) */
};

/* Writes the stack file: blobs = HOST array of n_layers HOST pointers (any
 * host memory) to blobs laid out as qlx_layer_blob_layout says, or as
 * qlx_layer_wire_layout says with flags = QLX_FILE_WIRE. Creates or
 * truncates path; fsyncs before returning. */
int qlx_layer_file_write(const char* path, const qlx_dims* d, const void* const* blobs, int flags);
/* Opens a stack file for the model dims d; QLX_EIO if it is missing or
 * shorter than n_layers * stride. flags: QLX_FILE_BUFFERED and/or
 * QLX_FILE_WIRE (as the file was written). */
int qlx_layer_file_open(qlx_layer_file** out, const char* path, const qlx_dims* d, int flags);
/* Waits for copies still reading its staging buffers, then frees it. NULL is
 * a no-op. QLX_EINVAL (and nothing freed) while a context still holds it:
 * detach it first (qlx_ctx_set_layer_source(ctx, NULL)) or destroy that
 * context. */
int qlx_layer_file_close(qlx_layer_file* f);
/* *direct (HOST) = 1 if reads bypass the page cache; *stride = blob stride. */
int qlx_layer_file_info(const qlx_layer_file* f, int* direct, uint64_t* stride);
/* Reads layer i's blob into dst (HOST, the size of one blob of the file's form, any
 * alignment). */
int qlx_layer_file_read(qlx_layer_file* f, int layer, void* dst);
/* Attaches f (NULL detaches) as the context's source for QLX_STREAMED_DISK.
 * The first attach allocates two pinned staging buffers of one stride each
 * on the context's device; a file stays bound to that device. */
int qlx_ctx_set_layer_source(qlx_ctx* ctx, qlx_layer_file* f);
/* `stream_source: auto`: *mode (HOST) = QLX_STREAMED if the stack
 * (stack_bytes) plus reserve_bytes fits in the host's available memory
 * (MemAvailable), else QLX_STREAMED_DISK. */
int qlx_stream_source_auto(uint64_t stack_bytes, uint64_t reserve_bytes, int* mode);

/* The model a step runs on.
 * layer_blobs: HOST array of n_layers pointers to layer blobs; in
 *   QLX_STREAMED mode they must be pinned host memory (hipHostMalloc or
 *   registered by the runtime's pinned allocator); in QLX_RESIDENT mode they
 *   are device memory and no copy happens; in QLX_STREAMED_DISK mode they are
 *   not read (may be NULL) and the layers come from the context's layer file,
 *   disk -> pinned staging -> device slot, with the same bits.
 * embed_f16, lm_head_f16: DEVICE fp16 [vocab, hidden] (untied, frozen).
 * final_norm: DEVICE fp32 [hidden]. lora: HOST array of n_layers qlx_lora.
 * blob_form: QLX_BLOB_FULL, or QLX_BLOB_WIRE for QLX_STREAMED host blobs in
 *   the wire form (QLX_STREAMED_DISK takes the form from the layer file). */
typedef struct {
    qlx_dims dims;
    const void* const* layer_blobs;
    const uint16_t* embed_f16;
    const uint16_t* lm_head_f16;
    const float* final_norm;
    const qlx_lora* lora;
    int blob_form;
} qlx_model;

/* Workspace of a step: two device slots of one full-form layer blob each
 * plus room for a wire-form tail (streamed modes), n_layers+1 fp32
 * layer-boundary checkpoints, one layer's workspace, the LM head's per-row
 * partials [T, vocab/64] (max and sum of exponentials, fp32), the fp32
 * logits [T, vocab] of the stream being trained (kept for the backward) and
 * one vocabulary chunk of fp16 logit gradients [T, 16384]. kind: 0 = SFT (batch = sequences),
 * 1 = DPO, ORPO or SimPO, 2 = KTO (batch = pairs; T = 2*pairs*seq; KTO adds
 * the mismatched pairs' tokens, two more fp32 hidden-state streams and
 * their CE statistics). */
size_t qlx_step_workspace_bytes(const qlx_dims* d, int kind, int batch, int seq);

/* One SFT step: embedding, n_layers decoder layers streamed one at a time
 * (double-buffered: the copy of layer i+1 overlaps compute on layer i; in
 * backward the layers are re-streamed in reverse and recomputed from the
 * layer-boundary checkpoints; the two layers still in the slots at the turn
 * are not copied again), final RMSNorm, fp16 LM head, next-token
 * cross-entropy averaged over batch*(seq-1) positions.
 * tokens: DEVICE int32 [batch, seq], batch >= 1, seq >= 2 (else QLX_EINVAL:
 * a next-token loss needs a second position). loss: DEVICE fp32 scalar.
 * grads: HOST array of n_layers qlx_lora_grad (device fp32 buffers, overwritten).
 * Streamed and resident modes give bit-identical loss and gradients. */
int stream_step_sft(qlx_ctx* ctx, const qlx_model* model, const int32_t* tokens, int batch,
                    int seq, int mode, float* loss, const qlx_lora_grad* grads,
                    void* ws, size_t ws_bytes, void* stream);

/* One DPO step (Rafailov et al. 2023, eq. 7; reference = the same layer
 * stream with LoRA off). chosen/rejected: DEVICE int32 [pairs, seq]; the
 * response of each sequence is positions prompt_len..seq-1 (1 <= prompt_len
 * < seq, 1 <= pairs <= 32, else QLX_EINVAL). The batch is
 * [chosen_1..chosen_P, rejected_1..rejected_P].
 * ref_schedule = QLX_DPO_REF_FUSED computes the reference forward on each
 *   layer while it is resident for the policy forward (layer reads as SFT);
 *   QLX_DPO_REF_SEPARATE runs a separate reference pass first (3L-2 reads).
 *   Both give identical bits.
 * loss: DEVICE fp32 scalar = mean over pairs of -log sigmoid(beta*Delta).
 * logps: DEVICE fp32 [4*pairs] = policy chosen, policy rejected, reference
 *   chosen, reference rejected (summed response-token log-probs). */
int stream_step_dpo(qlx_ctx* ctx, const qlx_model* model, const int32_t* chosen,
                    const int32_t* rejected, int pairs, int seq, int prompt_len, float beta,
                    int mode, int ref_schedule, float* loss, float* logps,
                    const qlx_lora_grad* grads, void* ws, size_t ws_bytes, void* stream);

/* The preference objectives the pages list on the same layer stream (rug.gal
 * article, intro and "En detalle"; imasters article, "Do SFT para os métodos
 * de preferência"): DPO, ORPO, SimPO and KTO, KTO with DPO's reference scheme
 * (adapters off). Each loss is the published one, a function of per-sequence
 * summed response log-probs s over n = seq - prompt_len tokens (l = s/n):
 *   QLX_PREF_DPO   (Rafailov et al. 2023, eq. 7): as stream_step_dpo; beta.
 *   QLX_PREF_ORPO  (Hong et al. 2024, eqs. 2-7): mean over pairs of
 *     -l_c + beta * -log sigmoid(log odds_c - log odds_r),
 *     log odds = l - log(1 - e^l); beta is ORPO's lambda (0.1). No reference.
 *   QLX_PREF_SIMPO (Meng et al. 2024, eq. 6): mean over pairs of
 *     -log sigmoid(beta (l_c - l_r) - gamma) (2.0, 0.5). No reference.
 *   QLX_PREF_KTO   (Ethayarajh et al. 2024, eq. 8): chosen desirable,
 *     rejected undesirable; r = s_pol - s_ref; z0 = max(0, mean over the
 *     mismatched pairs (prompt j + completion (j+1) mod 2P) of s_pol - s_ref),
 *     no gradient through z0; mean over examples of lambda_y - v with
 *     v = lambda_d sigmoid(beta (r - z0)) or lambda_u sigmoid(beta (z0 - r))
 *     (beta 0.1, lambdas 1).
 * ref_schedule applies to DPO and KTO (QLX_DPO_REF_FUSED / _SEPARATE); the
 * reference-free kinds read the stack as SFT does. logps as in
 * stream_step_dpo (reference entries 0 for ORPO and SimPO). Workspace kind
 * (qlx_step_workspace_bytes): 2 for KTO, 1 otherwise. Streamed and resident
 * modes give identical bits. */
enum { QLX_PREF_DPO = 0, QLX_PREF_ORPO = 1, QLX_PREF_SIMPO = 2, QLX_PREF_KTO = 3 };
typedef struct {
    int kind;
    int ref_schedule;
    float beta;
    float gamma;
    float lambda_d, lambda_u;
} qlx_pref_cfg;

int stream_step_pref(qlx_ctx* ctx, const qlx_model* model, const qlx_pref_cfg* cfg,
                     const int32_t* chosen, const int32_t* rejected, int pairs, int seq,
                     int prompt_len, int mode, float* loss, float* logps,
                     const qlx_lora_grad* grads, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Adapter merge (the pages' `soup merge`: guillermodelpino.com article,
 * command list; imasters article, closing section): fold one trained LoRA
 * adapter into its NF4 base matrix,
 *   W_merged = W' + scale * B A,  W' = fl32(c[code] * absmax),
 * summed in fp32 (B A accumulated over r in ascending order) and rounded once
 * to bf16 (RNE).
 * W: the NF4 matrix [rows, cols] (canonical layout; a projection inside a
 *   stacked q|k|v or gate|up matrix is addressed by offsetting packed by
 *   row0*cols/2 bytes and absmax by row0*cols/64 entries). A: DEVICE fp32
 *   [r, cols]; B: DEVICE fp32 [rows, r].
 * out_kind QLX_MERGE_BF16: out = DEVICE bf16 [rows, cols], out_absmax unused.
 * out_kind QLX_MERGE_NF4:  out = DEVICE packed NF4 [rows*cols/2], out_absmax
 *   = DEVICE fp32 [rows*cols/64]: the bf16 merged matrix re-quantized by
 *   nf4_quantize's rules (needs qlx_merge_workspace_bytes of workspace).
 * r >= 1; QLX_EINVAL on bad arguments (nothing runs).
 * ------------------------------------------------------------------------- */
enum { QLX_MERGE_BF16 = 0, QLX_MERGE_NF4 = 1 };
size_t qlx_merge_workspace_bytes(int64_t rows, int64_t cols, int out_kind);
int qlx_lora_merge(qlx_nf4 W, const float* A, const float* B, int r, float scale, int out_kind,
                   void* out, float* out_absmax, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Optimizer update of the training step: AdamW on every LoRA factor.
 * The pages set the learning rate (2e-5, training section of the example
 * configuration: guillermodelpino.com article, "Qué es Soup") and name no
 * optimizer; the reading is AdamW with decoupled weight decay (Loshchilov &
 * Hutter, "Decoupled Weight Decay Regularization", Algorithm 2), the decay
 * scaled by lr as in PyTorch's AdamW, bias-corrected moments:
 *   theta <- theta (1 - lr wd); m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
 *   theta <- theta - lr/(1 - b1^t) * m / (sqrt(v)/sqrt(1 - b2^t) + eps).
 * params, m, v: arrays of dims->n_layers qlx_lora_buf, each pointer a DEVICE
 *   fp32 tensor laid out like the LoRA factor (A[p] [r, in_p], B[p] [out_p, r]),
 *   updated in place (params are the same memory the model's qlx_lora
 *   points to). m and v start at zero.
 * grads: dims->n_layers qlx_lora_grad from the step.
 * t: 1-based count of updates so far including this one (t >= 1).
 * cfg: lr >= 0, 0 <= beta1, beta2 < 1, eps > 0, weight_decay >= 0.
 * Tensors whose length is a multiple of 4 must be 16-byte aligned. One
 * launch per layer on `stream`; QLX_EINVAL on bad arguments (nothing runs).
 * ------------------------------------------------------------------------- */
/* double so that 1 - beta is formed before any rounding (1 - fp32(0.999) is
 * off by 1.3e-5); the kernel computes in fp32 */
typedef struct { double lr, beta1, beta2, eps, weight_decay; } qlx_adamw_cfg;
typedef struct { float* A[7]; float* B[7]; } qlx_lora_buf;

int qlx_adamw_lora(const qlx_dims* dims, const qlx_lora_buf* params, const qlx_lora_grad* grads,
                   const qlx_lora_buf* m, const qlx_lora_buf* v, int64_t t, const qlx_adamw_cfg* cfg,
                   void* stream);

/* Fused AdamW (off by default). Registers AdamW on a context: every later
 * step on it (SFT or preference) updates layer i's adapters right after
 * layer i's backward, on the step's stream, where it overlaps the copies and
 * compute of the layers still to come (nothing later in the step reads
 * them). The result is bit-identical to qlx_adamw_lora with the same t after
 * the step. params, m, v: HOST arrays of n_layers qlx_lora_buf (device fp32
 * buffers, copied as pointers; the buffers must stay valid while
 * registered); params must be the adapters of the model each step runs on,
 * or the step fails with QLX_EINVAL before any launch. t_next: the update
 * count of the next step (>= 1); each step call that returns QLX_OK adds 1.
 * params = NULL switches it off. */
int qlx_ctx_set_adamw(qlx_ctx* ctx, int n_layers, const qlx_lora_buf* params, const qlx_lora_buf* m,
                      const qlx_lora_buf* v, const qlx_adamw_cfg* cfg, int64_t t_next);
/* *t_next (HOST) = the update count the next step will use; 0 when off. */
int qlx_ctx_adamw_t(const qlx_ctx* ctx, int64_t* t_next);

/* ---------------------------------------------------------------------------
 * Per-kernel timing (observability). Between qlx_profile_begin() and
 * qlx_profile_end() every kernel the library launches is bracketed by a pair
 * of HIP events on its own stream; qlx_profile_end() waits for them and
 * returns one row per kernel: launches, summed event time, and the summed
 * algorithmic flops and HBM bytes of those launches (operands read once,
 * outputs written once). Process-wide; not for concurrent use from several
 * threads. `out` may be NULL to only count rows.
 * ------------------------------------------------------------------------- */
typedef struct {
    char name[48];
    int64_t launches;
    double ms;
    double flops;
    double bytes;
} qlx_kernel_prof;

int qlx_profile_begin(void);
/* As qlx_profile_begin(), but only kernels whose row name starts with
 * `name_prefix` are bracketed (the others run with no events at all), so a
 * timed loop can measure one kernel family at almost no cost to the rest.
 * NULL or "" selects every kernel. The prefix is copied. */
int qlx_profile_begin_prefix(const char* name_prefix);
int qlx_profile_end(qlx_kernel_prof* out, int max_out, int* count);

/* Measured peaks of the device, for roofline figures (not part of a step).
 * qlx_peak_mfma: `workgroups` workgroups of 4 wavefronts, each wavefront
 *   running `iters` x (shape 0) 8 independent v_mfma_f32_16x16x32_bf16 or
 *   (shape 1) 4 independent v_mfma_f32_32x32x16_bf16 on register operands:
 *   131072 x iters flops per wavefront either way. out: DEVICE fp32
 *   [workgroups * 256], written to keep the loop alive.
 * qlx_peak_copy: a 16-byte grid-stride copy of `bytes` (multiple of 16,
 *   both buffers DEVICE and 16-byte aligned): bytes read + bytes written. */
int qlx_peak_mfma(int64_t iters, int workgroups, int shape, float* out, void* stream);
int qlx_peak_copy(const void* src, void* dst, uint64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QLX_H */
