"""ctypes binding of libqlx (include/qlx.h). Argument marshalling only: every
step of the path runs in the library's HIP kernels. torch supplies device and
pinned host memory and the current HIP stream; it does no math here.

The functions keep the C names: nf4_quantize, nf4_dequant, qlora_linear_fwd,
qlora_linear_bwd, layer_fwd, layer_bwd, stream_step_sft, stream_step_dpo.
A missing or unloadable library raises immediately; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Sequence

import torch

# QLX_LIB names another build of the same library (the host-sanitizer builds
# the CPU tests run under); by default the in-tree libqlx.so
LIB_PATH = os.environ.get("QLX_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlx.so")

QLX_OK, QLX_EINVAL, QLX_EUNSUPPORTED, QLX_EWORKSPACE, QLX_ENOTPINNED, QLX_EHIP, QLX_EIO = range(7)
QLX_F32, QLX_BF16 = 0, 1
QLX_STREAMED, QLX_RESIDENT, QLX_STREAMED_DISK = 0, 1, 2
QLX_FILE_BUFFERED, QLX_FILE_WIRE = 1, 2
QLX_BLOB_FULL, QLX_BLOB_WIRE = 0, 1
QLX_DEBUG_SERIALIZE, QLX_DEBUG_POISON, QLX_DEBUG_DELAY_COPY, QLX_DEBUG_DELAY_COMPUTE, QLX_DEBUG_POISON_LIVE = (
    1, 2, 4, 8, 16)
QLX_DPO_REF_FUSED, QLX_DPO_REF_SEPARATE = 0, 1
QLX_PREF_DPO, QLX_PREF_ORPO, QLX_PREF_SIMPO, QLX_PREF_KTO = 0, 1, 2, 3
QLX_MERGE_BF16, QLX_MERGE_NF4 = 0, 1
QLX_ACT_BF16, QLX_ACT_F16 = 0, 1
# 16-bit activation type of layer and step calls when the caller names none:
# fp16 (10 significand bits, the same MFMA rate as bf16; the weight operand
# is bf16 of its NF4 value either way). QLX_ACT=bf16 in the environment
# switches the default.
ACT_DEFAULT = QLX_ACT_BF16 if os.environ.get("QLX_ACT", "").lower() == "bf16" else QLX_ACT_F16
PREF_KINDS = {"dpo": QLX_PREF_DPO, "orpo": QLX_PREF_ORPO, "simpo": QLX_PREF_SIMPO, "kto": QLX_PREF_KTO}
# the readings' default hyperparameters (beta, gamma, lambda_d, lambda_u)
PREF_DEFAULTS = {"dpo": (0.1, 0.0, 1.0, 1.0), "orpo": (0.1, 0.0, 1.0, 1.0), "simpo": (2.0, 0.5, 1.0, 1.0),
                 "kto": (0.1, 0.0, 1.0, 1.0)}
BLOB_NSEG = 16
PROJ = ("q", "k", "v", "o", "gate", "up", "down")

EXPORTED = (
    "qlx_last_error", "qlx_version", "nf4_quantize", "nf4_dequant", "qlx_linear_workspace_bytes",
    "qlora_linear_fwd", "qlora_linear_bwd", "qlx_layer_blob_layout", "qlx_layer_workspace_bytes",
    "layer_fwd", "layer_bwd", "qlx_ctx_create", "qlx_ctx_destroy", "qlx_ctx_sync",
    "qlx_step_workspace_bytes", "stream_step_sft", "stream_step_dpo", "stream_step_pref", "qlx_merge_workspace_bytes", "qlx_lora_merge", "qlx_profile_begin", "qlx_profile_begin_prefix", "qlx_profile_end", "qlx_adamw_lora",
    "qlx_layer_file_write", "qlx_layer_file_open", "qlx_layer_file_close", "qlx_layer_file_info",
    "qlx_layer_file_read", "qlx_ctx_set_layer_source", "qlx_stream_source_auto", "qlx_ctx_set_debug",
    "qlx_peak_mfma", "qlx_peak_copy", "qlx_layer_wire_layout", "qlx_layer_blob_to_wire", "qlx_ctx_set_keep_layers",
    "qlx_ctx_set_adamw", "qlx_ctx_adamw_t", "qlora_linear_fwd_noalloc",
)


class QlxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qlx error {code}: {msg}")
        self.code = code


class Dims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("inter", C.c_int32), ("vocab", C.c_int32),
                ("n_layers", C.c_int32), ("lora_r", C.c_int32), ("lora_alpha", C.c_float),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("act_dtype", C.c_int32)]

    @classmethod
    def of(cls, d, act_dtype: int | None = None) -> "Dims":
        """C dims from any object with the decoder fields. act_dtype (QLX_ACT_BF16
        or QLX_ACT_F16): the 16-bit activation type of layer and step calls; by
        default d's own act_dtype if it has one, else ACT_DEFAULT."""
        if isinstance(d, Dims):
            if act_dtype is None or act_dtype == d.act_dtype:
                return d
            return cls(d.hidden, d.n_heads, d.n_kv_heads, d.head_dim, d.inter, d.vocab, d.n_layers, d.lora_r,
                       d.lora_alpha, d.rms_eps, d.rope_theta, int(act_dtype))
        act = act_dtype if act_dtype is not None else getattr(d, "act_dtype", ACT_DEFAULT)
        return cls(d.hidden, d.n_heads, d.n_kv_heads, d.head_dim, d.inter, d.vocab, d.n_layers,
                   d.lora_r, float(d.lora_alpha), float(d.rms_eps), float(d.rope_theta), int(act))


class NF4(C.Structure):
    _fields_ = [("packed", C.c_void_p), ("absmax", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64)]


class Lora(C.Structure):
    _fields_ = [("A", C.c_void_p * 7), ("B", C.c_void_p * 7)]


class LoraGrad(C.Structure):
    _fields_ = [("dA", C.c_void_p * 7), ("dB", C.c_void_p * 7)]


class LoraBuf(C.Structure):
    _fields_ = [("A", C.c_void_p * 7), ("B", C.c_void_p * 7)]


class AdamwCfg(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double), ("eps", C.c_double),
                ("weight_decay", C.c_double)]


class PrefCfg(C.Structure):
    _fields_ = [("kind", C.c_int), ("ref_schedule", C.c_int), ("beta", C.c_float), ("gamma", C.c_float),
                ("lambda_d", C.c_float), ("lambda_u", C.c_float)]


class Stats(C.Structure):
    _fields_ = [("layer_reads", C.c_int64), ("h2d_bytes", C.c_int64), ("layer_passes", C.c_int64),
                ("step_ms", C.c_float), ("h2d_ms", C.c_float), ("disk_bytes", C.c_int64), ("disk_ms", C.c_float)]


class KernelProf(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_int64), ("ms", C.c_double), ("flops", C.c_double),
                ("bytes", C.c_double)]


class Model(C.Structure):
    _fields_ = [("dims", Dims), ("layer_blobs", C.POINTER(C.c_void_p)), ("embed_f16", C.c_void_p),
                ("lm_head_f16", C.c_void_p), ("final_norm", C.c_void_p), ("lora", C.POINTER(Lora)),
                ("blob_form", C.c_int)]


_lib = None


def lib() -> C.CDLL:
    """The loaded libqlx; raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libqlx.so not built at {LIB_PATH}: run __graft_entry__.build()")
    L = C.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
    sig = {
        "qlx_last_error": (C.c_char_p, []),
        "qlx_version": (C.c_char_p, []),
        "nf4_quantize": (i32, [vp, i64, i64, vp, vp, vp]),
        "nf4_dequant": (i32, [vp, vp, i64, i64, i32, vp, vp]),
        "qlx_linear_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "qlora_linear_fwd": (i32, [vp, i64, NF4, vp, vp, i32, f32, vp, vp, sz, vp]),
        "qlora_linear_fwd_noalloc": (i32, [vp, i64, NF4, vp, vp, i32, f32, vp, vp]),
        "qlora_linear_bwd": (i32, [vp, vp, i64, NF4, vp, vp, i32, f32, vp, vp, vp, i32, vp, sz, vp]),
        "qlx_layer_blob_layout": (i32, [C.POINTER(Dims), C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]),
        "qlx_layer_wire_layout": (i32, [C.POINTER(Dims), C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]),
        "qlx_layer_blob_to_wire": (i32, [C.POINTER(Dims), vp, vp]),
        "qlx_layer_workspace_bytes": (sz, [C.POINTER(Dims), i32, i32]),
        "layer_fwd": (i32, [C.POINTER(Dims), vp, C.POINTER(Lora), vp, i32, i32, vp, vp, sz, vp]),
        "layer_bwd": (i32, [C.POINTER(Dims), vp, C.POINTER(Lora), vp, vp, i32, i32, vp, C.POINTER(LoraGrad),
                            vp, sz, vp]),
        "qlx_ctx_create": (i32, [C.POINTER(vp), i32]),
        "qlx_ctx_destroy": (i32, [vp]),
        "qlx_ctx_sync": (i32, [vp, C.POINTER(Stats)]),
        "qlx_step_workspace_bytes": (sz, [C.POINTER(Dims), i32, i32, i32]),
        "stream_step_sft": (i32, [vp, C.POINTER(Model), vp, i32, i32, i32, vp, C.POINTER(LoraGrad), vp, sz, vp]),
        "stream_step_dpo": (i32, [vp, C.POINTER(Model), vp, vp, i32, i32, i32, f32, i32, i32, vp, vp,
                                  C.POINTER(LoraGrad), vp, sz, vp]),
        "stream_step_pref": (i32, [vp, C.POINTER(Model), C.POINTER(PrefCfg), vp, vp, i32, i32, i32, i32, vp, vp,
                                   C.POINTER(LoraGrad), vp, sz, vp]),
        "qlx_merge_workspace_bytes": (sz, [C.c_int64, C.c_int64, i32]),
        "qlx_lora_merge": (i32, [NF4, vp, vp, i32, f32, i32, vp, vp, vp, sz, vp]),
        "qlx_profile_begin": (i32, []),
        "qlx_profile_begin_prefix": (i32, [C.c_char_p]),
        "qlx_adamw_lora": (i32, [C.POINTER(Dims), C.POINTER(LoraBuf), C.POINTER(LoraGrad), C.POINTER(LoraBuf),
                                 C.POINTER(LoraBuf), C.c_int64, C.POINTER(AdamwCfg), C.c_void_p]),
        "qlx_profile_end": (i32, [C.POINTER(KernelProf), i32, C.POINTER(C.c_int)]),
        "qlx_layer_file_write": (i32, [C.c_char_p, C.POINTER(Dims), C.POINTER(C.c_void_p), i32]),
        "qlx_layer_file_open": (i32, [C.POINTER(vp), C.c_char_p, C.POINTER(Dims), i32]),
        "qlx_layer_file_close": (i32, [vp]),
        "qlx_layer_file_info": (i32, [vp, C.POINTER(C.c_int), C.POINTER(C.c_uint64)]),
        "qlx_layer_file_read": (i32, [vp, i32, vp]),
        "qlx_ctx_set_layer_source": (i32, [vp, vp]),
        "qlx_stream_source_auto": (i32, [C.c_uint64, C.c_uint64, C.POINTER(C.c_int)]),
        "qlx_ctx_set_debug": (i32, [vp, i32, i32]),
        "qlx_ctx_set_keep_layers": (i32, [vp, i32]),
        "qlx_ctx_set_adamw": (i32, [vp, i32, C.POINTER(LoraBuf), C.POINTER(LoraBuf), C.POINTER(LoraBuf),
                                    C.POINTER(AdamwCfg), C.c_int64]),
        "qlx_ctx_adamw_t": (i32, [vp, C.POINTER(C.c_int64)]),
        "qlx_peak_mfma": (i32, [C.c_int64, i32, i32, vp, vp]),
        "qlx_peak_copy": (i32, [vp, vp, C.c_uint64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(code: int) -> None:
    if code != QLX_OK:
        raise QlxError(code, lib().qlx_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _bits16(t: torch.Tensor) -> torch.Tensor:
    assert t.dtype in (torch.bfloat16, torch.float16, torch.int16, torch.uint16), t.dtype
    return t


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------- NF4
def nf4_quantize(w: torch.Tensor, packed: torch.Tensor, absmax: torch.Tensor, stream=None) -> None:
    """w bf16 [rows, cols] (any shape, flattened) -> packed uint8 [ceil(n/2)], absmax fp32 [ceil(n/64)]."""
    _bits16(w)
    rows = w.shape[0] if w.dim() > 0 else 1
    cols = w.numel() // rows if rows else 0
    _check(lib().nf4_quantize(_ptr(w), rows, cols, _ptr(packed), _ptr(absmax), _stream(stream)))


def nf4_dequant(packed: torch.Tensor, absmax: torch.Tensor, rows: int, cols: int, out: torch.Tensor,
                stream=None) -> None:
    dt = QLX_BF16 if out.dtype == torch.bfloat16 else QLX_F32
    assert out.dtype in (torch.bfloat16, torch.float32)
    _check(lib().nf4_dequant(_ptr(packed), _ptr(absmax), rows, cols, dt, _ptr(out), _stream(stream)))


class NF4Matrix:
    """A canonical NF4 matrix [rows = out_features, cols = in_features] on the device."""

    def __init__(self, packed: torch.Tensor, absmax: torch.Tensor, rows: int, cols: int):
        self.packed, self.absmax, self.rows, self.cols = packed, absmax, int(rows), int(cols)

    @classmethod
    def quantize(cls, w: torch.Tensor, stream=None) -> "NF4Matrix":
        rows, cols = w.shape
        n = rows * cols
        packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=w.device)
        absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=w.device)
        nf4_quantize(w, packed, absmax, stream)
        return cls(packed, absmax, rows, cols)

    def c(self) -> NF4:
        return NF4(_ptr(self.packed), _ptr(self.absmax), self.rows, self.cols)


def lora_merge(W: NF4Matrix, A: torch.Tensor, B: torch.Tensor, scale: float, to_nf4: bool = False,
               stream=None):
    """qlx_lora_merge: W' + scale * B A rounded to bf16 [rows, cols], or (to_nf4)
    that matrix re-quantized to a new NF4Matrix."""
    r = A.shape[0]
    if A.shape != (r, W.cols) or B.shape != (W.rows, r):
        raise ValueError("A must be [r, cols] and B [rows, r]")
    dev = W.packed.device
    if not to_nf4:
        out = torch.empty(W.rows, W.cols, dtype=torch.bfloat16, device=dev)
        _check(lib().qlx_lora_merge(W.c(), _ptr(A), _ptr(B), r, float(scale), QLX_MERGE_BF16, _ptr(out), None, None,
                                    0, _stream(stream)))
        return out
    n = W.rows * W.cols
    packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=dev)
    ws = workspace(int(lib().qlx_merge_workspace_bytes(W.rows, W.cols, QLX_MERGE_NF4)), dev)
    _check(lib().qlx_lora_merge(W.c(), _ptr(A), _ptr(B), r, float(scale), QLX_MERGE_NF4, _ptr(packed), _ptr(absmax),
                                _ptr(ws), ws.numel(), _stream(stream)))
    return NF4Matrix(packed, absmax, W.rows, W.cols)


# -------------------------------------------------------------- QLoRA linear
def linear_workspace_bytes(T: int, in_f: int, out_f: int, r: int) -> int:
    return int(lib().qlx_linear_workspace_bytes(T, in_f, out_f, r))


def qlora_linear_fwd(x: torch.Tensor, W: NF4Matrix, A, B, scale: float, y: torch.Tensor,
                     ws: torch.Tensor | None = None, stream=None) -> None:
    T = x.shape[0]
    r = A.shape[0] if A is not None else 0
    if ws is None:
        ws = workspace(linear_workspace_bytes(T, W.cols, W.rows, r), x.device)
    _check(lib().qlora_linear_fwd(_ptr(x), T, W.c(), _ptr(A), _ptr(B), r, float(scale), _ptr(y), _ptr(ws),
                                  ws.numel(), _stream(stream)))


def qlora_linear_bwd(dy: torch.Tensor, x: torch.Tensor, W: NF4Matrix, A, B, scale: float, dx, dA, dB,
                     accumulate: bool = False, ws: torch.Tensor | None = None, stream=None) -> None:
    T = x.shape[0]
    r = A.shape[0] if A is not None else 0
    if ws is None:
        ws = workspace(linear_workspace_bytes(T, W.cols, W.rows, r), x.device)
    _check(lib().qlora_linear_bwd(_ptr(dy), _ptr(x), T, W.c(), _ptr(A), _ptr(B), r, float(scale), _ptr(dx),
                                  _ptr(dA), _ptr(dB), int(accumulate), _ptr(ws), ws.numel(), _stream(stream)))


# ------------------------------------------------------------------- layers
def blob_layout(dims) -> tuple[list[int], int]:
    d = Dims.of(dims)
    offs = (C.c_uint64 * BLOB_NSEG)()
    total = C.c_uint64()
    _check(lib().qlx_layer_blob_layout(C.byref(d), offs, C.byref(total)))
    return list(offs), int(total.value)


def wire_layout(dims) -> tuple[list[int], int]:
    """Offsets and size of the wire form of a layer blob (block maxima as bf16)."""
    d = Dims.of(dims)
    offs = (C.c_uint64 * BLOB_NSEG)()
    total = C.c_uint64()
    _check(lib().qlx_layer_wire_layout(C.byref(d), offs, C.byref(total)))
    return list(offs), int(total.value)


def blob_to_wire(dims, blob: torch.Tensor, pin_memory: bool = True) -> torch.Tensor:
    """Host full-form blob -> new host uint8 tensor in the wire form (pinned
    by default); raises QlxError if a block maximum is not a bf16 value."""
    if blob.is_cuda:
        raise ValueError("blob_to_wire converts host blobs")
    d = Dims.of(dims)
    _, total = wire_layout(d)
    out = torch.empty(total, dtype=torch.uint8, pin_memory=pin_memory)
    _check(lib().qlx_layer_blob_to_wire(C.byref(d), _ptr(blob), _ptr(out)))
    return out


def fill_blob(dims, blob: torch.Tensor, weights_bf16: dict, g1: torch.Tensor, g2: torch.Tensor,
              stream=None) -> None:
    """Quantize each projection's bf16 weight (device tensors [out, in]) with
    nf4_quantize straight into a device blob, and copy the RMSNorm gains."""
    offs, total = blob_layout(dims)
    assert blob.numel() >= total and blob.is_cuda
    base = blob.data_ptr()
    for p, name in enumerate(PROJ):
        w = weights_bf16[name]
        rows, cols = w.shape
        _check(lib().nf4_quantize(_ptr(w), rows, cols, base + offs[p], base + offs[7 + p], _stream(stream)))
    H = g1.numel()
    blob[offs[14]: offs[14] + 4 * H].copy_(g1.to(torch.float32).view(torch.uint8))
    blob[offs[15]: offs[15] + 4 * H].copy_(g2.to(torch.float32).view(torch.uint8))


class LoraLayer:
    """The 7 adapters of one layer: A [r, in], B [out, r] fp32 device tensors."""

    def __init__(self, A: Sequence[torch.Tensor], B: Sequence[torch.Tensor]):
        self.A, self.B = list(A), list(B)

    def c(self) -> Lora:
        return Lora((C.c_void_p * 7)(*[_ptr(a) for a in self.A]), (C.c_void_p * 7)(*[_ptr(b) for b in self.B]))


class LoraGrads:
    """Gradient buffers matching a LoraLayer (fp32, device)."""

    def __init__(self, like: LoraLayer):
        self.dA = [torch.empty_like(a) for a in like.A]
        self.dB = [torch.empty_like(b) for b in like.B]

    def c(self) -> LoraGrad:
        return LoraGrad((C.c_void_p * 7)(*[_ptr(a) for a in self.dA]), (C.c_void_p * 7)(*[_ptr(b) for b in self.dB]))


def _lora_buf(A: Sequence[torch.Tensor], B: Sequence[torch.Tensor]) -> LoraBuf:
    return LoraBuf((C.c_void_p * 7)(*[_ptr(a) for a in A]), (C.c_void_p * 7)(*[_ptr(b) for b in B]))


def adamw_lora(dims, params: Sequence[LoraLayer], grads: Sequence[LoraGrads], m: Sequence[LoraLayer],
               v: Sequence[LoraLayer], t: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
               eps: float = 1e-8, weight_decay: float = 0.0, stream=None) -> None:
    """qlx_adamw_lora: one AdamW update of every LoRA factor in place (params
    are the model's LoraLayer tensors; m, v LoraLayer-shaped moment buffers)."""
    d = Dims.of(dims)
    L = d.n_layers
    if not (len(params) == len(grads) == len(m) == len(v) == L):
        raise ValueError("params, grads, m, v need one entry per layer")
    P = (LoraBuf * L)(*[_lora_buf(x.A, x.B) for x in params])
    G = (LoraGrad * L)(*[g.c() for g in grads])
    Mb = (LoraBuf * L)(*[_lora_buf(x.A, x.B) for x in m])
    Vb = (LoraBuf * L)(*[_lora_buf(x.A, x.B) for x in v])
    cfg = AdamwCfg(lr, beta1, beta2, eps, weight_decay)
    _check(lib().qlx_adamw_lora(C.byref(d), P, G, Mb, Vb, int(t), C.byref(cfg), _stream(stream)))


class AdamW:
    """AdamW state for a list of LoraLayer (zero moments, step count)."""

    def __init__(self, dims, params: Sequence[LoraLayer], lr: float = 2e-5, beta1: float = 0.9,
                 beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0):
        self.dims, self.params = dims, list(params)
        self.m = [LoraLayer([torch.zeros_like(a) for a in p.A], [torch.zeros_like(b) for b in p.B]) for p in params]
        self.v = [LoraLayer([torch.zeros_like(a) for a in p.A], [torch.zeros_like(b) for b in p.B]) for p in params]
        self.t = 0
        self.hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)

    def step(self, grads: Sequence[LoraGrads], stream=None) -> None:
        self.t += 1
        adamw_lora(self.dims, self.params, grads, self.m, self.v, self.t, stream=stream, **self.hp)


def layer_workspace_bytes(dims, batch: int, seq: int) -> int:
    d = Dims.of(dims)
    return int(lib().qlx_layer_workspace_bytes(C.byref(d), batch, seq))


def layer_fwd(dims, blob: torch.Tensor, lora: LoraLayer | None, h_in: torch.Tensor, batch: int, seq: int,
              h_out: torch.Tensor, ws: torch.Tensor | None = None, stream=None) -> None:
    d = Dims.of(dims)
    if ws is None:
        ws = workspace(layer_workspace_bytes(d, batch, seq), h_in.device)
    lo = C.byref(lora.c()) if lora is not None else None
    _check(lib().layer_fwd(C.byref(d), _ptr(blob), lo, _ptr(h_in), batch, seq, _ptr(h_out), _ptr(ws),
                           ws.numel(), _stream(stream)))


def layer_bwd(dims, blob: torch.Tensor, lora: LoraLayer, h_in: torch.Tensor, dh_out: torch.Tensor, batch: int,
              seq: int, dh_in: torch.Tensor | None, grads: LoraGrads, ws: torch.Tensor | None = None,
              stream=None) -> None:
    d = Dims.of(dims)
    if ws is None:
        ws = workspace(layer_workspace_bytes(d, batch, seq), h_in.device)
    lc, gc = lora.c(), grads.c()
    _check(lib().layer_bwd(C.byref(d), _ptr(blob), C.byref(lc), _ptr(h_in), _ptr(dh_out), batch, seq,
                           _ptr(dh_in), C.byref(gc), _ptr(ws), ws.numel(), _stream(stream)))


# ------------------------------------------------------------------ streaming
class Context:
    """Streaming context (side stream, slot events, statistics)."""

    def __init__(self, device: int = 0):
        h = C.c_void_p()
        _check(lib().qlx_ctx_create(C.byref(h), device))
        self.h = h

    def set_adamw(self, opt: "AdamW | None") -> None:
        """Fused AdamW: each step on this context updates layer i's adapters
        right after layer i's backward (bit-identical to opt.step(grads)
        after the step); opt.t follows the steps. None switches it off."""
        if opt is None:
            _check(lib().qlx_ctx_set_adamw(self.h, 0, None, None, None, None, 0))
            self.adam = None
            return
        L = len(opt.params)
        P = (LoraBuf * L)(*[_lora_buf(x.A, x.B) for x in opt.params])
        Mb = (LoraBuf * L)(*[_lora_buf(x.A, x.B) for x in opt.m])
        Vb = (LoraBuf * L)(*[_lora_buf(x.A, x.B) for x in opt.v])
        h = opt.hp
        cfg = AdamwCfg(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"])
        _check(lib().qlx_ctx_set_adamw(self.h, L, P, Mb, Vb, C.byref(cfg), opt.t + 1))
        self.adam = opt

    def _stepped(self) -> None:
        """After a step call: the fused AdamW's update count moved on."""
        if getattr(self, "adam", None) is not None:
            t = C.c_int64()
            _check(lib().qlx_ctx_adamw_t(self.h, C.byref(t)))
            self.adam.t = int(t.value) - 1

    def set_keep_layers(self, on: bool = True) -> None:
        """Keep the two layers a step leaves in the slots for the next step
        (same workspace and blobs; see qlx_ctx_set_keep_layers)."""
        _check(lib().qlx_ctx_set_keep_layers(self.h, 1 if on else 0))

    def set_debug(self, flags: int, delay_us: int = 0) -> None:
        """Stream fault injection (QLX_DEBUG_*): serialize, poison freed slots, delay copies or compute."""
        _check(lib().qlx_ctx_set_debug(self.h, flags, delay_us))

    def set_layer_source(self, f: "LayerFile | None") -> None:
        """Attaches a stack file for QLX_STREAMED_DISK (None detaches)."""
        _check(lib().qlx_ctx_set_layer_source(self.h, f.h if f is not None else None))
        self.source = f  # keeps the file alive while attached

    def sync(self) -> dict:
        st = Stats()
        _check(lib().qlx_ctx_sync(self.h, C.byref(st)))
        return {k: getattr(st, k) for k, _ in Stats._fields_}

    def close(self) -> None:
        if self.h:
            lib().qlx_ctx_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LayerFile:
    """A stack file on disk (qlx_layer_file): blob i at i * stride. Reads go
    around the page cache (O_DIRECT) unless buffered=True or the file system
    refuses it."""

    @staticmethod
    def write(path: str, dims, blobs: Sequence, wire: bool = False) -> None:
        """blobs: host buffers (uint8 tensors or numpy arrays) of one layer blob
        each, in the wire form when wire=True."""
        d = Dims.of(dims)
        ptrs = [b.data_ptr() if isinstance(b, torch.Tensor) else b.ctypes.data for b in blobs]
        if len(ptrs) != d.n_layers:
            raise ValueError(f"{len(ptrs)} blobs for {d.n_layers} layers")
        for b in blobs:
            if isinstance(b, torch.Tensor) and b.is_cuda:
                raise ValueError("layer blobs for the file must be host memory")
        arr = (C.c_void_p * len(ptrs))(*ptrs)
        _check(lib().qlx_layer_file_write(os.fsencode(path), C.byref(d), C.cast(arr, C.POINTER(C.c_void_p)),
                                          QLX_FILE_WIRE if wire else 0))

    def __init__(self, path: str, dims, buffered: bool = False, wire: bool = False):
        self.dims = Dims.of(dims)
        self.wire = wire
        h = C.c_void_p()
        _check(lib().qlx_layer_file_open(C.byref(h), os.fsencode(path), C.byref(self.dims),
                                         (QLX_FILE_BUFFERED if buffered else 0) | (QLX_FILE_WIRE if wire else 0)))
        self.h = h
        self.path = path

    def info(self) -> dict:
        direct, stride = C.c_int(), C.c_uint64()
        _check(lib().qlx_layer_file_info(self.h, C.byref(direct), C.byref(stride)))
        return {"direct": bool(direct.value), "stride": int(stride.value)}

    def read(self, layer: int, out) -> None:
        """Reads layer `layer`'s blob into a host buffer (tensor or numpy array)."""
        ptr = out.data_ptr() if isinstance(out, torch.Tensor) else out.ctypes.data
        _check(lib().qlx_layer_file_read(self.h, layer, ptr))

    def close(self) -> None:
        """Frees the file; raises QlxError while a context still holds it."""
        if self.h:
            _check(lib().qlx_layer_file_close(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stream_source_auto(stack_bytes: int, reserve_bytes: int = 0) -> int:
    """QLX_STREAMED if the stack (plus reserve) fits in available host memory, else QLX_STREAMED_DISK."""
    mode = C.c_int()
    _check(lib().qlx_stream_source_auto(int(stack_bytes), int(reserve_bytes), C.byref(mode)))
    return mode.value


class StreamModel:
    """Holds the tensors of a model and the C struct pointing at them.
    blobs: pinned host uint8 tensors (streamed) or device uint8 tensors
    (resident); None for a model that only streams from a layer file.
    blob_form: QLX_BLOB_FULL, or QLX_BLOB_WIRE for streamed host blobs made
    by blob_to_wire."""

    def __init__(self, dims, blobs: Sequence[torch.Tensor] | None, embed_f16: torch.Tensor, head_f16: torch.Tensor,
                 final_norm: torch.Tensor, lora: Sequence[LoraLayer], blob_form: int = QLX_BLOB_FULL,
                 act_dtype: int | None = None):
        self.dims = Dims.of(dims, act_dtype)
        self.blob_form = blob_form
        _, total = wire_layout(self.dims) if blob_form == QLX_BLOB_WIRE else blob_layout(self.dims)
        for bl in blobs or ():
            if bl.numel() * bl.element_size() < total:
                raise ValueError(f"layer blob holds {bl.numel() * bl.element_size()} bytes, layout needs {total}")
        self.blobs = list(blobs) if blobs is not None else None
        self.embed, self.head, self.final_norm, self.lora = embed_f16, head_f16, final_norm, list(lora)
        if self.blobs is not None:
            self._blob_arr = (C.c_void_p * len(self.blobs))(*[_ptr(b) for b in self.blobs])
            blob_ptr = C.cast(self._blob_arr, C.POINTER(C.c_void_p))
        else:
            self._blob_arr, blob_ptr = None, None
        self._lora_arr = (Lora * len(self.lora))(*[l.c() for l in self.lora])
        self.c = Model(self.dims, blob_ptr, _ptr(embed_f16), _ptr(head_f16),
                       _ptr(final_norm), C.cast(self._lora_arr, C.POINTER(Lora)), blob_form)

    def with_blobs(self, blobs: Sequence[torch.Tensor], blob_form: int = QLX_BLOB_FULL) -> "StreamModel":
        return StreamModel(self.dims, blobs, self.embed, self.head, self.final_norm, self.lora, blob_form)

    def with_act(self, act_dtype: int) -> "StreamModel":
        """The same model computing with another 16-bit activation type."""
        return StreamModel(Dims.of(self.dims, act_dtype), self.blobs, self.embed, self.head, self.final_norm, self.lora,
                           self.blob_form)


def step_workspace_bytes(dims, kind: int, batch: int, seq: int) -> int:
    d = Dims.of(dims)
    return int(lib().qlx_step_workspace_bytes(C.byref(d), kind, batch, seq))


def _grad_arr(grads: Sequence[LoraGrads]):
    return (LoraGrad * len(grads))(*[g.c() for g in grads])


def stream_step_sft(ctx: Context, model: StreamModel, tokens: torch.Tensor, mode: int, loss: torch.Tensor,
                    grads: Sequence[LoraGrads], ws: torch.Tensor, stream=None) -> None:
    B, S = tokens.shape
    ga = _grad_arr(grads)
    _check(lib().stream_step_sft(ctx.h, C.byref(model.c), _ptr(tokens), B, S, mode, _ptr(loss), ga, _ptr(ws),
                                 ws.numel(), _stream(stream)))
    ctx._stepped()


def stream_step_dpo(ctx: Context, model: StreamModel, chosen: torch.Tensor, rejected: torch.Tensor,
                    prompt_len: int, beta: float, mode: int, ref_schedule: int, loss: torch.Tensor,
                    logps: torch.Tensor, grads: Sequence[LoraGrads], ws: torch.Tensor, stream=None) -> None:
    P, S = chosen.shape
    ga = _grad_arr(grads)
    _check(lib().stream_step_dpo(ctx.h, C.byref(model.c), _ptr(chosen), _ptr(rejected), P, S, prompt_len,
                                 float(beta), mode, ref_schedule, _ptr(loss), _ptr(logps), ga, _ptr(ws),
                                 ws.numel(), _stream(stream)))
    ctx._stepped()


def stream_step_pref(ctx: Context, model: StreamModel, kind: str, chosen: torch.Tensor, rejected: torch.Tensor,
                     prompt_len: int, mode: int, loss: torch.Tensor, logps: torch.Tensor, grads: Sequence[LoraGrads],
                     ws: torch.Tensor, ref_schedule: int = QLX_DPO_REF_FUSED, beta: float | None = None,
                     gamma: float | None = None, lambda_d: float | None = None, lambda_u: float | None = None,
                     stream=None) -> None:
    """stream_step_pref: kind "dpo" | "orpo" | "simpo" | "kto"; unset
    hyperparameters take the kind's defaults (PREF_DEFAULTS)."""
    b0, g0, ld0, lu0 = PREF_DEFAULTS[kind]
    cfg = PrefCfg(PREF_KINDS[kind], ref_schedule, b0 if beta is None else beta, g0 if gamma is None else gamma,
                  ld0 if lambda_d is None else lambda_d, lu0 if lambda_u is None else lambda_u)
    P, S = chosen.shape
    ga = _grad_arr(grads)
    _check(lib().stream_step_pref(ctx.h, C.byref(model.c), C.byref(cfg), _ptr(chosen), _ptr(rejected), P, S,
                                  prompt_len, mode, _ptr(loss), _ptr(logps), ga, _ptr(ws), ws.numel(),
                                  _stream(stream)))
    ctx._stepped()


# ------------------------------------------------------------------ profiling
def profile_begin(prefix: str | None = None) -> None:
    """Start per-kernel event timing; with `prefix`, only kernels whose row
    name starts with it are timed (the rest run with no events)."""
    if prefix:
        _check(lib().qlx_profile_begin_prefix(prefix.encode()))
    else:
        _check(lib().qlx_profile_begin())


def profile_end() -> dict:
    """{kernel name: {launches, ms, flops, bytes}} summed since profile_begin()."""
    n = C.c_int()
    out = (KernelProf * 64)()
    _check(lib().qlx_profile_end(out, 64, C.byref(n)))
    return {out[i].name.decode(): {"launches": out[i].launches, "ms": out[i].ms, "flops": out[i].flops,
                                   "bytes": out[i].bytes} for i in range(min(n.value, 64))}
