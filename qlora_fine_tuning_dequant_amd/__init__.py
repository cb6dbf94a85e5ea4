"""MI355X-native layer-streamed QLoRA training step (NF4 base + LoRA).

The compute lives in libqlx.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/qlx.h); ``binding`` marshals torch tensors to it."""
from . import binding
from .binding import (AdamW, Context, LayerFile, LoraGrads, LoraLayer, NF4Matrix, QlxError, StreamModel,
                      adamw_lora, layer_bwd, layer_fwd, lora_merge, nf4_dequant, nf4_quantize, qlora_linear_bwd,
                      qlora_linear_fwd, stream_source_auto, stream_step_dpo, stream_step_pref, stream_step_sft)

__all__ = ["binding", "AdamW", "adamw_lora", "lora_merge", "Context", "LayerFile", "LoraGrads", "LoraLayer",
           "NF4Matrix", "QlxError", "StreamModel", "layer_bwd", "layer_fwd", "nf4_dequant", "nf4_quantize",
           "qlora_linear_bwd", "qlora_linear_fwd", "stream_source_auto", "stream_step_dpo", "stream_step_pref",
           "stream_step_sft"]
