"""Oracle: a plain, slow, obviously correct CPU implementation of the
layer-streamed QLoRA training step (NF4 base + LoRA), written from the pages
and the published methods they name.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use it. It shares no code, table or constant with the
HIP path; both sides consume the seeded arrays from ``synth``.

Everything is numpy. Floating point is float32 unless a caller passes float64
arrays (the finite-difference checks do), in which case every step runs in
float64. There is no blocking, fusion or reordering beyond the definitions:
each function is the formula it cites, written out.

Sources (cited by page title and section; the pages give system-level facts,
the published methods fill in the mathematics):
  * rug.gal, "Soup: fine-tune an 8B model on a 4 GB laptop GPU (layer
    streaming)" (es/it/fr editions), sections intro and "En detalle":
    frozen NF4 base fed one decoder layer at a time, LoRA trainable and
    resident, bit-exact vs a non-streamed run, DPO reference = same stream
    with LoRA switched off.
  * guillermodelpino.com, "Soup: afinar un modelo de 8.000 millones de
    parámetros en un portátil con 4 GB de gráfica", sections "Qué es
    exactamente" (config: Llama-3.1-8B-Instruct, lora r 64 alpha 16,
    quantization 4bit) and "El streaming de capas".
  * imasters.com.br, "Soup promete fine-tuning de modelo 8B em GPU de notebook
    com 4 GB", sections "Como cabe um 8B em 4 GB" (NF4) and "Do SFT para os
    métodos de preferência" (DPO reference with adapters off).
  * QLoRA (Dettmers et al., 2023), NormalFloat section and the NF4 appendix.
  * LoRA (Hu et al., 2021), section 4.1.
  * Llama decoder: RMSNorm (Zhang & Sennrich, 2019), RoPE rotate-half
    (Su et al., 2021), SwiGLU (Shazeer, 2020), grouped-query attention.
  * DPO (Rafailov et al., 2023), the sigmoid objective (equation 7).
  * ORPO (Hong et al., 2024), SimPO (Meng et al., 2024), KTO (Ethayarajh et
    al., 2024) for the other preference objectives the pages list.
  * AdamW (Kingma & Ba, Algorithm 1; Loshchilov & Hutter, Algorithm 2) for
    the optimizer update (the pages give only the learning rate).

Parity status per function is stated in each module header; functions with
no independent pin say "parity unpinned".
"""
from .nf4 import (nf4_codebook, nf4_midpoints, nf4_quantize, nf4_dequant,
                  bf16_rne_bits, bf16_bits_to_f32, bf16_round)
from .layer import (rmsnorm_fwd, rmsnorm_bwd, rope_cos_sin, rope_fwd, rope_bwd,
                    attention_fwd, attention_bwd, swiglu_fwd, swiglu_bwd,
                    qlora_linear_fwd, qlora_linear_bwd, layer_fwd, layer_bwd,
                    dequant_layer)
from .model import (embed, head_ce, seq_logprobs, dpo_loss, model_forward,
                    sft_step, dpo_step, pref_step)
from .preference import orpo_loss, simpo_loss, kto_loss, kto_z0, kl_tokens
from .optim import adamw, adamw_lora
from .merge import lora_merge

__all__ = [n for n in dir() if not n.startswith("_")]
