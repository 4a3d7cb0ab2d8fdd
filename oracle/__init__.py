"""CPU oracle for the nanochat GPT forward+backward step.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package. The GPU library never
calls it, and it shares no code with the GPU library: it derives the
parameter layout, the per-layer window/value-embedding pattern and every
formula on its own, from the pages.

Pages cited (by title and section):
  * "NanoChat基础训练报告" (the nanochat d12 base-training report), block
    "模型架构" (model architecture): layer count, widths, vocabulary, the
    286.3M / 261.1M parameter totals, value embeddings on odd layers with a
    learned gate.
  * "Nanochat在nanoGPT之上的新增功能" (nanochat additions over nanoGPT),
    section 1 "模型架构（gpt.py）": the feature table (RoPE, parameter-free
    RMSNorm, ReLU^2, separate c_q/c_k/c_v/c_proj, GQA, QK-norm after RoPE, no
    bias, untied embeddings, no dropout, tanh logit softcap +-15, per-layer
    sliding windows, value residuals, per-layer resid/x0 lambdas, dynamic
    per-tensor fp8) and the notes under it ("关键架构更改说明").
  * "nanochat — 架构与原理" (nanochat architecture overview), section 4: the
    -1 ignore index of the loss, the fp8 matmul wrapper; section 5: the
    sliding window needs a flash-attention backend.

Functions whose result the pages do not fix, and how each is pinned, are
listed in ``oracle/model.py``'s module docstring. The gate form of the value
embedding is "parity unpinned" with respect to the pages (one reading of a
sentence that names a gate but not its form). The same holds for the two
model variants: the Smear gate's form and the Backout layer are readings of
the additions page's notes (stated in ``oracle/model.py``); the tests pin the
oracle's arithmetic for them, not the readings.
"""
from .model import (  # noqa: F401
    layer_is_full, layer_has_ve, layout, param_offsets, unpack,
    rms_fwd, rms_bwd, rope_tables, rope_fwd, rope_bwd, attention_fwd,
    attention_bwd, softcap_ce_fwd_bwd, forward_backward, forward_loss,
    visible, model_flops_per_token, smear_fwd, smear_bwd, backout_layer,
)
from . import fp8  # noqa: F401
from . import decode  # noqa: F401
from . import optim  # noqa: F401
