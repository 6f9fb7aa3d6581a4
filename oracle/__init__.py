"""Oracle: a plain, slow, fp64 CPU definition of one training step of the layer-sliding
offloaded fine-tuning method (SlideFormer, "An Efficient Heterogeneous Co-Design for
Fine-Tuning on a Single GPU", Yang & Wen).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package. The product path (the HIP library and its Python binding)
never imports it, and this package imports nothing from the product path.

What it computes. The pages define the method as exact full-parameter fine-tuning whose
offloaded schedule reaches the same result as plain training (abstract: ">95% of peak
performance"; gist.science summary, section 2C: the fused LinearCrossEntropy has no accuracy
loss). So the oracle is the plain definition of one training step of a Llama-style pre-norm
decoder (the model family the summary names in section 4), written with NumPy fp64 and a
library matrix product as its only primitive. Readings of what the pages leave open are
listed in the module docstrings.

Every function here is pinned by tests/test_oracle_*.py against mathematics or library
routines (finite differences, closed forms, invariants, torch CPU reference routines).
"""
from .model import (LayerShape, rmsnorm_fwd, rmsnorm_bwd, rope_tables, rope_rotate,
                    attention_fwd, attention_bwd, swiglu_fwd, swiglu_bwd, layer_fwd,
                    layer_bwd, ce_dense, ce_chunked, embedding_fwd, embedding_bwd,
                    ModelShape, model_loss_and_grads, LAYER_PARAM_NAMES)
from .adamw import (adamw_fp64, adamw_fp32, bf16_round_bits, bf16_bits_to_f32,
                    f16_round_bits, f16_bits_to_f32, AdamWHyper)

__all__ = [
    "LayerShape", "rmsnorm_fwd", "rmsnorm_bwd", "rope_tables", "rope_rotate",
    "attention_fwd", "attention_bwd", "swiglu_fwd", "swiglu_bwd", "layer_fwd", "layer_bwd",
    "ce_dense", "ce_chunked", "embedding_fwd", "embedding_bwd", "ModelShape",
    "model_loss_and_grads", "LAYER_PARAM_NAMES", "adamw_fp64", "adamw_fp32",
    "bf16_round_bits", "bf16_bits_to_f32", "f16_round_bits", "f16_bits_to_f32", "AdamWHyper",
]
