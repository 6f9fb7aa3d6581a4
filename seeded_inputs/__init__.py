"""Seeded synthetic inputs shared by the HIP path's tests, the oracle's tests and the benchmark.

This module holds workload shapes and random draws only: none of the method's arithmetic.
Every array is drawn with numpy.random.default_rng(seed) (PCG64) so that the oracle and the
HIP path consume exactly the same values. bf16 inputs are produced by rounding the fp32 draw
with torch's CPU conversion (round to nearest-even) and are handed over as uint16 bit
patterns together with their exact fp32 widening.

Workloads (SlideFormer pages: Llama-3-class full fine-tuning on one GPU; the shapes below are
the standard Llama-3-8B layer and a 123B-class layer, plus a tiny fp32 decoder):
  tiny   2 layers, hidden 256, 4 heads x 64 (no GQA), SwiGLU 688, vocab 1024, batch 2 x 128, fp32
  8b     32 layers, hidden 4096, 32 q / 8 kv heads x 128, SwiGLU 14336, vocab 128256,
         batch 8 x 1024, bf16 compute / fp32 master, 3-slot HBM ring
  ce     hidden 4096, 16384 tokens, vocab 128256, vocabulary chunks of 8192
  123b   hidden 12288, 96 q / 8 kv heads x 128, SwiGLU 28672, vocab 32768, batch 4 x 2048
Weights: matrices N(0, 0.02); RMSNorm gains 1 (optionally 1 + N(0, gain_std) for tests that
must see the gain). Tokens: uniform integers in [0, V).
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class LayerCfg:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def qkv_rows(self):
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def param_shapes(self):
        """Slot packing order: w_attn | Wqkv | Wo | w_mlp | Wgu | Wd (row-major [out, in])."""
        H, F = self.hidden, self.ffn
        return [("w_attn", (H,)), ("wqkv", (self.qkv_rows, H)),
                ("wo", (H, self.n_heads * self.head_dim)), ("w_mlp", (H,)),
                ("wgu", (2 * F, H)), ("wd", (H, F))]

    def param_count(self):
        return int(sum(np.prod(s) for _, s in self.param_shapes()))


@dataclass(frozen=True)
class Workload:
    name: str
    layer: LayerCfg
    n_layers: int
    vocab: int
    batch: int
    seq: int
    dtype: str            # "f32" or "bf16"
    ce_chunk: int = 8192
    ring_slots: int = 3


TINY = Workload("tiny-llama-fp32", LayerCfg(256, 4, 4, 64, 688), 2, 1024, 2, 128, "f32")
L8B = Workload("llama3-8b-shaped", LayerCfg(4096, 32, 8, 128, 14336), 32, 128256, 8, 1024,
               "bf16")
L123B = Workload("123b-shaped-slice", LayerCfg(12288, 96, 8, 128, 28672), 12, 32768, 4, 2048,
                 "bf16")
CE_ONLY = dict(name="lmhead-ce-128k", hidden=4096, tokens=16384, vocab=128256, chunk=8192)
WORKLOADS = {w.name: w for w in (TINY, L8B, L123B)}


def to_bf16_bits(a):
    """Round fp32 values to bf16 with torch's CPU conversion; returns uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_as_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """A seeded input: fp32 values (exact widening when dtype is bf16) and, for bf16, the bits."""
    f32: np.ndarray
    bits: np.ndarray = None

    @property
    def f64(self):
        return self.f32.astype(np.float64)


def _finish(a, dtype):
    a = np.asarray(a, np.float32)
    if dtype == "bf16":
        bits = to_bf16_bits(a)
        return Tensor(bf16_bits_as_f32(bits), bits)
    if dtype == "f16":     # IEEE binary16, round to nearest-even (NumPy's conversion)
        h = a.astype(np.float16)
        return Tensor(h.astype(np.float32), h.view(np.uint16))
    return Tensor(a)


def draw_layer(rng, cfg: LayerCfg, dtype, std=0.02, gain_std=0.0):
    """One layer's parameters in packing order from an existing generator."""
    out = {}
    for name, shape in cfg.param_shapes():
        if len(shape) == 1:
            a = np.ones(shape, np.float32)
            if gain_std:
                a = a + rng.standard_normal(shape, dtype=np.float32) * np.float32(gain_std)
        else:
            a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        out[name] = _finish(a, dtype)
    return out


def layer_params(cfg: LayerCfg, dtype, seed=0, std=0.02, gain_std=0.0):
    return draw_layer(np.random.default_rng(seed), cfg, dtype, std, gain_std)


def pack_layer(params, cfg: LayerCfg, dtype):
    """Concatenate one layer's parameters in slot packing order (flat array)."""
    parts = [(params[n].bits if dtype in ("bf16", "f16") else params[n].f32).reshape(-1)
             for n, _ in cfg.param_shapes()]
    return np.concatenate(parts)


def model_params(w: Workload, seed=0, std=0.02, gain_std=0.0):
    """Whole-model parameters drawn in order: embedding, each layer, final gain, LM head."""
    rng = np.random.default_rng(seed)
    H, V = w.layer.hidden, w.vocab
    embed = _finish(rng.standard_normal((V, H), dtype=np.float32) * np.float32(std), w.dtype)
    layers = [draw_layer(rng, w.layer, w.dtype, std, gain_std) for _ in range(w.n_layers)]
    g = np.ones(H, np.float32)
    if gain_std:
        g = g + rng.standard_normal(H, dtype=np.float32) * np.float32(gain_std)
    w_final = _finish(g, w.dtype)
    lm = _finish(rng.standard_normal((V, H), dtype=np.float32) * np.float32(std), w.dtype)
    return dict(embed=embed, layers=layers, w_final=w_final, lm_head=lm)


def tokens(batch, seq, vocab, seed=1):
    """Uniform int32 tokens [batch, seq+1]: inputs are [:, :seq], next-token targets [:, 1:]."""
    return np.random.default_rng(seed).integers(0, vocab, (batch, seq + 1), dtype=np.int32)


def activations(shape, dtype, seed, std=1.0):
    """N(0, std) activations (e.g. a layer input or an upstream gradient)."""
    rng = np.random.default_rng(seed)
    return _finish(rng.standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)


def ce_inputs(n_tokens, hidden, vocab, dtype="bf16", seed_h=2, seed_t=3, w_seed=4,
              std=0.02, ignore_frac=0.0):
    """LM-head CE inputs: h ~ N(0,1) [N,H], W ~ N(0, std) [V,H], uniform int32 targets
    (a fraction ignore_frac of them set to -1, i.e. ignored)."""
    h = activations((n_tokens, hidden), dtype, seed_h)
    w = _finish(np.random.default_rng(w_seed).standard_normal((vocab, hidden), dtype=np.float32)
                * np.float32(std), dtype)
    rng = np.random.default_rng(seed_t)
    t = rng.integers(0, vocab, n_tokens, dtype=np.int32)
    if ignore_frac:
        t[rng.random(n_tokens) < ignore_frac] = -1
    return h, w, t
