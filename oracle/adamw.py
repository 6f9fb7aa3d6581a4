"""AdamW for the host-side per-layer optimizer (SlideFormer's "Layer-Adam": optimizer state in
host memory, updated on the CPU layer by layer while the GPU runs the next layer's backward;
gist.science summary, sections 2A and 2B; abstract).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings (the pages name only "Layer-Adam"): decoupled weight decay (Loshchilov & Hutter)
applied uniformly to every parameter, bias correction on, step t starting at 1, eps 1e-8,
no gradient clipping (a global-norm clip needs every gradient before any update, which the
per-layer overlap rules out).

Two forms:
  adamw_fp64  the textbook update in float64;
  adamw_fp32  a fixed float32 operation order (every op rounded to nearest-even, no fused
              multiply-add) that a native implementation can match bit for bit:
                scalars, computed in double and cast once to float32:
                  b1t = b1^t, b2t = b2^t (t repeated double multiplications from 1.0),
                  c_dec = 1 - lr*wd, c_b1 = b1, c_1b1 = 1 - b1, c_b2 = b2, c_1b2 = 1 - b2,
                  c_step = lr / (1 - b1t), c_bc2 = sqrt(1 - b2t), c_eps = eps
                per element, in float32:
                  p1  = p * c_dec
                  m'  = (c_b1 * m) + (c_1b1 * g)
                  v'  = (c_b2 * v) + (c_1b2 * (g * g))
                  den = (sqrt(v') / c_bc2) + c_eps
                  p'  = p1 - c_step * (m' / den)
              plus the bf16 (or fp16) copy of p' rounded to nearest-even (NaN -> quiet NaN),
              which is the FP32 -> BF16/FP16 conversion the summary places in the shared host
              buffers (section 2B). With loss scaling (fp16 training) the gradient is first
              multiplied by float32(1 / scale).
The two agree to about 1e-6 relative (pinned in the tests).
"""
from dataclasses import dataclass
import math

import numpy as np


@dataclass(frozen=True)
class AdamWHyper:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def adamw_fp64(p, g, m, v, t, hp: AdamWHyper):
    """Textbook decoupled AdamW step t (t >= 1) in float64. Returns new (p, m, v)."""
    p, g, m, v = (np.asarray(a, np.float64) for a in (p, g, m, v))
    p = p * (1.0 - hp.lr * hp.weight_decay)
    m = hp.beta1 * m + (1.0 - hp.beta1) * g
    v = hp.beta2 * v + (1.0 - hp.beta2) * g * g
    mhat = m / (1.0 - hp.beta1 ** t)
    vhat = v / (1.0 - hp.beta2 ** t)
    p = p - hp.lr * mhat / (np.sqrt(vhat) + hp.eps)
    return p, m, v


def _scalars_fp32(t, hp: AdamWHyper):
    b1t = 1.0
    b2t = 1.0
    for _ in range(int(t)):
        b1t *= hp.beta1
        b2t *= hp.beta2
    f = np.float32
    return dict(
        c_dec=f(1.0 - hp.lr * hp.weight_decay),
        c_b1=f(hp.beta1), c_1b1=f(1.0 - hp.beta1),
        c_b2=f(hp.beta2), c_1b2=f(1.0 - hp.beta2),
        c_step=f(hp.lr / (1.0 - b1t)),
        c_bc2=f(math.sqrt(1.0 - b2t)),
        c_eps=f(hp.eps),
    )


def adamw_fp32(p, g, m, v, t, hp: AdamWHyper, grad_scale=1.0, copy="bf16"):
    """The fixed-order float32 AdamW step. p, g, m, v: float32 arrays (g may be any float
    array exactly representable in float32, e.g. widened bf16 or fp16). grad_scale: the loss
    scale the gradient carries (dynamic loss scaling): g is first multiplied by
    float32(1 / grad_scale), unless grad_scale is 0 or 1. Returns new (p, m, v, copy_bits) with
    the 16-bit copy of p ("bf16" or "f16", round to nearest-even) as uint16 bit patterns."""
    c = _scalars_fp32(t, hp)
    f32 = np.float32
    p = np.asarray(p, f32)
    g = np.asarray(g, f32)
    m = np.asarray(m, f32)
    v = np.asarray(v, f32)
    with np.errstate(all="ignore"):
        if grad_scale not in (0, 1, 0.0, 1.0):
            g = g * f32(1.0 / grad_scale)
        p1 = p * c["c_dec"]
        m2 = (c["c_b1"] * m) + (c["c_1b1"] * g)
        v2 = (c["c_b2"] * v) + (c["c_1b2"] * (g * g))
        den = (np.sqrt(v2) / c["c_bc2"]) + c["c_eps"]
        p2 = p1 - c["c_step"] * (m2 / den)
    bits = f16_round_bits(p2) if copy == "f16" else bf16_round_bits(p2)
    return p2.astype(f32), m2.astype(f32), v2.astype(f32), bits


def bf16_round_bits(x):
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even; NaN becomes a
    quiet NaN with its sign kept. Written from the IEEE-754 binary32 layout: bf16 keeps the
    top 16 bits, so round the discarded low half."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    is_nan = ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)
    lsb = (b >> 16) & 1
    rounded = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    quiet = ((b >> 16) | 0x0040) & 0xFFFF
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def f16_round_bits(x):
    """float32 -> IEEE binary16 bit pattern (uint16), round to nearest, ties to even, overflow
    to infinity (NumPy's float16 conversion, which implements the IEEE-754 rounding)."""
    with np.errstate(all="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits):
    """Exact widening of binary16 bit patterns to float32."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
