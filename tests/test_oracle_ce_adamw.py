"""Pins for the oracle's LM-head cross-entropy, whole-model step and AdamW against closed
forms, finite differences and torch CPU library routines."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import model as om
from oracle import adamw as oa


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)


def _ce_case(N=13, H=12, V=37, seed=0, ignore=True):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H))
    w = 0.5 * rng.standard_normal((V, H))
    t = rng.integers(0, V, N)
    if ignore:
        t[[1, N - 2]] = -1
    return h, w, t


def test_ce_zero_weights_gives_log_v():
    h, _, t = _ce_case()
    V = 37
    w = np.zeros((V, h.shape[1]))
    loss, dh, dw, lse = om.ce_dense(h, w, t)
    assert abs(loss - math.log(V)) < 1e-14
    assert np.all(dh == 0.0)
    valid = t >= 0
    dz = np.where(valid[:, None], np.full((len(t), V), 1.0 / V), 0.0)
    dz[np.nonzero(valid)[0], t[valid]] -= 1.0
    dz /= valid.sum()
    assert np.max(np.abs(dw - dz.T @ h)) < 1e-14


def test_ce_matches_torch_cross_entropy():
    h, w, t = _ce_case(seed=1)
    loss, dh, dw, lse = om.ce_dense(h, w, t)
    th = torch.from_numpy(h).requires_grad_()
    tw = torch.from_numpy(w).requires_grad_()
    tl = TF.cross_entropy(th @ tw.T, torch.from_numpy(t), ignore_index=-1, reduction="mean")
    tl.backward()
    assert abs(loss - tl.item()) < 1e-13
    assert _rel(dh, th.grad.numpy()) < 1e-12
    assert _rel(dw, tw.grad.numpy()) < 1e-12


@pytest.mark.parametrize("chunk", [1, 5, 8, 37, 64])
def test_chunked_equals_dense(chunk):
    h, w, t = _ce_case(seed=2)
    d = om.ce_dense(h, w, t)
    c = om.ce_chunked(h, w, t, chunk)
    assert abs(d[0] - c[0]) < 1e-12
    for a, b in zip(d[1:], c[1:]):
        assert np.max(np.abs(a - b)) < 1e-12


def test_ce_all_ignored_is_zero():
    h, w, t = _ce_case(seed=3)
    t[:] = -1
    for res in (om.ce_dense(h, w, t), om.ce_chunked(h, w, t, 8)):
        assert res[0] == 0.0 and np.all(res[1] == 0) and np.all(res[2] == 0)


def test_ce_central_differences():
    h, w, t = _ce_case(N=4, H=5, V=9, seed=4)
    loss, dh, dw, _ = om.ce_dense(h, w, t)
    eps = 1e-6
    for arr, g in ((h, dh), (w, dw)):
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            o = arr[i]
            arr[i] = o + eps
            lp = om.ce_dense(h, w, t)[0]
            arr[i] = o - eps
            lm = om.ce_dense(h, w, t)[0]
            arr[i] = o
            fd[i] = (lp - lm) / (2 * eps)
        assert _rel(g, fd) < 1e-7


def _tiny_model(seed=0):
    ls = om.LayerShape(8, 2, 1, 4, 12)
    shape = om.ModelShape(ls, n_layers=2, vocab=11)
    rng = np.random.default_rng(seed)

    def lp():
        return {n: (1.0 + 0.2 * rng.standard_normal(s)) if len(s) == 1
                else 0.4 * rng.standard_normal(s) for n, s in ls.param_shapes().items()}

    params = dict(embed=rng.standard_normal((11, 8)), layers=[lp(), lp()],
                  w_final=1.0 + 0.2 * rng.standard_normal(8),
                  lm_head=0.4 * rng.standard_normal((11, 8)))
    tok = rng.integers(0, 11, (2, 5))
    return shape, params, tok


def test_model_step_central_differences():
    shape, params, tok = _tiny_model()
    loss, grads = om.model_loss_and_grads(params, tok, shape)
    eps = 1e-6

    def check(arr, g):
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            o = arr[i]
            arr[i] = o + eps
            lp = om.model_loss_and_grads(params, tok, shape)[0]
            arr[i] = o - eps
            lm = om.model_loss_and_grads(params, tok, shape)[0]
            arr[i] = o
            fd[i] = (lp - lm) / (2 * eps)
        assert _rel(g, fd) < 1e-6

    check(params["embed"], grads["embed"])
    check(params["w_final"], grads["w_final"])
    check(params["lm_head"], grads["lm_head"])
    for li in range(2):
        for n in ("wqkv", "w_mlp"):
            check(params["layers"][li][n], grads["layers"][li][n])
    lc, gc = om.model_loss_and_grads(params, tok, shape, chunk=4)
    assert abs(lc - loss) < 1e-12
    assert np.max(np.abs(gc["embed"] - grads["embed"])) < 1e-12


def test_embedding_bwd_repeated_tokens():
    dx = np.arange(12, dtype=np.float64).reshape(1, 4, 3)
    tok = np.array([[2, 0, 2, 2]])
    de = om.embedding_bwd(dx, tok, 4)
    assert np.array_equal(de[2], dx[0, 0] + dx[0, 2] + dx[0, 3])
    assert np.array_equal(de[0], dx[0, 1])
    assert np.all(de[1] == 0) and np.all(de[3] == 0)


# ------------------------------------------------------------------------------- AdamW
HP = oa.AdamWHyper(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(0)
    p0 = rng.standard_normal(100)
    g = rng.standard_normal(100)
    p, m, v = oa.adamw_fp64(p0, g, np.zeros(100), np.zeros(100), 1, HP)
    ref = p0 * (1 - HP.lr * HP.weight_decay) - HP.lr * g / (np.abs(g) + HP.eps)
    assert np.max(np.abs(p - ref)) < 1e-15


def test_adamw_constant_gradient_and_zero_gradient_closed_forms():
    p0 = np.array([0.3, -1.2, 2.0])
    g = np.array([0.5, -2.0, 0.0])
    c = 1 - HP.lr * HP.weight_decay
    s = HP.lr * g / (np.abs(g) + HP.eps)
    p, m, v = p0.copy(), np.zeros(3), np.zeros(3)
    for t in range(1, 31):
        p, m, v = oa.adamw_fp64(p, g, m, v, t, HP)
        ref = p0 * c ** t - s * (1 - c ** t) / (1 - c)
        assert np.max(np.abs(p - ref)) < 1e-13
    assert abs(p[2] - p0[2] * c ** 30) < 1e-15


def test_adamw_fp32_contract_tracks_fp64():
    rng = np.random.default_rng(1)
    n = 10000
    p = rng.standard_normal(n).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    pd, md, vd = p.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        p, m, v, _ = oa.adamw_fp32(p, g, m, v, t, HP)
        pd, md, vd = oa.adamw_fp64(pd, g, md, vd, t, HP)
        assert np.max(np.abs(p - pd) / np.maximum(np.abs(pd), 1e-3)) < 2e-6
        assert _rel(m, md) < 1e-5
        assert _rel(v, vd) < 1e-5


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(5000).astype(np.float32) * 10.0 ** rng.integers(-40, 38, 5000),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45, -1e-45, 1.17e-38],
                 np.float32),
        # exact ties between two bf16 values: low 16 bits == 0x8000
        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ]).astype(np.float32)
    ours = oa.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = np.array([np.nan, -np.nan], np.float32)
    nb = oa.bf16_round_bits(nan)
    assert np.all(np.isnan(oa.bf16_bits_to_f32(nb))) and np.all(nb & 0x0040)
    assert np.array_equal(oa.bf16_bits_to_f32(ours[:5000]).view(np.uint32) & 0xFFFF,
                          np.zeros(5000, np.uint32))


def test_f16_rounding_matches_ieee_cases_and_torch():
    """binary16 round-to-nearest-even: hand-checked encodings (exact values, the halfway ties
    around 1, the largest finite value and the first value that rounds to infinity, the
    smallest subnormal), and agreement with torch's conversion over a wide sample."""
    cases = {1.0: 0x3C00, -2.0: 0xC000, 65504.0: 0x7BFF, 65520.0: 0x7C00, 2.0 ** -24: 0x0001,
             2.0 ** -14: 0x0400, 1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02,
             0.0: 0x0000, 1e-9: 0x0000}
    for x, bits in cases.items():
        assert int(oa.f16_round_bits(np.float32(x))) == bits, (x, hex(bits))
    assert float(oa.f16_bits_to_f32(np.uint16(0x3555))) == 0.333251953125
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oa.f16_round_bits(x), ref)


def test_adamw_loss_scaled_gradient_closed_form():
    """A gradient computed at loss scale S is unscaled before the update: at t = 1 from m = v = 0
    the step is p0 (1 - lr wd) - lr (g/S) / (|g/S| + eps), the same as the unscaled gradient's;
    with S a power of two the fp32 contract gives the unscaled result bit for bit."""
    hp = oa.AdamWHyper()
    rng = np.random.default_rng(4)
    p0 = rng.standard_normal(1000).astype(np.float32)
    g = (rng.standard_normal(1000) * 1e-3).astype(np.float32)
    S = 2.0 ** 16
    z = np.zeros(1000, np.float32)
    a = oa.adamw_fp32(p0, g, z, z, 1, hp)
    b = oa.adamw_fp32(p0, g * np.float32(S), z, z, 1, hp, grad_scale=S)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    ref = p0.astype(np.float64) * (1 - hp.lr * hp.weight_decay) - hp.lr * g / (np.abs(g) + hp.eps)
    assert np.max(np.abs(b[0] - ref)) <= 1e-6
    # the 16-bit copy in fp16
    assert np.array_equal(oa.adamw_fp32(p0, g, z, z, 1, hp, copy="f16")[3],
                          oa.f16_round_bits(a[0]))
