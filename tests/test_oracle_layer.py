"""Pins for the oracle's decoder layer (oracle/model.py) against mathematics and library
routines: central finite differences for every gradient, closed forms, invariants, and
torch CPU reference routines (rms_norm, scaled_dot_product_attention, silu, linear)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import model as om

SH = om.LayerShape(hidden=16, n_heads=2, n_kv_heads=1, head_dim=8, ffn=40, eps=1e-5,
                   rope_theta=10000.0)


def _params(shape, seed=0, std=0.3, gain_std=0.2):
    rng = np.random.default_rng(seed)
    p = {}
    for n, s in shape.param_shapes().items():
        if len(s) == 1:
            p[n] = 1.0 + gain_std * rng.standard_normal(s)
        else:
            p[n] = std * rng.standard_normal(s)
    return p


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)


def _loss(p, x, c, shape):
    y, _ = om.layer_fwd(p, x, shape)
    return float(np.sum(y * c))


@pytest.mark.parametrize("shape", [SH, om.LayerShape(16, 2, 2, 8, 24)])
def test_layer_grads_match_central_differences(shape):
    B, S = 1, 5
    rng = np.random.default_rng(1)
    p = _params(shape)
    x = rng.standard_normal((B, S, shape.hidden))
    c = rng.standard_normal((B, S, shape.hidden))
    y, cache = om.layer_fwd(p, x, shape)
    dx, grads = om.layer_bwd(p, c, cache, shape)
    eps = 1e-6
    fd = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        fd[i] = (_loss(p, xp, c, shape) - _loss(p, xm, c, shape)) / (2 * eps)
    assert _rel(dx, fd) < 1e-6
    for name in om.LAYER_PARAM_NAMES:
        w = p[name]
        fdw = np.zeros_like(w)
        for i in np.ndindex(w.shape):
            orig = w[i]
            w[i] = orig + eps
            lp = _loss(p, x, c, shape)
            w[i] = orig - eps
            lm = _loss(p, x, c, shape)
            w[i] = orig
            fdw[i] = (lp - lm) / (2 * eps)
        assert _rel(grads[name], fdw) < 1e-6, name


def test_causal_no_gradient_from_future_tokens():
    B, S = 2, 7
    rng = np.random.default_rng(2)
    p = _params(SH)
    x = rng.standard_normal((B, S, SH.hidden))
    y, cache = om.layer_fwd(p, x, SH)
    for t_star in range(S - 1):
        c = rng.standard_normal(y.shape)
        c[:, t_star + 1:] = 0.0          # loss only reads outputs at positions <= t_star
        dx, _ = om.layer_bwd(p, c, cache, SH)
        assert np.all(dx[:, t_star + 1:] == 0.0)
        assert np.any(dx[:, : t_star + 1] != 0.0)


def test_attention_rows_sum_to_one_and_equal_keys_average_prefix():
    rng = np.random.default_rng(3)
    B, S, nq, nkv, d = 2, 9, 4, 2, 8
    q = rng.standard_normal((B, S, nq, d))
    k = rng.standard_normal((B, S, nkv, d))
    v = rng.standard_normal((B, S, nkv, d))
    o, lse, P = om.attention_fwd(q, k, v)
    assert np.max(np.abs(P.sum(-1) - 1.0)) < 1e-12
    assert np.all(np.triu(P[0, 0], 1) == 0.0)
    # identical keys: every visible key has the same score, so o_i is the mean of v_0..v_i
    k_eq = np.broadcast_to(rng.standard_normal((1, 1, nkv, d)), k.shape).copy()
    o2, _, _ = om.attention_fwd(q, k_eq, v)
    G = nq // nkv
    for h in range(nq):
        prefix_mean = np.cumsum(v[:, :, h // G], axis=1) / np.arange(1, S + 1)[None, :, None]
        assert np.max(np.abs(o2[:, :, h] - prefix_mean)) < 1e-12
    # S = 1: the only key is the query's own, so o = v
    o1, _, _ = om.attention_fwd(q[:, :1], k[:, :1], v[:, :1])
    assert np.max(np.abs(o1 - np.repeat(v[:, :1], G, axis=2))) < 1e-12


def test_attention_matches_torch_sdpa_and_lse():
    rng = np.random.default_rng(4)
    B, S, nq, nkv, d = 2, 11, 6, 2, 16
    q = rng.standard_normal((B, S, nq, d))
    k = rng.standard_normal((B, S, nkv, d))
    v = rng.standard_normal((B, S, nkv, d))
    o, lse, _ = om.attention_fwd(q, k, v)
    G = nq // nkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, G, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, G, axis=2)).permute(0, 2, 1, 3)
    ref = TF.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(0, 2, 1, 3)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12
    s = (tq @ tk.transpose(-1, -2)) / np.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, -1).numpy())) < 1e-12


def test_gqa_equals_mha_with_replicated_kv_weights():
    g_shape = om.LayerShape(16, 4, 2, 4, 24)
    m_shape = om.LayerShape(16, 4, 4, 4, 24)
    rng = np.random.default_rng(5)
    p = _params(g_shape)
    nq, d = 4, 4
    wq = p["wqkv"][: nq * d]
    wk = p["wqkv"][nq * d: nq * d + 2 * d].reshape(2, d, 16)
    wv = p["wqkv"][nq * d + 2 * d:].reshape(2, d, 16)
    pm = dict(p)
    pm["wqkv"] = np.concatenate([wq, np.repeat(wk, 2, axis=0).reshape(-1, 16),
                                 np.repeat(wv, 2, axis=0).reshape(-1, 16)])
    x = rng.standard_normal((2, 6, 16))
    yg, _ = om.layer_fwd(p, x, g_shape)
    ym, _ = om.layer_fwd(pm, x, m_shape)
    assert np.max(np.abs(yg - ym)) < 1e-12


def test_rope_identity_norms_relative_and_complex_form():
    rng = np.random.default_rng(6)
    B, S, h, d = 1, 12, 3, 16
    x = rng.standard_normal((B, S, h, d))
    cos, sin = om.rope_tables(S, d, 10000.0)
    y = om.rope_rotate(x, cos, sin)
    assert np.array_equal(y[:, 0], x[:, 0])                          # position 0
    n_in = x[..., : d // 2] ** 2 + x[..., d // 2:] ** 2
    n_out = y[..., : d // 2] ** 2 + y[..., d // 2:] ** 2
    assert np.max(np.abs(n_in - n_out)) < 1e-12                      # pair norms kept
    assert np.max(np.abs(om.rope_rotate(y, cos, sin, inverse=True) - x)) < 1e-12
    # pair (i, i+d/2) as the complex number x_i + j x_{i+d/2}, times exp(j * s * theta_i)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    s = np.arange(S)[None, :, None, None]
    th = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    zr = z * np.exp(1j * s * th)
    assert np.max(np.abs(np.concatenate([zr.real, zr.imag], -1) - y)) < 1e-12
    # relative position: <R_m q, R_n k> depends on n - m only
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    cos2, sin2 = om.rope_tables(40, d, 10000.0)
    X = np.zeros((1, 40, 2, d))
    X[0, :, 0] = q
    X[0, :, 1] = k
    R = om.rope_rotate(X, cos2, sin2)
    for m, n, c in [(2, 7, 5), (0, 3, 30), (9, 1, 11)]:
        a = R[0, m, 0] @ R[0, n, 1]
        b = R[0, m + c, 0] @ R[0, n + c, 1]
        assert abs(a - b) < 1e-12


def test_rmsnorm_constant_row_and_torch():
    H = 32
    w = np.linspace(0.5, 1.5, H)
    for cval in (0.0, 1e-3, 2.5, -7.0):
        y, _ = om.rmsnorm_fwd(np.full((1, H), cval), w, 1e-5)
        assert np.max(np.abs(y - w * cval / np.sqrt(cval * cval + 1e-5))) < 1e-14
    x = np.random.default_rng(7).standard_normal((5, H))
    y, _ = om.rmsnorm_fwd(x, w, 1e-5)
    ref = TF.rms_norm(torch.from_numpy(x), (H,), torch.from_numpy(w), eps=1e-5).numpy()
    assert np.max(np.abs(y - ref)) < 1e-13


def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(8)
    g = rng.standard_normal(1000) * 6
    u = rng.standard_normal(1000)
    ref = (TF.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.max(np.abs(om.swiglu_fwd(g, u) - ref)) < 1e-13
    tg = torch.from_numpy(g).requires_grad_()
    tu = torch.from_numpy(u).requires_grad_()
    dm = rng.standard_normal(1000)
    (TF.silu(tg) * tu).backward(torch.from_numpy(dm))
    dg, du = om.swiglu_bwd(dm, g, u)
    assert np.max(np.abs(dg - tg.grad.numpy())) < 1e-13
    assert np.max(np.abs(du - tu.grad.numpy())) < 1e-13


def _torch_layer(p, x, shape):
    """The same block assembled from torch library routines (autograd gives its gradients)."""
    B, S, H = x.shape
    nq, nkv, d, F = shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn
    r = TF.rms_norm(x, (H,), p["w_attn"], eps=shape.eps)
    qkv = TF.linear(r, p["wqkv"])
    q = qkv[..., : nq * d].reshape(B, S, nq, d)
    k = qkv[..., nq * d: (nq + nkv) * d].reshape(B, S, nkv, d)
    v = qkv[..., (nq + nkv) * d:].reshape(B, S, nkv, d)
    pos = torch.arange(S, dtype=torch.float64)
    th = shape.rope_theta ** (-torch.arange(d // 2, dtype=torch.float64) * 2.0 / d)
    rot = torch.polar(torch.ones(S, d // 2, dtype=torch.float64), pos[:, None] * th[None])

    def rope(t):
        zc = torch.complex(t[..., : d // 2], t[..., d // 2:]) * rot[None, :, None, :]
        return torch.cat([zc.real, zc.imag], -1)

    q, k = rope(q), rope(k)
    G = nq // nkv
    k = k.repeat_interleave(G, dim=2)
    v = v.repeat_interleave(G, dim=2)
    o = TF.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                        is_causal=True).transpose(1, 2).reshape(B, S, nq * d)
    x2 = x + TF.linear(o, p["wo"])
    r2 = TF.rms_norm(x2, (H,), p["w_mlp"], eps=shape.eps)
    gu = TF.linear(r2, p["wgu"])
    return x2 + TF.linear(TF.silu(gu[..., :F]) * gu[..., F:], p["wd"])


def test_layer_matches_torch_composition():
    shape = om.LayerShape(32, 4, 2, 8, 48)
    p = _params(shape, seed=9)
    rng = np.random.default_rng(10)
    x = rng.standard_normal((2, 9, 32))
    c = rng.standard_normal((2, 9, 32))
    y, cache = om.layer_fwd(p, x, shape)
    dx, grads = om.layer_bwd(p, c, cache, shape)
    tp = {n: torch.from_numpy(v.copy()).requires_grad_() for n, v in p.items()}
    tx = torch.from_numpy(x).requires_grad_()
    ty = _torch_layer(tp, tx, shape)
    ty.backward(torch.from_numpy(c))
    assert _rel(y, ty.detach().numpy()) < 1e-12
    assert _rel(dx, tx.grad.numpy()) < 1e-11
    for n in om.LAYER_PARAM_NAMES:
        assert _rel(grads[n], tp[n].grad.numpy()) < 1e-11, n
