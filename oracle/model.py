"""fp64 reference of the decoder layer, the LM-head cross-entropy and the whole-model step.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product path imports it.

Sources and readings (the pages name the model family but never define the layer):
  * SlideFormer, gist.science summary, section 4: the system fine-tunes Llama-3, Qwen and
    Mistral with standard training objectives. Reading: the standard pre-norm Llama block,
    x2 = x + Attn(RMSNorm(x)), y = x2 + MLP(RMSNorm(x2)), no biases, no dropout, untied
    embedding and LM head, final RMSNorm before the LM head.
  * Same summary, section 2C: the optimised kernels are RoPE, RMSNorm and SwiGLU, and the
    projection plus loss is fused (LinearCrossEntropy). Readings: RMSNorm with a gain and
    eps inside the root; half-split ("rotate-half") RoPE with base theta and position s in
    [0, S) inside each sequence; SwiGLU m = silu(gate) * up; attention scaled by 1/sqrt(d),
    causal, query head h reads kv head h // (n_heads / n_kv_heads).
  * Loss: next-token cross-entropy, mean over valid targets (targets < 0 are ignored);
    if no target is valid the loss and all gradients are zero.
  * Chunked CE: vocabulary chunks [cC, min((c+1)C, V)) with the online max / sum-exp
    update s <- s*exp(m - m') + sum(exp(z - m')); equal to the dense CE in exact arithmetic.

Everything is computed in float64 from the given arrays; the only library primitive is the
matrix product (numpy @).
"""
from dataclasses import dataclass

import numpy as np

LAYER_PARAM_NAMES = ("w_attn", "wqkv", "wo", "w_mlp", "wgu", "wd")


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def qkv_rows(self):
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def param_shapes(self):
        H, F = self.hidden, self.ffn
        return {
            "w_attn": (H,),
            "wqkv": (self.qkv_rows, H),
            "wo": (H, self.n_heads * self.head_dim),
            "w_mlp": (H,),
            "wgu": (2 * F, H),
            "wd": (H, F),
        }


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------- RMSNorm
def rmsnorm_fwd(x, w, eps):
    """y = w * x * r with r = (mean_j x_j^2 + eps)^(-1/2), per row (last axis)."""
    x = _f64(x)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * _f64(w), r


def rmsnorm_bwd(dy, x, w, r):
    """Gradients of rmsnorm_fwd. With g = w*dy:
    dx = r*g - (r^3/H) * x * sum_j(g_j x_j);  dw = sum over rows of dy * x * r."""
    dy, x, w = _f64(dy), _f64(x), _f64(w)
    H = x.shape[-1]
    g = dy * w
    dx = r * g - (r ** 3 / H) * x * np.sum(g * x, axis=-1, keepdims=True)
    dw = np.sum((dy * x * r).reshape(-1, H), axis=0)
    return dx, dw


# ----------------------------------------------------------------------------- RoPE
def rope_tables(S, d, theta):
    """cos/sin of angle s * theta^(-2i/d) for positions s < S and pair index i < d/2."""
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / d)
    ang = np.arange(S, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope_rotate(x, cos, sin, inverse=False):
    """Rotate-half RoPE on x [B, S, heads, d]: pair (i, i + d/2) is turned by +angle
    (or -angle when inverse=True, which is the backward since the map is a rotation)."""
    x = _f64(x)
    h = x.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------- attention
def attention_fwd(q, k, v):
    """Causal grouped-query attention. q [B,S,nq,d]; k, v [B,S,nkv,d].
    Returns o [B,S,nq,d], lse [B,nq,S] and the probabilities P [B,nq,S,S] (for the bwd)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, nq, d = q.shape
    nkv = k.shape[2]
    G = nq // nkv
    scale = 1.0 / np.sqrt(d)
    future = np.triu(np.ones((S, S), dtype=bool), k=1)  # key j > query i is masked
    o = np.zeros_like(q)
    lse = np.zeros((B, nq, S))
    P = np.zeros((B, nq, S, S))
    for h in range(nq):
        qh = q[:, :, h, :]                      # [B,S,d]
        kh = k[:, :, h // G, :]
        vh = v[:, :, h // G, :]
        s = (qh @ kh.transpose(0, 2, 1)) * scale  # [B,S,S]
        s = np.where(future[None], -np.inf, s)
        m = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - m)
        l = np.sum(e, axis=-1, keepdims=True)
        p = e / l
        P[:, h] = p
        lse[:, h] = (m + np.log(l))[..., 0]
        o[:, :, h, :] = p @ vh
    return o, lse, P


def attention_bwd(do, q, k, v, P):
    """Backward of attention_fwd: dv = P^T do, dP = do v^T, dS = P*(dP - rowsum(dP*P)),
    dq = dS k / sqrt(d), dk = dS^T q / sqrt(d); dk and dv summed over each kv group."""
    do, q, k, v = _f64(do), _f64(q), _f64(k), _f64(v)
    B, S, nq, d = q.shape
    nkv = k.shape[2]
    G = nq // nkv
    scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(nq):
        p = P[:, h]
        doh = do[:, :, h, :]
        kh = k[:, :, h // G, :]
        vh = v[:, :, h // G, :]
        dv[:, :, h // G, :] += p.transpose(0, 2, 1) @ doh
        dp = doh @ vh.transpose(0, 2, 1)
        ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
        dq[:, :, h, :] = (ds @ kh) * scale
        dk[:, :, h // G, :] += (ds.transpose(0, 2, 1) @ q[:, :, h, :]) * scale
    return dq, dk, dv


# ----------------------------------------------------------------------------- SwiGLU
def _sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def swiglu_fwd(g, u):
    """m = silu(g) * u with silu(a) = a * sigmoid(a)."""
    g, u = _f64(g), _f64(u)
    return g * _sigmoid(g) * u


def swiglu_bwd(dm, g, u):
    """dg = dm * u * silu'(g) with silu'(a) = sig(a) * (1 + a*(1 - sig(a))); du = dm * silu(g)."""
    dm, g, u = _f64(dm), _f64(g), _f64(u)
    sg = _sigmoid(g)
    du = dm * g * sg
    dg = dm * u * sg * (1.0 + g * (1.0 - sg))
    return dg, du


# ----------------------------------------------------------------------------- layer
def layer_fwd(p, x, shape: LayerShape):
    """One pre-norm decoder layer on x [B,S,H]. p holds the parameters named in
    LAYER_PARAM_NAMES (y = x W^T for every matrix). Returns y and the cache for layer_bwd."""
    x = _f64(x)
    B, S, H = x.shape
    nq, nkv, d, F = shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn
    r, rr = rmsnorm_fwd(x, p["w_attn"], shape.eps)
    qkv = r @ _f64(p["wqkv"]).T
    q = qkv[..., : nq * d].reshape(B, S, nq, d)
    k = qkv[..., nq * d: (nq + nkv) * d].reshape(B, S, nkv, d)
    v = qkv[..., (nq + nkv) * d:].reshape(B, S, nkv, d)
    cos, sin = rope_tables(S, d, shape.rope_theta)
    qr = rope_rotate(q, cos, sin)
    kr = rope_rotate(k, cos, sin)
    o, lse, P = attention_fwd(qr, kr, v)
    o2 = o.reshape(B, S, nq * d)
    x2 = x + o2 @ _f64(p["wo"]).T
    r2, rr2 = rmsnorm_fwd(x2, p["w_mlp"], shape.eps)
    gu = r2 @ _f64(p["wgu"]).T
    g, u = gu[..., :F], gu[..., F:]
    m = swiglu_fwd(g, u)
    y = x2 + m @ _f64(p["wd"]).T
    cache = dict(x=x, r=r, rr=rr, qr=qr, kr=kr, v=v, o=o2, lse=lse, P=P, x2=x2, r2=r2,
                 rr2=rr2, g=g, u=u, m=m, cos=cos, sin=sin, qkv=qkv, gu=gu)
    return y, cache


def layer_bwd(p, dy, cache, shape: LayerShape):
    """Backward of layer_fwd. Returns dx [B,S,H] and a dict of parameter gradients."""
    dy = _f64(dy)
    c = cache
    B, S, H = dy.shape
    nq, nkv, d = shape.n_heads, shape.n_kv_heads, shape.head_dim
    N = B * S
    wd, wgu, wo, wqkv = (_f64(p[k]) for k in ("wd", "wgu", "wo", "wqkv"))
    grads = {}
    # MLP half: y = x2 + m Wd^T
    dm = dy @ wd
    grads["wd"] = dy.reshape(N, H).T @ c["m"].reshape(N, -1)
    dg, du = swiglu_bwd(dm, c["g"], c["u"])
    dgu = np.concatenate([dg, du], axis=-1)
    dr2 = dgu @ wgu
    grads["wgu"] = dgu.reshape(N, -1).T @ c["r2"].reshape(N, H)
    dx2n, grads["w_mlp"] = rmsnorm_bwd(dr2, c["x2"], p["w_mlp"], c["rr2"])
    dx2 = dy + dx2n
    # attention half: x2 = x + o Wo^T
    do = dx2 @ wo
    grads["wo"] = dx2.reshape(N, H).T @ c["o"].reshape(N, -1)
    dqr, dkr, dv = attention_bwd(do.reshape(B, S, nq, d), c["qr"], c["kr"], c["v"], c["P"])
    dq = rope_rotate(dqr, c["cos"], c["sin"], inverse=True)
    dk = rope_rotate(dkr, c["cos"], c["sin"], inverse=True)
    dqkv = np.concatenate([dq.reshape(B, S, -1), dk.reshape(B, S, -1), dv.reshape(B, S, -1)],
                          axis=-1)
    dr = dqkv @ wqkv
    grads["wqkv"] = dqkv.reshape(N, -1).T @ c["r"].reshape(N, H)
    dxn, grads["w_attn"] = rmsnorm_bwd(dr, c["x"], p["w_attn"], c["rr"])
    dx = dx2 + dxn
    return dx, grads


# ----------------------------------------------------------------------------- LM head CE
def ce_dense(h, w, targets):
    """Cross-entropy of logits z = h W^T. h [N,H], w [V,H], targets [N] (negative = ignored).
    Returns (loss, dh, dw, lse) with loss the mean over valid targets."""
    h, w = _f64(h), _f64(w)
    t = np.asarray(targets).astype(np.int64)
    N, V = h.shape[0], w.shape[0]
    valid = t >= 0
    nv = int(valid.sum())
    z = h @ w.T
    m = np.max(z, axis=1, keepdims=True)
    lse = (m + np.log(np.sum(np.exp(z - m), axis=1, keepdims=True)))[:, 0]
    if nv == 0:
        return 0.0, np.zeros_like(h), np.zeros_like(w), lse
    rows = np.nonzero(valid)[0]
    loss = float(np.sum(lse[rows] - z[rows, t[rows]]) / nv)
    dz = np.exp(z - lse[:, None])
    dz[rows, t[rows]] -= 1.0
    dz *= valid[:, None] / nv
    return loss, dz @ w, dz.T @ h, lse


def ce_chunked(h, w, targets, chunk):
    """The same loss and gradients, computed over vocabulary chunks [cC, min((c+1)C, V))
    with the online max / sum-exp update; the gradient pass recomputes each chunk's logits."""
    h, w = _f64(h), _f64(w)
    t = np.asarray(targets).astype(np.int64)
    N, V = h.shape[0], w.shape[0]
    valid = t >= 0
    nv = int(valid.sum())
    m = np.full(N, -np.inf)
    s = np.zeros(N)
    zt = np.zeros(N)
    for c0 in range(0, V, chunk):
        c1 = min(c0 + chunk, V)
        z = h @ w[c0:c1].T
        m_new = np.maximum(m, np.max(z, axis=1))
        s = s * np.exp(m - m_new) + np.sum(np.exp(z - m_new[:, None]), axis=1)
        m = m_new
        inside = valid & (t >= c0) & (t < c1)
        zt[inside] = z[inside, t[inside] - c0]
    lse = m + np.log(s)
    if nv == 0:
        return 0.0, np.zeros_like(h), np.zeros_like(w), lse
    loss = float(np.sum((lse - zt)[valid]) / nv)
    dh = np.zeros_like(h)
    dw = np.zeros_like(w)
    for c0 in range(0, V, chunk):
        c1 = min(c0 + chunk, V)
        z = h @ w[c0:c1].T
        dz = np.exp(z - lse[:, None])
        inside = valid & (t >= c0) & (t < c1)
        dz[inside, t[inside] - c0] -= 1.0
        dz *= valid[:, None] / nv
        dh += dz @ w[c0:c1]
        dw[c0:c1] = dz.T @ h
    return loss, dh, dw, lse


# ----------------------------------------------------------------------------- embedding
def embedding_fwd(e, tokens):
    return _f64(e)[np.asarray(tokens)]


def embedding_bwd(dx, tokens, vocab):
    """dE[v] = sum of dx over the positions whose token is v."""
    dx = _f64(dx)
    H = dx.shape[-1]
    de = np.zeros((vocab, H))
    np.add.at(de, np.asarray(tokens).reshape(-1), dx.reshape(-1, H))
    return de


# ----------------------------------------------------------------------------- whole model
@dataclass(frozen=True)
class ModelShape:
    layer: LayerShape
    n_layers: int
    vocab: int


def model_loss_and_grads(params, tokens, shape: ModelShape, chunk=None):
    """Loss and gradients of one step. params: {"embed": [V,H], "layers": [dict, ...],
    "w_final": [H], "lm_head": [V,H]}; tokens int [B, S+1]: inputs tokens[:, :S],
    targets tokens[:, 1:]. Returns (loss, grads) with grads shaped like params."""
    tok = np.asarray(tokens)
    inp, tgt = tok[:, :-1], tok[:, 1:]
    B, S = inp.shape
    H = shape.layer.hidden
    x = embedding_fwd(params["embed"], inp)
    caches = []
    for lp in params["layers"]:
        x, cache = layer_fwd(lp, x, shape.layer)
        caches.append(cache)
    hf, rf = rmsnorm_fwd(x, params["w_final"], shape.layer.eps)
    if chunk is None:
        loss, dhf, dlm, _ = ce_dense(hf.reshape(B * S, H), params["lm_head"], tgt.reshape(-1))
    else:
        loss, dhf, dlm, _ = ce_chunked(hf.reshape(B * S, H), params["lm_head"],
                                       tgt.reshape(-1), chunk)
    dx, dwf = rmsnorm_bwd(dhf.reshape(B, S, H), x, params["w_final"], rf)
    layer_grads = [None] * len(params["layers"])
    for i in range(len(params["layers"]) - 1, -1, -1):
        dx, layer_grads[i] = layer_bwd(params["layers"][i], dx, caches[i], shape.layer)
    de = embedding_bwd(dx, inp, shape.vocab)
    return loss, {"embed": de, "layers": layer_grads, "w_final": dwf, "lm_head": dlm}
