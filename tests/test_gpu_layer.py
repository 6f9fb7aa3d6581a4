"""GPU parity of slide_layer_fwd / slide_layer_bwd and slide_lmhead_ce against the fp64 oracle,
through the C ABI, on seeded inputs."""
import numpy as np
import pytest
import torch

import layer_sliding_offloaded_fwd_amd as sl
from oracle import model as om
from seeded_inputs import LayerCfg, TINY, activations, ce_inputs, layer_params, pack_layer
from tests._gpu import DEV, assert_close, dev, empty, host, rel_err, stream, ws

pytestmark = pytest.mark.gpu


def _oracle_shape(c: LayerCfg):
    return om.LayerShape(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, c.rms_eps,
                         c.rope_theta)


_TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _packed_to_device(params, c, dtype):
    flat = pack_layer(params, c, dtype)
    t = torch.from_numpy(flat.view(np.int16) if dtype != "f32" else flat).to(DEV)
    return t.view(_TDT[dtype]) if dtype != "f32" else t


def _unpack(g, c):
    out, o = {}, 0
    for name, shape in c.param_shapes():
        n = int(np.prod(shape))
        out[name] = g[o:o + n].reshape(shape)
        o += n
    return out


CASES = [
    ("tiny-fp32", TINY.layer, "f32", 2, 128, 0.0),
    ("bf16-gqa-ragged", LayerCfg(512, 8, 2, 64, 1376), "bf16", 2, 200, 0.1),
    ("bf16-d128", LayerCfg(1024, 8, 4, 128, 2816), "bf16", 1, 256, 0.1),
    ("f16-gqa-ragged", LayerCfg(512, 8, 2, 64, 1376), "f16", 2, 200, 0.1),
    ("f16-d128", LayerCfg(1024, 8, 4, 128, 2816), "f16", 1, 256, 0.1),
]


@pytest.mark.parametrize("name,c,dtype,B,S,gain_std", CASES, ids=[c[0] for c in CASES])
def test_layer_fwd_bwd_matches_oracle(name, c, dtype, B, S, gain_std):
    print(f"layer {name}: H={c.hidden} nq={c.n_heads} nkv={c.n_kv_heads} d={c.head_dim} "
          f"F={c.ffn} B={B} S={S} {dtype}", flush=True)
    N = B * S
    params = layer_params(c, dtype, seed=0, gain_std=gain_std)
    x = activations((N, c.hidden), dtype, 1)
    dy = activations((N, c.hidden), dtype, 2)
    cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, dtype, c.rms_eps,
                       c.rope_theta)
    w = _packed_to_device(params, c, dtype)
    tx, tdy = dev(x.f32, dtype), dev(dy.f32, dtype)
    y = empty((N, c.hidden), dtype)
    wf = sl.slide_layer_workspace_bytes(cfg, B, S, 0)
    sl.slide_layer_fwd(cfg, w, tx, y, B, S, ws(wf), wf, stream())
    dx = empty((N, c.hidden), dtype)
    g = torch.full_like(w, float("nan"))
    wb = sl.slide_layer_workspace_bytes(cfg, B, S, 1)
    sl.slide_layer_bwd(cfg, w, tx, tdy, dx, g, B, S, ws(wb), wb, stream())
    torch.cuda.synchronize()

    shape = _oracle_shape(c)
    p64 = {k: v.f64 for k, v in params.items()}
    ry, cache = om.layer_fwd(p64, x.f64.reshape(B, S, -1), shape)
    rdx, rg = om.layer_bwd(p64, dy.f64.reshape(B, S, -1), cache, shape)
    assert_close(host(y).reshape(B, S, -1), ry, dtype, "layer y")
    assert_close(host(dx).reshape(B, S, -1), rdx, dtype, "layer dx")
    gg = _unpack(host(g), c)
    for n in om.LAYER_PARAM_NAMES:
        assert_close(gg[n], rg[n], dtype, f"grad {n}")


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_saved_intermediates_give_identical_results(dtype):
    c, B, S = (LayerCfg(512, 8, 2, 64, 1376), 2, 200) if dtype != "f32" else (TINY.layer, 2, 128)
    print(f"layer fwd_save / bwd_saved vs recompute, {dtype}", flush=True)
    N = B * S
    params = layer_params(c, dtype, seed=7, gain_std=0.1)
    x = activations((N, c.hidden), dtype, 8)
    dy = activations((N, c.hidden), dtype, 9)
    cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, dtype)
    w = _packed_to_device(params, c, dtype)
    tx, tdy = dev(x.f32, dtype), dev(dy.f32, dtype)
    wb = sl.slide_layer_workspace_bytes(cfg, B, S, 1)
    y1, dx1, g1 = empty((N, c.hidden), dtype), empty((N, c.hidden), dtype), torch.empty_like(w)
    sl.slide_layer_fwd(cfg, w, tx, y1, B, S, ws(wb), wb, stream())
    sl.slide_layer_bwd(cfg, w, tx, tdy, dx1, g1, B, S, ws(wb), wb, stream())
    sb = sl.slide_layer_saved_bytes(cfg, B, S)
    w2 = sl.slide_layer_workspace_bytes(cfg, B, S, 2)
    assert 0 < w2 < wb and sb < wb
    saved = ws(sb)
    y2, dx2, g2 = empty((N, c.hidden), dtype), empty((N, c.hidden), dtype), torch.empty_like(w)
    sl.slide_layer_fwd_save(cfg, w, tx, y2, B, S, saved, sb, stream())
    sl.slide_layer_bwd_saved(cfg, w, tx, tdy, dx2, g2, B, S, saved, sb, ws(w2), w2, stream())
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if dtype != "f32" else (lambda t: t.view(torch.int32))
    assert torch.equal(bits(y1), bits(y2))
    assert torch.equal(bits(dx1), bits(dx2))
    assert torch.equal(bits(g1), bits(g2))


def test_layer_bwd_dy_may_alias_dx():
    c, dtype, B, S = LayerCfg(256, 4, 2, 64, 688), "bf16", 1, 96
    print("layer bwd with dy aliasing dx", flush=True)
    N = B * S
    params = layer_params(c, dtype, seed=3)
    x = activations((N, c.hidden), dtype, 4)
    dy = activations((N, c.hidden), dtype, 5)
    cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, dtype)
    w = _packed_to_device(params, c, dtype)
    tx = dev(x.f32, dtype)
    wb = sl.slide_layer_workspace_bytes(cfg, B, S, 1)
    W = ws(wb)
    dx1 = empty((N, c.hidden), dtype)
    g1 = torch.empty_like(w)
    sl.slide_layer_bwd(cfg, w, tx, dev(dy.f32, dtype), dx1, g1, B, S, W, wb, stream())
    buf = dev(dy.f32, dtype)
    g2 = torch.empty_like(w)
    sl.slide_layer_bwd(cfg, w, tx, buf, buf, g2, B, S, W, wb, stream())
    torch.cuda.synchronize()
    assert torch.equal(dx1.view(torch.int16), buf.view(torch.int16))
    assert torch.equal(g1.view(torch.int16), g2.view(torch.int16))


CE_CASES = [
    ("bf16-ragged-chunks", "bf16", 300, 256, 1000, 256, 0.1),   # last chunk 232 rows, ignored targets
    ("bf16-one-chunk", "bf16", 128, 512, 2048, 8192, 0.0),
    ("f32-tiny", "f32", 256, 256, 1024, 8192, 0.0),
    ("bf16-all-ignored", "bf16", 64, 256, 512, 128, 1.0),
    ("f16-ragged-chunks", "f16", 300, 256, 1000, 256, 0.1),
    ("f16-one-chunk", "f16", 128, 512, 2048, 8192, 0.0),
]


@pytest.mark.parametrize("name,dtype,N,H,V,chunk,ign", CE_CASES, ids=[c[0] for c in CE_CASES])
def test_lmhead_ce_matches_oracle(name, dtype, N, H, V, chunk, ign):
    print(f"lmhead ce {name}: N={N} H={H} V={V} chunk={chunk}", flush=True)
    h, w, t = ce_inputs(N, H, V, dtype, ignore_frac=ign)
    cfg = sl.CeCfg(H, V, chunk, sl.dtype_code(dtype))
    wsz = sl.slide_lmhead_ce_workspace_bytes(cfg, N)
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    dh = empty((N, H), dtype)
    dw = empty((V, H), dtype)
    sl.slide_lmhead_ce(cfg, dev(h.f32, dtype), dev(w.f32, dtype), torch.from_numpy(t).to(DEV), N,
                       loss, dh, dw, ws(wsz), wsz, stream())
    torch.cuda.synchronize()
    rl, rdh, rdw, _ = om.ce_dense(h.f64, w.f64, t)
    got = float(loss.item())
    print(f"  loss gpu {got:.6f} oracle {rl:.6f}", flush=True)
    if ign >= 1.0:
        assert got == 0.0
        assert float(dh.float().abs().max()) == 0.0 and float(dw.float().abs().max()) == 0.0
        return
    assert abs(got - rl) <= (1e-5 if dtype == "f32" else 2e-3) * max(1.0, abs(rl))
    assert_close(host(dh), rdh, dtype, "ce dh")
    assert_close(host(dw), rdw, dtype, "ce dw")


@pytest.mark.parametrize("dtype,N,H,V,chunk,ign", [("bf16", 300, 256, 1000, 256, 0.1),
                                                  ("f32", 200, 256, 1024, 384, 0.0),
                                                  ("f16", 300, 256, 1000, 256, 0.1)])
def test_lmhead_ce_phases_equal_single_call(dtype, N, H, V, chunk, ign):
    """The host-driven phases (stats per chunk in reverse order, loss, grad per chunk, dh) give
    the single call's results bit for bit."""
    print(f"lmhead ce phases {dtype}: N={N} H={H} V={V} chunk={chunk}", flush=True)
    h, w, t = ce_inputs(N, H, V, dtype, ignore_frac=ign)
    cfg = sl.CeCfg(H, V, chunk, sl.dtype_code(dtype))
    wsz = sl.slide_lmhead_ce_workspace_bytes(cfg, N)
    th, tw, tt = dev(h.f32, dtype), dev(w.f32, dtype), torch.from_numpy(t).to(DEV)
    loss1 = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    dh1, dw1 = empty((N, H), dtype), empty((V, H), dtype)
    sl.slide_lmhead_ce(cfg, th, tw, tt, N, loss1, dh1, dw1, ws(wsz), wsz, stream())
    nch = sl.slide_lmhead_ce_n_chunks(cfg)
    assert nch == (V + chunk - 1) // chunk
    W2 = ws(wsz)
    loss2 = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    dh2, dw2 = empty((N, H), dtype), torch.full((V, H), float("nan"), device=DEV,
                                               dtype=dh1.dtype)
    for ci in reversed(range(nch)):
        sl.slide_lmhead_ce_stats(cfg, th, tw, tt, N, ci, W2, wsz, stream())
    sl.slide_lmhead_ce_loss(cfg, tt, N, loss2, W2, wsz, stream())
    for ci in range(nch):
        sl.slide_lmhead_ce_grad(cfg, th, tw, tt, N, ci, True, dw2, W2, wsz, stream())
    sl.slide_lmhead_ce_dh(cfg, N, dh2, W2, wsz, stream())
    torch.cuda.synchronize()
    assert torch.equal(loss1, loss2)
    bits = (lambda x: x.view(torch.int16)) if dtype != "f32" else (lambda x: x.view(torch.int32))
    assert torch.equal(bits(dh1), bits(dh2))
    assert torch.equal(bits(dw1), bits(dw2))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_lmhead_ce_gradient_scale(dtype):
    """With grad_scale S (dynamic loss scaling) the CE returns the same loss and S times the
    gradients. In bf16 (fp32's exponent range) a power-of-two S scales every rounding point
    exactly, so dh and dW are S times the unscaled values exactly. In fp16 the unscaled dz
    (about 1 / (V N)) lies in the subnormal range and loses digits, which S restores: the
    scaled gradients match the oracle within the fp16 bound and more closely than the unscaled
    ones."""
    N, H, V, chunk = 300, 256, 1000, 256
    S = 1024.0
    print(f"lmhead ce {dtype} grad_scale {S}", flush=True)
    h, w, t = ce_inputs(N, H, V, dtype, ignore_frac=0.1)
    th, tw, tt = dev(h.f32, dtype), dev(w.f32, dtype), torch.from_numpy(t).to(DEV)
    out = []
    for scale in (0.0, S):
        cfg = sl.CeCfg(H, V, chunk, sl.dtype_code(dtype), scale)
        wsz = sl.slide_lmhead_ce_workspace_bytes(cfg, N)
        loss = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
        dh, dw = empty((N, H), dtype), empty((V, H), dtype)
        sl.slide_lmhead_ce(cfg, th, tw, tt, N, loss, dh, dw, ws(wsz), wsz, stream())
        torch.cuda.synchronize()
        out.append((float(loss.item()), host(dh), host(dw)))
    (l0, dh0, dw0), (l1, dh1, dw1) = out
    assert l0 == l1
    rl, rdh, rdw, _ = om.ce_dense(h.f64, w.f64, t)
    if dtype == "bf16":
        assert np.array_equal(dh1, S * dh0) and np.array_equal(dw1, S * dw0)
    else:
        # the largest errors sit in the target rows (dz near -1/N, normal range either way);
        # the underflow shows in the many small entries, so compare root-mean-square errors
        rms = lambda a: float(np.sqrt(np.mean((a - rdw) ** 2)) / np.sqrt(np.mean(rdw ** 2)))
        e0, e1 = rms(dw0), rms(dw1 / S)
        print(f"  fp16 dW rms rel err unscaled {e0:.3e}, scaled by {S:g} {e1:.3e}", flush=True)
        assert e1 < e0
    assert_close(dh1 / S, rdh, dtype, "ce dh / S")
    assert_close(dw1 / S, rdw, dtype, "ce dw / S")
