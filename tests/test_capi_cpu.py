"""CPU-side checks of the C ABI: the library loads and exports every declared entry point, the
host-side validation rejects bad arguments before anything is launched, the CPU AdamW matches the
oracle's fixed-order float32 contract bit for bit, and the slot ring's state machine (on its host
engine) enforces its transitions and reports copy failures and time-outs."""
import ctypes
import os
import re

import numpy as np
import pytest

import layer_sliding_offloaded_fwd_amd as sl
from layer_sliding_offloaded_fwd_amd import _capi
from oracle import adamw as oa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "slide.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slide_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sl.lib()
    names = _declared_functions()
    assert len(names) >= 30
    for n in names:
        assert hasattr(L, n), n
        assert n in _capi.SIGNATURES, f"{n} has no ctypes signature"
    assert b"gfx950" in L.slide_version()


def test_validation_errors_before_any_launch():
    cfg = sl.layer_cfg(100, 4, 3, 64, 688, "bf16")          # 4 % 3 != 0 and H % 8 != 0
    with pytest.raises(sl.SlideError) as e:
        sl.slide_layer_fwd(cfg, 16, 16, 32, 1, 8, 64, 1 << 20)
    assert e.value.code in (_capi.SLIDE_E_SHAPE,)
    cfg = sl.layer_cfg(256, 4, 4, 96, 688, "bf16")          # head_dim 96 unsupported
    with pytest.raises(sl.SlideError) as e:
        sl.slide_layer_fwd(cfg, 16, 16, 32, 1, 8, 64, 1 << 20)
    assert e.value.code == _capi.SLIDE_E_SHAPE and "head_dim" in str(e.value)
    cfg = sl.layer_cfg(256, 4, 4, 64, 688, "bf16")
    need = sl.slide_layer_workspace_bytes(cfg, 2, 128, 0)
    assert need > 0 and sl.slide_layer_workspace_bytes(cfg, 2, 128, 1) > need
    with pytest.raises(sl.SlideError) as e:                 # workspace one byte short
        sl.slide_layer_fwd(cfg, 256, 512, 1024, 2, 128, 2048, need - 1)
    assert e.value.code == _capi.SLIDE_E_WORKSPACE
    with pytest.raises(sl.SlideError) as e:                 # misaligned pointer
        sl.slide_layer_fwd(cfg, 258, 512, 1024, 2, 128, 2048, need)
    assert e.value.code == _capi.SLIDE_E_ARG
    with pytest.raises(sl.SlideError) as e:                 # null weight slot
        sl.slide_layer_bwd(cfg, None, 512, 1024, 2048, 4096, 2, 128, 8192, 1 << 40)
    assert e.value.code == _capi.SLIDE_E_ARG
    ce = sl.CeCfg(4096, 1001, 8192, sl.SLIDE_BF16)          # vocab not a multiple of 8
    assert sl.slide_lmhead_ce_workspace_bytes(ce, 16) == 0
    with pytest.raises(sl.SlideError) as e:
        sl.slide_gemm(64, 64, 60, 256, 64, True, 512, 64, True, 1024, 64, sl.SLIDE_BF16)
    assert e.value.code == _capi.SLIDE_E_SHAPE              # K-contiguous K % 8 != 0
    with pytest.raises(sl.SlideError) as e:
        sl.slide_attention_fwd(256, 512, 1024, 1, 16, 6, 4, 128, sl.SLIDE_BF16)
    assert e.value.code == _capi.SLIDE_E_SHAPE


def test_rmsnorm_noalloc_size_limit_checked_before_any_launch():
    """The no-allocation RMSNorm backward refuses a size whose scratch exceeds its fixed array
    (16 MiB) with SLIDE_E_WORKSPACE before touching the device."""
    assert sl.slide_rmsnorm_bwd_noalloc_max_bytes() == 16 << 20
    N, H = 65536, 8192
    assert sl.slide_rmsnorm_bwd_workspace_bytes(N, H) > 16 << 20
    with pytest.raises(sl.SlideError) as e:
        sl.slide_rmsnorm_bwd_noalloc(None, None, None, None, None, None, N, H, 1e-5,
                                     sl.SLIDE_BF16)
    assert e.value.code == _capi.SLIDE_E_WORKSPACE


def test_nonfinite_count_validation():
    cnt = np.zeros(1, np.int32)
    for args, code in [((None, sl.SLIDE_BF16, 16, cnt.ctypes.data), _capi.SLIDE_E_ARG),
                       ((cnt.ctypes.data, 7, 16, cnt.ctypes.data), _capi.SLIDE_E_ARG),
                       ((cnt.ctypes.data + 2, sl.SLIDE_F32, 16, cnt.ctypes.data), _capi.SLIDE_E_ARG),
                       ((cnt.ctypes.data, sl.SLIDE_F32, 16, None), _capi.SLIDE_E_ARG)]:
        with pytest.raises(sl.SlideError) as e:
            sl.slide_nonfinite_count(*args)
        assert e.value.code == code


def test_ce_phase_validation():
    ce = sl.CeCfg(4096, 128256, 8192, sl.SLIDE_BF16)
    assert sl.slide_lmhead_ce_n_chunks(ce) == 16            # 15 full chunks and one of 5376 rows
    assert sl.slide_lmhead_ce_n_chunks(sl.CeCfg(256, 1024, 0, sl.SLIDE_F32)) == 1
    assert sl.slide_lmhead_ce_n_chunks(sl.CeCfg(256, 1024, 256, sl.SLIDE_F32)) == 4
    need = sl.slide_lmhead_ce_workspace_bytes(ce, 64)
    for chunk in (-1, 16):                                  # chunk index out of range
        with pytest.raises(sl.SlideError) as e:
            sl.slide_lmhead_ce_stats(ce, 256, 512, 1024, 64, chunk, 2048, need)
        assert e.value.code == _capi.SLIDE_E_ARG and "chunk" in str(e.value)
        with pytest.raises(sl.SlideError) as e:
            sl.slide_lmhead_ce_grad(ce, 256, 512, 1024, 64, chunk, 1, 4096, 2048, need)
        assert e.value.code == _capi.SLIDE_E_ARG
    with pytest.raises(sl.SlideError) as e:                 # workspace one byte short
        sl.slide_lmhead_ce_loss(ce, 1024, 64, 4096, 2048, need - 1)
    assert e.value.code == _capi.SLIDE_E_WORKSPACE
    with pytest.raises(sl.SlideError) as e:                 # null dh
        sl.slide_lmhead_ce_dh(ce, 64, None, 2048, need)
    assert e.value.code == _capi.SLIDE_E_ARG
    with pytest.raises(sl.SlideError) as e:                 # bad cfg
        sl.slide_lmhead_ce_n_chunks(sl.CeCfg(4096, 1001, 8192, sl.SLIDE_BF16))


def test_param_count_and_offsets_match_packing():
    from seeded_inputs import L8B, TINY
    for w in (TINY, L8B):
        c = w.layer
        cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, w.dtype)
        assert sl.slide_layer_param_count(cfg) == c.param_count()
        off = sl.slide_layer_param_offsets(cfg)
        sizes = [int(np.prod(s)) for _, s in c.param_shapes()]
        assert off == list(np.concatenate([[0], np.cumsum(sizes)[:-1]]))
    assert L8B.layer.param_count() == 218_112_000


# ------------------------------------------------------------------------------ AdamW
HP = oa.AdamWHyper(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
CHP = sl.AdamWHp(HP.lr, HP.beta1, HP.beta2, HP.eps, HP.weight_decay)


def _adversarial(n, rng):
    g = (rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17e-38, 3e38, -3e38, 1e-20, 65504.0,
                        np.inf, -np.inf, np.nan], np.float32)
    g[: len(special)] = special
    return g


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
@pytest.mark.parametrize("threads", [1, 7])
def test_cpu_adamw_bit_exact_vs_oracle(gdt, threads):
    rng = np.random.default_rng(11)
    n = 100_003                       # odd size: scalar head and tail around the vector loop
    p = rng.standard_normal(n).astype(np.float32)
    p[:4] = [0.0, -0.0, 1e-40, 3e38]
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    po, mo, vo = p.copy(), m.copy(), v.copy()
    for t in range(1, 5):
        g32 = _adversarial(n, rng) if t == 2 else (rng.standard_normal(n) * 1e-3).astype(np.float32)
        if gdt == "bf16":
            gbits = oa.bf16_round_bits(g32)
            g_in, g_or = gbits.copy(), oa.bf16_bits_to_f32(gbits)
            code = sl.SLIDE_BF16
        else:
            g_in, g_or, code = g32.copy(), g32, sl.SLIDE_F32
        out = np.zeros(n, np.uint16)
        sl.slide_cpu_adamw(p, g_in, code, m, v, out, n, t, CHP, threads)
        po, mo, vo, bo = oa.adamw_fp32(po, g_or, mo, vo, t, HP)
        np.testing.assert_array_equal(p.view(np.uint32), po.view(np.uint32))
        np.testing.assert_array_equal(m.view(np.uint32), mo.view(np.uint32))
        np.testing.assert_array_equal(v.view(np.uint32), vo.view(np.uint32))
        np.testing.assert_array_equal(out, bo)


def _same_f32_nan(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    assert np.array_equal(na, nb)
    assert np.array_equal(a.view(np.uint32)[~na], b.view(np.uint32)[~nb])


@pytest.mark.parametrize("threads", [1, 5])
def test_cpu_adamw_fp16_gradient_with_loss_scale_bit_exact_vs_oracle(threads):
    """fp16 gradients at a loss scale of 2^16 (including values that overflowed to infinity):
    the update unscales them and writes an fp16 copy, bit for bit as the oracle's contract (NaN
    results compared as NaN)."""
    rng = np.random.default_rng(14)
    n = 50_001
    S = 2.0 ** 16
    p = rng.standard_normal(n).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    po, mo, vo = p.copy(), m.copy(), v.copy()
    hp = sl.AdamWHp(HP.lr, HP.beta1, HP.beta2, HP.eps, HP.weight_decay, S)
    for t in range(1, 4):
        g = (rng.standard_normal(n) * 1e-3 * S).astype(np.float32)
        if t == 2:
            g[:3] = [np.inf, -np.inf, 70000.0]
        gbits = oa.f16_round_bits(g)
        out = np.zeros(n, np.uint16)
        sl.slide_cpu_adamw(p, gbits.copy(), sl.SLIDE_F16, m, v, out, n, t, hp, threads)
        po, mo, vo, bo = oa.adamw_fp32(po, oa.f16_bits_to_f32(gbits), mo, vo, t, HP,
                                       grad_scale=S, copy="f16")
        _same_f32_nan(p, po)
        _same_f32_nan(m, mo)
        _same_f32_nan(v, vo)
        _same_f32_nan(oa.f16_bits_to_f32(out), oa.f16_bits_to_f32(bo))


def test_cpu_convert_f32_matches_oracle_rounding():
    rng = np.random.default_rng(15)
    x = (rng.standard_normal(70_001) * 10.0 ** rng.integers(-10, 6, 70_001)).astype(np.float32)
    x[:4] = [np.inf, -np.inf, 65520.0, 1e-9]
    for code, ref in ((sl.SLIDE_BF16, oa.bf16_round_bits(x)), (sl.SLIDE_F16, oa.f16_round_bits(x))):
        out = np.zeros(x.size, np.uint16)
        sl.slide_cpu_convert_f32(x, out, code, x.size, 3)
        assert np.array_equal(out, ref)
    with pytest.raises(sl.SlideError):
        sl.slide_cpu_convert_f32(x, np.zeros(4, np.float32), sl.SLIDE_F32, 4)


def test_cpu_adamw_shared_grad_and_bf16_buffer_and_scalar_path():
    """The bf16 gradient landing buffer may double as the bf16 weight output (in place)."""
    rng = np.random.default_rng(12)
    n = 4099
    p = rng.standard_normal(n).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    g = oa.bf16_round_bits((rng.standard_normal(n) * 1e-2).astype(np.float32))
    po, mo, vo, bo = oa.adamw_fp32(p, oa.bf16_bits_to_f32(g), m, v, 7, HP)
    p2, m2, v2, shared = p.copy(), m.copy(), v.copy(), g.copy()
    sl.slide_cpu_adamw(p2, shared, sl.SLIDE_BF16, m2, v2, shared, n, 7, CHP, 3)
    np.testing.assert_array_equal(shared, bo)
    np.testing.assert_array_equal(p2.view(np.uint32), po.view(np.uint32))
    p3, m3, v3, out3 = p.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
    _capi.call("slide_cpu_adamw_scalar_for_test", p3.ctypes.data, g.ctypes.data, sl.SLIDE_BF16,
               m3.ctypes.data, v3.ctypes.data, out3.ctypes.data, n, 7, ctypes.byref(CHP))
    np.testing.assert_array_equal(p3.view(np.uint32), po.view(np.uint32))
    np.testing.assert_array_equal(out3, bo)


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
@pytest.mark.parametrize("zero_grad", [False, True])
def test_cpu_adamw_rows_bit_exact_vs_oracle(gdt, zero_grad):
    """Listed rows get the fixed-order AdamW of their gradient (zero when g is NULL), bit for
    bit; rows not listed are untouched."""
    rng = np.random.default_rng(13)
    R, W = 37, 1000                     # odd row length: vector loop with a scalar tail per row
    p = rng.standard_normal(R * W).astype(np.float32)
    m = (rng.standard_normal(R * W) * 1e-3).astype(np.float32)
    v = (rng.random(R * W) * 1e-6).astype(np.float32)
    g32 = (rng.standard_normal(R * W) * 1e-2).astype(np.float32)
    rows = np.array([0, 5, 6, 17, 36], np.int32)
    if gdt == "bf16":
        gbits = oa.bf16_round_bits(g32)
        g_in, g_or, code = gbits, oa.bf16_bits_to_f32(gbits), sl.SLIDE_BF16
    else:
        g_in, g_or, code = g32, g32, sl.SLIDE_F32
    if zero_grad:
        g_or = np.zeros_like(g32)
    p2, m2, v2, out = p.copy(), m.copy(), v.copy(), np.full(R * W, 7, np.uint16)
    sl.slide_cpu_adamw_rows(p2, None if zero_grad else g_in, code, m2, v2, out, W, R, rows,
                            len(rows), 3, CHP, 4)
    po, mo, vo, bo = oa.adamw_fp32(p, g_or, m, v, 3, HP)
    sel = np.zeros(R, bool)
    sel[rows] = True
    sel = np.repeat(sel, W)
    np.testing.assert_array_equal(p2[sel].view(np.uint32), po[sel].view(np.uint32))
    np.testing.assert_array_equal(m2[sel].view(np.uint32), mo[sel].view(np.uint32))
    np.testing.assert_array_equal(v2[sel].view(np.uint32), vo[sel].view(np.uint32))
    np.testing.assert_array_equal(out[sel], bo[sel])
    np.testing.assert_array_equal(p2[~sel].view(np.uint32), p[~sel].view(np.uint32))
    assert np.all(out[~sel] == 7)
    with pytest.raises(sl.SlideError):            # a row outside the arrays
        sl.slide_cpu_adamw_rows(p2, None, code, m2, v2, None, W, R,
                                np.array([R], np.int32), 1, 1, CHP)
    p3 = p2.copy()
    with pytest.raises(sl.SlideError):            # a row listed twice: refused, nothing changed
        sl.slide_cpu_adamw_rows(p3, None, code, m2, v2, None, W, R,
                                np.array([3, 9, 3], np.int32), 3, 1, CHP)
    np.testing.assert_array_equal(p3.view(np.uint32), p2.view(np.uint32))


@pytest.mark.parametrize("gdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("in_place", [False, True])
def test_cpu_adamw_rows_packed_bit_exact_vs_oracle(gdt, in_place):
    """Packed gradient rows (row k for row rows[k], rows in any order): the listed rows get the
    fixed-order AdamW of their gradient bit for bit, the 16-bit copy lands in both the full
    table's rows and the packed rows (in place over the gradient when asked), fp32 rows are
    packed as they are; rows not listed are untouched."""
    rng = np.random.default_rng(17)
    R, W = 41, 1000
    p = rng.standard_normal(R * W).astype(np.float32)
    m = (rng.standard_normal(R * W) * 1e-3).astype(np.float32)
    v = (rng.random(R * W) * 1e-6).astype(np.float32)
    rows = np.array([33, 0, 7, 40, 12], np.int32)
    K = len(rows)
    g32 = (rng.standard_normal(K * W) * 1e-2).astype(np.float32)
    if gdt == "bf16":
        g_in = oa.bf16_round_bits(g32)
        g_or, code = oa.bf16_bits_to_f32(g_in), sl.SLIDE_BF16
    elif gdt == "f16":
        g_in = oa.f16_round_bits(g32)
        g_or, code = oa.f16_bits_to_f32(g_in), sl.SLIDE_F16
    else:
        g_in, g_or, code = g32, g32, sl.SLIDE_F32
    g_full = np.zeros(R * W, np.float32)
    for k, r in enumerate(rows):
        g_full[r * W:(r + 1) * W] = g_or[k * W:(k + 1) * W]
    p2, m2, v2 = p.copy(), m.copy(), v.copy()
    full = np.full(R * W, 7, np.uint16) if gdt != "f32" else None
    g_buf = g_in.copy()
    packed = g_buf if in_place else np.zeros_like(g_in)
    sl.slide_cpu_adamw_rows_packed(p2, m2, v2, W, R, rows, K, g_buf, code, full, packed, 3,
                                   CHP, 4)
    po, mo, vo, bo = oa.adamw_fp32(p, g_full, m, v, 3, HP, copy="f16" if gdt == "f16" else "bf16")
    sel = np.zeros(R, bool)
    sel[rows] = True
    sel = np.repeat(sel, W)
    np.testing.assert_array_equal(p2[sel].view(np.uint32), po[sel].view(np.uint32))
    np.testing.assert_array_equal(m2[sel].view(np.uint32), mo[sel].view(np.uint32))
    np.testing.assert_array_equal(v2[sel].view(np.uint32), vo[sel].view(np.uint32))
    np.testing.assert_array_equal(p2[~sel].view(np.uint32), p[~sel].view(np.uint32))
    for k, r in enumerate(rows):
        want = bo[r * W:(r + 1) * W] if gdt != "f32" else po[r * W:(r + 1) * W]
        got = packed[k * W:(k + 1) * W]
        np.testing.assert_array_equal(got.view(want.dtype), want)
    if full is not None:
        np.testing.assert_array_equal(full[sel], bo[sel])
        assert np.all(full[~sel] == 7)
    with pytest.raises(sl.SlideError):            # a row outside the table
        sl.slide_cpu_adamw_rows_packed(p2, m2, v2, W, R, np.array([R], np.int32), 1, g_buf,
                                       code, None, None, 1, CHP)
    with pytest.raises(sl.SlideError):            # a row listed twice
        sl.slide_cpu_adamw_rows_packed(p2, m2, v2, W, R, np.array([5, 5], np.int32), 2, g_buf,
                                       code, None, None, 1, CHP)
    if gdt == "f32":
        with pytest.raises(sl.SlideError):        # no 16-bit copy of an fp32 gradient
            sl.slide_cpu_adamw_rows_packed(p2, m2, v2, W, R, rows, K, g_buf, code,
                                           np.zeros(R * W, np.uint16), None, 1, CHP)
    with pytest.raises(sl.SlideError):            # packed output partly over the gradient
        sl.slide_cpu_adamw_rows_packed(p2, m2, v2, W, R, rows, K, g_buf, code, None,
                                       g_buf.ctypes.data + 2, 1, CHP)


def test_copy_rows_validates_before_any_launch():
    a = np.zeros(64, np.float32)
    for args in [(a, None, 4, a, None, 4, 2, 24),       # row_bytes not a multiple of 16
                 (a, None, 1, a, None, 4, 2, 16),       # two rows in order from a 1-row source
                 (a, None, 4, a, None, 4, -1, 16)]:     # negative count
        with pytest.raises(sl.SlideError) as e:
            sl.slide_copy_rows(*args)
        assert e.value.code == _capi.SLIDE_E_SHAPE
    sl.slide_copy_rows(a, None, 4, a, None, 4, 0, 16)     # nothing to copy: no launch


def test_gpu_adamw_validates_before_any_launch():
    a = np.zeros(16, np.float32)
    with pytest.raises(sl.SlideError) as e:
        sl.slide_gpu_adamw(None, a, sl.SLIDE_F32, a, a, None, 16, 1, CHP)
    assert e.value.code == _capi.SLIDE_E_ARG
    with pytest.raises(sl.SlideError):            # step 0
        sl.slide_gpu_adamw(a, a, sl.SLIDE_F32, a, a, None, 16, 0, CHP)
    with pytest.raises(sl.SlideError):            # fp32 gradient aliasing the bf16 output
        sl.slide_gpu_adamw(a, a, sl.SLIDE_F32, a.copy(), a.copy(), a, 16, 1, CHP)


def test_host_triad_measures_and_validates():
    best, med = sl.slide_host_triad(1 << 20, 2, 3)
    assert best >= med > 0.0
    with pytest.raises(sl.SlideError):
        sl.slide_host_triad(8, 1, 1)
    with pytest.raises(sl.SlideError):
        sl.slide_host_triad(1 << 20, 1, 0)


def test_cpu_adamw_rejects_bad_arguments():
    a = np.zeros(64, np.float32)
    g = np.zeros(64, np.uint16)
    with pytest.raises(sl.SlideError):
        sl.slide_cpu_adamw(a, g, sl.SLIDE_BF16, a.copy(), a.copy(), None, 64, 0, CHP)
    bad = sl.AdamWHp(1e-4, 1.0, 0.999, 1e-8, 0.0)
    with pytest.raises(sl.SlideError):
        sl.slide_cpu_adamw(a, g, sl.SLIDE_BF16, a.copy(), a.copy(), None, 64, 1, bad)
    with pytest.raises(sl.SlideError):     # partially overlapping output
        sl.slide_cpu_adamw(a, g, sl.SLIDE_BF16, a.copy(), a.copy(), g.ctypes.data + 2, 64, 1, CHP)


# ------------------------------------------------------------------------------ slot ring
def _host_ring(n_slots=3, wb=1024, gb=512):
    dev = np.zeros(n_slots * (wb + gb), np.uint8)
    ring = sl.SlotRing(n_slots, wb, gb, dev, engine=sl.SLIDE_ENGINE_HOST)
    return ring, dev


def test_ring_sliding_schedule_moves_the_right_bytes():
    wb, gb, L = 1024, 512, 7
    ring, dev = _host_ring(3, wb, gb)
    host_w = [np.full(wb, 10 + i, np.uint8) for i in range(L)]
    host_g = [np.zeros(gb, np.uint8) for _ in range(L)]
    loaded = {}
    for i in range(min(3, L)):
        loaded[i] = ring.load(i, host_w[i])
    for i in range(L):                      # forward sweep, prefetch depth 2
        s = loaded.pop(i)
        wptr, gptr = ring.acquire(s)
        off = wptr - dev.ctypes.data
        assert np.all(dev[off: off + wb] == 10 + i)
        ring.release(s)
        if i + 3 < L:
            loaded[i + 3] = ring.load(i + 3, host_w[i + 3])
    # turnaround: the last three layers are still resident
    for i in (L - 1, L - 2, L - 3):
        loaded[i] = ring.reuse(i)
    with pytest.raises(sl.SlideError) as e:
        ring.reuse(0)
    assert e.value.code == _capi.SLIDE_E_STATE
    tickets = []
    for i in range(L - 1, -1, -1):          # backward sweep
        s = loaded.pop(i)
        wptr, gptr = ring.acquire(s)
        off = wptr - dev.ctypes.data
        assert np.all(dev[off: off + wb] == 10 + i)
        goff = gptr - dev.ctypes.data
        dev[goff: goff + gb] = 100 + i      # "compute" the gradients
        tickets.append((i, ring.flush(s, host_g[i])))
        ring.release(s)
        if i - 3 >= 0:
            loaded[i - 3] = ring.load(i - 3, host_w[i - 3])
    import time
    for i, t in tickets:
        ring.wait_flush(t, 5000)
        assert np.all(host_g[i] == 100 + i)
        # the copy thread's completion time is on time.perf_counter's clock
        assert 0 < ring.ticket_time(t) <= time.perf_counter()
    with pytest.raises(sl.SlideError) as e:
        ring.ticket_time(tickets[-1][1] + 1)
    assert e.value.code == _capi.SLIDE_E_ARG
    ring.close()


def test_ring_copies_stay_inside_engine_sized_host_buffers():
    """hidden 520 in bf16: a layer's bytes are not a multiple of 256, the slot ring copies its
    256-byte-padded slot size, and the engine sizes its pinned layer buffers for that copy.
    Guard bytes after each buffer must survive a load and a flush."""
    from layer_sliding_offloaded_fwd_amd.engine import _align, pinned_bytes
    cfg = sl.layer_cfg(520, 4, 2, 64, 1040, "bf16")
    P = sl.slide_layer_param_count(cfg)
    assert (P * 2) % 256 != 0
    wb = _align(P * 2)
    nb = pinned_bytes(P, 2, wb)
    assert nb >= wb and nb % 256 == 0
    ring, dev = _host_ring(2, wb, wb)
    guard = 4096
    hw = np.full(nb + guard, 0xA5, np.uint8)
    hg = np.full(nb + guard, 0x5A, np.uint8)
    hw[:P * 2] = np.arange(P * 2, dtype=np.uint64).astype(np.uint8)
    s = ring.load(0, hw)
    wptr, gptr = ring.acquire(s)
    off = wptr - dev.ctypes.data
    assert np.array_equal(dev[off: off + P * 2], hw[:P * 2])
    goff = gptr - dev.ctypes.data
    dev[goff: goff + wb] = 7
    t = ring.flush(s, hg)
    ring.release(s)
    ring.wait_flush(t, 5000)
    assert np.all(hg[:wb] == 7)
    assert np.all(hw[nb:] == 0xA5) and np.all(hg[nb:] == 0x5A), "copy ran past the buffer"
    ring.close()


def test_ring_state_errors():
    ring, dev = _host_ring(2)
    w = np.ones(1024, np.uint8)
    g = np.zeros(512, np.uint8)
    a = ring.load(0, w)
    b = ring.load(1, w)
    assert {a, b} == {0, 1}
    with pytest.raises(sl.SlideError) as e:           # no FREE slot left
        ring.load(2, w)
    assert e.value.code == _capi.SLIDE_E_STATE
    with pytest.raises(sl.SlideError) as e:           # release before acquire
        ring.release(a)
    assert e.value.code == _capi.SLIDE_E_STATE
    with pytest.raises(sl.SlideError) as e:           # flush before acquire
        ring.flush(a, g)
    assert e.value.code == _capi.SLIDE_E_STATE
    ring.acquire(a)
    with pytest.raises(sl.SlideError) as e:           # double acquire
        ring.acquire(a)
    assert e.value.code == _capi.SLIDE_E_STATE
    assert ring.state(a) == (_capi.SLOT_IN_USE, 0)
    t = ring.flush(a, g)
    assert ring.state(a)[0] == _capi.SLOT_FLUSHING
    with pytest.raises(sl.SlideError):                # double flush
        ring.flush(a, g)
    ring.release(a)
    assert ring.state(a)[0] == _capi.SLOT_FREE
    ring.wait_flush(t, 5000)
    with pytest.raises(sl.SlideError) as e:
        ring.wait_flush(t + 100, 10)
    assert e.value.code == _capi.SLIDE_E_ARG
    with pytest.raises(sl.SlideError) as e:
        ring.acquire(7)
    assert e.value.code == _capi.SLIDE_E_ARG
    assert ring.find(1) == b and ring.find(5) == -1
    ring.close()


def test_ring_copy_failure_and_timeout_are_reported():
    ring, dev = _host_ring(2)
    w = np.ones(1024, np.uint8)
    g = np.zeros(512, np.uint8)
    ring.inject_fault(1, 1)                           # next copy fails
    s = ring.load(0, w)
    with pytest.raises(sl.SlideError) as e:
        ring.acquire(s)
    assert e.value.code == _capi.SLIDE_E_HIP and "copy failed" in str(e.value)
    s2 = ring.load(1, w)
    ring.acquire(s2)
    ring.inject_fault(2, 1)                           # next copy never completes
    t = ring.flush(s2, g)
    with pytest.raises(sl.SlideError) as e:
        ring.wait_flush(t, 50)
    assert e.value.code == _capi.SLIDE_E_TIMEOUT
    with pytest.raises(sl.SlideError) as e:
        sl.SlotRing(2, 1024, 512, dev, engine=sl.SLIDE_ENGINE_HIP).inject_fault(1, 1)
    assert e.value.code == _capi.SLIDE_E_UNSUPPORTED
    ring.close()


def test_ring_rejects_bad_geometry():
    dev = np.zeros(4096, np.uint8)
    for args in [(0, 1024, 512), (2, 1000, 512), (2, 0, 0)]:
        with pytest.raises(sl.SlideError) as e:
            sl.SlotRing(*args, dev, engine=sl.SLIDE_ENGINE_HOST)
        assert e.value.code == _capi.SLIDE_E_ARG


def test_ring_ranged_flush_and_load_move_exactly_their_parts():
    """A layer flushed and loaded in parts (the step boundary's layer 0): each part's ticket
    covers its bytes, parts land at their offsets, the slot stays FLUSHING / LOADING between
    parts, and acquire after the last load part sees the whole layer."""
    wb, gb = 1024, 1024
    ring, dev = _host_ring(2, wb, gb)
    w = np.arange(wb, dtype=np.uint16).astype(np.uint8)
    s = ring.load(0, w)
    wptr, gptr = ring.acquire(s)
    goff = gptr - dev.ctypes.data
    dev[goff: goff + gb] = (np.arange(gb) % 251).astype(np.uint8)
    hg = np.zeros(gb + 256, np.uint8)
    parts = [(0, 256), (256, 512), (768, 256)]
    tickets = []
    for off, n in parts:
        tickets.append(ring.flush_range(s, hg, off, n))
        assert ring.state(s)[0] == _capi.SLOT_FLUSHING
    for (off, n), t in zip(parts, tickets):
        ring.wait_flush(t, 5000)
        assert np.array_equal(hg[off: off + n], dev[goff + off: goff + off + n])
    assert np.all(hg[gb:] == 0)
    ring.release(s)
    # load layer 1 in parts into the other slot, then acquire
    w1 = (np.arange(wb) * 7 % 253).astype(np.uint8)
    slot = -1
    for off, n in parts:
        slot = ring.load_range(1, w1, off, n, slot)
        assert ring.state(slot) == (_capi.SLOT_LOADING, 1)
    wptr, _ = ring.acquire(slot)
    woff = wptr - dev.ctypes.data
    assert np.array_equal(dev[woff: woff + wb], w1)
    ring.release(slot)
    ring.close()


def test_ring_ranged_copies_validate_before_copying():
    ring, dev = _host_ring(2, 1024, 512)
    w = np.ones(1024, np.uint8)
    g = np.zeros(512, np.uint8)
    for off, n in [(0, 0), (1024, 1), (1000, 100)]:
        with pytest.raises(sl.SlideError) as e:
            ring.load_range(0, w, off, n, -1)
        assert e.value.code == _capi.SLIDE_E_ARG
    s = ring.load_range(0, w, 0, 512, -1)
    with pytest.raises(sl.SlideError) as e:          # continue a load of another layer
        ring.load_range(1, w, 512, 512, s)
    assert e.value.code == _capi.SLIDE_E_STATE
    with pytest.raises(sl.SlideError) as e:          # flush a part of a slot not in use
        ring.flush_range(s, g, 0, 256)
    assert e.value.code == _capi.SLIDE_E_STATE
    ring.load_range(0, w, 512, 512, s)
    ring.acquire(s)
    with pytest.raises(sl.SlideError) as e:          # outside the gradient bytes
        ring.flush_range(s, g, 256, 512)
    assert e.value.code == _capi.SLIDE_E_ARG
    t = ring.flush_range(s, g, 0, 256)
    with pytest.raises(sl.SlideError) as e:          # a whole flush needs an IN_USE slot
        ring.flush(s, g)
    assert e.value.code == _capi.SLIDE_E_STATE
    ring.flush_range(s, g, 256, 256)
    ring.release(s)
    ring.wait_flush(t, 5000)
    ring.close()
