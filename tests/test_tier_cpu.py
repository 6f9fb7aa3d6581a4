"""CPU tests of the disk tier of the optimizer state (slide_tier_*): bytes written come back
unchanged, with and without O_DIRECT, across chunk and page boundaries; the streamed AdamW over
state held in the file gives the same bits as the oracle's fixed-order float32 AdamW over state
held in memory, for every placement of p, m and v and both gradient types; bad offsets, sizes
and paths are rejected before any file traffic."""
import os

import numpy as np
import pytest

import layer_sliding_offloaded_fwd_amd as sl
from layer_sliding_offloaded_fwd_amd import _capi
from layer_sliding_offloaded_fwd_amd.binding import StateTier
from oracle import adamw as oa

HP = oa.AdamWHyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
CHP = sl.AdamWHp(HP.lr, HP.beta1, HP.beta2, HP.eps, HP.weight_decay)
PAGE = 4096


@pytest.mark.parametrize("flags", [_capi.SLIDE_TIER_DIRECT | _capi.SLIDE_TIER_UNLINK,
                                   _capi.SLIDE_TIER_UNLINK])
def test_round_trip_across_chunks_and_pages(tmp_path, flags):
    path = tmp_path / "state.bin"
    # chunk of 3000 elements -> 3072 (a whole number of pages); pieces of 3 x 3072 floats
    t = StateTier(path, 64 << 20, chunk_elems=3000, io_threads=3, flags=flags)
    try:
        info = t.info()
        assert info["chunk"] == 3072 and info["capacity"] == 64 << 20
        assert not path.exists()                       # unlinked right after creation
        rng = np.random.default_rng(0)
        a = rng.standard_normal(50_001).astype(np.float32)     # ragged: not a page multiple
        b = rng.integers(0, 2 ** 32, 9_216 * 3, dtype=np.uint32)  # exactly one piece
        off_a, off_b = PAGE, PAGE + sl.slide_tier_region_bytes(a.size)
        t.write(off_a, a)
        t.write(off_b, b)
        ra, rb = np.empty_like(a), np.empty_like(b)
        t.read(off_a, ra)
        t.read(off_b, rb)
        assert np.array_equal(ra.view(np.uint32), a.view(np.uint32))
        assert np.array_equal(rb, b)
        # the tail of a's last page reads back as zeros; unwritten space reads as zeros
        full = np.full(sl.slide_tier_region_bytes(a.size) // 4, 7, np.float32)
        t.read(off_a, full)
        assert full.size > a.size and np.all(full[a.size:] == 0)
        z = np.ones(1000, np.float32)
        t.read(32 << 20, z)
        assert np.all(z == 0)
        # a write of zeros (no source)
        t.write(off_a, None, 4 * 10_000)
        t.read(off_a, ra)
        assert np.all(ra[:10_000] == 0) and np.array_equal(ra[10_240:], a[10_240:])
        s = t.stats()
        assert s["bytes_written"] >= a.nbytes + b.nbytes and s["bytes_read"] > 0
    finally:
        t.close()


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
@pytest.mark.parametrize("placement", ["pmv", "mv", "p"])
def test_tier_adamw_bit_exact_vs_oracle(tmp_path, gdt, placement):
    """placement: which of p, m, v live in the file (the rest in host memory)."""
    rng = np.random.default_rng(5)
    n = 2 * 4096 + 1234          # chunks of 4096: two full ones and a ragged third
    p0 = rng.standard_normal(n).astype(np.float32)
    p0[:4] = [0.0, -0.0, 1e-40, 3e38]
    reg = sl.slide_tier_region_bytes(n)
    offs = {"p": PAGE, "m": PAGE + reg, "v": PAGE + 2 * reg}
    t = StateTier(tmp_path / "s.bin", PAGE + 3 * reg, chunk_elems=4096, io_threads=4)
    try:
        host = {"p": p0.copy(), "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32)}
        for k in placement:
            t.write(offs[k], host[k])
            host[k] = None
        po, mo, vo = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        for step in range(1, 5):
            g32 = (rng.standard_normal(n) * 10.0 ** rng.integers(-6, 2, n)).astype(np.float32)
            g32[:3] = [0.0, np.inf, np.nan] if step == 3 else g32[:3]
            if gdt == "bf16":
                gbits = oa.bf16_round_bits(g32)
                g_in, g_or, code = gbits.copy(), oa.bf16_bits_to_f32(gbits), sl.SLIDE_BF16
                out = g_in                      # the bf16 weight copy overwrites the gradient
            else:
                g_in, g_or, code = g32.copy(), g32, sl.SLIDE_F32
                out = np.zeros(n, np.uint16)
            t.adamw(host["p"], offs["p"], host["m"], offs["m"], host["v"], offs["v"], g_in, code,
                    out, n, step, CHP, n_threads=3)
            po, mo, vo, bo = oa.adamw_fp32(po, g_or, mo, vo, step, HP)
            got = {}
            for k in "pmv":
                if host[k] is None:
                    got[k] = np.empty(n, np.float32)
                    t.read(offs[k], got[k])
                else:
                    got[k] = host[k]
            np.testing.assert_array_equal(got["p"].view(np.uint32), po.view(np.uint32))
            np.testing.assert_array_equal(got["m"].view(np.uint32), mo.view(np.uint32))
            np.testing.assert_array_equal(got["v"].view(np.uint32), vo.view(np.uint32))
            np.testing.assert_array_equal(out, bo)
        s = t.stats()
        n_tiered = len(placement)
        assert s["bytes_read"] >= 4 * n_tiered * reg and s["bytes_written"] >= 4 * n_tiered * reg
    finally:
        t.close()


def test_tier_rejects_bad_arguments(tmp_path):
    with pytest.raises(sl.SlideError) as e:
        StateTier(tmp_path / "missing-dir" / "s.bin", 1 << 20)
    assert e.value.code == _capi.SLIDE_E_IO
    with pytest.raises(sl.SlideError) as e:
        StateTier(tmp_path / "s.bin", 1000)                  # not a page multiple
    assert e.value.code == _capi.SLIDE_E_ARG
    t = StateTier(tmp_path / "s.bin", 1 << 20, chunk_elems=1024)
    try:
        a = np.zeros(1000, np.float32)
        for off in (100, (1 << 20) - PAGE // 2):
            with pytest.raises(sl.SlideError) as e:
                t.write(off, a)
            assert e.value.code == _capi.SLIDE_E_ARG
        with pytest.raises(sl.SlideError) as e:
            t.read(1 << 20, a)                                # past the capacity
        assert e.value.code == _capi.SLIDE_E_ARG
        g = np.zeros(5000, np.float32)
        with pytest.raises(sl.SlideError) as e:               # p and m regions overlap
            t.adamw(None, 0, None, PAGE, np.zeros(5000, np.float32), 0, g, sl.SLIDE_F32, None,
                    5000, 1, CHP)
        assert e.value.code == _capi.SLIDE_E_ARG
        with pytest.raises(sl.SlideError) as e:               # step 0
            t.adamw(None, 0, None, 8 * PAGE, None, 16 * PAGE, g, sl.SLIDE_F32, None, 5000, 0, CHP)
        assert e.value.code == _capi.SLIDE_E_ARG
    finally:
        t.close()
    assert not os.path.exists(tmp_path / "s.bin")
