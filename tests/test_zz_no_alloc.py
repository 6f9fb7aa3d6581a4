"""The RMSNorm backward's no-allocation entry point (scratch in the library's fixed device
array) against the entry point with a caller workspace: bit-identical results on two calls in
a row, the second smaller (a short input after a long one must not see the first call's
scratch), and the size limit reported before any launch."""
import numpy as np
import pytest
import torch

import layer_sliding_offloaded_fwd_amd as sl
from seeded_inputs import activations
from tests._gpu import DEV, dev, ws

pytestmark = pytest.mark.gpu


def _inputs(N, H, dtype, seed):
    rng = np.random.default_rng(seed)
    x = dev(activations((N, H), dtype, seed).f32, dtype)
    dy = dev(activations((N, H), dtype, seed + 1).f32, dtype)
    dres = dev(activations((N, H), dtype, seed + 2).f32, dtype)
    w = dev((1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32), dtype)
    return x, dy, dres, w


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_workspace_variant_on_consecutive_calls(dtype):
    code = sl.dtype_code(dtype)
    st = torch.cuda.current_stream()
    for N, H, seed in ((8192, 4096, 1), (300, 264, 7)):
        print(f"rmsnorm_bwd_noalloc {dtype} N={N} H={H}", flush=True)
        x, dy, dres, w = _inputs(N, H, dtype, seed)
        dx_a, dx_b = torch.empty_like(x), torch.empty_like(x)
        dw_a, dw_b = torch.empty_like(w), torch.empty_like(w)
        nb = sl.slide_rmsnorm_bwd_workspace_bytes(N, H)
        assert nb <= sl.slide_rmsnorm_bwd_noalloc_max_bytes()
        work = ws(nb)
        work.view(torch.uint8).fill_(0xFF)          # NaN patterns: every read must be written
        sl.slide_rmsnorm_bwd(dy, x, w, dres, dx_a, dw_a, N, H, 1e-5, code, work, nb, st)
        sl.slide_rmsnorm_bwd_noalloc(dy, x, w, dres, dx_b, dw_b, N, H, 1e-5, code, st)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(dx_a), _bits(dx_b)), "dx differs"
        assert np.array_equal(_bits(dw_a), _bits(dw_b)), "dw differs"
        assert np.isfinite(dw_b.float().cpu().numpy()).all()


def test_noalloc_rejects_sizes_beyond_its_array():
    N, H = 65536, 8192
    assert sl.slide_rmsnorm_bwd_workspace_bytes(N, H) > sl.slide_rmsnorm_bwd_noalloc_max_bytes()
    x = torch.empty((1, H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sl.SlideError) as e:
        sl.slide_rmsnorm_bwd_noalloc(x, x, x[0], None, x.clone(), x[0].clone(), N, H, 1e-5,
                                     sl.SLIDE_BF16, torch.cuda.current_stream())
    assert "fixed array" in str(e.value)
