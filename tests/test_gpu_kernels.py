"""GPU parity of libslide's kernels against the fp64 oracle (and, for the GEMM, the library
matrix product the oracle uses), on seeded inputs whose sizes span several tiles and end in a
ragged tail. Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import layer_sliding_offloaded_fwd_amd as sl
from oracle import model as om
from seeded_inputs import activations
from tests._gpu import DEV, assert_close, dev, empty, host, stream, ws

pytestmark = pytest.mark.gpu


def _rng(seed):
    return np.random.default_rng(seed)


def _round(a, dtype):
    """Values the device tensor will hold (bf16 rounding via torch, as the inputs are made)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16).float()
    elif dtype == "f16":
        t = t.to(torch.float16).float()
    return t.numpy().astype(np.float64)


GEMM_SHAPES = [
    (328, 200, 136),      # small-tile path: 3 x 2 tiles of 128 with ragged edges, 3 k-tiles
    (2088, 4120, 136),    # large-tile path: 9 x 17 tiles of 256 with ragged edges
    (2090, 4121, 136),    # large-tile path, odd N and ldc: per-element stores at every row
    (4608, 4096, 520),    # full 256 x 256 tiles, more than one per compute unit (288): the
                          # bf16 store walks tiles, each next tile's loads under the last store
]


def _r8(v):
    return (v + 7) // 8 * 8


# the fp32 kernel (tiny fp32 model) has a single tile shape: only the small shape applies to it
GEMM_CASES = ([("bf16",) + s for s in GEMM_SHAPES] + [("f16",) + s for s in GEMM_SHAPES]
              + [("f32",) + s for s in GEMM_SHAPES if s[0] <= 1000])
GEMM_TOL = {"bf16": 1e-2, "f16": 2e-3, "f32": 1e-5}


@pytest.mark.parametrize("ak,bk", [(True, True), (True, False), (False, True), (False, False)])
@pytest.mark.parametrize("dtype,M,N,K", GEMM_CASES)
def test_gemm_layouts_and_ragged_tails(dtype, ak, bk, M, N, K):
    print(f"gemm {dtype} a_kmajor={ak} b_kmajor={bk} M={M} N={N} K={K}", flush=True)
    rng = _rng(1)
    A = _round(rng.standard_normal((M, K)), dtype)
    B = _round(rng.standard_normal((K, N)), dtype)
    R = _round(rng.standard_normal((M, N)), dtype)
    ref = A @ B
    # ak: [M][K] else [K][M]; bk: [N][K] else [K][N]; an outer-K operand's rows are padded to 8
    lda = K if ak else _r8(M)
    ldb = K if bk else _r8(N)
    a_mem = A if ak else np.pad(A.T, ((0, 0), (0, lda - M)))
    b_mem = B.T.copy() if bk else np.pad(B, ((0, 0), (0, ldb - N)))
    dA, dB = dev(a_mem, dtype), dev(b_mem, dtype)
    code = sl.dtype_code(dtype)
    C = empty((M, N), dtype)
    sl.slide_gemm(M, N, K, dA, lda, ak, dB, ldb, bk, C, N, code, dtype=code, stream=stream())
    torch.cuda.synchronize()
    assert_close(host(C), ref, dtype, "C = A B", tol=GEMM_TOL[dtype])
    C2 = empty((M, N), dtype)
    sl.slide_gemm(M, N, K, dA, lda, ak, dB, ldb, bk, C2, N, code, R=dev(R, dtype), ldr=N,
                  alpha=0.5, dtype=code, stream=stream())
    C3 = torch.full((M, N), 1.0, dtype=torch.float32, device=DEV)
    sl.slide_gemm(M, N, K, dA, lda, ak, dB, ldb, bk, C3, N, sl.SLIDE_F32, accumulate=True,
                  dtype=code, stream=stream())
    C4 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    sl.slide_gemm(M, N, K, dA, lda, ak, dB, ldb, bk, C4, N, sl.SLIDE_F32, dtype=code,
                  stream=stream())
    torch.cuda.synchronize()
    assert_close(host(C2), 0.5 * ref + R, dtype, "C = R + 0.5 A B", tol=GEMM_TOL[dtype])
    assert_close(host(C3), 1.0 + ref, "f32", "C += A B (fp32 accumulate)", tol=1e-5)
    assert_close(host(C4), ref, "f32", "C = A B (fp32 output)", tol=1e-5)


# Tile counts just past whole waves of the 256 compute units (384 = 1.5 waves), so the last
# 128 tiles run as two K halves each when a workspace is given; one shape with ragged edges.
TAIL_SHAPES = [(6144, 4096, 264), (6100, 4090, 264)]


@pytest.mark.parametrize("ak,bk", [(True, True), (True, False), (False, True), (False, False)])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_gemm_split_tail_matches_oracle_and_unsplit(ak, bk, M, N, K):
    print(f"gemm tail split a_kmajor={ak} b_kmajor={bk} M={M} N={N} K={K}", flush=True)
    dtype, code = "bf16", sl.SLIDE_BF16
    rng = _rng(3)
    A = _round(rng.standard_normal((M, K)), dtype)
    B = _round(rng.standard_normal((K, N)), dtype)
    R = _round(rng.standard_normal((M, N)), dtype)
    ref = A @ B
    lda = K if ak else _r8(M)
    ldb = K if bk else _r8(N)
    dA = dev(A if ak else np.pad(A.T, ((0, 0), (0, lda - M))), dtype)
    dB = dev(B.T.copy() if bk else np.pad(B, ((0, 0), (0, ldb - N))), dtype)
    nb = sl.slide_gemm_tail_workspace_bytes()
    buf = ws(nb)
    C1, C2 = empty((M, N), dtype), empty((M, N), dtype)
    sl.slide_gemm_ws(M, N, K, dA, lda, ak, dB, ldb, bk, C1, N, code, dtype=code, ws=buf,
                     ws_bytes=nb, stream=stream())
    sl.slide_gemm(M, N, K, dA, lda, ak, dB, ldb, bk, C2, N, code, dtype=code, stream=stream())
    R1 = empty((M, N), dtype)
    sl.slide_gemm_ws(M, N, K, dA, lda, ak, dB, ldb, bk, R1, N, code, R=dev(R, dtype), ldr=N,
                     alpha=0.5, dtype=code, ws=buf, ws_bytes=nb, stream=stream())
    F1 = torch.full((M, N), 1.0, dtype=torch.float32, device=DEV)
    sl.slide_gemm_ws(M, N, K, dA, lda, ak, dB, ldb, bk, F1, N, sl.SLIDE_F32, accumulate=True,
                     dtype=code, ws=buf, ws_bytes=nb, stream=stream())
    torch.cuda.synchronize()
    assert_close(host(C1), ref, dtype, "C = A B (split tail)", tol=GEMM_TOL[dtype])
    assert_close(host(R1), 0.5 * ref + R, dtype, "C = R + 0.5 A B (split tail)",
                 tol=GEMM_TOL[dtype])
    assert_close(host(F1), 1.0 + ref, "f32", "C += A B (split tail, fp32)", tol=1e-5)
    # tiles outside the tail are computed exactly as without the split; the tail's 128 tiles
    # differ at most by the rounding of the one addition of the two halves
    ndiff = int((_bits(C1) != _bits(C2)).sum())
    print(f"  elements differing from the unsplit GEMM: {ndiff}", flush=True)
    assert ndiff <= 128 * 256 * 256
    assert_close(host(C1), host(C2), dtype, "split vs unsplit", tol=1e-2)


# (M, F, K): fused launches (both directions) with ragged rows, a ragged last tile (F % 128 and
# F % 256 != 0) and a partial k-tile; the same with full tiles and a steady k loop; a size below
# the pipelined kernel's threshold (the GEMM and the elementwise kernel run instead)
SWIGLU_SHAPES = [(2088, 4040, 136), (2048, 4096, 520), (300, 264, 72)]


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,F,K", SWIGLU_SHAPES)
def test_gemm_swiglu_fused_equals_separate_and_oracle(dtype, M, F, K):
    print(f"gemm+swiglu {dtype} M={M} F={F} K={K}", flush=True)
    rng = _rng(7)
    code = sl.dtype_code(dtype)
    x = _round(rng.standard_normal((M, K)), dtype)
    w = _round(rng.standard_normal((2 * F, K)) / np.sqrt(K), dtype)
    dx, dw = dev(x, dtype), dev(w, dtype)
    gu1, m1 = empty((M, 2 * F), dtype), empty((M, F), dtype)
    sl.slide_gemm_swiglu_fwd(M, F, K, dx, K, dw, K, gu1, m1, code, stream())
    gu2, m2 = empty((M, 2 * F), dtype), empty((M, F), dtype)
    sl.slide_gemm(M, 2 * F, K, dx, K, True, dw, K, True, gu2, 2 * F, code, dtype=code,
                  stream=stream())
    sl.slide_swiglu_fwd(gu2, m2, M, F, code, stream())
    torch.cuda.synchronize()
    assert torch.equal(_bits(gu1), _bits(gu2)), "fused gu differs from the plain GEMM's"
    assert torch.equal(_bits(m1), _bits(m2)), "fused m differs from the elementwise kernel's"
    ref = x @ w.T
    assert_close(host(gu1), ref, dtype, "gu = x W_gu^T", tol=GEMM_TOL[dtype])
    assert_close(host(m1), om.swiglu_fwd(ref[:, :F], ref[:, F:]), dtype, "m = SwiGLU(gu)")

    # backward: dm = dy W_d (W_d [K][F]), then SwiGLU's backward at the stored gu
    dy = _round(rng.standard_normal((M, K)), dtype)
    wd = _round(rng.standard_normal((K, F)) / np.sqrt(K), dtype)
    ddy, dwd = dev(dy, dtype), dev(wd, dtype)
    need = sl.slide_gemm_swiglu_bwd_workspace_bytes(M, F, code)
    dgu1 = empty((M, 2 * F), dtype)
    buf = ws(need) if need else None
    sl.slide_gemm_swiglu_bwd(M, F, K, ddy, K, dwd, F, gu1, dgu1, code, buf, need, stream())
    dm2, dgu2 = empty((M, F), dtype), empty((M, 2 * F), dtype)
    sl.slide_gemm(M, F, K, ddy, K, True, dwd, F, False, dm2, F, code, dtype=code, stream=stream())
    sl.slide_swiglu_bwd(dm2, gu1, dgu2, M, F, code, stream())
    torch.cuda.synchronize()
    assert torch.equal(_bits(dgu1), _bits(dgu2)), "fused dgu differs from the separate kernels'"
    g, u = host(gu1)[:, :F], host(gu1)[:, F:]
    dg_ref, du_ref = om.swiglu_bwd(dy @ wd, g, u)
    got = host(dgu1)
    assert_close(got[:, :F], dg_ref, dtype, "dg")
    assert_close(got[:, F:], du_ref, dtype, "du")
    print(f"  fused launch: {need == 0}", flush=True)


# N = 300 and 517: several 64-row partial sums of the weight gradient, the last one ragged
@pytest.mark.parametrize("dtype,H,N", [("bf16", 4096, 37), ("f32", 256, 37), ("bf16", 264, 300),
                                       ("f32", 200, 517), ("f16", 4096, 37), ("f16", 264, 300)])
def test_rmsnorm_fwd_bwd(dtype, H, N):
    print(f"rmsnorm {dtype} N={N} H={H}", flush=True)
    x = activations((N, H), dtype, 5).f64
    w = _round(1.0 + 0.1 * _rng(6).standard_normal(H), dtype)
    dy = activations((N, H), dtype, 7).f64
    dres = activations((N, H), dtype, 8).f64
    code = sl.dtype_code(dtype)
    dx_, x_, w_, dy_, dres_ = (dev(a, dtype) for a in (x, x, w, dy, dres))
    y = empty((N, H), dtype)
    rstd = torch.empty(N, dtype=torch.float32, device=DEV)
    sl.slide_rmsnorm_fwd(x_, w_, y, rstd, N, H, 1e-5, code, stream())
    dx = empty((N, H), dtype)
    dw = empty((H,), dtype)
    wsz = sl.slide_rmsnorm_bwd_workspace_bytes(N, H)
    sl.slide_rmsnorm_bwd(dy_, x_, w_, dres_, dx, dw, N, H, 1e-5, code, ws(wsz), wsz, stream())
    torch.cuda.synchronize()
    ry, rr = om.rmsnorm_fwd(x, w, 1e-5)
    rdx, rdw = om.rmsnorm_bwd(dy, x, w, rr)
    assert_close(host(y), ry, dtype, "rmsnorm y")
    assert_close(host(rstd), rr[:, 0], "f32", "rmsnorm rstd", tol=1e-5)
    assert_close(host(dx), rdx + dres, dtype, "rmsnorm dx + residual")
    assert_close(host(dw), rdw, dtype, "rmsnorm dw")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f16", 128)])
def test_rope_forward_and_inverse(dtype, d):
    B, S, nq, nkv = 2, 77, 4, 2
    print(f"rope {dtype} d={d} S={S}", flush=True)
    QR = (nq + 2 * nkv) * d
    qkv = activations((B * S, QR), dtype, 9).f64
    t = dev(qkv, dtype)
    code = sl.dtype_code(dtype)
    wsz = 2 * 4 * S * d + 1024
    w = ws(wsz)
    sl.slide_rope(t, B, S, nq, nkv, d, 10000.0, 0, code, w, wsz, stream())
    torch.cuda.synchronize()
    out = host(t).reshape(B, S, -1)
    cos, sin = om.rope_tables(S, d, 10000.0)
    x = qkv.reshape(B, S, -1)
    rq = om.rope_rotate(x[..., : nq * d].reshape(B, S, nq, d), cos, sin).reshape(B, S, -1)
    rk = om.rope_rotate(x[..., nq * d:(nq + nkv) * d].reshape(B, S, nkv, d), cos, sin).reshape(B, S, -1)
    assert_close(out[..., : nq * d], rq, dtype, "rope q")
    assert_close(out[..., nq * d:(nq + nkv) * d], rk, dtype, "rope k")
    assert np.array_equal(out[..., (nq + nkv) * d:], x[..., (nq + nkv) * d:]), "v must be untouched"
    sl.slide_rope(t, B, S, nq, nkv, d, 10000.0, 1, code, w, wsz, stream())
    torch.cuda.synchronize()
    assert_close(host(t), qkv, dtype, "rope inverse restores the input")


@pytest.mark.parametrize("dtype,B,S,nq,nkv,d", [
    ("bf16", 2, 200, 8, 2, 128),     # GQA, ragged sequence (not a multiple of 64 or 128)
    ("bf16", 1, 128, 4, 4, 64),      # MHA, head_dim 64
    ("bf16", 1, 1, 4, 1, 128),       # a single token: o = v
    ("f32", 2, 128, 4, 4, 64),
    ("f16", 2, 200, 8, 2, 128),
    ("f16", 1, 128, 4, 4, 64),
])
def test_attention_fwd_bwd(dtype, B, S, nq, nkv, d):
    print(f"attention {dtype} B={B} S={S} nq={nq} nkv={nkv} d={d}", flush=True)
    QR = (nq + 2 * nkv) * d
    qkv = activations((B * S, QR), dtype, 21).f64
    do = activations((B * S, nq * d), dtype, 22).f64
    code = sl.dtype_code(dtype)
    t_qkv, t_do = dev(qkv, dtype), dev(do, dtype)
    o = empty((B * S, nq * d), dtype)
    lse = torch.empty(B * nq * S, dtype=torch.float32, device=DEV)
    sl.slide_attention_fwd(t_qkv, o, lse, B, S, nq, nkv, d, code, stream())
    dqkv = torch.full((B * S, QR), float("nan"), dtype=o.dtype, device=DEV)
    wsz = sl.slide_attention_bwd_workspace_bytes(B, S, nq)
    sl.slide_attention_bwd(t_qkv, o, lse, t_do, dqkv, B, S, nq, nkv, d, code, ws(wsz), wsz,
                           stream())
    torch.cuda.synchronize()
    x = qkv.reshape(B, S, -1)
    q = x[..., : nq * d].reshape(B, S, nq, d)
    k = x[..., nq * d:(nq + nkv) * d].reshape(B, S, nkv, d)
    v = x[..., (nq + nkv) * d:].reshape(B, S, nkv, d)
    ro, rlse, P = om.attention_fwd(q, k, v)
    # the backward consumes the o the GPU stored (bf16-rounded), as the layer does
    dq, dk, dv = om.attention_bwd(do.reshape(B, S, nq, d), q, k, v, P)
    assert_close(host(o).reshape(B, S, nq, d), ro, dtype, "attention o")
    assert_close(host(lse).reshape(B, nq, S), rlse, "f32", "attention lse",
                 tol=1e-4 if dtype == "f32" else 2e-3)
    g = host(dqkv).reshape(B, S, -1)
    # with one token dS = P (dP - D) is exactly zero: measure dq, dk against the size of dv
    assert_close(g[..., : nq * d].reshape(B, S, nq, d), dq, dtype, "attention dq",
                 scale=float(np.max(np.abs(dv))))
    assert_close(g[..., nq * d:(nq + nkv) * d].reshape(B, S, nkv, d), dk, dtype, "attention dk",
                 scale=float(np.max(np.abs(dv))))
    assert_close(g[..., (nq + nkv) * d:].reshape(B, S, nkv, d), dv, dtype, "attention dv")


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_embedding_fwd_bwd_repeated_tokens(dtype):
    N, H, V = 300, 264, 40           # small vocabulary: every token repeats several times
    print(f"embedding {dtype} N={N} H={H} V={V}", flush=True)
    E = activations((V, H), dtype, 31).f64
    tok = _rng(32).integers(0, V, N).astype(np.int32)
    tok[5] = 7
    tok[6] = 7
    dx = activations((N, H), dtype, 33).f64
    code = sl.dtype_code(dtype)
    t_tok = torch.from_numpy(tok).to(DEV)
    x = empty((N, H), dtype)
    sl.slide_embed_fwd(dev(E, dtype), t_tok, x, N, H, V, code, stream())
    dE = torch.full((V, H), float("nan"), dtype=x.dtype, device=DEV)
    wsz = sl.slide_embed_bwd_workspace_bytes(N, V)
    sl.slide_embed_bwd(dev(dx, dtype), t_tok, dE, N, H, V, code, ws(wsz), wsz, stream())
    torch.cuda.synchronize()
    assert np.array_equal(host(x), E[tok]), "gather must be exact"
    assert_close(host(dE), om.embedding_bwd(dx, tok, V), dtype, "embedding dE")
    # deterministic: a second run gives identical bits
    dE2 = torch.empty_like(dE)
    sl.slide_embed_bwd(dev(dx, dtype), t_tok, dE2, N, H, V, code, ws(wsz), wsz, stream())
    torch.cuda.synchronize()
    assert torch.equal(dE.view(torch.int16) if dtype != "f32" else dE,
                       dE2.view(torch.int16) if dtype != "f32" else dE2)


@pytest.mark.parametrize("row_bytes", [16, 528, 8192])
def test_copy_rows_gather_scatter_exact(row_bytes):
    """Row gather (listed source rows into a packed matrix), scatter (packed rows into listed
    destination rows) and both at once move exactly the listed rows, bit for bit; rows not
    listed stay as they were; listed indices outside a matrix are skipped."""
    print(f"copy_rows row_bytes={row_bytes}", flush=True)
    rng = np.random.default_rng(5)
    V, n = 37, 12
    w = row_bytes // 4
    table = torch.from_numpy(rng.integers(0, 2**31, (V, w), dtype=np.int64).astype(np.int32)).to(DEV)
    rows = np.array([36, 0, 5, 17, 3, 30, 31, 9, 12, 1, 22, 8], np.int32)
    t_rows = torch.from_numpy(rows).to(DEV)
    packed = torch.full((n, w), -1, dtype=torch.int32, device=DEV)
    sl.slide_copy_rows(table, t_rows, V, packed, None, n, n, row_bytes, stream())
    torch.cuda.synchronize()
    assert torch.equal(packed.cpu(), table.cpu()[torch.from_numpy(rows).long()])
    dst = torch.zeros((V, w), dtype=torch.int32, device=DEV)
    sl.slide_copy_rows(packed, None, n, dst, t_rows, V, n, row_bytes, stream())
    torch.cuda.synchronize()
    want = torch.zeros((V, w), dtype=torch.int32)
    want[torch.from_numpy(rows).long()] = table.cpu()[torch.from_numpy(rows).long()]
    assert torch.equal(dst.cpu(), want)
    # both lists at once, with two indices out of range (skipped, nothing else touched)
    src_rows = torch.from_numpy(np.array([2, 40, 7, -1], np.int32)).to(DEV)
    dst_rows = torch.from_numpy(np.array([10, 11, 99, 12], np.int32)).to(DEV)
    dst2 = torch.zeros((V, w), dtype=torch.int32, device=DEV)
    sl.slide_copy_rows(table, src_rows, V, dst2, dst_rows, V, 4, row_bytes, stream())
    torch.cuda.synchronize()
    want2 = torch.zeros((V, w), dtype=torch.int32)
    want2[10] = table.cpu()[2]
    assert torch.equal(dst2.cpu(), want2)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("n", [0, 5, 8, 1000003])
def test_nonfinite_count_exact(dtype, n):
    """Exact count of NaN / +inf / -inf among finite values of every size class (including the
    largest finite value and denormals), with a ragged tail; the counter is overwritten."""
    print(f"nonfinite count {dtype} n={n}", flush=True)
    rng = _rng(40)
    a = rng.standard_normal(n).astype(np.float32)
    big = {"bf16": 3.3e38, "f32": 3.4e38, "f16": 65504.0}[dtype]
    special = np.array([np.nan, np.inf, -np.inf, big, -big, 1e-40, 0.0, -0.0], np.float32)
    if n:
        idx = rng.choice(n, size=min(n, 64), replace=False)
        a[idx] = special[rng.integers(0, len(special), len(idx))]
        a[-1] = np.inf                                  # the last element sits in the tail
    t = dev(a, dtype) if n else empty((8,), dtype)
    want = int(np.sum(~np.isfinite(_round(a, dtype)))) if n else 0
    cnt = torch.full((1,), 12345, dtype=torch.int32, device=DEV)
    sl.slide_nonfinite_count(t, sl.dtype_code(dtype), n, cnt, stream())
    torch.cuda.synchronize()
    print(f"  count {int(cnt.item())} expected {want}", flush=True)
    assert int(cnt.item()) == want


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_convert_f32_matches_oracle_rounding(dtype):
    """The GPU fp32 -> 16-bit conversion rounds to nearest-even exactly as the oracle's rounding
    and the host conversion do, for every non-NaN input: random bit patterns cover every exponent
    (subnormals and overflow to infinity included), plus signed zeros, infinities, ties and the
    half-precision limits; NaN stays NaN. The length spans many workgroups with a ragged tail."""
    print(f"convert_f32 {dtype}", flush=True)
    from oracle import adamw as oa
    code = sl.dtype_code(dtype)
    rng = np.random.default_rng(11)
    n = 70_001
    x = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32).copy()
    special = [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-45, 65504.0,
               65520.0, 1.00390625, 1.01171875, 1.0 + 2.0**-11, np.nan]
    x[:len(special)] = np.array(special, np.float32)
    ref = oa.bf16_round_bits(x) if dtype == "bf16" else oa.f16_round_bits(x)
    host_out = np.zeros(n, np.uint16)
    sl.slide_cpu_convert_f32(x, host_out, code, n, 4)
    out = torch.empty(n, dtype=torch.int16, device=DEV)
    sl.slide_convert_f32(torch.from_numpy(x).to(DEV), out, code, n, stream())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    nan_in = np.isnan(x)
    exp_mask, man_mask = (0x7F80, 0x007F) if dtype == "bf16" else (0x7C00, 0x03FF)
    got_nan = ((got & exp_mask) == exp_mask) & ((got & man_mask) != 0)
    assert np.array_equal(got_nan, nan_in)
    assert np.array_equal(got[~nan_in], ref[~nan_in])
    assert np.array_equal(got[~nan_in], host_out[~nan_in])
    with pytest.raises(sl.SlideError):
        sl.slide_convert_f32(torch.from_numpy(x).to(DEV), out, sl.SLIDE_F32, n, stream())


def test_host_link_engine_rates_time_every_engine():
    """The host-link diagnostic times a copy on every copy engine in both directions (16 MB),
    reports the engine counts and preferred masks, moves the bytes it claims to (the host buffer
    ends up holding the device bytes after the device-to-host copies) and refuses unpinned host
    memory."""
    print("host_link_engine_rates 16 MB", flush=True)
    n = 16 << 20
    dev = torch.full((n,), 7, dtype=torch.uint8, device=DEV)
    host = torch.zeros(n, dtype=torch.uint8, pin_memory=True)
    d2h, h2d, info = sl.slide_host_link_engine_rates(dev, host, n, 1)
    timed = [e for e in range(32) if d2h[e] > 0 and h2d[e] > 0]
    assert len(timed) >= 1 and info[0] + info[1] >= len(timed)
    assert all(t == -1.0 for e, t in enumerate(d2h) if e not in timed and h2d[e] < 0)
    if info[2]:
        assert any(info[2] >> e & 1 for e in timed)
    assert bool(torch.all(host == 7))   # the last copy before the h2d pass was device -> host
    with pytest.raises(sl.SlideError):
        sl.slide_host_link_engine_rates(dev, np.zeros(n, np.uint8), n, 1)
