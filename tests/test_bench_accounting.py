"""The bench's work accounting against the algorithmic totals worked out independently for the
Llama-3-8B-shaped step (hot-path scope table): a wrong flop or byte count would misstate every
reported rate, so these are pinned on the CPU."""
import types

import pytest

import bench
from seeded_inputs import L8B

LAYER_FWD = ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attn_fwd")
LAYER_BWD = ("gemm_qkv_dx", "gemm_qkv_dw", "gemm_o_dx", "gemm_o_dw", "gemm_gate_up_dx",
             "gemm_gate_up_dw", "gemm_down_dx", "gemm_down_dw", "attn_bwd_dkv", "attn_bwd_dq")


def _spec():
    c = L8B.layer
    return types.SimpleNamespace(hidden=c.hidden, ffn=c.ffn, head_dim=c.head_dim,
                                 n_heads=c.n_heads, n_kv_heads=c.n_kv_heads, vocab=L8B.vocab)


def test_layer_flops_match_the_algorithmic_totals():
    alg, exe = bench.kernel_flops(_spec(), L8B.batch, L8B.seq, L8B.ce_chunk)
    # one causal S x S x d product over all heads: d * S(S+1) * B * nq (2 flops per pair / 2)
    U = 128 * 1024 * 1025 * 8 * 32
    assert alg["attn_fwd"] == 2 * U
    assert alg["attn_bwd_dkv"] + alg["attn_bwd_dq"] == 4 * U
    fwd = sum(alg[k] for k in LAYER_FWD)
    bwd = sum(alg[k] for k in LAYER_BWD)
    assert fwd == pytest.approx(3.642e12, rel=1e-3)        # 444.6 MF/token at N = 8192
    assert bwd == pytest.approx(2 * fwd, rel=1e-12)         # every product twice
    assert fwd + bwd == pytest.approx(1333.8e6 * 8192, rel=1e-3)
    # projections: 2 M N K
    assert alg["gemm_gate_up"] == 2 * 8192 * 2 * 14336 * 4096
    assert alg["gemm_qkv"] == 2 * 8192 * (32 + 16) * 128 * 4096
    # executed attention work includes the recomputed scores (twice in the dK / dV launch, once
    # per output) and dP (in its dK half and in the dQ kernel)
    assert exe["attn_bwd_dkv"] == 5 * U and exe["attn_bwd_dq"] == 3 * U


def test_cross_entropy_flops_per_chunk():
    alg, exe = bench.kernel_flops(_spec(), L8B.batch, L8B.seq, L8B.ce_chunk)
    nch = -(-L8B.vocab // L8B.ce_chunk)
    per = 2 * 8192 * L8B.vocab * 4096 / nch
    # algorithmically the logits once, dh and dW once; the logits GEMM runs twice
    assert alg["ce_stats_gemm"] + alg["ce_dz_gemm"] == pytest.approx(per)
    assert exe["ce_stats_gemm"] == exe["ce_dz_gemm"] == pytest.approx(per)
    assert alg["ce_dh_gemm"] == alg["ce_dw_gemm"] == pytest.approx(per)
    # the 8B step's CE: three 2 N V H products = 25.8 TF
    assert 3 * per * nch == pytest.approx(25.8e12, rel=2e-3)


def test_hbm_bytes_of_the_memory_bound_kernels():
    b = bench.kernel_bytes(_spec(), L8B.batch, L8B.seq)
    N, H, F = 8192, 4096, 14336
    assert b["rmsnorm_fwd"] == 2 * N * H * 2                 # read x, write y
    assert b["swiglu_fwd"] == 3 * N * F * 2                  # read g, u; write m
    assert b["swiglu_bwd"] == 5 * N * F * 2                  # read dm, g, u; write dg, du
    assert b["rope_fwd"] == 2 * N * 40 * 128 * 2             # q and k heads, read and written
    assert b["attn_delta"] == 2 * N * 4096 * 2 + N * 32 * 12


def test_step_host_bytes():
    """Per step: AdamW moves 28 B per parameter (224.8 GB), the uploads are 28.7 GB and the
    gradient flushes 16.1 GB."""
    assert L8B.layer.param_count() == 218_112_000
    adam, h2d, d2h = bench.step_host_bytes(L8B)
    assert adam == 28 * 8_030_261_248
    assert adam == pytest.approx(224.8e9, rel=1e-3)
    assert h2d == pytest.approx(28.7e9, rel=2e-3)
    assert d2h == pytest.approx(16.06e9, rel=1e-3)


def test_overlap_table_checks_the_pages_condition(tmp_path):
    """Layer i is covered when the backward of layer i-1 takes at least T_d2h(i) + T_update(i);
    only the last step's rows are written, from the last layer down."""
    rows = []
    for step in (1, 2):
        for i, (tb, td, tu) in enumerate([(10.0, 3.0, 6.0), (9.0, 3.0, 6.0), (8.0, 4.0, 5.0)]):
            rows.append(dict(step=step, layer=i, t_bwd_ms=tb + step, t_d2h_ms=td, t_update_ms=tu))
    path = tmp_path / "t.csv"
    bench._write_overlap_table(str(path), rows)
    lines = path.read_text().strip().split("\n")
    assert lines[0].startswith("layer,t_bwd_ms")
    got = [line.split(",") for line in lines[1:]]
    assert [int(r[0]) for r in got] == [2, 1, 0]
    # layer 2: below it layer 1 takes 11 >= 4 + 5; layer 1: layer 0 takes 12 >= 3 + 6; layer 0:
    # nothing below
    assert [int(r[-1]) for r in got] == [1, 1, 0]
    assert got[0][4] == "11.000" and got[2][4] == "nan"


def test_tier_report_rates():
    class Eng:
        tier_layers = [30, 31]
        def tier_stats(self):
            return dict(bytes_read=3 * 10**9 + 100, bytes_written=3 * 10**9 + 100, busy_s=2.5,
                        stall_s=1.0, direct=True, capacity=5 * 10**9, chunk=4 << 20)
    before = dict(bytes_read=100, bytes_written=100, busy_s=0.5, stall_s=0.0)
    r = bench._tier_report(Eng(), before, steps=2, step_s=2.0)
    assert r["read_bytes_per_step"] == r["write_bytes_per_step"] == 1.5e9
    assert r["update_s_per_step"] == 1.0 and r["io_wait_s_per_step"] == 0.5
    assert r["read_plus_write_gbs"] == 3.0          # 6 GB over 2 s of tier calls
    assert r["frac_of_step"] == 0.5 and r["layers"] == 2 and r["direct_io"] is True


def test_text_timeline_lanes():
    """A column shows the activity covering at least half of it, ':' when 10-50% of it is
    busy, '.' when idle."""
    from layer_sliding_offloaded_fwd_amd.engine import SlideEngine
    tl = dict(gpu=[("F", "layer0 fwd", 0, 9), ("C", "ce", 30, 45), ("B", "layer0 bwd", 50, 58)],
              d2h=[("#", "layer0 grads", 58, 66)],
              cpu=[("e", "embed0", 5, 14), ("u", "layer0", 66, 85)])
    out = SlideEngine.render_timeline(tl, 5.0).split("\n")
    assert out[0] == "GPU |FF....CCC.BB.....|"
    assert out[1] == "D2H |...........:#:...|"      # 58-66 ms: 40%, 100%, 20% of columns
    assert out[2] == "CPU |.ee..........uuuu|"


def test_noop_step_replay_worked_example():
    """4 layers through 2 slots, worked out by hand: loads of layers 0, 1 and the embedding end
    at 1.5, 3, 4; the forward runs 4.5-9.5 (layer 2 waits for its load until 7, layer 3 until
    8.5); the head 9.5-12.5; the backward's reloads of layers 1 and 0 end at 16 and 18, so the
    backward runs 12.5-20.5; the embedding's backward ends the step at 21."""
    t = bench.noop_step_replay([1, 1, 1, 1], [2, 2, 2, 2], 2, 0.5, 3.0, 0.5, 1.5, 1.0, 1.0)
    assert t == pytest.approx(21.0, abs=1e-12)


def test_noop_step_replay_limits():
    L, S = 32, 3
    # uploads free: the step is the GPU's work
    t = bench.noop_step_replay([2.0] * L, [5.0] * L, S, 0.1, 20.0, 1.0, 0.0, 0.0, 0.0)
    assert t == pytest.approx(2.0 * L + 5.0 * L + 20.0 + 1.1)
    # GPU free: the step is the upload link's work (every layer twice except the resident
    # slots, the embedding and the LM head), plus nothing else
    t = bench.noop_step_replay([0.0] * L, [0.0] * L, S, 0.0, 0.0, 0.0, 8.0, 18.0, 18.0)
    assert t == pytest.approx((2 * L - S) * 8.0 + 18.0 + 18.0)
    # one slot: no load can run ahead of the layer that holds the slot
    t = bench.noop_step_replay([1.0] * 4, [1.0] * 4, 1, 0.0, 0.0, 0.0, 2.0, 0.0, 0.0)
    assert t == pytest.approx(4 * (2.0 + 1.0) + 1.0 + 3 * (2.0 + 1.0))
