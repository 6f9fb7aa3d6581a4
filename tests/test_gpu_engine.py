"""GPU tests of the whole training step (embedding, layers through the slot ring, final norm,
chunked CE, backward with gradient flushes and the CPU AdamW worker) against the oracle, and
the scheduler-invariance property: offloading and overlap must not change a single bit of the
result (the pages' offloaded training keeps the semantics of plain training)."""
import numpy as np
import pytest
import torch

from layer_sliding_offloaded_fwd_amd.engine import AdamW, ModelSpec, SlideEngine
from oracle import adamw as oa
from oracle import model as om
from seeded_inputs import TINY, LayerCfg, Workload, model_params, tokens
from tests._gpu import assert_close

pytestmark = pytest.mark.gpu

HP = AdamW()
OHP = oa.AdamWHyper(HP.lr, HP.beta1, HP.beta2, HP.eps, HP.weight_decay)


def _spec(w: Workload):
    c = w.layer
    return ModelSpec(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, w.vocab, w.n_layers,
                     w.dtype, c.rms_eps, c.rope_theta)


def _flat_layers(params, w):
    return [np.concatenate([lp[n].f32.reshape(-1) for n, _ in w.layer.param_shapes()])
            for lp in params["layers"]]


def _oracle_params(params):
    return dict(embed=params["embed"].f64,
                layers=[{k: v.f64 for k, v in lp.items()} for lp in params["layers"]],
                w_final=params["w_final"].f64, lm_head=params["lm_head"].f64)


def _flat_grads(g, w):
    return [np.concatenate([lg[n].reshape(-1) for n, _ in w.layer.param_shapes()])
            for lg in g["layers"]]


@pytest.mark.parametrize("ce_chunk", [8192, 256])
def test_tiny_fp32_step_matches_oracle(ce_chunk):
    """ce_chunk 8192: one LM-head chunk; 256: four, each updated, uploaded and flushed on its
    own schedule."""
    w = TINY
    print(f"engine step {w.name}: L={w.n_layers} H={w.layer.hidden} V={w.vocab} "
          f"B={w.batch} S={w.seq} ce_chunk={ce_chunk}", flush=True)
    params = model_params(w, seed=0)
    tok = tokens(w.batch, w.seq, w.vocab, seed=1)
    eng = SlideEngine(_spec(w), w.batch, w.seq, n_slots=3, hp=HP, adam_threads=4,
                      ce_chunk=ce_chunk)
    try:
        eng.load_params(params["embed"].f32, _flat_layers(params, w), params["w_final"].f32,
                        params["lm_head"].f32)
        eng.step(tok)
        loss = eng.loss()
        eng.wait_updates()
        sh = om.ModelShape(om.LayerShape(256, 4, 4, 64, 688), w.n_layers, w.vocab)
        rloss, rg = om.model_loss_and_grads(_oracle_params(params), tok, sh)
        print(f"  loss gpu {loss:.7f} oracle {rloss:.7f}", flush=True)
        assert abs(loss - rloss) <= 1e-4 * abs(rloss)
        # gradients landed in the pinned host buffers (fp32 compute keeps them separate)
        assert_close(eng.embed.grad_host.numpy(), rg["embed"].reshape(-1), "f32", "grad embed")
        assert_close(eng.final.grad_host.numpy(), rg["w_final"], "f32", "grad w_final")
        assert_close(eng.lm.grad_host.numpy(), rg["lm_head"].reshape(-1), "f32", "grad lm_head")
        for i, (gg, rr) in enumerate(zip([p.grad_host.numpy() for p in eng.layers],
                                         _flat_grads(rg, w))):
            assert_close(gg, rr, "f32", f"grad layer {i}")
        # the update applied on the host is the fixed-order fp32 AdamW of those gradients
        got = eng.master_params()
        for name, prm, p0 in [("embed", eng.embed, params["embed"].f32),
                              ("lm_head", eng.lm, params["lm_head"].f32)]:
            ref = oa.adamw_fp32(p0.reshape(-1), prm.grad_host.numpy(), np.zeros(prm.n, np.float32),
                                np.zeros(prm.n, np.float32), 1, OHP)[0]
            assert np.array_equal(got[name].view(np.uint32), ref.view(np.uint32)), name
        # a second step sees every updated parameter (synchronous semantics): its loss is the
        # oracle's loss at the parameters the first step produced
        tok2 = tokens(w.batch, w.seq, w.vocab, seed=2)
        eng.step(tok2)
        loss2 = eng.loss()
        p1 = dict(embed=got["embed"].astype(np.float64).reshape(w.vocab, -1),
                  w_final=got["w_final"].astype(np.float64),
                  lm_head=got["lm_head"].astype(np.float64).reshape(w.vocab, -1), layers=[])
        for flat in got["layers"]:
            d, o = {}, 0
            for n, shp in w.layer.param_shapes():
                k = int(np.prod(shp))
                d[n] = flat[o:o + k].astype(np.float64).reshape(shp)
                o += k
            p1["layers"].append(d)
        rloss2, _ = om.model_loss_and_grads(p1, tok2, sh)
        print(f"  step 2 loss gpu {loss2:.7f} oracle {rloss2:.7f}", flush=True)
        assert abs(loss2 - rloss2) <= 1e-4 * abs(rloss2)
    finally:
        eng.close()


SMALL = Workload("small-bf16", LayerCfg(256, 4, 2, 64, 688), 5, 1024, 2, 64, "bf16")


def _run(n_slots, serialize, steps=2, save=True, ce_chunk=256, activations=None, x_slots=4,
         w=SMALL, **kw):
    params = model_params(w, seed=0, gain_std=0.1)
    eng = SlideEngine(_spec(w), w.batch, w.seq, n_slots=n_slots, hp=HP, adam_threads=3,
                      serialize=serialize, save_activations=save, ce_chunk=ce_chunk,
                      activations=activations, x_slots=x_slots, **kw)
    try:
        eng.load_params(params["embed"].f32, _flat_layers(params, w), params["w_final"].f32,
                        params["lm_head"].f32)
        losses = []
        for s in range(steps):
            eng.step(tokens(w.batch, w.seq, w.vocab, seed=10 + s))
            losses.append(eng.loss())
        return losses, eng.master_params()
    finally:
        eng.close()


def test_offload_and_overlap_do_not_change_results():
    print("scheduler invariance: 3 slots overlapped vs serialized vs one slot per layer",
          flush=True)
    la, pa = _run(3, False)
    lb, pb = _run(3, True)
    lc, pc = _run(SMALL.n_layers, False)
    lone, pone = _run(1, False)
    lrec, prec = _run(3, False, save=False)       # backward recomputes the forward instead
    lsteps, psteps = _run(3, False, steps=3)
    # layer inputs slide to host memory (3 device slots for 5 layers) and come back
    lhost, phost = _run(3, False, activations="host", x_slots=3)
    lhost1, phost1 = _run(1, True, activations="host", x_slots=3)
    # layer 0 moved whole at the step boundary instead of in parts, and in 3 uneven parts
    lwhole, pwhole = _run(3, False, boundary_parts=1)
    lp3, pp3 = _run(3, True, boundary_parts=3)
    # only the selected embedding rows cross the link at the step boundary (packed)
    lsp, psp = _run(3, False, steps=3, embed_split=True)
    assert lsp == lsteps
    for k in ("embed", "w_final", "lm_head"):
        assert np.array_equal(psteps[k].view(np.uint32), psp[k].view(np.uint32)), k
    for x, y in zip(psteps["layers"], psp["layers"]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    # the same in fp32 (packed fp32 rows), three steps
    lt, pt = _run(3, False, steps=3, w=TINY)
    lts, pts = _run(3, False, steps=3, w=TINY, embed_split=True)
    assert lt == lts
    for k in ("embed", "w_final", "lm_head"):
        assert np.array_equal(pt[k].view(np.uint32), pts[k].view(np.uint32)), k
    for x, y in zip(pt["layers"], pts["layers"]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    print(f"  losses {la} {lb} {lc} {lone} {lrec} {lsteps} {lhost} {lhost1} {lwhole} {lp3}",
          flush=True)
    assert la == lb == lc == lone == lrec == lsteps[:2] == lhost == lhost1 == lwhole == lp3
    # one LM-head chunk instead of four: the same step up to rounding (an AdamW step moves a
    # weight by at most about lr, so rounding-level gradient differences stay below 2 lr)
    l_ch, p_ch = _run(3, True, ce_chunk=1024)
    assert all(abs(x - y) <= 2e-3 * abs(y) for x, y in zip(l_ch, la))
    assert float(np.max(np.abs(p_ch["lm_head"] - pa["lm_head"]))) <= 2.5 * HP.lr
    for other in (pb, pc, pone, prec, phost, phost1, pwhole, pp3):
        for k in ("embed", "w_final", "lm_head"):
            assert np.array_equal(pa[k].view(np.uint32), other[k].view(np.uint32)), k
        for x, y in zip(pa["layers"], other["layers"]):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_hsa_copy_engine_changes_no_bit_and_times_the_copies():
    """The slot ring's copies on chosen copy engines through the HSA runtime (copy_engine="hsa",
    the default) move the same bytes in the same order as hipMemcpyAsync ("hip"): the same losses and fp32 masters to
    the bit, overlapped and serialized; the timeline's gradient copies are timed from the copy
    threads' clocks."""
    print("copy engine: hsa vs hip", flush=True)
    la, pa = _run(3, False, steps=3, copy_engine="hip")
    lb, pb = _run(3, False, steps=3, copy_engine="hsa")
    lc, pc = _run(1, True, steps=2, copy_engine="hip")
    ld, pd = _run(1, True, steps=2, copy_engine="hsa")
    assert la == lb and lc == ld and la[:2] == lc
    for ref, other in ((pa, pb), (pc, pd)):
        for k in ("embed", "w_final", "lm_head"):
            assert np.array_equal(ref[k].view(np.uint32), other[k].view(np.uint32)), k
        for x, y in zip(ref["layers"], other["layers"]):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    params = model_params(SMALL, seed=0, gain_std=0.1)
    eng = SlideEngine(_spec(SMALL), SMALL.batch, SMALL.seq, n_slots=3, hp=HP, adam_threads=3,
                      ce_chunk=256, timeline=True, copy_engine="hsa")
    try:
        eng.load_params(params["embed"].f32, _flat_layers(params, SMALL), params["w_final"].f32,
                        params["lm_head"].f32)
        for s in range(2):
            eng.step(tokens(SMALL.batch, SMALL.seq, SMALL.vocab, seed=10 + s))
        eng.wait_updates()
        ana = eng.analyse(list(eng.records)[-1:])
        assert all(r["t_d2h_ms"] >= 0 for r in ana["layers"])
        assert sum(r["t_d2h_ms"] for r in ana["layers"]) > 0
        tl = eng.timeline_of(list(eng.records)[-1:])
        assert len(tl["d2h"]) == SMALL.n_layers
    finally:
        eng.close()


def test_bf16_model_loss_matches_oracle():
    w = SMALL
    print(f"engine step {w.name}", flush=True)
    params = model_params(w, seed=0, gain_std=0.1)
    tok = tokens(w.batch, w.seq, w.vocab, seed=10)
    eng = SlideEngine(_spec(w), w.batch, w.seq, n_slots=3, hp=HP, adam_threads=3)
    try:
        eng.load_params(params["embed"].f32, _flat_layers(params, w), params["w_final"].f32,
                        params["lm_head"].f32)
        eng.step(tok)
        loss = eng.loss()
    finally:
        eng.close()
    c = w.layer
    sh = om.ModelShape(om.LayerShape(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn),
                       w.n_layers, w.vocab)
    rloss, _ = om.model_loss_and_grads(_oracle_params(params), tok, sh)
    print(f"  loss gpu {loss:.6f} oracle {rloss:.6f}", flush=True)
    assert abs(loss - rloss) <= 2e-3 * abs(rloss)


def _block_of(name):
    """Block a CPU job belongs to: "embed3" -> "embed", "lm_head0" -> "lm_head"."""
    for b in ("embed", "lm_head"):
        if name.startswith(b):
            return b
    return name


def _oracle_from_flat(flat, w):
    """fp64 oracle parameters from flat fp32 blocks (embed, layer0.., w_final, lm_head)."""
    V, H = w.vocab, w.layer.hidden
    out = dict(embed=flat["embed"].astype(np.float64).reshape(V, H),
               w_final=flat["w_final"].astype(np.float64),
               lm_head=flat["lm_head"].astype(np.float64).reshape(V, H), layers=[])
    for i in range(w.n_layers):
        d, o = {}, 0
        for n, shp in w.layer.param_shapes():
            k = int(np.prod(shp))
            d[n] = flat[f"layer{i}"][o:o + k].astype(np.float64).reshape(shp)
            o += k
        out["layers"].append(d)
    return out


@pytest.mark.parametrize("activations", ["hbm", "host", "recompute", "hbm-embed-split"])
def test_bf16_step_gradients_updates_and_uploads_match_oracle(activations):
    """The benchmarked bf16 path, where one pinned buffer per block is both the gradient landing
    zone and the upload source and the CPU AdamW writes the new bf16 weights into it in place.
    For two steps (the second on the weights the first produced; a large learning rate makes a
    stale or misrouted upload visible in the second step's loss and gradients):
    - the loss matches the oracle's at the bf16 rounding of the current fp32 masters;
    - every gradient that lands in host memory matches the oracle's gradient (bf16 tolerance);
    - every fp32 master, first and second moment equals the fixed-order fp32 AdamW of the
      landed gradient, bit for bit;
    - every pinned buffer (the next upload source) and every resident device copy holds the
      bf16 rounding of its master, bit for bit."""
    w = SMALL
    c = w.layer
    hp = AdamW(lr=1e-2)
    ohp = oa.AdamWHyper(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
    print(f"bf16 engine vs oracle after updates: {w.name} activations={activations} "
          f"lr={hp.lr}", flush=True)
    params = model_params(w, seed=0, gain_std=0.1)
    H, V, P = c.hidden, w.vocab, c.param_count()
    sizes = dict(embed=V * H, w_final=H, lm_head=V * H, **{f"layer{i}": P
                                                              for i in range(w.n_layers)})
    landed = {}

    def on_gradient(name, step, off, g):
        blk = _block_of(name)
        arr = landed.setdefault((step, blk), np.full(sizes[blk], np.nan, np.float32))
        vals = oa.bf16_bits_to_f32(g.numpy().view(np.uint16))
        if isinstance(off, np.ndarray):       # packed rows of the split embedding
            for k, r in enumerate(off):
                arr[r * H:(r + 1) * H] = vals[k * H:(k + 1) * H]
        else:
            arr[off:off + g.numel()] = vals

    p = dict(embed=params["embed"].f32.reshape(-1), w_final=params["w_final"].f32,
             lm_head=params["lm_head"].f32.reshape(-1))
    for i, flat in enumerate(_flat_layers(params, w)):
        p[f"layer{i}"] = flat.astype(np.float32)
    m = {k: np.zeros(v.size, np.float32) for k, v in p.items()}
    vv = {k: np.zeros(v.size, np.float32) for k, v in p.items()}
    sh = om.ModelShape(om.LayerShape(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn),
                       w.n_layers, w.vocab)
    split = activations.endswith("-embed-split")
    eng = SlideEngine(_spec(w), w.batch, w.seq, n_slots=3, hp=hp, adam_threads=3, ce_chunk=256,
                      activations=activations.split("-")[0], x_slots=3,
                      on_gradient=on_gradient, embed_split=split)
    try:
        eng.load_params(p["embed"], [p[f"layer{i}"] for i in range(w.n_layers)], p["w_final"],
                        p["lm_head"])
        prm_of = dict(embed=eng.embed, w_final=eng.final, lm_head=eng.lm,
                      **{f"layer{i}": eng.layers[i] for i in range(w.n_layers)})
        for step in (1, 2):
            tok = tokens(w.batch, w.seq, w.vocab, seed=40 + step)
            eng.step(tok)
            loss = eng.loss()
            eng.wait_updates()
            torch.cuda.synchronize()
            # the oracle runs on the bf16 rounding of the masters the GPU computed with
            cur = {k: oa.bf16_bits_to_f32(oa.bf16_round_bits(a)) for k, a in p.items()}
            rloss, rg = om.model_loss_and_grads(_oracle_from_flat(cur, w), tok, sh)
            print(f"  step {step}: loss gpu {loss:.6f} oracle {rloss:.6f}", flush=True)
            assert abs(loss - rloss) <= 2e-3 * abs(rloss)
            rflat = dict(embed=rg["embed"].reshape(-1), w_final=rg["w_final"],
                         lm_head=rg["lm_head"].reshape(-1))
            for i, fl in enumerate(_flat_grads(rg, w)):
                rflat[f"layer{i}"] = fl
            got = eng.master_params()
            got_flat = dict(embed=got["embed"], w_final=got["w_final"], lm_head=got["lm_head"],
                            **{f"layer{i}": a for i, a in enumerate(got["layers"])})
            for blk in sizes:
                g = landed.pop((step, blk))
                if split and blk == "embed":
                    # only the selected rows leave the GPU; every other row's gradient is
                    # exactly zero (the oracle's gradient below must agree)
                    sel = np.zeros(V, bool)
                    sel[np.unique(tok[:, :-1])] = True
                    assert not np.isnan(g.reshape(V, H)[sel]).any(), f"step {step}: embed"
                    g.reshape(V, H)[~sel] = 0.0
                assert not np.isnan(g).any(), f"step {step} {blk}: a part never landed"
                if blk.startswith("layer"):
                    o = 0
                    for n, shp in c.param_shapes():
                        k = int(np.prod(shp))
                        assert_close(g[o:o + k], rflat[blk][o:o + k], "bf16",
                                     f"step {step} {blk} landed grad {n}")
                        o += k
                else:
                    assert_close(g, rflat[blk], "bf16", f"step {step} {blk} landed grad")
                pn, mn, vn, bits = oa.adamw_fp32(p[blk], g, m[blk], vv[blk], step, ohp)
                prm = prm_of[blk]
                assert np.array_equal(got_flat[blk].view(np.uint32), pn.view(np.uint32)), \
                    f"step {step} {blk}: master is not AdamW of the landed gradient"
                assert np.array_equal(prm.m.numpy().view(np.uint32), mn.view(np.uint32)), blk
                assert np.array_equal(prm.v.numpy().view(np.uint32), vn.view(np.uint32)), blk
                assert np.array_equal(prm.shared.numpy().view(np.uint16), bits), \
                    f"step {step} {blk}: upload buffer is not the bf16 rounding of the master"
                if hasattr(prm, "dev"):
                    dbits = prm.dev.view(torch.int16).cpu().numpy().view(np.uint16)
                    assert np.array_equal(dbits, bits), f"step {step} {blk}: device copy"
                p[blk], m[blk], vv[blk] = pn, mn, vn
        assert not landed, sorted(landed)
    finally:
        eng.close()


RAGGED = Workload("ragged-vocab-bf16", LayerCfg(256, 4, 2, 64, 688), 3, 1000, 2, 64, "bf16")


def test_ragged_vocab_chunks_match_oracle_and_serialized_run():
    """A vocabulary of 1000 rows: LM-head chunks of 256 with a ragged last one (232 rows) and
    embedding row chunks of 125 rows, each flushed, updated and uploaded on its own. Step 1's
    loss matches the oracle; two overlapped steps equal two serialized ones bit for bit."""
    w = RAGGED
    print(f"engine step {w.name}: V={w.vocab}", flush=True)
    params = model_params(w, seed=0, gain_std=0.1)
    toks = [tokens(w.batch, w.seq, w.vocab, seed=20 + s) for s in range(2)]

    def run(serialize):
        eng = SlideEngine(_spec(w), w.batch, w.seq, n_slots=2, hp=HP, adam_threads=3,
                          serialize=serialize, ce_chunk=256)
        try:
            eng.load_params(params["embed"].f32, _flat_layers(params, w),
                            params["w_final"].f32, params["lm_head"].f32)
            losses = []
            for t in toks:
                eng.step(t)
                losses.append(eng.loss())
            return losses, eng.master_params()
        finally:
            eng.close()

    la, pa = run(False)
    lb, pb = run(True)
    c = w.layer
    sh = om.ModelShape(om.LayerShape(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn),
                       w.n_layers, w.vocab)
    rloss, _ = om.model_loss_and_grads(_oracle_params(params), toks[0], sh)
    print(f"  losses overlapped {la} serialized {lb}, oracle step 1 {rloss:.6f}", flush=True)
    assert abs(la[0] - rloss) <= 2e-3 * abs(rloss)
    assert la == lb
    for k in ("embed", "w_final", "lm_head"):
        assert np.array_equal(pa[k].view(np.uint32), pb[k].view(np.uint32)), k
    for x, y in zip(pa["layers"], pb["layers"]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("w", [SMALL, TINY], ids=["bf16", "f32"])
def test_disk_tier_of_optimizer_state_changes_no_bit(tmp_path, w):
    """The optimizer state of some or all layers lives in a file (O_DIRECT where the file system
    allows; for bf16 the fp32 master too, for fp32 the moments only): three steps give the same
    losses and master weights, bit for bit, as with every state in host memory."""
    print(f"disk tier: {w.name} L={w.n_layers}", flush=True)
    la, pa = _run(3, False, steps=3, w=w)
    for layers in (None, [0, w.n_layers - 1]):
        lt, pt = _run(3, False, steps=3, w=w, state_tier=str(tmp_path / "state.bin"),
                      tier_layers=layers, tier_chunk=4096 * 3)
        print(f"  tier layers {layers}: losses {lt} (host memory {la})", flush=True)
        assert lt == la
        for k in ("embed", "w_final", "lm_head"):
            assert np.array_equal(pa[k].view(np.uint32), pt[k].view(np.uint32)), k
        for x, y in zip(pa["layers"], pt["layers"]):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert not (tmp_path / "state.bin").exists()


def test_checkpoint_resume_is_bit_exact(tmp_path):
    """Two steps in one run equal one step, a checkpoint, a new engine that loads it and one more
    step, bit for bit; also when the resumed engine keeps its optimizer state in the disk tier."""
    w = SMALL
    print(f"checkpoint/resume: {w.name}", flush=True)
    params = model_params(w, seed=0, gain_std=0.1)
    toks = [tokens(w.batch, w.seq, w.vocab, seed=30 + s) for s in range(2)]

    def engine(**kw):
        return SlideEngine(_spec(w), w.batch, w.seq, n_slots=3, hp=HP, adam_threads=3,
                           ce_chunk=256, **kw)

    def load(e):
        e.load_params(params["embed"].f32, _flat_layers(params, w), params["w_final"].f32,
                      params["lm_head"].f32)

    ref = engine()
    try:
        load(ref)
        losses = []
        for t in toks:
            ref.step(t)
            losses.append(ref.loss())
        pref = ref.master_params()
    finally:
        ref.close()
    first = engine()
    try:
        load(first)
        first.step(toks[0])
        l0 = first.loss()
        first.save_checkpoint(tmp_path / "ck")
    finally:
        first.close()
    for kw in ({}, {"state_tier": str(tmp_path / "state.bin")}):
        e = engine(**kw)
        try:
            e.load_checkpoint(tmp_path / "ck")
            assert e.step_count == 1
            e.step(toks[1])
            l1 = e.loss()
            pe = e.master_params()
        finally:
            e.close()
        print(f"  {sorted(kw)}: losses {[l0, l1]} vs uninterrupted {losses}", flush=True)
        assert [l0, l1] == losses
        for k in ("embed", "w_final", "lm_head"):
            assert np.array_equal(pref[k].view(np.uint32), pe[k].view(np.uint32)), k
        for x, y in zip(pref["layers"], pe["layers"]):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_nonfinite_gradient_check(tmp_path):
    """With check_finite the results are the same bits as without; a layer weight set to
    infinity makes that step's gradients non-finite, and the engine refuses their updates with
    SLIDE_E_NONFINITE instead of writing them into the fp32 master weights."""
    from layer_sliding_offloaded_fwd_amd._capi import SLIDE_E_NONFINITE, SlideError
    w = SMALL
    print(f"non-finite check: {w.name}", flush=True)
    la, pa = _run(3, False)
    lc, pc = _run(3, False, check_finite=True)
    assert la == lc
    for k in ("embed", "w_final", "lm_head"):
        assert np.array_equal(pa[k].view(np.uint32), pc[k].view(np.uint32)), k
    for x, y in zip(pa["layers"], pc["layers"]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))

    params = model_params(w, seed=0, gain_std=0.1)
    layers = _flat_layers(params, w)
    layers[2] = layers[2].copy()
    layers[2][w.layer.hidden + 5] = np.inf          # one entry of layer 2's Wqkv
    eng = SlideEngine(_spec(w), w.batch, w.seq, n_slots=3, hp=HP, adam_threads=3, ce_chunk=256,
                      check_finite=True)
    closed = False
    try:
        eng.load_params(params["embed"].f32, layers, params["w_final"].f32,
                        params["lm_head"].f32)
        eng.step(tokens(w.batch, w.seq, w.vocab, seed=10))
        with pytest.raises(SlideError) as e:
            eng.wait_updates()
        print(f"  raised: {e.value}", flush=True)
        assert e.value.code == SLIDE_E_NONFINITE
        # every update was refused: each master is still the loaded value (or its infinity)
        for i, prm in enumerate(eng.layers):
            assert np.array_equal(prm.master.numpy().view(np.uint32),
                                  layers[i].astype(np.float32).view(np.uint32)), i
        # close() frees everything and raises the error once more
        with pytest.raises(SlideError):
            eng.close()
        closed = True
    finally:
        if not closed:
            try:
                eng.close()
            except SlideError:
                pass


SMALL16 = Workload("small-f16", LayerCfg(256, 4, 2, 64, 688), 5, 1024, 2, 64, "f16")


def test_f16_loss_scaled_steps_match_oracle_and_overflow_skips_the_step():
    """fp16 compute with dynamic loss scaling (scale 2^16, doubled after 2 good steps):
    - steps 1 and 2: the loss matches the oracle at the fp16 rounding of the masters; every
      landed gradient divided by the step's scale matches the oracle's gradient (fp16 bound);
      masters and moments equal the fp32 AdamW contract of the landed (scaled) gradient with
      that scale, bit for bit; every upload buffer and resident device copy holds the fp16
      rounding of its master;
    - step 3 at a scale of 2^40 overflows (the CE's dz alone exceeds fp16's range): the whole
      step is skipped, so every master, moment, upload buffer and device copy keeps its bits,
      the optimizer's step count stays, and the scale is halved;
    - step 4 at 2^16 applies again, as the optimizer's third step."""
    w = SMALL16
    c = w.layer
    hp = AdamW(lr=1e-2)
    ohp = oa.AdamWHyper(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
    print(f"fp16 engine with loss scaling: {w.name}", flush=True)
    params = model_params(w, seed=0, gain_std=0.1)
    H, V, P = c.hidden, w.vocab, c.param_count()
    sizes = dict(embed=V * H, w_final=H, lm_head=V * H, **{f"layer{i}": P
                                                              for i in range(w.n_layers)})
    landed = {}

    def on_gradient(name, step, off, g):
        blk = _block_of(name)
        arr = landed.setdefault((step, blk), np.full(sizes[blk], np.nan, np.float32))
        arr[off:off + g.numel()] = oa.f16_bits_to_f32(g.numpy().view(np.uint16))

    p = dict(embed=params["embed"].f32.reshape(-1), w_final=params["w_final"].f32,
             lm_head=params["lm_head"].f32.reshape(-1))
    for i, flat in enumerate(_flat_layers(params, w)):
        p[f"layer{i}"] = flat.astype(np.float32)
    m = {k: np.zeros(v.size, np.float32) for k, v in p.items()}
    vv = {k: np.zeros(v.size, np.float32) for k, v in p.items()}
    sh = om.ModelShape(om.LayerShape(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn),
                       w.n_layers, w.vocab)
    eng = SlideEngine(_spec(w), w.batch, w.seq, n_slots=3, hp=hp, adam_threads=3, ce_chunk=256,
                      on_gradient=on_gradient, loss_scale=2.0 ** 16, scale_growth_interval=2)
    try:
        eng.load_params(p["embed"], [p[f"layer{i}"] for i in range(w.n_layers)], p["w_final"],
                        p["lm_head"])
        prm_of = dict(embed=eng.embed, w_final=eng.final, lm_head=eng.lm,
                      **{f"layer{i}": eng.layers[i] for i in range(w.n_layers)})

        def state_bits():
            out = {}
            for blk, prm in prm_of.items():
                out[blk] = (prm.master.numpy().copy(), prm.m.numpy().copy(),
                            prm.v.numpy().copy(), prm.shared.numpy().copy(),
                            prm.dev.view(torch.int16).cpu().numpy() if hasattr(prm, "dev")
                            else None)
            return out

        def applied_step(step, seed):
            scale = eng.loss_scale
            tok = tokens(w.batch, w.seq, w.vocab, seed=seed)
            eng.step(tok)
            loss = eng.loss()
            eng.wait_updates()
            torch.cuda.synchronize()
            cur = {k: oa.f16_bits_to_f32(oa.f16_round_bits(a)) for k, a in p.items()}
            rloss, rg = om.model_loss_and_grads(_oracle_from_flat(cur, w), tok, sh)
            print(f"  step {step} (scale {scale:g}): loss gpu {loss:.6f} oracle {rloss:.6f}",
                  flush=True)
            assert abs(loss - rloss) <= 2e-3 * abs(rloss)
            rflat = dict(embed=rg["embed"].reshape(-1), w_final=rg["w_final"],
                         lm_head=rg["lm_head"].reshape(-1))
            for i, fl in enumerate(_flat_grads(rg, w)):
                rflat[f"layer{i}"] = fl
            got = eng.master_params()
            got_flat = dict(embed=got["embed"], w_final=got["w_final"], lm_head=got["lm_head"],
                            **{f"layer{i}": a for i, a in enumerate(got["layers"])})
            t_adam = eng.opt_step
            for blk in sizes:
                g = landed.pop((eng.step_count, blk))
                assert not np.isnan(g).any(), f"step {step} {blk}: a part never landed"
                if blk.startswith("layer"):
                    o = 0
                    for n, shp in c.param_shapes():
                        k = int(np.prod(shp))
                        assert_close(g[o:o + k] / scale, rflat[blk][o:o + k], "f16",
                                     f"step {step} {blk} landed grad / scale {n}")
                        o += k
                else:
                    assert_close(g / scale, rflat[blk], "f16", f"step {step} {blk} landed grad")
                pn, mn, vn, bits = oa.adamw_fp32(p[blk], g, m[blk], vv[blk], t_adam, ohp,
                                                 grad_scale=scale, copy="f16")
                prm = prm_of[blk]
                assert np.array_equal(got_flat[blk].view(np.uint32), pn.view(np.uint32)), blk
                assert np.array_equal(prm.m.numpy().view(np.uint32), mn.view(np.uint32)), blk
                assert np.array_equal(prm.v.numpy().view(np.uint32), vn.view(np.uint32)), blk
                assert np.array_equal(prm.shared.numpy().view(np.uint16), bits), blk
                if hasattr(prm, "dev"):
                    dbits = prm.dev.view(torch.int16).cpu().numpy().view(np.uint16)
                    assert np.array_equal(dbits, bits), f"step {step} {blk}: device copy"
                p[blk], m[blk], vv[blk] = pn, mn, vn

        applied_step(1, 60)
        assert eng.loss_scale == 2.0 ** 16 and eng.opt_step == 1
        applied_step(2, 61)
        assert eng.loss_scale == 2.0 ** 17 and eng.opt_step == 2 and eng.skipped_steps == 0
        # step 3 overflows
        before = state_bits()
        eng.loss_scale = 2.0 ** 40
        eng.step(tokens(w.batch, w.seq, w.vocab, seed=62))
        eng.wait_updates()
        torch.cuda.synchronize()
        print(f"  step 3 (scale 2^40): skipped {eng.skipped_steps}, scale now "
              f"{eng.loss_scale:g}", flush=True)
        assert eng.skipped_steps == 1 and eng.loss_scale == 2.0 ** 39 and eng.opt_step == 2
        after = state_bits()
        for blk in before:
            for a, b in zip(before[blk], after[blk]):
                if a is not None:
                    assert np.array_equal(a, b), f"step 3 changed {blk}"
        assert not [k for k in landed if k[0] == 3], "a skipped step's gradient reached AdamW"
        # step 4 applies again, as the optimizer's third step
        eng.loss_scale = 2.0 ** 16
        applied_step(4, 63)
        assert eng.opt_step == 3 and eng.step_count == 4
    finally:
        eng.close()
