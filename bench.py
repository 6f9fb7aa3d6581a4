#!/usr/bin/env python3
"""Train tokens/s of the layer-sliding offloaded fine-tuning step on one MI355X.

Workload: a Llama-3-8B-shaped decoder (32 layers, hidden 4096, 32 q / 8 kv heads x 128, SwiGLU
14336, vocab 128256), batch 8 x 1024 uniform random tokens, weights N(0, 0.02), bf16 compute with
fp32 master weights and AdamW state in host memory, layers streamed through a 3-slot HBM ring.
One step = embedding, 32 layer forwards, final norm + chunked LM-head CE (fwd+bwd), 32 layer
backwards, every gradient flushed to host memory and every parameter updated by the CPU AdamW,
including the weight uploads the next step needs. The token batch is resident on the GPU when
the timed region starts; weight streaming is part of the method and stays inside the step.

Prints ONE JSON line. `roofline` is for the dominant GPU kernel (by total time), timed with HIP
events on the stream it runs on; `cpu_baseline` is the fp64 oracle timed on a bounded sample on
this host's cores and scaled to the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def _die_multi_gpu(n):
    print(f"bench.py runs on one GPU only (asked for --gpus {n}); this build has no multi-GPU "
          f"path.", file=sys.stderr)
    sys.exit(2)


def kernel_flops(spec, B, S, ce_chunk):
    """Algorithmic and executed flops per launch of each named MFMA kernel."""
    N, H, F, d = B * S, spec.hidden, spec.ffn, spec.head_dim
    nq, nkv, V = spec.n_heads, spec.n_kv_heads, spec.vocab
    QR, OD = (nq + 2 * nkv) * d, nq * d
    g = {
        "gemm_qkv": 2 * N * QR * H, "gemm_o": 2 * N * H * OD, "gemm_gate_up": 2 * N * 2 * F * H,
        "gemm_down": 2 * N * H * F,
    }
    for k in list(g):
        g[k + "_dx"] = g[k]
        g[k + "_dw"] = g[k]
    U = d * S * (S + 1) * B * nq        # one causal S x S x d matrix product, all heads
    alg = dict(g)
    exe = dict(g)
    # backward, algorithmically dV, dP, dK and dQ once each; the kernels recompute the scores
    # (dV, dK and dQ kernels) and dP (dK and dQ kernels)
    # dK and dV run as one launch: 2 causal matmuls for dK (dS^T Q and dP), 1 for dV (P^T dO);
    # executed, the scores are recomputed in both halves and dP in the dK half
    alg.update(attn_fwd=2 * U, attn_bwd_dkv=3 * U, attn_bwd_dq=1 * U)
    exe.update(attn_fwd=2 * U, attn_bwd_dkv=5 * U, attn_bwd_dq=3 * U)
    nch = (V + ce_chunk - 1) // ce_chunk
    per = 2 * N * V * H / nch           # average per chunk launch
    # the logits run twice (statistics pass, then recomputed with dz fused); algorithmically once
    alg.update(ce_stats_gemm=per / 2, ce_dz_gemm=per / 2, ce_logits_gemm=per / 2, ce_dh_gemm=per,
               ce_dw_gemm=per)
    exe.update(ce_stats_gemm=per, ce_dz_gemm=per, ce_logits_gemm=per, ce_dh_gemm=per,
               ce_dw_gemm=per)
    return alg, exe


LAYER_KERNEL_PREFIXES = ("gemm_", "attn_", "rmsnorm_", "rope", "swiglu_")


def _layer_kernel_ms(kernels):
    """Total time of the decoder layers' kernels (projections, attention, RMSNorm, RoPE, SwiGLU);
    the LM head's cross-entropy GEMMs are named ce_*."""
    return sum(k["total_ms"] for n, k in kernels.items() if n.startswith(LAYER_KERNEL_PREFIXES))


def kernel_bytes(spec, B, S):
    """Algorithmic HBM bytes per launch of the memory-bound kernels (bf16 tensors)."""
    N, H, F, d = B * S, spec.hidden, spec.ffn, spec.head_dim
    QR = (spec.n_heads + 2 * spec.n_kv_heads) * d
    OD = spec.n_heads * d
    return {"rmsnorm_fwd": 2 * N * H * 2, "rmsnorm_bwd": 4 * N * H * 2,
            "rmsnorm_dw": 2 * N * H * 2,             # dy and x read; the partials are small
            "swiglu_fwd": 3 * N * F * 2, "swiglu_bwd": 5 * N * F * 2,
            "rope_fwd": 2 * N * (QR - spec.n_kv_heads * d) * 2,
            "rope_bwd": 2 * N * (QR - spec.n_kv_heads * d) * 2,
            # O and dO read; per query and head D written, lse read, lse * log2(e) written
            "attn_delta": 2 * N * OD * 2 + N * spec.n_heads * 12}


def cpu_baseline(w, B1=2, S1=1024, n_ce=1024, ad_frac=1.0):
    """The oracle (NumPy fp64) timed on a bounded sample of the same workload, scaled to the
    workload's tokens/s: one layer fwd+bwd at B1 x S1 tokens, the LM-head CE on n_ce tokens at
    the full vocabulary, and the fp32 AdamW on ad_frac of one layer's parameters (about 10 s of
    CPU work for the 8B shapes)."""
    from oracle import adamw as oa
    from oracle import model as om
    from seeded_inputs import activations, layer_params
    c = w.layer
    shape = om.LayerShape(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn)
    p = {k: v.f64 for k, v in layer_params(c, "bf16", seed=0).items()}
    x = activations((B1, S1, c.hidden), "bf16", 1).f64
    dy = activations((B1, S1, c.hidden), "bf16", 2).f64
    t0 = time.perf_counter()
    y, cache = om.layer_fwd(p, x, shape)
    om.layer_bwd(p, dy, cache, shape)
    t_layer = time.perf_counter() - t0
    del p, cache
    rng = np.random.default_rng(3)
    h = rng.standard_normal((n_ce, c.hidden))
    wl = rng.standard_normal((w.vocab, c.hidden)) * 0.02
    t = rng.integers(0, w.vocab, n_ce)
    t0 = time.perf_counter()
    om.ce_chunked(h, wl, t, w.ce_chunk)
    t_ce = time.perf_counter() - t0
    del wl
    n_ad = int(c.param_count() * ad_frac)
    pa = rng.standard_normal(n_ad).astype(np.float32)
    ga = (rng.standard_normal(n_ad) * 1e-3).astype(np.float32)
    z = np.zeros(n_ad, np.float32)
    t0 = time.perf_counter()
    oa.adamw_fp32(pa, ga, z, z, 1, oa.AdamWHyper())
    t_ad = time.perf_counter() - t0
    n_params = w.n_layers * c.param_count() + 2 * w.vocab * c.hidden + c.hidden
    tokens = w.batch * w.seq
    step_s = (tokens / (B1 * S1)) * w.n_layers * t_layer + (tokens / n_ce) * t_ce + \
        (n_params / n_ad) * t_ad
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = len(os.sched_getaffinity(0))
    return {"value": tokens / step_s, "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "sample": (f"fp64 oracle: one {w.name} layer fwd+bwd at B={B1} S={S1} "
                       f"({t_layer:.2f} s), LM-head CE on {n_ce} tokens at V={w.vocab} "
                       f"({t_ce:.2f} s), fp32 AdamW on {n_ad} params ({t_ad:.2f} s, "
                       f"one thread); scaled to {w.n_layers} layers, {tokens} tokens and "
                       f"{n_params} parameters per step; cores = BLAS threads"),
            "sample_seconds": round(t_layer + t_ce + t_ad, 2)}


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3-8b-shaped",
                    choices=["llama3-8b-shaped", "123b-shaped-slice", "lmhead-ce-128k",
                             "critical-batch-sweep", "layer-kernels-8b", "host-link-engines"],
                    help="llama3-8b-shaped (default: the headline step), 123b-shaped-slice, "
                         "lmhead-ce-128k (the chunked CE alone), critical-batch-sweep, "
                         "layer-kernels-8b (one 8B-shaped layer's kernels alone, plus a 1 GiB "
                         "device copy that calibrates HBM byte counters), host-link-engines (one "
                         "8B layer's bytes over the host link on each copy engine, and through "
                         "hipMemcpyAsync)")
    ap.add_argument("--batch", type=int, default=0,
                    help="sequences of 1024 tokens per step of the llama3-8b-shaped workload "
                         "(default 8); at the critical batch the CPU updates hide behind the "
                         "backward")
    ap.add_argument("--slots", type=int, default=0,
                    help="HBM slots of the layer ring for the llama3-8b-shaped workload (default "
                         "3; with one slot per layer the backward re-uploads no layer)")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers of the 123b slice (default 12, fewer if host RAM is short)")
    ap.add_argument("--copy-engine", default="hsa", choices=["hip", "hsa"],
                    help="slot-ring copies on two host-optimised copy engines chosen through "
                         "the HSA runtime (default) or through hipMemcpyAsync")
    ap.add_argument("--activations", default="hbm", choices=["hbm", "recompute", "host"],
                    help="forward state for the backward: intermediates kept in HBM (default), "
                         "layer inputs kept and the forward recomputed, or layer inputs slid to "
                         "host memory and back (with recompute)")
    ap.add_argument("--state-tier", default=None, metavar="DIR",
                    help="keep the optimizer state (fp32 master, m, v) of --tier-layers layers in "
                         "a file under DIR (O_DIRECT where the file system allows; unlinked at "
                         "once) instead of host memory: the pages' optional NVMe tier")
    ap.add_argument("--tier-layers", type=int, default=0,
                    help="with --state-tier: how many layers (the last ones) keep their state "
                         "in the file (default: all)")
    ap.add_argument("--overlap-table", default=None, metavar="PATH",
                    help="write the last timed step's per-layer T_bwd, T_d2h and T_update (the "
                         "pages' overlap condition, layer by layer) as a CSV file")
    ap.add_argument("--trace", default=None, metavar="PREFIX",
                    help="write PREFIX.json (Chrome trace of the timed steps: GPU layer and CE "
                         "intervals, gradient D2H, CPU updates) and PREFIX.txt (text timeline of "
                         "the last two steps, 10 ms per column)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle CPU baseline (e.g. under a profiler)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"],
                    help="compute dtype of the step and layer-kernel workloads (f16: with dynamic "
                         "loss scaling)")
    ap.add_argument("--embed-split", action="store_true",
                    help="update the embedding's rows that no token selects during the step and "
                         "only the selected rows after the backward")
    ap.add_argument("--gap-ms", type=float, default=0.0,
                    help="layer-kernels-8b only: leave the GPU idle this long after each layer "
                         "(the host-bound step's duty cycle: the GPU waits on the CPU between "
                         "layers); the kernel table then shows the kernels at the clocks such "
                         "a duty cycle runs at, and ms_per_step is the kernels' sum")
    ap.add_argument("--adam-threads", type=int, default=0,
                    help="CPU AdamW threads (default: cores - 3, leaving cores to the engine thread and the HIP runtime)")
    return ap.parse_args()


def _kernel_table(prof, alg, exe, byt):
    kernels = {}
    for name, (cnt, ms) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        avg_ms = ms / max(cnt, 1)
        k = {"launches": cnt, "total_ms": round(ms, 3), "avg_ms": round(avg_ms, 4)}
        if name in alg:
            k["tflops_alg"] = round(alg[name] / (avg_ms * 1e-3) / 1e12, 1)
            k["tflops_exec"] = round(exe[name] / (avg_ms * 1e-3) / 1e12, 1)
        if name in byt:
            k["gbs"] = round(byt[name] / (avg_ms * 1e-3) / 1e9, 1)
        kernels[name] = k
    return kernels


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_8b_layer_hbm_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "layer_sliding_offloaded_fwd_amd", "csrc", f)
                for f in ("gemm.hip", "gemm.h")]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` at the 8B layer shapes, from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE passes scaled by a 1 GiB copy), or None when there is no
    figure for it or the GEMM sources changed since the counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    sha, table = None, {}
    for line in open(TRAFFIC_FILE):
        parts = line.split()
        if len(parts) == 2 and parts[0] == "source_sha256":
            sha = parts[1]
        elif len(parts) == 3 and parts[0] == "traffic":
            table[parts[1]] = int(parts[2])
    if sha != h.hexdigest():
        return None
    return table.get(kernel)


STEP_PROFILE = os.path.join(ROOT, "profiles", "llama3-8b-shaped_step_kernels.md")


def profiled_figures(kernel):
    """The committed rocprofv3 summaries' averages for `kernel` (ms): under kernel tracing in the
    step (the runtime then copies gradients with blit kernels on the compute units) and alone on
    the GPU (layer-kernels workload); None where a summary has no figure for it."""
    out = {"step_profile_avg_ms": None, "layer_kernels_avg_ms": None}
    if not os.path.exists(STEP_PROFILE):
        return out
    for line in open(STEP_PROFILE):
        parts = line.split()
        if len(parts) == 3 and parts[1] == kernel:
            if parts[0] == "profiled_step_avg_ms":
                out["step_profile_avg_ms"] = float(parts[2])
            elif parts[0] == "layer_kernels_avg_ms":
                out["layer_kernels_avg_ms"] = float(parts[2])
    return out


def _roofline(kernels, alg, profiled=False):
    """Roofline of the dominant MFMA kernel. `profiled`: the launch is the one the committed
    counter and trace summaries cover (the 8B-shaped layer at 8 x 1024 tokens in bf16), so
    their HBM traffic and profiled averages apply; otherwise both are null."""
    mfma_names = [n for n in kernels if n in alg]
    dom = max(mfma_names, key=lambda n: kernels[n]["total_ms"])
    dk = kernels[dom]
    achieved = alg[dom] / (dk["avg_ms"] * 1e-3) / 1e12
    check = None
    if profiled:
        check = profiled_figures(dom)
        for k in list(check):
            if check[k] is not None:
                check[k.replace("avg_ms", "frac")] = round(
                    alg[dom] / (check[k] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        check["source"] = os.path.relpath(STEP_PROFILE, ROOT)
    return {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(dom) if profiled else None,
            "avg_launch_ms": dk["avg_ms"], "flops_per_launch": alg[dom], "check": check}


def _is_profiled_launch(layer, tokens, dtype):
    from seeded_inputs import L8B
    return layer == L8B.layer and tokens == 8 * 1024 and dtype == "bf16"


def _host_bytes_needed(w, args=None):
    """fp32 master + m + v (12 B) and the pinned bf16 buffer (2 B) per parameter; layers whose
    optimizer state is in the disk tier keep only the bf16 buffer in host memory."""
    c = w.layer
    n = w.n_layers * c.param_count() + 2 * w.vocab * c.hidden + c.hidden
    tiered = 0
    if args is not None and getattr(args, "state_tier", None):
        tiered = min(args.tier_layers or w.n_layers, w.n_layers) * c.param_count()
    return n * 14 - tiered * 12


def step_host_bytes(w):
    """Host bytes of one offloaded step: the CPU AdamW's 28 B per parameter (fp32 master, m, v
    read and written, the bf16 gradient read and the bf16 weight written); the uploads (every
    layer twice except the ring's slots reused at the turnaround, the resident embedding, final
    gain and LM head once); the gradient flushes (every parameter once, bf16)."""
    c = w.layer
    n = c.param_count()
    n_all = w.n_layers * n + 2 * w.vocab * c.hidden + c.hidden
    h2d = 2 * (2 * w.n_layers - w.ring_slots) * n + 2 * (2 * w.vocab * c.hidden + c.hidden)
    return 28 * n_all, h2d, 2 * n_all


def host_roofline(w, threads, step_s):
    """The step's host-memory bound. Every parameter's CPU AdamW moves 28 bytes through host
    DRAM (fp32 master, m, v read and written, the bf16 gradient read and the bf16 weight
    written), and the weight uploads and gradient flushes cross it once more. The peak is a
    STREAM triad (slide_host_triad) on the optimizer's threads over one layer's worth of
    elements (at most 2^28 per array) on huge pages, the better of one run before and one after
    the AdamW timing; the bound is the step's host bytes (AdamW + copies) at that rate.
    The AdamW's own rate alone on the same host is reported beside it (its fraction of the
    triad is the optimizer's efficiency)."""
    import layer_sliding_offloaded_fwd_amd as sl
    from layer_sliding_offloaded_fwd_amd.engine import _host_f32
    import torch
    c = w.layer
    n = c.param_count()
    n_triad = min(n, 1 << 28)       # 1 GiB per array, several times the last-level cache
    triad_best, triad_med = sl.slide_host_triad(n_triad, threads, 5)
    p, m, v = _host_f32(n), _host_f32(n), _host_f32(n)
    for t in (p, m, v):
        t.fill_(0.0)                 # touch every page before timing
    p.fill_(0.01)
    # the gradient / bf16-weight buffer is pinned, as the engine's shared buffers are
    g = torch.zeros(n, dtype=torch.int16, pin_memory=True).numpy()
    hp = sl.AdamWHp(1e-4, 0.9, 0.999, 1e-8, 0.01)
    ts = []
    for k in range(6):
        a = time.perf_counter()
        sl.slide_cpu_adamw(p, g, sl.SLIDE_BF16, m, v, g, n, k + 1, hp, threads)
        ts.append(time.perf_counter() - a)
    del p, m, v, g
    bw = 28 * n / min(ts[1:])        # best of the timed calls: the host's DRAM is shared
    # a second triad after the AdamW; the peak is the better of the two (right after a large
    # engine is torn down the kernel may still be reclaiming its pinned memory)
    tb2, tm2 = sl.slide_host_triad(n_triad, threads, 5)
    if tb2 > triad_best:
        triad_best, triad_med = tb2, tm2
    adam_bytes, h2d, d2h = step_host_bytes(w)
    host_bytes = adam_bytes + h2d + d2h
    bound_s = host_bytes / (triad_best * 1e9)
    link = host_link(2 * n)
    # both directions at once at the probe's rate, scaled (per direction) from the engine the
    # runtime used to the best engine where the probe's own copy ran slower than that
    f_up = max(1.0, link["engine_best_h2d_gbs"] / link["h2d_alone_gbs"])
    f_dn = max(1.0, link["engine_best_d2h_gbs"] / link["d2h_alone_gbs"])
    link_s = max(h2d / (link["h2d_both_gbs"] * f_up * 1e9), d2h / (link["d2h_both_gbs"] * f_dn * 1e9))
    placed_s = max(h2d / (link["h2d_both_gbs"] * 1e9), d2h / (link["d2h_both_gbs"] * 1e9))
    link.update(step_bound_ms=round(link_s * 1e3, 1), frac=round(link_s / step_s, 4),
                frac_as_placed=round(placed_s / step_s, 4))
    return {"bound": "host_dram", "adamw_bytes": adam_bytes, "h2d_bytes": h2d, "d2h_bytes": d2h,
            "peak_triad_gbs": round(triad_best, 1), "triad_median_gbs": round(triad_med, 1),
            "triad_threads": threads,
            "adamw_alone_gbs": round(bw / 1e9, 1),
            "adamw_frac_of_triad": round(bw / 1e9 / triad_best, 3),
            "step_bound_ms": round(bound_s * 1e3, 1),
            "frac": round(bound_s / step_s, 4),
            # achieved rates over the whole step (bytes per step / time per step)
            "host_dram_gbs": round(host_bytes / step_s / 1e9, 1),
            "h2d_link_gbs": round(h2d / step_s / 1e9, 1),
            "d2h_link_gbs": round(d2h / step_s / 1e9, 1),
            "link": link,
            "note": "bound = the step's AdamW and copy bytes at the STREAM-triad rate"}


def host_link(nbytes, reps=3):
    """Host-link rates of the slot-ring copies, measured alone: one layer's bf16 weights
    (nbytes) between pinned host memory and HBM with hipMemcpyAsync on side streams, each
    direction alone and both at once (the backward's weight reloads run beside its gradient
    flushes), each copy timed with events on its own stream. Best of `reps`. The step's link
    bound is its upload and flush bytes at the rates of both directions at once."""
    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    h_src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h_dst = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d_dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    d_src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    up, down = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(h2d, d2h):
        """(up GB/s, down GB/s), best of reps, each direction timed on its own stream"""
        best = [float("inf"), float("inf")]
        for _ in range(reps):
            torch.cuda.synchronize()
            ev = []
            for on, st, dst, src in ((h2d, up, d_dst, h_src), (d2h, down, h_dst, d_src)):
                if not on:
                    ev.append(None)
                    continue
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(st):
                    e0.record(st)
                    dst.copy_(src, non_blocking=True)
                    e1.record(st)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            for i, e in enumerate(ev):
                if e:
                    best[i] = min(best[i], e[0].elapsed_time(e[1]) * 1e-3)
        return tuple(nbytes / t / 1e9 if t < float("inf") else 0.0 for t in best)

    timed(True, True)   # warm-up
    h2d_alone, d2h_alone = timed(True, False)[0], timed(False, True)[1]
    h2d_both, d2h_both = timed(True, True)
    # The rate a copy gets depends on the copy engine the runtime places it on (the engines built
    # for copies between GPUs run the host link at a fraction of the host-optimised ones' rate),
    # and hipMemcpyAsync's placement can stay on a slow engine for a while. The link's own rate
    # is that of the best engine, timed one engine at a time.
    d2h_ms, h2d_ms, _ = sl.slide_host_link_engine_rates(d_src, h_dst, nbytes, 1)
    best = lambda ms: max((nbytes / (t * 1e-3) / 1e9 for t in ms if t > 0), default=0.0)
    return {"bytes_per_copy": nbytes, "h2d_alone_gbs": round(h2d_alone, 1),
            "d2h_alone_gbs": round(d2h_alone, 1), "h2d_both_gbs": round(h2d_both, 1),
            "d2h_both_gbs": round(d2h_both, 1),
            "engine_best_h2d_gbs": round(best(h2d_ms), 1),
            "engine_best_d2h_gbs": round(best(d2h_ms), 1)}


def run_step(w, args):
    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    from layer_sliding_offloaded_fwd_amd.engine import AdamW, ModelSpec, SlideEngine
    from seeded_inputs import tokens as draw_tokens

    c = w.layer
    spec = ModelSpec(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, w.vocab, w.n_layers,
                     args.dtype, c.rms_eps, c.rope_theta)
    cores = len(os.sched_getaffinity(0))
    threads = args.adam_threads or max(1, cores - 3)
    t_init = time.perf_counter()
    print(f"[bench] {w.name}: {w.n_layers} layers, host state {_host_bytes_needed(w, args) / 1e9:.1f} GB;"
          f" allocating", file=sys.stderr, flush=True)
    tier_kw = {}
    if args.state_tier:
        # the last layers: their gradients land first in the backward and the next forward
        # needs them last, so their slower updates have the most time to hide
        k = min(args.tier_layers or w.n_layers, w.n_layers)
        tier_kw = dict(state_tier=os.path.join(args.state_tier, f"slide-state-{os.getpid()}.bin"),
                       tier_layers=list(range(w.n_layers - k, w.n_layers)))
        need = k * 3 * sl.slide_tier_region_bytes(c.param_count())
        st = os.statvfs(args.state_tier)
        if need > 0.95 * st.f_bavail * st.f_frsize:
            print(f"[bench] --state-tier {args.state_tier}: {k} layers need {need / 1e9:.1f} GB, "
                  f"only {st.f_bavail * st.f_frsize / 1e9:.1f} GB free", file=sys.stderr)
            sys.exit(1)
    eng = SlideEngine(spec, w.batch, w.seq, n_slots=w.ring_slots, ce_chunk=w.ce_chunk,
                      hp=AdamW(), adam_threads=threads, timeline=True,
                      activations=args.activations, keep_records=args.steps + args.warmup,
                      embed_split=args.embed_split, copy_engine=args.copy_engine, **tier_kw)
    copy_engine = eng.copy_engine     # "hip" if the HSA ring could not be created
    eng.init_random(seed=0, std=0.02,
                    progress=lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True))
    toks = [draw_tokens(w.batch, w.seq, w.vocab, seed=1 + i)
            for i in range(args.warmup + args.steps)]
    t_init = time.perf_counter() - t_init
    print(f"[bench] init {t_init:.1f} s; warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        eng.step(toks[i])
        print(f"[bench] warmup step {i + 1}: loss {eng.loss():.4f}", file=sys.stderr, flush=True)
    eng.wait_updates()
    torch.cuda.synchronize()
    tier0 = eng.tier_stats()
    sl.slide_prof_reset()
    sl.slide_prof_enable(True)
    t0 = time.perf_counter()
    t_ret = []
    for i in range(args.steps):
        eng.step(toks[args.warmup + i])
        t_ret.append(time.perf_counter())
    eng.wait_updates()       # the last step's pending CPU updates are part of the timed work
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sl.slide_prof_enable(False)
    prof = sl.slide_prof_read()
    loss = eng.loss()
    step_s = (t1 - t0) / args.steps
    tok_s = w.batch * w.seq / step_s
    periods = np.diff(np.asarray(t_ret)) * 1e3
    steady_ms = float(np.median(periods)) if len(periods) else step_s * 1e3
    print(f"[bench] {args.steps} steps: {step_s * 1e3:.1f} ms/step ({steady_ms:.1f} ms steady), "
          f"{tok_s:.0f} tokens/s, loss {loss:.4f}", file=sys.stderr, flush=True)

    alg, exe = kernel_flops(spec, w.batch, w.seq, w.ce_chunk)
    kernels = _kernel_table(prof, alg, exe, kernel_bytes(spec, w.batch, w.seq))
    # forward projections and attention run once per step when the forward's intermediates are
    # kept (the engine's default); with the recompute they would run twice
    fwd_names = {"gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attn_fwd"}
    layer_names = [n for n in kernels if n in alg and n.startswith(("gemm_", "attn_"))]
    lt = sum(kernels[n]["total_ms"] for n in layer_names) * 1e-3
    fwd_runs = 1 if eng.save_activations else 2
    l_alg = sum(alg[n] * kernels[n]["launches"] / (fwd_runs if n in fwd_names else 1)
                for n in layer_names)
    l_exe = sum(exe[n] * kernels[n]["launches"] for n in layer_names)
    # the layer's whole kernel time (the elementwise and normalisation kernels too), so that work
    # fused into a GEMM's epilogue neither hides nor inflates the figure
    lt_all = _layer_kernel_ms(kernels) * 1e-3
    mfma_util_alg = 100.0 * l_alg / lt_all / 1e12 / PEAK_BF16_TFLOPS if lt_all else 0.0
    mfma_util_exec = 100.0 * l_exe / lt_all / 1e12 / PEAK_BF16_TFLOPS if lt_all else 0.0
    mfma_kernels_util = 100.0 * l_alg / lt / 1e12 / PEAK_BF16_TFLOPS if lt else 0.0
    ana = eng.analyse(list(eng.records)[-args.steps:])
    if args.overlap_table:
        _write_overlap_table(args.overlap_table, ana["layers"])
    if args.trace:
        recs = list(eng.records)[-args.steps:]
        eng.export_trace(recs, args.trace + ".json")
        _write_text_timeline(eng, recs[-3:], args.trace + ".txt")
    tier = _tier_report(eng, tier0, args.steps, step_s) if eng.tier is not None else None
    eng_scale, eng_skipped = eng.loss_scale, eng.skipped_steps
    eng.close()
    del eng
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    print("[bench] resident (non-offloaded) baseline", file=sys.stderr, flush=True)
    resident = (run_resident(w, args) if args.dtype == "bf16" else
                {"skipped": "the resident baseline runs the bf16 step"})
    if "tokens_per_s" in resident:
        resident["offloaded_fraction_of_resident"] = round(tok_s / resident["tokens_per_s"], 4)
    host = host_roofline(w, threads, step_s)
    # exposed-time overlap: the step replayed with the gradient copies and CPU updates taking no
    # time, from the measured per-layer GPU times, the other GPU work and the upload rate
    L = w.n_layers
    fwd_ms = [float(np.mean([li["t_fwd_ms"] for li in ana["layers"] if li["layer"] == i]))
              for i in range(L)]
    bwd_ms = [float(np.mean([li["t_bwd_ms"] for li in ana["layers"] if li["layer"] == i]))
              for i in range(L)]
    busy = sum(k["total_ms"] for k in kernels.values()) / args.steps
    avg = lambda n: kernels[n]["total_ms"] / args.steps if n in kernels else 0.0
    t_ef = avg("embed_fwd")
    t_eb = avg("embed_bwd") + avg("convert_f32")
    t_head = max(0.0, busy - sum(fwd_ms) - sum(bwd_ms) - t_ef - t_eb)
    up = host["link"]["h2d_alone_gbs"] * 1e6          # bytes per ms
    t_noop = noop_step_replay(fwd_ms, bwd_ms, w.ring_slots, t_ef, t_head, t_eb,
                              2 * c.param_count() / up, 2 * w.vocab * c.hidden / up,
                              2 * w.vocab * c.hidden / up)
    work_ms = ana["t_d2h_total_ms"] + ana["t_update_all_ms"]
    t_exposed = max(0.0, steady_ms - t_noop)
    overlap_exposed = 100.0 * (1.0 - t_exposed / work_ms) if work_ms > 0 else 100.0
    layer_bytes = w.n_layers * c.param_count() * 28
    n_all = w.n_layers * c.param_count() + 2 * w.vocab * c.hidden + c.hidden
    return {
        "metric": "train tokens/sec (1 GPU) + layer MFMA util % + backward/update overlap %",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "hidden": c.hidden,
                   "heads": c.n_heads, "kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                   "ffn": c.ffn, "vocab": w.vocab, "global_batch": w.batch, "seq_len": w.seq,
                   "ring_slots": w.ring_slots, "ce_chunk": w.ce_chunk,
                   "parallelism": "single GPU, layers streamed from host",
                   "adam_threads": threads, "copy_engine": copy_engine,
                   "activations": {"hbm": "intermediates kept in HBM (no recompute)",
                                   "recompute": "layer inputs kept in HBM, forward recomputed",
                                   "host": "layer inputs slid to host memory, forward "
                                           "recomputed"}[args.activations]},
        "layer_mfma_util_pct": round(mfma_util_alg, 2),
        "layer_mfma_util_exec_pct": round(mfma_util_exec, 2),
        "mfma_kernels_util_pct": round(mfma_kernels_util, 2),
        # 1 - T_exposed / sum(T_d2h + T_update): T_exposed = T_step - T_step(copies and
        # updates as no-ops), the latter from noop_step_replay
        "overlap_pct": round(overlap_exposed, 1),
        "overlap": {"definition": "1 - (T_step - T_step_noop) / (sum of layer gradient D2H "
                                  "times + sum of all CPU update times)",
                    "t_step_noop_replay_ms": round(t_noop, 1),
                    "t_exposed_ms": round(t_exposed, 1),
                    "d2h_plus_update_ms": round(work_ms, 1),
                    "gpu_busy_ms_per_step": round(busy, 1),
                    # share of the D2H + update intervals that ran while the GPU computed
                    "interval_pct": round(ana["overlap_pct"], 1),
                    "t_bwd_total_ms": round(ana["t_bwd_total_ms"], 1),
                    "t_d2h_total_ms": round(ana["t_d2h_total_ms"], 1),
                    "t_update_total_ms": round(ana["t_update_total_ms"], 1),
                    # every CPU update of the step (layers, embedding, final gain, LM head)
                    "t_update_all_blocks_ms": round(ana["t_update_all_ms"], 1),
                    # GPU idle between a backward's end and the next layer-0 forward (median)
                    "step_boundary_gap_ms": (round(ana["boundary_ms"], 1)
                                             if ana["boundary_ms"] is not None else None),
                    "layers_meeting_T_bwd_ge_T_d2h_plus_T_update": ana["predicate_layers_met"],
                    "gpu_span_ms_per_step": round(ana["gpu_ms"], 1)},
        # CPU AdamW of the layer parameters: fp32 master, m, v read and written (24 B), the
        # bf16 gradient read and the bf16 weight written (4 B)
        "host_adamw_gbs": round(layer_bytes / (ana["t_update_total_ms"] * 1e-3) / 1e9, 1)
        if ana["t_update_total_ms"] else None,
        "loss_last_step": round(loss, 4),
        "ms_per_step_steady": round(steady_ms, 2),
        **({"loss_scaling": {"final_scale": eng_scale, "skipped_steps": eng_skipped}}
           if args.dtype == "f16" else {}),
        "step_periods_ms": [round(float(x), 1) for x in periods],
        "first_step_ms": round((t_ret[0] - t0) * 1e3, 1) if t_ret else None,
        "drain_ms": round((t1 - t_ret[-1]) * 1e3, 1) if t_ret else None,
        "host_roofline": host,
        # the pages compare offloaded training with training whose state stays on the GPU:
        # measured on the same GPU with the same kernels (paper page abstract: over 95%)
        "resident": resident,
        "roofline": _roofline(kernels, alg, profiled=_is_profiled_launch(
            w.layer, w.batch * w.seq, args.dtype)),
        **({"state_tier": tier} if tier is not None else {}),
        "kernels": kernels,
        "init_s": round(t_init, 1),
    }


def run_resident(w, args, steps=5, warmup=2):
    """The non-offloaded baseline on the same GPU: every parameter, gradient and AdamW state in
    HBM (ResidentTrainer: the engine's library calls with slide_gpu_adamw instead of the gradient
    flushes, CPU updates and uploads; results equal the offloaded step's bit for bit), same
    seeded weights and tokens. Returns its tokens/s, or None where the state does not fit."""
    import torch
    from layer_sliding_offloaded_fwd_amd.engine import AdamW, ModelSpec
    from layer_sliding_offloaded_fwd_amd.resident import ResidentTrainer
    from seeded_inputs import tokens as draw_tokens
    import layer_sliding_offloaded_fwd_amd as sl
    c = w.layer
    n_all = w.n_layers * c.param_count() + 2 * w.vocab * c.hidden + c.hidden
    cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, "bf16")
    # bf16 weights, fp32 master, m, v (14 B per parameter), the embedding's and LM head's
    # gradients, every layer's saved intermediates and input
    need = (14 * n_all + 4 * w.vocab * c.hidden
            + w.n_layers * (sl.slide_layer_saved_bytes(cfg, w.batch, w.seq)
                            + 2 * w.batch * w.seq * c.hidden))
    free, _ = torch.cuda.mem_get_info()
    if need > 0.9 * free:
        return {"skipped": f"needs about {need / 1e9:.0f} GB of HBM, {free / 1e9:.0f} GB free"}
    spec = ModelSpec(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, w.vocab, w.n_layers,
                     "bf16", c.rms_eps, c.rope_theta)
    tr = ResidentTrainer(spec, w.batch, w.seq, ce_chunk=w.ce_chunk, hp=AdamW())
    tr.init_random(seed=0, std=0.02)
    toks = [draw_tokens(w.batch, w.seq, w.vocab, seed=1 + i) for i in range(warmup + steps)]
    for i in range(warmup):
        tr.step(toks[i])
    tr.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        tr.step(toks[warmup + i])
    tr.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    loss = tr.loss()
    del tr
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(w.batch * w.seq / step_s, 1),
            "ms_per_step": round(step_s * 1e3, 2), "steps": steps, "warmup": warmup,
            "loss_last_step": round(loss, 4),
            "what": "every parameter, gradient and AdamW state in HBM, GPU AdamW with the CPU "
                    "optimizer's operation order (bit-identical results)"}


def noop_step_replay(fwd_ms, bwd_ms, n_slots, t_embed_fwd, t_head, t_embed_bwd, u_layer,
                     u_embed, u_lm, steps=4):
    """Period (ms) of the engine's step with the gradient copies and the CPU updates taking no
    time: the second term of the exposed-time overlap, 1 - T_exposed / sum(T_d2h + T_update)
    with T_exposed = T_step - T_step(copies and updates as no-ops). The engine's dependencies
    are replayed with measured durations on two resources, the compute stream and the upload
    stream:
      forward   the loads of layers 0 .. n_slots-1, then the embedding's upload (the previous
                step's update), are queued when the step starts; the gather waits for the
                embedding; layer i's forward waits for its load; the load of layer i + n_slots
                waits for the slot that layer i's forward releases;
      head      final norm and the fused CE (t_head, GPU time); the LM head's re-upload (its
                update, done at once) is queued when the head starts;
      backward  the last n_slots layers are still resident; every other layer i waits for its
                load, queued when layer i + n_slots's backward releases its slot;
      boundary  the embedding's backward; the next step starts when the GPU is done (the engine's
                host thread waits for it).
    fwd_ms, bwd_ms: per-layer GPU times; u_*: upload times at the link's measured rate. Returns
    the steady period (the last of `steps` replayed steps)."""
    L = len(fwd_ms)
    S = max(1, min(n_slots, L))
    t0 = 0.0
    periods = []
    for _ in range(steps):
        gpu = h2d = t0
        load_end = {}
        for i in range(min(S, L)):            # every slot is free when a step starts
            h2d += u_layer
            load_end[i] = h2d
        h2d += u_embed
        gpu = max(gpu, h2d) + t_embed_fwd
        for i in range(L):
            gpu = max(gpu, load_end[i]) + fwd_ms[i]
            if i + S < L:                     # the slot layer i released takes layer i + S
                h2d = max(h2d, gpu) + u_layer
                load_end[i + S] = h2d
        h2d = max(h2d, gpu) + u_lm
        gpu += t_head
        for i in range(L - 1, -1, -1):
            if i < L - S:
                gpu = max(gpu, load_end[i])
            gpu += bwd_ms[i]
            if i - S >= 0:
                h2d = max(h2d, gpu) + u_layer
                load_end[i - S] = h2d
        gpu += t_embed_bwd
        periods.append(gpu - t0)
        t0 = gpu
    return periods[-1]


def _write_text_timeline(eng, recs, path, ms_per_col=10.0):
    """Text lanes from the start of the second of `recs` to the end: GPU (F layer forward, B
    layer backward, C CE), D2H (# gradient copies) and CPU (u layer, e embedding, l LM head, f
    final gain updates), with the first step's updates included where they run into the
    second; ':' marks a partly busy column."""
    tl = eng.timeline_of(recs)
    t0 = (recs[1]["host_t0"] - recs[0]["host_t0"]) * 1e3 if len(recs) > 1 else 0.0
    with open(path, "w") as f:
        f.write(f"steps {recs[min(1, len(recs) - 1)]['step']}-{recs[-1]['step']}, "
                f"{ms_per_col:g} ms per column\n")
        f.write(eng.render_timeline(tl, ms_per_col, t_start=t0) + "\n")


def _write_overlap_table(path, per_layer):
    """Per layer of the last timed step: its backward time, the D2H of its gradients, its CPU
    update, and whether the backward of the layer below covers them (the pages' condition)."""
    last = max(li["step"] for li in per_layer)
    rows = sorted((li for li in per_layer if li["step"] == last), key=lambda li: -li["layer"])
    by = {li["layer"]: li for li in rows}
    with open(path, "w") as f:
        f.write("layer,t_bwd_ms,t_d2h_ms,t_update_ms,t_bwd_next_layer_ms,covered\n")
        for li in rows:
            nxt = by.get(li["layer"] - 1)
            tb = nxt["t_bwd_ms"] if nxt else float("nan")
            ok = nxt is not None and tb >= li["t_d2h_ms"] + li["t_update_ms"]
            f.write(f"{li['layer']},{li['t_bwd_ms']:.3f},{li['t_d2h_ms']:.3f},"
                    f"{li['t_update_ms']:.3f},{tb:.3f},{int(ok)}\n")


def _tier_report(eng, before, steps, step_s):
    """Disk-tier traffic of the timed steps: the optimizer state of each tiered layer (fp32
    master, m and v for bf16 compute: 12 B per parameter) is read and written once per step,
    streamed through the update; the rate is those bytes over the time the tier's calls took,
    and the bound is the step's tier bytes at that rate."""
    after = eng.tier_stats()
    rd = after["bytes_read"] - before["bytes_read"]
    wr = after["bytes_written"] - before["bytes_written"]
    busy = after["busy_s"] - before["busy_s"]
    stall = after["stall_s"] - before["stall_s"]
    return {"layers": len(eng.tier_layers), "direct_io": after["direct"],
            "chunk_elems": after["chunk"], "file_bytes": after["capacity"],
            "read_bytes_per_step": rd // steps, "write_bytes_per_step": wr // steps,
            "update_s_per_step": round(busy / steps, 3),
            "io_wait_s_per_step": round(stall / steps, 3),
            "read_plus_write_gbs": round((rd + wr) / busy / 1e9, 2) if busy else None,
            "frac_of_step": round(busy / steps / step_s, 4)}


def run_ce(args):
    """The chunked LM-head CE alone: 16384 tokens, hidden 4096, vocab 128256, chunks of 8192."""
    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    from seeded_inputs import CE_ONLY
    N, H, V, C = CE_ONLY["tokens"], CE_ONLY["hidden"], CE_ONLY["vocab"], CE_ONLY["chunk"]
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    h = torch.empty(N, H, device=dev, dtype=torch.float32).normal_(0, 1, generator=gen).bfloat16()
    w = torch.empty(V, H, device=dev, dtype=torch.float32).normal_(0, 0.02, generator=gen).bfloat16()
    t = torch.randint(0, V, (N,), device=dev, dtype=torch.int32, generator=gen)
    cfg = sl.CeCfg(H, V, C, sl.SLIDE_BF16)
    wsz = sl.slide_lmhead_ce_workspace_bytes(cfg, N)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    loss = torch.zeros(1, dtype=torch.float32, device=dev)
    dh = torch.empty_like(h)
    dw = torch.empty_like(w)
    st = torch.cuda.current_stream()
    for _ in range(args.warmup):
        sl.slide_lmhead_ce(cfg, h, w, t, N, loss, dh, dw, ws, wsz, st)
    torch.cuda.synchronize()
    sl.slide_prof_reset()
    sl.slide_prof_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        sl.slide_lmhead_ce(cfg, h, w, t, N, loss, dh, dw, ws, wsz, st)
    e1.record(st)
    torch.cuda.synchronize()
    sl.slide_prof_enable(False)
    ms = e0.elapsed_time(e1) / args.steps
    flops_alg = 3 * 2 * N * H * V
    flops_exec = 4 * 2 * N * H * V
    nch = (V + C - 1) // C
    per = 2 * N * V * H / nch
    alg = {"ce_stats_gemm": per / 2, "ce_dz_gemm": per / 2, "ce_dh_gemm": per, "ce_dw_gemm": per}
    exe = {"ce_stats_gemm": per, "ce_dz_gemm": per, "ce_dh_gemm": per, "ce_dw_gemm": per}
    kernels = _kernel_table(sl.slide_prof_read(), alg, exe, {})
    return {
        "metric": "chunked LM-head cross-entropy fwd+bwd tokens/sec (1 GPU)",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "lmhead-ce-128k", "tokens": N, "hidden": H, "vocab": V, "chunk": C},
        "tflops_alg": round(flops_alg / (ms * 1e-3) / 1e12, 1),
        "tflops_exec": round(flops_exec / (ms * 1e-3) / 1e12, 1),
        "mfma_util_alg_pct": round(100 * flops_alg / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "workspace_bytes": wsz, "dense_fp32_logits_bytes": N * V * 4,
        "workspace_vs_dense_logits_pct": round(100.0 * wsz / (N * V * 4), 1),
        "loss": round(float(loss.item()), 5),
        "roofline": _roofline(kernels, alg), "kernels": kernels,
        "cpu_baseline": None if args.no_cpu_baseline else ce_cpu_baseline(N, H, V, C),
    }


def ce_cpu_baseline(N, H, V, C, n_s=1024):
    """The oracle's chunked CE (fwd+bwd, fp64) on n_s of the N tokens at the full vocabulary,
    scaled to N tokens (the CE is linear in the token count)."""
    from oracle import model as om
    rng = np.random.default_rng(3)
    h = rng.standard_normal((n_s, H))
    w = rng.standard_normal((V, H)) * 0.02
    t = rng.integers(0, V, n_s)
    t0 = time.perf_counter()
    om.ce_chunked(h, w, t, C)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = len(os.sched_getaffinity(0))
    return {"value": N / (dt * N / n_s), "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "sample": f"fp64 oracle chunked CE fwd+bwd on {n_s} tokens at V={V}, H={H} "
                      f"({dt:.2f} s), scaled to {N} tokens; cores = BLAS threads",
            "sample_seconds": round(dt, 2)}


def run_sweep(args):
    """The pages' critical batch (figure 4 of the paper page): for one 8B-shaped layer at
    S = 1024 and B = 1..32, the layer backward time on the GPU against the D2H time of its
    gradients plus the CPU AdamW time of its parameters."""
    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    from seeded_inputs import L8B
    c, S = L8B.layer, 1024
    dev = "cuda:0"
    cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, "bf16")
    P = sl.slide_layer_param_count(cfg)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    w = (torch.empty(P, device=dev).normal_(0, 0.02, generator=gen)).bfloat16()
    offs = sl.slide_layer_param_offsets(cfg)
    w[offs[0]:offs[0] + c.hidden] = 1.0
    w[offs[3]:offs[3] + c.hidden] = 1.0
    g = torch.empty_like(w)
    st = torch.cuda.current_stream()
    # T_grad_d2h: the layer's bf16 gradients to pinned host memory
    cores = len(os.sched_getaffinity(0))
    threads = args.adam_threads or max(1, cores - 3)
    host_g = torch.empty(P, dtype=torch.bfloat16, pin_memory=True)
    for _ in range(2):
        host_g.copy_(g, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(5):
        host_g.copy_(g, non_blocking=True)
    e1.record(st)
    torch.cuda.synchronize()
    t_d2h = e0.elapsed_time(e1) / 5
    # T_update: the CPU AdamW of the layer's parameters
    from layer_sliding_offloaded_fwd_amd.engine import _host_f32
    pm, mm, vv = _host_f32(P), _host_f32(P), _host_f32(P)     # as the engine holds them
    pm.fill_(0.01)
    gb = host_g.view(torch.int16).numpy()
    hp = sl.AdamWHp(1e-4, 0.9, 0.999, 1e-8, 0.01)
    ts = []
    for k in range(4):
        a = time.perf_counter()
        # in place, as in the step: the bf16 gradient buffer receives the new bf16 weights
        sl.slide_cpu_adamw(pm, gb, sl.SLIDE_BF16, mm, vv, gb, P, k + 1, hp, threads)
        ts.append(time.perf_counter() - a)
    t_upd = min(ts[1:]) * 1e3
    rows = []
    crit = None
    for Bb in (1, 2, 4, 8, 16, 32):
        N = Bb * S
        x = torch.empty(N, c.hidden, device=dev).normal_(0, 1, generator=gen).bfloat16()
        dy = torch.empty_like(x).normal_(0, 1, generator=gen)
        y = torch.empty_like(x)
        dx = torch.empty_like(x)
        sb = sl.slide_layer_saved_bytes(cfg, Bb, S)
        wb = sl.slide_layer_workspace_bytes(cfg, Bb, S, 2)
        saved = torch.empty(sb, dtype=torch.uint8, device=dev)
        ws = torch.empty(wb, dtype=torch.uint8, device=dev)
        sl.slide_layer_fwd_save(cfg, w, x, y, Bb, S, saved, sb, st)
        sl.slide_layer_bwd_saved(cfg, w, x, dy, dx, g, Bb, S, saved, sb, ws, wb, st)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(3):
            sl.slide_layer_bwd_saved(cfg, w, x, dy, dx, g, Bb, S, saved, sb, ws, wb, st)
        e1.record(st)
        torch.cuda.synchronize()
        t_bwd = e0.elapsed_time(e1) / 3
        ok = t_bwd >= t_d2h + t_upd
        if ok and crit is None:
            crit = Bb
        rows.append({"batch": Bb, "tokens": N, "t_bwd_ms": round(t_bwd, 3),
                     "t_grad_d2h_ms": round(t_d2h, 3), "t_update_ms": round(t_upd, 3),
                     "full_overlap": ok})
        print(f"[bench] B={Bb}: T_bwd {t_bwd:.2f} ms vs T_d2h {t_d2h:.2f} + T_update "
              f"{t_upd:.2f} ms", file=sys.stderr, flush=True)
        del x, dy, y, dx, saved, ws
    per_seq = rows[-1]["t_bwd_ms"] / rows[-1]["batch"]
    extrap = int(np.ceil((t_d2h + t_upd) / per_seq))
    return {
        "metric": "critical batch size: smallest B with T_bwd >= T_grad_d2h + T_update",
        "value": crit if crit is not None else extrap, "unit": "sequences of 1024 tokens",
        "n_gpus": 1, "higher_is_better": False, "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "measured": crit is not None,
        "config": {"workload": "critical-batch-sweep", "layer": "llama3-8b-shaped", "seq_len": S,
                   "params_per_layer": P, "adam_threads": threads},
        "rows": rows,
        "d2h_gbs": round(P * 2 / (t_d2h * 1e-3) / 1e9, 1),
        "adamw_host_gbs": round(P * 28 / (t_upd * 1e-3) / 1e9, 1),
    }


def run_layer_kernels(args):
    """One 8B-shaped layer's forward (keeping its intermediates) and backward at batch 8 x 1024,
    alone on the GPU: the same kernels at the same shapes as in the step, without the host
    traffic. Then a plain 1 GiB device-to-device copy, the reference a byte counter is scaled
    by."""
    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    from seeded_inputs import L8B
    c, Bb, S = L8B.layer, L8B.batch, L8B.seq
    N = Bb * S
    dev = "cuda:0"
    cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, args.dtype)
    tdt = torch.float16 if args.dtype == "f16" else torch.bfloat16
    P = sl.slide_layer_param_count(cfg)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    w = torch.empty(P, device=dev).normal_(0, 0.02, generator=gen).to(tdt)
    offs = sl.slide_layer_param_offsets(cfg)
    w[offs[0]:offs[0] + c.hidden] = 1.0
    w[offs[3]:offs[3] + c.hidden] = 1.0
    g = torch.empty_like(w)
    x = torch.empty(N, c.hidden, device=dev).normal_(0, 1, generator=gen).to(tdt)
    dy = torch.empty_like(x).normal_(0, 1, generator=gen)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    sb = sl.slide_layer_saved_bytes(cfg, Bb, S)
    wb = sl.slide_layer_workspace_bytes(cfg, Bb, S, 2)
    saved = torch.empty(sb, dtype=torch.uint8, device=dev)
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()

    def one():
        sl.slide_layer_fwd_save(cfg, w, x, y, Bb, S, saved, sb, st)
        sl.slide_layer_bwd_saved(cfg, w, x, dy, dx, g, Bb, S, saved, sb, ws, wb, st)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    sl.slide_prof_reset()
    sl.slide_prof_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        one()
        if args.gap_ms > 0:
            torch.cuda.synchronize()
            time.sleep(args.gap_ms * 1e-3)
    e1.record(st)
    torch.cuda.synchronize()
    sl.slide_prof_enable(False)
    ms = e0.elapsed_time(e1) / args.steps
    spec = type("Spec", (), dict(hidden=c.hidden, ffn=c.ffn, head_dim=c.head_dim,
                                 n_heads=c.n_heads, n_kv_heads=c.n_kv_heads, vocab=L8B.vocab))
    alg, exe = kernel_flops(spec, Bb, S, L8B.ce_chunk)
    kernels = _kernel_table(sl.slide_prof_read(), alg, exe, kernel_bytes(spec, Bb, S))
    lt = sum(k["total_ms"] for n, k in kernels.items() if n in alg) * 1e-3
    l_alg = sum(alg[n] * k["launches"] for n, k in kernels.items() if n in alg)
    if args.gap_ms > 0:   # the idle gaps are not the layer's time
        ms = sum(k["total_ms"] for k in kernels.values()) / args.steps
    # the calibration copy: 1 GiB read and 1 GiB written by the runtime's copy kernel
    del saved, ws
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(3):
        dst.copy_(src)
    e1.record(st)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / 3
    copy_gbs = 2 * nbytes / (copy_ms * 1e-3) / 1e9
    for k in kernels.values():   # the HBM-bound kernels against the measured copy rate
        if "gbs" in k:
            k["frac_of_copy"] = round(k["gbs"] / copy_gbs, 3)
    return {
        "metric": "one decoder layer fwd+bwd, kernels alone (1 GPU)",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": "layer-kernels-8b", "hidden": c.hidden, "heads": c.n_heads,
                   "kv_heads": c.n_kv_heads, "head_dim": c.head_dim, "ffn": c.ffn,
                   "global_batch": Bb, "seq_len": S, "idle_gap_ms": args.gap_ms},
        "layer_mfma_util_pct": round(100 * l_alg / (_layer_kernel_ms(kernels) * 1e-3) / 1e12 /
                                     PEAK_BF16_TFLOPS, 2),
        "mfma_kernels_util_pct": round(100 * l_alg / lt / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": _roofline(kernels, alg, profiled=_is_profiled_launch(c, Bb * S, args.dtype)),
        "kernels": kernels,
        "copy_ref": {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(copy_ms, 4),
                     "gbs_read_plus_write": round(copy_gbs, 1)},
    }


def run_host_link_engines(args):
    """One 8B layer's bf16 weights (436 MB) between pinned host memory and HBM on each of the
    GPU's copy engines, both directions, against hipMemcpyAsync on a side stream (the slot ring's
    copies): the host link's rate depends on the engine a copy lands on."""
    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    from seeded_inputs import L8B
    c = L8B.layer
    cfg = sl.layer_cfg(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, "bf16")
    nbytes = sl.slide_layer_param_count(cfg) * 2
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dev.fill_(1)
    host.fill_(2)
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    d2h, h2d, info = sl.slide_host_link_engine_rates(dev, host, nbytes, reps)
    s = torch.cuda.Stream()
    rt = {}
    for name, dst, src in (("d2h", host, dev), ("h2d", dev, host)):
        best = 1e30
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(s):
                e0.record(s)
                dst.copy_(src, non_blocking=True)
                e1.record(s)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        rt[name] = best
    eng = {e: {"d2h_ms": round(d2h[e], 3), "h2d_ms": round(h2d[e], 3),
               "d2h_gbs": round(nbytes / d2h[e] / 1e6, 1) if d2h[e] > 0 else None,
               "h2d_gbs": round(nbytes / h2d[e] / 1e6, 1) if h2d[e] > 0 else None}
           for e in range(32) if d2h[e] > 0 or h2d[e] > 0}
    for e, r in eng.items():
        print(f"[bench] engine {e:2d}: d2h {r['d2h_ms']:7.2f} ms ({r['d2h_gbs']} GB/s)  "
              f"h2d {r['h2d_ms']:7.2f} ms ({r['h2d_gbs']} GB/s)", file=sys.stderr, flush=True)
    return {"metric": "host-link copy time per copy engine (1 GPU)", "unit": "ms",
            "value": round(rt["d2h"], 3), "n_gpus": 1, "steps": reps, "warmup": 0,
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
            "data": "synthetic",
            "config": {"workload": "host-link-engines", "bytes_per_copy": nbytes},
            "engines": eng, "n_host_optimized_engines": info[0], "n_xgmi_engines": info[1],
            "preferred_mask_d2h": hex(info[2]), "preferred_mask_h2d": hex(info[3]),
            "hipMemcpyAsync_ms": {k: round(v, 3) for k, v in rt.items()}}


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _die_multi_gpu(max(args.gpus, world))
    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    from seeded_inputs import L8B, L123B
    import dataclasses

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sl.lib()  # fail loudly if libslide.so is missing
    if args.workload == "lmhead-ce-128k":
        print(json.dumps(run_ce(args)))
        return
    if args.workload == "critical-batch-sweep":
        print(json.dumps(run_sweep(args)))
        return
    if args.workload == "layer-kernels-8b":
        print(json.dumps(run_layer_kernels(args)))
        return
    if args.workload == "host-link-engines":
        print(json.dumps(run_host_link_engines(args)))
        return
    if args.workload == "123b-shaped-slice":
        layers = args.layers or L123B.n_layers
        w = dataclasses.replace(L123B, n_layers=layers)
        try:
            import psutil
            avail = psutil.virtual_memory().available
            while layers > 1 and _host_bytes_needed(w, args) > 0.85 * avail:
                layers -= 1
                w = dataclasses.replace(L123B, n_layers=layers)
        except ImportError:
            pass
        result = run_step(w, args)
        if not args.no_cpu_baseline:
            print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
            result["cpu_baseline"] = cpu_baseline(w, B1=1, S1=512, n_ce=1024, ad_frac=0.125)
        else:
            result["cpu_baseline"] = None
        print(json.dumps(result))
        return
    w = dataclasses.replace(L8B, batch=args.batch) if args.batch else L8B
    if args.slots:
        w = dataclasses.replace(w, ring_slots=args.slots)
    result = run_step(w, args)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
