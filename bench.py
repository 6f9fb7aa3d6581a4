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
    alg.update(attn_fwd=2 * U, attn_bwd_dkv=3 * U, attn_bwd_dq=1 * U)
    exe.update(attn_fwd=2 * U, attn_bwd_dkv=4 * U, attn_bwd_dq=3 * U)
    nch = (V + ce_chunk - 1) // ce_chunk
    per = 2 * N * V * H / nch           # average per chunk launch
    alg.update(ce_logits_gemm=per / 2, ce_dh_gemm=per, ce_dw_gemm=per)   # logits recomputed
    exe.update(ce_logits_gemm=per, ce_dh_gemm=per, ce_dw_gemm=per)
    return alg, exe


def kernel_bytes(spec, B, S):
    """Algorithmic HBM bytes per launch of the memory-bound kernels (bf16 tensors)."""
    N, H, F, d = B * S, spec.hidden, spec.ffn, spec.head_dim
    QR = (spec.n_heads + 2 * spec.n_kv_heads) * d
    return {"rmsnorm_fwd": 2 * N * H * 2, "rmsnorm_bwd": 4 * N * H * 2,
            "swiglu_fwd": 3 * N * F * 2, "swiglu_bwd": 5 * N * F * 2,
            "rope_fwd": 2 * N * (QR - spec.n_kv_heads * d) * 2,
            "rope_bwd": 2 * N * (QR - spec.n_kv_heads * d) * 2}


def cpu_baseline(w, budget_note=True):
    """The oracle (NumPy fp64) timed on a bounded sample of the same workload, scaled to the
    workload's tokens/s: one layer fwd+bwd at B=1 x S=1024, the LM-head CE on 256 tokens at the
    full vocabulary, and the fp32 AdamW on 1/8 of one layer's parameters."""
    from oracle import adamw as oa
    from oracle import model as om
    from seeded_inputs import activations, layer_params
    c = w.layer
    shape = om.LayerShape(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn)
    S1 = 1024
    p = {k: v.f64 for k, v in layer_params(c, "bf16", seed=0).items()}
    x = activations((1, S1, c.hidden), "bf16", 1).f64
    dy = activations((1, S1, c.hidden), "bf16", 2).f64
    t0 = time.perf_counter()
    y, cache = om.layer_fwd(p, x, shape)
    om.layer_bwd(p, dy, cache, shape)
    t_layer = time.perf_counter() - t0
    del p, cache
    n_ce = 256
    rng = np.random.default_rng(3)
    h = rng.standard_normal((n_ce, c.hidden))
    wl = rng.standard_normal((w.vocab, c.hidden)) * 0.02
    t = rng.integers(0, w.vocab, n_ce)
    t0 = time.perf_counter()
    om.ce_chunked(h, wl, t, w.ce_chunk)
    t_ce = time.perf_counter() - t0
    del wl
    n_ad = c.param_count() // 8
    pa = rng.standard_normal(n_ad).astype(np.float32)
    ga = (rng.standard_normal(n_ad) * 1e-3).astype(np.float32)
    z = np.zeros(n_ad, np.float32)
    t0 = time.perf_counter()
    oa.adamw_fp32(pa, ga, z, z, 1, oa.AdamWHyper())
    t_ad = time.perf_counter() - t0
    n_params = w.n_layers * c.param_count() + 2 * w.vocab * c.hidden + c.hidden
    tokens = w.batch * w.seq
    step_s = (tokens / S1) * w.n_layers * t_layer + (tokens / n_ce) * t_ce + \
        (n_params / n_ad) * t_ad
    cores = len(os.sched_getaffinity(0))
    return {"value": tokens / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 oracle: one {w.name} layer fwd+bwd at B=1 S=1024 ({t_layer:.2f} s), "
                       f"LM-head CE on {n_ce} tokens at V={w.vocab} ({t_ce:.2f} s), fp32 AdamW on "
                       f"{n_ad} params ({t_ad:.2f} s); scaled to {w.n_layers} layers, "
                       f"{tokens} tokens and {n_params} parameters per step"),
            "sample_seconds": round(t_layer + t_ce + t_ad, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle CPU baseline (e.g. under a profiler)")
    ap.add_argument("--adam-threads", type=int, default=0,
                    help="CPU AdamW threads (default: cores - 1)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _die_multi_gpu(max(args.gpus, world))

    import torch
    import layer_sliding_offloaded_fwd_amd as sl
    from layer_sliding_offloaded_fwd_amd.engine import AdamW, ModelSpec, SlideEngine
    from seeded_inputs import L8B, tokens as draw_tokens

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sl.lib()  # fail loudly if libslide.so is missing
    w = L8B
    c = w.layer
    spec = ModelSpec(c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, w.vocab, w.n_layers,
                     "bf16", c.rms_eps, c.rope_theta)
    cores = len(os.sched_getaffinity(0))
    threads = args.adam_threads or max(1, cores - 1)
    t_init = time.perf_counter()
    eng = SlideEngine(spec, w.batch, w.seq, n_slots=w.ring_slots, ce_chunk=w.ce_chunk,
                      hp=AdamW(), adam_threads=threads, timeline=True)
    print("[bench] allocating host and device state", file=sys.stderr, flush=True)
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
    sl.slide_prof_reset()
    sl.slide_prof_enable(True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        eng.step(toks[args.warmup + i])
    eng.wait_updates()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sl.slide_prof_enable(False)
    prof = sl.slide_prof_read()
    loss = eng.loss()
    step_s = (t1 - t0) / args.steps
    tok_s = w.batch * w.seq / step_s
    print(f"[bench] {args.steps} steps: {step_s * 1e3:.1f} ms/step, {tok_s:.0f} tokens/s, "
          f"loss {loss:.4f}", file=sys.stderr, flush=True)

    # ---- kernels
    alg, exe = kernel_flops(spec, w.batch, w.seq, w.ce_chunk)
    byt = kernel_bytes(spec, w.batch, w.seq)
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
    mfma_names = [n for n in kernels if n in alg]
    dom = max(mfma_names, key=lambda n: kernels[n]["total_ms"])
    dk = kernels[dom]
    achieved = alg[dom] / (dk["avg_ms"] * 1e-3) / 1e12
    # forward projections and attention run twice per step (forward and recompute in the
    # backward): the algorithmic count takes them once
    fwd_names = {"gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attn_fwd"}
    layer_names = [n for n in mfma_names if n.startswith(("gemm_", "attn_"))]
    lt = sum(kernels[n]["total_ms"] for n in layer_names) * 1e-3
    l_alg = sum(alg[n] * kernels[n]["launches"] * (0.5 if n in fwd_names else 1.0)
                for n in layer_names)
    l_exe = sum(exe[n] * kernels[n]["launches"] for n in layer_names)
    mfma_util_alg = 100.0 * l_alg / lt / 1e12 / PEAK_BF16_TFLOPS if lt else 0.0
    mfma_util_exec = 100.0 * l_exe / lt / 1e12 / PEAK_BF16_TFLOPS if lt else 0.0

    # ---- overlap (timed steps)
    ana = eng.analyse(eng.records[-args.steps:])
    gpu_ms = ana["gpu_ms"]
    eng.close()

    result = {
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "hidden": c.hidden,
                   "heads": c.n_heads, "kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                   "ffn": c.ffn, "vocab": w.vocab, "global_batch": w.batch, "seq_len": w.seq,
                   "ring_slots": w.ring_slots, "ce_chunk": w.ce_chunk,
                   "parallelism": "single GPU, layers streamed from host",
                   "adam_threads": threads},
        "layer_mfma_util_pct": round(mfma_util_alg, 2),
        "layer_mfma_util_exec_pct": round(mfma_util_exec, 2),
        "overlap_pct": round(ana["overlap_pct"], 1),
        "overlap": {"t_bwd_total_ms": round(ana["t_bwd_total_ms"], 1),
                    "t_d2h_total_ms": round(ana["t_d2h_total_ms"], 1),
                    "t_update_total_ms": round(ana["t_update_total_ms"], 1),
                    "layers_meeting_T_bwd_ge_T_d2h_plus_T_update": ana["predicate_layers_met"],
                    "gpu_span_ms_per_step": round(gpu_ms, 1)},
        "loss_last_step": round(loss, 4),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": dk["avg_ms"], "flops_per_launch": alg[dom]},
        "kernels": kernels,
        "init_s": round(t_init, 1),
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
