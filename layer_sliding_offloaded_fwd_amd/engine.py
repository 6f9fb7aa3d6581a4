"""Thread-based step engine of the layer-sliding method (SlideFormer summary, section 2A:
a lightweight thread-based engine with separate streams for transfers and computation; the
GPU is a sliding window over the layers; while the CPU updates layer i the GPU runs the backward
of layer i-1 and prefetches layer i-2; figures 3-5 of the paper page).

One training step:
  forward   embedding gather; layers 0..L-1 through the slot ring (weights loaded ahead on the
            H2D stream as slots free up); each layer's input and (by default) its forward
            intermediates stay in HBM, so the backward does not recompute the forward.
  loss      final RMSNorm, chunked LM-head cross-entropy (loss, dh, dW_lm).
  backward  layers L-1..0: the last n_slots layers are still resident (re-claimed without a
            copy); every other layer is prefetched n_slots layers ahead; after each layer's
            backward its gradients are flushed to host memory on the D2H stream and a CPU worker
            thread runs AdamW on that layer as soon as they land, while the GPU continues.
  glue      embedding, final gain and LM head are updated the same way; their device copies are
            refreshed by the worker as soon as their update is done.
The host keeps fp32 master weights and AdamW moments per layer. For bf16 compute each layer has
one pinned bf16 buffer that is both the upload source of its weights and the landing buffer of
its gradients; AdamW reads the gradients from it and writes the new bf16 weights back into it
(summary, section 2B: gradients and FP32->BF16 conversions share fixed host buffers).
Every device buffer is allocated once, up front (section 2B: pre-allocated, no fragmentation).

All numerical work runs in libslide (HIP kernels and the C++ AdamW); this module only orders
calls on streams and threads. PyTorch provides device memory, pinned host memory and streams.
"""
import collections
import dataclasses
import json
import mmap
import os
import threading
import sys
import time
from dataclasses import dataclass, field

import numpy as np
import torch

from . import binding as B
from ._capi import SLIDE_BF16, SLIDE_E_NONFINITE, SLIDE_F16, SLIDE_F32

# compute dtype -> (library code, torch dtype of the compute copies, bytes per element)
_DTYPES = {"bf16": (SLIDE_BF16, torch.bfloat16, 2), "f16": (SLIDE_F16, torch.float16, 2),
           "f32": (SLIDE_F32, torch.float32, 4)}


@dataclass(frozen=True)
class ModelSpec:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    dtype: str = "bf16"          # compute dtype: "bf16", "f16" (with loss scaling) or "f32"
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0


@dataclass(frozen=True)
class AdamW:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def _align(n, a=256):
    return (n + a - 1) // a * a


def pinned_bytes(n, esize, min_bytes=0):
    """Bytes allocated for a pinned buffer of n elements of esize bytes that the slot ring may
    copy min_bytes of: the larger of the two, at least 64, rounded up to 256."""
    return _align(max(n * esize, int(min_bytes), 64))


class _Job:
    __slots__ = ("name", "wait", "p", "g", "m", "v", "out", "n", "post", "done", "t_start",
                 "t_end", "t_ready", "t_landed", "step", "priority", "seq", "tier", "nonfinite",
                 "off",
                 "rows", "row_len", "adam_t", "hp", "cancelled", "packed")

    def __init__(self, name, wait, p, g, m, v, out, n, step, priority, post=None, tier=None,
                 off=0, rows=None, row_len=0):
        self.name, self.wait, self.p, self.g, self.m, self.v = name, wait, p, g, m, v
        self.off = off        # element offset of this job's part within its block
        # rows: update only these rows of row_len elements (int32 indices into p, m, v, out,
        # which then hold n // row_len rows); g None: their gradient is exactly zero
        self.rows, self.row_len = rows, row_len
        # packed: g holds only the listed rows (row k for rows[k]); the new rows' upload copy
        # is written over g (and into out, the whole table's upload buffer, for 16-bit)
        self.packed = False
        self.adam_t = step     # AdamW's step count (bias correction); the engine sets it
        self.hp = None         # per-job hyper-parameters (loss-scaled gradients), else the engine's
        self.cancelled = False  # the step was skipped (fp16 overflow): apply nothing
        self.out, self.n, self.post, self.step, self.priority = out, n, post, step, priority
        self.tier = tier      # (p, m, v) offsets in the disk tier (None: in host memory)
        self.nonfinite = None  # (pinned count array, index) when the gradient is checked
        self.seq = 0
        self.done = threading.Event()
        self.t_start = self.t_end = self.t_ready = 0.0
        self.t_landed = None   # host time its gradient copy landed (host-timed copy engines)


class _PinnedPool:
    """Exact-size pinned host buffers from hipHostMalloc (PyTorch's pinned allocator rounds each
    request up to a power of two, which wastes up to half of the host RAM the method needs)."""

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                            ctypes.c_uint]
        self._hip.hipHostFree.argtypes = [ctypes.c_void_p]
        self._ptrs = []

    def tensor(self, n, dtype, min_bytes=0):
        """n elements of dtype; the allocation spans at least min_bytes and is rounded up to
        256 bytes, so a copy of a 256-byte-padded size (the slot ring's) stays inside it."""
        ct = self._ct
        esize = torch.empty(0, dtype=dtype).element_size()
        nbytes = pinned_bytes(n, esize, min_bytes)
        ptr = ct.c_void_p()
        rc = self._hip.hipHostMalloc(ct.byref(ptr), nbytes, 0)
        if rc != 0 or not ptr.value:
            raise MemoryError(f"hipHostMalloc({nbytes}) failed with {rc}")
        self._ptrs.append(ptr.value)
        buf = (ct.c_uint8 * nbytes).from_address(ptr.value)
        return torch.frombuffer(buf, dtype=dtype, count=n)

    def free(self):
        for p in self._ptrs:
            self._hip.hipHostFree(self._ct.c_void_p(p))
        self._ptrs = []


def _host_f32(n):
    """Zero-filled pageable fp32 host array on transparent huge pages where the kernel allows
    (fewer TLB misses for the CPU optimizer's streaming passes)."""
    nbytes = max(4 * n, 4)
    try:
        mm = mmap.mmap(-1, nbytes, flags=mmap.MAP_PRIVATE | mmap.MAP_ANONYMOUS)
        if hasattr(mmap, "MADV_HUGEPAGE"):
            mm.madvise(mmap.MADV_HUGEPAGE)
        return torch.from_numpy(np.frombuffer(mm, dtype=np.float32, count=n))
    except (OSError, ValueError):
        return torch.zeros(n, dtype=torch.float32)


class _Param:
    """Host state of one parameter block: fp32 master, AdamW moments, the pinned buffer that
    serves as upload source and gradient landing zone, and (for resident blocks) the device
    copy and device gradient.
    tier: (p, m, v) byte offsets of the arrays that live in the disk tier instead of host memory
    (the moments always; the master too for bf16 compute, where the pinned bf16 buffer is the
    upload source; None where an array stays in host memory)."""

    def __init__(self, n, dtype, pinned, device=None, resident=False, tier=None, copy_bytes=0,
                 separate_grad=False):
        """copy_bytes: how many bytes the slot ring copies into / out of the pinned buffers
        (its slot size, n elements rounded up to 256 bytes); they are allocated that large.
        separate_grad: for 16-bit compute, the gradient lands in its own pinned buffer instead of the
        upload buffer (the embedding: the update of its untouched rows writes the upload buffer
        while the gradient of the touched rows is still on its way)."""
        self.n = n
        self.dtype = dtype
        self.tier = tier
        if dtype != "f32":
            self.master = _host_f32(n) if tier is None or tier[0] is None else None
            self.shared = pinned.tensor(n, torch.int16, copy_bytes)        # 16-bit bits
            self.grad_host = (pinned.tensor(n, torch.int16) if separate_grad
                              else self.shared)
        else:
            self.master = pinned.tensor(n, torch.float32, copy_bytes)      # upload source
            self.shared = self.master
            self.grad_host = pinned.tensor(n, torch.float32, copy_bytes)
        self.m = _host_f32(n) if tier is None else None
        self.v = _host_f32(n) if tier is None else None
        self.job = None
        self.part_jobs = None   # the last update, when it ran in parts (layer 0)
        if resident:
            tdt = _DTYPES[dtype][1]
            self.dev = torch.empty(n, dtype=tdt, device=device)
            self.grad = torch.empty(n, dtype=tdt, device=device)
            self.ready_ev = None      # h2d of the current device copy
            self.flushed_ev = None    # d2h of the last device gradient


class SlideEngine:
    def __init__(self, spec: ModelSpec, batch, seq, n_slots=3, ce_chunk=8192, hp=AdamW(),
                 adam_threads=0, device="cuda:0", serialize=False, timeline=False,
                 save_activations=True, activations=None, x_slots=4, state_tier=None,
                 tier_layers=None, tier_chunk=0, tier_io_threads=8, check_finite=False,
                 keep_records=64, on_gradient=None, embed_split=False, loss_scale=2.0 ** 16,
                 scale_growth_interval=2000, min_loss_scale=1.0, boundary_parts=8,
                 copy_engine="hsa"):
        """activations: where the forward's state for the backward lives.
          "hbm" (default): every layer's intermediates stay in HBM; no recompute.
          "recompute": only each layer's input stays in HBM; the backward re-runs the forward.
          "host": layer inputs slide to pinned host memory after the forward and come back
            before the backward (the pages' sliding activations), with recompute; only
            x_slots layer-input buffers stay on the device.
        save_activations=False is the older spelling of activations="recompute".
        state_tier: path of a file that holds the optimizer state (AdamW moments, and the fp32
          master for bf16 compute) of the layers in tier_layers (default: every layer) instead
          of host memory (the pages' optional NVMe tier of the CPU optimizer's state). The file
          is opened with O_DIRECT where the file system allows and unlinked at once, so it
          takes disk space only while the engine lives. tier_chunk (elements) and
          tier_io_threads size its streaming.
        check_finite: count the NaN / infinite elements of every gradient on the GPU before it
          is flushed; the CPU worker then refuses the update of a block whose gradient is not
          finite (SlideError SLIDE_E_NONFINITE, raised by the next wait), so the fp32 master
          weights are never overwritten from it.
        copy_engine: "hsa" (default: the slot ring's copies on two host-optimised copy engines
          chosen through the HSA runtime, ordered by host threads; the ring's acquire then
          blocks until the slot's load is in) or "hip" (hipMemcpyAsync, which picks the copy
          engine itself and has put whole steps' gradient copies on engines that run the host
          link at a quarter of its rate). If the HSA ring cannot be created, the engine falls
          back to "hip" with a warning; copy_engine then says which one runs.
        keep_records: how many of the latest steps' records (events, job timings) are kept for
          analyse(); older ones are dropped, so a long run does not accumulate them.
        loss_scale, scale_growth_interval, min_loss_scale: dynamic loss scaling of fp16 compute
          (spec.dtype "f16"). The gradients are computed for loss_scale times the loss; every
          block's gradient is checked for NaN / infinity on the GPU, and a step's CPU updates
          start only once the whole step has passed (they then overlap the next step's forward
          instead of this step's backward). A step with a non-finite gradient is skipped whole:
          no parameter, moment or step count changes, and the scale is halved (not below
          min_loss_scale); after scale_growth_interval good steps in a row it is doubled.
        embed_split: update the embedding's rows that no input token selects (an exactly zero
          gradient) while the step runs, and only the selected rows after the backward (False:
          the whole embedding after the backward, chunk by chunk). Same results either way.
        boundary_parts: layer 0, the last layer of the backward and the first the next forward
          needs, is flushed, updated and uploaded in this many parts (byte ranges of its slot),
          so that its gradient copy, its CPU update and its upload overlap one another at the
          step boundary instead of running back to back; 1 moves it whole. (Not for a layer 0
          whose optimizer state is in the disk tier.)
        on_gradient: optional callable(name, step, offset, grad) run on the CPU worker once a
          gradient has landed in host memory and before the update that consumes it (for bf16
          compute the update overwrites the gradient with the new weights). name is the block
          ("layer3", "embed2", "lm_head0", "w_final"), offset the element offset of this part
          within its block (with embed_split, an embedding part holds only selected rows:
          offset is then the int32 array of their row numbers, grad their rows in that order),
          grad the host tensor (bf16 bits as int16, or fp32). For gradient statistics and
          inspection; it must not modify grad.
        """
        assert spec.dtype in _DTYPES, spec.dtype
        self.fp16 = spec.dtype == "f16"
        assert not (self.fp16 and serialize), "serialize is not supported with fp16 compute"
        if activations is None:
            activations = "hbm" if save_activations else "recompute"
        assert activations in ("hbm", "recompute", "host"), activations
        self.activations = activations
        save_activations = activations == "hbm"
        self.spec, self.B, self.S, self.N = spec, batch, seq, batch * seq
        self.L = spec.n_layers
        self.n_slots = max(1, min(n_slots, self.L))
        self.hp = B.AdamWHp(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
        self.adam_threads = adam_threads
        self.device = torch.device(device)
        self.serialize = serialize
        self.timeline = timeline
        self.save_activations = save_activations
        self.code, self.tdt, self.ts = _DTYPES[spec.dtype]
        # dynamic loss scaling (fp16): the scale, good steps in a row, skipped steps; the
        # optimizer's own step count advances only on applied steps; a step's CPU updates are
        # released (opened_step) once its gradients have been checked
        self.loss_scale = float(loss_scale) if self.fp16 else 1.0
        self.scale_growth_interval = scale_growth_interval
        self.min_loss_scale = min_loss_scale
        self.good_steps = 0
        self.skipped_steps = 0
        self.opt_step = 0
        self.opened_step = 0 if self.fp16 else float("inf")
        s = spec
        self.cfg = B.layer_cfg(s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.ffn, s.dtype,
                               s.rms_eps, s.rope_theta)
        self.ce_cfg = B.CeCfg(s.hidden, s.vocab, ce_chunk, self.code)
        self.P = B.slide_layer_param_count(self.cfg)
        self.w_bytes = _align(self.P * self.ts)
        H, V, N = s.hidden, s.vocab, self.N

        # streams: one for compute, one per copy direction (default priority)
        self.compute = torch.cuda.Stream(device=self.device)
        self.h2d = torch.cuda.Stream(device=self.device)
        self.d2h = torch.cuda.Stream(device=self.device)

        # host parameter blocks
        self.pinned = _PinnedPool()
        self.tier = None
        tiered = set()
        if state_tier is not None:
            tiered = set(range(self.L) if tier_layers is None else tier_layers)
            assert tiered <= set(range(self.L)), tier_layers
            reg = B.slide_tier_region_bytes(self.P)
            arrays = 3 if s.dtype != "f32" else 2
            self.tier = B.StateTier(state_tier, max(arrays * reg * len(tiered), 4096),
                                    tier_chunk, tier_io_threads)
        self.tier_layers = sorted(tiered)
        self.layers = []
        o = 0
        for i in range(self.L):
            offs = None
            if i in tiered:
                if s.dtype != "f32":
                    offs, o = (o, o + reg, o + 2 * reg), o + 3 * reg
                else:
                    offs, o = (None, o, o + reg), o + 2 * reg
            self.layers.append(_Param(self.P, s.dtype, self.pinned, tier=offs,
                                      copy_bytes=self.w_bytes))
        # layer 0 in parts at the step boundary: element ranges starting on 256-byte boundaries
        self.l0_parts = None
        if boundary_parts > 1 and 0 not in tiered:
            step_el = _align(-(-self.P * self.ts // boundary_parts)) // self.ts
            self.l0_parts = [(a, min(a + step_el, self.P)) for a in range(0, self.P, step_el)]
        self.embed_split = embed_split
        self.embed = _Param(V * H, s.dtype, self.pinned, self.device, resident=True)
        self.final = _Param(H, s.dtype, self.pinned, self.device, resident=True)
        self.lm = _Param(V * H, s.dtype, self.pinned, self.device, resident=True)
        # The LM head is updated, uploaded and flushed per vocabulary chunk of the fused CE, so
        # the CE's first pass starts on chunk c as soon as that chunk is updated, and the CPU
        # starts on chunk c's next update as soon as the second pass has produced its dW.
        self.lm_nch = B.slide_lmhead_ce_n_chunks(self.ce_cfg)
        C = min(ce_chunk if ce_chunk > 0 else 8192, V)
        self.lm_rows = [(ci * C, min((ci + 1) * C, V)) for ci in range(self.lm_nch)]
        self.lm_job = [None] * self.lm_nch        # pending CPU update per chunk
        self.lm_ready = [None] * self.lm_nch      # H2D of the chunk's current device copy
        self.lm_flushed = [None] * self.lm_nch    # D2H of the chunk's last device gradient
        # The embedding is flushed, updated and uploaded in row chunks too: at the step boundary
        # its gradient's D2H, CPU update and upload overlap chunk by chunk instead of running one
        # after the other before the next forward can start.
        self.emb_nch = min(8, V)
        er = -(-V // self.emb_nch)
        self.emb_rows = [(ci * er, min((ci + 1) * er, V)) for ci in range(self.emb_nch)
                         if ci * er < V]
        self.emb_nch = len(self.emb_rows)
        self.emb_job = [None] * self.emb_nch
        self.emb_ready = [None] * self.emb_nch
        self.emb_flushed = [None] * self.emb_nch
        # Rows of the embedding that no input token of a step selects have an exactly zero
        # gradient: their update needs no gradient copy, so it runs as soon as the step's gather
        # has been issued (off the step boundary); after the backward only the selected rows
        # are updated, chunk by chunk.
        self.emb_zero_job = None
        self.emb_present = None
        # With the split, only the selected rows cross the link at the step boundary: their
        # gradient rows are packed on the device, copied out, updated and copied back packed,
        # then scattered into the table; the rest of the table goes up after its zero-gradient
        # update, during the step.
        self.emb_scatter_n = 0          # selected rows whose new values wait to be scattered
        self.emb_zero_up_ev = None      # upload of the table after the zero-row update
        if embed_split:
            R = min(N, V)
            self.emb_rows_host = self.pinned.tensor(R, torch.int32)
            self.emb_rows_dev = torch.empty(R, dtype=torch.int32, device=self.device)
            self.emb_gc_dev = torch.empty(R * H, dtype=self.tdt, device=self.device)
            self.emb_gc_host = self.pinned.tensor(
                R * H, torch.int16 if s.dtype != "f32" else torch.float32)

        # device memory, allocated once
        dev = self.device
        # fp16 counts every block's non-finite gradient elements for its loss-scale check
        self.check_finite = check_finite or self.fp16
        self.on_gradient = on_gradient
        if self.check_finite:
            names = ([f"layer{i}" for i in range(self.L)] + ["w_final"]
                     + [f"lm_head{ci}" for ci in range(self.lm_nch)]
                     + [f"embed{ci}" for ci in range(self.emb_nch)])
            self.nf_index = {n: k for k, n in enumerate(names)}
            self.nf_dev = torch.zeros(len(names), dtype=torch.int32, device=dev)
            self.nf_host = self.pinned.tensor(len(names), torch.int32)
        self.ring_mem = torch.empty(self.n_slots * 2 * self.w_bytes, dtype=torch.uint8, device=dev)
        if copy_engine not in ("hip", "hsa"):
            raise ValueError(f"copy_engine must be 'hip' or 'hsa', not {copy_engine!r}")
        self.copy_engine = copy_engine
        if copy_engine == "hsa":
            try:
                self.ring = B.SlotRing(self.n_slots, self.w_bytes, self.w_bytes, self.ring_mem,
                                       self.h2d, self.d2h, engine=B.SLIDE_ENGINE_HSA)
            except B.SlideError as e:
                print(f"[slide] HSA copy engines unavailable ({e}); using hipMemcpyAsync",
                      file=sys.stderr, flush=True)
                self.copy_engine = "hip"
        if self.copy_engine == "hip":
            self.ring = B.SlotRing(self.n_slots, self.w_bytes, self.w_bytes, self.ring_mem,
                                   self.h2d, self.d2h, engine=B.SLIDE_ENGINE_HIP)
        if activations == "host":
            # a ring of x_slots device buffers: layer input i lives in slot i % x_slots; the
            # inputs a later layer's output would overwrite are copied to pinned host memory
            self.x_slots = max(3, min(x_slots, self.L + 1))
            self.xs = torch.empty((self.x_slots, N, H), dtype=self.tdt, device=dev)
            self.x_host = self.pinned.tensor((self.L + 1) * N * H,
                                             torch.int16 if s.dtype != "f32" else torch.float32)
            self.x_d2h_ev = [None] * (self.L + 1)
            self.x_h2d_ev = [None] * (self.L + 1)
        else:
            self.x_slots = self.L + 1
            self.xs = torch.empty((self.L + 1, N, H), dtype=self.tdt, device=dev)   # layer inputs
        self.grad_x = torch.empty((N, H), dtype=self.tdt, device=dev)
        self.hf = torch.empty((N, H), dtype=self.tdt, device=dev)
        self.dhf = torch.empty((N, H), dtype=self.tdt, device=dev)
        self.tok_in = torch.empty(N, dtype=torch.int32, device=dev)
        self.tok_tgt = torch.empty(N, dtype=torch.int32, device=dev)
        self.loss_dev = torch.zeros(1, dtype=torch.float32, device=dev)
        # forward intermediates of every layer stay in HBM (no recompute in the backward), or
        # only the layer inputs are kept and the backward recomputes the forward
        if save_activations:
            self.saved_bytes = _align(B.slide_layer_saved_bytes(self.cfg, batch, seq))
            self.saved = torch.empty((self.L, self.saved_bytes), dtype=torch.uint8, device=dev)
            layer_ws = B.slide_layer_workspace_bytes(self.cfg, batch, seq, 2)
        else:
            self.saved_bytes, self.saved = 0, None
            layer_ws = max(B.slide_layer_workspace_bytes(self.cfg, batch, seq, 1),
                           B.slide_layer_workspace_bytes(self.cfg, batch, seq, 0))
        ws = max(layer_ws,
                 B.slide_lmhead_ce_workspace_bytes(self.ce_cfg, N),
                 B.slide_embed_bwd_workspace_bytes(N, V),
                 B.slide_rmsnorm_bwd_workspace_bytes(N, H))
        self.ws_bytes = _align(ws)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

        # CPU optimizer worker: runs, among the updates whose gradients have landed, the one the
        # next forward needs first (embedding, then layers in forward order, LM head last), so
        # the updates still pending at the end of a backward overlap the next forward
        self.jobs = []
        self.jobs_cv = threading.Condition()
        self.job_seq = 0
        self.worker_stop = False
        self.worker_error = None
        self.workers = [threading.Thread(target=self._worker_loop, daemon=True, name="slide-adamw")]
        if self.tier is not None:
            # the tier's updates stream their state through the file; their arithmetic needs few
            # cores, so they get a share of the optimizer threads and run beside the others
            self.tier_threads = max(2, (adam_threads or 12) // 3)
            self.workers.append(threading.Thread(target=self._worker_loop, args=(True,),
                                                 daemon=True, name="slide-adamw-tier"))
        for t in self.workers:
            t.start()
        self.step_count = 0
        self.records = collections.deque(maxlen=max(1, keep_records))

    # ------------------------------------------------------------------ parameters
    def load_params(self, embed, layers, w_final, lm_head):
        """Set fp32 master weights (numpy or torch, any shape; layers in slot packing order)
        and derive the compute copies. Moments are reset to zero and the step counter to 0."""
        self.wait_updates()

        def put(prm, arr):
            t = torch.as_tensor(np.ascontiguousarray(arr, dtype=np.float32)
                                if isinstance(arr, np.ndarray) else arr).reshape(-1).float()
            assert t.numel() == prm.n
            self._set_master(prm, t)
            self._zero_moments(prm)

        put(self.embed, embed)
        put(self.final, w_final)
        put(self.lm, lm_head)
        assert len(layers) == self.L
        for prm, arr in zip(self.layers, layers):
            put(prm, arr)
        self._upload_all_resident()
        self._reset_counts()

    def init_random(self, seed=0, std=0.02, progress=None):
        """Seeded synthetic weights drawn on the GPU (matrices N(0, std), norm gains 1).
        progress(msg) is called every few layers."""
        self.wait_updates()
        gen = torch.Generator(device=self.device)
        gen.manual_seed(seed)
        offs = B.slide_layer_param_offsets(self.cfg)
        H = self.spec.hidden

        def draw(prm, gains=()):
            t = torch.empty(prm.n, dtype=torch.float32, device=self.device)
            t.normal_(0.0, std, generator=gen)
            for o in gains:
                t[o:o + H] = 1.0
            self._set_master(prm, t)
            if self.step_count:          # moments are zero from construction until a step ran
                self._zero_moments(prm)

        draw(self.embed)
        for i, prm in enumerate(self.layers):
            draw(prm, gains=(offs[0], offs[3]))
            if progress is not None and (i + 1) % 8 == 0:
                progress(f"initialised {i + 1}/{self.L} layers")
        self.final.master.fill_(1.0)
        self._refresh_shared(self.final)
        draw(self.lm)
        self._upload_all_resident()
        self._reset_counts()

    def _reset_counts(self, step=0, opt_step=None):
        self.step_count = step
        self.opt_step = step if opt_step is None else opt_step
        if self.fp16:
            self.opened_step = step

    def _refresh_shared(self, prm, src=None):
        """The 16-bit compute copy (the upload buffer) of a block from its fp32 master (or from
        src, a host fp32 tensor of the same values), rounded by the library."""
        if prm.dtype != "f32":
            if src is None:
                src = prm.master if prm.master is not None else torch.from_numpy(
                    self._get_master(prm))
            B.slide_cpu_convert_f32(src, prm.shared, self.code, prm.n, self.adam_threads)

    def _set_master(self, prm, t):
        """fp32 master weights of a block (a float32 tensor of prm.n elements, any device), and
        the 16-bit compute copy derived from them."""
        host = t.detach().to("cpu").float().contiguous()
        if prm.master is not None:
            prm.master.copy_(host)
        else:
            self.tier.write(prm.tier[0], host)
        self._refresh_shared(prm, host)

    def _zero_moments(self, prm):
        if prm.tier is None:
            prm.m.zero_()
            prm.v.zero_()
        else:
            self.tier.write(prm.tier[1], None, 4 * prm.n)
            self.tier.write(prm.tier[2], None, 4 * prm.n)

    def _get_master(self, prm):
        if prm.master is not None:
            return prm.master.numpy().copy()
        out = np.empty(prm.n, np.float32)
        self.tier.read(prm.tier[0], out)
        return out

    # ------------------------------------------------------------------ checkpoint
    def _blocks(self):
        out = {"embed": self.embed, "w_final": self.final, "lm_head": self.lm}
        out.update({f"layer{i}": p for i, p in enumerate(self.layers)})
        return out

    def _state(self, prm, kind):
        """fp32 master ("master"), first ("m") or second ("v") moment of a block as a numpy copy,
        from host memory or the disk tier."""
        arr = {"master": prm.master, "m": prm.m, "v": prm.v}[kind]
        if arr is not None:
            return arr.numpy().copy()
        out = np.empty(prm.n, np.float32)
        self.tier.read(prm.tier[{"master": 0, "m": 1, "v": 2}[kind]], out)
        return out

    def save_checkpoint(self, path):
        """Write the host state after every pending update: each block's fp32 master weights and
        AdamW moments as .npy files under `path`, and a manifest with the step count, the model
        shape and the hyper-parameters. The bf16 compute copies are not saved; they are the
        rounding of the master weights."""
        self.wait_updates()
        os.makedirs(path, exist_ok=True)
        blocks = self._blocks()
        for name, prm in blocks.items():
            for kind in ("master", "m", "v"):
                np.save(os.path.join(path, f"{name}.{kind}.npy"), self._state(prm, kind),
                        allow_pickle=False)
        manifest = dict(step=self.step_count, opt_step=self.opt_step,
                        loss_scale=self.loss_scale, good_steps=self.good_steps,
                        spec=dataclasses.asdict(self.spec),
                        hp=dict(lr=self.hp.lr, beta1=self.hp.beta1, beta2=self.hp.beta2,
                                eps=self.hp.eps, weight_decay=self.hp.weight_decay),
                        blocks={name: prm.n for name, prm in blocks.items()})
        with open(os.path.join(path, "manifest.json"), "w") as f:
            json.dump(manifest, f, indent=1)

    def load_checkpoint(self, path):
        """Restore what save_checkpoint wrote (same model shape): master weights, moments, the
        derived compute copies and the step count. The next step continues exactly as the
        saved run would have."""
        self.wait_updates()
        with open(os.path.join(path, "manifest.json")) as f:
            manifest = json.load(f)
        if manifest["spec"] != dataclasses.asdict(self.spec):
            raise ValueError(f"checkpoint of {manifest['spec']}, engine is {self.spec}")
        blocks = self._blocks()
        if manifest["blocks"] != {name: prm.n for name, prm in blocks.items()}:
            raise ValueError("checkpoint block sizes differ from the engine's")
        for name, prm in blocks.items():
            ld = lambda kind: np.load(os.path.join(path, f"{name}.{kind}.npy"), allow_pickle=False)
            self._set_master(prm, torch.from_numpy(ld("master")))
            for kind, idx in (("m", 1), ("v", 2)):
                arr = ld(kind)
                if prm.tier is None:
                    getattr(prm, kind).copy_(torch.from_numpy(arr))
                else:
                    self.tier.write(prm.tier[idx], arr)
        self._upload_all_resident()
        self._reset_counts(int(manifest["step"]), int(manifest.get("opt_step", manifest["step"])))
        if self.fp16 and "loss_scale" in manifest:
            self.loss_scale = float(manifest["loss_scale"])
            self.good_steps = int(manifest.get("good_steps", 0))

    def tier_stats(self):
        """Traffic and time of the disk tier so far (None without a tier)."""
        return None if self.tier is None else dict(self.tier.stats(), **self.tier.info())

    def _upload_all_resident(self):
        for prm in (self.embed, self.final, self.lm):
            self._upload_resident(prm)
        self.lm_ready = [self.lm.ready_ev] * self.lm_nch
        self.lm_job = [None] * self.lm_nch
        self.emb_ready = [self.embed.ready_ev] * self.emb_nch
        self.emb_job = [None] * self.emb_nch
        self.emb_flushed = [None] * self.emb_nch
        self.emb_zero_job = None
        self.emb_scatter_n = 0
        self.emb_zero_up_ev = None
        torch.cuda.synchronize(self.device)

    def _upload_resident(self, prm):
        with torch.cuda.stream(self.h2d):
            src = prm.shared.view(self.tdt) if prm.dtype != "f32" else prm.shared
            prm.dev.copy_(src, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(self.h2d)
        prm.ready_ev = ev

    def master_params(self):
        """fp32 master weights as numpy arrays (after waiting for pending updates)."""
        self.wait_updates()
        return dict(embed=self.embed.master.numpy().copy(),
                    layers=[self._get_master(p) for p in self.layers],
                    w_final=self.final.master.numpy().copy(),
                    lm_head=self.lm.master.numpy().copy())

    # ------------------------------------------------------------------ CPU worker
    def _landed(self, job):
        """Non-blocking: have this job's gradients arrived in host memory (and, for fp16 compute,
        has its step passed the overflow check)?"""
        if job.step > self.opened_step:
            return False
        if job.wait is None:
            return True
        if isinstance(job.wait, int):
            try:
                self.ring.wait_flush(job.wait, 0)
                if self.copy_engine == "hsa" and job.t_landed is None:
                    job.t_landed = self.ring.ticket_time(job.wait)
                return True
            except B.SlideError as e:
                if e.code == -6:   # SLIDE_E_TIMEOUT: still in flight
                    return False
                raise
        return job.wait.query()

    def _worker_loop(self, tiered=False):
        """One CPU worker: the updates of blocks whose state is in host memory, or (tiered)
        those whose state is in the disk tier, which wait mostly on the file and so run beside
        the in-memory ones instead of holding them up."""
        def mine():
            return [j for j in self.jobs if (j.tier is not None) == tiered]

        while True:
            with self.jobs_cv:
                while not mine() and not self.worker_stop:
                    self.jobs_cv.wait()
                pending = mine()
                if not pending and self.worker_stop:
                    return
            try:
                ready = [j for j in pending if self._landed(j)]
            except Exception as e:
                self.worker_error = e
                ready = pending
            if not ready:
                time.sleep(50e-6)
                continue
            # a step's updates before the next step's (every one is needed by that step's
            # forward), then the one the next forward needs first
            job = min(ready, key=lambda j: (j.step, j.priority, j.seq))
            with self.jobs_cv:
                self.jobs.remove(job)
            try:
                if self.worker_error is None and not job.cancelled:
                    if job.nonfinite is not None:
                        arr, k = job.nonfinite
                        bad = int(arr[k])
                        if bad:
                            raise B.SlideError(
                                SLIDE_E_NONFINITE, "slide_nonfinite_count",
                                f"{job.name}: {bad} NaN or infinite gradient elements in step "
                                f"{job.step}; its update was not applied")
                    if self.on_gradient is not None and job.g is not None:
                        self.on_gradient(job.name, job.step,
                                         job.rows if job.packed else job.off, job.g)
                    job.t_ready = time.perf_counter()
                    hp = job.hp if job.hp is not None else self.hp
                    if job.packed:
                        B.slide_cpu_adamw_rows_packed(
                            job.p, job.m, job.v, job.row_len, job.n // job.row_len, job.rows,
                            len(job.rows), job.g, self.code, job.out, job.g, job.adam_t, hp,
                            self.adam_threads)
                    elif job.rows is not None:
                        if len(job.rows):
                            B.slide_cpu_adamw_rows(job.p, job.g, self.code, job.m, job.v,
                                                   job.out, job.row_len, job.n // job.row_len,
                                                   job.rows, len(job.rows), job.adam_t, hp,
                                                   self.adam_threads)
                    elif job.tier is None:
                        B.slide_cpu_adamw(job.p, job.g, self.code, job.m, job.v, job.out, job.n,
                                          job.adam_t, hp, self.adam_threads)
                    else:
                        po, mo, vo = job.tier
                        self.tier.adamw(job.p, po or 0, job.m, mo, job.v, vo, job.g, self.code,
                                        job.out, job.n, job.adam_t, hp, self.tier_threads)
                    job.t_start = job.t_ready
                    job.t_end = time.perf_counter()
                    if job.post is not None:
                        job.post()
            except Exception as e:  # surfaced on the main thread by wait_updates / step
                self.worker_error = e
            finally:
                job.done.set()

    def _submit(self, prm, wait, name, priority, post=None):
        out = prm.shared if prm.dtype != "f32" else None
        job = _Job(name, wait, prm.master, prm.grad_host, prm.m, prm.v, out, prm.n,
                   self.step_count, priority, post, prm.tier)
        self._nf_attach(job)
        prm.job, prm.part_jobs = job, None
        return self._enqueue(job)

    def _submit_parts(self, prm, tickets, name, priority):
        """The update of a layer flushed in parts (l0_parts): one job per part, each waiting for
        its own gradient copy; the parts' uploads follow as each job finishes."""
        jobs = []
        for (a, b), t in zip(self.l0_parts, tickets):
            out = prm.shared[a:b] if prm.dtype != "f32" else None
            job = _Job(name, t, prm.master[a:b], prm.grad_host[a:b], prm.m[a:b], prm.v[a:b],
                       out, b - a, self.step_count, priority, off=a)
            self._nf_attach(job)
            jobs.append(self._enqueue(job))
        prm.job, prm.part_jobs = None, jobs
        return jobs

    # ------------------------------------------------------------------ non-finite check
    def _nf_count(self, grad, n, name):
        """On the compute stream, after the gradient is complete: count its non-finite
        elements into the block's device counter (check_finite only)."""
        if self.check_finite:
            k = self.nf_index[name]
            B.slide_nonfinite_count(grad, self.code, n, self.nf_dev[k:k + 1], self.compute)

    def _nf_fetch(self, name):
        """On the D2H stream, ahead of the gradient copy: the counter to pinned host memory, so
        the gradient's arrival implies the count's."""
        if self.check_finite:
            k = self.nf_index[name]
            self.nf_host[k:k + 1].copy_(self.nf_dev[k:k + 1], non_blocking=True)

    def _nf_attach(self, job):
        """The worker refuses a non-finite update (check_finite); with fp16 compute the engine
        decides for the whole step instead."""
        if self.check_finite and not self.fp16 and job.name in self.nf_index:
            job.nonfinite = (self.nf_host, self.nf_index[job.name])

    def _enqueue(self, job):
        job.adam_t = self.opt_step + 1
        if self.fp16:
            h = self.hp
            job.hp = B.AdamWHp(h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, self.loss_scale)
        with self.jobs_cv:
            self.job_seq += 1
            job.seq = self.job_seq
            self.jobs.append(job)
            self.jobs_cv.notify_all()
        if self.serialize:
            job.done.wait()
        return job

    def _wait_param(self, prm):
        self._wait_job(prm.job)
        for j in prm.part_jobs or ():
            self._wait_job(j)

    def _wait_job(self, job):
        if job is not None:
            job.done.wait()
            if self.worker_error is not None:
                raise self.worker_error

    def wait_updates(self):
        for prm in self.layers + [self.embed, self.final, self.lm]:
            self._wait_param(prm)
        for ci in range(self.lm_nch):
            self._wait_job(self.lm_job[ci])
        for ci in range(self.emb_nch):
            self._wait_job(self.emb_job[ci])
        self._wait_job(self.emb_zero_job)
        self._embed_catch_up()           # the device table holds the updated rows too

    def close(self):
        """Wait for the pending updates and free every resource. A worker error is raised after
        the clean-up (the updates after it were not applied)."""
        err = None
        try:
            self.wait_updates()
        except Exception as e:  # noqa: BLE001 - re-raised below, after the clean-up
            err = e
        with self.jobs_cv:
            self.worker_stop = True
            self.jobs_cv.notify_all()
        for t in self.workers:
            t.join()
        self.ring.close()
        torch.cuda.synchronize(self.device)
        for prm in self.layers + [self.embed, self.final, self.lm]:
            prm.master = prm.shared = prm.grad_host = None
        self.pinned.free()
        if self.tier is not None:
            self.tier.close()
        if err is not None:
            raise err

    # ------------------------------------------------------------------ step
    def _sync(self):
        if self.serialize:
            torch.cuda.synchronize(self.device)

    def _ev(self, stream):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        return ev

    def _flush_resident(self, prm, name, priority):
        """D2H of a resident block's device gradient after the compute stream, then AdamW, then
        the refreshed device copy goes back up on the H2D stream."""
        self._nf_count(prm.grad, prm.n, name)
        ev_c = torch.cuda.Event()
        ev_c.record(self.compute)
        self.d2h.wait_event(ev_c)
        with torch.cuda.stream(self.d2h):
            self._nf_fetch(name)
            dst = prm.grad_host.view(self.tdt) if prm.dtype != "f32" else prm.grad_host
            dst.copy_(prm.grad, non_blocking=True)
            done = torch.cuda.Event()
            done.record(self.d2h)
        prm.flushed_ev = done
        return self._submit(prm, done, name, priority, post=lambda: self._upload_resident(prm))

    # ------------------------------------------------------------------ sliding activations
    def _x(self, i):
        """Device buffer of layer input i (i = L: the last layer's output)."""
        return self.xs[i % self.x_slots]

    def _x_host(self, i):
        n = self.N * self.spec.hidden
        t = self.x_host[i * n:(i + 1) * n]
        return (t.view(self.tdt) if self.spec.dtype != "f32" else t).view(self.N, -1)

    def _x_offload(self, i):
        """After the compute stream's work so far (the forward of layer i), copy layer input i
        to host memory; its slot may be overwritten once the copy is done."""
        ev = torch.cuda.Event()
        ev.record(self.compute)
        self.d2h.wait_event(ev)
        with torch.cuda.stream(self.d2h):
            self._x_host(i).copy_(self._x(i), non_blocking=True)
            done = torch.cuda.Event()
            done.record(self.d2h)
        self.x_d2h_ev[i] = done

    def _x_reload(self, i):
        """After the compute stream's work so far (which last used slot i % x_slots), bring
        layer input i back from host memory into its slot."""
        ev = torch.cuda.Event()
        ev.record(self.compute)
        self.h2d.wait_event(ev)
        self.h2d.wait_event(self.x_d2h_ev[i])
        with torch.cuda.stream(self.h2d):
            self._x(i).copy_(self._x_host(i), non_blocking=True)
            done = torch.cuda.Event()
            done.record(self.h2d)
        self.x_h2d_ev[i] = done

    def _flush_chunk(self, prm, r0, r1, name, priority, rec, on_ready, rows=None):
        """D2H of rows [r0, r1) of a resident block's gradient once the compute stream has
        produced them, then those rows' AdamW, then the refreshed rows go back up on the H2D
        stream (on_ready(event) is called with the upload's event). rows: update only these
        rows (int32, relative to r0; the others were updated already). Returns (job, flush
        event)."""
        H = self.spec.hidden
        sl = slice(r0 * H, r1 * H)
        self._nf_count(prm.grad[sl], (r1 - r0) * H, name)
        ev_c = torch.cuda.Event()
        ev_c.record(self.compute)
        self.d2h.wait_event(ev_c)
        with torch.cuda.stream(self.d2h):
            self._nf_fetch(name)
            dst = prm.grad_host[sl]
            dst = dst.view(self.tdt) if prm.dtype != "f32" else dst
            dst.copy_(prm.grad[sl], non_blocking=True)
            done = torch.cuda.Event()
            done.record(self.d2h)

        def upload():
            with torch.cuda.stream(self.h2d):
                src = prm.shared[sl]
                src = src.view(self.tdt) if prm.dtype != "f32" else src
                prm.dev[sl].copy_(src, non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(self.h2d)
            on_ready(ev)

        out = prm.shared[sl] if prm.dtype != "f32" else None
        job = _Job(name, done, prm.master[sl], prm.grad_host[sl], prm.m[sl], prm.v[sl], out,
                   (r1 - r0) * H, self.step_count, priority, upload, off=r0 * H, rows=rows,
                   row_len=H)
        self._nf_attach(job)
        rec["other_jobs"].append(job)
        return job, done

    def _flush_lm_chunk(self, ci, rec):
        """LM-head chunk ci: flushed, updated and uploaded on its own (see _flush_chunk)."""
        r0, r1 = self.lm_rows[ci]

        def ready(ev):
            self.lm_ready[ci] = ev
        job, done = self._flush_chunk(self.lm, r0, r1, f"lm_head{ci}",
                                      self.L + 1 + ci / self.lm_nch, rec, ready)
        self.lm_flushed[ci] = done
        self.lm_job[ci] = job
        return self._enqueue(job)

    def _update_embed_zero_rows(self, rec):
        """After this step's gather has been issued (and every earlier update of the embedding
        is done): update the rows that no input token selects, whose gradient this step is
        exactly zero, with no gradient copy. Their upload goes with the chunks after the
        backward; this update runs before those chunks' (priority -2)."""
        V, H = self.spec.vocab, self.spec.hidden
        zero = np.ones(V, bool)
        zero[self.emb_present] = False
        rows = np.flatnonzero(zero).astype(np.int32)
        prm = self.embed
        out = prm.shared if prm.dtype != "f32" else None
        ev_g = torch.cuda.Event()
        ev_g.record(self.compute)        # the gather that reads the current table

        def upload():
            # the whole table goes up (its selected rows still hold the values the device
            # has; their new values are scattered over them before the next gather)
            self.h2d.wait_event(ev_g)
            with torch.cuda.stream(self.h2d):
                src = prm.shared.view(self.tdt) if prm.dtype != "f32" else prm.shared
                prm.dev.copy_(src, non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(self.h2d)
            self.emb_zero_up_ev = ev
        job = _Job("embed_zero", None, prm.master, None, prm.m, prm.v, out, V * H,
                   self.step_count, -2, post=upload, rows=rows, row_len=H)
        rec["other_jobs"].append(job)
        self.emb_zero_job = job
        self._enqueue(job)

    def _embed_catch_up(self):
        """Order the compute stream after the embedding's last updates and uploads (its chunks
        or packed parts, and with embed_split the table after its zero-row update), and
        scatter the packed rows into the table: from here the device table is current. The
        updates themselves must be done (their jobs issue the uploads)."""
        c, H, V = self.compute, self.spec.hidden, self.spec.vocab
        for ci in range(self.emb_nch):
            if self.emb_ready[ci] is not None:
                c.wait_event(self.emb_ready[ci])
            if self.emb_flushed[ci] is not None:
                c.wait_event(self.emb_flushed[ci])
        self._wait_job(self.emb_zero_job)
        if self.emb_zero_up_ev is not None:
            c.wait_event(self.emb_zero_up_ev)
            self.emb_zero_up_ev = None
        if self.emb_scatter_n:
            n = self.emb_scatter_n
            B.slide_copy_rows(self.emb_gc_dev, None, n, self.embed.dev, self.emb_rows_dev, V, n,
                              H * self.ts, c)
            self.emb_scatter_n = 0

    def _flush_embed_packed(self, rec):
        """embed_split: the selected rows' gradient, packed on the device, leaves in parts; each
        part is updated (priorities -1 .. -1/n, before every layer) and its new rows go back
        packed; the next forward scatters them into the table before its gather."""
        prm, H, V = self.embed, self.spec.hidden, self.spec.vocab
        pres = self.emb_present
        n = len(pres)
        c = self.compute
        B.slide_copy_rows(prm.grad, self.emb_rows_dev, V, self.emb_gc_dev, None, n, n,
                          H * self.ts, c)
        nch = self.emb_nch
        per = -(-n // nch) if n else 0
        for ci in range(nch):
            k0, k1 = min(ci * per, n), min((ci + 1) * per, n)
            self.emb_job[ci] = self.emb_ready[ci] = self.emb_flushed[ci] = None
            if k0 >= k1:
                continue
            sl = slice(k0 * H, k1 * H)
            self._nf_count(self.emb_gc_dev[sl], (k1 - k0) * H, f"embed{ci}")
            ev_c = torch.cuda.Event()
            ev_c.record(c)
            self.d2h.wait_event(ev_c)
            gh = self.emb_gc_host[sl]
            with torch.cuda.stream(self.d2h):
                self._nf_fetch(f"embed{ci}")
                (gh.view(self.tdt) if prm.dtype != "f32" else gh).copy_(self.emb_gc_dev[sl],
                                                                       non_blocking=True)
                done = torch.cuda.Event()
                done.record(self.d2h)

            def upload(ci=ci, sl=sl, gh=gh):
                with torch.cuda.stream(self.h2d):
                    self.emb_gc_dev[sl].copy_(gh.view(self.tdt) if prm.dtype != "f32" else gh,
                                              non_blocking=True)
                    ev = torch.cuda.Event()
                    ev.record(self.h2d)
                self.emb_ready[ci] = ev
            out = prm.shared if prm.dtype != "f32" else None
            job = _Job(f"embed{ci}", done, prm.master, gh, prm.m, prm.v, out, V * H,
                       self.step_count, -1 + ci / nch, post=upload, rows=pres[k0:k1],
                       row_len=H)
            job.packed = True
            self._nf_attach(job)
            rec["other_jobs"].append(job)
            self.emb_flushed[ci] = done
            self.emb_job[ci] = job
            self._enqueue(job)
        self.emb_scatter_n = n

    def _flush_embed(self, rec):
        """The embedding's gradient in row chunks, each flushed, updated (before every layer:
        priorities -1 .. -1/n) and uploaded on its own."""
        for ci, (r0, r1) in enumerate(self.emb_rows):
            def ready(ev, ci=ci):
                self.emb_ready[ci] = ev
            job, done = self._flush_chunk(self.embed, r0, r1, f"embed{ci}",
                                          -1 + ci / self.emb_nch, rec, ready)
            self.emb_flushed[ci] = done
            self.emb_job[ci] = job
            self._enqueue(job)

    def step(self, tokens):
        """One training step on int32 tokens [B, S+1] (inputs [:, :S], targets [:, 1:]).
        Returns the loss (float)."""
        if self.worker_error is not None:
            raise self.worker_error
        spec, N, H, V, L = self.spec, self.N, self.spec.hidden, self.spec.vocab, self.L
        c = self.compute
        tok = torch.as_tensor(np.asarray(tokens, dtype=np.int32))
        assert tok.shape == (self.B, self.S + 1), tok.shape
        self.step_count += 1
        rec = dict(step=self.step_count, layers={}, jobs=[], other_jobs=[])
        t_step0 = time.perf_counter()
        ev0 = self._ev(c)          # the compute stream is idle here: ev0 ~ host time t_step0
        rec["host_t0"] = t_step0
        with torch.cuda.stream(c):
            self.tok_in.copy_(tok[:, :-1].reshape(-1), non_blocking=False)
            self.tok_tgt.copy_(tok[:, 1:].reshape(-1), non_blocking=False)

        # ---- forward
        host_x = self.activations == "host"
        K = self.x_slots
        # Prefetch: load layers in order into free slots as soon as their update is done,
        # without blocking; block only for the layer the forward needs next.
        slots = {}
        nxt = [0]
        free = [self.n_slots]
        part = dict(slot=-1, k=0)   # progress of a layer uploaded in parts

        def load_parts(j, prm, need):
            """Upload the parts of layer j whose updates are done, in order; True once all
            are on their way."""
            jobs = prm.part_jobs
            while part["k"] < len(jobs):
                k = part["k"]
                if not jobs[k].done.is_set():
                    if need != j:
                        return False
                    self._wait_job(jobs[k])
                a, b = self.l0_parts[k]
                part["slot"] = self.ring.load_range(j, prm.shared, a * self.ts, (b - a) * self.ts,
                                                    part["slot"])
                part["k"] += 1
            return True

        def prefetch(need=None):
            while nxt[0] < L and free[0] > 0:
                j = nxt[0]
                prm = self.layers[j]
                if prm.part_jobs:
                    if not load_parts(j, prm, need):
                        return
                    slots[j] = part["slot"]
                else:
                    job = prm.job
                    if job is not None and not job.done.is_set():
                        if need != j:
                            return
                        self._wait_param(prm)
                    slots[j] = self.ring.load(j, prm.shared)
                nxt[0] += 1
                free[0] -= 1

        # layers already updated start uploading while the embedding's chunks are still being
        # updated; the gather waits for every chunk's upload
        prefetch()
        for ci in range(self.emb_nch):
            self._wait_job(self.emb_job[ci])
            prefetch()
        self._embed_catch_up()
        B.slide_embed_fwd(self.embed.dev, self.tok_in, self._x(0), N, H, V, self.code, c)
        if self.embed_split:
            pres = np.unique(np.asarray(tok[:, :-1])).astype(np.int32)
            self.emb_present = pres
            self.emb_rows_host[:len(pres)].copy_(torch.from_numpy(pres))
            with torch.cuda.stream(c):
                self.emb_rows_dev[:len(pres)].copy_(self.emb_rows_host[:len(pres)],
                                                    non_blocking=True)
            self._update_embed_zero_rows(rec)
        for i in range(L):
            if i not in slots:
                prefetch(need=i)
            s = slots.pop(i)
            w, _ = self.ring.acquire(s, c)
            if host_x and i + 1 >= K:          # the output overwrites input i + 1 - K: copied?
                c.wait_event(self.x_d2h_ev[i + 1 - K])
            e_a = self._ev(c) if self.timeline else None
            if self.save_activations:
                B.slide_layer_fwd_save(self.cfg, w, self._x(i), self._x(i + 1), self.B, self.S,
                                       self.saved[i], self.saved_bytes, c)
            else:
                B.slide_layer_fwd(self.cfg, w, self._x(i), self._x(i + 1), self.B, self.S,
                                  self.ws, self.ws_bytes, c)
            if self.timeline:
                rec["layers"].setdefault(i, {})["fwd"] = (e_a, self._ev(c))
            if host_x and i <= L - K:          # inputs L-K+1 .. L stay in their slots
                self._x_offload(i)
            self.ring.release(s, c)
            free[0] += 1
            self._sync()
            prefetch()

        # ---- loss: the fused CE in its phases, chunk by chunk of the LM head
        self._wait_param(self.final)
        c.wait_event(self.final.ready_ev)
        if self.final.flushed_ev is not None:
            c.wait_event(self.final.flushed_ev)
        B.slide_rmsnorm_fwd(self._x(L), self.final.dev, self.hf, None, N, H, spec.rms_eps,
                            self.code, c)
        ce, lm = self.ce_cfg, self.lm
        ce.grad_scale = self.loss_scale if self.fp16 else 0.0
        ce_iv = rec["ce_iv"] = []         # GPU intervals of the CE, without its waits
        for ci in range(self.lm_nch):
            self._wait_job(self.lm_job[ci])       # this chunk's previous update, then its upload
            c.wait_event(self.lm_ready[ci])
            e_a = self._ev(c) if self.timeline else None
            B.slide_lmhead_ce_stats(ce, self.hf, lm.dev, self.tok_tgt, N, ci, self.ws,
                                    self.ws_bytes, c)
            if self.timeline:
                ce_iv.append((e_a, self._ev(c)))
        e_ce = self._ev(c) if self.timeline else None
        B.slide_lmhead_ce_loss(ce, self.tok_tgt, N, self.loss_dev, self.ws, self.ws_bytes, c)
        for ci in range(self.lm_nch):
            if self.lm_flushed[ci] is not None:   # the previous gradient of these rows is out
                c.wait_event(self.lm_flushed[ci])
            B.slide_lmhead_ce_grad(ce, self.hf, lm.dev, self.tok_tgt, N, ci, True, lm.grad,
                                   self.ws, self.ws_bytes, c)
            self._flush_lm_chunk(ci, rec)
        B.slide_lmhead_ce_dh(ce, N, self.dhf, self.ws, self.ws_bytes, c)
        if self.timeline:
            ce_iv.append((e_ce, self._ev(c)))
        B.slide_rmsnorm_bwd(self.dhf, self._x(L), self.final.dev, None, self.grad_x,
                            self.final.grad, N, H, spec.rms_eps, self.code, self.ws,
                            self.ws_bytes, c)
        rec["other_jobs"].append(self._flush_resident(self.final, "w_final", L))
        self._sync()

        # ---- backward: the last n_slots layers are still in their slots; claim them all
        # before the first prefetch so that no load can pick one of their slots
        for i in range(L - 1, L - 1 - self.n_slots, -1):
            slots[i] = self.ring.reuse(i)
        if host_x and L - K >= 0:             # slot of x_L is free after the final norm
            self._x_reload(L - K)
        for i in range(L - 1, -1, -1):
            s = slots.pop(i)
            w, g = self.ring.acquire(s, c)
            if host_x and i <= L - K:
                c.wait_event(self.x_h2d_ev[i])
            e_a = self._ev(c) if self.timeline else None
            if self.save_activations:
                B.slide_layer_bwd_saved(self.cfg, w, self._x(i), self.grad_x, self.grad_x, g,
                                        self.B, self.S, self.saved[i], self.saved_bytes, self.ws,
                                        self.ws_bytes, c)
            else:
                B.slide_layer_bwd(self.cfg, w, self._x(i), self.grad_x, self.grad_x, g, self.B,
                                  self.S, self.ws, self.ws_bytes, c)
            if host_x and i - K >= 0:          # slot i % K is free again: input i - K comes back
                self._x_reload(i - K)
            e_b = self._ev(c) if self.timeline else None
            if self.check_finite:
                self._nf_count(g, self.P, f"layer{i}")
                self.d2h.wait_event(self._ev(c))
                with torch.cuda.stream(self.d2h):
                    self._nf_fetch(f"layer{i}")
            if i == 0 and self.l0_parts is not None:
                gh = self.layers[0].grad_host
                tickets = [self.ring.flush_range(s, gh, a * self.ts, (b - a) * self.ts, c)
                           for a, b in self.l0_parts]
            else:
                ticket = self.ring.flush(s, self.layers[i].grad_host, c)
            if self.timeline:
                rec["layers"].setdefault(i, {})["bwd"] = (e_a, e_b)
                if self.copy_engine == "hip":   # else: the landed times of the layer's jobs
                    rec["layers"][i]["d2h_end"] = self._ev(self.d2h)
            if i == 0 and self.l0_parts is not None:
                rec["jobs"].extend(self._submit_parts(self.layers[0], tickets, "layer0", 0))
            else:
                rec["jobs"].append(self._submit(self.layers[i], ticket, f"layer{i}", i))
            self.ring.release(s, c)
            self._sync()
            j = i - self.n_slots
            if j >= 0:
                slots[j] = self.ring.load(j, self.layers[j].shared)

        # ---- embedding gradient
        B.slide_embed_bwd(self.grad_x, self.tok_in, self.embed.grad, N, H, V, self.code,
                          self.ws, self.ws_bytes, c)
        if self.embed_split:
            self._flush_embed_packed(rec)
        else:
            self._flush_embed(rec)
        # the host sleeps until the GPU is done (a blocking event), leaving every core to the
        # CPU optimizer instead of spinning on one
        e_end = torch.cuda.Event(enable_timing=True, blocking=True)
        e_end.record(c)
        e_end.synchronize()
        rec["ev0"], rec["ev_end"] = ev0, e_end
        rec["host_gpu_done"] = time.perf_counter()
        if self.fp16:
            self._loss_scale_check(rec)
        else:
            self.opt_step += 1
        self._sync()
        self.records.append(rec)
        return rec

    def _loss_scale_check(self, rec):
        """fp16: once the step's gradients are complete, release its CPU updates if every
        gradient is finite, or skip the whole step: cancel the updates (none has started: they
        wait for this release), put the fp32 masters' 16-bit copies back into the upload buffers
        (where the gradients landed) and halve the loss scale."""
        bad = int(self.nf_dev.cpu().sum())
        rec["loss_scale"], rec["nonfinite"] = self.loss_scale, bad
        jobs = rec["jobs"] + rec["other_jobs"]
        if bad:
            for j in jobs:
                j.cancelled = True
        with self.jobs_cv:
            self.opened_step = self.step_count
            self.jobs_cv.notify_all()
        if not bad:
            self.opt_step += 1
            self.good_steps += 1
            if self.good_steps >= self.scale_growth_interval:
                self.loss_scale *= 2.0
                self.good_steps = 0
            return
        for j in jobs:
            j.done.wait()
        self.emb_scatter_n = 0           # the device still holds every current row
        self.d2h.synchronize()           # every gradient copy has landed
        for prm in self.layers + [self.embed, self.final, self.lm]:
            self._refresh_shared(prm)
        self.loss_scale = max(self.loss_scale * 0.5, self.min_loss_scale)
        self.good_steps = 0
        self.skipped_steps += 1

    def loss(self):
        return float(self.loss_dev.item())

    # ------------------------------------------------------------------ timeline analysis
    def timeline_of(self, recs):
        """Intervals of consecutive recorded steps (timeline=True), in ms from the first one's
        start: GPU layer forwards ("F"), backwards ("B") and CE phases ("C"); the layers'
        gradient D2H copies ("#"); and the CPU updates ("u" layer, "e" embedding, "l" LM head,
        "f" final gain), each under the step that produced its gradient -- the pages' timeline
        figures (paper page, figures 3 and 5) for this build."""
        if isinstance(recs, dict):
            recs = [recs]
        origin = recs[0]["host_t0"]
        gpu, d2h, cpu = [], [], []
        kind = {"layer": "u", "embed": "e", "lm_head": "l", "w_final": "f"}
        for rec in recs:
            for j in rec["jobs"] + rec["other_jobs"]:
                j.done.wait()
            ev0, shift = rec["ev0"], (rec["host_t0"] - origin) * 1e3
            gms = lambda e, ev0=ev0, shift=shift: shift + ev0.elapsed_time(e)
            for i, lr in sorted(rec["layers"].items()):
                for key, ch in (("fwd", "F"), ("bwd", "B")):
                    if key in lr:
                        gpu.append((ch, f"step{rec['step']} layer{i} {key}", gms(lr[key][0]),
                                    gms(lr[key][1])))
            for a, b in rec.get("ce_iv", []):
                gpu.append(("C", f"step{rec['step']} lm-head CE", gms(a), gms(b)))
            prev = -1e30
            for i in range(self.L - 1, -1, -1):
                lr = rec["layers"].get(i, {})
                landed = self._landed_at(rec, i)
                if "bwd" in lr and ("d2h_end" in lr or landed is not None):
                    end = gms(lr["d2h_end"]) if landed is None else (landed - origin) * 1e3
                    start = max(gms(lr["bwd"][1]), prev)
                    prev = end
                    d2h.append(("#", f"step{rec['step']} layer{i} grads", start, end))
            for j in rec["jobs"] + rec["other_jobs"]:
                if j.t_end > j.t_start:
                    ch = next((v for k, v in kind.items() if j.name.startswith(k)), "?")
                    cpu.append((ch, f"step{rec['step']} {j.name}", (j.t_start - origin) * 1e3,
                                (j.t_end - origin) * 1e3))
        return dict(gpu=gpu, d2h=d2h, cpu=cpu)

    @staticmethod
    def render_timeline(tl, ms_per_col=10.0, t_end=None, t_start=0.0):
        """Three text lanes (GPU, D2H, CPU) of a timeline_of(), one column per ms_per_col: each
        column shows the activity that covers at least half of it, ':' when activities cover
        10-50% of it, '.' when idle."""
        lanes = (("GPU", tl["gpu"]), ("D2H", tl["d2h"]), ("CPU", tl["cpu"]))
        end = t_end or max((iv[3] for _, ivs in lanes for iv in ivs), default=0.0)
        ncol = max(1, int((end - t_start) / ms_per_col + 0.999))
        out = []
        for name, ivs in lanes:
            row = []
            for c in range(ncol):
                lo, hi = t_start + c * ms_per_col, t_start + (c + 1) * ms_per_col
                cover = {}
                for ch, _, a, b in ivs:
                    ov = min(b, hi) - max(a, lo)
                    if ov > 0:
                        cover[ch] = cover.get(ch, 0.0) + ov
                best = max(cover.items(), key=lambda kv: kv[1]) if cover else None
                busy = sum(cover.values())
                row.append(best[0] if best and best[1] >= 0.5 * ms_per_col
                           else ":" if busy >= 0.1 * ms_per_col else ".")
            out.append(f"{name} |{''.join(row)}|")
        return "\n".join(out)

    def export_trace(self, recs, path):
        """Chrome trace-event JSON (chrome://tracing, Perfetto) of recorded steps."""
        events = []
        tl = self.timeline_of(recs)
        for tid, lane in ((1, "gpu"), (2, "d2h"), (3, "cpu")):
            for _, name, a, b in tl[lane]:
                events.append(dict(name=name, ph="X", pid=0, tid=tid, ts=a * 1e3,
                                   dur=max(0.0, (b - a) * 1e3)))
        with open(path, "w") as f:
            json.dump({"traceEvents": events}, f)

    @staticmethod
    def _boundary_gaps(recs):
        """Median GPU time between the end of a step's backward and the start of the next step's
        layer-0 forward (the iteration-boundary bubble: the next forward needs the embedding and
        layer 0 first, and they are the last to get their gradients), over consecutive records;
        None with fewer than two."""
        gaps = []
        for a, b in zip(recs[:-1], recs[1:]):
            f0 = b["layers"].get(0, {}).get("fwd")
            if b["step"] == a["step"] + 1 and f0 is not None:
                gaps.append(a["ev_end"].elapsed_time(f0[0]))
        return float(np.median(gaps)) if gaps else None

    def _landed_at(self, rec, i):
        """Host time at which layer i's gradient copies of this step had all landed, from the
        copy threads' clocks (copy_engine "hsa"); None where GPU events time the copies."""
        if self.copy_engine != "hsa":
            return None
        ts = [j.t_landed for j in rec["jobs"] if j.name == f"layer{i}"]
        return max(ts) if ts and all(t is not None for t in ts) else None

    def analyse(self, recs):
        """Timeline of recorded steps (timeline=True): per-layer backward, gradient D2H and CPU
        update times; the pages' per-layer overlap predicate T_bwd >= T_d2h + T_update (figure 4
        caption of the paper page), checked as: the update of layer i is hidden by the backward
        of layer i-1; and the share of the D2H + update work that ran while the GPU was busy with
        layer or loss kernels (of the same step or the next one)."""
        if isinstance(recs, dict):
            recs = [recs]
        L = self.L
        gpu_iv, work_iv, per_layer = [], [], []
        cpu_all = 0.0
        for rec in recs:
            for j in rec["jobs"] + rec["other_jobs"]:
                j.done.wait()
            cpu_all += sum(j.t_end - j.t_start for j in rec["jobs"] + rec["other_jobs"])
            ev0, t0 = rec["ev0"], rec["host_t0"]
            to_host = lambda e: t0 + ev0.elapsed_time(e) / 1e3
            for i, lr in rec["layers"].items():
                for key in ("fwd", "bwd"):
                    if key in lr:
                        gpu_iv.append((to_host(lr[key][0]), to_host(lr[key][1])))
            for a, b in rec.get("ce_iv", []):
                gpu_iv.append((to_host(a), to_host(b)))
            jobs = {}
            for j in rec["jobs"]:
                jobs.setdefault(j.name, []).append(j)
            prev_end = -1e30
            for i in range(L - 1, -1, -1):
                lr = rec["layers"][i]
                bs, be = to_host(lr["bwd"][0]), to_host(lr["bwd"][1])
                landed = self._landed_at(rec, i)
                d_end = to_host(lr["d2h_end"]) if landed is None else landed
                d_start = max(be, prev_end)   # the copy starts after its backward and the
                prev_end = d_end              # previous copy on the D2H stream
                parts = jobs[f"layer{i}"]
                work_iv.append((d_start, d_end))
                work_iv.extend((j.t_start, j.t_end) for j in parts)
                fw = lr.get("fwd")
                t_fwd = fw[0].elapsed_time(fw[1]) if fw is not None else None
                per_layer.append(dict(step=rec["step"], layer=i, t_fwd_ms=t_fwd,
                                      t_bwd_ms=(be - bs) * 1e3,
                                      t_d2h_ms=max(0.0, d_end - d_start) * 1e3,
                                      t_update_ms=sum(j.t_end - j.t_start for j in parts) * 1e3))
        # merge GPU intervals
        gpu_iv.sort()
        merged = []
        for a, b in gpu_iv:
            if merged and a <= merged[-1][1]:
                merged[-1][1] = max(merged[-1][1], b)
            else:
                merged.append([a, b])

        def covered(iv):
            tot = 0.0
            for a, b in merged:
                lo, hi = max(iv[0], a), min(iv[1], b)
                if hi > lo:
                    tot += hi - lo
            return tot

        work = sum(b - a for a, b in work_iv)
        hid = sum(covered(iv) for iv in work_iv)
        by = {(li["step"], li["layer"]): li for li in per_layer}
        met = 0
        for li in per_layer:
            nxt = by.get((li["step"], li["layer"] - 1))
            if nxt is not None and nxt["t_bwd_ms"] >= li["t_d2h_ms"] + li["t_update_ms"]:
                met += 1
        n = max(len(recs), 1)
        return dict(
            overlap_pct=100.0 * hid / work if work > 0 else 100.0,
            t_bwd_total_ms=sum(li["t_bwd_ms"] for li in per_layer) / n,
            t_update_total_ms=sum(li["t_update_ms"] for li in per_layer) / n,
            t_d2h_total_ms=sum(li["t_d2h_ms"] for li in per_layer) / n,
            predicate_layers_met=met / n,
            gpu_ms=sum(r["ev0"].elapsed_time(r["ev_end"]) for r in recs) / n,
            t_update_all_ms=cpu_all * 1e3 / n,
            boundary_ms=self._boundary_gaps(recs),
            layers=per_layer)
