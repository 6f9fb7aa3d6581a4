"""Training with every parameter, gradient and optimizer state resident in HBM: the
non-offloaded baseline that the layer-sliding method is measured against (paper page,
abstract: offloaded training keeps over 95% of the performance of training without offloading).

One step runs the same library calls, in the same order, as SlideEngine.step: embedding gather,
the layers' forward keeping their intermediates, final RMSNorm, the fused LM-head CE in its
phases, the final norm's backward, the layers' backward, the embedding's backward. The only
difference is where the optimizer runs: every block's AdamW is slide_gpu_adamw on the compute
stream right after the block's gradient is complete, instead of a gradient flush, a CPU update
and an upload. slide_gpu_adamw has slide_cpu_adamw's operation order, so a resident step equals
an offloaded step bit for bit.

All numerical work runs in libslide; this module only orders calls on one stream.
"""
import numpy as np
import torch

from . import binding as B
from ._capi import SLIDE_BF16, SLIDE_F32
from .engine import AdamW, ModelSpec


class _Block:
    """One parameter block in HBM: compute copy, fp32 master (the compute copy itself for fp32
    compute), AdamW moments and gradient."""

    def __init__(self, n, dtype, device, rows=1):
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        ts = 2 if dtype == "bf16" else 4
        self.n = n

        def alloc(dt, esize):
            if rows == 1:
                return torch.zeros(n, dtype=dt, device=device)
            # each row starts on a 256-byte boundary, as a slot of the offloaded ring does
            stride = -(-n * esize // 256) * 256 // esize
            return torch.zeros((rows, stride), dtype=dt, device=device)[:, :n]

        self.dev = alloc(tdt, ts)
        self.master = alloc(torch.float32, 4) if dtype == "bf16" else self.dev
        self.m = alloc(torch.float32, 4)
        self.v = alloc(torch.float32, 4)


class ResidentTrainer:
    def __init__(self, spec: ModelSpec, batch, seq, ce_chunk=8192, hp=AdamW(),
                 device="cuda:0"):
        assert spec.dtype in ("bf16", "f32")
        self.spec, self.B, self.S, self.N = spec, batch, seq, batch * seq
        self.L = spec.n_layers
        self.device = torch.device(device)
        self.hp = B.AdamWHp(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
        self.code = SLIDE_BF16 if spec.dtype == "bf16" else SLIDE_F32
        self.tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        s = spec
        self.cfg = B.layer_cfg(s.hidden, s.n_heads, s.n_kv_heads, s.head_dim, s.ffn, s.dtype,
                               s.rms_eps, s.rope_theta)
        self.ce_cfg = B.CeCfg(s.hidden, s.vocab, ce_chunk, self.code)
        self.P = B.slide_layer_param_count(self.cfg)
        self.lm_nch = B.slide_lmhead_ce_n_chunks(self.ce_cfg)
        H, V, N, dev = s.hidden, s.vocab, self.N, self.device
        self.compute = torch.cuda.Stream(device=dev)
        self.layers = _Block(self.P, s.dtype, dev, rows=self.L)
        self.embed = _Block(V * H, s.dtype, dev)
        self.final = _Block(H, s.dtype, dev)
        self.lm = _Block(V * H, s.dtype, dev)
        self.g_layer = torch.empty(self.P, dtype=self.tdt, device=dev)
        self.g_embed = torch.empty(V * H, dtype=self.tdt, device=dev)
        self.g_final = torch.empty(H, dtype=self.tdt, device=dev)
        self.g_lm = torch.empty(V * H, dtype=self.tdt, device=dev)
        self.xs = torch.empty((self.L + 1, N, H), dtype=self.tdt, device=dev)
        self.grad_x = torch.empty((N, H), dtype=self.tdt, device=dev)
        self.hf = torch.empty((N, H), dtype=self.tdt, device=dev)
        self.dhf = torch.empty((N, H), dtype=self.tdt, device=dev)
        self.tok_in = torch.empty(N, dtype=torch.int32, device=dev)
        self.tok_tgt = torch.empty(N, dtype=torch.int32, device=dev)
        self.loss_dev = torch.zeros(1, dtype=torch.float32, device=dev)
        self.saved_bytes = (B.slide_layer_saved_bytes(self.cfg, batch, seq) + 255) // 256 * 256
        self.saved = torch.empty((self.L, self.saved_bytes), dtype=torch.uint8, device=dev)
        ws = max(B.slide_layer_workspace_bytes(self.cfg, batch, seq, 2),
                 B.slide_lmhead_ce_workspace_bytes(self.ce_cfg, N),
                 B.slide_embed_bwd_workspace_bytes(N, V),
                 B.slide_rmsnorm_bwd_workspace_bytes(N, H))
        self.ws_bytes = (ws + 255) // 256 * 256
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.step_count = 0

    # ------------------------------------------------------------------ parameters
    def _set(self, blk, t, row=None):
        """fp32 master of a block (or of one layer row) and its compute copy, rounded by the
        library (the offloaded engine rounds its copies with the same rule on the host)."""
        dst_m = blk.master if row is None else blk.master[row]
        dst_m.copy_(t.reshape(dst_m.shape))
        if self.spec.dtype == "bf16":
            dst = blk.dev if row is None else blk.dev[row]
            B.slide_convert_f32(dst_m, dst, self.code, blk.n,
                                torch.cuda.current_stream(self.device))

    def load_params(self, embed, layers, w_final, lm_head):
        """fp32 master weights (numpy or torch; layers in slot packing order); moments and the
        step counter are reset."""
        def t(a):
            return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)
                                   if isinstance(a, np.ndarray) else a).float().to(self.device)
        self._set(self.embed, t(embed))
        self._set(self.final, t(w_final))
        self._set(self.lm, t(lm_head))
        assert len(layers) == self.L
        for i, a in enumerate(layers):
            self._set(self.layers, t(a), row=i)
        self._zero_moments()

    def init_random(self, seed=0, std=0.02):
        """The offloaded engine's seeded synthetic weights (SlideEngine.init_random draws the
        same values: matrices N(0, std) on a torch generator in the same order, norm gains 1)."""
        gen = torch.Generator(device=self.device)
        gen.manual_seed(seed)
        offs = B.slide_layer_param_offsets(self.cfg)
        H = self.spec.hidden

        def draw(n, gains=()):
            x = torch.empty(n, dtype=torch.float32, device=self.device)
            x.normal_(0.0, std, generator=gen)
            for o in gains:
                x[o:o + H] = 1.0
            return x

        self._set(self.embed, draw(self.embed.n))
        for i in range(self.L):
            self._set(self.layers, draw(self.P, gains=(offs[0], offs[3])), row=i)
        self._set(self.final, torch.ones(H, device=self.device))
        self._set(self.lm, draw(self.lm.n))
        self._zero_moments()

    def _zero_moments(self):
        for blk in (self.embed, self.final, self.lm, self.layers):
            blk.m.zero_()
            blk.v.zero_()
        torch.cuda.synchronize(self.device)
        self.step_count = 0

    def master_params(self):
        torch.cuda.synchronize(self.device)
        return dict(embed=self.embed.master.cpu().numpy().copy(),
                    layers=[self.layers.master[i].cpu().numpy().copy() for i in range(self.L)],
                    w_final=self.final.master.cpu().numpy().copy(),
                    lm_head=self.lm.master.cpu().numpy().copy())

    # ------------------------------------------------------------------ step
    def _adam(self, master, g, m, v, dev, n):
        out = dev if self.spec.dtype == "bf16" else None
        B.slide_gpu_adamw(master, g, self.code, m, v, out, n, self.step_count, self.hp,
                          self.compute)

    def step(self, tokens):
        """One training step on int32 tokens [B, S+1] (inputs [:, :S], targets [:, 1:])."""
        spec, N, H, V, L = self.spec, self.N, self.spec.hidden, self.spec.vocab, self.L
        c = self.compute
        tok = torch.as_tensor(np.asarray(tokens, dtype=np.int32))
        assert tok.shape == (self.B, self.S + 1), tok.shape
        self.step_count += 1
        with torch.cuda.stream(c):
            self.tok_in.copy_(tok[:, :-1].reshape(-1), non_blocking=False)
            self.tok_tgt.copy_(tok[:, 1:].reshape(-1), non_blocking=False)
        B.slide_embed_fwd(self.embed.dev, self.tok_in, self.xs[0], N, H, V, self.code, c)
        for i in range(L):
            B.slide_layer_fwd_save(self.cfg, self.layers.dev[i], self.xs[i], self.xs[i + 1],
                                   self.B, self.S, self.saved[i], self.saved_bytes, c)
        B.slide_rmsnorm_fwd(self.xs[L], self.final.dev, self.hf, None, N, H, spec.rms_eps,
                            self.code, c)
        ce, ws, wb = self.ce_cfg, self.ws, self.ws_bytes
        for ci in range(self.lm_nch):
            B.slide_lmhead_ce_stats(ce, self.hf, self.lm.dev, self.tok_tgt, N, ci, ws, wb, c)
        B.slide_lmhead_ce_loss(ce, self.tok_tgt, N, self.loss_dev, ws, wb, c)
        for ci in range(self.lm_nch):
            B.slide_lmhead_ce_grad(ce, self.hf, self.lm.dev, self.tok_tgt, N, ci, True,
                                   self.g_lm, ws, wb, c)
        B.slide_lmhead_ce_dh(ce, N, self.dhf, ws, wb, c)
        B.slide_rmsnorm_bwd(self.dhf, self.xs[L], self.final.dev, None, self.grad_x,
                            self.g_final, N, H, spec.rms_eps, self.code, ws, wb, c)
        self._adam(self.lm.master, self.g_lm, self.lm.m, self.lm.v, self.lm.dev, self.lm.n)
        self._adam(self.final.master, self.g_final, self.final.m, self.final.v, self.final.dev,
                   H)
        lay = self.layers
        for i in range(L - 1, -1, -1):
            B.slide_layer_bwd_saved(self.cfg, lay.dev[i], self.xs[i], self.grad_x, self.grad_x,
                                    self.g_layer, self.B, self.S, self.saved[i],
                                    self.saved_bytes, ws, wb, c)
            self._adam(lay.master[i], self.g_layer, lay.m[i], lay.v[i], lay.dev[i], self.P)
        B.slide_embed_bwd(self.grad_x, self.tok_in, self.g_embed, N, H, V, self.code, ws, wb, c)
        self._adam(self.embed.master, self.g_embed, self.embed.m, self.embed.v, self.embed.dev,
                   self.embed.n)

    def loss(self):
        self.compute.synchronize()
        return float(self.loss_dev.item())

    def synchronize(self):
        self.compute.synchronize()
