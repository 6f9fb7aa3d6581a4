"""Thin Python binding of libslide with the C ABI's names (include/slide.h).

Argument marshalling only: tensors are passed by address (torch tensors, or plain integers
holding an address), streams as torch streams or raw hipStream_t integers. Every computation
runs in libslide's kernels; a non-zero status raises SlideError carrying slide_last_error().
"""
import ctypes

from ._capi import (AdamWHp, CeCfg, LayerCfg, SlideError, call, lib, SLIDE_BF16, SLIDE_F16,
                    SLIDE_F32, SLIDE_ENGINE_HIP, SLIDE_ENGINE_HOST, SLIDE_ENGINE_HSA,
                    SLIDE_TIER_DIRECT,
                    SLIDE_TIER_UNLINK)

__all__ = [
    "LayerCfg", "CeCfg", "AdamWHp", "SlideError", "SLIDE_BF16", "SLIDE_F16", "SLIDE_F32",
    "SLIDE_ENGINE_HIP", "SLIDE_ENGINE_HSA",
    "SLIDE_ENGINE_HOST", "slide_layer_param_count", "slide_layer_param_offsets",
    "slide_layer_workspace_bytes", "slide_layer_fwd", "slide_layer_bwd",
    "slide_layer_saved_bytes", "slide_layer_fwd_save", "slide_layer_bwd_saved",
    "slide_lmhead_ce_workspace_bytes", "slide_lmhead_ce", "slide_lmhead_ce_n_chunks",
    "slide_lmhead_ce_stats", "slide_lmhead_ce_loss", "slide_lmhead_ce_grad", "slide_lmhead_ce_dh",
    "slide_embed_fwd",
    "slide_embed_bwd_workspace_bytes", "slide_embed_bwd", "slide_rmsnorm_fwd",
    "slide_rmsnorm_bwd_workspace_bytes", "slide_rmsnorm_bwd", "slide_rmsnorm_bwd_noalloc",
    "slide_rmsnorm_bwd_noalloc_max_bytes", "slide_gemm", "slide_gemm_tail_workspace_bytes",
    "slide_gemm_ws", "slide_swiglu_fwd", "slide_swiglu_bwd",
    "slide_gemm_swiglu_fwd", "slide_gemm_swiglu_bwd_workspace_bytes", "slide_gemm_swiglu_bwd",
    "slide_attention_fwd", "slide_attention_bwd_workspace_bytes", "slide_attention_bwd",
    "slide_rope", "SlotRing", "slide_cpu_adamw", "slide_cpu_adamw_rows",
    "slide_cpu_adamw_rows_packed", "slide_copy_rows", "slide_gpu_adamw", "slide_convert_f32",
    "slide_host_link_engine_rates",
    "slide_cpu_convert_f32", "slide_host_triad", "StateTier",
    "slide_tier_region_bytes",
    "slide_nonfinite_count",
    "SLIDE_TIER_DIRECT", "SLIDE_TIER_UNLINK", "slide_prof_enable", "slide_prof_reset",
    "slide_prof_read", "dtype_code", "layer_cfg",
]


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if hasattr(t, "data_ptr"):
        return ctypes.c_void_p(t.data_ptr())
    if hasattr(t, "ctypes"):           # numpy array
        return ctypes.c_void_p(t.ctypes.data)
    raise TypeError(f"cannot pass {type(t)} as a pointer")


def _s(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(dt):
    """'bf16' / 'f16' / 'f32' / torch dtype -> SLIDE_BF16 / SLIDE_F16 / SLIDE_F32."""
    s = str(dt)
    if "bf16" in s or "bfloat16" in s:
        return SLIDE_BF16
    if s in ("f16", "torch.float16", "float16"):
        return SLIDE_F16
    if "f32" in s or "float32" in s:
        return SLIDE_F32
    raise ValueError(f"unsupported dtype {dt}")


def layer_cfg(hidden, n_heads, n_kv_heads, head_dim, ffn, dtype, rms_eps=1e-5,
              rope_theta=10000.0):
    return LayerCfg(hidden, n_heads, n_kv_heads, head_dim, ffn, dtype_code(dtype), rms_eps,
                    rope_theta)


# ------------------------------------------------------------------------------ layer
def slide_layer_param_count(cfg):
    return int(lib().slide_layer_param_count(ctypes.byref(cfg)))


def slide_layer_param_offsets(cfg):
    off = (ctypes.c_size_t * 6)()
    call("slide_layer_param_offsets", ctypes.byref(cfg), off)
    return list(off)


def slide_layer_workspace_bytes(cfg, B, S, bwd):
    return int(lib().slide_layer_workspace_bytes(ctypes.byref(cfg), B, S, int(bwd)))


def slide_layer_fwd(cfg, w_slot, x, y, B, S, ws, ws_bytes, stream=None):
    call("slide_layer_fwd", ctypes.byref(cfg), _p(w_slot), _p(x), _p(y), B, S, _p(ws),
         ws_bytes, _s(stream))


def slide_layer_bwd(cfg, w_slot, x, dy, dx, g_slot, B, S, ws, ws_bytes, stream=None):
    call("slide_layer_bwd", ctypes.byref(cfg), _p(w_slot), _p(x), _p(dy), _p(dx), _p(g_slot),
         B, S, _p(ws), ws_bytes, _s(stream))


def slide_layer_saved_bytes(cfg, B, S):
    return int(lib().slide_layer_saved_bytes(ctypes.byref(cfg), B, S))


def slide_layer_fwd_save(cfg, w_slot, x, y, B, S, saved, saved_bytes, stream=None):
    call("slide_layer_fwd_save", ctypes.byref(cfg), _p(w_slot), _p(x), _p(y), B, S, _p(saved),
         saved_bytes, _s(stream))


def slide_layer_bwd_saved(cfg, w_slot, x, dy, dx, g_slot, B, S, saved, saved_bytes, ws,
                          ws_bytes, stream=None):
    call("slide_layer_bwd_saved", ctypes.byref(cfg), _p(w_slot), _p(x), _p(dy), _p(dx),
         _p(g_slot), B, S, _p(saved), saved_bytes, _p(ws), ws_bytes, _s(stream))


# ------------------------------------------------------------------------------ LM head CE
def slide_lmhead_ce_workspace_bytes(cfg, N):
    return int(lib().slide_lmhead_ce_workspace_bytes(ctypes.byref(cfg), N))


def slide_lmhead_ce(cfg, h, w, targets, N, loss_dev, dh, dw, ws, ws_bytes, stream=None):
    call("slide_lmhead_ce", ctypes.byref(cfg), _p(h), _p(w), _p(targets), N, _p(loss_dev),
         _p(dh), _p(dw), _p(ws), ws_bytes, _s(stream))


def slide_lmhead_ce_n_chunks(cfg):
    n = int(lib().slide_lmhead_ce_n_chunks(ctypes.byref(cfg)))
    if n < 1:
        raise SlideError(n, "slide_lmhead_ce_n_chunks",
                         lib().slide_last_error().decode(errors="replace"))
    return n


def slide_lmhead_ce_stats(cfg, h, w, targets, N, chunk, ws, ws_bytes, stream=None):
    call("slide_lmhead_ce_stats", ctypes.byref(cfg), _p(h), _p(w), _p(targets), N, chunk, _p(ws),
         ws_bytes, _s(stream))


def slide_lmhead_ce_loss(cfg, targets, N, loss_dev, ws, ws_bytes, stream=None):
    call("slide_lmhead_ce_loss", ctypes.byref(cfg), _p(targets), N, _p(loss_dev), _p(ws),
         ws_bytes, _s(stream))


def slide_lmhead_ce_grad(cfg, h, w, targets, N, chunk, with_dh, dw, ws, ws_bytes, stream=None):
    call("slide_lmhead_ce_grad", ctypes.byref(cfg), _p(h), _p(w), _p(targets), N, chunk,
         int(with_dh), _p(dw), _p(ws), ws_bytes, _s(stream))


def slide_lmhead_ce_dh(cfg, N, dh, ws, ws_bytes, stream=None):
    call("slide_lmhead_ce_dh", ctypes.byref(cfg), N, _p(dh), _p(ws), ws_bytes, _s(stream))


# ------------------------------------------------------------------------------ glue
def slide_embed_fwd(E, tokens, x, N, H, V, dtype, stream=None):
    call("slide_embed_fwd", _p(E), _p(tokens), _p(x), N, H, V, dtype, _s(stream))


def slide_embed_bwd_workspace_bytes(N, V):
    return int(lib().slide_embed_bwd_workspace_bytes(N, V))


def slide_embed_bwd(dx, tokens, dE, N, H, V, dtype, ws, ws_bytes, stream=None):
    call("slide_embed_bwd", _p(dx), _p(tokens), _p(dE), N, H, V, dtype, _p(ws), ws_bytes,
         _s(stream))


def slide_copy_rows(src, src_rows, src_n_rows, dst, dst_rows, dst_n_rows, n_rows, row_bytes,
                    stream=None):
    """Row gather / scatter on the device (src_rows / dst_rows: int32 device lists or None)."""
    call("slide_copy_rows", _p(src), _p(src_rows), src_n_rows, _p(dst), _p(dst_rows),
         dst_n_rows, n_rows, row_bytes, _s(stream))


def slide_rmsnorm_fwd(x, w, y, rstd, N, H, eps, dtype, stream=None):
    call("slide_rmsnorm_fwd", _p(x), _p(w), _p(y), _p(rstd), N, H, ctypes.c_float(eps), dtype,
         _s(stream))


def slide_rmsnorm_bwd_workspace_bytes(N, H):
    return int(lib().slide_rmsnorm_bwd_workspace_bytes(N, H))


def slide_rmsnorm_bwd(dy, x, w, dres, dx, dw, N, H, eps, dtype, ws, ws_bytes, stream=None):
    call("slide_rmsnorm_bwd", _p(dy), _p(x), _p(w), _p(dres), _p(dx), _p(dw), N, H,
         ctypes.c_float(eps), dtype, _p(ws), ws_bytes, _s(stream))


def slide_rmsnorm_bwd_noalloc_max_bytes():
    return int(lib().slide_rmsnorm_bwd_noalloc_max_bytes())


def slide_rmsnorm_bwd_noalloc(dy, x, w, dres, dx, dw, N, H, eps, dtype, stream=None):
    call("slide_rmsnorm_bwd_noalloc", _p(dy), _p(x), _p(w), _p(dres), _p(dx), _p(dw), N, H,
         ctypes.c_float(eps), dtype, _s(stream))


# ------------------------------------------------------------------------------ kernels
def slide_gemm(M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, C, ldc, c_dtype, R=None, ldr=0,
               alpha=1.0, accumulate=False, dtype=SLIDE_BF16, stream=None):
    call("slide_gemm", M, N, K, _p(A), lda, int(a_kmajor), _p(B), ldb, int(b_kmajor), _p(C), ldc,
         c_dtype, _p(R), ldr, ctypes.c_float(alpha), int(accumulate), dtype, _s(stream))


def slide_gemm_tail_workspace_bytes():
    return int(lib().slide_gemm_tail_workspace_bytes())


def slide_gemm_ws(M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, C, ldc, c_dtype, R=None, ldr=0,
                  alpha=1.0, accumulate=False, dtype=SLIDE_BF16, ws=None, ws_bytes=0,
                  stream=None):
    call("slide_gemm_ws", M, N, K, _p(A), lda, int(a_kmajor), _p(B), ldb, int(b_kmajor), _p(C),
         ldc, c_dtype, _p(R), ldr, ctypes.c_float(alpha), int(accumulate), dtype, _p(ws),
         ws_bytes, _s(stream))


def slide_swiglu_fwd(gu, m, N, F, dtype, stream=None):
    call("slide_swiglu_fwd", _p(gu), _p(m), N, F, dtype, _s(stream))


def slide_swiglu_bwd(dm, gu, dgu, N, F, dtype, stream=None):
    call("slide_swiglu_bwd", _p(dm), _p(gu), _p(dgu), N, F, dtype, _s(stream))


def slide_gemm_swiglu_fwd(M, F, K, x, ldx, w_gu, ldw, gu, m, dtype, stream=None):
    call("slide_gemm_swiglu_fwd", M, F, K, _p(x), ldx, _p(w_gu), ldw, _p(gu), _p(m), dtype,
         _s(stream))


def slide_gemm_swiglu_bwd_workspace_bytes(M, F, dtype):
    return int(lib().slide_gemm_swiglu_bwd_workspace_bytes(M, F, dtype))


def slide_gemm_swiglu_bwd(M, F, K, dy, lddy, w_down, ldw, gu, dgu, dtype, ws=None, ws_bytes=0,
                          stream=None):
    call("slide_gemm_swiglu_bwd", M, F, K, _p(dy), lddy, _p(w_down), ldw, _p(gu), _p(dgu), dtype,
         _p(ws), ws_bytes, _s(stream))


def slide_attention_fwd(qkv, o, lse, B, S, nq, nkv, d, dtype, stream=None):
    call("slide_attention_fwd", _p(qkv), _p(o), _p(lse), B, S, nq, nkv, d, dtype, _s(stream))


def slide_attention_bwd_workspace_bytes(B, S, nq):
    return int(lib().slide_attention_bwd_workspace_bytes(B, S, nq))


def slide_attention_bwd(qkv, o, lse, d_o, dqkv, B, S, nq, nkv, d, dtype, ws, ws_bytes,
                        stream=None):
    call("slide_attention_bwd", _p(qkv), _p(o), _p(lse), _p(d_o), _p(dqkv), B, S, nq, nkv, d,
         dtype, _p(ws), ws_bytes, _s(stream))


def slide_rope(qkv, B, S, nq, nkv, d, theta, inverse, dtype, ws, ws_bytes, stream=None):
    call("slide_rope", _p(qkv), B, S, nq, nkv, d, ctypes.c_float(theta), int(inverse), dtype,
         _p(ws), ws_bytes, _s(stream))


# ------------------------------------------------------------------------------ slot ring
class SlotRing:
    """Handle around slide_slot_ring_*: the fixed queue of identical HBM slots."""

    def __init__(self, n_slots, w_bytes, g_bytes, dev_base, h2d_stream=None, d2h_stream=None,
                 engine=SLIDE_ENGINE_HIP):
        self._h = ctypes.c_void_p()
        call("slide_slot_ring_create", ctypes.byref(self._h), n_slots, w_bytes, g_bytes,
             _p(dev_base), _s(h2d_stream), _s(d2h_stream), engine)

    def load(self, layer, host_w):
        s = ctypes.c_int()
        call("slide_slot_ring_load", self._h, layer, _p(host_w), ctypes.byref(s))
        return s.value

    def load_range(self, layer, host_w, offset, nbytes, slot=-1):
        """Part [offset, offset + nbytes) of a layer's weights; slot -1 starts the load on the
        next FREE slot, a slot number continues it. Returns the slot."""
        s = ctypes.c_int(slot)
        call("slide_slot_ring_load_range", self._h, layer, _p(host_w), offset, nbytes,
             ctypes.byref(s))
        return s.value

    def reuse(self, layer):
        s = ctypes.c_int()
        call("slide_slot_ring_reuse", self._h, layer, ctypes.byref(s))
        return s.value

    def acquire(self, slot, compute_stream=None):
        w = ctypes.c_void_p()
        g = ctypes.c_void_p()
        call("slide_slot_ring_acquire", self._h, slot, _s(compute_stream), ctypes.byref(w),
             ctypes.byref(g))
        return w.value, g.value

    def flush(self, slot, host_g, compute_stream=None):
        t = ctypes.c_uint64()
        call("slide_slot_ring_flush", self._h, slot, _p(host_g), _s(compute_stream),
             ctypes.byref(t))
        return t.value

    def flush_range(self, slot, host_g, offset, nbytes, compute_stream=None):
        t = ctypes.c_uint64()
        call("slide_slot_ring_flush_range", self._h, slot, _p(host_g), offset, nbytes,
             _s(compute_stream), ctypes.byref(t))
        return t.value

    def wait_flush(self, ticket, timeout_ms=-1):
        call("slide_slot_ring_wait_flush", self._h, ctypes.c_uint64(ticket), timeout_ms)

    def release(self, slot, compute_stream=None):
        call("slide_slot_ring_release", self._h, slot, _s(compute_stream))

    def ticket_time(self, ticket):
        """Host time (time.perf_counter's clock) at which a flush landed (host-timed engines)."""
        t = ctypes.c_double()
        call("slide_slot_ring_ticket_time", self._h, ctypes.c_uint64(ticket), ctypes.byref(t))
        return t.value

    def state(self, slot):
        st = ctypes.c_int()
        ly = ctypes.c_int()
        call("slide_slot_ring_state", self._h, slot, ctypes.byref(st), ctypes.byref(ly))
        return st.value, ly.value

    def find(self, layer):
        s = ctypes.c_int()
        call("slide_slot_ring_find", self._h, layer, ctypes.byref(s))
        return s.value

    def inject_fault(self, mode, count):
        call("slide_slot_ring_inject_fault", self._h, mode, count)

    def close(self):
        if self._h:
            call("slide_slot_ring_destroy", self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------------ AdamW
def slide_cpu_adamw(p, g, g_dtype, m, v, p_bf16_out, n, step, hp, n_threads=0):
    """p, m, v: float32 host buffers; g: host bf16 (uint16) or float32; hp: AdamWHp."""
    call("slide_cpu_adamw", _p(p), _p(g), g_dtype, _p(m), _p(v), _p(p_bf16_out), n, step,
         ctypes.byref(hp), n_threads)


def slide_cpu_adamw_rows(p, g, g_dtype, m, v, p_bf16_out, row_len, n_rows_total, rows, n_rows,
                         step, hp, n_threads=0):
    """Rows of row_len elements (int32 row indices); g None: zero gradient on those rows."""
    call("slide_cpu_adamw_rows", _p(p), _p(g), g_dtype, _p(m), _p(v), _p(p_bf16_out), row_len,
         n_rows_total, _p(rows), n_rows, step, ctypes.byref(hp), n_threads)


def slide_cpu_adamw_rows_packed(p, m, v, row_len, n_rows_total, rows, n_rows, g_packed, g_dtype,
                                out_full, out_packed, step, hp, n_threads=0):
    """Rows rows[k] updated from packed gradient rows k; new rows to out_full / out_packed."""
    call("slide_cpu_adamw_rows_packed", _p(p), _p(m), _p(v), row_len, n_rows_total, _p(rows),
         n_rows, _p(g_packed), g_dtype, _p(out_full), _p(out_packed), step, ctypes.byref(hp),
         n_threads)


def slide_gpu_adamw(p, g, g_dtype, m, v, p_bf16_out, n, step, hp, stream=None):
    """p, m, v: float32 device tensors; g: device bf16 or float32; hp: AdamWHp."""
    call("slide_gpu_adamw", _p(p), _p(g), g_dtype, _p(m), _p(v), _p(p_bf16_out), n, step,
         ctypes.byref(hp), _s(stream))


def slide_cpu_convert_f32(src, dst, dst_dtype, n, n_threads=0):
    """fp32 host array -> bf16 / fp16 bit patterns (round to nearest-even)."""
    call("slide_cpu_convert_f32", _p(src), _p(dst), dst_dtype, n, n_threads)


def slide_convert_f32(src, dst, dst_dtype, n, stream=None):
    """fp32 device tensor -> bf16 / fp16 device tensor (round to nearest-even), on stream."""
    call("slide_convert_f32", _p(src), _p(dst), dst_dtype, n, _s(stream))


def slide_host_link_engine_rates(dev, host, nbytes, reps=3):
    """Per copy engine: best time (ms) of an nbytes copy device -> host and host -> device
    between `dev` (device tensor) and `host` (pinned tensor); -1 where absent. Returns
    (d2h_ms[32], h2d_ms[32], (n_host_engines, n_xgmi_engines, pref_d2h_mask, pref_h2d_mask))."""
    d2h, h2d = (ctypes.c_double * 32)(), (ctypes.c_double * 32)()
    info = (ctypes.c_uint32 * 4)()
    call("slide_host_link_engine_rates", _p(dev), _p(host), nbytes, reps, d2h, h2d, info)
    return list(d2h), list(h2d), tuple(info)


def slide_host_triad(n, n_threads=0, reps=3):
    """STREAM-triad host-DRAM bandwidth (GB/s): (best, median) over reps repetitions."""
    best, med = ctypes.c_double(), ctypes.c_double()
    call("slide_host_triad", n, n_threads, reps, ctypes.byref(best), ctypes.byref(med))
    return best.value, med.value


def slide_nonfinite_count(x, dtype, n, count_dev, stream=None):
    """count_dev: a 4-byte device buffer (e.g. an int32 tensor element) that receives the number
    of NaN or infinite elements of x[:n]."""
    call("slide_nonfinite_count", _p(x), dtype, n, _p(count_dev), _s(stream))


# ------------------------------------------------------------------------------ disk tier
def slide_tier_region_bytes(n_floats):
    return lib().slide_tier_region_bytes(n_floats)


class StateTier:
    """Handle of a disk tier of fp32 optimizer state (slide_tier_*). Offsets are bytes, multiples
    of 4096; arrays are host buffers (numpy or CPU torch)."""

    def __init__(self, path, capacity_bytes, chunk_elems=0, io_threads=8,
                 flags=SLIDE_TIER_DIRECT | SLIDE_TIER_UNLINK):
        h = ctypes.c_void_p()
        call("slide_tier_create", ctypes.byref(h), str(path).encode(), capacity_bytes,
             chunk_elems, io_threads, flags)
        self.h = h

    def info(self):
        d, cap, ch = ctypes.c_int(), ctypes.c_uint64(), ctypes.c_size_t()
        call("slide_tier_info", self.h, ctypes.byref(d), ctypes.byref(cap), ctypes.byref(ch))
        return dict(direct=bool(d.value), capacity=cap.value, chunk=ch.value)

    def stats(self):
        r, w = ctypes.c_uint64(), ctypes.c_uint64()
        busy, stall = ctypes.c_double(), ctypes.c_double()
        call("slide_tier_stats", self.h, ctypes.byref(r), ctypes.byref(w), ctypes.byref(busy),
             ctypes.byref(stall))
        return dict(bytes_read=r.value, bytes_written=w.value, busy_s=busy.value,
                    stall_s=stall.value)

    def write(self, off, src, nbytes=None):
        """src: host array, or None to write nbytes of zeros."""
        if nbytes is None:
            nbytes = src.nbytes if hasattr(src, "nbytes") else src.numel() * src.element_size()
        call("slide_tier_write", self.h, off, _p(src), nbytes)

    def read(self, off, dst):
        nbytes = dst.nbytes if hasattr(dst, "nbytes") else dst.numel() * dst.element_size()
        call("slide_tier_read", self.h, off, _p(dst), nbytes)

    def adamw(self, p, p_off, m, m_off, v, v_off, g, g_dtype, p_bf16_out, n, step, hp,
              n_threads=0):
        """p, m, v: a host float32 buffer, or None for the array at the given tier offset."""
        call("slide_tier_adamw", self.h, _p(p), p_off, _p(m), m_off, _p(v), v_off, _p(g), g_dtype,
             _p(p_bf16_out), n, step, ctypes.byref(hp), n_threads)

    def close(self):
        if self.h is not None and self.h.value:
            call("slide_tier_destroy", self.h)
        self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------------ profiler
def slide_prof_enable(on=True):
    call("slide_prof_enable", int(on))


def slide_prof_reset():
    call("slide_prof_reset")


def slide_prof_read(max_entries=256):
    """{kernel name: (launches, total_ms)} since the last reset (synchronizes the events)."""
    names = (ctypes.c_char * 64 * max_entries)()
    counts = (ctypes.c_int64 * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    n = ctypes.c_int()
    call("slide_prof_read", ctypes.cast(names, ctypes.c_void_p), counts, ms, max_entries,
         ctypes.byref(n))
    return {bytes(names[i]).split(b"\0")[0].decode(): (counts[i], ms[i]) for i in range(n.value)}
