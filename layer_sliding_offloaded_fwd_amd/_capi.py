"""ctypes declarations of libslide's C ABI (include/slide.h). Argument marshalling only."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libslide.so")

SLIDE_OK = 0
SLIDE_E_ARG, SLIDE_E_SHAPE, SLIDE_E_WORKSPACE, SLIDE_E_HIP = -1, -2, -3, -4
SLIDE_E_STATE, SLIDE_E_TIMEOUT, SLIDE_E_UNSUPPORTED, SLIDE_E_NONFINITE = -5, -6, -7, -8
SLIDE_E_IO = -9
SLIDE_TIER_DIRECT, SLIDE_TIER_UNLINK = 1, 2
SLIDE_F32, SLIDE_BF16, SLIDE_F16 = 0, 1, 2
SLIDE_ENGINE_HIP, SLIDE_ENGINE_HOST, SLIDE_ENGINE_HSA = 0, 1, 2
SLOT_FREE, SLOT_LOADING, SLOT_IN_USE, SLOT_FLUSHING = 0, 1, 2, 3
ERROR_NAMES = {0: "SLIDE_OK", -1: "SLIDE_E_ARG", -2: "SLIDE_E_SHAPE", -3: "SLIDE_E_WORKSPACE",
               -4: "SLIDE_E_HIP", -5: "SLIDE_E_STATE", -6: "SLIDE_E_TIMEOUT",
               -7: "SLIDE_E_UNSUPPORTED", -8: "SLIDE_E_NONFINITE", -9: "SLIDE_E_IO"}


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class CeCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("grad_scale", ctypes.c_float)]


class AdamWHp(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("grad_scale", ctypes.c_double)]


P = ctypes.c_void_p
I = ctypes.c_int
SZ = ctypes.c_size_t
F = ctypes.c_float
LCP = ctypes.POINTER(LayerCfg)
CCP = ctypes.POINTER(CeCfg)

SIGNATURES = {
    "slide_last_error": (ctypes.c_char_p, []),
    "slide_version": (ctypes.c_char_p, []),
    "slide_layer_param_count": (SZ, [LCP]),
    "slide_layer_param_offsets": (I, [LCP, ctypes.POINTER(SZ)]),
    "slide_layer_workspace_bytes": (SZ, [LCP, I, I, I]),
    "slide_layer_fwd": (I, [LCP, P, P, P, I, I, P, SZ, P]),
    "slide_layer_bwd": (I, [LCP, P, P, P, P, P, I, I, P, SZ, P]),
    "slide_layer_saved_bytes": (SZ, [LCP, I, I]),
    "slide_layer_fwd_save": (I, [LCP, P, P, P, I, I, P, SZ, P]),
    "slide_layer_bwd_saved": (I, [LCP, P, P, P, P, P, I, I, P, SZ, P, SZ, P]),
    "slide_lmhead_ce_workspace_bytes": (SZ, [CCP, I]),
    "slide_lmhead_ce": (I, [CCP, P, P, P, I, P, P, P, P, SZ, P]),
    "slide_lmhead_ce_n_chunks": (I, [CCP]),
    "slide_lmhead_ce_stats": (I, [CCP, P, P, P, I, I, P, SZ, P]),
    "slide_lmhead_ce_loss": (I, [CCP, P, I, P, P, SZ, P]),
    "slide_lmhead_ce_grad": (I, [CCP, P, P, P, I, I, I, P, P, SZ, P]),
    "slide_lmhead_ce_dh": (I, [CCP, I, P, P, SZ, P]),
    "slide_embed_fwd": (I, [P, P, P, I, I, I, I, P]),
    "slide_embed_bwd_workspace_bytes": (SZ, [I, I]),
    "slide_embed_bwd": (I, [P, P, P, I, I, I, I, P, SZ, P]),
    "slide_copy_rows": (I, [P, P, ctypes.c_int64, P, P, ctypes.c_int64, ctypes.c_int64, SZ, P]),
    "slide_rmsnorm_fwd": (I, [P, P, P, P, I, I, F, I, P]),
    "slide_rmsnorm_bwd_workspace_bytes": (SZ, [I, I]),
    "slide_rmsnorm_bwd": (I, [P, P, P, P, P, P, I, I, F, I, P, SZ, P]),
    "slide_rmsnorm_bwd_noalloc_max_bytes": (SZ, []),
    "slide_rmsnorm_bwd_noalloc": (I, [P, P, P, P, P, P, I, I, F, I, P]),
    "slide_gemm": (I, [I, I, I, P, I, I, P, I, I, P, I, I, P, I, F, I, I, P]),
    "slide_gemm_tail_workspace_bytes": (SZ, []),
    "slide_gemm_ws": (I, [I, I, I, P, I, I, P, I, I, P, I, I, P, I, F, I, I, P, SZ, P]),
    "slide_swiglu_fwd": (I, [P, P, I, I, I, P]),
    "slide_swiglu_bwd": (I, [P, P, P, I, I, I, P]),
    "slide_gemm_swiglu_fwd": (I, [I, I, I, P, I, P, I, P, P, I, P]),
    "slide_gemm_swiglu_bwd_workspace_bytes": (SZ, [I, I, I]),
    "slide_gemm_swiglu_bwd": (I, [I, I, I, P, I, P, I, P, P, I, P, SZ, P]),
    "slide_attention_fwd": (I, [P, P, P, I, I, I, I, I, I, P]),
    "slide_attention_bwd_workspace_bytes": (SZ, [I, I, I]),
    "slide_attention_bwd": (I, [P, P, P, P, P, I, I, I, I, I, I, P, SZ, P]),
    "slide_rope": (I, [P, I, I, I, I, I, F, I, I, P, SZ, P]),
    "slide_slot_ring_create": (I, [ctypes.POINTER(P), I, SZ, SZ, P, P, P, I]),
    "slide_slot_ring_load": (I, [P, I, P, ctypes.POINTER(I)]),
    "slide_slot_ring_load_range": (I, [P, I, P, SZ, SZ, ctypes.POINTER(I)]),
    "slide_slot_ring_reuse": (I, [P, I, ctypes.POINTER(I)]),
    "slide_slot_ring_acquire": (I, [P, I, P, ctypes.POINTER(P), ctypes.POINTER(P)]),
    "slide_slot_ring_flush": (I, [P, I, P, P, ctypes.POINTER(ctypes.c_uint64)]),
    "slide_slot_ring_flush_range": (I, [P, I, P, SZ, SZ, P, ctypes.POINTER(ctypes.c_uint64)]),
    "slide_slot_ring_wait_flush": (I, [P, ctypes.c_uint64, I]),
    "slide_slot_ring_release": (I, [P, I, P]),
    "slide_slot_ring_state": (I, [P, I, ctypes.POINTER(I), ctypes.POINTER(I)]),
    "slide_slot_ring_find": (I, [P, I, ctypes.POINTER(I)]),
    "slide_slot_ring_destroy": (I, [P]),
    "slide_slot_ring_ticket_time": (I, [P, ctypes.c_uint64, ctypes.POINTER(ctypes.c_double)]),
    "slide_slot_ring_inject_fault": (I, [P, I, I]),
    "slide_cpu_adamw": (I, [P, P, I, P, P, P, SZ, ctypes.c_int64, ctypes.POINTER(AdamWHp), I]),
    "slide_cpu_adamw_scalar_for_test": (I, [P, P, I, P, P, P, SZ, ctypes.c_int64,
                                            ctypes.POINTER(AdamWHp)]),
    "slide_cpu_adamw_rows_packed": (I, [P, P, P, SZ, SZ, P, SZ, P, I, P, P, ctypes.c_int64,
                                        ctypes.POINTER(AdamWHp), I]),
    "slide_cpu_adamw_rows": (I, [P, P, I, P, P, P, SZ, SZ, P, SZ, ctypes.c_int64,
                                 ctypes.POINTER(AdamWHp), I]),
    "slide_gpu_adamw": (I, [P, P, I, P, P, P, SZ, ctypes.c_int64, ctypes.POINTER(AdamWHp), P]),
    "slide_cpu_convert_f32": (I, [P, P, I, SZ, I]),
    "slide_host_link_engine_rates": (I, [P, P, SZ, I, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_uint32)]),
    "slide_convert_f32": (I, [P, P, I, SZ, P]),
    "slide_host_triad": (I, [SZ, I, I, ctypes.POINTER(ctypes.c_double),
                             ctypes.POINTER(ctypes.c_double)]),
    "slide_nonfinite_count": (I, [P, I, SZ, P, P]),
    "slide_tier_region_bytes": (SZ, [SZ]),
    "slide_tier_create": (I, [ctypes.POINTER(P), ctypes.c_char_p, ctypes.c_uint64, SZ, I, I]),
    "slide_tier_destroy": (I, [P]),
    "slide_tier_info": (I, [P, ctypes.POINTER(I), ctypes.POINTER(ctypes.c_uint64),
                            ctypes.POINTER(SZ)]),
    "slide_tier_stats": (I, [P, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64),
                             ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    "slide_tier_write": (I, [P, ctypes.c_uint64, P, SZ]),
    "slide_tier_read": (I, [P, ctypes.c_uint64, P, SZ]),
    "slide_tier_adamw": (I, [P, P, ctypes.c_uint64, P, ctypes.c_uint64, P, ctypes.c_uint64, P, I,
                             P, SZ, ctypes.c_int64, ctypes.POINTER(AdamWHp), I]),
    "slide_prof_enable": (I, [I]),
    "slide_prof_reset": (I, []),
    "slide_prof_read": (I, [P, P, P, I, ctypes.POINTER(I)]),
}

_lib = None


class SlideError(RuntimeError):
    def __init__(self, code, func, message):
        super().__init__(f"{func} -> {ERROR_NAMES.get(code, code)}: {message}")
        self.code = code
        self.func = func


def lib():
    """Load libslide.so (built in-tree). There is no fallback: without the library the
    product path cannot run."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m layer_sliding_offloaded_fwd_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def call(name, *args):
    """Call an int-returning entry point; raise SlideError on a non-zero status."""
    L = lib()
    rc = getattr(L, name)(*args)
    if rc != SLIDE_OK:
        raise SlideError(rc, name, L.slide_last_error().decode(errors="replace"))
    return rc
