// One decoder layer, forward and backward, composed from the GEMM, attention and memory-bound
// kernels, plus the C-ABI entry points of the model glue (RMSNorm, RoPE, embedding).
//
// The layer runs on a weight slot of the sliding window (SlideFormer summary, section 2A: only
// the active layers live on the GPU). Between the forward and the backward sweep only the
// layer's input x is kept; the backward recomputes the forward's intermediates into its
// workspace (the summary's section 2B keeps the activation window small), then runs:
//   dm = dy Wd, dWd = dy^T m; SwiGLU backward; dr2 = dgu Wgu, dWgu = dgu^T r2;
//   dx2 = dy + RMSNorm_bwd(dr2); do = dx2 Wo, dWo = dx2^T o; attention backward; inverse RoPE;
//   dr = dqkv Wqkv, dWqkv = dqkv^T r; dx = dx2 + RMSNorm_bwd(dr).
#include <mutex>

#include "attention.h"
#include "gemm.h"
#include "pointwise.h"

namespace slide {
namespace {

struct Dims {
  int H, nq, nkv, d, F, dt, B, S, N, QR, OD;
  size_t ts;
};

int check_cfg(const slide_layer_cfg* c) {
  SLIDE_REQUIRE(c, SLIDE_E_ARG, "layer: null cfg");
  SLIDE_REQUIRE(dtype_valid(c->dtype), SLIDE_E_ARG, "layer: bad dtype %d", c->dtype);
  SLIDE_REQUIRE(c->hidden > 0 && c->hidden % 8 == 0, SLIDE_E_SHAPE, "layer: hidden %d must be a positive multiple of 8", c->hidden);
  SLIDE_REQUIRE(c->ffn > 0 && c->ffn % 8 == 0, SLIDE_E_SHAPE, "layer: ffn %d must be a positive multiple of 8", c->ffn);
  SLIDE_REQUIRE(c->head_dim == 64 || c->head_dim == 128, SLIDE_E_SHAPE, "layer: head_dim %d (64 or 128)", c->head_dim);
  SLIDE_REQUIRE(c->n_heads > 0 && c->n_kv_heads > 0 && c->n_heads % c->n_kv_heads == 0,
                SLIDE_E_SHAPE, "layer: n_heads %d must be a positive multiple of n_kv_heads %d",
                c->n_heads, c->n_kv_heads);
  SLIDE_REQUIRE(c->rms_eps > 0.f && c->rope_theta > 0.f, SLIDE_E_ARG, "layer: rms_eps and rope_theta must be > 0");
  return SLIDE_OK;
}

Dims dims_of(const slide_layer_cfg& c, int B, int S) {
  Dims d;
  d.H = c.hidden;
  d.nq = c.n_heads;
  d.nkv = c.n_kv_heads;
  d.d = c.head_dim;
  d.F = c.ffn;
  d.dt = c.dtype;
  d.B = B;
  d.S = S;
  d.N = B * S;
  d.QR = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  d.OD = c.n_heads * c.head_dim;
  d.ts = (size_t)dtype_size(c.dtype);
  return d;
}

void param_offsets(const Dims& d, size_t off[6]) {
  const size_t H = d.H, F = d.F;
  off[0] = 0;                             // w_attn [H]
  off[1] = off[0] + H;                    // Wqkv [QR, H]
  off[2] = off[1] + (size_t)d.QR * H;     // Wo [H, OD]
  off[3] = off[2] + H * (size_t)d.OD;     // w_mlp [H]
  off[4] = off[3] + H;                    // Wgu [2F, H]
  off[5] = off[4] + 2 * F * H;            // Wd [H, F]
}
size_t param_count(const Dims& d) {
  size_t off[6];
  param_offsets(d, off);
  return off[5] + (size_t)d.H * d.F;
}

// Workspace carving; with a null base only the size is computed.
struct Ws {
  void *r, *qkv, *o, *x2, *r2, *gu, *m;
  float *lse, *cos_t, *sin_t;
  void *dm, *dgu, *dr2, *dx2, *dO, *dqkv, *dr;
  void *rms_ws, *attn_ws;
  float* tail_ws;
  size_t bytes;
};

// Forward intermediates (everything the backward reads): the forward workspace, or the
// per-layer "saved" buffer that lets the backward skip the recompute.
size_t carve_fwd(void* base, const Dims& d, Ws& w) {
  Carver c(base);
  const size_t N = d.N;
  auto T = [&](size_t n) { return (void*)c.take<char>(n * d.ts); };
  w.cos_t = c.take<float>((size_t)d.S * (d.d / 2));
  w.sin_t = c.take<float>((size_t)d.S * (d.d / 2));
  w.r = T(N * d.H);
  w.qkv = T(N * d.QR);
  w.o = T(N * d.OD);
  w.lse = c.take<float>((size_t)d.B * d.nq * d.S);
  w.x2 = T(N * d.H);
  w.r2 = T(N * d.H);
  w.gu = T(N * 2 * (size_t)d.F);
  w.m = T(N * d.F);
  return align_up(c.used, 256);
}

// Backward-only buffers.
size_t carve_bwd(void* base, const Dims& d, Ws& w) {
  Carver c(base);
  const size_t N = d.N;
  auto T = [&](size_t n) { return (void*)c.take<char>(n * d.ts); };
  w.dm = T(N * d.F);
  w.dgu = T(N * 2 * (size_t)d.F);
  w.dr2 = T(N * d.H);
  w.dx2 = T(N * d.H);
  w.dO = T(N * d.OD);
  w.dqkv = T(N * d.QR);
  w.dr = T(N * d.H);
  w.rms_ws = c.take<char>(rmsnorm_bwd_ws(d.N, d.H));
  w.attn_ws = c.take<char>(attention_bwd_ws(d.B, d.S, d.nq));
  w.tail_ws = d.dt == SLIDE_F32 ? nullptr : (float*)c.take<char>(kTailWsBytes);
  return align_up(c.used, 256);
}

// Recompute layout: forward intermediates followed by the backward buffers in one workspace.
Ws carve(void* base, const Dims& d, bool bwd) {
  Ws w{};
  const size_t fb = carve_fwd(base, d, w);
  w.bytes = fb;
  if (bwd) w.bytes += carve_bwd(base ? (char*)base + fb : nullptr, d, w);
  return w;
}

inline const void* at(const void* p, size_t elems, size_t ts) { return (const char*)p + elems * ts; }
inline void* at(void* p, size_t elems, size_t ts) { return (char*)p + elems * ts; }

// tail_ws (kTailWsBytes, or null) lets a GEMM whose last wave of tiles is at most half full
// split those tiles over K
int gemm(int M, int N, int K, const void* A, int lda, bool ak, const void* B, int ldb, bool bk,
         void* C, int ldc, const void* R, int dt, const char* name, int site, hipStream_t st,
         float* tail_ws = nullptr) {
  GemmArgs g{M, N, K, A, lda, ak, B, ldb, bk, C, ldc, dt, R, R ? ldc : 0, 1.0f, false, dt, name,
             site};
  g.tail_ws = tail_ws;
  g.tail_ws_bytes = tail_ws ? kTailWsBytes : 0;
  return gemm_launch(g, st);
}

// forward through SwiGLU (everything the backward needs); y written when y != nullptr
int forward(const Dims& d, const slide_layer_cfg& c, const void* w, const void* x, void* y,
            const Ws& ws, hipStream_t st) {
  size_t off[6];
  param_offsets(d, off);
  const size_t ts = d.ts;
  SLIDE_TRY(rope_tables(ws.cos_t, ws.sin_t, d.S, d.d, c.rope_theta, st));
  SLIDE_TRY(rmsnorm_fwd(x, at(w, off[0], ts), ws.r, nullptr, d.N, d.H, c.rms_eps, d.dt, st));
  SLIDE_TRY(gemm(d.N, d.QR, d.H, ws.r, d.H, true, at(w, off[1], ts), d.H, true, ws.qkv, d.QR,
                 nullptr, d.dt, "gemm_qkv", SITE_QKV, st));
  SLIDE_TRY(rope_apply(ws.qkv, ws.cos_t, ws.sin_t, d.B, d.S, d.nq, d.nkv, d.d, 0, d.dt, st));
  SLIDE_TRY(attention_fwd(ws.qkv, ws.o, ws.lse, d.B, d.S, d.nq, d.nkv, d.d, d.dt, st));
  SLIDE_TRY(gemm(d.N, d.H, d.OD, ws.o, d.OD, true, at(w, off[2], ts), d.OD, true, ws.x2, d.H, x,
                 d.dt, "gemm_o", SITE_O, st));
  SLIDE_TRY(rmsnorm_fwd(ws.x2, at(w, off[3], ts), ws.r2, nullptr, d.N, d.H, c.rms_eps, d.dt, st));
  SLIDE_TRY(gemm_swiglu_fwd(d.N, d.F, d.H, ws.r2, d.H, at(w, off[4], ts), d.H, ws.gu, ws.m, d.dt,
                            "gemm_gate_up", SITE_GATE_UP, st));
  if (y)
    SLIDE_TRY(gemm(d.N, d.H, d.F, ws.m, d.F, true, at(w, off[5], ts), d.F, true, y, d.H, ws.x2,
                   d.dt, "gemm_down", SITE_DOWN, st));
  return SLIDE_OK;
}

int backward(const Dims& d, const slide_layer_cfg& c, const void* w, const void* x,
             const void* dy, void* dx, void* g, const Ws& ws, bool recompute, hipStream_t st) {
  size_t off[6];
  param_offsets(d, off);
  const size_t ts = d.ts;
  const int N = d.N, H = d.H, F = d.F;
  if (recompute) SLIDE_TRY(forward(d, c, w, x, nullptr, ws, st));
  // MLP half
  SLIDE_TRY(gemm_swiglu_bwd(N, F, H, dy, H, at(w, off[5], ts), F, ws.gu, ws.dgu, ws.dm, d.dt,
                            "gemm_down_dx", SITE_DOWN_DX, st));
  SLIDE_TRY(gemm(H, F, N, dy, H, false, ws.m, F, false, at(g, off[5], ts), F, nullptr, d.dt,
                 "gemm_down_dw", SITE_DOWN_DW, st, ws.tail_ws));
  SLIDE_TRY(gemm(N, H, 2 * F, ws.dgu, 2 * F, true, at(w, off[4], ts), H, false, ws.dr2, H,
                 nullptr, d.dt, "gemm_gate_up_dx", SITE_GATE_UP_DX, st, ws.tail_ws));
  SLIDE_TRY(gemm(2 * F, H, N, ws.dgu, 2 * F, false, ws.r2, H, false, at(g, off[4], ts), H,
                 nullptr, d.dt, "gemm_gate_up_dw", SITE_GATE_UP_DW, st, ws.tail_ws));
  SLIDE_TRY(rmsnorm_bwd(ws.dr2, ws.x2, at(w, off[3], ts), dy, ws.dx2, at(g, off[3], ts), N, H,
                        c.rms_eps, d.dt, ws.rms_ws, st));
  // attention half
  SLIDE_TRY(gemm(N, d.OD, H, ws.dx2, H, true, at(w, off[2], ts), d.OD, false, ws.dO, d.OD,
                 nullptr, d.dt, "gemm_o_dx", SITE_O_DX, st, ws.tail_ws));
  SLIDE_TRY(gemm(H, d.OD, N, ws.dx2, H, false, ws.o, d.OD, false, at(g, off[2], ts), d.OD,
                 nullptr, d.dt, "gemm_o_dw", SITE_O_DW, st, ws.tail_ws));
  SLIDE_TRY(attention_bwd(ws.qkv, ws.o, ws.lse, ws.dO, ws.dqkv, d.B, d.S, d.nq, d.nkv, d.d,
                          d.dt, ws.attn_ws, st));
  SLIDE_TRY(rope_apply(ws.dqkv, ws.cos_t, ws.sin_t, d.B, d.S, d.nq, d.nkv, d.d, 1, d.dt, st));
  SLIDE_TRY(gemm(N, H, d.QR, ws.dqkv, d.QR, true, at(w, off[1], ts), H, false, ws.dr, H, nullptr,
                 d.dt, "gemm_qkv_dx", SITE_QKV_DX, st, ws.tail_ws));
  SLIDE_TRY(gemm(d.QR, H, N, ws.dqkv, d.QR, false, ws.r, H, false, at(g, off[1], ts), H, nullptr,
                 d.dt, "gemm_qkv_dw", SITE_QKV_DW, st, ws.tail_ws));
  SLIDE_TRY(rmsnorm_bwd(ws.dr, x, at(w, off[0], ts), ws.dx2, dx, at(g, off[0], ts), N, H,
                        c.rms_eps, d.dt, ws.rms_ws, st));
  return SLIDE_OK;
}

int check_ptrs(const Dims& d, std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    SLIDE_REQUIRE(p, SLIDE_E_ARG, "layer: null pointer");
    SLIDE_REQUIRE(aligned16(p), SLIDE_E_ARG, "layer: pointers must be 16-byte aligned");
  }
  (void)d;
  return SLIDE_OK;
}

}  // namespace
}  // namespace slide

using namespace slide;

extern "C" size_t slide_layer_param_count(const slide_layer_cfg* cfg) {
  if (check_cfg(cfg) != SLIDE_OK) return 0;
  return param_count(dims_of(*cfg, 0, 0));
}

extern "C" int slide_layer_param_offsets(const slide_layer_cfg* cfg, size_t off[6]) {
  SLIDE_TRY(check_cfg(cfg));
  SLIDE_REQUIRE(off, SLIDE_E_ARG, "slide_layer_param_offsets: null output");
  param_offsets(dims_of(*cfg, 0, 0), off);
  return SLIDE_OK;
}

extern "C" size_t slide_layer_workspace_bytes(const slide_layer_cfg* cfg, int B, int S, int bwd) {
  if (check_cfg(cfg) != SLIDE_OK || B < 0 || S < 0) return 0;
  if (bwd == 2) {  // slide_layer_bwd_saved: the backward-only buffers
    Ws w{};
    return carve_bwd(nullptr, dims_of(*cfg, B, S), w);
  }
  return carve(nullptr, dims_of(*cfg, B, S), bwd != 0).bytes;
}

extern "C" int slide_layer_fwd(const slide_layer_cfg* cfg, const void* w_slot, const void* x,
                               void* y, int B, int S, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_TRY(check_cfg(cfg));
  SLIDE_REQUIRE(B >= 0 && S >= 0, SLIDE_E_SHAPE, "slide_layer_fwd: negative B or S");
  const Dims d = dims_of(*cfg, B, S);
  if (d.N == 0) return SLIDE_OK;
  SLIDE_TRY(check_ptrs(d, {w_slot, x, y, ws}));
  SLIDE_REQUIRE(x != y, SLIDE_E_ARG, "slide_layer_fwd: y must not alias x");
  const Ws w0 = carve(nullptr, d, false);
  SLIDE_REQUIRE(ws_bytes >= w0.bytes, SLIDE_E_WORKSPACE, "slide_layer_fwd: workspace %zu < %zu",
                ws_bytes, w0.bytes);
  return forward(d, *cfg, w_slot, x, y, carve(ws, d, false), (hipStream_t)stream);
}

extern "C" int slide_layer_bwd(const slide_layer_cfg* cfg, const void* w_slot, const void* x,
                               const void* dy, void* dx, void* g_slot, int B, int S, void* ws,
                               size_t ws_bytes, void* stream) {
  SLIDE_TRY(check_cfg(cfg));
  SLIDE_REQUIRE(B >= 0 && S >= 0, SLIDE_E_SHAPE, "slide_layer_bwd: negative B or S");
  const Dims d = dims_of(*cfg, B, S);
  SLIDE_TRY(check_ptrs(d, {w_slot, g_slot, ws}));
  if (d.N == 0)  // no tokens: every parameter gradient is zero
    return fill_zero(g_slot, param_count(d), d.dt, (hipStream_t)stream);
  SLIDE_TRY(check_ptrs(d, {x, dy, dx}));
  SLIDE_REQUIRE(x != dx, SLIDE_E_ARG, "slide_layer_bwd: dx must not alias x");
  const Ws w0 = carve(nullptr, d, true);
  SLIDE_REQUIRE(ws_bytes >= w0.bytes, SLIDE_E_WORKSPACE, "slide_layer_bwd: workspace %zu < %zu",
                ws_bytes, w0.bytes);
  return backward(d, *cfg, w_slot, x, dy, dx, g_slot, carve(ws, d, true), true,
                  (hipStream_t)stream);
}

extern "C" size_t slide_layer_saved_bytes(const slide_layer_cfg* cfg, int B, int S) {
  if (check_cfg(cfg) != SLIDE_OK || B < 0 || S < 0) return 0;
  Ws w{};
  return carve_fwd(nullptr, dims_of(*cfg, B, S), w);
}

extern "C" int slide_layer_fwd_save(const slide_layer_cfg* cfg, const void* w_slot, const void* x,
                                    void* y, int B, int S, void* saved, size_t saved_bytes,
                                    void* stream) {
  return slide_layer_fwd(cfg, w_slot, x, y, B, S, saved, saved_bytes, stream);
}

extern "C" int slide_layer_bwd_saved(const slide_layer_cfg* cfg, const void* w_slot,
                                     const void* x, const void* dy, void* dx, void* g_slot,
                                     int B, int S, const void* saved, size_t saved_bytes,
                                     void* ws, size_t ws_bytes, void* stream) {
  SLIDE_TRY(check_cfg(cfg));
  SLIDE_REQUIRE(B >= 0 && S >= 0, SLIDE_E_SHAPE, "slide_layer_bwd_saved: negative B or S");
  const Dims d = dims_of(*cfg, B, S);
  SLIDE_TRY(check_ptrs(d, {w_slot, g_slot}));
  if (d.N == 0) return fill_zero(g_slot, param_count(d), d.dt, (hipStream_t)stream);
  SLIDE_TRY(check_ptrs(d, {x, dy, dx, saved, ws}));
  SLIDE_REQUIRE(x != dx, SLIDE_E_ARG, "slide_layer_bwd_saved: dx must not alias x");
  Ws w{};
  const size_t fb = carve_fwd(nullptr, d, w);
  const size_t bb = carve_bwd(nullptr, d, w);
  SLIDE_REQUIRE(saved_bytes >= fb, SLIDE_E_WORKSPACE, "slide_layer_bwd_saved: saved %zu < %zu",
                saved_bytes, fb);
  SLIDE_REQUIRE(ws_bytes >= bb, SLIDE_E_WORKSPACE, "slide_layer_bwd_saved: workspace %zu < %zu",
                ws_bytes, bb);
  carve_fwd(const_cast<void*>(saved), d, w);
  carve_bwd(ws, d, w);
  return backward(d, *cfg, w_slot, x, dy, dx, g_slot, w, false, (hipStream_t)stream);
}

extern "C" int slide_rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd_out, int N,
                                 int H, float eps, int dtype, void* stream) {
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "rmsnorm: bad dtype");
  SLIDE_REQUIRE(N >= 0 && H > 0 && H % 8 == 0, SLIDE_E_SHAPE, "rmsnorm: H %d must be a positive multiple of 8", H);
  SLIDE_REQUIRE(eps > 0.f, SLIDE_E_ARG, "rmsnorm: eps must be > 0");
  if (N == 0) return SLIDE_OK;
  SLIDE_REQUIRE(x && w && y && aligned16(x) && aligned16(w) && aligned16(y), SLIDE_E_ARG,
                "rmsnorm: null or misaligned pointer");
  return rmsnorm_fwd(x, w, y, rstd_out, N, H, eps, dtype, (hipStream_t)stream);
}

extern "C" size_t slide_rmsnorm_bwd_workspace_bytes(int N, int H) {
  return rmsnorm_bwd_ws(N < 0 ? 0 : N, H < 0 ? 0 : H);
}

extern "C" int slide_rmsnorm_bwd(const void* dy, const void* x, const void* w, const void* dres,
                                 void* dx, void* dw, int N, int H, float eps, int dtype, void* ws,
                                 size_t ws_bytes, void* stream) {
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "rmsnorm: bad dtype");
  SLIDE_REQUIRE(N >= 0 && H > 0 && H % 8 == 0, SLIDE_E_SHAPE, "rmsnorm: H %d must be a positive multiple of 8", H);
  SLIDE_REQUIRE(ws && ws_bytes >= rmsnorm_bwd_ws(N, H), SLIDE_E_WORKSPACE,
                "rmsnorm_bwd: workspace %zu < %zu", ws_bytes, rmsnorm_bwd_ws(N, H));
  SLIDE_REQUIRE(N == 0 || (dy && x && w && dx), SLIDE_E_ARG, "rmsnorm_bwd: null pointer");
  SLIDE_REQUIRE(dy != dx, SLIDE_E_ARG, "rmsnorm_bwd: dx must not alias dy");
  return rmsnorm_bwd(dy, x, w, dres, dx, dw, N, H, eps, dtype, ws, (hipStream_t)stream);
}

// ------------------------------------------------------------------ no-allocation variant
// The RMSNorm backward's scratch (per-row 1/rms and the 64-row partial sums of the weight
// gradient) in a fixed device array, for callers that cannot allocate. Each GPU holds its own
// copy of the array; its device address is looked up once per device and kept.
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream` (the current device for the
// null stream).
int scratch_for_stream(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(SLIDE_E_HIP, "no-alloc scratch: hipGetDevice: %s", hipGetErrorString(e));
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess)
      return fail(SLIDE_E_HIP, "no-alloc scratch: hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SLIDE_E_UNSUPPORTED, "no-alloc scratch: device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(SLIDE_E_HIP, "no-alloc scratch: hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) hipSetDevice(cur);
    if (e != hipSuccess || !ptr)
      return fail(SLIDE_E_HIP, "no-alloc scratch: hipGetSymbolAddress on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SLIDE_OK;
}
}  // namespace

extern "C" size_t slide_rmsnorm_bwd_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int slide_rmsnorm_bwd_noalloc(const void* dy, const void* x, const void* w,
                                         const void* dres, void* dx, void* dw, int N, int H,
                                         float eps, int dtype, void* stream) {
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "rmsnorm: bad dtype");
  SLIDE_REQUIRE(N >= 0 && H > 0 && H % 8 == 0, SLIDE_E_SHAPE, "rmsnorm: H %d must be a positive multiple of 8", H);
  const size_t need = rmsnorm_bwd_ws(N, H);
  SLIDE_REQUIRE(need <= kNoAllocScratchBytes, SLIDE_E_WORKSPACE,
                "rmsnorm_bwd_noalloc: N=%d H=%d needs %zu bytes of scratch, the fixed array holds %zu",
                N, H, need, kNoAllocScratchBytes);
  SLIDE_REQUIRE(N == 0 || (dy && x && w && dx), SLIDE_E_ARG, "rmsnorm_bwd: null pointer");
  SLIDE_REQUIRE(dy != dx, SLIDE_E_ARG, "rmsnorm_bwd: dx must not alias dy");
  void* ptr = nullptr;
  SLIDE_TRY(scratch_for_stream((hipStream_t)stream, &ptr));
  // every scratch element the kernels read is written earlier in the same call: nothing needs
  // clearing, and a previous call's contents are never read
  return rmsnorm_bwd(dy, x, w, dres, dx, dw, N, H, eps, dtype, ptr, (hipStream_t)stream);
}

extern "C" int slide_nonfinite_count(const void* x, int dtype, size_t n, uint32_t* count_dev,
                                     void* stream) {
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "nonfinite_count: bad dtype");
  SLIDE_REQUIRE(count_dev && (n == 0 || x), SLIDE_E_ARG, "nonfinite_count: null pointer");
  SLIDE_REQUIRE(n == 0 || aligned16(x), SLIDE_E_ARG, "nonfinite_count: x must be 16-byte aligned");
  SLIDE_REQUIRE(((uintptr_t)count_dev & 3) == 0, SLIDE_E_ARG, "nonfinite_count: count must be 4-byte aligned");
  return nonfinite_count(x, n, dtype, count_dev, (hipStream_t)stream);
}

extern "C" int slide_rope(void* qkv, int B, int S, int nq, int nkv, int d, float theta,
                          int inverse, int dtype, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_TRY(attention_check(B, S, nq, nkv, d, dtype));
  SLIDE_REQUIRE(theta > 0.f, SLIDE_E_ARG, "rope: theta must be > 0");
  const size_t need = 2 * align_up((size_t)S * (d / 2) * 4, 256);
  SLIDE_REQUIRE(ws && ws_bytes >= need, SLIDE_E_WORKSPACE, "rope: workspace %zu < %zu", ws_bytes, need);
  if ((size_t)B * S == 0) return SLIDE_OK;
  SLIDE_REQUIRE(qkv, SLIDE_E_ARG, "rope: null qkv");
  Carver c(ws);
  float* cs = c.take<float>((size_t)S * (d / 2));
  float* sn = c.take<float>((size_t)S * (d / 2));
  SLIDE_TRY(rope_tables(cs, sn, S, d, theta, (hipStream_t)stream));
  return rope_apply(qkv, cs, sn, B, S, nq, nkv, d, inverse, dtype, (hipStream_t)stream);
}

namespace {
int swiglu_args(const void* a, const void* b, const void* c, int N, int F, int dtype,
                const char* what) {
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "%s: bad dtype", what);
  SLIDE_REQUIRE(N >= 0 && F > 0 && F % 8 == 0, SLIDE_E_SHAPE,
                "%s: N %d must be >= 0 and F %d a positive multiple of 8", what, N, F);
  if (N == 0) return SLIDE_OK;
  SLIDE_REQUIRE(a && b && c, SLIDE_E_ARG, "%s: null pointer", what);
  SLIDE_REQUIRE(aligned16(a) && aligned16(b) && aligned16(c), SLIDE_E_ARG,
                "%s: pointers must be 16-byte aligned", what);
  return SLIDE_OK;
}
}  // namespace

extern "C" int slide_swiglu_fwd(const void* gu, void* m, int N, int F, int dtype, void* stream) {
  SLIDE_TRY(swiglu_args(gu, m, m, N, F, dtype, "swiglu_fwd"));
  return swiglu_fwd(gu, m, N, F, dtype, (hipStream_t)stream);
}

extern "C" int slide_swiglu_bwd(const void* dm, const void* gu, void* dgu, int N, int F, int dtype,
                                void* stream) {
  SLIDE_TRY(swiglu_args(dm, gu, dgu, N, F, dtype, "swiglu_bwd"));
  return swiglu_bwd(dm, gu, dgu, N, F, dtype, (hipStream_t)stream);
}

extern "C" int slide_embed_fwd(const void* E, const int32_t* tokens, void* x, int N, int H, int V,
                               int dtype, void* stream) {
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "embed: bad dtype");
  SLIDE_REQUIRE(N >= 0 && V > 0 && H > 0 && H % 8 == 0, SLIDE_E_SHAPE, "embed: bad sizes N %d H %d V %d", N, H, V);
  if (N == 0) return SLIDE_OK;
  SLIDE_REQUIRE(E && tokens && x && aligned16(E) && aligned16(x), SLIDE_E_ARG, "embed: null or misaligned pointer");
  return embed_fwd(E, tokens, x, N, H, V, dtype, (hipStream_t)stream);
}

extern "C" int slide_copy_rows(const void* src, const int32_t* src_rows, int64_t src_n_rows,
                               void* dst, const int32_t* dst_rows, int64_t dst_n_rows,
                               int64_t n_rows, size_t row_bytes, void* stream) {
  SLIDE_REQUIRE(n_rows >= 0 && n_rows < (1LL << 31) && src_n_rows >= 0 && dst_n_rows >= 0,
                SLIDE_E_SHAPE, "copy_rows: bad row counts %lld %lld %lld", (long long)n_rows,
                (long long)src_n_rows, (long long)dst_n_rows);
  SLIDE_REQUIRE(row_bytes > 0 && row_bytes % 16 == 0, SLIDE_E_SHAPE,
                "copy_rows: row_bytes %zu is not a positive multiple of 16", row_bytes);
  SLIDE_REQUIRE((src_rows || n_rows <= src_n_rows) && (dst_rows || n_rows <= dst_n_rows),
                SLIDE_E_SHAPE, "copy_rows: %lld rows in order exceed a matrix", (long long)n_rows);
  if (n_rows == 0) return SLIDE_OK;
  SLIDE_REQUIRE(src && dst && aligned16(src) && aligned16(dst), SLIDE_E_ARG,
                "copy_rows: null or misaligned pointer");
  return copy_rows(src, src_rows, src_n_rows, dst, dst_rows, dst_n_rows, n_rows, row_bytes,
                   (hipStream_t)stream);
}

extern "C" int slide_convert_f32(const float* src, void* dst, int dst_dtype, size_t n,
                                 void* stream) {
  SLIDE_REQUIRE(dst_dtype == SLIDE_BF16 || dst_dtype == SLIDE_F16, SLIDE_E_ARG,
                "convert_f32: dst_dtype %d is not a 16-bit type", dst_dtype);
  if (n == 0) return SLIDE_OK;
  SLIDE_REQUIRE(src && dst, SLIDE_E_ARG, "convert_f32: null pointer");
  return convert_from_f32(src, dst, n, dst_dtype, (hipStream_t)stream);
}

extern "C" size_t slide_embed_bwd_workspace_bytes(int N, int V) { return embed_bwd_ws(N < 0 ? 0 : N, V); }

extern "C" int slide_embed_bwd(const void* dx, const int32_t* tokens, void* dE, int N, int H, int V,
                               int dtype, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "embed_bwd: bad dtype");
  SLIDE_REQUIRE(N >= 0 && N <= (1 << 30) && V > 0 && H > 0 && H % 8 == 0, SLIDE_E_SHAPE,
                "embed_bwd: bad sizes N %d H %d V %d", N, H, V);
  SLIDE_REQUIRE(ws && ws_bytes >= embed_bwd_ws(N, V), SLIDE_E_WORKSPACE, "embed_bwd: workspace %zu < %zu",
                ws_bytes, embed_bwd_ws(N, V));
  SLIDE_REQUIRE(dE && aligned16(dE) && (N == 0 || (dx && tokens && aligned16(dx))), SLIDE_E_ARG,
                "embed_bwd: null or misaligned pointer");
  return embed_bwd(dx, tokens, dE, N, H, V, dtype, ws, (hipStream_t)stream);
}
