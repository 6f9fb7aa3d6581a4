// Fused LM-head cross-entropy in vocabulary chunks (SlideFormer summary, section 2C: the
// projection and the loss are fused so that the [N, V] logit tensor of a large vocabulary never
// exists, cutting the output layer's memory without changing the result).
//
//   pass 1, per chunk c of C vocabulary rows: z_c^T = W_c h^T (MFMA GEMM); per token and block
//           of 64 vocabulary rows the max and sum of exp(z - max), and the target logit.
//   combine: lse_t from the partials in a fixed order; loss = mean over valid t of lse_t - z_t[y_t]
//   pass 2, per chunk: recompute z_c^T, dz = (exp(z - lse_t) - [v == y_t]) / N_valid,
//           dh += dz^T W_c (fp32 accumulator), dW_c = dz h.
// bf16: the statistics of pass 1 and the dz of pass 2 are computed in the logits GEMM's
// epilogue, so no logit is ever stored; fp32 (the small configuration): the logits of one chunk
// go to an fp32 buffer that small kernels then reduce. Every reduction has a fixed order, so the
// results are deterministic. The workspace holds one chunk's dz, O(C*N), instead of O(V*N).
#include "ce.h"

#include "gemm.h"
#include "pointwise.h"

namespace slide {
namespace {

// The statistics pass keeps one (max, sum-exp) partial per token and block of kCeRowsPerPart
// vocabulary rows of a chunk (the bf16 path computes them in the logits GEMM's epilogue).
__host__ __device__ inline int ce_parts(int rows) { return (rows + kCeRowsPerPart - 1) / kCeRowsPerPart; }

// partial (max, sum exp(z - max)) of rows [r0, r1) of a [rows][ldz] fp32 chunk, per token column
__global__ __launch_bounds__(256) void ce_stats_kernel(const float* __restrict__ z, int rows,
                                                       int N, int ldz, int c0,
                                                       const int32_t* __restrict__ tgt,
                                                       float* __restrict__ pm,
                                                       float* __restrict__ ps,
                                                       float* __restrict__ zt, int splits) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= N) return;
  const int sp = blockIdx.y;
  const int per = (rows + splits - 1) / splits;
  const int r0 = sp * per, r1 = min(rows, r0 + per);
  float m = -INFINITY, s = 0.f;
  for (int r = r0; r < r1; ++r) {
    const float v = z[(size_t)r * ldz + t];
    if (v > m) {
      s = s * __expf(m - v) + 1.f;
      m = v;
    } else {
      s += __expf(v - m);
    }
  }
  pm[(size_t)sp * N + t] = m;
  ps[(size_t)sp * N + t] = s;
  const int y = tgt[t] - c0;
  if (y >= r0 && y < r1) zt[t] = z[(size_t)y * ldz + t];
}

// lse_t from the partials of every chunk (chunk c holds ce_parts(rows of c) partials starting
// at slot c * ppc) and the per-token loss term. Thread (t, g) of a 32 x 8 block folds the slots
// g, g + 8, ... of every chunk for token t (running max, rescaled sum), then the 8 folds of each
// token are combined in the order g = 0..7: a fixed order, so the result is deterministic.
__global__ __launch_bounds__(256) void ce_lse_kernel(const float* __restrict__ pm,
                                                     const float* __restrict__ ps, int nchunks,
                                                     int C, int ppc, int N,
                                                     const int32_t* __restrict__ tgt, int V,
                                                     const float* __restrict__ zt,
                                                     float* __restrict__ lse,
                                                     float* __restrict__ lt) {
  __shared__ float sm[8][32], ss[8][32];
  const int tl = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int t = blockIdx.x * 32 + tl;
  float m = -INFINITY, s = 0.f;
  if (t < N) {
    for (int c = 0; c < nchunks; ++c) {
      const int np = ce_parts(min(C, V - c * C));
      for (int p = g; p < np; p += 8) {
        const size_t at = (size_t)(c * ppc + p) * N + t;
        const float pmv = pm[at];
        if (pmv == -INFINITY) continue;
        const float psv = ps[at];
        if (pmv > m) {
          s = s * __expf(m - pmv) + psv;
          m = pmv;
        } else {
          s += psv * __expf(pmv - m);
        }
      }
    }
  }
  sm[g][tl] = m;
  ss[g][tl] = s;
  __syncthreads();
  if (g != 0 || t >= N) return;
  float mm = -INFINITY;
  for (int k = 0; k < 8; ++k) mm = fmaxf(mm, sm[k][tl]);
  float sum = 0.f;
  for (int k = 0; k < 8; ++k)
    if (sm[k][tl] != -INFINITY) sum += ss[k][tl] * __expf(sm[k][tl] - mm);
  const float l = mm + logf(sum);
  lse[t] = l;
  const int y = tgt[t];
  lt[t] = (y >= 0 && y < V) ? l - zt[t] : 0.f;
}

// loss = sum(lt over valid) / N_valid with a fixed reduction tree; also 1/N_valid for pass 2
__global__ __launch_bounds__(1024) void ce_loss_kernel(const float* __restrict__ lt,
                                                       const int32_t* __restrict__ tgt, int N,
                                                       int V, float* loss, float* inv_nv,
                                                       float scale) {
  __shared__ float ss[1024];
  __shared__ int sc[1024];
  float s = 0.f;
  int c = 0;
  for (int t = threadIdx.x; t < N; t += 1024) {
    const int y = tgt[t];
    if (y >= 0 && y < V) {
      s += lt[t];
      ++c;
    }
  }
  ss[threadIdx.x] = s;
  sc[threadIdx.x] = c;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      ss[threadIdx.x] += ss[threadIdx.x + o];
      sc[threadIdx.x] += sc[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int nv = sc[0];
    *loss = nv > 0 ? ss[0] / (float)nv : 0.f;
    *inv_nv = nv > 0 ? scale / (float)nv : 0.f;
  }
}

// dz[v][t] = (exp(z[v][t] - lse_t) - [c0 + v == y_t]) / N_valid for valid t, 0 otherwise
template <typename T>
__global__ __launch_bounds__(256) void ce_dz_kernel(const float* __restrict__ z,
                                                    T* __restrict__ dz, int rows, int N, int ldz,
                                                    int c0, int V, const int32_t* __restrict__ tgt,
                                                    const float* __restrict__ lse,
                                                    const float* __restrict__ inv_nv) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * ldz) return;
  const int r = (int)(idx / ldz), t = (int)(idx % ldz);
  float g = 0.f;
  if (t < N) {
    const int y = tgt[t];
    if (y >= 0 && y < V) {
      g = __expf(z[idx] - lse[t]);
      if (c0 + r == y) g -= 1.f;
      g *= *inv_nv;
    }
  }
  Elem<T>::store(dz + idx, g);
}

template <typename T>
__global__ void fill_zero_kernel(T* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) Elem<T>::store(p + i, 0.f);
}

__global__ void write_scalar_kernel(float* p, float v) { *p = v; }

struct CeLayout {
  int C, nchunks, ldz, ppc;   // ppc: partial slots per chunk
  size_t zbuf, dz, pm, ps, zt, lse, lt, scal, dh, total;
};

CeLayout ce_layout(const slide_ce_cfg& c, int N, bool want_dh) {
  CeLayout L{};
  L.C = c.chunk > 0 ? c.chunk : 8192;
  if (L.C > c.vocab) L.C = c.vocab;
  L.nchunks = (c.vocab + L.C - 1) / L.C;
  L.ldz = ((N + 7) / 8) * 8;
  const size_t ts = (size_t)dtype_size(c.dtype);
  size_t off = 0;
  auto put = [&](size_t bytes) {
    off = align_up(off, 256);
    size_t at = off;
    off += bytes;
    return at;
  };
  L.ppc = ce_parts(L.C);
  // fp32 logits of one chunk: only the fp32 path stores them (the bf16 path fuses the
  // statistics and dz into the logits GEMM)
  L.zbuf = c.dtype == SLIDE_F32 ? put((size_t)L.C * L.ldz * 4) : 0;
  L.dz = put((size_t)L.C * L.ldz * ts);
  L.pm = put((size_t)L.nchunks * L.ppc * N * 4);
  L.ps = put((size_t)L.nchunks * L.ppc * N * 4);
  L.zt = put((size_t)N * 4);
  L.lse = put((size_t)N * 4);
  L.lt = put((size_t)N * 4);
  L.scal = put(256);
  L.dh = want_dh ? put((size_t)N * c.hidden * 4) : 0;
  L.total = align_up(off, 256);
  return L;
}

inline unsigned nblk(size_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

size_t ce_workspace_bytes(const slide_ce_cfg& c, int N) { return ce_layout(c, N, true).total; }

int ce_check(const slide_ce_cfg* c, int N) {
  SLIDE_REQUIRE(c, SLIDE_E_ARG, "lmhead_ce: null cfg");
  SLIDE_REQUIRE(dtype_valid(c->dtype), SLIDE_E_ARG, "lmhead_ce: bad dtype");
  SLIDE_REQUIRE(c->grad_scale >= 0.f && c->grad_scale < 3.0e38f, SLIDE_E_ARG,
                "lmhead_ce: grad_scale must be a finite value >= 0");
  SLIDE_REQUIRE(c->hidden > 0 && c->hidden % 8 == 0, SLIDE_E_SHAPE, "lmhead_ce: hidden %d must be a positive multiple of 8", c->hidden);
  SLIDE_REQUIRE(c->vocab > 0 && c->vocab % 8 == 0, SLIDE_E_SHAPE, "lmhead_ce: vocab %d must be a positive multiple of 8", c->vocab);
  SLIDE_REQUIRE(c->chunk >= 0 && c->chunk % 8 == 0, SLIDE_E_SHAPE, "lmhead_ce: chunk %d must be a multiple of 8", c->chunk);
  SLIDE_REQUIRE(N >= 0, SLIDE_E_SHAPE, "lmhead_ce: negative token count");
  return SLIDE_OK;
}

// Workspace views shared by the phases below.
struct CeBufs {
  CeLayout L;
  float *zbuf, *pm, *ps, *zt, *lse, *lt, *inv_nv, *dh_acc;
  void* dz;
};

CeBufs ce_bufs(const slide_ce_cfg& c, int N, void* ws) {
  CeBufs b;
  b.L = ce_layout(c, N, true);
  char* base = (char*)ws;
  b.zbuf = (float*)(base + b.L.zbuf);
  b.dz = base + b.L.dz;
  b.pm = (float*)(base + b.L.pm);
  b.ps = (float*)(base + b.L.ps);
  b.zt = (float*)(base + b.L.zt);
  b.lse = (float*)(base + b.L.lse);
  b.lt = (float*)(base + b.L.lt);
  b.inv_nv = (float*)(base + b.L.scal);
  b.dh_acc = (float*)(base + b.L.dh);
  return b;
}

int ce_n_chunks(const slide_ce_cfg& c) { return ce_layout(c, 0, false).nchunks; }

namespace {

// z^T[v][t] = sum_k W[c0+v][k] h[t][k] for the rows of chunk ci. fp32: stored in the chunk
// buffer. bf16: the epilogue `special` consumes it (statistics or dz) and nothing is stored.
int ce_logits(const slide_ce_cfg& c, const CeBufs& b, const void* h, const void* w,
              const int32_t* tgt, int N, int ci, int special, hipStream_t st) {
  const int c0 = ci * b.L.C, rows = std::min(b.L.C, c.vocab - c0);
  const size_t ts = (size_t)dtype_size(c.dtype);
  const bool fused = c.dtype != SLIDE_F32;
  GemmArgs g{rows, N, c.hidden, (const char*)w + (size_t)c0 * c.hidden * ts, c.hidden, true, h,
             c.hidden, true, b.zbuf, b.L.ldz, SLIDE_F32, nullptr, 0, 1.0f, false, c.dtype,
             "ce_logits_gemm", SITE_GENERIC};
  if (fused) {
    g.special = special;
    g.tgt = tgt;
    g.c0 = c0;
    g.V = c.vocab;
    if (special == SPECIAL_CE_STATS) {
      g.site = SITE_CE_STATS;
      g.name = "ce_stats_gemm";
      g.C = b.pm;                 // not written; any non-null pointer
      g.pm = b.pm + (size_t)ci * b.L.ppc * N;
      g.ps = b.ps + (size_t)ci * b.L.ppc * N;
      g.zt = b.zt;
    } else {
      g.site = SITE_CE_DZ;
      g.name = "ce_dz_gemm";
      g.C = b.dz;
      g.c_dtype = c.dtype;
      g.lse = b.lse;
      g.inv_nv = b.inv_nv;
    }
  }
  return gemm_launch(g, st);
}

}  // namespace

// pass 1 for vocabulary chunk ci: logits, then per (token, row split) max / sum-exp partials and
// the target logit of targets inside the chunk
int ce_stats(const slide_ce_cfg& c, const void* h, const void* w, const int32_t* tgt, int N,
             int ci, void* ws, hipStream_t st) {
  if (N == 0) return SLIDE_OK;
  const CeBufs b = ce_bufs(c, N, ws);
  const int c0 = ci * b.L.C, rows = std::min(b.L.C, c.vocab - c0);
  SLIDE_TRY(ce_logits(c, b, h, w, tgt, N, ci, SPECIAL_CE_STATS, st));
  if (c.dtype != SLIDE_F32) return SLIDE_OK;   // the partials came out of the GEMM
  ProfScope ps_("ce_stats", st);
  const int parts = ce_parts(rows);
  hipLaunchKernelGGL(ce_stats_kernel, dim3(nblk(N, 256), parts), dim3(256), 0, st, b.zbuf,
                     rows, N, b.L.ldz, c0, tgt, b.pm + (size_t)ci * b.L.ppc * N,
                     b.ps + (size_t)ci * b.L.ppc * N, b.zt, parts);
  return check_launch("ce_stats");
}

// lse_t from the partials of every chunk (fixed order), the per-token loss and the mean
int ce_loss(const slide_ce_cfg& c, const int32_t* tgt, int N, float* loss, void* ws,
            hipStream_t st) {
  if (N == 0) {
    hipLaunchKernelGGL(write_scalar_kernel, dim3(1), dim3(1), 0, st, loss, 0.f);
    return check_launch("lmhead_ce(empty)");
  }
  const CeBufs b = ce_bufs(c, N, ws);
  ProfScope ps_("ce_lse", st);
  hipLaunchKernelGGL(ce_lse_kernel, dim3(nblk(N, 32)), dim3(256), 0, st, b.pm, b.ps,
                     b.L.nchunks, b.L.C, b.L.ppc, N, tgt, c.vocab, b.zt, b.lse, b.lt);
  const float scale = c.grad_scale > 0.f ? c.grad_scale : 1.0f;
  hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(1024), 0, st, b.lt, tgt, N, c.vocab, loss,
                     b.inv_nv, scale);
  return check_launch("ce_lse");
}

// pass 2 for vocabulary chunk ci: recomputed logits, dz, dh (fp32 accumulator in the workspace;
// chunk 0 initialises it) and the chunk's rows of dW
int ce_grad(const slide_ce_cfg& c, const void* h, const void* w, const int32_t* tgt, int N,
            int ci, bool with_dh, void* dw, void* ws, hipStream_t st) {
  const int H = c.hidden, V = c.vocab, dt = c.dtype;
  const size_t ts = (size_t)dtype_size(dt);
  const CeBufs b = ce_bufs(c, N, ws);
  const int c0 = ci * b.L.C, rows = std::min(b.L.C, V - c0);
  if (N == 0) {
    if (dw) {
      const size_t n = (size_t)rows * H;
      char* d = (char*)dw + (size_t)c0 * H * ts;
      SLIDE_DISPATCH(dt, T, hipLaunchKernelGGL(fill_zero_kernel<T>, dim3(nblk(n, 256)), dim3(256),
                                               0, st, (T*)d, n));
    }
    return check_launch("lmhead_ce(empty)");
  }
  SLIDE_TRY(ce_logits(c, b, h, w, tgt, N, ci, SPECIAL_CE_DZ, st));
  if (dt == SLIDE_F32) {   // the 16-bit path computed dz in the logits GEMM's epilogue
    ProfScope ps_("ce_dz", st);
    const size_t n = (size_t)rows * b.L.ldz;
    hipLaunchKernelGGL(ce_dz_kernel<float>, dim3(nblk(n, 256)), dim3(256), 0, st, b.zbuf,
                       (float*)b.dz, rows, N, b.L.ldz, c0, V, tgt, b.lse, b.inv_nv);
    SLIDE_TRY(check_launch("ce_dz"));
  }
  const void* wc = (const char*)w + (size_t)c0 * H * ts;
  if (with_dh) {
    // dh[t][i] (+)= sum_v dz[v][t] W[c0+v][i]
    GemmArgs g{N, H, rows, b.dz, b.L.ldz, false, wc, H, false, b.dh_acc, H, SLIDE_F32, nullptr,
               0, 1.0f, ci > 0, dt, "ce_dh_gemm", SITE_CE_DH};
    SLIDE_TRY(gemm_launch(g, st));
  }
  if (dw) {
    // dW[c0+v][i] = sum_t dz[v][t] h[t][i]
    GemmArgs g{rows, H, N, b.dz, b.L.ldz, true, h, H, false, (char*)dw + (size_t)c0 * H * ts, H,
               dt, nullptr, 0, 1.0f, false, dt, "ce_dw_gemm", SITE_CE_DW};
    SLIDE_TRY(gemm_launch(g, st));
  }
  return SLIDE_OK;
}

// dh in the storage type from the fp32 accumulator
int ce_dh(const slide_ce_cfg& c, int N, void* dh, void* ws, hipStream_t st) {
  if (N == 0) return SLIDE_OK;
  const CeBufs b = ce_bufs(c, N, ws);
  return convert_from_f32(b.dh_acc, dh, (size_t)N * c.hidden, c.dtype, st);
}

int ce_run(const slide_ce_cfg& c, const void* h, const void* w, const int32_t* tgt, int N,
           float* loss, void* dh, void* dw, void* ws, hipStream_t st) {
  const int nch = ce_n_chunks(c);
  if (N > 0)
    for (int ci = 0; ci < nch; ++ci) SLIDE_TRY(ce_stats(c, h, w, tgt, N, ci, ws, st));
  SLIDE_TRY(ce_loss(c, tgt, N, loss, ws, st));
  if (!dh && !dw) return SLIDE_OK;
  for (int ci = 0; ci < nch; ++ci) SLIDE_TRY(ce_grad(c, h, w, tgt, N, ci, dh != nullptr, dw, ws, st));
  if (dh) SLIDE_TRY(ce_dh(c, N, dh, ws, st));
  return SLIDE_OK;
}

}  // namespace slide

extern "C" size_t slide_lmhead_ce_workspace_bytes(const slide_ce_cfg* cfg, int N) {
  if (!cfg || slide::ce_check(cfg, N) != SLIDE_OK) return 0;
  return slide::ce_workspace_bytes(*cfg, N);
}

namespace {
int ce_common_check(const slide_ce_cfg* cfg, int N, const void* ws, size_t ws_bytes,
                    const char* fn) {
  SLIDE_TRY(slide::ce_check(cfg, N));
  SLIDE_REQUIRE(ws, SLIDE_E_ARG, "%s: null workspace", fn);
  const size_t need = slide::ce_workspace_bytes(*cfg, N);
  SLIDE_REQUIRE(ws_bytes >= need, SLIDE_E_WORKSPACE, "%s: workspace %zu < %zu", fn, ws_bytes, need);
  return SLIDE_OK;
}
int ce_chunk_check(const slide_ce_cfg* cfg, int chunk, const char* fn) {
  const int n = slide::ce_n_chunks(*cfg);
  SLIDE_REQUIRE(chunk >= 0 && chunk < n, SLIDE_E_ARG, "%s: chunk %d outside [0, %d)", fn, chunk, n);
  return SLIDE_OK;
}
}  // namespace

extern "C" int slide_lmhead_ce_n_chunks(const slide_ce_cfg* cfg) {
  if (slide::ce_check(cfg, 0) != SLIDE_OK) return slide::fail(SLIDE_E_ARG, "slide_lmhead_ce_n_chunks: bad cfg");
  return slide::ce_n_chunks(*cfg);
}

extern "C" int slide_lmhead_ce_stats(const slide_ce_cfg* cfg, const void* h, const void* w,
                                     const int32_t* targets, int N, int chunk, void* ws,
                                     size_t ws_bytes, void* stream) {
  SLIDE_TRY(ce_common_check(cfg, N, ws, ws_bytes, "slide_lmhead_ce_stats"));
  SLIDE_TRY(ce_chunk_check(cfg, chunk, "slide_lmhead_ce_stats"));
  SLIDE_REQUIRE(N == 0 || (h && w && targets), SLIDE_E_ARG, "slide_lmhead_ce_stats: null pointer");
  SLIDE_REQUIRE(slide::aligned16(h) && slide::aligned16(w), SLIDE_E_ARG,
                "slide_lmhead_ce_stats: tensors must be 16-byte aligned");
  return slide::ce_stats(*cfg, h, w, targets, N, chunk, ws, (hipStream_t)stream);
}

extern "C" int slide_lmhead_ce_loss(const slide_ce_cfg* cfg, const int32_t* targets, int N,
                                    float* loss_dev, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_TRY(ce_common_check(cfg, N, ws, ws_bytes, "slide_lmhead_ce_loss"));
  SLIDE_REQUIRE(loss_dev && (N == 0 || targets), SLIDE_E_ARG, "slide_lmhead_ce_loss: null pointer");
  return slide::ce_loss(*cfg, targets, N, loss_dev, ws, (hipStream_t)stream);
}

extern "C" int slide_lmhead_ce_grad(const slide_ce_cfg* cfg, const void* h, const void* w,
                                    const int32_t* targets, int N, int chunk, int with_dh,
                                    void* dw, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_TRY(ce_common_check(cfg, N, ws, ws_bytes, "slide_lmhead_ce_grad"));
  SLIDE_TRY(ce_chunk_check(cfg, chunk, "slide_lmhead_ce_grad"));
  SLIDE_REQUIRE(N == 0 || (h && w && targets), SLIDE_E_ARG, "slide_lmhead_ce_grad: null pointer");
  SLIDE_REQUIRE(slide::aligned16(h) && slide::aligned16(w) && (!dw || slide::aligned16(dw)),
                SLIDE_E_ARG, "slide_lmhead_ce_grad: tensors must be 16-byte aligned");
  return slide::ce_grad(*cfg, h, w, targets, N, chunk, with_dh != 0, dw, ws, (hipStream_t)stream);
}

extern "C" int slide_lmhead_ce_dh(const slide_ce_cfg* cfg, int N, void* dh, void* ws,
                                  size_t ws_bytes, void* stream) {
  SLIDE_TRY(ce_common_check(cfg, N, ws, ws_bytes, "slide_lmhead_ce_dh"));
  SLIDE_REQUIRE(dh || N == 0, SLIDE_E_ARG, "slide_lmhead_ce_dh: null dh");
  SLIDE_REQUIRE(slide::aligned16(dh), SLIDE_E_ARG, "slide_lmhead_ce_dh: dh must be 16-byte aligned");
  return slide::ce_dh(*cfg, N, dh, ws, (hipStream_t)stream);
}

extern "C" int slide_lmhead_ce(const slide_ce_cfg* cfg, const void* h, const void* w,
                               const int32_t* targets, int N, float* loss_dev, void* dh,
                               void* dw, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_TRY(slide::ce_check(cfg, N));
  SLIDE_REQUIRE(loss_dev && ws && (N == 0 || (h && w && targets)), SLIDE_E_ARG,
                "slide_lmhead_ce: null pointer");
  SLIDE_REQUIRE(slide::aligned16(h) && slide::aligned16(w) && (!dh || slide::aligned16(dh)) &&
                    (!dw || slide::aligned16(dw)),
                SLIDE_E_ARG, "slide_lmhead_ce: tensors must be 16-byte aligned");
  const size_t need = slide::ce_workspace_bytes(*cfg, N);
  SLIDE_REQUIRE(ws_bytes >= need, SLIDE_E_WORKSPACE, "slide_lmhead_ce: workspace %zu < %zu",
                ws_bytes, need);
  return slide::ce_run(*cfg, h, w, targets, N, loss_dev, dh, dw, ws, (hipStream_t)stream);
}
