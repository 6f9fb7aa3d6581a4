// Memory-bound kernels of the layer and the model glue: RMSNorm forward/backward, RoPE,
// SwiGLU forward/backward, token embedding gather and its deterministic backward, plus small
// fill/convert helpers. The pages name RoPE, RMSNorm and SwiGLU as the kernels their system
// rewrote (SlideFormer summary, section 2C); the formulas are the standard ones for the Llama
// family the summary names in section 4.
//
// Layout: rows of H (or 2F) contiguous elements; one 64-lane wavefront per row for the row
// reductions, 16-byte vector accesses (8 bf16 or 2x4 fp32) so every wave reads whole 128-byte
// lines. All arithmetic is fp32; bf16 is converted on load and rounded (nearest-even) on store.
#include "pointwise.h"
#include "swiglu.h"

namespace slide {
namespace {

// ---------------------------------------------------------------- 8-element vector I/O
template <typename T> struct V8;
template <> struct V8<bf16_t> {
  __device__ __forceinline__ static void load(const bf16_t* p, float (&v)[8]) {
    uint4 u = *(const uint4*)p;
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store(bf16_t* p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct V8<f16_t> {
  __device__ __forceinline__ static void load(const f16_t* p, float (&v)[8]) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = *(const h8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  }
  __device__ __forceinline__ static void store(f16_t* p, const float (&v)[8]) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)v[i];
    *(h8*)p = h;
  }
};
template <> struct V8<float> {
  __device__ __forceinline__ static void load(const float* p, float (&v)[8]) {
    float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&v)[8]) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// ---------------------------------------------------------------- RMSNorm
// y = w * x * r, r = 1/sqrt(mean(x^2) + eps); one wave per row, 4 rows per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ w,
                                                          T* __restrict__ y, float* rstd,
                                                          int N, int H, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= N) return;
  const T* xr = x + (size_t)row * H;
  float ss = 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    float v[8];
    V8<T>::load(xr + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  }
  ss = warp_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (rstd && lane == 0) rstd[row] = r;
  T* yr = y + (size_t)row * H;
  for (int c = lane * 8; c < H; c += 512) {
    float v[8], g[8];
    V8<T>::load(xr + c, v);
    V8<T>::load(w + c, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = g[i] * (v[i] * r);
    V8<T>::store(yr + c, v);
  }
}

// dx = dres + r*g - (r^3/H) * x * sum(g*x), g = w*dy; also stores r per row for the dw pass.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const T* __restrict__ dy,
                                                          const T* __restrict__ x,
                                                          const T* __restrict__ w,
                                                          const T* dres, T* dx, float* rstd,
                                                          int N, int H, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= N) return;
  const T* xr = x + (size_t)row * H;
  const T* dyr = dy + (size_t)row * H;
  float ss = 0.f, gx = 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    float xv[8], dv[8], wv[8];
    V8<T>::load(xr + c, xv);
    V8<T>::load(dyr + c, dv);
    V8<T>::load(w + c, wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ss += xv[i] * xv[i];
      gx += (wv[i] * dv[i]) * xv[i];
    }
  }
  ss = warp_sum(ss);
  gx = warp_sum(gx);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  const float coef = r * r * r * gx / (float)H;
  if (lane == 0) rstd[row] = r;
  T* dxr = dx + (size_t)row * H;
  const T* drr = dres ? dres + (size_t)row * H : nullptr;
  for (int c = lane * 8; c < H; c += 512) {
    float xv[8], dv[8], wv[8], o[8];
    V8<T>::load(xr + c, xv);
    V8<T>::load(dyr + c, dv);
    V8<T>::load(w + c, wv);
    if (drr) V8<T>::load(drr + c, o);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] += r * (wv[i] * dv[i]) - coef * xv[i];
    V8<T>::store(dxr + c, o);
  }
}

// Single-pass variants for rows of H = 512 * NI elements: each lane keeps its NI 8-element
// pieces of the row in registers (as loaded, 16 or 32 bytes each), so the row is read from
// memory once, with all of a lane's loads in flight together. Same operations in the same
// order as the two-pass kernels above, so the results are the same bits.
template <typename T>
struct Raw8 {
  uint4 u[sizeof(T) / 2];
  __device__ __forceinline__ void load(const T* p) {
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 2); ++k) u[k] = ((const uint4*)p)[k];
  }
  __device__ __forceinline__ void get(float (&v)[8]) const { V8<T>::load((const T*)u, v); }
};

template <typename T, int NI>
__global__ __launch_bounds__(256) void rmsnorm_fwd_reg_kernel(const T* __restrict__ x,
                                                              const T* __restrict__ w,
                                                              T* __restrict__ y, float* rstd,
                                                              int N, float eps) {
  constexpr int H = NI * 512;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= N) return;
  const T* xr = x + (size_t)row * H + lane * 8;
  Raw8<T> xv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) xv[i].load(xr + i * 512);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float v[8];
    xv[i].get(v);
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += v[k] * v[k];
  }
  ss = warp_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (rstd && lane == 0) rstd[row] = r;
  T* yr = y + (size_t)row * H + lane * 8;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float v[8], g[8];
    xv[i].get(v);
    V8<T>::load(w + i * 512 + lane * 8, g);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = g[k] * (v[k] * r);
    V8<T>::store(yr + i * 512, v);
  }
}

template <typename T, int NI>
__global__ __launch_bounds__(256) void rmsnorm_bwd_reg_kernel(const T* __restrict__ dy,
                                                              const T* __restrict__ x,
                                                              const T* __restrict__ w,
                                                              const T* dres, T* dx, float* rstd,
                                                              int N, float eps) {
  constexpr int H = NI * 512;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= N) return;
  const size_t o0 = (size_t)row * H + lane * 8;
  Raw8<T> xv[NI], dv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    xv[i].load(x + o0 + i * 512);
    dv[i].load(dy + o0 + i * 512);
  }
  float ss = 0.f, gx = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float a[8], d[8], g[8];
    xv[i].get(a);
    dv[i].get(d);
    V8<T>::load(w + i * 512 + lane * 8, g);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ss += a[k] * a[k];
      gx += (g[k] * d[k]) * a[k];
    }
  }
  ss = warp_sum(ss);
  gx = warp_sum(gx);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  const float coef = r * r * r * gx / (float)H;
  if (lane == 0) rstd[row] = r;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float a[8], d[8], g[8], o[8];
    xv[i].get(a);
    dv[i].get(d);
    V8<T>::load(w + i * 512 + lane * 8, g);
    if (dres) V8<T>::load(dres + o0 + i * 512, o);
    else
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] += r * (g[k] * d[k]) - coef * a[k];
    V8<T>::store(dx + o0 + i * 512, o);
  }
}

// dw partials: part[rb][j] = sum over rows of block rb of dy*x*r (rows in increasing order).
// One lane per 8 consecutive columns (16- or 32-byte loads), one wave per workgroup.
template <typename T>
__global__ __launch_bounds__(64) void rmsnorm_dw_partial_kernel(const T* __restrict__ dy,
                                                                const T* __restrict__ x,
                                                                const float* __restrict__ rstd,
                                                                float* __restrict__ part, int N,
                                                                int H, int rows_per_block) {
  const int j = (blockIdx.x * 64 + threadIdx.x) * 8;
  if (j >= H) return;
  const int r0 = blockIdx.y * rows_per_block, r1 = min(N, r0 + rows_per_block);
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  // 16 rows' loads in flight at a time; the sums still run row by row in order
  constexpr int U = 16;
  int t = r0;
  for (; t + U <= r1; t += U) {
    Raw8<T> a[U], b[U];
    float r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u].load(dy + (size_t)(t + u) * H + j);
      b[u].load(x + (size_t)(t + u) * H + j);
      r[u] = rstd[t + u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float av[8], bv[8];
      a[u].get(av);
      b[u].get(bv);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += av[k] * bv[k] * r[u];
    }
  }
  for (; t < r1; ++t) {
    float a[8], b[8];
    V8<T>::load(dy + (size_t)t * H + j, a);
    V8<T>::load(x + (size_t)t * H + j, b);
    const float r = rstd[t];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += a[k] * b[k] * r;
  }
  V8<float>::store(part + (size_t)blockIdx.y * H + j, acc);
}

// Sum of nparts rows of H floats (H a multiple of 4), per column: 64 columns per workgroup as 16
// groups of 4 (16-byte loads); the parts split over 16 slices (slice s takes parts s, s + 16,
// ..., with up to 8 loads in flight per thread, summed in increasing part order), the slices
// combined in slice order: the result is deterministic.
template <typename T>
__global__ __launch_bounds__(256) void reduce_rows_kernel(const float* __restrict__ part, T* out,
                                                          int nparts, int H) {
  __shared__ float red[16][64];
  const int cg = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int j = blockIdx.x * 64 + cg * 4;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  if (j < H) {
    for (int p0 = sl; p0 < nparts; p0 += 16 * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p0 + 16 * u < nparts) v[u] = *(const float4*)(part + (size_t)(p0 + 16 * u) * H + j);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p0 + 16 * u < nparts) {
          a[0] += v[u].x;
          a[1] += v[u].y;
          a[2] += v[u].z;
          a[3] += v[u].w;
        }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[sl][cg * 4 + e] = a[e];
  __syncthreads();
  if (threadIdx.x < 64 && blockIdx.x * 64 + (int)threadIdx.x < H) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][threadIdx.x];
    Elem<T>::store(out + blockIdx.x * 64 + threadIdx.x, t);
  }
}

// ---------------------------------------------------------------- RoPE
__global__ void rope_table_kernel(float* cos_t, float* sin_t, int S, int half, int d, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= S * half) return;
  const int s = idx / half, i = idx % half;
  const double inv = pow(theta, -2.0 * (double)i / (double)d);
  const double a = (double)s * inv;
  cos_t[idx] = (float)cos(a);
  sin_t[idx] = (float)sin(a);
}

// One thread per 8 consecutive rotation pairs (i .. i+7, i+d/2 .. i+d/2+7) of one (token, head)
// of the q and k parts: 16-byte loads and stores of both halves.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T* qkv, const float* __restrict__ cos_t,
                                                   const float* __restrict__ sin_t, int N, int S,
                                                   int heads, int d, int row_stride, float sgn) {
  const int half = d >> 1, groups = half >> 3;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)N * heads * groups;
  if (idx >= total) return;
  const int i0 = (int)(idx % groups) * 8;
  const size_t th = idx / groups;
  const int h = (int)(th % heads);
  const int t = (int)(th / heads);
  const int s = t % S;
  T* p = qkv + (size_t)t * row_stride + (size_t)h * d;
  float x1[8], x2[8], c[8], sn[8], o1[8], o2[8];
  V8<T>::load(p + i0, x1);
  V8<T>::load(p + i0 + half, x2);
  V8<float>::load(cos_t + (size_t)s * half + i0, c);
  V8<float>::load(sin_t + (size_t)s * half + i0, sn);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float sk = sgn * sn[k];
    o1[k] = x1[k] * c[k] - x2[k] * sk;
    o2[k] = x2[k] * c[k] + x1[k] * sk;
  }
  V8<T>::store(p + i0, o1);
  V8<T>::store(p + i0 + half, o2);
}

// ---------------------------------------------------------------- SwiGLU

template <typename T>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const T* __restrict__ gu,
                                                         T* __restrict__ m, int N, int F) {
  const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (idx >= (size_t)N * F) return;
  const size_t t = idx / F, j = idx % F;
  float g[8], u[8], o[8];
  V8<T>::load(gu + t * 2 * F + j, g);
  V8<T>::load(gu + t * 2 * F + F + j, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = swiglu_fwd_1(g[i], u[i]);
  V8<T>::store(m + idx, o);
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T* __restrict__ dm,
                                                         const T* __restrict__ gu,
                                                         T* __restrict__ dgu, int N, int F) {
  const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (idx >= (size_t)N * F) return;
  const size_t t = idx / F, j = idx % F;
  float g[8], u[8], d[8], dg[8], du[8];
  V8<T>::load(gu + t * 2 * F + j, g);
  V8<T>::load(gu + t * 2 * F + F + j, u);
  V8<T>::load(dm + idx, d);
#pragma unroll
  for (int i = 0; i < 8; ++i) swiglu_bwd_1(d[i], g[i], u[i], dg[i], du[i]);
  V8<T>::store(dgu + t * 2 * F + j, dg);
  V8<T>::store(dgu + t * 2 * F + F + j, du);
}

// ---------------------------------------------------------------- embedding
template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_kernel(const T* __restrict__ E,
                                                        const int32_t* __restrict__ tok,
                                                        T* __restrict__ x, int N, int H, int V) {
  const int row = blockIdx.x;
  const int v = tok[row];
  T* xr = x + (size_t)row * H;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float o[8];
    if (v >= 0 && v < V) V8<T>::load(E + (size_t)v * H + c, o);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = 0.f;
    V8<T>::store(xr + c, o);
  }
}

// keys[t] = (token << 32) | t for valid tokens, all-ones for padding and invalid tokens
__global__ void embed_keys_kernel(const int32_t* __restrict__ tok, uint64_t* keys, int N, int P,
                                  int V) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= P) return;
  uint64_t k = ~0ull;
  if (t < N) {
    int v = tok[t];
    if (v >= 0 && v < V) k = ((uint64_t)(uint32_t)v << 32) | (uint32_t)t;
  }
  keys[t] = k;
}

// one compare-exchange stage of a bitonic sort over P = 2^p keys (ascending)
__global__ void bitonic_step_kernel(uint64_t* keys, int P, int j, int k) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  const int l = i ^ j;
  if (l > i) {
    const uint64_t a = keys[i], b = keys[l];
    const bool up = (i & k) == 0;
    if ((a > b) == up) {
      keys[i] = b;
      keys[l] = a;
    }
  }
}

// dE[v] = sum of dx rows of the positions holding token v, in position order.
template <typename T>
__global__ __launch_bounds__(256) void embed_sum_kernel(const T* __restrict__ dx,
                                                        const uint64_t* __restrict__ keys, int P,
                                                        T* __restrict__ dE, int H) {
  const uint32_t v = blockIdx.x;
  // lower bound of (v << 32) in the sorted keys
  int lo = 0, hi = P;
  const uint64_t target = (uint64_t)v << 32;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (keys[mid] < target) lo = mid + 1;
    else hi = mid;
  }
  T* out = dE + (size_t)v * H;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int p = lo; p < P && (uint32_t)(keys[p] >> 32) == v; ++p) {
      const uint32_t t = (uint32_t)keys[p];
      float r[8];
      V8<T>::load(dx + (size_t)t * H + c, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += r[i];
    }
    V8<T>::store(out + c, acc);
  }
}

// ---------------------------------------------------------------- helpers
// ---------------------------------------------------------------- non-finite count
// Number of NaN or infinite elements (exponent bits all ones): 8 elements per thread and step
// (one 16-byte load for bf16, two for fp32) in a grid-stride loop, a wave sum, one integer atomic
// per wave (exact, whatever the order).
template <typename T>
__global__ __launch_bounds__(256) void nonfinite_count_kernel(const T* __restrict__ x, size_t n,
                                                              uint32_t* __restrict__ count) {
  const size_t n8 = n / 8;
  uint32_t c = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    if constexpr (sizeof(T) == 2) {
      // exponent field of bf16 (8 bits) or fp16 (5 bits), in both halves of a word
      constexpr uint32_t e = __is_same(T, f16_t) ? 0x7C00u : 0x7F80u;
      const uint4 u = *(const uint4*)(x + i * 8);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        c += ((w[k] & e) == e) + ((w[k] & (e << 16)) == (e << 16));
    } else {
      const uint4 a = *(const uint4*)(x + i * 8), b = *(const uint4*)(x + i * 8 + 4);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) c += (w[k] & 0x7F800000u) == 0x7F800000u;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < n - n8 * 8) {   // the last n % 8 elements
    const size_t i = n8 * 8 + threadIdx.x;
    constexpr uint32_t e = __is_same(T, f16_t) ? 0x7C00u : 0x7F80u;
    if constexpr (sizeof(T) == 2) c += (((const uint16_t*)x)[i] & e) == e;
    else c += (((const uint32_t*)x)[i] & 0x7F800000u) == 0x7F800000u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(count, c);
}

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

__global__ void fill_f32_kernel(float* p, size_t n, float v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void fill_u16_kernel(uint16_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
template <typename T>
__global__ void convert_f32_kernel(const float* __restrict__ src, T* __restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) Elem<T>::store(dst + i, src[i]);
}

inline unsigned blocks_for(size_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

// ------------------------------------------------------------------------ launchers
int rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd, int N, int H, float eps,
                int dtype, hipStream_t st) {
  if (N == 0) return SLIDE_OK;
  ProfScope ps("rmsnorm_fwd", st);
  dim3 grid(blocks_for(N, 4)), block(256);
#define SLIDE_RMS_FWD_REG(NI)                                                                  \
  case NI:                                                                                     \
    SLIDE_DISPATCH(dtype, T,                                                                   \
                   hipLaunchKernelGGL((rmsnorm_fwd_reg_kernel<T, NI>), grid, block, 0, st,     \
                                      (const T*)x, (const T*)w, (T*)y, rstd, N, eps));         \
    return check_launch("rmsnorm_fwd");
  if (H % 512 == 0) switch (H / 512) {
      SLIDE_RMS_FWD_REG(1) SLIDE_RMS_FWD_REG(2) SLIDE_RMS_FWD_REG(4) SLIDE_RMS_FWD_REG(8)
      SLIDE_RMS_FWD_REG(16) SLIDE_RMS_FWD_REG(24)
      default: break;
    }
#undef SLIDE_RMS_FWD_REG
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(rmsnorm_fwd_kernel<T>, grid, block, 0, st, (const T*)x,
                                    (const T*)w, (T*)y, rstd, N, H, eps));
  return check_launch("rmsnorm_fwd");
}

size_t rmsnorm_bwd_ws(int N, int H) {
  const int parts = (N + kRmsRowsPerPart - 1) / kRmsRowsPerPart;
  return align_up((size_t)N * 4, 256) + align_up((size_t)parts * H * 4, 256);
}

int rmsnorm_bwd(const void* dy, const void* x, const void* w, const void* dres, void* dx,
                void* dw, int N, int H, float eps, int dtype, void* ws, hipStream_t st) {
  Carver cv(ws);
  float* rstd = cv.take<float>((size_t)N);
  const int parts = (N + kRmsRowsPerPart - 1) / kRmsRowsPerPart;
  float* part = cv.take<float>((size_t)std::max(parts, 1) * H);
  {
    ProfScope ps("rmsnorm_bwd", st);
    if (N > 0) {
      dim3 grid(blocks_for(N, 4)), block(256);
      bool done = false;
#define SLIDE_RMS_BWD_REG(NI)                                                                  \
  case NI:                                                                                     \
    SLIDE_DISPATCH(dtype, T,                                                                   \
                   hipLaunchKernelGGL((rmsnorm_bwd_reg_kernel<T, NI>), grid, block, 0, st,     \
                                      (const T*)dy, (const T*)x, (const T*)w, (const T*)dres,  \
                                      (T*)dx, rstd, N, eps));                                  \
    done = true;                                                                               \
    break;
      if (H % 512 == 0) switch (H / 512) {
          SLIDE_RMS_BWD_REG(1) SLIDE_RMS_BWD_REG(2) SLIDE_RMS_BWD_REG(4) SLIDE_RMS_BWD_REG(8)
          SLIDE_RMS_BWD_REG(16)
          default: break;
        }
#undef SLIDE_RMS_BWD_REG
      if (!done)
        SLIDE_DISPATCH(dtype, T,
                       hipLaunchKernelGGL(rmsnorm_bwd_kernel<T>, grid, block, 0, st,
                                          (const T*)dy, (const T*)x, (const T*)w,
                                          (const T*)dres, (T*)dx, rstd, N, H, eps));
    }
  }
  SLIDE_TRY(check_launch("rmsnorm_bwd"));
  if (!dw) return SLIDE_OK;
  ProfScope ps("rmsnorm_dw", st);
  if (N == 0) {
    hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(H, 256)), dim3(256), 0, st, part, (size_t)H, 0.f);
  } else {
    dim3 g1(blocks_for(H / 8, 64), parts), b1(64);
    SLIDE_DISPATCH(dtype, T,
                   hipLaunchKernelGGL(rmsnorm_dw_partial_kernel<T>, g1, b1, 0, st,
                                      (const T*)dy, (const T*)x, rstd, part, N, H,
                                      kRmsRowsPerPart));
  }
  dim3 g2(blocks_for(H, 64)), b2(256);
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(reduce_rows_kernel<T>, g2, b2, 0, st, part, (T*)dw,
                                    std::max(parts, 1), H));
  return check_launch("rmsnorm_dw");
}

int nonfinite_count(const void* x, size_t n, int dtype, uint32_t* count, hipStream_t st) {
  ProfScope ps("nonfinite_count", st);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, st, count);
  if (n > 0) {
    const unsigned grid = std::min<size_t>(std::max<size_t>(blocks_for(n / 8, 256), 1), 2048);
    SLIDE_DISPATCH(dtype, T,
                   hipLaunchKernelGGL(nonfinite_count_kernel<T>, dim3(grid), dim3(256), 0, st,
                                      (const T*)x, n, count));
  }
  return check_launch("nonfinite_count");
}

int rope_tables(float* cos_t, float* sin_t, int S, int d, float theta, hipStream_t st) {
  ProfScope ps("rope_table", st);
  const int half = d / 2;
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks_for((size_t)S * half, 256)), dim3(256), 0, st,
                     cos_t, sin_t, S, half, d, (double)theta);
  return check_launch("rope_table");
}

int rope_apply(void* qkv, const float* cos_t, const float* sin_t, int B, int S, int nq, int nkv,
               int d, int inverse, int dtype, hipStream_t st) {
  const int N = B * S, heads = nq + nkv, stride = (nq + 2 * nkv) * d;
  const size_t total = (size_t)N * heads * (d / 16);   // threads: 8 pairs each (d % 16 == 0)
  if (total == 0) return SLIDE_OK;
  ProfScope ps(inverse ? "rope_bwd" : "rope_fwd", st);
  const float sgn = inverse ? -1.f : 1.f;
  dim3 grid(blocks_for(total, 256)), block(256);
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(rope_kernel<T>, grid, block, 0, st, (T*)qkv, cos_t, sin_t,
                                    N, S, heads, d, stride, sgn));
  return check_launch("rope");
}

int swiglu_fwd(const void* gu, void* m, int N, int F, int dtype, hipStream_t st) {
  const size_t n8 = (size_t)N * F / 8;
  if (n8 == 0) return SLIDE_OK;
  ProfScope ps("swiglu_fwd", st);
  dim3 grid(blocks_for(n8, 256)), block(256);
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(swiglu_fwd_kernel<T>, grid, block, 0, st, (const T*)gu,
                                    (T*)m, N, F));
  return check_launch("swiglu_fwd");
}

int swiglu_bwd(const void* dm, const void* gu, void* dgu, int N, int F, int dtype, hipStream_t st) {
  const size_t n8 = (size_t)N * F / 8;
  if (n8 == 0) return SLIDE_OK;
  ProfScope ps("swiglu_bwd", st);
  dim3 grid(blocks_for(n8, 256)), block(256);
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(swiglu_bwd_kernel<T>, grid, block, 0, st, (const T*)dm,
                                    (const T*)gu, (T*)dgu, N, F));
  return check_launch("swiglu_bwd");
}

int embed_fwd(const void* E, const int32_t* tok, void* x, int N, int H, int V, int dtype,
              hipStream_t st) {
  if (N == 0) return SLIDE_OK;
  ProfScope ps("embed_fwd", st);
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(embed_fwd_kernel<T>, dim3(N), dim3(256), 0, st,
                                    (const T*)E, tok, (T*)x, N, H, V));
  return check_launch("embed_fwd");
}

// One workgroup per row pair, 16-byte accesses.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4* __restrict__ src,
                                                        const int32_t* __restrict__ src_rows,
                                                        long long src_n, uint4* __restrict__ dst,
                                                        const int32_t* __restrict__ dst_rows,
                                                        long long dst_n, long long row_vec) {
  const long long k = blockIdx.x;
  const long long rs = src_rows ? (long long)src_rows[k] : k;
  const long long rd = dst_rows ? (long long)dst_rows[k] : k;
  if (rs < 0 || rs >= src_n || rd < 0 || rd >= dst_n) return;
  const uint4* s = src + rs * row_vec;
  uint4* d = dst + rd * row_vec;
  for (long long i = threadIdx.x; i < row_vec; i += 256) d[i] = s[i];
}

int copy_rows(const void* src, const int32_t* src_rows, long long src_n, void* dst,
              const int32_t* dst_rows, long long dst_n, long long n_rows, size_t row_bytes,
              hipStream_t st) {
  if (n_rows == 0) return SLIDE_OK;
  ProfScope ps("copy_rows", st);
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)n_rows), dim3(256), 0, st,
                     (const uint4*)src, src_rows, src_n, (uint4*)dst, dst_rows, dst_n,
                     (long long)(row_bytes / 16));
  return check_launch("copy_rows");
}

static int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

size_t embed_bwd_ws(int N, int V) {
  (void)V;
  return align_up((size_t)pow2_at_least(std::max(N, 1)) * 8, 256);
}

int embed_bwd(const void* dx, const int32_t* tok, void* dE, int N, int H, int V, int dtype,
              void* ws, hipStream_t st) {
  ProfScope ps("embed_bwd", st);
  const int P = pow2_at_least(std::max(N, 1));
  uint64_t* keys = (uint64_t*)ws;
  hipLaunchKernelGGL(embed_keys_kernel, dim3(blocks_for(P, 256)), dim3(256), 0, st, tok, keys, N,
                     P, V);
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1)
      hipLaunchKernelGGL(bitonic_step_kernel, dim3(blocks_for(P, 256)), dim3(256), 0, st, keys, P,
                         j, k);
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(embed_sum_kernel<T>, dim3(V), dim3(256), 0, st,
                                    (const T*)dx, keys, P, (T*)dE, H));
  return check_launch("embed_bwd");
}

int fill_zero(void* p, size_t n, int dtype, hipStream_t st) {
  if (n == 0) return SLIDE_OK;
  if (dtype != SLIDE_F32) {
    // a 16-bit zero is the all-zero bit pattern: fill as fp32 words plus a possible odd tail
    if (n >= 2)
      hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(n / 2, 256)), dim3(256), 0, st, (float*)p, n / 2, 0.f);
    if (n & 1)
      hipLaunchKernelGGL(fill_u16_kernel, dim3(1), dim3(1), 0, st, (uint16_t*)p + (n - 1), (size_t)1);
  } else {
    hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, (float*)p, n, 0.f);
  }
  return check_launch("fill_zero");
}

int fill_f32(float* p, size_t n, float v, hipStream_t st) {
  if (n == 0) return SLIDE_OK;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, p, n, v);
  return check_launch("fill");
}

int convert_from_f32(const float* src, void* dst, size_t n, int dtype, hipStream_t st) {
  if (n == 0) return SLIDE_OK;
  ProfScope ps("convert_f32", st);
  SLIDE_DISPATCH(dtype, T,
                 hipLaunchKernelGGL(convert_f32_kernel<T>, dim3(blocks_for(n, 256)), dim3(256),
                                    0, st, src, (T*)dst, n));
  return check_launch("convert_f32");
}

}  // namespace slide
