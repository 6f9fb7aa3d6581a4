// CPU AdamW: the per-layer host optimizer of the layer-sliding method ("Layer-Adam": optimizer
// state kept in host memory and updated on the CPU layer by layer while the GPU runs the next
// layer's backward; SlideFormer summary, sections 2A and 2B).
//
// Fixed float32 operation order, every operation rounded to nearest-even and no fused
// multiply-add, so that the result is reproducible bit for bit on any x86-64 host:
//   p1 = p*c_dec; m' = c_b1*m + c_1b1*g; v' = c_b2*v + c_1b2*(g*g);
//   den = sqrt(v')/c_bc2 + c_eps; p' = p1 - c_step*(m'/den); bf16 copy = rne(p').
// The AVX-512 path and the scalar path perform the same IEEE operations element by element.
// This file must be compiled with -ffp-contract=off and without fast-math.
#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/slide.h"
#include "adamw_consts.h"

namespace slide {
int fail(int code, const char* fmt, ...);
}

namespace {

// Helper threads kept alive per calling thread: a layer's update is one call, about seventy per
// training step, and creating and joining a dozen threads for each of them costs more than the
// dispatch below. Each calling thread (the engine's in-memory and tiered workers, a test) owns
// its own helpers, so concurrent callers never wait for one another; they end with it.
class Helpers {
 public:
  ~Helpers() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  // Run body(i) for i in [0, n): i = 0 on the caller, the others on helpers; returns when all
  // are done.
  void run(int n, const std::function<void(int)>& body) {
    if (n <= 1) {
      if (n == 1) body(0);
      return;
    }
    while ((int)th_.size() < n - 1) {
      const int k = (int)th_.size();
      th_.emplace_back([this, k] { loop(k + 1); });
    }
    {
      std::lock_guard<std::mutex> lk(mu_);
      body_ = &body;
      n_ = n;
      left_ = n - 1;
      ++gen_;
    }
    cv_.notify_all();
    body(0);
    std::unique_lock<std::mutex> lk(mu_);
    done_.wait(lk, [&] { return left_ == 0; });
    body_ = nullptr;
  }

 private:
  void loop(int idx) {
    uint64_t seen = 0;
    {
      std::lock_guard<std::mutex> lk(mu_);
      seen = gen_;   // a helper created for a call joins it below: gen_ already counts it
      if (body_ && idx < n_) --seen;
    }
    for (;;) {
      const std::function<void(int)>* b;
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
        if (idx >= n_) continue;   // not needed in this call
        b = body_;
      }
      (*b)(idx);
      {
        std::lock_guard<std::mutex> lk(mu_);
        if (--left_ == 0) done_.notify_all();
      }
    }
  }
  std::vector<std::thread> th_;
  std::mutex mu_;
  std::condition_variable cv_, done_;
  const std::function<void(int)>* body_ = nullptr;
  int n_ = 0, left_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

thread_local Helpers tl_helpers;

// body(lo, hi) over [0, n) split into at most nt ranges of `align`-multiple length
void parallel_ranges(size_t n, int nt, size_t align, const std::function<void(size_t, size_t)>& body) {
  size_t per = (n + nt - 1) / nt;
  per = (per + align - 1) / align * align;
  const int parts = (int)((n + per - 1) / per);
  tl_helpers.run(parts, [&](int i) {
    const size_t lo = (size_t)i * per, hi = std::min(n, lo + per);
    if (lo < hi) body(lo, hi);
  });
}

using Consts = slide::AdamConsts;

Consts make_consts(const slide_adamw_hp& hp, int64_t t) { return slide::adam_consts(hp, t); }

// Every listed row inside [0, n_total) and listed once (a repeated row would be updated twice,
// by two threads at once); -1 if so, else the position of the first offending entry.
long long bad_row(const int32_t* rows, size_t n, size_t n_total) {
  std::vector<uint64_t> seen((n_total + 63) / 64, 0);
  for (size_t k = 0; k < n; ++k) {
    const int32_t r = rows[k];
    if (r < 0 || (size_t)r >= n_total) return (long long)k;
    uint64_t& w = seen[(size_t)r >> 6];
    const uint64_t bit = uint64_t(1) << (r & 63);
    if (w & bit) return (long long)k;
    w |= bit;
  }
  return -1;
}

inline float widen_bf16(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

__attribute__((target("f16c"))) inline float widen_f16(uint16_t h) { return _cvtsh_ss(h); }
__attribute__((target("f16c"))) inline uint16_t f16_rne(float f) {
  return (uint16_t)_cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
}

inline uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Gradient element i of g_dtype as float (exact), unscaled by c_gs when the gradient carries a
// loss scale.
inline float grad_at(const void* g, int gdt, size_t i, const Consts& c) {
  float gi = gdt == SLIDE_BF16   ? widen_bf16(((const uint16_t*)g)[i])
             : gdt == SLIDE_F16 ? widen_f16(((const uint16_t*)g)[i])
                                : ((const float*)g)[i];
  if (c.c_gs != 1.0f) gi = gi * c.c_gs;
  return gi;
}

// One element; g is already widened to float. The 16-bit copy is fp16 when the gradient is
// (f16_out), else bf16.
inline void step1(float& p, float g, float& m, float& v, uint16_t* out, const Consts& c,
                  bool f16_out = false) {
  float p1 = p * c.c_dec;
  float a = c.c_b1 * m;
  float b = c.c_1b1 * g;
  float m2 = a + b;
  float gg = g * g;
  float e = c.c_b2 * v;
  float f = c.c_1b2 * gg;
  float v2 = e + f;
  float sq = sqrtf(v2);
  float q = sq / c.c_bc2;
  float den = q + c.c_eps;
  float r = m2 / den;
  float s = c.c_step * r;
  float p2 = p1 - s;
  p = p2;
  m = m2;
  v = v2;
  if (out) *out = f16_out ? f16_rne(p2) : bf16_rne(p2);
}

void range_scalar(float* p, const void* g, int gdt, float* m, float* v, uint16_t* out,
                  size_t lo, size_t hi, const Consts& c) {
  for (size_t i = lo; i < hi; ++i)
    step1(p[i], grad_at(g, gdt, i, c), m[i], v[i], out ? out + i : nullptr, c,
          gdt == SLIDE_F16);
}

__attribute__((target("avx512f,avx512bw"))) void range_avx512(float* p, const void* g, int gdt,
                                                                float* m, float* v,
                                                                uint16_t* out, size_t lo,
                                                                size_t hi, const Consts& c) {
  const __m512 c_dec = _mm512_set1_ps(c.c_dec), c_b1 = _mm512_set1_ps(c.c_b1),
               c_1b1 = _mm512_set1_ps(c.c_1b1), c_b2 = _mm512_set1_ps(c.c_b2),
               c_1b2 = _mm512_set1_ps(c.c_1b2), c_step = _mm512_set1_ps(c.c_step),
               c_bc2 = _mm512_set1_ps(c.c_bc2), c_eps = _mm512_set1_ps(c.c_eps);
  const __m512i exp_mask = _mm512_set1_epi32(0x7fffffff), inf_bits = _mm512_set1_epi32(0x7f800000),
                bias = _mm512_set1_epi32(0x7fff), one = _mm512_set1_epi32(1),
                quiet = _mm512_set1_epi32(0x40);
  const __m512 c_gs = _mm512_set1_ps(c.c_gs);
  const bool scaled = c.c_gs != 1.0f, f16 = gdt == SLIDE_F16;
  size_t i = lo;
  // scalar head up to 64-byte alignment of p
  while (i < hi && (((uintptr_t)(p + i)) & 63u)) {
    step1(p[i], grad_at(g, gdt, i, c), m[i], v[i], out ? out + i : nullptr, c, f16);
    ++i;
  }
  for (; i + 16 <= hi; i += 16) {
    __m512 gv;
    if (gdt == SLIDE_BF16) {
      __m256i gb = _mm256_loadu_si256((const __m256i*)((const uint16_t*)g + i));
      gv = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(gb), 16));
    } else if (f16) {
      gv = _mm512_cvtph_ps(_mm256_loadu_si256((const __m256i*)((const uint16_t*)g + i)));
    } else {
      gv = _mm512_loadu_ps((const float*)g + i);
    }
    if (scaled) gv = _mm512_mul_ps(gv, c_gs);
    __m512 pv = _mm512_load_ps(p + i);
    __m512 mv = _mm512_loadu_ps(m + i);
    __m512 vv = _mm512_loadu_ps(v + i);
    __m512 p1 = _mm512_mul_ps(pv, c_dec);
    __m512 m2 = _mm512_add_ps(_mm512_mul_ps(c_b1, mv), _mm512_mul_ps(c_1b1, gv));
    __m512 v2 = _mm512_add_ps(_mm512_mul_ps(c_b2, vv), _mm512_mul_ps(c_1b2, _mm512_mul_ps(gv, gv)));
    __m512 den = _mm512_add_ps(_mm512_div_ps(_mm512_sqrt_ps(v2), c_bc2), c_eps);
    __m512 p2 = _mm512_sub_ps(p1, _mm512_mul_ps(c_step, _mm512_div_ps(m2, den)));
    _mm512_store_ps(p + i, p2);
    _mm512_storeu_ps(m + i, m2);
    _mm512_storeu_ps(v + i, v2);
    if (out && f16) {
      _mm256_storeu_si256((__m256i*)(out + i),
                          _mm512_cvtps_ph(p2, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC));
    } else if (out) {
      __m512i u = _mm512_castps_si512(p2);
      __mmask16 isnan = _mm512_cmpgt_epu32_mask(_mm512_and_si512(u, exp_mask), inf_bits);
      __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(u, 16), one);
      __m512i rnd = _mm512_srli_epi32(_mm512_add_epi32(_mm512_add_epi32(u, bias), lsb), 16);
      __m512i qn = _mm512_or_si512(_mm512_srli_epi32(u, 16), quiet);
      __m512i res = _mm512_mask_mov_epi32(rnd, isnan, qn);
      _mm256_storeu_si256((__m256i*)(out + i), _mm512_cvtepi32_epi16(res));
    }
  }
  for (; i < hi; ++i)
    step1(p[i], grad_at(g, gdt, i, c), m[i], v[i], out ? out + i : nullptr, c, f16);
}

}  // namespace

int slide::adamw_check(const char* who, const void* p, const void* g, int g_dtype,
                       const void* m, const void* v, const void* p_bf16_out, size_t n,
                       int64_t step, const slide_adamw_hp* hp) {
  using slide::fail;
  if (!p || !g || !m || !v || !hp) return fail(SLIDE_E_ARG, "%s: null pointer", who);
  if (g_dtype != SLIDE_BF16 && g_dtype != SLIDE_F16 && g_dtype != SLIDE_F32)
    return fail(SLIDE_E_ARG, "%s: g_dtype must be SLIDE_BF16, SLIDE_F16 or SLIDE_F32", who);
  if (!(hp->grad_scale >= 0))
    return fail(SLIDE_E_ARG, "%s: grad_scale must be >= 0", who);
  if (step < 1) return fail(SLIDE_E_ARG, "%s: step must be >= 1 (got %lld)", who, (long long)step);
  if (!(hp->beta1 >= 0 && hp->beta1 < 1 && hp->beta2 >= 0 && hp->beta2 < 1 && hp->eps > 0 &&
        hp->lr >= 0 && hp->weight_decay >= 0))
    return fail(SLIDE_E_ARG, "%s: hyper-parameters out of range", who);
  if (p_bf16_out && p_bf16_out != g) {
    // overlapping but not identical buffers would read already-written values
    const char* a = (const char*)p_bf16_out;
    const char* b = (const char*)g;
    size_t gb = n * (g_dtype == SLIDE_F32 ? 4 : 2);
    if (a < b + gb && b < a + n * 2)
      return fail(SLIDE_E_ARG, "%s: p_bf16_out partially overlaps g", who);
  }
  if (p_bf16_out && p_bf16_out == g && g_dtype == SLIDE_F32)
    return fail(SLIDE_E_ARG, "%s: p_bf16_out may alias g only for a 16-bit g", who);
  return SLIDE_OK;
}

extern "C" int slide_cpu_adamw(float* p, const void* g, int g_dtype, float* m, float* v,
                               uint16_t* p_bf16_out, size_t n, int64_t step,
                               const slide_adamw_hp* hp, int n_threads) {
  if (n == 0) return SLIDE_OK;
  int rc = slide::adamw_check("slide_cpu_adamw", p, g, g_dtype, m, v, p_bf16_out, n, step, hp);
  if (rc != SLIDE_OK) return rc;
  const Consts c = make_consts(*hp, step);
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  size_t min_per = 1 << 16;
  nt = (int)std::max<size_t>(1, std::min<size_t>((size_t)nt, (n + min_per - 1) / min_per));
  const bool avx512 = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
  auto work = [&](size_t lo, size_t hi) {
    if (avx512)
      range_avx512(p, g, g_dtype, m, v, p_bf16_out, lo, hi, c);
    else
      range_scalar(p, g, g_dtype, m, v, p_bf16_out, lo, hi, c);
  };
  if (nt == 1) {
    work(0, n);
    return SLIDE_OK;
  }
  parallel_ranges(n, nt, 16, work);
  return SLIDE_OK;
}

// The same update on a list of rows of row_len elements (row r = elements [r*row_len,
// (r+1)*row_len) of p, m, v, g and the bf16 copy); g may be NULL for rows whose gradient is
// exactly zero (an embedding's rows that no token of the batch selected). Rows are split evenly
// over the threads; each row runs the element loop of slide_cpu_adamw, so the results are the
// same bits as a whole-array call with those gradient values.
extern "C" int slide_cpu_adamw_rows(float* p, const void* g, int g_dtype, float* m, float* v,
                                    uint16_t* p_bf16_out, size_t row_len, size_t n_rows_total,
                                    const int32_t* rows, size_t n_rows, int64_t step,
                                    const slide_adamw_hp* hp, int n_threads) {
  using slide::fail;
  if (n_rows == 0 || row_len == 0) return SLIDE_OK;
  const size_t n = row_len * n_rows_total;
  const void* gchk = g ? g : (const void*)p;   // the checks below need a gradient address
  int rc = slide::adamw_check("slide_cpu_adamw_rows", p, gchk, g ? g_dtype : SLIDE_F32, m, v,
                              g ? p_bf16_out : nullptr, n, step, hp);
  if (rc != SLIDE_OK) return rc;
  if (!rows) return fail(SLIDE_E_ARG, "slide_cpu_adamw_rows: null row list");
  if (const long long k = bad_row(rows, n_rows, n_rows_total); k >= 0)
    return fail(SLIDE_E_ARG, "slide_cpu_adamw_rows: row %d (entry %lld) outside [0, %zu) or repeated",
                rows[k], k, n_rows_total);
  const Consts c = make_consts(*hp, step);
  const bool avx512 = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
  const size_t gsz = g_dtype == SLIDE_F32 ? 4 : 2;
  auto work = [&](size_t k0, size_t k1) {
    std::vector<uint16_t> zeros(g ? 0 : row_len, 0);   // bf16 +0.0 widens to +0.0f
    for (size_t k = k0; k < k1; ++k) {
      const size_t o = (size_t)rows[k] * row_len;
      // zero rows: +0.0 in the gradient's 16-bit type (widens to +0.0f), so the copy keeps it
      const void* gr = g ? (const void*)((const char*)g + o * gsz) : (const void*)zeros.data();
      const int gd = g ? g_dtype : (g_dtype == SLIDE_F16 ? SLIDE_F16 : SLIDE_BF16);
      uint16_t* outr = p_bf16_out ? p_bf16_out + o : nullptr;
      if (avx512) range_avx512(p + o, gr, gd, m + o, v + o, outr, 0, row_len, c);
      else range_scalar(p + o, gr, gd, m + o, v + o, outr, 0, row_len, c);
    }
  };
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = (int)std::max<size_t>(1, std::min<size_t>((size_t)nt, (n_rows * row_len + 65535) / 65536));
  nt = (int)std::min<size_t>((size_t)nt, n_rows);
  if (nt == 1) {
    work(0, n_rows);
    return SLIDE_OK;
  }
  parallel_ranges(n_rows, nt, 1, work);
  return SLIDE_OK;
}

// Listed rows whose gradients arrive packed (row k of g_packed belongs to row rows[k]): each row
// runs the element loop of slide_cpu_adamw with the new 16-bit copy written into out_full's
// row, then that row is copied into out_packed's row k (which may be g_packed's, already
// consumed). For fp32 gradients the new fp32 row itself is copied into out_packed.
extern "C" int slide_cpu_adamw_rows_packed(float* p, float* m, float* v, size_t row_len,
                                           size_t n_rows_total, const int32_t* rows,
                                           size_t n_rows, const void* g_packed, int g_dtype,
                                           void* out_full, void* out_packed, int64_t step,
                                           const slide_adamw_hp* hp, int n_threads) {
  using slide::fail;
  if (n_rows == 0 || row_len == 0) return SLIDE_OK;
  int rc = slide::adamw_check("slide_cpu_adamw_rows_packed", p, g_packed, g_dtype, m, v,
                              nullptr, row_len * n_rows, step, hp);
  if (rc != SLIDE_OK) return rc;
  if (!rows) return fail(SLIDE_E_ARG, "slide_cpu_adamw_rows_packed: null row list");
  if (n_rows > n_rows_total)
    return fail(SLIDE_E_ARG, "slide_cpu_adamw_rows_packed: %zu rows of %zu", n_rows,
                n_rows_total);
  const bool g16 = g_dtype != SLIDE_F32;
  if (!g16 && out_full)
    return fail(SLIDE_E_ARG, "slide_cpu_adamw_rows_packed: out_full needs a 16-bit gradient");
  const size_t gsz = g16 ? 2 : 4;
  if (out_packed && out_packed != g_packed) {
    const char* a = (const char*)out_packed;
    const char* b = (const char*)g_packed;
    const size_t nb = n_rows * row_len * gsz;
    if (a < b + nb && b < a + nb)
      return fail(SLIDE_E_ARG, "slide_cpu_adamw_rows_packed: out_packed partially overlaps g");
  }
  if (const long long k = bad_row(rows, n_rows, n_rows_total); k >= 0)
    return fail(SLIDE_E_ARG,
                "slide_cpu_adamw_rows_packed: row %d (entry %lld) outside [0, %zu) or repeated",
                rows[k], k, n_rows_total);
  const Consts c = make_consts(*hp, step);
  const bool avx512 = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
  auto work = [&](size_t k0, size_t k1) {
    std::vector<uint16_t> tmp(g16 && !out_full ? row_len : 0);
    for (size_t k = k0; k < k1; ++k) {
      const size_t o = (size_t)rows[k] * row_len;
      const void* gr = (const char*)g_packed + k * row_len * gsz;
      uint16_t* o16 = nullptr;
      if (g16) o16 = out_full ? (uint16_t*)out_full + o : tmp.data();
      if (avx512) range_avx512(p + o, gr, g_dtype, m + o, v + o, o16, 0, row_len, c);
      else range_scalar(p + o, gr, g_dtype, m + o, v + o, o16, 0, row_len, c);
      if (out_packed) {
        char* dst = (char*)out_packed + k * row_len * gsz;
        if (g16) memcpy(dst, o16, row_len * 2);
        else memcpy(dst, p + o, row_len * 4);
      }
    }
  };
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = (int)std::max<size_t>(1, std::min<size_t>((size_t)nt, (n_rows * row_len + 65535) / 65536));
  nt = (int)std::min<size_t>((size_t)nt, n_rows);
  if (nt == 1) {
    work(0, n_rows);
    return SLIDE_OK;
  }
  parallel_ranges(n_rows, nt, 1, work);
  return SLIDE_OK;
}

// Scalar-only entry used by tests to check that both code paths agree bit for bit.
extern "C" int slide_cpu_adamw_scalar_for_test(float* p, const void* g, int g_dtype, float* m,
                                               float* v, uint16_t* out, size_t n, int64_t step,
                                               const slide_adamw_hp* hp) {
  if (!p || !g || !m || !v || !hp || step < 1) return SLIDE_E_ARG;
  range_scalar(p, g, g_dtype, m, v, out, 0, n, make_consts(*hp, step));
  return SLIDE_OK;
}

extern "C" int slide_cpu_convert_f32(const float* src, void* dst, int dst_dtype, size_t n,
                                     int n_threads) {
  using slide::fail;
  if (n == 0) return SLIDE_OK;
  if (!src || !dst) return fail(SLIDE_E_ARG, "slide_cpu_convert_f32: null pointer");
  if (dst_dtype != SLIDE_BF16 && dst_dtype != SLIDE_F16)
    return fail(SLIDE_E_ARG, "slide_cpu_convert_f32: dst_dtype must be SLIDE_BF16 or SLIDE_F16");
  uint16_t* d = (uint16_t*)dst;
  const bool f16 = dst_dtype == SLIDE_F16;
  auto work = [&](size_t lo, size_t hi) {
    for (size_t i = lo; i < hi; ++i) d[i] = f16 ? f16_rne(src[i]) : bf16_rne(src[i]);
  };
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = (int)std::max<size_t>(1, std::min<size_t>((size_t)nt, (n + 65535) / 65536));
  if (nt == 1) {
    work(0, n);
    return SLIDE_OK;
  }
  parallel_ranges(n, nt, 1, work);
  return SLIDE_OK;
}

// ------------------------------------------------------------------ host-DRAM roofline
// STREAM triad (McCalpin): a[i] = b[i] + s * c[i] over three float arrays, each thread on its
// own contiguous range, 64-byte vector loads and streaming (non-temporal) stores. The arrays
// are mapped with transparent huge pages and first touched by the threads that use them, as
// the optimizer state is. Bytes counted: 12 per element (two reads, one write). The streaming
// stores write a line without reading it first, so the counted bytes are the bytes that move;
// with ordinary stores each written line would also be read (an uncounted third read), while
// the in-place AdamW reads every line it writes anyway.
#include <sys/mman.h>

#include <chrono>

namespace {

__attribute__((target("avx512f"))) void triad_range(float* a, const float* b, const float* c,
                                                    float s, size_t lo, size_t hi) {
  const __m512 sv = _mm512_set1_ps(s);
  size_t i = lo;
  for (; i + 16 <= hi; i += 16)
    _mm512_stream_ps(a + i, _mm512_add_ps(_mm512_load_ps(b + i),
                                          _mm512_mul_ps(sv, _mm512_load_ps(c + i))));
  for (; i < hi; ++i) a[i] = b[i] + s * c[i];
  _mm_sfence();
}

void triad_range_scalar(float* a, const float* b, const float* c, float s, size_t lo, size_t hi) {
  for (size_t i = lo; i < hi; ++i) a[i] = b[i] + s * c[i];
}

}  // namespace

extern "C" int slide_host_triad(size_t n, int n_threads, int reps, double* gbs_best,
                                double* gbs_median) {
  using slide::fail;
  if (n < 16 || reps < 1 || !gbs_best)
    return fail(SLIDE_E_ARG, "slide_host_triad: need n >= 16, reps >= 1 and an output");
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  const size_t bytes = (n * sizeof(float) + 4095) / 4096 * 4096;
  float* arr[3] = {nullptr, nullptr, nullptr};
  for (int k = 0; k < 3; ++k) {
    void* p = mmap(nullptr, bytes, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
    if (p == MAP_FAILED) {
      for (int j = 0; j < k; ++j) munmap(arr[j], bytes);
      return fail(SLIDE_E_ARG, "slide_host_triad: cannot map %zu bytes", bytes);
    }
    madvise(p, bytes, MADV_HUGEPAGE);
    arr[k] = (float*)p;
  }
  size_t per = (n + nt - 1) / nt;
  per = (per + 15) / 16 * 16;
  const bool avx512 = __builtin_cpu_supports("avx512f");
  // the optimizer's helper threads, each on the range it first touched
  auto parallel = [&](auto&& body) {
    parallel_ranges(n, nt, 16, [&](size_t lo, size_t hi) { body(lo, hi); });
  };
  parallel([&](size_t lo, size_t hi) {
    for (size_t i = lo; i < hi; ++i) {
      arr[0][i] = 0.f;
      arr[1][i] = 1.f;
      arr[2][i] = 2.f;
    }
  });
  std::vector<double> rates;
  for (int r = 0; r < reps; ++r) {
    const auto t0 = std::chrono::steady_clock::now();
    parallel([&](size_t lo, size_t hi) {
      if (avx512) triad_range(arr[0], arr[1], arr[2], 3.f, lo, hi);
      else triad_range_scalar(arr[0], arr[1], arr[2], 3.f, lo, hi);
    });
    const double s = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    rates.push_back(12.0 * (double)n / s / 1e9);
  }
  const bool ok = arr[0][n - 1] == 7.f;
  for (int k = 0; k < 3; ++k) munmap(arr[k], bytes);
  if (!ok) return fail(SLIDE_E_STATE, "slide_host_triad: wrong result");
  std::sort(rates.begin(), rates.end());
  *gbs_best = rates.back();
  if (gbs_median) *gbs_median = rates[rates.size() / 2];
  return SLIDE_OK;
}
