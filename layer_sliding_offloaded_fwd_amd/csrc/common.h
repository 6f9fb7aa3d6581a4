// Internal helpers shared by the HIP kernels and the C-ABI glue of libslide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/slide.h"

namespace slide {

// ---------------------------------------------------------------- errors (thread-local)
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char* what);  // hipGetLastError -> SLIDE_E_HIP with a message

#define SLIDE_REQUIRE(cond, code, ...)                 \
  do {                                                 \
    if (!(cond)) return ::slide::fail((code), __VA_ARGS__); \
  } while (0)

#define SLIDE_TRY(expr)                \
  do {                                 \
    int _rc = (expr);                  \
    if (_rc != SLIDE_OK) return _rc;   \
  } while (0)

// ---------------------------------------------------------------- kernel timing
// Brackets a launch with events on `stream` when profiling is on (no-op otherwise).
struct ProfScope {
  ProfScope(const char* name, hipStream_t stream);
  ~ProfScope();
  int slot = -1;
  hipStream_t stream;
};

// ---------------------------------------------------------------- element types
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float -> bf16, round to nearest-even (gfx950 v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Load/store one element of either storage type as float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f2bf(v); }
};

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

inline bool aligned16(const void* p) { return (((uintptr_t)p) & 15u) == 0; }
inline int dtype_size(int dt) { return dt == SLIDE_BF16 ? 2 : 4; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Carves consecutive 256-byte aligned regions out of a caller workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T> T* take(size_t count) {
    used = align_up(used, 256);
    T* p = (T*)(base ? base + used : nullptr);
    used += count * sizeof(T);
    return p;
  }
};

}  // namespace slide
