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
// bf16 is handled as its uint16 bit pattern; fp16 (SLIDE_F16) as the compiler's _Float16, a
// distinct type, so that kernels templated on the storage type tell the two apart.
typedef uint16_t bf16_t;
typedef _Float16 f16_t;

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
template <> struct Elem<f16_t> {
  __device__ __forceinline__ static float load(const f16_t* p) { return (float)*p; }
  __device__ __forceinline__ static void store(f16_t* p, float v) { *p = (f16_t)v; }  // RNE
};

// 16-bit storage codes as bit patterns (for kernels that move raw 16-bit words):
// to_f widens exactly, from_f rounds to nearest-even (NaN stays NaN).
template <int DT> struct Bits16;
template <> struct Bits16<SLIDE_BF16> {
  __device__ __forceinline__ static float to_f(uint16_t b) { return bf2f(b); }
  __device__ __forceinline__ static uint16_t from_f(float f) { return f2bf(f); }
};
template <> struct Bits16<SLIDE_F16> {
  __device__ __forceinline__ static float to_f(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  __device__ __forceinline__ static uint16_t from_f(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
};

// ---------------------------------------------------------------- MFMA operands
// 8 x 16-bit MFMA operand per lane (moved as raw words; DT says how the MFMA reads them) and the
// 32x32 fp32 accumulator block.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// One v_mfma_f32_32x32x16 on bf16 (DT = SLIDE_BF16) or fp16 (DT = SLIDE_F16) operands.
template <int DT>
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  if constexpr (DT == SLIDE_F16) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a),
                                                  __builtin_bit_cast(h8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
}

// 8 floats rounded (nearest-even) to an MFMA operand of type DT.
template <int DT>
__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  if constexpr (DT == SLIDE_F16) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 r = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3],
            (_Float16)v[4], (_Float16)v[5], (_Float16)v[6], (_Float16)v[7]};
    return __builtin_bit_cast(bf16x8_t, r);
  } else {
    bf16x8_t r = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3],
                  (__bf16)v[4], (__bf16)v[5], (__bf16)v[6], (__bf16)v[7]};
    return r;
  }
}

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
inline int dtype_size(int dt) { return dt == SLIDE_F32 ? 4 : 2; }
inline bool dtype_valid(int dt) { return dt == SLIDE_F32 || dt == SLIDE_BF16 || dt == SLIDE_F16; }

// Run `...` with T the storage type of dtype (float, bf16_t or f16_t).
#define SLIDE_DISPATCH(dtype, T, ...)            \
  switch (dtype) {                               \
    case SLIDE_BF16: {                           \
      typedef ::slide::bf16_t T;                 \
      __VA_ARGS__;                               \
    } break;                                     \
    case SLIDE_F16: {                            \
      typedef ::slide::f16_t T;                  \
      __VA_ARGS__;                               \
    } break;                                     \
    default: {                                   \
      typedef float T;                           \
      __VA_ARGS__;                               \
    } break;                                     \
  }
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
