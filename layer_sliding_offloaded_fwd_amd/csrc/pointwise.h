// Launchers of the memory-bound kernels (RMSNorm, RoPE, SwiGLU, embedding, helpers).
#pragma once
#include <algorithm>

#include "common.h"

namespace slide {

constexpr int kRmsRowsPerPart = 64;  // rows per partial sum of the RMSNorm weight gradient

int rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd, int N, int H, float eps,
                int dtype, hipStream_t st);
size_t rmsnorm_bwd_ws(int N, int H);
// dx = dres + RMSNorm backward of dy; dres may alias dx, dy must not. dw may be null.
int rmsnorm_bwd(const void* dy, const void* x, const void* w, const void* dres, void* dx,
                void* dw, int N, int H, float eps, int dtype, void* ws, hipStream_t st);
int rope_tables(float* cos_t, float* sin_t, int S, int d, float theta, hipStream_t st);
int rope_apply(void* qkv, const float* cos_t, const float* sin_t, int B, int S, int nq, int nkv,
               int d, int inverse, int dtype, hipStream_t st);
int swiglu_fwd(const void* gu, void* m, int N, int F, int dtype, hipStream_t st);
int swiglu_bwd(const void* dm, const void* gu, void* dgu, int N, int F, int dtype,
               hipStream_t st);
int embed_fwd(const void* E, const int32_t* tok, void* x, int N, int H, int V, int dtype,
              hipStream_t st);
size_t embed_bwd_ws(int N, int V);
// dst row (dst_rows ? dst_rows[k] : k) = src row (src_rows ? src_rows[k] : k), k < n_rows;
// rows of row_bytes (a multiple of 16); a pair with an index outside [0, src_n) or
// [0, dst_n) is skipped
int copy_rows(const void* src, const int32_t* src_rows, long long src_n, void* dst,
              const int32_t* dst_rows, long long dst_n, long long n_rows, size_t row_bytes,
              hipStream_t st);
int embed_bwd(const void* dx, const int32_t* tok, void* dE, int N, int H, int V, int dtype,
              void* ws, hipStream_t st);
// *count (device) = number of NaN or infinite elements of x[n]
int nonfinite_count(const void* x, size_t n, int dtype, uint32_t* count, hipStream_t st);
int fill_f32(float* p, size_t n, float v, hipStream_t st);
int fill_zero(void* p, size_t n, int dtype, hipStream_t st);
int convert_from_f32(const float* src, void* dst, size_t n, int dtype, hipStream_t st);

}  // namespace slide
