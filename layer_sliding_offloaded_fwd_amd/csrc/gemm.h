// GEMM launcher shared by the layer, the LM-head cross-entropy and the C ABI.
#pragma once
#include "common.h"

namespace slide {

enum { EPI_STORE_BF16 = 0, EPI_STORE_F32 = 1, EPI_RESID = 2, EPI_ACCUM_F32 = 3 };

// C[M,N] = alpha * A(m,k) B(k,n) (+ R) (or C += ... when accumulate); see slide_gemm in slide.h.
struct GemmArgs {
  int M, N, K;
  const void* A;
  int lda;
  bool a_kmajor;
  const void* B;
  int ldb;
  bool b_kmajor;
  void* C;
  int ldc;
  int c_dtype;
  const void* R;
  int ldr;
  float alpha;
  bool accumulate;
  int dtype;
  const char* name;  // kernel-timer label
};

int gemm_check(const GemmArgs& g);
int gemm_launch(const GemmArgs& g, hipStream_t st);

}  // namespace slide
