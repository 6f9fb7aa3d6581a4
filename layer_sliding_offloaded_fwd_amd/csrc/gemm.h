// GEMM launcher shared by the layer, the LM-head cross-entropy and the C ABI.
#pragma once
#include "common.h"

namespace slide {

enum { EPI_STORE_BF16 = 0, EPI_STORE_F32 = 1, EPI_RESID = 2, EPI_ACCUM_F32 = 3 };

// Call sites of the layer and the LM head. Each site with its usual layout gets its own kernel
// symbol (the site is a template tag with no effect on the code), so that profilers report the
// projections separately; any other combination runs the generic instantiation.
enum GemmSite {
  SITE_GENERIC = 0, SITE_QKV, SITE_O, SITE_GATE_UP, SITE_DOWN,
  SITE_DOWN_DX, SITE_DOWN_DW, SITE_GATE_UP_DX, SITE_GATE_UP_DW, SITE_O_DX, SITE_O_DW,
  SITE_QKV_DX, SITE_QKV_DW, SITE_CE_LOGITS, SITE_CE_DH, SITE_CE_DW
};

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
  int site;          // GemmSite (0 = generic)
};

int gemm_check(const GemmArgs& g);
int gemm_launch(const GemmArgs& g, hipStream_t st);

}  // namespace slide
