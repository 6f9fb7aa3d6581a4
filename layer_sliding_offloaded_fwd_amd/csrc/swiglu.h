// SwiGLU of the decoder MLP, m = silu(g) * u with silu(g) = g * sigmoid(g), and its derivatives
// (An Efficient Heterogeneous Co-Design for Fine-Tuning on a Single GPU: the Llama-style decoder
// layer whose MLP the method trains). One definition for the elementwise kernels and the GEMM
// epilogues that fuse them, so that both give the same bits.
#pragma once
#include "common.h"

namespace slide {

__device__ __forceinline__ float swiglu_sigmoid(float a) { return 1.0f / (1.0f + __expf(-a)); }

// The results leave as fp32 values: without this the compiler folds a final multiply and the
// narrowing to fp16 into one mixed-precision FMA (one rounding instead of two) in some callers
// and not in others, and the fused and separate kernels would disagree in the last bit.
__device__ __forceinline__ float swiglu_out(float x) {
  asm("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float swiglu_fwd_1(float g, float u) {
  return swiglu_out(g * swiglu_sigmoid(g) * u);
}

// dm -> (dg, du)
__device__ __forceinline__ void swiglu_bwd_1(float d, float g, float u, float& dg, float& du) {
  const float sg = swiglu_sigmoid(g);
  du = swiglu_out(d * g * sg);
  dg = swiglu_out(d * u * sg * (1.0f + g * (1.0f - sg)));
}

}  // namespace slide
