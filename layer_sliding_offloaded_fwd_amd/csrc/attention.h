// Launchers of the causal GQA attention kernels.
#pragma once
#include "common.h"

namespace slide {

int attention_check(int B, int S, int nq, int nkv, int d, int dtype);
int attention_fwd(const void* qkv, void* o, float* lse, int B, int S, int nq, int nkv, int d,
                  int dtype, hipStream_t st);
size_t attention_bwd_ws(int B, int S, int nq);
int attention_bwd(const void* qkv, const void* o, const float* lse, const void* dout, void* dqkv,
                  int B, int S, int nq, int nkv, int d, int dtype, void* ws, hipStream_t st);

}  // namespace slide
