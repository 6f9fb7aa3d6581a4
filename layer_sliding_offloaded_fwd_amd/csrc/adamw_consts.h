// Scalar constants of the fixed-order float32 AdamW step, shared by the CPU optimizer
// (adamw.cpp) and its GPU counterpart (adamw_gpu.hip) so that both round them identically.
#pragma once

#include <math.h>
#include <stdint.h>

#include "../../include/slide.h"

namespace slide {

struct AdamConsts {
  float c_dec, c_b1, c_1b1, c_b2, c_1b2, c_step, c_bc2, c_eps;
  float c_gs;   // 1 / grad_scale (the loss scale the gradient was computed at), 1 if unscaled
};

// Computed in double and cast once to float: b1t = beta1^t and b2t = beta2^t by t repeated
// multiplications from 1.0, c_dec = 1 - lr*wd, c_step = lr / (1 - b1t), c_bc2 = sqrt(1 - b2t).
inline AdamConsts adam_consts(const slide_adamw_hp& hp, int64_t t) {
  double b1t = 1.0, b2t = 1.0;
  for (int64_t i = 0; i < t; ++i) {
    b1t *= hp.beta1;
    b2t *= hp.beta2;
  }
  AdamConsts c;
  c.c_dec = (float)(1.0 - hp.lr * hp.weight_decay);
  c.c_b1 = (float)hp.beta1;
  c.c_1b1 = (float)(1.0 - hp.beta1);
  c.c_b2 = (float)hp.beta2;
  c.c_1b2 = (float)(1.0 - hp.beta2);
  c.c_step = (float)(hp.lr / (1.0 - b1t));
  c.c_bc2 = (float)sqrt(1.0 - b2t);
  c.c_eps = (float)hp.eps;
  c.c_gs = (float)(1.0 / (hp.grad_scale > 0 ? hp.grad_scale : 1.0));
  return c;
}

// Argument checks common to both optimizers (0 when valid, else a SLIDE_E_* code with the
// message left in slide_last_error()).
int adamw_check(const char* who, const void* p, const void* g, int g_dtype, const void* m,
                const void* v, const void* p_bf16_out, size_t n, int64_t step,
                const slide_adamw_hp* hp);

}  // namespace slide
