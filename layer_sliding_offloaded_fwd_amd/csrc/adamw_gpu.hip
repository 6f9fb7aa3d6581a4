// GPU AdamW with the CPU optimizer's fixed float32 operation order (adamw.cpp), for training
// whose optimizer state stays in HBM: the non-offloaded baseline the pages compare the
// layer-sliding method with (paper page abstract: offloaded training keeps over 95% of the
// performance of training without offloading).
//
// Per element, every operation rounded to nearest-even, no fused multiply-add (this file is
// compiled with -ffp-contract=off; division and square root are the correctly rounded ones):
//   p1 = p*c_dec; m' = c_b1*m + c_1b1*g; v' = c_b2*v + c_1b2*(g*g);
//   den = sqrt(v')/c_bc2 + c_eps; p' = p1 - c_step*(m'/den); bf16 copy = rne(p').
// So the result equals slide_cpu_adamw's bit for bit, and an HBM-resident training step equals
// the offloaded one bit for bit. HBM-bound: 28 bytes per element with a bf16 gradient and copy.
#include "adamw_consts.h"
#include "common.h"

namespace slide {
namespace {

__device__ __forceinline__ uint16_t rne_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// the 16-bit copy: fp16 for an fp16 gradient, bf16 otherwise (both round to nearest-even)
template <int GDT>
__device__ __forceinline__ uint16_t copy16(float f) {
  if constexpr (GDT == SLIDE_F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
  else return rne_bf16(f);
}
template <int GDT>
__device__ __forceinline__ float widen16(uint16_t b) {
  if constexpr (GDT == SLIDE_F16) return (float)__builtin_bit_cast(_Float16, b);
  else return bf2f(b);
}

__device__ __forceinline__ void adam1(float& p, float g, float& m, float& v, const AdamConsts& c) {
  const float p1 = p * c.c_dec;
  const float m2 = c.c_b1 * m + c.c_1b1 * g;
  const float v2 = c.c_b2 * v + c.c_1b2 * (g * g);
  const float den = sqrtf(v2) / c.c_bc2 + c.c_eps;
  p = p1 - c.c_step * (m2 / den);
  m = m2;
  v = v2;
}

// 8 consecutive elements per thread with 16-byte accesses (all pointers 16-byte aligned and
// n8 = n / 8 groups), or one element per thread (scalar = true) for the rest.
template <int GDT, bool SCALAR>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const void* g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    uint16_t* out, size_t lo, size_t n,
                                                    AdamConsts c) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if constexpr (SCALAR) {
    const size_t i = lo + t;
    if (i >= n) return;
    float gi = GDT == SLIDE_F32 ? ((const float*)g)[i] : widen16<GDT>(((const uint16_t*)g)[i]);
    if (c.c_gs != 1.0f) gi = gi * c.c_gs;
    float pi = p[i], mi = m[i], vi = v[i];
    adam1(pi, gi, mi, vi, c);
    p[i] = pi;
    m[i] = mi;
    v[i] = vi;
    if (out) out[i] = copy16<GDT>(pi);
  } else {
    const size_t i = t * 8;
    if (i + 8 > n) return;
    float pp[8], mm[8], vv[8], gg[8];
    *(float4*)&pp[0] = *(const float4*)(p + i);
    *(float4*)&pp[4] = *(const float4*)(p + i + 4);
    *(float4*)&mm[0] = *(const float4*)(m + i);
    *(float4*)&mm[4] = *(const float4*)(m + i + 4);
    *(float4*)&vv[0] = *(const float4*)(v + i);
    *(float4*)&vv[4] = *(const float4*)(v + i + 4);
    if constexpr (GDT != SLIDE_F32) {
      const uint4 gb = *(const uint4*)((const uint16_t*)g + i);
      const uint32_t w[4] = {gb.x, gb.y, gb.z, gb.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        gg[2 * k] = widen16<GDT>((uint16_t)(w[k] & 0xffffu));
        gg[2 * k + 1] = widen16<GDT>((uint16_t)(w[k] >> 16));
      }
    } else {
      *(float4*)&gg[0] = *(const float4*)((const float*)g + i);
      *(float4*)&gg[4] = *(const float4*)((const float*)g + i + 4);
    }
    if (c.c_gs != 1.0f)
#pragma unroll
      for (int k = 0; k < 8; ++k) gg[k] = gg[k] * c.c_gs;
#pragma unroll
    for (int k = 0; k < 8; ++k) adam1(pp[k], gg[k], mm[k], vv[k], c);
    *(float4*)(p + i) = *(float4*)&pp[0];
    *(float4*)(p + i + 4) = *(float4*)&pp[4];
    *(float4*)(m + i) = *(float4*)&mm[0];
    *(float4*)(m + i + 4) = *(float4*)&mm[4];
    *(float4*)(v + i) = *(float4*)&vv[0];
    *(float4*)(v + i + 4) = *(float4*)&vv[4];
    if (out) {
      uint4 o;
      o.x = (uint32_t)copy16<GDT>(pp[0]) | ((uint32_t)copy16<GDT>(pp[1]) << 16);
      o.y = (uint32_t)copy16<GDT>(pp[2]) | ((uint32_t)copy16<GDT>(pp[3]) << 16);
      o.z = (uint32_t)copy16<GDT>(pp[4]) | ((uint32_t)copy16<GDT>(pp[5]) << 16);
      o.w = (uint32_t)copy16<GDT>(pp[6]) | ((uint32_t)copy16<GDT>(pp[7]) << 16);
      *(uint4*)(out + i) = o;
    }
  }
}

template <int GDT>
void launch(float* p, const void* g, float* m, float* v, uint16_t* out, size_t n,
            const AdamConsts& c, hipStream_t st) {
  const bool vec = aligned16(p) && aligned16(g) && aligned16(m) && aligned16(v) &&
                   (!out || aligned16(out));
  size_t done = 0;
  if (vec && n >= 8) {
    const size_t groups = n / 8;
    hipLaunchKernelGGL((adamw_kernel<GDT, false>), dim3((unsigned)((groups + 255) / 256)),
                       dim3(256), 0, st, p, g, m, v, out, (size_t)0, n, c);
    done = groups * 8;
  }
  if (done < n)
    hipLaunchKernelGGL((adamw_kernel<GDT, true>), dim3((unsigned)((n - done + 255) / 256)),
                       dim3(256), 0, st, p, g, m, v, out, done, n, c);
}

}  // namespace
}  // namespace slide

extern "C" int slide_gpu_adamw(float* p, const void* g, int g_dtype, float* m, float* v,
                               uint16_t* p_bf16_out, size_t n, int64_t step,
                               const slide_adamw_hp* hp, void* stream) {
  using namespace slide;
  if (n == 0) return SLIDE_OK;
  SLIDE_TRY(adamw_check("slide_gpu_adamw", p, g, g_dtype, m, v, p_bf16_out, n, step, hp));
  SLIDE_REQUIRE(n / 8 < (size_t)1 << 38, SLIDE_E_SHAPE, "slide_gpu_adamw: n too large");
  const AdamConsts c = adam_consts(*hp, step);
  ProfScope ps("gpu_adamw", (hipStream_t)stream);
  if (g_dtype == SLIDE_BF16)
    launch<SLIDE_BF16>(p, g, m, v, p_bf16_out, n, c, (hipStream_t)stream);
  else if (g_dtype == SLIDE_F16)
    launch<SLIDE_F16>(p, g, m, v, p_bf16_out, n, c, (hipStream_t)stream);
  else
    launch<SLIDE_F32>(p, g, m, v, p_bf16_out, n, c, (hipStream_t)stream);
  return check_launch("slide_gpu_adamw");
}
