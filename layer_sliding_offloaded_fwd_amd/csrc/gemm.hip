// GEMMs of the decoder layer and the LM head (projections y = x W^T, their input gradients
// dX = dY W and weight gradients dW = dY^T X).
//
// bf16 path: gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation. One workgroup of 256
// threads (4 waves, 2x2) computes a 128x128 tile of C; each wave owns 64x64 = 2x2 MFMA blocks.
// K is consumed in 64-wide tiles staged through LDS (double buffered: the next tile is fetched
// into registers while the current one feeds the MFMAs). In LDS both operands are stored
// K-contiguous, one 128-byte row (64 bf16) per M (or N) index, with the 16-byte chunk index
// XOR-swizzled by (row + row/8) & 7 so that both the MFMA reads (8 consecutive rows, same chunk)
// and the transposed writes (8 rows spaced 8 apart) hit distinct banks. An operand whose K is
// the outer dimension in memory (dW = dY^T X, dX = dY W) is loaded as 8x8 blocks and transposed
// in registers before the LDS write, so every layout shares the same inner loop.
// fp32 path (the small fp32 configuration): a plain LDS-tiled SIMT kernel, 64x64 per workgroup.
#include "gemm.h"

namespace slide {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

namespace {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;

__device__ __forceinline__ int swz(int r) { return (r + (r >> 3)) & 7; }
// element offset of (row, 16-byte chunk) in a [rows][64] bf16 LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

// ---- K-major operand: rows x 64 k, 16-byte chunks, 4 per thread
__device__ __forceinline__ void load_kmajor(uint4 (&reg)[4], const bf16_t* __restrict__ P, int ld,
                                            int row0, int rows_total, int k0, int K) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int id = t + NT * i;
    int r = id >> 3, c = id & 7;
    int gr = row0 + r, gk = k0 + c * 8;
    if (gr < rows_total && gk < K)
      reg[i] = *(const uint4*)(P + (size_t)gr * ld + gk);
    else
      reg[i] = make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void store_kmajor(const uint4 (&reg)[4], bf16_t* s) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int id = t + NT * i;
    int r = id >> 3, c = id & 7;
    *(uint4*)(s + lds_off(r, c)) = reg[i];
  }
}

// ---- outer-K operand: memory holds [k][row], row contiguous. Thread t < 128 owns the 8x8
// block (k-block kb = t/16, row-block rb = t%16) and transposes it in registers.
__device__ __forceinline__ void load_outerk(uint4 (&reg)[8], const bf16_t* __restrict__ P, int ld,
                                            int row0, int rows_total, int k0, int K) {
  const int t = threadIdx.x;
  if (t >= 128) return;
  int kb = t >> 4, rb = t & 15;
  int gr = row0 + rb * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int gk = k0 + kb * 8 + j;
    if (gr < rows_total && gk < K)
      reg[j] = *(const uint4*)(P + (size_t)gk * ld + gr);
    else
      reg[j] = make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ uint32_t dw(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ void store_outerk(const uint4 (&reg)[8], bf16_t* s) {
  const int t = threadIdx.x;
  if (t >= 128) return;
  int kb = t >> 4, rb = t & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // row rb*8+i gets k = kb*8 .. kb*8+7: dword w = (k=2w, k=2w+1) from element i of v[2w], v[2w+1]
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o0 = __builtin_amdgcn_perm(dw(reg[1], i >> 1), dw(reg[0], i >> 1), sel);
    uint32_t o1 = __builtin_amdgcn_perm(dw(reg[3], i >> 1), dw(reg[2], i >> 1), sel);
    uint32_t o2 = __builtin_amdgcn_perm(dw(reg[5], i >> 1), dw(reg[4], i >> 1), sel);
    uint32_t o3 = __builtin_amdgcn_perm(dw(reg[7], i >> 1), dw(reg[6], i >> 1), sel);
    *(uint4*)(s + lds_off(rb * 8 + i, kb)) = make_uint4(o0, o1, o2, o3);
  }
}

template <bool AK, bool BKM, int EPI, int SITE>
__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];

  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  // XCD-aware order: workgroup w runs on XCD w % 8; give each XCD a contiguous range of
  // logical tiles so the tiles sharing A rows / B columns share that XCD's L2.
  int wg = blockIdx.x, nwg = gridDim.x, logical = wg;
  if ((nwg & 7) == 0) logical = (wg & 7) * (nwg >> 3) + (wg >> 3);
  constexpr int GM = 8;
  int group = logical / (GM * tiles_n);
  int first_m = group * GM;
  int gsize = min(tiles_m - first_m, GM);
  int in_group = logical % (GM * tiles_n);
  int tm = first_m + in_group % gsize, tn = in_group / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16_t* A = (const bf16_t*)g.A;
  const bf16_t* B = (const bf16_t*)g.B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint4 ra[AK ? 4 : 8], rb[BKM ? 4 : 8];
  auto gload = [&](int k0) {
    if constexpr (AK) load_kmajor(ra, A, g.lda, m0, g.M, k0, g.K);
    else load_outerk(ra, A, g.lda, m0, g.M, k0, g.K);
    if constexpr (BKM) load_kmajor(rb, B, g.ldb, n0, g.N, k0, g.K);
    else load_outerk(rb, B, g.ldb, n0, g.N, k0, g.K);
  };
  auto lstore = [&](int buf) {
    if constexpr (AK) store_kmajor(ra, sA[buf]);
    else store_outerk(ra, sA[buf]);
    if constexpr (BKM) store_kmajor(rb, sB[buf]);
    else store_outerk(rb, sB[buf]);
  };

  const int nk = (g.K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const bf16_t* a_s = sA[cur];
    const bf16_t* b_s = sB[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int r = wm * 64 + i * 32 + (lane & 31);
        af[i] = *(const bf16x8_t*)(a_s + lds_off(r, ch));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int r = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *(const bf16x8_t*)(b_s + lds_off(r, ch));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: acc[i][j][e] is C(row, col) with col = lane%32, row = (e/4)*8 + (lane/32)*4 + e%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= g.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row >= g.M) continue;
        float v = acc[i][j][e] * g.alpha;
        if constexpr (EPI == EPI_STORE_BF16) {
          ((bf16_t*)g.C)[(size_t)row * g.ldc + col] = f2bf(v);
        } else if constexpr (EPI == EPI_STORE_F32) {
          ((float*)g.C)[(size_t)row * g.ldc + col] = v;
        } else if constexpr (EPI == EPI_RESID) {
          v += bf2f(((const bf16_t*)g.R)[(size_t)row * g.ldr + col]);
          ((bf16_t*)g.C)[(size_t)row * g.ldc + col] = f2bf(v);
        } else {  // EPI_ACCUM_F32
          float* c = (float*)g.C + (size_t)row * g.ldc + col;
          *c = *c + v;
        }
      }
    }
}

// ------------------------------------------------------------------ fp32 SIMT GEMM
constexpr int SB = 64, SK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float sA[SK][SB + 1];
  __shared__ float sB[SK][SB + 1];
  const float* A = (const float*)g.A;
  const float* B = (const float*)g.B;
  const int m0 = blockIdx.y * SB, n0 = blockIdx.x * SB;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += SK) {
    for (int idx = threadIdx.x; idx < SB * SK; idx += 256) {
      int r = idx / SK, k = idx % SK;  // used for k-major loads
      int r2 = idx % SB, k2 = idx / SB;  // used for outer-k loads (coalesced along rows)
      {
        int rr = g.a_kmajor ? r : r2, kk = g.a_kmajor ? k : k2;
        int gm = m0 + rr, gk = k0 + kk;
        float v = 0.f;
        if (gm < g.M && gk < g.K)
          v = g.a_kmajor ? A[(size_t)gm * g.lda + gk] : A[(size_t)gk * g.lda + gm];
        sA[kk][rr] = v;
      }
      {
        int rr = g.b_kmajor ? r : r2, kk = g.b_kmajor ? k : k2;
        int gn = n0 + rr, gk = k0 + kk;
        float v = 0.f;
        if (gn < g.N && gk < g.K)
          v = g.b_kmajor ? B[(size_t)gn * g.ldb + gk] : B[(size_t)gk * g.ldb + gn];
        sB[kk][rr] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int row = m0 + ty * 4 + i;
    if (row >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int col = n0 + tx * 4 + j;
      if (col >= g.N) continue;
      float v = acc[i][j] * g.alpha;
      if constexpr (EPI == EPI_RESID) {
        v += ((const float*)g.R)[(size_t)row * g.ldr + col];
        ((float*)g.C)[(size_t)row * g.ldc + col] = v;
      } else if constexpr (EPI == EPI_ACCUM_F32) {
        float* c = (float*)g.C + (size_t)row * g.ldc + col;
        *c = *c + v;
      } else {
        ((float*)g.C)[(size_t)row * g.ldc + col] = v;
      }
    }
  }
}

template <bool AK, bool BKM, int EPI, int SITE>
void launch_one(const GemmArgs& g, hipStream_t st) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, EPI, SITE>), dim3(tiles), dim3(NT), 0, st, g);
}

template <bool AK, bool BKM>
void launch_generic(const GemmArgs& g, hipStream_t st, int epi) {
  switch (epi) {
    case EPI_STORE_BF16: launch_one<AK, BKM, EPI_STORE_BF16, SITE_GENERIC>(g, st); break;
    case EPI_STORE_F32: launch_one<AK, BKM, EPI_STORE_F32, SITE_GENERIC>(g, st); break;
    case EPI_RESID: launch_one<AK, BKM, EPI_RESID, SITE_GENERIC>(g, st); break;
    default: launch_one<AK, BKM, EPI_ACCUM_F32, SITE_GENERIC>(g, st); break;
  }
}

// (site, a_kmajor, b_kmajor, epilogue) -> dedicated instantiation, else generic
void launch_bf16(const GemmArgs& g, hipStream_t st, int epi) {
#define SLIDE_SITE(S, AK_, BK_, EPI_)                                              \
  if (g.site == S && g.a_kmajor == AK_ && g.b_kmajor == BK_ && epi == EPI_) {    \
    launch_one<AK_, BK_, EPI_, S>(g, st);                                        \
    return;                                                                      \
  }
  SLIDE_SITE(SITE_QKV, true, true, EPI_STORE_BF16)
  SLIDE_SITE(SITE_O, true, true, EPI_RESID)
  SLIDE_SITE(SITE_GATE_UP, true, true, EPI_STORE_BF16)
  SLIDE_SITE(SITE_DOWN, true, true, EPI_RESID)
  SLIDE_SITE(SITE_DOWN_DX, true, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_DOWN_DW, false, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_GATE_UP_DX, true, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_GATE_UP_DW, false, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_O_DX, true, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_O_DW, false, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_QKV_DX, true, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_QKV_DW, false, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_CE_LOGITS, true, true, EPI_STORE_F32)
  SLIDE_SITE(SITE_CE_DH, false, false, EPI_ACCUM_F32)
  SLIDE_SITE(SITE_CE_DW, true, false, EPI_STORE_BF16)
#undef SLIDE_SITE
  if (g.a_kmajor && g.b_kmajor) launch_generic<true, true>(g, st, epi);
  else if (g.a_kmajor) launch_generic<true, false>(g, st, epi);
  else if (g.b_kmajor) launch_generic<false, true>(g, st, epi);
  else launch_generic<false, false>(g, st, epi);
}

}  // namespace

int gemm_epilogue_of(const GemmArgs& g) {
  if (g.accumulate) return EPI_ACCUM_F32;
  if (g.R) return EPI_RESID;
  return g.c_dtype == SLIDE_F32 ? EPI_STORE_F32 : EPI_STORE_BF16;
}

int gemm_check(const GemmArgs& g) {
  SLIDE_REQUIRE(g.M >= 0 && g.N >= 0 && g.K >= 0, SLIDE_E_SHAPE, "gemm: negative size");
  SLIDE_REQUIRE(g.A && g.B && g.C, SLIDE_E_ARG, "gemm: null operand");
  SLIDE_REQUIRE(g.dtype == SLIDE_BF16 || g.dtype == SLIDE_F32, SLIDE_E_ARG, "gemm: bad dtype");
  SLIDE_REQUIRE(!g.accumulate || g.c_dtype == SLIDE_F32, SLIDE_E_ARG,
                "gemm: accumulate needs an fp32 C");
  SLIDE_REQUIRE(!(g.accumulate && g.R), SLIDE_E_ARG, "gemm: residual and accumulate are exclusive");
  SLIDE_REQUIRE(!g.R || g.c_dtype == g.dtype, SLIDE_E_ARG, "gemm: residual output must be in dtype");
  SLIDE_REQUIRE(g.lda >= (g.a_kmajor ? g.K : g.M) && g.ldb >= (g.b_kmajor ? g.K : g.N) &&
                    g.ldc >= g.N && (!g.R || g.ldr >= g.N),
                SLIDE_E_SHAPE, "gemm: leading dimension smaller than the row");
  if (g.dtype == SLIDE_BF16) {
    SLIDE_REQUIRE(aligned16(g.A) && aligned16(g.B), SLIDE_E_ARG, "gemm: operands must be 16-byte aligned");
    SLIDE_REQUIRE(g.lda % 8 == 0 && g.ldb % 8 == 0, SLIDE_E_SHAPE, "gemm: lda/ldb must be multiples of 8");
    // 16-byte vector loads: a K-contiguous operand needs K % 8 == 0; an operand whose rows run
    // along M (or N) may be ragged as long as the padded row fits its leading dimension.
    auto r8 = [](int v) { return (v + 7) / 8 * 8; };
    SLIDE_REQUIRE((g.a_kmajor ? g.K % 8 == 0 : g.lda >= r8(g.M)) &&
                      (g.b_kmajor ? g.K % 8 == 0 : g.ldb >= r8(g.N)),
                  SLIDE_E_SHAPE, "gemm: K must be a multiple of 8 for a K-contiguous operand, "
                  "and ld >= M (N) rounded up to 8 otherwise");
    SLIDE_REQUIRE(g.c_dtype == SLIDE_BF16 || g.c_dtype == SLIDE_F32, SLIDE_E_ARG, "gemm: bad c_dtype");
  } else {
    SLIDE_REQUIRE(g.c_dtype == SLIDE_F32, SLIDE_E_ARG, "gemm: fp32 operands need an fp32 C");
  }
  return SLIDE_OK;
}

int gemm_launch(const GemmArgs& g, hipStream_t st) {
  if (g.M == 0 || g.N == 0) return SLIDE_OK;
  ProfScope ps(g.name ? g.name : "gemm", st);
  const int epi = gemm_epilogue_of(g);
  if (g.dtype == SLIDE_BF16) {
    launch_bf16(g, st, epi);
  } else {
    dim3 grid((g.N + SB - 1) / SB, (g.M + SB - 1) / SB), block(256);
    switch (epi) {
      case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, block, 0, st, g); break;
      case EPI_ACCUM_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_ACCUM_F32>, grid, block, 0, st, g); break;
      default: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE_F32>, grid, block, 0, st, g); break;
    }
  }
  return check_launch(g.name ? g.name : "gemm");
}

}  // namespace slide

extern "C" int slide_gemm(int M, int N, int K, const void* A, int lda, int a_kmajor, const void* B,
                          int ldb, int b_kmajor, void* C, int ldc, int c_dtype, const void* R,
                          int ldr, float alpha, int accumulate, int dtype, void* stream) {
  slide::GemmArgs g{M, N, K, A, lda, a_kmajor != 0, B, ldb, b_kmajor != 0, C, ldc, c_dtype,
                    R, ldr, alpha, accumulate != 0, dtype, "gemm", slide::SITE_GENERIC};
  SLIDE_TRY(slide::gemm_check(g));
  return slide::gemm_launch(g, (hipStream_t)stream);
}
