// GEMMs of the decoder layer and the LM head (projections y = x W^T, their input gradients
// dX = dY W and weight gradients dW = dY^T X).
//
// 16-bit path (bf16 or fp16 operands): gfx950 MFMA v_mfma_f32_32x32x16_bf16 / _f16, fp32
// accumulation, two kernels:
//   pipelined (problems with at least 128 tiles of 256 x 256, i.e. every projection of the
//     step): 256 x 256 tile, 8 waves, k-tiles streamed global -> LDS by direct loads; see the
//     comment above gemm_pipe_kernel.
//   register-staged (smaller problems): 128 x 128 tile, 4 waves (2 x 2), wave tile 64 x 64,
//     K consumed in 64-wide tiles staged through registers into LDS (double buffered, one
//     barrier per tile). Both operands are stored K-contiguous in LDS, one 128-byte row per M
//     (or N) index, the 16-byte chunk index XOR-swizzled by (row + row/8) & 7 so that both the
//     MFMA reads (8 consecutive rows, same chunk) and the transposed writes (8 rows spaced 8
//     apart) hit distinct banks. An operand whose K is the outer dimension in memory is loaded as
//     8x8 blocks and transposed in registers before the LDS write.
// Tiles are ordered XCD-aware and grouped along M for L2 reuse.
// fp32 path (the small fp32 configuration): a plain LDS-tiled SIMT kernel, 64x64 per workgroup.
#include <atomic>

#include "gemm.h"
#include "pointwise.h"
#include "swiglu.h"

namespace slide {

namespace {

// the two 16-bit values of a 32-bit word, widened
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) { return Bits16<DT>::to_f((uint16_t)(w & 0xffffu)); }
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) { return Bits16<DT>::to_f((uint16_t)(w >> 16)); }
template <int DT>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  return (uint32_t)Bits16<DT>::from_f(a) | ((uint32_t)Bits16<DT>::from_f(b) << 16);
}

constexpr int BK = 64;

__device__ __forceinline__ int swz(int r) { return (r + (r >> 3)) & 7; }
// element offset of (row, 16-byte chunk) in a [rows][64] bf16 LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

__device__ __forceinline__ uint32_t dw(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Epilogue of a wave tile of MI x NJ 32x32 MFMA blocks whose top-left element is (rw0, cw0):
// acc[i][j][e] is C(row, col) with col = cw0 + 32 j + lane%32,
// row = rw0 + 32 i + (e/4)*8 + (lane/32)*4 + e%4.
template <int EPI, int MI, int NJ, int DT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, f32x16_t (&acc)[MI][NJ],
                                              int rw0, int cw0, int lane) {
  if constexpr (EPI == EPI_CE_STATS) {
    static_assert((MI * 32) % kCeRowsPerPart == 0, "whole row blocks per wave");
    constexpr int PARTS = MI * 32 / kCeRowsPerPart;
    const int hl = lane >> 5;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = cw0 + j * 32 + (lane & 31);
      const bool cok = col < g.N;
      const int y = cok ? g.tgt[col] - g.c0 : -1;
#pragma unroll
      for (int p = 0; p < PARTS; ++p) {
        // rows of part p: blocks i in [p * MI / PARTS, (p + 1) * MI / PARTS)
        float m = -INFINITY;
#pragma unroll
        for (int i = p * MI / PARTS; i < (p + 1) * MI / PARTS; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = rw0 + i * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
            const float v = acc[i][j][e] * g.alpha;
            if (row < g.M) m = fmaxf(m, v);
            if (row == y && row < g.M) g.zt[col] = v;
          }
        float s = 0.f;
        if (m != -INFINITY) {
#pragma unroll
          for (int i = p * MI / PARTS; i < (p + 1) * MI / PARTS; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int row = rw0 + i * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
              if (row < g.M) s += __expf(acc[i][j][e] * g.alpha - m);
            }
        }
        // combine with the other half of the rows (lane +- 32)
        const float m2 = __shfl_xor(m, 32, 64), s2 = __shfl_xor(s, 32, 64);
        const float mm = fmaxf(m, m2);
        float ss = 0.f;
        if (mm != -INFINITY) ss = s * __expf(m - mm) + s2 * __expf(m2 - mm);
        if (hl == 0 && cok) {
          const size_t at = (size_t)((rw0 + p * kCeRowsPerPart) / kCeRowsPerPart) * g.N + col;
          g.pm[at] = mm;
          g.ps[at] = ss;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = cw0 + j * 32 + (lane & 31);
        if constexpr (EPI == EPI_CE_DZ) {
          if (col >= g.ldc) continue;
        } else {
          if (col >= g.N) continue;
        }
        float dzs = 0.f, lse_t = 0.f;
        int y = -1;
        if constexpr (EPI == EPI_CE_DZ) {
          if (col < g.N) {
            const int yt = g.tgt[col];
            if (yt >= 0 && yt < g.V) {
              y = yt;
              lse_t = g.lse[col];
              dzs = *g.inv_nv;
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rw0 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          if (row >= g.M) continue;
          float v = acc[i][j][e] * g.alpha;
          if constexpr (EPI == EPI_STORE_BF16) {
            ((bf16_t*)g.C)[(size_t)row * g.ldc + col] = Bits16<DT>::from_f(v);
          } else if constexpr (EPI == EPI_STORE_F32) {
            ((float*)g.C)[(size_t)row * g.ldc + col] = v;
          } else if constexpr (EPI == EPI_RESID) {
            v += Bits16<DT>::to_f(((const bf16_t*)g.R)[(size_t)row * g.ldr + col]);
            ((bf16_t*)g.C)[(size_t)row * g.ldc + col] = Bits16<DT>::from_f(v);
          } else if constexpr (EPI == EPI_ACCUM_F32) {
            float* c = (float*)g.C + (size_t)row * g.ldc + col;
            *c = *c + v;
          } else {  // EPI_CE_DZ
            float d = 0.f;
            if (y >= 0) {
              d = __expf(v - lse_t);
              if (g.c0 + row == y) d -= 1.f;
              d *= dzs;
            }
            if (g.c_dtype != SLIDE_F32) ((bf16_t*)g.C)[(size_t)row * g.ldc + col] = Bits16<DT>::from_f(d);
            else ((float*)g.C)[(size_t)row * g.ldc + col] = d;
          }
        }
      }
  }
}

// Operand staging. Threads [0, NT/2) stage the A tile and threads [NT/2, NT) the B tile, each
// through the same 8 x 16-byte registers: a K-major operand (memory row = M or N index) as 8
// chunks per thread (8 consecutive threads cover one 128-byte row segment), an outer-K operand
// (memory holds [k][row]) as one 8x8 block per thread (k-block kb, row-block rb), transposed in
// registers before the LDS write. Requires ROWS * 8 == 8 * (NT / 2), i.e. ROWS == NT / 2.
struct Stage {
  uint4 r[8];

  template <int ROWS, bool KMAJ>
  __device__ __forceinline__ void load(int u, const bf16_t* __restrict__ P, int ld, int row0,
                                       int rows_total, int k0, int K) {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = u + ROWS * i;
        const int rr = id >> 3, c = id & 7;
        const int gr = row0 + rr, gk = k0 + c * 8;
        r[i] = (gr < rows_total && gk < K) ? *(const uint4*)(P + (size_t)gr * ld + gk)
                                           : make_uint4(0, 0, 0, 0);
      }
    } else {
      const int kb = u / (ROWS / 8), rb = u % (ROWS / 8);
      const int gr = row0 + rb * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        r[j] = (gr < rows_total && gk < K) ? *(const uint4*)(P + (size_t)gk * ld + gr)
                                           : make_uint4(0, 0, 0, 0);
      }
    }
  }

  template <int ROWS, bool KMAJ>
  __device__ __forceinline__ void store(int u, bf16_t* s) const {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = u + ROWS * i;
        *(uint4*)(s + lds_off(id >> 3, id & 7)) = r[i];
      }
    } else {
      const int kb = u / (ROWS / 8), rb = u % (ROWS / 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // row rb*8+i gets k = kb*8 .. kb*8+7: dword w = (k=2w, k=2w+1), element i of r[2w], r[2w+1]
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t o0 = __builtin_amdgcn_perm(dw(r[1], i >> 1), dw(r[0], i >> 1), sel);
        const uint32_t o1 = __builtin_amdgcn_perm(dw(r[3], i >> 1), dw(r[2], i >> 1), sel);
        const uint32_t o2 = __builtin_amdgcn_perm(dw(r[5], i >> 1), dw(r[4], i >> 1), sel);
        const uint32_t o3 = __builtin_amdgcn_perm(dw(r[7], i >> 1), dw(r[6], i >> 1), sel);
        *(uint4*)(s + lds_off(rb * 8 + i, kb)) = make_uint4(o0, o1, o2, o3);
      }
    }
  }
};

template <int BM_, int BN_, int NT_, int WGM_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, NT = NT_, WGM = WGM_;
  static constexpr int NW = NT / 64, WGN = NW / WGM;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
  static constexpr int MI = WTM / 32, NJ = WTN / 32;     // 32x32 MFMA blocks per wave
};
using TileS = Tile<128, 128, 256, 2>;

template <class TL, bool AK, bool BKM, int EPI, int SITE, int DT>
__global__ __launch_bounds__(TL::NT, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BN = TL::BN, NT = TL::NT, MI = TL::MI, NJ = TL::NJ;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];

  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  // XCD-aware order: workgroup w runs on XCD w % 8; give each XCD a contiguous range of
  // logical tiles so the tiles sharing A rows / B columns share that XCD's L2.
  int wg = blockIdx.x, nwg = gridDim.x, logical = wg;
  if ((nwg & 7) == 0) logical = (wg & 7) * (nwg >> 3) + (wg >> 3);
  constexpr int GM = 8;
  const int group = logical / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = logical % (GM * tiles_n);
  const int tm = first_m + in_group % gsize, tn = in_group / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16_t* A = (const bf16_t*)g.A;
  const bf16_t* B = (const bf16_t*)g.B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % TL::WGM, wn = wave / TL::WGM;

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  static_assert(BM == NT / 2 && BN == NT / 2, "staging splits the threads evenly between A and B");
  Stage st;
  const bool is_a = threadIdx.x < NT / 2;
  const int u = is_a ? threadIdx.x : threadIdx.x - NT / 2;
  auto gload = [&](int k0) {
    if (is_a) st.load<BM, AK>(u, A, g.lda, m0, g.M, k0, g.K);
    else st.load<BN, BKM>(u, B, g.ldb, n0, g.N, k0, g.K);
  };
  auto lstore = [&](int buf) {
    if (is_a) st.store<BM, AK>(u, sA[buf]);
    else st.store<BN, BKM>(u, sB[buf]);
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
      bf16x8_t af[MI], bfr[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = *(const bf16x8_t*)(a_s + lds_off(wm * TL::WTM + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bfr[j] = *(const bf16x8_t*)(b_s + lds_off(wn * TL::WTN + j * 32 + (lane & 31), ch));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = mfma32<DT>(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  gemm_epilogue<EPI, MI, NJ, DT>(g, acc, m0 + wm * TL::WTM, n0 + wn * TL::WTN, lane);
}

// ------------------------------------------------------------------ pipelined bf16 GEMM
// 256 x 256 tile, 8 waves (2 x 4, wave tile 128 x 64), k-tiles of 64 in 2 LDS stages of 64 KB
// fed by direct global -> LDS loads (global_load_lds_dwordx4: lane l's 16 bytes land at the
// wave's LDS destination + 16 l), so the next k-tile streams in without holding registers.
// Each wave issues 4 loads per operand per stage whatever the layout:
//   K-major operand: stage = [256 rows][64 k] (128-byte rows, 8 chunks, whole cache lines); a
//     wave load covers 8 rows; the chunk order inside a row is swizzled by (r ^ (r >> 3)) & 7.
//   outer-K operand: stage = [64 k][256 rows] (512-byte rows, 32 chunks); a wave load covers 2
//     k-rows; chunks swizzled by (0, 4, 10, 14)[k % 4]. MFMA fragments come out through the LDS
//     transpose read ds_read_b64_tr_b16 (16-lane groups: lanes addressing 4 consecutive k-rows x
//     16 rows deliver 4 consecutive k of one row per lane).
// The swizzles keep both the 16-byte fragment reads and the transpose reads free of bank
// conflicts (checked for 32 and 64 banks). Out-of-range lanes load from a zero page. MFMA
// fragments are double buffered in registers: the LDS reads of the next 16-k step are in flight
// while the MFMAs of the current one run, and are interleaved with them instruction by
// instruction; the one barrier per stage sits where the last step's MFMAs can cover it. Each
// lane's load addresses are computed once and advanced per stage. Every layout (forward, dX,
// dW) runs this kernel.
namespace pipe {

// BM x BN output tiles computed by NT threads in a WGM x (waves / WGM) wave grid; NS stages of
// BK-deep k-tiles of both operands in LDS ((BM + BN) * BK * 2 bytes a stage); MINB workgroups
// share a compute unit.
template <int NT_, int WGM_, int NS_, int BK_, int BM_ = 256, int BN_ = 256, int MINB_ = 1>
struct PCfg {
  static constexpr int BM = BM_, BN = BN_, MINB = MINB_;
  static constexpr int NT = NT_, NW = NT / 64, WGM = WGM_, WGN = NW / WGM, NS = NS_, BK = BK_;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN, MI = WTM / 32, NJ = WTN / 32;
  static constexpr int SEA = BM * BK, SEB = BN * BK;   // elements of each operand in a stage
  static constexpr int SE2 = SEA + SEB;
  static constexpr int LPS = SE2 / 512 / NW;  // this wave's 1 KB loads per stage (both operands)
  static constexpr int KS = BK / 16;          // MFMA k steps per stage
  static_assert(NS * SE2 * 2 * MINB <= 160 * 1024, "LDS");
  static_assert(SEA % (512 * NW) == 0 && SEB % (512 * NW) == 0, "whole loads per wave");
  static_assert(KS % 2 == 0, "fragment sets alternate within a stage");
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_s4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glob_void_t;

__device__ uint4 zero_page[4];

// chunk swizzle of K-major rows: 4 chunks of 16 bytes per row (BK = 32) or 8 (BK = 64)
template <int BK>
__device__ __forceinline__ int swzk(int r) {
  if constexpr (BK == 32) return ((r >> 1) ^ (r >> 3)) & 3;
  else return (r ^ (r >> 3)) & 7;
}
// (0, 4, 10, 14)[k % 4], branch-free (k differs between lanes)
__device__ __forceinline__ int swzt(int k) { return (0xEA40 >> ((k & 3) << 2)) & 15; }

// Issue this wave's loads of one operand (R rows of the tile) for one stage: R * BK / 512
// wave-loads of 1 KB cover the stage, 1 / NW of them per wave. An operand read along M (N) keeps
// a 256-element row per k, 32 swizzled chunks.
template <bool KMAJ, int NW, int BK, int R>
__device__ __forceinline__ void issue(bf16_t* stage, const bf16_t* __restrict__ P, int ld,
                                      int row0, int rows_total, int k0, int K, int wave,
                                      int lane, int split = 0) {
  constexpr int LPR = BK / 8;       // lanes per K-major row (16 bytes each)
  static_assert(KMAJ || R == 256, "outer-k stages hold 256 rows");
#pragma unroll
  for (int q = 0; q < R * BK / 512 / NW; ++q) {
    const int instr = wave + NW * q;
    const void* src = zero_page;
    if constexpr (KMAJ) {
      const int r = instr * (64 / LPR) + lane / LPR;
      const int c = (lane % LPR) ^ swzk<BK>(r);
      int gr = row0 + r;
      bool ok = gr < rows_total;
      if (split) {   // rows R/2 .. R - 1 of the tile come from the matrix's second half
        gr = row0 + r % (R / 2) + (r >= R / 2 ? split : 0);
        ok = row0 + r % (R / 2) < split;
      }
      const int gk = k0 + c * 8;
      if (ok && gk < K) src = P + (size_t)gr * ld + gk;
    } else {
      const int kr = instr * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swzt(kr);
      const int gk = k0 + kr, gr = row0 + c * 8;
      if (gk < K && gr < rows_total) src = P + (size_t)gk * ld + gr;
    }
    __builtin_amdgcn_global_load_lds((glob_void_t*)src, (lds_void_t*)(stage + instr * 512), 16,
                                     0, 0);
  }
}

// The same loads with the per-lane addressing computed once: each lane keeps one source pointer
// per load of the stage and advances it by a per-load byte step (0 for a lane outside the
// matrix, which keeps reading the zero page) each time a stage is issued. Stages are issued in
// order; a stage that reaches past K goes through the bounds-checked issue() instead.
template <bool KMAJ, int NW, int BK, int R>
struct Streamer {
  static constexpr int NL = R * BK / 512 / NW;   // this wave's loads per stage of one operand
  static_assert(KMAJ || R == 256, "outer-k stages hold 256 rows");
  const char* ptr[NL];
  int step[NL];
  int dst0;                                // element offset of this wave's first load in a stage

  __device__ __forceinline__ void init(const bf16_t* __restrict__ P, int ld, int row0,
                                       int rows_total, int wave, int lane, int split = 0,
                                       int k0 = 0) {
    constexpr int LPR = BK / 8;
    dst0 = wave * 512;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int instr = wave + NW * q;
      bool ok;
      size_t off;
      if constexpr (KMAJ) {
        const int r = instr * (64 / LPR) + lane / LPR;
        const int c = (lane % LPR) ^ swzk<BK>(r);
        int gr = row0 + r;
        ok = gr < rows_total;
        if (split) {   // as in issue()
          gr = row0 + r % (R / 2) + (r >= R / 2 ? split : 0);
          ok = row0 + r % (R / 2) < split;
        }
        off = (size_t)gr * ld + k0 + c * 8;
      } else {
        const int kr = instr * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swzt(kr);
        ok = row0 + c * 8 < rows_total;
        off = (size_t)(k0 + kr) * ld + row0 + c * 8;
      }
      ptr[q] = ok ? (const char*)(P + off) : (const char*)zero_page;
      step[q] = ok ? (KMAJ ? BK * 2 : BK * ld * 2) : 0;
    }
  }
  __device__ __forceinline__ void issue_next(bf16_t* stage) {
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      __builtin_amdgcn_global_load_lds((glob_void_t*)ptr[q],
                                       (lds_void_t*)(stage + dst0 + NW * 512 * q), 16, 0, 0);
      ptr[q] += step[q];
    }
  }
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// 8 bf16 of MFMA fragment row `r` (0..255 within the stage), k = 16 kk + 8 h .. + 7
template <bool KMAJ, int BK>
__device__ __forceinline__ bf16x8_t frag(const bf16_t* stage, int rbase, int kk, int lane) {
  if constexpr (KMAJ) {
    const int r = rbase + (lane & 31);
    const int c = (kk * 2 + (lane >> 5)) ^ swzk<BK>(r);
    return *(const bf16x8_t*)(stage + r * BK + c * 8);
  } else {
    const int g = lane >> 4, i = lane & 15;
    const int m = rbase + 16 * (g & 1) + 4 * (i & 3);
    const int k = kk * 16 + 8 * (g >> 1) + (i >> 2);
    const bf16_t* p0 = stage + k * 256 + (((m >> 3) ^ swzt(k)) << 3) + (m & 7);
    const bf16_t* p1 = stage + (k + 4) * 256 + (((m >> 3) ^ swzt(k + 4)) << 3) + (m & 7);
    // inline asm: the compiler would drain all in-flight direct-to-LDS loads before each
    // builtin transpose read; the caller waits on the results with frag_wait()
    short4_t lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(lds_addr(p0)));
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hi) : "v"(lds_addr(p1)));
    typedef short short8_t __attribute__((ext_vector_type(8)));
    const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt with vmcnt = N (bits 3:0 and 15:14), expcnt and lgkmcnt at their maxima (no wait)
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// vmcnt wait that leaves the loads of `later` stages (LPS loads each) in flight, later <= L
template <int L, int LPS>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (L == 0) {
    wait_vm<0>();
  } else {
    if (later >= L) wait_vm<L * LPS>();
    else wait_later<L - 1, LPS>(later);
  }
}

// Wait for this wave's LDS reads into fragment sets a, b and pin the registers after the wait:
// one statement, so no read of the set can be scheduled after the wait.
__device__ __forceinline__ void frag_wait(bf16x8_t (&a)[4], bf16x8_t (&b)[2]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1])
               :
               : "memory");
}
__device__ __forceinline__ void frag_wait(bf16x8_t (&a)[4], bf16x8_t (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                 "+v"(b[2]), "+v"(b[3])
               :
               : "memory");
}

// 8 16-bit values (one 16-byte chunk) of gate and up -> 8 values of silu(g) u
template <int DT>
__device__ __forceinline__ uint4 swiglu_fwd8(const uint4& gv, const uint4& uv) {
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack16<DT>(swiglu_fwd_1(lo16<DT>(gw[i]), lo16<DT>(uw[i])),
                      swiglu_fwd_1(hi16<DT>(gw[i]), hi16<DT>(uw[i])));
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// dm, g, u chunks -> dg, du chunks
template <int DT>
__device__ __forceinline__ void swiglu_bwd8(const uint4& dv, const uint4& gv, const uint4& uv,
                                            uint4& dgv, uint4& duv) {
  const uint32_t dw_[4] = {dv.x, dv.y, dv.z, dv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w},
                 uw[4] = {uv.x, uv.y, uv.z, uv.w};
  uint32_t og[4], ou[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float g0, u0, g1, u1;
    swiglu_bwd_1(lo16<DT>(dw_[i]), lo16<DT>(gw[i]), lo16<DT>(uw[i]), g0, u0);
    swiglu_bwd_1(hi16<DT>(dw_[i]), hi16<DT>(gw[i]), hi16<DT>(uw[i]), g1, u1);
    og[i] = pack16<DT>(g0, g1);
    ou[i] = pack16<DT>(u0, u1);
  }
  dgv = make_uint4(og[0], og[1], og[2], og[3]);
  duv = make_uint4(ou[0], ou[1], ou[2], ou[3]);
}

// The SwiGLU epilogues: the tile rounded to 16 bits into LDS, as the plain 16-bit store does
// (so g, u and dm carry the bits the separate kernels would read), then 16-byte chunks.
//   forward: a tile's columns 0 .. BN/2 - 1 are gate columns n0 .., the rest the matching up
//     columns; both go to gu and silu(g) u to m.
//   backward: columns n0 .. of dm; g and u are read from gu (row stride 2F) a group of chunks at
//     a time, all issued before the first is waited for.
template <int EPI, class PC, int DT>
__device__ __forceinline__ void swiglu_epilogue(const GemmArgs& g,
                                                f32x16_t (&acc)[PC::MI][PC::NJ], float* lds,
                                                int m0, int n0, int wm, int wn, int lane) {
  constexpr int WTM = PC::WTM, WTN = PC::WTN, MI = PC::MI, NJ = PC::NJ, NT = PC::NT;
  constexpr int BM = PC::BM, BN = PC::BN;
  static_assert(BM * BN * 2 <= PC::NS * PC::SE2 * 2, "a 16-bit tile fits the stages");
  const int hl = lane >> 5;
  bf16_t* lb = (bf16_t*)lds;
  __syncthreads();   // the main loop's LDS reads are done
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * WTM + i * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
        const int c = (wn * WTN + j * 32 + (lane & 31)) ^ (hl << 5);
        lb[r * BN + c] = Bits16<DT>::from_f(acc[i][j][e] * g.alpha);
      }
  __syncthreads();
  auto chunk = [&](int r, int c) {
    return *(const uint4*)(lb + r * BN + (c ^ (((r >> 2) & 1) << 5)));
  };
  const int F = g.ffn;
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    constexpr int CPH = BN / 2 / 8, PER = BM * CPH / NT;
    static_assert(BM * CPH % NT == 0, "whole chunks per thread");
    bf16_t* gu = (bf16_t*)g.C;
    bf16_t* mo = (bf16_t*)g.aux_out;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int k = threadIdx.x + NT * q;
      const int r = k / CPH, cc = k % CPH;
      const int gr = m0 + r, col = n0 + cc * 8;
      if (gr < g.M && col < F) {
        const uint4 gv = chunk(r, cc * 8), uv = chunk(r, BN / 2 + cc * 8);
        *(uint4*)(gu + (size_t)gr * g.ldc + col) = gv;
        *(uint4*)(gu + (size_t)gr * g.ldc + F + col) = uv;
        *(uint4*)(mo + (size_t)gr * F + col) = swiglu_fwd8<DT>(gv, uv);
      }
    }
  } else {
    constexpr int CPR = BN / 8, PER = BM * CPR / NT, GRP = 4;
    static_assert(BM * CPR % NT == 0 && PER % GRP == 0, "whole groups per thread");
    const bf16_t* gu = (const bf16_t*)g.aux_in;
    bf16_t* dgu = (bf16_t*)g.C;
#pragma unroll
    for (int q0 = 0; q0 < PER; q0 += GRP) {
      uint4 gv[GRP], uv[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const int k = threadIdx.x + NT * (q0 + j);
        const int gr = m0 + k / CPR, col = n0 + (k % CPR) * 8;
        if (gr < g.M && col < F) {
          gv[j] = *(const uint4*)(gu + (size_t)gr * 2 * F + col);
          uv[j] = *(const uint4*)(gu + (size_t)gr * 2 * F + F + col);
        }
      }
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const int k = threadIdx.x + NT * (q0 + j);
        const int r = k / CPR, cc = k % CPR;
        const int gr = m0 + r, col = n0 + cc * 8;
        if (gr < g.M && col < F) {
          uint4 dgv, duv;
          swiglu_bwd8<DT>(chunk(r, cc * 8), gv[j], uv[j], dgv, duv);
          *(uint4*)(dgu + (size_t)gr * g.ldc + col) = dgv;
          *(uint4*)(dgu + (size_t)gr * g.ldc + F + col) = duv;
        }
      }
    }
  }
}

// Stores through LDS. The accumulators of a 32 x 32 MFMA block give each lane one column, so
// direct stores are one element per lane. Instead, in pass h the waves of wave row h write
// alpha * acc as fp32 into LDS (WTM x BN floats; the 32-column half is flipped for rows with bit 2
// set, so the two half-waves of a write hit different banks), and then every thread reads 4
// consecutive values of a row and stores them with one vector access (8 bytes of bf16, 16 of
// fp32): one wave instruction covers a whole 256-column row. The residual (bf16) and the fp32
// accumulation target are read the same way. Ragged or unaligned edges fall back to per-element
// accesses. The cross-entropy dz (softmax - onehot of a vocabulary chunk, per token column) is
// formed from the same staged values.
template <int EPI, class PC, int DT>
__device__ __forceinline__ void staged_epilogue(const GemmArgs& g,
                                                f32x16_t (&acc)[PC::MI][PC::NJ], float* lds,
                                                int m0, int n0, int wm, int wn, int lane) {
  constexpr int WTM = PC::WTM, WTN = PC::WTN, MI = PC::MI, NJ = PC::NJ, NT = PC::NT;
  constexpr int BM = PC::BM, BN = PC::BN;
  constexpr int CPR = BN / 4;                 // 4-column chunks per row
  constexpr int PER = WTM * CPR / NT;         // chunks per thread and pass
  constexpr bool F32 = EPI == EPI_STORE_F32 || EPI == EPI_ACCUM_F32;
  static_assert(WTM * CPR % NT == 0, "whole chunks per thread");
  if constexpr (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD) {
    swiglu_epilogue<EPI, PC, DT>(g, acc, lds, m0, n0, wm, wn, lane);
    return;
  }
  static_assert(WTM * BN * 4 <= PC::NS * PC::SE2 * 2, "one wave row of fp32 fits the stages");
  const int hl = lane >> 5;
  const bool c_f32 = F32 || (EPI == EPI_CE_DZ && g.c_dtype == SLIDE_F32);
  const bool vec = (g.ldc % 4 == 0) && ((uintptr_t)g.C % (c_f32 ? 16 : 8) == 0) &&
                   (EPI != EPI_RESID || ((g.ldr % 4 == 0) && ((uintptr_t)g.R % 8 == 0)));
  // A thread's chunks all lie in the same 4 columns (NT is a multiple of the chunks per row):
  // for dz, their targets and log-sum-exps are read once.
  static_assert(NT % CPR == 0, "fixed chunk column per thread");
  int dz_y[4] = {-1, -1, -1, -1};
  float dz_lse[4] = {0.f, 0.f, 0.f, 0.f}, inv_nv = 0.f;
  if constexpr (EPI == EPI_CE_DZ) {
    inv_nv = *g.inv_nv;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int col = n0 + (threadIdx.x % CPR) * 4 + t;
      if (col < g.N) {
        const int yt = g.tgt[col];
        if (yt >= 0 && yt < g.V) {
          dz_y[t] = yt;
          dz_lse[t] = g.lse[col];
        }
      }
    }
  }
  // A plain bf16 store of a tile inside an aligned matrix: one pass. The whole tile, rounded to
  // bf16 (the only rounding either way), fits the stages, so every wave writes at once and each
  // thread then stores 16-byte row chunks.
  if constexpr (EPI == EPI_STORE_BF16) {
    if (g.ldc % 8 == 0 && (uintptr_t)g.C % 16 == 0 && m0 + BM <= g.M && n0 + BN <= g.N) {
      static_assert(BM * BN * 2 <= PC::NS * PC::SE2 * 2, "a bf16 tile fits the stages");
      constexpr int CPR8 = BN / 8, PER8 = BM * CPR8 / NT;
      bf16_t* lb = (bf16_t*)lds;
      __syncthreads();   // the main loop's LDS reads are done
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = wm * WTM + i * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
            const int c = (wn * WTN + j * 32 + (lane & 31)) ^ (hl << 5);
            lb[r * BN + c] = Bits16<DT>::from_f(acc[i][j][e] * g.alpha);
          }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < PER8; ++q) {
        const int k = threadIdx.x + NT * q;
        const int r = k / CPR8, cc = k % CPR8;
        const uint4 v = *(const uint4*)(lb + r * BN + ((cc * 8) ^ (((r >> 2) & 1) << 5)));
        *(uint4*)((bf16_t*)g.C + (size_t)(m0 + r) * g.ldc + n0 + cc * 8) = v;
      }
      return;
    }
  }
#pragma unroll
  for (int h = 0; h < PC::WGM; ++h) {
    __syncthreads();   // the main loop's (or the previous pass's) LDS reads are done
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = i * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
            const int c = (wn * WTN + j * 32 + (lane & 31)) ^ (hl << 5);
            lds[r * BN + c] = acc[i][j][e] * g.alpha;
          }
    }
    __syncthreads();
    // the cross-entropy dz also writes zeros into the padding columns [N, ldc)
    const int col_lim = EPI == EPI_CE_DZ ? g.ldc : g.N;
    if (vec && n0 + BN <= col_lim && m0 + h * WTM + WTM <= g.M) {
      // the whole pass is inside the matrix: groups of GRP chunks with no per-chunk checks, so
      // a group's global reads (residual, accumulation target) and LDS reads are all issued
      // before the first of them is waited for
      constexpr int GRP = 8;
      static_assert(PER % GRP == 0, "whole groups per pass");
#pragma unroll
      for (int q0 = 0; q0 < PER; q0 += GRP) {
        uint2 rres[GRP];
        float4 cold[GRP], v[GRP];
#pragma unroll
        for (int j = 0; j < GRP; ++j) {
          const int k = threadIdx.x + NT * (q0 + j);
          const int gr = m0 + h * WTM + k / CPR, gc = n0 + (k % CPR) * 4;
          if constexpr (EPI == EPI_RESID)
            rres[j] = *(const uint2*)((const bf16_t*)g.R + (size_t)gr * g.ldr + gc);
          if constexpr (EPI == EPI_ACCUM_F32)
            cold[j] = *(const float4*)((const float*)g.C + (size_t)gr * g.ldc + gc);
        }
#pragma unroll
        for (int j = 0; j < GRP; ++j) {
          const int k = threadIdx.x + NT * (q0 + j);
          const int r = k / CPR, cc = k % CPR;
          v[j] = *(const float4*)(lds + r * BN + ((cc * 4) ^ (((r >> 2) & 1) << 5)));
        }
#pragma unroll
        for (int j = 0; j < GRP; ++j) {
          const int k = threadIdx.x + NT * (q0 + j);
          const int gr = m0 + h * WTM + k / CPR, gc = n0 + (k % CPR) * 4;
          const size_t at = (size_t)gr * g.ldc + gc;
          float o[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
          bool f32_out = F32;
          if constexpr (EPI == EPI_RESID) {
            o[0] += lo16<DT>(rres[j].x);
            o[1] += hi16<DT>(rres[j].x);
            o[2] += lo16<DT>(rres[j].y);
            o[3] += hi16<DT>(rres[j].y);
          }
          if constexpr (EPI == EPI_ACCUM_F32) {
            o[0] += cold[j].x;
            o[1] += cold[j].y;
            o[2] += cold[j].z;
            o[3] += cold[j].w;
          }
          if constexpr (EPI == EPI_CE_DZ) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              float d = 0.f;
              if (dz_y[t] >= 0) {
                d = __expf(o[t] - dz_lse[t]);
                if (g.c0 + gr == dz_y[t]) d -= 1.f;
                d *= inv_nv;
              }
              o[t] = d;
            }
            f32_out = c_f32;
          }
          if (f32_out) {
            *(float4*)((float*)g.C + at) = make_float4(o[0], o[1], o[2], o[3]);
          } else {
            uint2 w;
            w.x = pack16<DT>(o[0], o[1]);
            w.y = pack16<DT>(o[2], o[3]);
            *(uint2*)((bf16_t*)g.C + at) = w;
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int k = threadIdx.x + NT * q;
      const int r = k / CPR, cc = k % CPR;
      const int gr = m0 + h * WTM + r, gc = n0 + cc * 4;
      if (gr >= g.M || gc >= col_lim) continue;
      const float4 v = *(const float4*)(lds + r * BN + ((cc * 4) ^ (((r >> 2) & 1) << 5)));
      float o[4] = {v.x, v.y, v.z, v.w};
      const size_t at = (size_t)gr * g.ldc + gc;
      if constexpr (EPI == EPI_CE_DZ) {
        // dz = (softmax - onehot) / N_valid of vocabulary row c0 + gr for tokens gc .. gc + 3;
        // 0 for ignored targets and padding columns
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float d = 0.f;
          if (dz_y[t] >= 0) {
            d = __expf(o[t] - dz_lse[t]);
            if (g.c0 + gr == dz_y[t]) d -= 1.f;
            d *= inv_nv;
          }
          o[t] = d;
        }
        if (vec && gc + 3 < g.ldc) {
          if (g.c_dtype != SLIDE_F32) {
            uint2 w;
            w.x = pack16<DT>(o[0], o[1]);
            w.y = pack16<DT>(o[2], o[3]);
            *(uint2*)((bf16_t*)g.C + at) = w;
          } else {
            *(float4*)((float*)g.C + at) = make_float4(o[0], o[1], o[2], o[3]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (gc + t >= g.ldc) break;
            if (g.c_dtype != SLIDE_F32) ((bf16_t*)g.C)[at + t] = Bits16<DT>::from_f(o[t]);
            else ((float*)g.C)[at + t] = o[t];
          }
        }
        continue;
      }
      if (vec && gc + 3 < g.N) {
        if constexpr (F32) {
          float4* c = (float4*)((float*)g.C + at);
          if constexpr (EPI == EPI_ACCUM_F32) {
            const float4 old = *c;
            o[0] += old.x;
            o[1] += old.y;
            o[2] += old.z;
            o[3] += old.w;
          }
          *c = make_float4(o[0], o[1], o[2], o[3]);
        } else {
          if constexpr (EPI == EPI_RESID) {
            const uint2 rr = *(const uint2*)((const bf16_t*)g.R + (size_t)gr * g.ldr + gc);
            o[0] += lo16<DT>(rr.x);
            o[1] += hi16<DT>(rr.x);
            o[2] += lo16<DT>(rr.y);
            o[3] += hi16<DT>(rr.y);
          }
          uint2 w;
          w.x = pack16<DT>(o[0], o[1]);
          w.y = pack16<DT>(o[2], o[3]);
          *(uint2*)((bf16_t*)g.C + at) = w;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (gc + t >= g.N) break;
          float x = o[t];
          if constexpr (EPI == EPI_STORE_F32) {
            ((float*)g.C)[at + t] = x;
          } else if constexpr (EPI == EPI_ACCUM_F32) {
            ((float*)g.C)[at + t] += x;
          } else {
            if constexpr (EPI == EPI_RESID)
              x += Bits16<DT>::to_f(((const bf16_t*)g.R)[(size_t)gr * g.ldr + gc + t]);
            ((bf16_t*)g.C)[at + t] = Bits16<DT>::from_f(x);
          }
        }
      }
    }
  }
}

// Tile (tm, tn) of a logical tile index: groups of GM tile rows walked column by column, so that
// consecutive tiles share B columns and a group's A rows stay in L2.
__device__ __forceinline__ void tile_coords(int logical, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  constexpr int GM = 4;
  const int group = logical / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = logical % (GM * tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// compile-time selector of the steady-state or the checked stage body
template <bool V>
struct StageTag {
  static constexpr bool value = V;
};

}  // namespace pipe

// HALF = true: the launch for the tail tiles of a split GEMM (see launch_pipe); workgroup w
// computes K half w % 2 of tail tile w / 2 and stores its fp32 partial sums.
template <class PC, bool AK, bool BKM, int EPI, int SITE, int DT, bool HALF = false>
__global__ __launch_bounds__(PC::NT, PC::MINB) void gemm_pipe_kernel(GemmArgs g) {
  using namespace pipe;
  constexpr int NS = PC::NS, NW = PC::NW, WGM = PC::WGM, WTM = PC::WTM, WTN = PC::WTN;
  constexpr int MI = PC::MI, NJ = PC::NJ, BK = PC::BK, SE2 = PC::SE2, KS = PC::KS;
  constexpr int BM = PC::BM, BN = PC::BN;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NS * SE2];

  // SwiGLU forward: a tile's B rows are BN / 2 gate rows and the matching up rows (F later)
  constexpr bool SPLIT = EPI == EPI_SWIGLU_FWD;
  static_assert(!SPLIT || (AK && BKM), "split tiles read a K-major B");
  const int split = SPLIT ? g.ffn : 0;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = SPLIT ? (g.ffn + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
  // Whole tiles in an XCD-aware order (workgroup w runs on XCD w % 8, so each XCD takes a
  // contiguous range of tiles); a split GEMM's tail tiles follow the whole ones (HALF launch).
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int n_full = tiles_m * tiles_n - g.tail_split;
  int logical = wg, half = 0;
  if constexpr (HALF) {
    logical = n_full + (wg >> 1);
    half = wg & 1;
  } else if ((nwg & 7) == 0) {
    logical = (wg & 7) * (nwg >> 3) + (wg >> 3);
  }
  int tm, tn;
  tile_coords(logical, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * (SPLIT ? BN / 2 : BN);
  int kb = 0, ke = g.K;              // this workgroup's K range
  if constexpr (HALF) {
    const int mid = (g.K + BK - 1) / BK / 2 * BK;
    if (half == 0) ke = mid;
    else kb = mid;
  }

  const bf16_t* A = (const bf16_t*)g.A;
  const bf16_t* B = (const bf16_t*)g.B;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WGM, wn = wave / WGM;

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (ke - kb + BK - 1) / BK;
  auto stage_a = [&](int b) { return smem + b * SE2; };
  auto stage_b = [&](int b) { return smem + b * SE2 + PC::SEA; };
  Streamer<AK, NW, BK, BM> sta;
  Streamer<BKM, NW, BK, BN> stb;
  sta.init(A, g.lda, m0, g.M, wave, lane, 0, kb);
  stb.init(B, g.ldb, n0, g.N, wave, lane, split, kb);
  auto issue_stage = [&](int kt) {   // stages are issued in order 0, 1, 2, ...
    const int b = kt % NS;
    if (kb + (kt + 1) * BK <= ke) {
      sta.issue_next(stage_a(b));
      stb.issue_next(stage_b(b));
    } else {                         // the last, partial stage: bounds-checked per lane
      issue<AK, NW, BK, BM>(stage_a(b), A, g.lda, m0, g.M, kb + kt * BK, ke, wave, lane);
      issue<BKM, NW, BK, BN>(stage_b(b), B, g.ldb, n0, g.N, kb + kt * BK, ke, wave, lane, split);
    }
  };
  // Wait until stage kt has landed (this wave's loads; the barrier that follows covers the
  // other waves'): the loads of the stages issued after it, up to stage `last`, may stay in
  // flight.
  auto wait_stage = [&](int kt, int last) {
    wait_later<NS - 1, PC::LPS>(min(nk - 1, last) - kt);
  };
  // Fragments of one 16-wide k step, double buffered: the LDS reads of the next step are in
  // flight while the MFMAs of the current one run.
  bf16x8_t fa[2][MI], fb[2][NJ];
  auto load_frags = [&](int buf, int kt, int kk) {
    const bf16_t* sa = stage_a(kt % NS);
    const bf16_t* sb = stage_b(kt % NS);
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[buf][i] = frag<AK, BK>(sa, wm * WTM + i * 32, kk, lane);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[buf][j] = frag<BKM, BK>(sb, wn * WTN + j * 32, kk, lane);
  };
  // Wait for this wave's LDS reads of fragment set `buf` and pin the registers after the wait:
  // one statement, so no read of the set can be scheduled after the wait. Required before a
  // barrier that lets other waves overwrite the stage, and before inline-asm (transpose) reads
  // are consumed.
  auto wait_frags = [&](int buf) { frag_wait(fa[buf], fb[buf]); };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = mfma32<DT>(fa[buf][i], fb[buf][j], acc[i][j]);
  };

  // All NS stages start in flight; stage kt + NS reuses stage kt's buffer once every wave has
  // read stage kt (the barrier in iteration kt).
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nk) issue_stage(s);
  if (nk > 0) {
    wait_stage(0, NS - 1);
    asm volatile("s_barrier" ::: "memory");
    load_frags(0, 0, 0);
  }
  // Steps of 16 k alternate between the two fragment sets. The last step of a stage passes the
  // barrier after which stage kt's buffer is refilled and stage kt + 1's first fragments are
  // read, then runs its MFMAs while those reads are in flight. sched_barrier(0) keeps the
  // compiler from moving MFMAs across steps.
  //
  // A steady-state stage (stage kt + NS is a full stage, issued in this iteration) is
  // straight-line code: its last step's MFMAs interleave with the barrier, the stage loads and
  // the next fragment reads. The last NS stages take the same steps with runtime checks.
  auto run_stage = [&](int kt, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int cur = kk & 1;
      wait_frags(cur);
      if (kk + 1 < KS) {
        load_frags(cur ^ 1, kt, kk + 1);
      } else if constexpr (STEADY) {
        // stages kt + 2 .. kt + NS - 1 stay in flight
        wait_vm<(NS - 2) * PC::LPS>();
        asm volatile("s_barrier" ::: "memory");
        sta.issue_next(stage_a(kt % NS));
        stb.issue_next(stage_b(kt % NS));
        load_frags(cur ^ 1, kt + 1, 0);
      } else if (kt + 1 < nk) {
        wait_stage(kt + 1, kt + NS - 1);
        // Plain barrier: the explicit vmcnt wait covers this wave's loads of stage kt + 1, and
        // the later stages' loads stay in flight across it.
        asm volatile("s_barrier" ::: "memory");
        if (kt + NS < nk) issue_stage(kt + NS);
        load_frags(cur ^ 1, kt + 1, 0);
      }
      mfmas(cur);
      // Interleave this step's MFMAs with the other work (the next set's LDS reads, a stage's
      // direct-to-LDS loads, address arithmetic): each MFMA is followed by one or two memory
      // instructions and a few ALU instructions, which issue while it runs.
      if constexpr (STEADY) {
        if (kk + 1 == KS) {
#pragma unroll
          for (int q = 0; q < MI * NJ - 1; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100 | 0x020, 2, 0);   // LDS read, VMEM read
            __builtin_amdgcn_sched_group_barrier(0x002 | 0x004, 4, 0);   // VALU, SALU
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
      }
#pragma unroll
      for (int q = 0; q < MI * NJ - 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100 | 0x020, 1, 0);   // LDS read, VMEM read
        __builtin_amdgcn_sched_group_barrier(0x002 | 0x004, 5, 0);   // VALU, SALU
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // iterations whose stage kt + NS is a full stage
  const int n_steady = max(0, (ke - kb) / BK - NS);
  int kt = 0;
  for (; kt < n_steady; ++kt) run_stage(kt, StageTag<true>{});
  for (; kt < nk; ++kt) run_stage(kt, StageTag<false>{});

  if constexpr (HALF) {   // a K half of a tail tile: its fp32 partial sums, in register order
    float* p = g.tail_ws + ((size_t)wg * (BM * BN));
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          p[(((wave * MI + i) * NJ + j) * 16 + e) * 64 + lane] = acc[i][j][e];
    (void)half;
  } else if constexpr (EPI != EPI_CE_STATS)
    staged_epilogue<EPI, PC, DT>(g, acc, (float*)smem, m0, n0, wm, wn, lane);
  else
    gemm_epilogue<EPI, MI, NJ, DT>(g, acc, m0 + wm * WTM, n0 + wn * WTN, lane);
}

// The tail tiles of a split launch: the two K halves' partial sums added in a fixed order (the
// first half's plus the second's), then the tile's usual epilogue.
template <class PC, int EPI, int DT>
__global__ __launch_bounds__(PC::NT, PC::MINB) void gemm_tail_combine_kernel(GemmArgs g) {
  using namespace pipe;
  constexpr int NW = PC::NW, WGM = PC::WGM, MI = PC::MI, NJ = PC::NJ, BM = PC::BM, BN = PC::BN;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[PC::NS * PC::SE2];
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int n_full = tiles_m * tiles_n - g.tail_split;
  int tm, tn;
  tile_coords(n_full + (int)blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  static_assert(NW == PC::NT / 64, "waves");
  const float* p0 = g.tail_ws + (size_t)blockIdx.x * 2 * (BM * BN);
  const float* p1 = p0 + BM * BN;
  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const size_t at = (size_t)(((wave * MI + i) * NJ + j) * 16 + e) * 64 + lane;
        acc[i][j][e] = p0[at] + p1[at];
      }
  staged_epilogue<EPI, PC, DT>(g, acc, (float*)smem, tm * BM, tn * BN, wave % WGM, wave / WGM,
                               lane);
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

// Two 64-deep stages where an operand is K-major (its 128-byte rows swizzle conflict-free); when
// both operands are read through transpose reads (the weight-gradient GEMMs), four 32-deep
// stages, which keep more loads in flight.
using PipeL = pipe::PCfg<512, 2, 2, 64>;
using PipeT = pipe::PCfg<512, 2, 4, 32>;
template <bool AK, bool BKM>
struct PipeFor {
  using type = PipeL;
};
template <>
struct PipeFor<false, false> {
  using type = PipeT;
};

// Large tiles when they alone give at least half a wave of workgroups per compute unit.
inline bool use_large(const GemmArgs& g) {
  const long tiles = (long)((g.M + 255) / 256) * ((g.N + 255) / 256);
  return tiles >= 128;
}

// compute units of the current device (cached per device)
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <bool AK, bool BKM, int EPI, int SITE, int DT>
void launch_pipe(const GemmArgs& g_in, hipStream_t st) {
  using PC = typename PipeFor<AK, BKM>::type;
  GemmArgs g = g_in;
  const int tiles_n = EPI == EPI_SWIGLU_FWD ? (g.ffn + PC::BN / 2 - 1) / (PC::BN / 2)
                                            : (g.N + PC::BN - 1) / PC::BN;
  const int tiles = ((g.M + PC::BM - 1) / PC::BM) * tiles_n;
  // A last wave of at most half the compute units would leave the others idle for a whole tile:
  // with a workspace, the whole waves run first, then the tail tiles as two K halves each (one
  // workgroup per half, so the halves fill the compute units), then a launch that adds them.
  g.tail_split = 0;
  constexpr bool CAN_SPLIT = EPI == EPI_STORE_BF16 || EPI == EPI_STORE_F32 || EPI == EPI_RESID ||
                             EPI == EPI_ACCUM_F32;
  const int cus = cu_count();
  if (CAN_SPLIT && g.tail_ws && cus > 0 && tiles > cus && g.K >= 4 * PC::BK) {
    const int tail = tiles % cus;
    if (tail > 0 && 2 * tail <= cus && tail <= kTailMaxTiles &&
        (size_t)tail * 2 * PC::BM * PC::BN * 4 <= g.tail_ws_bytes)
      g.tail_split = tail;
  }
  hipLaunchKernelGGL((gemm_pipe_kernel<PC, AK, BKM, EPI, SITE, DT>), dim3(tiles - g.tail_split),
                     dim3(PC::NT), 0, st, g);
  if constexpr (CAN_SPLIT) {
    if (g.tail_split) {
      hipLaunchKernelGGL((gemm_pipe_kernel<PC, AK, BKM, EPI, SITE, DT, true>),
                         dim3(2 * g.tail_split), dim3(PC::NT), 0, st, g);
      hipLaunchKernelGGL((gemm_tail_combine_kernel<PC, EPI, DT>), dim3(g.tail_split),
                         dim3(PC::NT), 0, st, g);
    }
  }
}

template <bool AK, bool BKM, int EPI, int SITE, int DT>
void launch_one(const GemmArgs& g, hipStream_t st) {
  if constexpr (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD) {
    launch_pipe<AK, BKM, EPI, SITE, DT>(g, st);   // callers checked use_large
  } else if (use_large(g)) {
    launch_pipe<AK, BKM, EPI, SITE, DT>(g, st);
  } else {
    const int tiles = ((g.M + TileS::BM - 1) / TileS::BM) * ((g.N + TileS::BN - 1) / TileS::BN);
    hipLaunchKernelGGL((gemm_bf16_kernel<TileS, AK, BKM, EPI, SITE, DT>), dim3(tiles),
                       dim3(TileS::NT), 0, st, g);
  }
}

template <bool AK, bool BKM, int DT>
void launch_generic(const GemmArgs& g, hipStream_t st, int epi) {
  switch (epi) {
    case EPI_STORE_BF16: launch_one<AK, BKM, EPI_STORE_BF16, SITE_GENERIC, DT>(g, st); break;
    case EPI_STORE_F32: launch_one<AK, BKM, EPI_STORE_F32, SITE_GENERIC, DT>(g, st); break;
    case EPI_RESID: launch_one<AK, BKM, EPI_RESID, SITE_GENERIC, DT>(g, st); break;
    default: launch_one<AK, BKM, EPI_ACCUM_F32, SITE_GENERIC, DT>(g, st); break;
  }
}

// (site, a_kmajor, b_kmajor, epilogue) -> dedicated instantiation, else generic; DT is the
// 16-bit operand type (SLIDE_BF16 or SLIDE_F16)
template <int DT>
void launch_16(const GemmArgs& g, hipStream_t st, int epi) {
#define SLIDE_SITE(S, AK_, BK_, EPI_)                                              \
  if (g.site == S && g.a_kmajor == AK_ && g.b_kmajor == BK_ && epi == EPI_) {    \
    launch_one<AK_, BK_, EPI_, S, DT>(g, st);                                    \
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
  SLIDE_SITE(SITE_CE_STATS, true, true, EPI_CE_STATS)
  SLIDE_SITE(SITE_CE_DZ, true, true, EPI_CE_DZ)
  SLIDE_SITE(SITE_CE_DH, false, false, EPI_ACCUM_F32)
  SLIDE_SITE(SITE_CE_DW, true, false, EPI_STORE_BF16)
  SLIDE_SITE(SITE_GATE_UP, true, true, EPI_SWIGLU_FWD)
  SLIDE_SITE(SITE_DOWN_DX, true, false, EPI_SWIGLU_BWD)
#undef SLIDE_SITE
  if (g.a_kmajor && g.b_kmajor) launch_generic<true, true, DT>(g, st, epi);
  else if (g.a_kmajor) launch_generic<true, false, DT>(g, st, epi);
  else if (g.b_kmajor) launch_generic<false, true, DT>(g, st, epi);
  else launch_generic<false, false, DT>(g, st, epi);
}

}  // namespace

int gemm_epilogue_of(const GemmArgs& g) {
  if (g.special == SPECIAL_CE_STATS) return EPI_CE_STATS;
  if (g.special == SPECIAL_CE_DZ) return EPI_CE_DZ;
  if (g.special == SPECIAL_SWIGLU_FWD) return EPI_SWIGLU_FWD;
  if (g.special == SPECIAL_SWIGLU_BWD) return EPI_SWIGLU_BWD;
  if (g.accumulate) return EPI_ACCUM_F32;
  if (g.R) return EPI_RESID;
  return g.c_dtype == SLIDE_F32 ? EPI_STORE_F32 : EPI_STORE_BF16;
}

int gemm_check(const GemmArgs& g) {
  SLIDE_REQUIRE(g.M >= 0 && g.N >= 0 && g.K >= 0, SLIDE_E_SHAPE, "gemm: negative size");
  SLIDE_REQUIRE(g.A && g.B && g.C, SLIDE_E_ARG, "gemm: null operand");
  SLIDE_REQUIRE(dtype_valid(g.dtype), SLIDE_E_ARG, "gemm: bad dtype");
  SLIDE_REQUIRE(!g.accumulate || g.c_dtype == SLIDE_F32, SLIDE_E_ARG,
                "gemm: accumulate needs an fp32 C");
  SLIDE_REQUIRE(!(g.accumulate && g.R), SLIDE_E_ARG, "gemm: residual and accumulate are exclusive");
  SLIDE_REQUIRE(!g.R || g.c_dtype == g.dtype, SLIDE_E_ARG, "gemm: residual output must be in dtype");
  SLIDE_REQUIRE(g.lda >= (g.a_kmajor ? g.K : g.M) && g.ldb >= (g.b_kmajor ? g.K : g.N) &&
                    g.ldc >= g.N && (!g.R || g.ldr >= g.N),
                SLIDE_E_SHAPE, "gemm: leading dimension smaller than the row");
  if (g.dtype != SLIDE_F32) {
    SLIDE_REQUIRE(aligned16(g.A) && aligned16(g.B), SLIDE_E_ARG, "gemm: operands must be 16-byte aligned");
    SLIDE_REQUIRE(g.lda % 8 == 0 && g.ldb % 8 == 0, SLIDE_E_SHAPE, "gemm: lda/ldb must be multiples of 8");
    // 16-byte vector loads: a K-contiguous operand needs K % 8 == 0; an operand whose rows run
    // along M (or N) may be ragged as long as the padded row fits its leading dimension.
    auto r8 = [](int v) { return (v + 7) / 8 * 8; };
    SLIDE_REQUIRE((g.a_kmajor ? g.K % 8 == 0 : g.lda >= r8(g.M)) &&
                      (g.b_kmajor ? g.K % 8 == 0 : g.ldb >= r8(g.N)),
                  SLIDE_E_SHAPE, "gemm: K must be a multiple of 8 for a K-contiguous operand, "
                  "and ld >= M (N) rounded up to 8 otherwise");
    SLIDE_REQUIRE(g.c_dtype == g.dtype || g.c_dtype == SLIDE_F32, SLIDE_E_ARG,
                  "gemm: c_dtype must be the operands' dtype or SLIDE_F32");
  } else {
    SLIDE_REQUIRE(g.c_dtype == SLIDE_F32, SLIDE_E_ARG, "gemm: fp32 operands need an fp32 C");
  }
  return SLIDE_OK;
}

int gemm_launch(const GemmArgs& g, hipStream_t st) {
  if (g.M == 0 || g.N == 0) return SLIDE_OK;
  // the cross-entropy and SwiGLU epilogues exist for their GEMMs' own instantiations only
  SLIDE_REQUIRE(g.special == SPECIAL_NONE || g.special == SPECIAL_SWIGLU_FWD ||
                    g.special == SPECIAL_SWIGLU_BWD ||
                    (g.dtype != SLIDE_F32 && g.a_kmajor && g.b_kmajor &&
                     g.site == (g.special == SPECIAL_CE_STATS ? SITE_CE_STATS : SITE_CE_DZ)),
                SLIDE_E_ARG, "gemm: cross-entropy epilogue with another site or layout");
  SLIDE_REQUIRE(g.special != SPECIAL_SWIGLU_FWD ||
                    (g.dtype != SLIDE_F32 && g.a_kmajor && g.b_kmajor && g.site == SITE_GATE_UP &&
                     use_large(g) && g.N == 2 * g.ffn && g.aux_out),
                SLIDE_E_ARG, "gemm: SwiGLU forward epilogue with another site, layout or size");
  SLIDE_REQUIRE(g.special != SPECIAL_SWIGLU_BWD ||
                    (g.dtype != SLIDE_F32 && g.a_kmajor && !g.b_kmajor && g.site == SITE_DOWN_DX &&
                     use_large(g) && g.N == g.ffn && g.aux_in),
                SLIDE_E_ARG, "gemm: SwiGLU backward epilogue with another site, layout or size");
  ProfScope ps(g.name ? g.name : "gemm", st);
  const int epi = gemm_epilogue_of(g);
  if (g.dtype == SLIDE_BF16) {
    launch_16<SLIDE_BF16>(g, st, epi);
  } else if (g.dtype == SLIDE_F16) {
    launch_16<SLIDE_F16>(g, st, epi);
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

int gemm_swiglu_fwd(int M, int F, int K, const void* x, int ldx, const void* w, int ldw, void* gu,
                    void* m, int dtype, const char* name, int site, hipStream_t st) {
  GemmArgs g{M, 2 * F, K, x, ldx, true, w, ldw, true, gu, 2 * F, dtype, nullptr, 0, 1.0f,
             false, dtype, name, site};
  if (dtype == SLIDE_F32 || !use_large(g)) {
    SLIDE_TRY(gemm_launch(g, st));
    return swiglu_fwd(gu, m, M, F, dtype, st);
  }
  SLIDE_REQUIRE(F % 8 == 0 && aligned16(gu) && aligned16(m), SLIDE_E_ARG,
                "gemm_swiglu_fwd: F must be a multiple of 8 and gu, m 16-byte aligned");
  g.special = SPECIAL_SWIGLU_FWD;
  g.ffn = F;
  g.aux_out = m;
  return gemm_launch(g, st);
}

bool gemm_swiglu_bwd_needs_dm(int M, int F, int dtype) {
  GemmArgs g{};
  g.M = M;
  g.N = F;
  return dtype == SLIDE_F32 || !use_large(g);
}

int gemm_swiglu_bwd(int M, int F, int K, const void* dy, int lddy, const void* w, int ldw,
                    const void* gu, void* dgu, void* dm_ws, int dtype, const char* name, int site,
                    hipStream_t st) {
  GemmArgs g{M, F, K, dy, lddy, true, w, ldw, false, dm_ws, F, dtype, nullptr, 0, 1.0f, false,
             dtype, name, site};
  if (gemm_swiglu_bwd_needs_dm(M, F, dtype)) {
    SLIDE_REQUIRE(dm_ws, SLIDE_E_ARG, "gemm_swiglu_bwd: these sizes need the dm workspace");
    SLIDE_TRY(gemm_launch(g, st));
    return swiglu_bwd(dm_ws, gu, dgu, M, F, dtype, st);
  }
  SLIDE_REQUIRE(F % 8 == 0 && aligned16(gu) && aligned16(dgu), SLIDE_E_ARG,
                "gemm_swiglu_bwd: F must be a multiple of 8 and gu, dgu 16-byte aligned");
  g.C = dgu;
  g.ldc = 2 * F;
  g.special = SPECIAL_SWIGLU_BWD;
  g.ffn = F;
  g.aux_in = gu;
  return gemm_launch(g, st);
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

extern "C" size_t slide_gemm_tail_workspace_bytes(void) { return slide::kTailWsBytes; }

extern "C" int slide_gemm_ws(int M, int N, int K, const void* A, int lda, int a_kmajor,
                             const void* B, int ldb, int b_kmajor, void* C, int ldc, int c_dtype,
                             const void* R, int ldr, float alpha, int accumulate, int dtype,
                             void* ws, size_t ws_bytes, void* stream) {
  slide::GemmArgs g{M, N, K, A, lda, a_kmajor != 0, B, ldb, b_kmajor != 0, C, ldc, c_dtype,
                    R, ldr, alpha, accumulate != 0, dtype, "gemm", slide::SITE_GENERIC};
  SLIDE_TRY(slide::gemm_check(g));
  SLIDE_REQUIRE(!ws || slide::aligned16(ws), SLIDE_E_ARG, "gemm_ws: workspace must be 16-byte aligned");
  g.tail_ws = (float*)ws;
  g.tail_ws_bytes = ws ? ws_bytes : 0;
  return slide::gemm_launch(g, (hipStream_t)stream);
}

extern "C" int slide_gemm_swiglu_fwd(int M, int F, int K, const void* x, int ldx, const void* w_gu,
                                     int ldw, void* gu, void* m, int dtype, void* stream) {
  SLIDE_REQUIRE(slide::dtype_valid(dtype), SLIDE_E_ARG, "gemm_swiglu_fwd: bad dtype");
  SLIDE_REQUIRE(M >= 0 && K >= 0 && F > 0 && F % 8 == 0, SLIDE_E_SHAPE,
                "gemm_swiglu_fwd: M %d, K %d must be >= 0 and F %d a positive multiple of 8", M,
                K, F);
  SLIDE_REQUIRE(m && slide::aligned16(m) && slide::aligned16(gu), SLIDE_E_ARG,
                "gemm_swiglu_fwd: gu and m must be non-null and 16-byte aligned");
  slide::GemmArgs g{M, 2 * F, K, x, ldx, true, w_gu, ldw, true, gu, 2 * F, dtype, nullptr, 0,
                    1.0f, false, dtype, "gemm_swiglu_fwd", slide::SITE_GATE_UP};
  SLIDE_TRY(slide::gemm_check(g));
  if (M == 0) return SLIDE_OK;
  return slide::gemm_swiglu_fwd(M, F, K, x, ldx, w_gu, ldw, gu, m, dtype, "gemm_swiglu_fwd",
                                slide::SITE_GATE_UP, (hipStream_t)stream);
}

extern "C" size_t slide_gemm_swiglu_bwd_workspace_bytes(int M, int F, int dtype) {
  if (M <= 0 || F <= 0 || !slide::dtype_valid(dtype)) return 0;
  if (!slide::gemm_swiglu_bwd_needs_dm(M, F, dtype)) return 0;
  return slide::align_up((size_t)M * F * slide::dtype_size(dtype), 256);
}

extern "C" int slide_gemm_swiglu_bwd(int M, int F, int K, const void* dy, int lddy,
                                     const void* w_down, int ldw, const void* gu, void* dgu,
                                     int dtype, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_REQUIRE(slide::dtype_valid(dtype), SLIDE_E_ARG, "gemm_swiglu_bwd: bad dtype");
  SLIDE_REQUIRE(M >= 0 && K >= 0 && F > 0 && F % 8 == 0, SLIDE_E_SHAPE,
                "gemm_swiglu_bwd: M %d, K %d must be >= 0 and F %d a positive multiple of 8", M,
                K, F);
  SLIDE_REQUIRE(gu && dgu && slide::aligned16(gu) && slide::aligned16(dgu), SLIDE_E_ARG,
                "gemm_swiglu_bwd: gu and dgu must be non-null and 16-byte aligned");
  const size_t need = slide_gemm_swiglu_bwd_workspace_bytes(M, F, dtype);
  SLIDE_REQUIRE(ws_bytes >= need && (need == 0 || (ws && slide::aligned16(ws))), SLIDE_E_WORKSPACE,
                "gemm_swiglu_bwd: workspace %zu < %zu", ws_bytes, need);
  slide::GemmArgs g{M, F, K, dy, lddy, true, w_down, ldw, false, dgu, 2 * F, dtype, nullptr, 0,
                    1.0f, false, dtype, "gemm_swiglu_bwd", slide::SITE_DOWN_DX};
  SLIDE_TRY(slide::gemm_check(g));
  if (M == 0) return SLIDE_OK;
  return slide::gemm_swiglu_bwd(M, F, K, dy, lddy, w_down, ldw, gu, dgu, need ? ws : nullptr,
                                dtype, "gemm_swiglu_bwd", slide::SITE_DOWN_DX, (hipStream_t)stream);
}
