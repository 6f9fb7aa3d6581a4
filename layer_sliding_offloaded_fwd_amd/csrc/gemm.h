// GEMM launcher shared by the layer, the LM-head cross-entropy and the C ABI.
#pragma once
#include "common.h"

namespace slide {

enum { EPI_STORE_BF16 = 0, EPI_STORE_F32 = 1, EPI_RESID = 2, EPI_ACCUM_F32 = 3,
       EPI_CE_STATS = 4, EPI_CE_DZ = 5, EPI_SWIGLU_FWD = 6, EPI_SWIGLU_BWD = 7 };

// Fused epilogues of the LM-head cross-entropy's logits GEMM (C = z^T, [vocab rows][tokens]):
//   CE_STATS: per token column, the max and sum of exp(z - max) over each block of kCeRowsPerPart
//     vocabulary rows, into pm / ps[(row / kCeRowsPerPart) * N + t]; the target logit into zt[t].
//     z itself is not stored.
//   CE_DZ: dz = (exp(z - lse_t) - [c0 + row == y_t]) * inv_nv for valid targets, else 0, stored
//     in C (the storage type) for columns up to ldc (columns past N get 0).
constexpr int kCeRowsPerPart = 64;
enum { SPECIAL_NONE = 0, SPECIAL_CE_STATS = 1, SPECIAL_CE_DZ = 2, SPECIAL_SWIGLU_FWD = 3,
       SPECIAL_SWIGLU_BWD = 4 };

// Fused SwiGLU epilogues of the MLP GEMMs (16-bit operands, pipelined kernel):
//   SWIGLU_FWD (gate/up projection, A and B K-major, B = W_gu [2F][K] with the gate rows first):
//     each tile holds 128 gate and the matching 128 up columns; it stores them into C = gu
//     [M][2F] (ldc) and m = silu(g) u of the 16-bit g and u into aux_out [M][F].
//   SWIGLU_BWD (down projection's input gradient, N = F): the 16-bit dm of each tile is not
//     stored; with g, u read from aux_in = gu [M][2F] (ld 2F) it gives dg, du into C = dgu
//     [M][2F] (ldc).

// Call sites of the layer and the LM head. Each site with its usual layout gets its own kernel
// symbol (the site is a template tag with no effect on the code), so that profilers report the
// projections separately; any other combination runs the generic instantiation.
enum GemmSite {
  SITE_GENERIC = 0, SITE_QKV, SITE_O, SITE_GATE_UP, SITE_DOWN,
  SITE_DOWN_DX, SITE_DOWN_DW, SITE_GATE_UP_DX, SITE_GATE_UP_DW, SITE_O_DX, SITE_O_DW,
  SITE_QKV_DX, SITE_QKV_DW, SITE_CE_STATS, SITE_CE_DZ, SITE_CE_DH, SITE_CE_DW
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
  // cross-entropy epilogues (special != SPECIAL_NONE; A and B K-major)
  int special;
  const int32_t* tgt;    // [N] targets (vocabulary index, < 0 ignored)
  const float* lse;      // [N] (CE_DZ)
  const float* inv_nv;   // 1 / number of valid targets (CE_DZ)
  float* pm;             // [parts][N] (CE_STATS)
  float* ps;
  float* zt;             // [N] target logit (CE_STATS)
  int c0;                // first vocabulary row of this chunk
  int V;                 // vocabulary size
  // SwiGLU epilogues
  int ffn;               // F
  void* aux_out;         // m (SWIGLU_FWD)
  const void* aux_in;    // gu (SWIGLU_BWD)
  // Optional fp32 workspace for the last, partial wave of tiles (see gemm_launch); the launcher
  // sets tail_split, the number of trailing tiles computed as two K halves.
  float* tail_ws;
  size_t tail_ws_bytes;
  int tail_split;
};

// Workspace that lets gemm_launch split a partial last wave of up to kTailMaxTiles tiles
constexpr int kTailMaxTiles = 128;
constexpr size_t kTailWsBytes = (size_t)kTailMaxTiles * 2 * 256 * 256 * 4;

int gemm_check(const GemmArgs& g);
int gemm_launch(const GemmArgs& g, hipStream_t st);

// The MLP's gate/up projection and SwiGLU: gu[M][2F] = x[M][K] W_gu^T (W_gu [2F][K], gate rows
// first, row stride ldw), m[M][F] = silu(g) u. One fused launch when the pipelined kernel
// applies, else the GEMM and the elementwise kernel; the results are the same bits either way.
int gemm_swiglu_fwd(int M, int F, int K, const void* x, int ldx, const void* w, int ldw, void* gu,
                    void* m, int dtype, const char* name, int site, hipStream_t st);
// The down projection's input gradient and SwiGLU's backward: dm = dy[M][K] W_d (W_d [K][F]),
// dgu[M][2F] = (dm * u * silu'(g), dm * silu(g)) from gu. dm_ws ([M][F], 16-byte aligned) is
// written only when the fused launch does not apply.
int gemm_swiglu_bwd(int M, int F, int K, const void* dy, int lddy, const void* w, int ldw,
                    const void* gu, void* dgu, void* dm_ws, int dtype, const char* name, int site,
                    hipStream_t st);
// whether gemm_swiglu_bwd writes dm_ws for these sizes
bool gemm_swiglu_bwd_needs_dm(int M, int F, int dtype);

}  // namespace slide
