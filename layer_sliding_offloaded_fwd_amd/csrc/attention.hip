// Causal grouped-query attention, forward and backward, on the packed qkv buffer of a layer
// (rows of (nq + 2 nkv) * d: q heads, then k heads, then v heads). Query head h reads kv head
// h / (nq / nkv); scores are scaled by 1/sqrt(d); key j is visible to query i iff j <= i.
// The pages leave attention itself unspecified (they optimise RoPE, RMSNorm and SwiGLU around
// it: SlideFormer summary, section 2C); this is the standard definition for the Llama family.
//
// 16-bit path (bf16 or fp16 operands: gfx950 MFMA v_mfma_f32_32x32x16_bf16 / _f16, fp32
// accumulation, flash-style, no [S, S] tensor in memory):
//  * every operand tile is [64 rows][d] of q, k, v or dO rows, copied global -> LDS by
//    direct-to-LDS buffer loads into 2 pipelined stages (the next block in flight while one is
//    computed); the range check of the buffer descriptor turns rows past the sequence into
//    zeros. The forward and dQ kernels are held to 256 registers per lane so that two
//    workgroups share a compute unit: one wave's softmax runs beside the other's MFMAs.
//    A tile is read either as rows (16-byte reads: MFMA fragments of q, k, v or dO) or, through
//    the LDS transpose read ds_read_b64_tr_b16, as columns (fragments of v^T, k^T, q^T, dO^T),
//    so no operand is ever transposed in registers. The 16-byte chunks of row r are XOR-swizzled
//    by f(r) (d = 64: 2(r&3) ^ ((r>>2)&3); d = 128: 2(r&3) ^ 5((r>>2)&3)), which keeps both read
//    kinds free of bank conflicts.
//  * forward and dQ: 128 queries per workgroup (32 per wave), keys in blocks of 64. Each wave
//    computes S^T = K Q^T so that a lane owns one query: row max / row sum are in-lane plus one
//    exchange with the lane 32 away. O^T += V^T P^T (and dQ^T += K^T dS^T) take P (dS) straight
//    from the score accumulators as the B operand; the 16 keys an MFMA consumes are ordered the
//    way the accumulator holds them, and the transpose reads fetch V^T (K^T) in that order.
//  * dK and dV: two workgroup bodies (one accumulator each, so each fits 256 registers) in one
//    launch, 128 keys per workgroup, looping over the G query heads of the kv group and over
//    the query blocks on or after the diagonal, so dK and dV are summed without atomics (the
//    result is deterministic). dQ runs as its own kernel. Every grid is flat and ordered
//    heaviest block first.
//  * D_i = rowsum(dO_i * O_i) is formed in the dQ kernel's prologue (which holds the dO rows) and
//    written, with the log-sum-exps in log2 units, for the dK/dV kernel.
// fp32 path (the small fp32 configuration): straightforward SIMT kernels, one thread per query
// (forward, dQ) or per key (dK/dV).
#include "attention.h"

namespace slide {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// the forward's running maximum (log2 units) lags the true one by at most this much
constexpr float kLazy = 8.0f;
// LDS stages of the key (or query) block pipeline: two (64 KB at d = 128), so that two
// workgroups (two waves per SIMD) fit a compute unit
constexpr int NSTAGE = 2;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_s4_t;
typedef __attribute__((address_space(3))) void lds_void_t;


template <int D>
__device__ __forceinline__ int fsw(int r) {
  return D == 128 ? ((2 * (r & 3)) ^ (5 * ((r >> 2) & 3))) : ((2 * (r & 3)) ^ ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {  // element offset of (row, 16-B chunk c)
  return r * D + ((c ^ fsw<D>(r)) << 3);
}

// Buffer descriptor of nbytes of global memory from p: a raw buffer load whose byte offset
// reaches nbytes is out of range and returns zeros (the range check of raw buffer accesses).
// Every field is uniform; readfirstlane keeps the compiler from building the descriptor in
// vector registers (and looping over lanes to use it). Word 3: 32-bit data format, the value
// for raw buffer accesses on this architecture family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* p, int nbytes) {
  const int nrec = __builtin_amdgcn_readfirstlane(nbytes > 0 ? nbytes : 0);
  const uintptr_t a = (uintptr_t)p;
  const uintptr_t au = ((uintptr_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc((void*)au, (short)0, nrec, 0x00020000);
}
// Rows [row0, row0 + nvalid) of a strided 16-bit matrix whose columns of interest start at g:
// loads of rows at or past nvalid return zeros, which is how a sequence's partial last block
// reads as zero rows. Each row's D columns end within its stride, so every in-range row is
// whole.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* g, int stride, int row0,
                                                          int nvalid) {
  return span_rsrc((const char*)g + (size_t)row0 * stride * 2, nvalid * stride * 2);
}

// Per-wave direct-to-LDS loads of a [64][D] tile (rows row0.. of a strided global matrix; rows
// at or past nvalid read as zeros). The tile's D*128 bytes are split into 1 KB wave loads; wave
// w issues loads w, w+4, ... . Across a wave's loads a lane keeps the same row within the load
// and the same swizzled chunk (the swizzle depends on the row mod 16, and the loads are 16 rows
// apart for d = 128, 32 for d = 64), so its byte offsets differ by a constant and the base is
// one descriptor in scalar registers.
template <int D>
__device__ __forceinline__ void tile_issue(bf16_t* tile, const bf16_t* g, int stride, int row0,
                                           int nvalid, int wave, int lane) {
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int RPL = 64 / CH;          // rows per 1 KB wave load
  constexpr int LOADS = 64 / RPL;       // wave loads per tile
  constexpr int PW = LOADS / 4;         // loads per wave
  static_assert((4 * RPL) % 16 == 0, "a wave's loads keep the row mod 16");
  const int rl = wave * RPL + lane / CH;
  const int c = (lane % CH) ^ fsw<D>(rl);
  const uint32_t voff = (uint32_t)(rl * stride + c * 8) * 2u;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(g, stride, row0, nvalid);
#pragma unroll
  for (int j = 0; j < PW; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + (wave + 4 * j) * 512), 16,
                                             voff + (uint32_t)(j * 4 * RPL * stride * 2), 0, 0,
                                             0);
}
template <int D> constexpr int tile_loads_per_wave() { return (64 / (64 / (D / 8))) / 4; }

// 16-byte row read: row r, chunk c (8 consecutive columns)
template <int D>
__device__ __forceinline__ bf16x8_t rows_read(const bf16_t* t, int r, int c) {
  return *(const bf16x8_t*)(t + tile_off<D>(r, c));
}

// LDS transpose read ds_read_b64_tr_b16 issued through inline asm. (With direct-to-LDS loads in
// flight the compiler would otherwise drain every outstanding load before each transpose read,
// including the next stages', which serializes the pipeline.) The result is only valid after
// tr_wait() on it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ short4_t tr_issue(const bf16_t* p) {
  short4_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(lds_addr(p)));
  return v;
}
// Wait for all outstanding LDS reads of this wave, then pin the N values after the wait so that
// no use of them can be scheduled before it.
template <int N>
__device__ __forceinline__ void tr_wait(bf16x8_t (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}
// The same with the last K LDS operations of this wave still in flight (the reads of the next
// step, issued after v's): LDS operations complete in order, so v's have landed. Only for code
// with no scalar memory loads outstanding, which share the counter and complete out of order.
template <int K, int N>
__device__ __forceinline__ void tr_wait_keep(bf16x8_t (&v)[N]) {
  static_assert(K >= 0 && K < 16, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(K) : "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Column fragment through two transpose reads: A operand of an MFMA whose row index is the tile
// column d0 + lane%32 and whose 8 k values are tile rows 16ks + 4h + {0..3} and
// 16ks + 8 + 4h + {0..3} (h = lane/32), i.e. the key order of a score accumulator.
template <int D>
__device__ __forceinline__ bf16x8_t t_read(const bf16_t* t, int d0, int ks, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int col = d0 + 16 * (g & 1) + 4 * (i & 3);
  const int r0 = ks * 16 + 4 * (g >> 1) + (i >> 2);
  const int r1 = r0 + 8;
  const short4_t lo = tr_issue(t + tile_off<D>(r0, col >> 3) + (col & 7));
  const short4_t hi = tr_issue(t + tile_off<D>(r1, col >> 3) + (col & 7));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// The same column fragment from per-lane byte offsets computed once: the swizzle depends on the
// row mod 16, so a k step (16 rows) moves both reads by 32 D bytes, which the instruction takes
// as an immediate offset, and only the stage's base is added per block.
template <int D>
struct ColOffs {
  uint32_t o[D / 32][2];
  __device__ __forceinline__ explicit ColOffs(int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int r0 = 4 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * (g & 1) + 4 * (i & 3);
      o[db][0] = 2u * (uint32_t)(tile_off<D>(r0, col >> 3) + (col & 7));
      o[db][1] = 2u * (uint32_t)(tile_off<D>(r0 + 8, col >> 3) + (col & 7));
    }
  }
};
template <int D>
__device__ __forceinline__ short4_t tr_issue_ks(uint32_t addr, int ks) {
  short4_t v;
  switch (ks) {   // ks is a constant of the unrolled caller
    case 0: asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr)); break;
    case 1: asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(32 * D)); break;
    case 2: asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(64 * D)); break;
    default: asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(96 * D)); break;
  }
  return v;
}
template <int D>
__device__ __forceinline__ bf16x8_t t_read_at(uint32_t tile, const ColOffs<D>& co, int db, int ks) {
  const short4_t lo = tr_issue_ks<D>(tile + co.o[db][0], ks);
  const short4_t hi = tr_issue_ks<D>(tile + co.o[db][1], ks);
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// score accumulator element i of sub-block kb (32 keys) -> key offset within the 64-key block
__device__ __forceinline__ int acc_key(int kb, int i, int hf) {
  return kb * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
}

// 2^x by the hardware instruction alone. exp2f adds a range reduction so that results below
// 2^-126 come out as denormals; here such values are weights next to a row maximum of 1 and
// contribute nothing, so the flush to zero is immaterial.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held by the lane 32 away (the other half of a score column):
// v_permlane32_swap hands every lane the pair (value of lane l mod 32, value of lane l mod 32 +
// 32) without a trip through the LDS. The pair is combined in the same order in both halves, and
// max and + are commutative, so every lane gets the same bits as with a shuffle.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// Wait until at most `later` stages of `per` loads each are still outstanding.
template <int PER>
__device__ __forceinline__ void wait_stage(int later) {
  if (later >= 2) wait_vm<(2 * PER < 16 ? 2 * PER : 15)>();
  else if (later == 1) wait_vm<PER>();
  else wait_vm<0>();
}
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Stage a wave's 32 x D output tile (held transposed in accumulators) through LDS and write
// 16-byte row chunks: out row r (0..31) of this wave goes to dst + (row0 + r) * stride.
template <int D, int DT>
__device__ __forceinline__ void store_tile_t(bf16_t* stage, const f32x16_t* acc, float scale,
                                             bf16_t* dst, int stride, int row0, int nvalid,
                                             int lane) {
  constexpr int LS = D + 8;
  const int lr = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = db * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
      stage[lr * LS + d] = Bits16<DT>::from_f(acc[db][e] * scale);
    }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  for (int id = lane; id < 32 * (D / 8); id += 64) {
    const int r = id / (D / 8), c = id % (D / 8);
    if (r < nvalid) *(uint4*)(dst + (size_t)(row0 + r) * stride + c * 8) = *(const uint4*)(stage + r * LS + c * 8);
  }
}

__device__ __forceinline__ bf16x8_t zero8() { return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0)); }

template <int D> constexpr int stage_elems() { return 128 * (D + 8); }
template <int D> constexpr int smem_elems(int tiles) {
  return NSTAGE * tiles * 64 * D > stage_elems<D>() ? NSTAGE * tiles * 64 * D : stage_elems<D>();
}

// ------------------------------------------------------------------ forward
template <int D, int DT>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const bf16_t* __restrict__ qkv,
                                                       bf16_t* __restrict__ out,
                                                       float* __restrict__ lse, int S, int nq,
                                                       int nkv, float scale) {
  constexpr int NKK = D / 16, NDB = D / 32, PER = 2 * tile_loads_per_wave<D>();
  __shared__ __attribute__((aligned(1024))) bf16_t smem[smem_elems<D>(2)];
  auto tK = [&](int b) { return smem + b * 2 * 64 * D; };
  auto tV = [&](int b) { return smem + b * 2 * 64 * D + 64 * D; };

  // one flat grid, heaviest (latest) query blocks of every head and sequence first: the
  // hardware dispatches in order, so the light blocks fill the compute units at the end
  const int nqb = (S + 127) / 128;
  const int per = gridDim.x / nqb;       // heads x sequences
  const int qb = nqb - 1 - (int)blockIdx.x / per;
  const int h = (int)blockIdx.x % per % nq, b = (int)blockIdx.x % per / nq;
  const int g = h / (nq / nkv);
  const int QS = (nq + 2 * nkv) * D;
  const int lane = threadIdx.x & 63, hf = lane >> 5, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wq0 = qb * 128 + wave * 32;
  const int q = wq0 + lr;
  const bf16_t* base = qkv + (size_t)b * S * QS;
  const float sl2 = scale * kLog2e;

  bf16x8_t qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = q < S ? *(const bf16x8_t*)(base + (size_t)q * QS + h * D + kk * 16 + hf * 8) : zero8();

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m2 = -INFINITY, l = 0.f;
  const ColOffs<D> co(lane);

  const int q_last = min(S - 1, qb * 128 + 127);
  const int nkvb = q_last / 64 + 1;
  const bf16_t* kbase = base + (nq + g) * D;
  const bf16_t* vbase = base + (nq + nkv + g) * D;
  auto issue = [&](int jb) {
    const int kv0 = jb * 64, st = jb % NSTAGE;
    tile_issue<D>(tK(st), kbase, QS, kv0, min(64, S - kv0), wave, lane);
    tile_issue<D>(tV(st), vbase, QS, kv0, min(64, S - kv0), wave, lane);
  };
#pragma unroll
  for (int j = 0; j < NSTAGE - 1; ++j)
    if (j < nkvb) issue(j);

  for (int jb = 0; jb < nkvb; ++jb) {
    const int kv0 = jb * 64;
    wait_stage<PER>(min(nkvb - 1, jb + NSTAGE - 2) - jb);
    plain_barrier();
    if (jb + NSTAGE - 1 < nkvb) issue(jb + NSTAGE - 1);
    if (kv0 > wq0 + 31) continue;  // every key of this block is after every query of the wave
    const bf16_t* sK = tK(jb % NSTAGE);
    const bf16_t* sV = tV(jb % NSTAGE);

    // the two 32-key halves alternate, so consecutive MFMAs do not depend on each other and
    // each K-row read has a step more to arrive
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = mfma32<DT>(rows_read<D>(sK, kb * 32 + lr, kk * 2 + hf), qf[kk], sacc[kb]);
    // V^T fragments of the first 16 keys: they do not depend on the scores, so they are read
    // before the softmax, whose VALU work covers their latency; each later step's are read
    // while the previous step's MFMAs run
    bf16x8_t vt[2][NDB];
    const uint32_t aV = lds_addr(sV);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vt[0][db] = t_read_at<D>(aV, co, db, 0);
    // the mask only on blocks that reach the diagonal or the end (one branch per block, not
    // one per score)
    const bool need_mask = (kv0 + 63 > wq0) || (kv0 + 64 > S);
    // The row maximum is taken over the raw scores and scaled once: the scale is positive and
    // rounding is monotonic, so this is the maximum of the scaled scores, and the scale goes
    // into each exponent's argument as a fused multiply-add.
    float mx = -INFINITY;
    if (need_mask) {
      // key kv0 + acc_key(kb, i, hf) is masked iff it is past min(q, S - 1); acc_key without
      // its lane term is a constant of the unrolled loop
      const int lim = min(q, S - 1) - kv0 - hf * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float s = acc_key(kb, i, 0) > lim ? -INFINITY : sacc[kb][i];
          sacc[kb][i] = s;
          mx = fmaxf(mx, s);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    }
    mx = halves_max(mx) * sl2;
    // The reference maximum m2 of the exponents moves only when some lane's block maximum
    // exceeds it by more than 2^kLazy: otherwise the weights exp2(s - m2) stay at most 2^kLazy
    // (no overflow in fp32 or in the 16-bit P), and O and l keep their scale, so the rescale of
    // O (64 products per lane) is skipped for the wave. O / l and the log-sum-exp m2 + log2 l
    // do not depend on which reference is used. The first block always moves it (m2 = -inf).
    if (__builtin_amdgcn_ballot_w64(mx > m2 + kLazy) != 0) {
      const float m_new = fmaxf(m2, mx);
      const float alpha = fast_exp2(m2 - (m_new == -INFINITY ? 0.f : m_new));
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      m2 = m_new;
    }
    const float m_use = m2 == -INFINITY ? 0.f : m2;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[kb][i], sl2, -m_use));
        sacc[kb][i] = p;
        rs += p;
      }
    l += halves_sum(rs);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = sacc[ks >> 1][8 * (ks & 1) + j];
      const bf16x8_t pf = pack8<DT>(pv);
      if (ks < 3) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) vt[(ks + 1) & 1][db] = t_read_at<D>(aV, co, db, ks + 1);
        tr_wait_keep<2 * NDB>(vt[ks & 1]);     // two transpose reads per fragment
      } else {
        tr_wait(vt[ks & 1]);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32<DT>(vt[ks & 1][db], pf, oacc[db]);
    }
  }
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  if (hf == 0 && q < S) lse[((size_t)b * nq + h) * S + q] = m2 * kLn2 + logf(l);
  wait_vm<0>();
  __syncthreads();
  bf16_t* stage = smem + wave * 32 * (D + 8);
  store_tile_t<D, DT>(stage, oacc, inv_l, out + (size_t)b * S * nq * D + h * D, nq * D, wq0,
                  min(32, S - wq0), lane);
}

// ------------------------------------------------------------------ D = rowsum(dO * O)
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 u = *(const uint4*)p;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<f16_t>(const f16_t* p, float (&v)[8]) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 h = *(const h8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// D_i = rowsum(dO_i * O_i): the (token, head) rows of o and dO are contiguous runs of D values;
// D / 8 lanes per row, 8 values (one 16- or 32-byte load) per lane, then a shuffle tree.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T* __restrict__ o,
                                                         const T* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         float* __restrict__ delta,
                                                         float* __restrict__ lse2, int B, int S,
                                                         int nq) {
  constexpr int LPR = D / 8;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / LPR;
  const int sub = (int)(gid % LPR);
  const bool ok = row < (size_t)B * S * nq;
  float s = 0.f;
  if (ok) {
    float a[8], c[8];
    load8<T>(o + row * D + sub * 8, a);
    load8<T>(dout + row * D + sub * 8, c);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += a[i] * c[i];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (ok && sub == 0) {
    const size_t t = row / nq;
    const int h = (int)(row % nq);
    const int b = (int)(t / S), sp = (int)(t % S);
    const size_t at = ((size_t)b * nq + h) * S + sp;
    delta[at] = s;
    lse2[at] = lse[at] * kLog2e;
  }
}

// ------------------------------------------------------------------ dQ
template <int D, int DT>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(const bf16_t* __restrict__ qkv,
                                                      const bf16_t* __restrict__ dout,
                                                      const bf16_t* __restrict__ o,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ delta_out,
                                                      float* __restrict__ lse2_out,
                                                      bf16_t* __restrict__ dqkv, int S, int nq,
                                                      int nkv, float scale) {
  constexpr int NKK = D / 16, NDB = D / 32, PER = 2 * tile_loads_per_wave<D>();
  __shared__ __attribute__((aligned(1024))) bf16_t smem[smem_elems<D>(2)];
  auto tK = [&](int b) { return smem + b * 2 * 64 * D; };
  auto tV = [&](int b) { return smem + b * 2 * 64 * D + 64 * D; };

  const int nqb = (S + 127) / 128;       // flat grid, heaviest first (as in the forward)
  const int per = gridDim.x / nqb;
  const int qb = nqb - 1 - (int)blockIdx.x / per;
  const int h = (int)blockIdx.x % per % nq, b = (int)blockIdx.x % per / nq;
  const int g = h / (nq / nkv);
  const int QS = (nq + 2 * nkv) * D, OS = nq * D;
  const int lane = threadIdx.x & 63, hf = lane >> 5, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wq0 = qb * 128 + wave * 32;
  const int q = wq0 + lr;
  const bf16_t* base = qkv + (size_t)b * S * QS;
  const bf16_t* dobase = dout + (size_t)b * S * OS;
  const float sl2 = scale * kLog2e;

  bf16x8_t qf[NKK], df[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = q < S ? *(const bf16x8_t*)(base + (size_t)q * QS + h * D + kk * 16 + hf * 8) : zero8();
    df[kk] = q < S ? *(const bf16x8_t*)(dobase + (size_t)q * OS + h * D + kk * 16 + hf * 8) : zero8();
  }
  const ColOffs<D> co(lane);
  // D = rowsum(dO * O) of this lane's query: the lane holds half of its dO row (d = 16 kk + 8 hf
  // .. + 7), reads O at the same places, and the lane 32 away adds the other half. D and the
  // log-sum-exp in log2 units go to the workspace for the dK/dV kernel, which runs after this.
  float dsum = 0.f;
  if (q < S) {
    const bf16_t* orow = o + ((size_t)b * S + q) * OS + h * D + hf * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const auto ov = __builtin_bit_cast(short8_t, *(const bf16x8_t*)(orow + kk * 16));
      const auto dv = __builtin_bit_cast(short8_t, df[kk]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dsum += Bits16<DT>::to_f((uint16_t)ov[i]) * Bits16<DT>::to_f((uint16_t)dv[i]);
    }
  }
  const float dl = halves_sum(dsum);
  const size_t at = ((size_t)b * nq + h) * S + q;
  const float lse2 = q < S ? lse[at] * kLog2e : 0.f;
  if (hf == 0 && q < S) {
    delta_out[at] = dl;
    lse2_out[at] = lse2;
  }

  f32x16_t dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;

  const int q_last = min(S - 1, qb * 128 + 127);
  const int nkvb = q_last / 64 + 1;
  const bf16_t* kbase = base + (nq + g) * D;
  const bf16_t* vbase = base + (nq + nkv + g) * D;
  auto issue = [&](int jb) {
    const int kv0 = jb * 64, st = jb % NSTAGE;
    tile_issue<D>(tK(st), kbase, QS, kv0, min(64, S - kv0), wave, lane);
    tile_issue<D>(tV(st), vbase, QS, kv0, min(64, S - kv0), wave, lane);
  };
#pragma unroll
  for (int j = 0; j < NSTAGE - 1; ++j)
    if (j < nkvb) issue(j);

  for (int jb = 0; jb < nkvb; ++jb) {
    const int kv0 = jb * 64;
    wait_stage<PER>(min(nkvb - 1, jb + NSTAGE - 2) - jb);
    plain_barrier();
    if (jb + NSTAGE - 1 < nkvb) issue(jb + NSTAGE - 1);
    if (kv0 > wq0 + 31) continue;
    const bf16_t* sK = tK(jb % NSTAGE);
    const bf16_t* sV = tV(jb % NSTAGE);

    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[kb][e] = 0.f;
        pacc[kb][e] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        sacc[kb] = mfma32<DT>(rows_read<D>(sK, kb * 32 + lr, kk * 2 + hf), qf[kk], sacc[kb]);
        pacc[kb] = mfma32<DT>(rows_read<D>(sV, kb * 32 + lr, kk * 2 + hf), df[kk], pacc[kb]);
      }
    }
    // The mask only in blocks on the diagonal or at the end of the sequence, as one branch per
    // block that sets masked scores to -inf (exp2 gives 0; every dP is finite, rows past the end
    // being zeros): key kv0 + acc_key(kb, i, hf) is masked iff it is past the query (which also
    // covers keys past the end), and every key is masked for a query past the end.
    const bool need_mask = (kv0 + 63 > wq0) || (kv0 + 64 > S) || (wq0 + 32 > S);
    if (need_mask) {
      const int lim = (q < S ? q : -1) - kv0 - hf * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (acc_key(kb, i, 0) > lim) sacc[kb][i] = -INFINITY;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sacc[kb][i] = fast_exp2(fmaf(sacc[kb][i], sl2, -lse2)) * (pacc[kb][i] - dl);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float sv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = sacc[ks >> 1][8 * (ks & 1) + j];
      const bf16x8_t sf = pack8<DT>(sv);
      bf16x8_t kt[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) kt[db] = t_read_at<D>(lds_addr(sK), co, db, ks);
      tr_wait(kt);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dq[db] = mfma32<DT>(kt[db], sf, dq[db]);
    }
  }
  wait_vm<0>();
  __syncthreads();
  bf16_t* stage = smem + wave * 32 * (D + 8);
  store_tile_t<D, DT>(stage, dq, scale, dqkv + (size_t)b * S * QS + h * D, QS, wq0, min(32, S - wq0),
                  lane);
}

// ------------------------------------------------------------------ dK, dV
// One workgroup body per output: MODE_DV accumulates dV = sum P^T dO, MODE_DK accumulates
// dK = scale * sum dS^T Q with dS = P (dP - D). Each recomputes the scores it needs; split this
// way a wave holds one 32 x d accumulator instead of two, and both stay within 256 registers
// per lane, so two workgroups share a compute unit.
constexpr int MODE_DV = 0, MODE_DK = 1;

template <int D, int MODE, int DT>
__device__ __forceinline__ void dkv_block(bf16_t* smem, float (*sL)[64], float (*sDl)[64],
                                          int kblk, int g, int b,
                                          const bf16_t* __restrict__ qkv,
                                          const bf16_t* __restrict__ dout,
                                          const float* __restrict__ lse2,
                                          const float* __restrict__ delta,
                                          bf16_t* __restrict__ dqkv, int S, int nq, int nkv,
                                          float scale) {
  constexpr bool DK = MODE == MODE_DK;
  constexpr int NKK = D / 16, NDB = D / 32, PER = 2 * tile_loads_per_wave<D>();
  auto tQ = [&](int b) { return smem + b * 2 * 64 * D; };
  auto tO = [&](int b) { return smem + b * 2 * 64 * D + 64 * D; };  // dO rows

  const int G = nq / nkv;
  const int QS = (nq + 2 * nkv) * D, OS = nq * D;
  const int lane = threadIdx.x & 63, hf = lane >> 5, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k0 = kblk * 128;
  const int wk0 = k0 + wave * 32;
  const int key = wk0 + lr;
  const bf16_t* base = qkv + (size_t)b * S * QS;
  const bf16_t* dobase = dout + (size_t)b * S * OS;
  const float sl2 = scale * kLog2e;

  bf16x8_t kf[NKK], vf[DK ? NKK : 1];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    kf[kk] = key < S ? *(const bf16x8_t*)(base + (size_t)key * QS + (nq + g) * D + kk * 16 + hf * 8) : zero8();
    if constexpr (DK)
      vf[kk] = key < S ? *(const bf16x8_t*)(base + (size_t)key * QS + (nq + nkv + g) * D + kk * 16 + hf * 8) : zero8();
  }
  const ColOffs<D> co(lane);
  f32x16_t acc[NDB];   // dK or dV, transposed: [d][key]
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;

  // flattened (head of the group, query block on or after the diagonal) sequence
  const int qb0 = k0 / 64, nqblk = (S + 63) / 64, per_head = nqblk - qb0;
  const int total = G * per_head;
  auto issue = [&](int it) {
    const int hh = it / per_head, jb = qb0 + it % per_head, st = it % NSTAGE;
    const int h = g * G + hh, q0 = jb * 64, nvalid = min(64, S - q0);
    tile_issue<D>(tQ(st), base + h * D, QS, q0, nvalid, wave, lane);
    tile_issue<D>(tO(st), dobase + h * D, OS, q0, nvalid, wave, lane);
    // the block's log-sum-exp in log2 units (wave 0) and D = rowsum(dO * O) (wave 1), 4 bytes
    // per lane; queries past the sequence read zeros
    if (wave < 2) {
      const float* src = (wave == 0 ? lse2 : delta) + ((size_t)b * nq + h) * S + q0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(span_rsrc(src, (S - q0) * 4),
                                               (lds_void_t*)(wave == 0 ? sL[st] : sDl[st]), 4,
                                               (uint32_t)lane * 4u, 0, 0, 0);
    }
  };
#pragma unroll
  for (int j = 0; j < NSTAGE - 1; ++j)
    if (j < total) issue(j);

  for (int it = 0; it < total; ++it) {
    const int jb = qb0 + it % per_head, st = it % NSTAGE;
    const int q0 = jb * 64;
    const int later = min(total - 1, it + NSTAGE - 2) - it;
    if (wave < 2) wait_stage<PER + 1>(later);  // waves 0 and 1 issue one extra load per stage
    else wait_stage<PER>(later);
    plain_barrier();
    if (it + NSTAGE - 1 < total) issue(it + NSTAGE - 1);
    if (q0 + 63 < wk0) continue;  // every query of this block precedes every key of the wave
    const bf16_t* sQ = tQ(st);
    const bf16_t* sO = tO(st);

    const bool need_mask = (q0 < wk0 + 31) || (q0 + 64 > S) || (wk0 + 32 > S);
    // the 64 queries in two halves of 32
#pragma unroll
    for (int qb2 = 0; qb2 < 2; ++qb2) {
      f32x16_t sacc, pacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[e] = 0.f;
        pacc[e] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        sacc = mfma32<DT>(rows_read<D>(sQ, qb2 * 32 + lr, kk * 2 + hf), kf[kk], sacc);
        if constexpr (DK)
          pacc = mfma32<DT>(rows_read<D>(sO, qb2 * 32 + lr, kk * 2 + hf), vf[kk], pacc);
      }
      // dV += P^T dO (columns of dO), dK += dS^T Q (columns of Q), in two steps of 16 queries.
      // The column reads do not depend on the scores: the first step's (both steps' for dV,
      // which has the registers) are issued before the softmax so that it covers their latency.
      const bf16_t* sT = DK ? sQ : sO;
      bf16x8_t tf0[NDB], tf1[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) tf0[db] = t_read_at<D>(lds_addr(sT), co, db, 2 * qb2);
      if constexpr (!DK) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          tf1[db] = t_read_at<D>(lds_addr(sT), co, db, 2 * qb2 + 1);
      }
      // element i is (query q0 + acc_key(qb2, i), this lane's key). Query q0 + acc_key(qb2, i,
      // hf) is masked iff it precedes this lane's key or is past the end: a compare pair and a
      // select per score, only in the blocks on the diagonal or at the end of the sequence.
      const int lo = key - q0 - hf * 4, hi = S - 1 - q0 - hf * 4;
      if constexpr (DK) {
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ql = acc_key(qb2, i, hf), c = acc_key(qb2, i, 0);
            float p = fast_exp2(fmaf(sacc[i], sl2, -sL[st][ql]));
            p = (c < lo || c > hi) ? 0.f : p;
            sacc[i] = p * (pacc[i] - sDl[st][ql]);   // dS
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ql = acc_key(qb2, i, hf);
            const float p = fast_exp2(fmaf(sacc[i], sl2, -sL[st][ql]));
            sacc[i] = p * (pacc[i] - sDl[st][ql]);   // dS
          }
        }
      } else {
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ql = acc_key(qb2, i, hf), c = acc_key(qb2, i, 0);
            const float p = fast_exp2(fmaf(sacc[i], sl2, -sL[st][ql]));
            sacc[i] = (c < lo || c > hi) ? 0.f : p;                    // P
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sacc[i] = fast_exp2(fmaf(sacc[i], sl2, -sL[st][acc_key(qb2, i, hf)]));   // P
        }
      }
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = sacc[j];
      const bf16x8_t wf0 = pack8<DT>(w);
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = sacc[8 + j];
      const bf16x8_t wf1 = pack8<DT>(w);
      tr_wait(tf0);
      if constexpr (DK) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          tf1[db] = t_read_at<D>(lds_addr(sT), co, db, 2 * qb2 + 1);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma32<DT>(tf0[db], wf0, acc[db]);
      tr_wait(tf1);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma32<DT>(tf1[db], wf1, acc[db]);
    }
  }
  wait_vm<0>();
  __syncthreads();
  bf16_t* stage = smem + wave * 32 * (D + 8);
  const int nv = min(32, S - wk0);
  if (nv > 0)
    store_tile_t<D, DT>(stage, acc, DK ? scale : 1.0f,
                    dqkv + (size_t)b * S * QS + (nq + (DK ? 0 : nkv) + g) * D, QS, wk0, nv, lane);
}

// dK and dV in one launch, one workgroup per (key block, output, kv head, sequence), in one
// flat grid ordered by key block: the earliest keys, which see the most query blocks, of both
// outputs go first. A key block's work shrinks along the sequence (8 : 1 at S = 1024), so with
// each output launched alone (512 workgroups, all resident at once) every launch waited for its
// heaviest blocks; in one grid the lighter blocks of both fill the compute units behind the
// heavy ones. The two bodies share the LDS and the register budget is their maximum.
template <int D, int DT>
__global__ __launch_bounds__(256, 2) void attn_dkdv_kernel(const bf16_t* __restrict__ qkv,
                                                           const bf16_t* __restrict__ dout,
                                                           const float* __restrict__ lse2,
                                                           const float* __restrict__ delta,
                                                           bf16_t* __restrict__ dqkv, int S,
                                                           int nq, int nkv, float scale) {
  __shared__ __attribute__((aligned(1024))) bf16_t smem[smem_elems<D>(2)];
  __shared__ float sL[NSTAGE][64], sDl[NSTAGE][64];
  const int nkb = (S + 127) / 128;
  const int per = gridDim.x / nkb;     // 2 outputs x kv heads x sequences
  const int kblk = (int)blockIdx.x / per, r = (int)blockIdx.x % per;
  const int mode = r & 1, g = (r >> 1) % nkv, b = (r >> 1) / nkv;
  if (mode == MODE_DK)
    dkv_block<D, MODE_DK, DT>(smem, sL, sDl, kblk, g, b, qkv, dout, lse2, delta, dqkv, S, nq, nkv,
                              scale);
  else
    dkv_block<D, MODE_DV, DT>(smem, sL, sDl, kblk, g, b, qkv, dout, lse2, delta, dqkv, S, nq, nkv,
                              scale);
}

// ------------------------------------------------------------------ fp32 SIMT kernels
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(const float* __restrict__ qkv,
                                                          float* __restrict__ out,
                                                          float* __restrict__ lse, int S, int nq,
                                                          int nkv, float scale) {
  const int q = blockIdx.x * 64 + threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (q >= S) return;
  const int g = h / (nq / nkv), QS = (nq + 2 * nkv) * D;
  const float* base = qkv + (size_t)b * S * QS;
  float qv[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qv[i] = base[(size_t)q * QS + h * D + i] * scale;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= q; ++j) {
    const float* kr = base + (size_t)j * QS + (nq + g) * D;
    const float* vr = base + (size_t)j * QS + (nq + nkv + g) * D;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) s += qv[i] * kr[i];
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn), p = expf(s - mn);
    l = l * a + p;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = o[i] * a + p * vr[i];
    m = mn;
  }
  float* orow = out + ((size_t)b * S + q) * nq * D + h * D;
#pragma unroll
  for (int i = 0; i < D; ++i) orow[i] = o[i] / l;
  lse[((size_t)b * nq + h) * S + q] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(64) void attn_dq_f32_kernel(const float* __restrict__ qkv,
                                                         const float* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ delta,
                                                         float* __restrict__ dqkv, int S, int nq,
                                                         int nkv, float scale) {
  const int q = blockIdx.x * 64 + threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (q >= S) return;
  const int g = h / (nq / nkv), QS = (nq + 2 * nkv) * D, OS = nq * D;
  const float* base = qkv + (size_t)b * S * QS;
  float qv[D], dov[D], dq[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qv[i] = base[(size_t)q * QS + h * D + i];
    dov[i] = dout[((size_t)b * S + q) * OS + h * D + i];
    dq[i] = 0.f;
  }
  const float L = lse[((size_t)b * nq + h) * S + q], Dl = delta[((size_t)b * nq + h) * S + q];
  for (int j = 0; j <= q; ++j) {
    const float* kr = base + (size_t)j * QS + (nq + g) * D;
    const float* vr = base + (size_t)j * QS + (nq + nkv + g) * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      s += qv[i] * kr[i];
      dp += dov[i] * vr[i];
    }
    const float p = expf(s * scale - L);
    const float ds = p * (dp - Dl);
#pragma unroll
    for (int i = 0; i < D; ++i) dq[i] += ds * kr[i];
  }
  float* out = dqkv + ((size_t)b * S + q) * QS + h * D;
#pragma unroll
  for (int i = 0; i < D; ++i) out[i] = dq[i] * scale;
}

template <int D>
__global__ __launch_bounds__(64) void attn_dkv_f32_kernel(const float* __restrict__ qkv,
                                                          const float* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ delta,
                                                          float* __restrict__ dqkv, int S, int nq,
                                                          int nkv, float scale) {
  const int j = blockIdx.x * 64 + threadIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (j >= S) return;
  const int G = nq / nkv, QS = (nq + 2 * nkv) * D, OS = nq * D;
  const float* base = qkv + (size_t)b * S * QS;
  float kv[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    kv[i] = base[(size_t)j * QS + (nq + g) * D + i];
    vv[i] = base[(size_t)j * QS + (nq + nkv + g) * D + i];
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    for (int q = j; q < S; ++q) {
      const float* qr = base + (size_t)q * QS + h * D;
      const float* dor = dout + ((size_t)b * S + q) * OS + h * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s += qr[i] * kv[i];
        dp += dor[i] * vv[i];
      }
      const float p = expf(s * scale - lse[((size_t)b * nq + h) * S + q]);
      const float ds = p * (dp - delta[((size_t)b * nq + h) * S + q]);
#pragma unroll
      for (int i = 0; i < D; ++i) {
        dv[i] += p * dor[i];
        dk[i] += ds * qr[i];
      }
    }
  }
  float* ok = dqkv + ((size_t)b * S + j) * QS + (nq + g) * D;
  float* ov = dqkv + ((size_t)b * S + j) * QS + (nq + nkv + g) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    ok[i] = dk[i] * scale;
    ov[i] = dv[i];
  }
}

}  // namespace

int attention_check(int B, int S, int nq, int nkv, int d, int dtype) {
  SLIDE_REQUIRE(B >= 0 && S >= 0, SLIDE_E_SHAPE, "attention: negative batch or sequence");
  SLIDE_REQUIRE(nq > 0 && nkv > 0 && nq % nkv == 0, SLIDE_E_SHAPE,
                "attention: n_heads %d must be a positive multiple of n_kv_heads %d", nq, nkv);
  SLIDE_REQUIRE(d == 64 || d == 128, SLIDE_E_SHAPE, "attention: head_dim %d (64 or 128)", d);
  SLIDE_REQUIRE(dtype_valid(dtype), SLIDE_E_ARG, "attention: bad dtype");
  return SLIDE_OK;
}

namespace {

template <int DT>
void launch_fwd16(const void* qkv, void* o, float* lse, int B, int S, int nq, int nkv, int d,
                  float scale, hipStream_t st) {
  dim3 grid((unsigned)((S + 127) / 128 * nq * B)), block(256);
  if (d == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, DT>), grid, block, 0, st, (const bf16_t*)qkv,
                       (bf16_t*)o, lse, S, nq, nkv, scale);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, DT>), grid, block, 0, st, (const bf16_t*)qkv,
                       (bf16_t*)o, lse, S, nq, nkv, scale);
}

template <typename T>
void launch_delta(const void* o, const void* dout, const float* lse, float* delta, float* lse2,
                  int B, int S, int nq, int d, hipStream_t st) {
  const size_t rows = (size_t)B * S * nq;
  dim3 grid((unsigned)((rows * (d / 8) + 255) / 256)), block(256);
  if (d == 128)
    hipLaunchKernelGGL((attn_delta_kernel<T, 128>), grid, block, 0, st, (const T*)o,
                       (const T*)dout, lse, delta, lse2, B, S, nq);
  else
    hipLaunchKernelGGL((attn_delta_kernel<T, 64>), grid, block, 0, st, (const T*)o,
                       (const T*)dout, lse, delta, lse2, B, S, nq);
}

template <int DT>
int launch_bwd16(const void* qkv, const void* o, const float* lse, const void* dout, void* dqkv,
                 float* delta, float* lse2, int B, int S, int nq, int nkv, int d, float scale,
                 hipStream_t st) {
  const bf16_t* q = (const bf16_t*)qkv;
  const bf16_t* g = (const bf16_t*)dout;
  bf16_t* out = (bf16_t*)dqkv;
  {
    ProfScope ps("attn_bwd_dq", st);
    dim3 grid((unsigned)((S + 127) / 128 * nq * B)), block(256);
    if (d == 128)
      hipLaunchKernelGGL((attn_dq_kernel<128, DT>), grid, block, 0, st, q, g,
                         (const bf16_t*)o, lse, delta, lse2, out, S, nq, nkv, scale);
    else
      hipLaunchKernelGGL((attn_dq_kernel<64, DT>), grid, block, 0, st, q, g, (const bf16_t*)o,
                         lse, delta, lse2, out, S, nq, nkv, scale);
  }
  SLIDE_TRY(check_launch("attn_bwd_dq"));
  {
    ProfScope ps("attn_bwd_dkv", st);
    dim3 grid((unsigned)((S + 127) / 128 * 2 * nkv * B)), block(256);
    if (d == 128)
      hipLaunchKernelGGL((attn_dkdv_kernel<128, DT>), grid, block, 0, st, q, g, lse2, delta, out, S,
                         nq, nkv, scale);
    else
      hipLaunchKernelGGL((attn_dkdv_kernel<64, DT>), grid, block, 0, st, q, g, lse2, delta, out, S,
                         nq, nkv, scale);
  }
  return check_launch("attn_bwd_dkv");
}

}  // namespace

int attention_fwd(const void* qkv, void* o, float* lse, int B, int S, int nq, int nkv, int d,
                  int dtype, hipStream_t st) {
  if (B == 0 || S == 0) return SLIDE_OK;
  ProfScope ps("attn_fwd", st);
  const float scale = 1.0f / sqrtf((float)d);
  if (dtype == SLIDE_BF16) {
    launch_fwd16<SLIDE_BF16>(qkv, o, lse, B, S, nq, nkv, d, scale, st);
  } else if (dtype == SLIDE_F16) {
    launch_fwd16<SLIDE_F16>(qkv, o, lse, B, S, nq, nkv, d, scale, st);
  } else {
    dim3 grid((S + 63) / 64, nq, B), block(64);
    if (d == 128)
      hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, block, 0, st, (const float*)qkv, (float*)o, lse, S, nq, nkv, scale);
    else
      hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, block, 0, st, (const float*)qkv, (float*)o, lse, S, nq, nkv, scale);
  }
  return check_launch("attn_fwd");
}

// D = rowsum(dO * O) and the log-sum-exps in log2 units, fp32 [B, nq, S] each
size_t attention_bwd_ws(int B, int S, int nq) { return 2 * align_up((size_t)B * nq * S * 4, 256); }

int attention_bwd(const void* qkv, const void* o, const float* lse, const void* dout, void* dqkv,
                  int B, int S, int nq, int nkv, int d, int dtype, void* ws, hipStream_t st) {
  if (B == 0 || S == 0) return SLIDE_OK;
  float* delta = (float*)ws;
  float* lse2 = (float*)((char*)ws + attention_bwd_ws(B, S, nq) / 2);
  const float scale = 1.0f / sqrtf((float)d);
  // 16-bit: the dQ kernel forms D and the log2-unit log-sum-exps itself
  if (dtype == SLIDE_BF16)
    return launch_bwd16<SLIDE_BF16>(qkv, o, lse, dout, dqkv, delta, lse2, B, S, nq, nkv, d,
                                    scale, st);
  if (dtype == SLIDE_F16)
    return launch_bwd16<SLIDE_F16>(qkv, o, lse, dout, dqkv, delta, lse2, B, S, nq, nkv, d, scale,
                                   st);
  {
    ProfScope ps("attn_delta", st);
    SLIDE_DISPATCH(dtype, T, launch_delta<T>(o, dout, lse, delta, lse2, B, S, nq, d, st));
  }
  SLIDE_TRY(check_launch("attn_delta"));
  {
    ProfScope ps("attn_bwd_dq", st);
    dim3 grid((S + 63) / 64, nq, B), block(64);
    if (d == 128)
      hipLaunchKernelGGL(attn_dq_f32_kernel<128>, grid, block, 0, st, (const float*)qkv, (const float*)dout, lse, delta, (float*)dqkv, S, nq, nkv, scale);
    else
      hipLaunchKernelGGL(attn_dq_f32_kernel<64>, grid, block, 0, st, (const float*)qkv, (const float*)dout, lse, delta, (float*)dqkv, S, nq, nkv, scale);
  }
  {
    ProfScope ps("attn_bwd_dkv", st);
    dim3 grid((S + 63) / 64, nkv, B), block(64);
    if (d == 128)
      hipLaunchKernelGGL(attn_dkv_f32_kernel<128>, grid, block, 0, st, (const float*)qkv, (const float*)dout, lse, delta, (float*)dqkv, S, nq, nkv, scale);
    else
      hipLaunchKernelGGL(attn_dkv_f32_kernel<64>, grid, block, 0, st, (const float*)qkv, (const float*)dout, lse, delta, (float*)dqkv, S, nq, nkv, scale);
  }
  return check_launch("attn_bwd");
}

}  // namespace slide

extern "C" int slide_attention_fwd(const void* qkv, void* o, float* lse, int B, int S, int nq,
                                   int nkv, int d, int dtype, void* stream) {
  SLIDE_TRY(slide::attention_check(B, S, nq, nkv, d, dtype));
  SLIDE_REQUIRE(qkv && o && lse, SLIDE_E_ARG, "slide_attention_fwd: null pointer");
  return slide::attention_fwd(qkv, o, lse, B, S, nq, nkv, d, dtype, (hipStream_t)stream);
}

extern "C" size_t slide_attention_bwd_workspace_bytes(int B, int S, int nq) {
  return slide::attention_bwd_ws(B, S, nq);
}

extern "C" int slide_attention_bwd(const void* qkv, const void* o, const float* lse,
                                   const void* d_o, void* dqkv, int B, int S, int nq, int nkv,
                                   int d, int dtype, void* ws, size_t ws_bytes, void* stream) {
  SLIDE_TRY(slide::attention_check(B, S, nq, nkv, d, dtype));
  SLIDE_REQUIRE(qkv && o && lse && d_o && dqkv && ws, SLIDE_E_ARG,
                "slide_attention_bwd: null pointer");
  SLIDE_REQUIRE(ws_bytes >= slide::attention_bwd_ws(B, S, nq), SLIDE_E_WORKSPACE,
                "slide_attention_bwd: workspace %zu < %zu", ws_bytes,
                slide::attention_bwd_ws(B, S, nq));
  return slide::attention_bwd(qkv, o, lse, d_o, dqkv, B, S, nq, nkv, d, dtype, ws,
                              (hipStream_t)stream);
}
