/* slide.h — C ABI of the layer-sliding offloaded fine-tuning hot path for AMD MI355X (gfx950).
 *
 * The method (SlideFormer: "An Efficient Heterogeneous Co-Design for Fine-Tuning on a Single
 * GPU", Yang & Wen; abstract and the gist.science technical summary, section 2) treats the GPU
 * as a sliding window over the decoder layers: a layer's weights are streamed into a fixed queue
 * of pre-allocated GPU buffers, its forward and backward run there, its gradients go back to host
 * memory asynchronously, and a CPU optimizer updates the layer while the GPU runs the backward of
 * the layer below (summary, sections 2A and 2B; figure 3 and figure 4 of the paper page, whose
 * caption states the overlap condition T_bwd >= T_grad_d2h + T_update).
 *
 * Conventions shared by every call
 *  - Return value: SLIDE_OK (0) or a negative SLIDE_E_* code. slide_last_error() returns a
 *    thread-local message describing the last failure on the calling thread. No C++ exception
 *    crosses this boundary.
 *  - Ownership: every device buffer, workspace and pinned host buffer is allocated and owned by
 *    the caller. The library never allocates device memory. It owns only host bookkeeping and
 *    the HIP events inside a ring handle and the profiler.
 *  - Streams and events are passed as `void*` holding a hipStream_t / hipEvent_t (NULL = the
 *    default stream). GPU calls are asynchronous on the given stream; launch failures return
 *    SLIDE_E_HIP. Arguments and shapes are validated on the host before anything is launched.
 *  - Element types: SLIDE_BF16 tensors are uint16 bf16 bit patterns, SLIDE_F16 tensors IEEE
 *    binary16, SLIDE_F32 tensors float. Accumulation, softmax, log-sum-exp and norm statistics
 *    are always fp32.
 *  - Layouts are row-major. A weight matrix W is [out, in] and a projection is y = x W^T.
 *    Activations are [N, features] with N = B*S tokens, token t = b*S + s at position s.
 *  - Device pointers must be 16-byte aligned; feature sizes must be multiples of 8.
 *  - No aliasing between inputs and outputs unless a call says otherwise.
 */
#ifndef SLIDE_H
#define SLIDE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SLIDE_OK = 0,
  SLIDE_E_ARG = -1,          /* null pointer, bad enum or hyper-parameter */
  SLIDE_E_SHAPE = -2,        /* unsupported or inconsistent sizes */
  SLIDE_E_WORKSPACE = -3,    /* workspace too small (see the *_workspace_bytes query) */
  SLIDE_E_HIP = -4,          /* a HIP runtime call or a kernel launch failed */
  SLIDE_E_STATE = -5,        /* slot-ring call not allowed in the slot's current state */
  SLIDE_E_TIMEOUT = -6,      /* a bounded host wait ran out */
  SLIDE_E_UNSUPPORTED = -7,  /* valid request this build does not implement */
  SLIDE_E_NONFINITE = -8,    /* non-finite gradient found where checked (engine option) */
  SLIDE_E_IO = -9            /* a file operation of the disk tier failed (errno in the message) */
};

/* SLIDE_F16: IEEE binary16 compute (the pages name FP16 beside BF16 for the GPU's compute and
 * the host buffers' conversions, summary section 2B), used with dynamic loss scaling. */
typedef enum { SLIDE_F32 = 0, SLIDE_BF16 = 1, SLIDE_F16 = 2 } slide_dtype;

const char* slide_last_error(void);
const char* slide_version(void);

/* ------------------------------------------------------------------------------------------
 * Decoder layer (pre-norm Llama block; the pages name Llama-3, Qwen and Mistral as the models
 * the system fine-tunes, summary section 4, and RoPE / RMSNorm / SwiGLU as its kernels,
 * summary section 2C):
 *   r  = RMSNorm(x; w_attn)               r_t = w * x_t / sqrt(mean(x_t^2) + eps)
 *   q,k,v = split(r Wqkv^T)               rows of Wqkv: n_heads*d q rows, then k, then v
 *   q,k = RoPE(q,k)                       rotate-half pairs (i, i+d/2), angle s*theta^(-2i/d)
 *   o  = softmax(q k^T / sqrt(d) + causal) v   query head h reads kv head h/(n_heads/n_kv_heads)
 *   x2 = x + o Wo^T
 *   r2 = RMSNorm(x2; w_mlp)
 *   g,u = split(r2 Wgu^T)                 rows of Wgu: ffn gate rows, then ffn up rows
 *   y  = x2 + (silu(g) * u) Wd^T
 * Slot packing (one contiguous buffer per layer, elements of cfg.dtype, in this order):
 *   w_attn[H] | Wqkv[(nq+2nkv)d, H] | Wo[H, nq d] | w_mlp[H] | Wgu[2F, H] | Wd[H, F]
 * The gradient buffer of a layer uses the same packing.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  int32_t hidden;      /* H, multiple of 8 */
  int32_t n_heads;     /* nq */
  int32_t n_kv_heads;  /* nkv, divides nq */
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t ffn;         /* F, multiple of 8 */
  int32_t dtype;       /* slide_dtype of weights, activations and gradients */
  float rms_eps;
  float rope_theta;
} slide_layer_cfg;

/* Number of elements in one layer's packed parameters (0 if cfg is invalid). */
size_t slide_layer_param_count(const slide_layer_cfg* cfg);
/* Element offsets of the six packed tensors, in packing order. */
int slide_layer_param_offsets(const slide_layer_cfg* cfg, size_t off[6]);
/* Workspace bytes needed by slide_layer_fwd (bwd = 0), slide_layer_bwd (bwd = 1) or
 * slide_layer_bwd_saved (bwd = 2). */
size_t slide_layer_workspace_bytes(const slide_layer_cfg* cfg, int B, int S, int bwd);

/* Forward of one layer. w_slot: packed weights (device). x, y: [B*S, H] (device), y != x.
 * ws: device workspace of at least slide_layer_workspace_bytes(cfg, B, S, 0) bytes. */
int slide_layer_fwd(const slide_layer_cfg* cfg, const void* w_slot, const void* x, void* y,
                    int B, int S, void* ws, size_t ws_bytes, void* stream);

/* Backward of one layer from its input checkpoint x: the layer's forward is recomputed inside
 * the workspace (only layer inputs are kept between the sweeps), then dx = dL/dx and the packed
 * parameter gradients g_slot = dL/dw are written (g_slot is overwritten, not accumulated).
 * dy may alias dx (dy is fully read before dx is written). ws: at least
 * slide_layer_workspace_bytes(cfg, B, S, 1) bytes. */
int slide_layer_bwd(const slide_layer_cfg* cfg, const void* w_slot, const void* x,
                    const void* dy, void* dx, void* g_slot, int B, int S, void* ws,
                    size_t ws_bytes, void* stream);

/* Keeping the forward's intermediates instead of recomputing them. The pages keep only a small
 * window of activations on the GPU (summary, section 2B, "sliding activations"); with 288 GB of
 * HBM the window can hold every layer's intermediates, which removes the backward's recompute.
 * slide_layer_saved_bytes: bytes of one layer's forward intermediates for B x S tokens.
 * slide_layer_fwd_save: slide_layer_fwd that leaves them in `saved` (caller-owned, per layer).
 * slide_layer_bwd_saved: slide_layer_bwd that reads them from `saved` instead of recomputing;
 * ws needs slide_layer_workspace_bytes(cfg, B, S, 2) bytes. Results are identical to the
 * recompute path given the same inputs. */
size_t slide_layer_saved_bytes(const slide_layer_cfg* cfg, int B, int S);
int slide_layer_fwd_save(const slide_layer_cfg* cfg, const void* w_slot, const void* x, void* y,
                         int B, int S, void* saved, size_t saved_bytes, void* stream);
int slide_layer_bwd_saved(const slide_layer_cfg* cfg, const void* w_slot, const void* x,
                          const void* dy, void* dx, void* g_slot, int B, int S,
                          const void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------------------------------------------
 * Fused LM-head cross-entropy in vocabulary chunks (summary, section 2C: projection and loss
 * fused so that the [N, V] logit tensor never exists).
 *   z = h W^T (chunk by chunk), loss = mean over valid t of (logsumexp(z_t) - z_t[y_t]),
 *   dz = (softmax(z) - onehot(y)) / N_valid, dh = dz W, dW = dz^T h.
 * Targets < 0 are ignored; with no valid target the loss and both gradients are 0.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  int32_t hidden;  /* H, multiple of 8 */
  int32_t vocab;   /* V, multiple of 8 */
  int32_t chunk;   /* vocabulary chunk C (multiple of 8); 0 selects 8192 */
  int32_t dtype;   /* slide_dtype of h, W, dh, dW */
  /* Gradient scale S (dynamic loss scaling of fp16 training): dh and dW are the gradients of S
   * times the mean loss (dz carries S / N_valid); the reported loss is not scaled. 0 means 1. */
  float grad_scale;
} slide_ce_cfg;

size_t slide_lmhead_ce_workspace_bytes(const slide_ce_cfg* cfg, int N);
/* h [N, H], w [V, H], targets int32 [N] (device). loss_dev: one float on the device.
 * dh [N, H] and dw [V, H] may each be NULL to skip that gradient. */
int slide_lmhead_ce(const slide_ce_cfg* cfg, const void* h, const void* w,
                    const int32_t* targets, int N, float* loss_dev, void* dh, void* dw,
                    void* ws, size_t ws_bytes, void* stream);

/* The same computation in host-driven phases over one workspace and one stream, so that a
 * caller can start each vocabulary chunk as soon as that chunk's weights are on the device and
 * ship each chunk of dW as soon as it is computed (the chunked fused cross-entropy of the
 * SlideFormer summary, section 2C, with the chunks exposed). Chunk ci covers vocabulary rows
 * [ci * C, min((ci + 1) * C, V)) with C = cfg->chunk (8192 if 0, at most V).
 *   1. slide_lmhead_ce_stats for every chunk, in any order (pass 1: logits and softmax partials);
 *   2. slide_lmhead_ce_loss (lse per token, the mean loss into loss_dev);
 *   3. slide_lmhead_ce_grad for every chunk in increasing order (pass 2: recomputed logits,
 *      dz, the fp32 dh accumulator in the workspace if with_dh, and rows of dw if dw != NULL;
 *      chunk 0 initialises the accumulator);
 *   4. slide_lmhead_ce_dh once if with_dh was set (dh in the storage type).
 * Arguments mean what they mean for slide_lmhead_ce; ws must hold
 * slide_lmhead_ce_workspace_bytes(cfg, N) bytes and stays owned by the caller. The results are
 * bit-identical to slide_lmhead_ce's. A chunk index outside [0, n_chunks) is SLIDE_E_ARG. */
int slide_lmhead_ce_n_chunks(const slide_ce_cfg* cfg);   /* >= 1, or a negative status */
int slide_lmhead_ce_stats(const slide_ce_cfg* cfg, const void* h, const void* w,
                          const int32_t* targets, int N, int chunk, void* ws, size_t ws_bytes,
                          void* stream);
int slide_lmhead_ce_loss(const slide_ce_cfg* cfg, const int32_t* targets, int N, float* loss_dev,
                         void* ws, size_t ws_bytes, void* stream);
int slide_lmhead_ce_grad(const slide_ce_cfg* cfg, const void* h, const void* w,
                         const int32_t* targets, int N, int chunk, int with_dh, void* dw,
                         void* ws, size_t ws_bytes, void* stream);
int slide_lmhead_ce_dh(const slide_ce_cfg* cfg, int N, void* dh, void* ws, size_t ws_bytes,
                       void* stream);

/* ------------------------------------------------------------------------------------------
 * Model glue around the layers: token embedding and the final RMSNorm.
 * ------------------------------------------------------------------------------------------ */
/* x[t] = E[tokens[t]]; E [V, H], x [N, H]. Tokens outside [0, V) -> SLIDE_E_ARG is not
 * detectable on the host; such rows are written as zeros. */
int slide_embed_fwd(const void* E, const int32_t* tokens, void* x, int N, int H, int V,
                    int dtype, void* stream);
size_t slide_embed_bwd_workspace_bytes(int N, int V);
/* dE = sum over positions of dx rows, grouped by token, summed in position order (so the
 * result is deterministic). dE [V, H] is fully overwritten (rows of absent tokens are 0). */
int slide_embed_bwd(const void* dx, const int32_t* tokens, void* dE, int N, int H, int V,
                    int dtype, void* ws, size_t ws_bytes, void* stream);
/* Row gather / scatter in device memory: row (dst_rows ? dst_rows[k] : k) of dst = row
 * (src_rows ? src_rows[k] : k) of src for k < n_rows, rows of row_bytes (a positive multiple of
 * 16; src and dst 16-byte aligned). src holds src_n_rows rows and dst dst_n_rows; a listed index
 * outside them is skipped (it cannot be checked on the host: the lists are device memory), an
 * implicit one outside them is SLIDE_E_SHAPE. Used to move only the embedding rows a batch
 * selected between the device table and the host (summary, section 2A: transfers kept off the
 * compute path; here the step boundary). */
int slide_copy_rows(const void* src, const int32_t* src_rows, int64_t src_n_rows, void* dst,
                    const int32_t* dst_rows, int64_t dst_n_rows, int64_t n_rows,
                    size_t row_bytes, void* stream);
/* y = RMSNorm(x; w). x, y [N, H]; rstd_out: optional fp32 [N] (may be NULL). */
int slide_rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd_out, int N, int H,
                      float eps, int dtype, void* stream);
size_t slide_rmsnorm_bwd_workspace_bytes(int N, int H);
/* dx = dres + dRMSNorm/dx (dres may be NULL), dw = sum over rows. dw is written, not added. */
int slide_rmsnorm_bwd(const void* dy, const void* x, const void* w, const void* dres, void* dx,
                      void* dw, int N, int H, float eps, int dtype, void* ws, size_t ws_bytes,
                      void* stream);
/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): slide_rmsnorm_bwd with its scratch in a fixed
 * device array of the library instead of a caller workspace. Results are bit-identical to
 * slide_rmsnorm_bwd. Calls no hipMalloc / hipFree. SLIDE_E_WORKSPACE if the call needs more
 * than slide_rmsnorm_bwd_noalloc_max_bytes() (16 MiB) of scratch, i.e. if
 * slide_rmsnorm_bwd_workspace_bytes(N, H) exceeds it. Each GPU has one such array, held until
 * the process ends and shared by every call on that GPU: calls that overlap on one GPU (other
 * streams, other threads) race on it and must be serialized by the caller. */
size_t slide_rmsnorm_bwd_noalloc_max_bytes(void);
int slide_rmsnorm_bwd_noalloc(const void* dy, const void* x, const void* w, const void* dres,
                              void* dx, void* dw, int N, int H, float eps, int dtype,
                              void* stream);

/* ------------------------------------------------------------------------------------------
 * Kernel-level entry points (the building blocks of the layer; used by tests and benches).
 * ------------------------------------------------------------------------------------------ */
/* C[M,N] = alpha * sum_k A(m,k) B(k,n)  (+ R[M,N] if R != NULL) (+ C if accumulate).
 * a_kmajor = 1: A(m,k) = A[m*lda + k] else A[k*lda + m]
 * b_kmajor = 1: B(k,n) = B[n*ldb + k] else B[k*ldb + n]
 * A, B, R in dtype; C in c_dtype (accumulate requires c_dtype = SLIDE_F32). */
int slide_gemm(int M, int N, int K, const void* A, int lda, int a_kmajor, const void* B,
               int ldb, int b_kmajor, void* C, int ldc, int c_dtype, const void* R, int ldr,
               float alpha, int accumulate, int dtype, void* stream);
/* slide_gemm with a workspace of slide_gemm_tail_workspace_bytes() (or NULL): when the last
 * wave of 256 x 256 tiles would occupy at most half of the compute units, those tiles are
 * computed as two halves of K each, whose fp32 partial sums a second launch adds (the first
 * half's plus the second's) before the usual epilogue. Results then differ from slide_gemm's
 * only in the rounding of that one addition; they are deterministic. The layer backward's GEMMs
 * use this with a slice of the layer workspace. */
size_t slide_gemm_tail_workspace_bytes(void);
int slide_gemm_ws(int M, int N, int K, const void* A, int lda, int a_kmajor, const void* B,
                  int ldb, int b_kmajor, void* C, int ldc, int c_dtype, const void* R, int ldr,
                  float alpha, int accumulate, int dtype, void* ws, size_t ws_bytes,
                  void* stream);
/* SwiGLU of the layer's MLP (An Efficient Heterogeneous Co-Design for Fine-Tuning on a Single
 * GPU, the summary's section 2C names SwiGLU among the kernels the system rewrote; the formula is
 * the Llama MLP's): gu [N][2F] holds g in columns 0 .. F-1 and u in F .. 2F-1 of each row,
 * m [N][F] = silu(g) * u with silu(g) = g / (1 + exp(-g)), computed in fp32 from the stored
 * 16-bit (or fp32) values and rounded once. F must be a positive multiple of 8 and every pointer
 * 16-byte aligned; device pointers, caller-owned; stream-ordered. */
int slide_swiglu_fwd(const void* gu, void* m, int N, int F, int dtype, void* stream);
/* Backward: dgu [N][2F] = (dm * u * s * (1 + g (1 - s)), dm * g * s) with s = sigmoid(g). */
int slide_swiglu_bwd(const void* dm, const void* gu, void* dgu, int N, int F, int dtype,
                     void* stream);
/* The gate/up projection fused with SwiGLU: gu = x w_gu^T (x [M][K] row stride ldx, w_gu
 * [2F][K] row stride ldw with the F gate rows first) and m = SwiGLU(gu), both written. For
 * 16-bit dtypes on problems large enough for the pipelined GEMM one launch does both (each tile
 * computes 128 gate and the matching 128 up columns); otherwise slide_gemm's kernel and the
 * elementwise kernel run. The bits are the same either way: m is computed from the 16-bit g, u. */
int slide_gemm_swiglu_fwd(int M, int F, int K, const void* x, int ldx, const void* w_gu, int ldw,
                          void* gu, void* m, int dtype, void* stream);
/* The down projection's input gradient fused with SwiGLU's backward: dm = dy w_down (dy [M][K]
 * row stride lddy, w_down [K][F] row stride ldw), dgu = SwiGLU backward of dm at gu; dm itself is
 * not stored by the fused launch. ws (ws_bytes >= slide_gemm_swiglu_bwd_workspace_bytes, 0 when
 * the fused launch applies) holds dm otherwise. */
size_t slide_gemm_swiglu_bwd_workspace_bytes(int M, int F, int dtype);
int slide_gemm_swiglu_bwd(int M, int F, int K, const void* dy, int lddy, const void* w_down,
                          int ldw, const void* gu, void* dgu, int dtype, void* ws,
                          size_t ws_bytes, void* stream);
/* Causal GQA attention on a packed qkv buffer [B*S, (nq+2nkv)*d] (RoPE already applied).
 * o [B*S, nq*d]; lse fp32 [B, nq, S]. */
int slide_attention_fwd(const void* qkv, void* o, float* lse, int B, int S, int nq, int nkv,
                        int d, int dtype, void* stream);
size_t slide_attention_bwd_workspace_bytes(int B, int S, int nq);
/* dqkv [B*S, (nq+2nkv)*d] fully written (dq, dk, dv before the inverse RoPE). */
int slide_attention_bwd(const void* qkv, const void* o, const float* lse, const void* d_o,
                        void* dqkv, int B, int S, int nq, int nkv, int d, int dtype, void* ws,
                        size_t ws_bytes, void* stream);
/* In-place RoPE on the q and k parts of a packed qkv buffer; inverse = 1 rotates by -angle. */
int slide_rope(void* qkv, int B, int S, int nq, int nkv, int d, float theta, int inverse,
               int dtype, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Slot ring: the pre-allocated GPU cache queue (summary, section 2B: a fixed queue of
 * identical buffers holding only the active layers' parameters and gradients, reused as soon
 * as they are free). Slot k occupies [dev_base + k*(w_bytes+g_bytes), +w_bytes) for weights
 * and the following g_bytes for gradients.
 * Slot states: FREE -> LOADING (load) -> IN_USE (acquire) -> FLUSHING (flush) -> FREE (release)
 *              IN_USE -> FREE (release without a flush, e.g. after a forward).
 * Every transition is stream-ordered: a release records an event on the compute stream and
 * the next load into that slot makes the copy stream wait for it (and for a pending flush), so
 * no call here blocks the host except slide_slot_ring_wait_flush.
 * ------------------------------------------------------------------------------------------ */
typedef struct slide_ring slide_ring;
enum { SLIDE_SLOT_FREE = 0, SLIDE_SLOT_LOADING = 1, SLIDE_SLOT_IN_USE = 2,
       SLIDE_SLOT_FLUSHING = 3 };
/* engine: SLIDE_ENGINE_HIP moves data with hipMemcpyAsync on the h2d / d2h streams;
 * SLIDE_ENGINE_HOST treats dev_base as host memory and copies with memcpy on a host thread
 * (events become host flags), which lets the state machine run and be tested without a GPU;
 * SLIDE_ENGINE_HSA copies on two chosen host-optimised copy engines (one per direction) through
 * the HSA runtime, from a host thread per direction that waits on the host for the HIP events
 * a copy depends on and for the copy's completion (the h2d / d2h streams are unused). With it,
 * slide_slot_ring_acquire blocks the calling thread until the slot's load, and any flush still
 * reading the slot, has completed (at most 60 s, then SLIDE_E_TIMEOUT); no GPU queue waits on
 * the host. dev_base must be device memory and the host buffers pinned memory. */
enum { SLIDE_ENGINE_HIP = 0, SLIDE_ENGINE_HOST = 1, SLIDE_ENGINE_HSA = 2 };
int slide_slot_ring_create(slide_ring** out, int n_slots, size_t w_bytes, size_t g_bytes,
                           void* dev_base, void* h2d_stream, void* d2h_stream, int engine);
/* Pick the next FREE slot (round-robin), start the copy host_w -> slot weights, mark LOADING.
 * The copy is w_bytes long: host_w must span w_bytes bytes (pinned memory for an asynchronous
 * copy), also where the layer's own bytes end before w_bytes.
 * SLIDE_E_STATE if no slot is FREE. */
int slide_slot_ring_load(slide_ring* r, int layer, const void* host_w, int* slot_out);
/* Make `compute_stream` wait for the slot's load; LOADING -> IN_USE. Also returns the slot's
 * weight and gradient device addresses (either out pointer may be NULL). */
int slide_slot_ring_acquire(slide_ring* r, int slot, void* compute_stream, void** w_dev,
                            void** g_dev);
/* After the work on compute_stream that writes the slot's gradients: copy them to host_g on
 * the d2h stream; IN_USE -> FLUSHING. The copy is g_bytes long, so host_g must span g_bytes
 * bytes. *ticket identifies this flush for wait_flush. */
int slide_slot_ring_flush(slide_ring* r, int slot, void* host_g, void* compute_stream,
                          uint64_t* ticket);
/* Part of a load or of a flush, so that a layer's copies, its CPU update and its upload can be
 * pipelined in pieces (summary, section 2A: transfers and updates overlap one another; here the
 * step boundary, where the last layer of the backward is the first of the next forward).
 * load_range: copy weight bytes [offset, offset + nbytes) from host_w + offset (host_w is the
 *   start of the layer's whole host buffer). *slot_inout < 0 starts a load on the next FREE
 *   slot (FREE -> LOADING, the slot is written back); otherwise *slot_inout must be LOADING
 *   with the same layer and the part is appended. The parts must cover the bytes the layer
 *   needs before slide_slot_ring_acquire, which orders the compute stream after every part
 *   issued so far (they run in order on the h2d stream).
 * flush_range: after the work queued so far on compute_stream, copy gradient bytes
 *   [offset, offset + nbytes) of the slot to host_g + offset; the slot must be IN_USE (the first
 *   part: -> FLUSHING) or FLUSHING. Each part gets its own ticket; the slot's pending-flush
 *   event is the last part's.
 * Both: SLIDE_E_ARG if the bytes fall outside the slot's w_bytes / g_bytes or nbytes is 0,
 * SLIDE_E_STATE for a slot in the wrong state (nothing is copied then). */
int slide_slot_ring_load_range(slide_ring* r, int layer, const void* host_w, size_t offset,
                               size_t nbytes, int* slot_inout);
int slide_slot_ring_flush_range(slide_ring* r, int slot, void* host_g, size_t offset,
                                size_t nbytes, void* compute_stream, uint64_t* ticket);
/* Block until the flush named by ticket has landed in host memory; SLIDE_E_TIMEOUT after
 * timeout_ms milliseconds (a negative value waits without a limit). */
int slide_slot_ring_wait_flush(slide_ring* r, uint64_t ticket, int timeout_ms);
/* Return the slot to FREE once the work queued so far on compute_stream is done with it
 * (stream-ordered; from IN_USE or FLUSHING). */
int slide_slot_ring_release(slide_ring* r, int slot, void* compute_stream);
/* Re-claim a FREE slot whose weights still hold `layer` (nothing was loaded over them since its
 * release) without copying; FREE -> LOADING. SLIDE_E_STATE if no such slot. Used at the turn
 * from the forward to the backward sweep, where the last layers are still resident. The caller
 * must know that the host copy of those weights has not changed since they were loaded. */
int slide_slot_ring_reuse(slide_ring* r, int layer, int* slot_out);
int slide_slot_ring_state(slide_ring* r, int slot, int* state, int* layer);
/* Find the slot currently holding `layer` (LOADING / IN_USE / FLUSHING), or -1. */
int slide_slot_ring_find(slide_ring* r, int layer, int* slot_out);
/* Host time (CLOCK_MONOTONIC seconds) at which the flush named by ticket landed, for the
 * host-timed engines (HOST, HSA; SLIDE_E_UNSUPPORTED for HIP). SLIDE_E_STATE before it has
 * landed; SLIDE_E_ARG for an unknown ticket or one whose record was reused (the last 1024
 * flushes are kept). */
int slide_slot_ring_ticket_time(slide_ring* r, uint64_t ticket, double* t_done);
int slide_slot_ring_destroy(slide_ring* r);

/* Host-link diagnostic (summary, section 2A: layers and gradients cross the host link
 * asynchronously; the ring's copies run on whichever copy engine the runtime picks): the best of
 * `reps` times (ms) of one nbytes copy between `dev` (device memory) and `host` (pinned host
 * memory) on each copy engine of the GPU, device to host into d2h_ms[e] and host to device into
 * h2d_ms[e] for engine e < 32 (-1 where an engine is absent or refuses). info4 receives the
 * number of host-optimized engines, the number of engines optimized for copies between GPUs,
 * and the runtime's preferred engine masks for device to host and host to device. Overwrites
 * both buffers; synchronizes the device first and blocks until done. SLIDE_E_ARG for null or
 * unpinned buffers, SLIDE_E_TIMEOUT if a copy does not finish within its bound. */
int slide_host_link_engine_rates(void* dev, void* host, size_t nbytes, int reps, double* d2h_ms,
                                 double* h2d_ms, uint32_t* info4);
/* Host engine only: make the next `count` copies fail (fail_mode 1) or never complete
 * (fail_mode 2). Returns SLIDE_E_UNSUPPORTED for the HIP engine. */
int slide_slot_ring_inject_fault(slide_ring* r, int fail_mode, int count);

/* Non-finite check of a gradient before it leaves the GPU: *count_dev (device memory, 4 bytes,
 * overwritten) receives the number of NaN or infinite elements of x[n] (dtype SLIDE_BF16 or
 * SLIDE_F32; x 16-byte aligned). The pages leave failure handling open; an update computed from
 * such a gradient would corrupt the fp32 master weights, so the engine checks each layer's
 * gradient with this call and refuses the update (SLIDE_E_NONFINITE) instead of applying it. */
int slide_nonfinite_count(const void* x, int dtype, size_t n, uint32_t* count_dev, void* stream);

/* ------------------------------------------------------------------------------------------
 * CPU AdamW (the per-layer host optimizer, "Layer-Adam": summary, section 2B).
 * Decoupled weight decay, bias correction, step t >= 1, fixed float32 operation order:
 *   scalars (double, each cast once to float): b1t = beta1^t, b2t = beta2^t (t repeated
 *   multiplications), c_dec = 1 - lr*wd, c_1b1 = 1 - beta1, c_1b2 = 1 - beta2,
 *   c_step = lr / (1 - b1t), c_bc2 = sqrt(1 - b2t)
 *   per element (float32, round to nearest-even, no fused multiply-add):
 *   p1 = p*c_dec; m = beta1*m + c_1b1*g; v = beta2*v + c_1b2*(g*g);
 *   den = sqrt(v)/c_bc2 + eps; p = p1 - c_step*(m/den); p_bf16 = bf16_rne(p)
 * with g read as float (exact widening) and multiplied by c_gs = float(1/hp->grad_scale) when
 * hp->grad_scale is neither 0 nor 1.
 * p, m, v: float [n] host memory, updated in place. g: [n] of g_dtype (SLIDE_BF16, SLIDE_F16 or
 * SLIDE_F32). p_bf16_out: optional uint16 [n] 16-bit copy of p, rounded to nearest-even, in
 * g's type when g is 16-bit (bf16 for an fp32 g); it may alias g when g is 16-bit (the
 * gradient landing buffer and the 16-bit weight copy are one shared host buffer).
 * n_threads <= 0 uses the available cores. Blocks until done.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
  /* The loss scale the gradient was computed at (dynamic loss scaling of fp16 training): the
   * update uses g * c_gs with c_gs = float(1 / grad_scale), a power of two in practice, so the
   * product is exact. 0 or 1: unscaled (c_gs = 1, no change to any result). */
  double grad_scale;
} slide_adamw_hp;
int slide_cpu_adamw(float* p, const void* g, int g_dtype, float* m, float* v,
                    uint16_t* p_bf16_out, size_t n, int64_t step, const slide_adamw_hp* hp,
                    int n_threads);
/* slide_cpu_adamw on a list of rows: row r is elements [r*row_len, (r+1)*row_len) of p, m, v,
 * g and p_bf16_out (all indexed alike, n_rows_total rows in each). g = NULL means an exactly
 * zero gradient for every listed row (summary, section 2B, Layer-Adam; for an embedding, the
 * rows that no token of the batch selected: their update needs no gradient copy and can run
 * before the backward ends). rows: n_rows distinct indices in [0, n_rows_total), else
 * SLIDE_E_ARG. Same bits as slide_cpu_adamw over the whole arrays with those gradients. */
int slide_cpu_adamw_rows(float* p, const void* g, int g_dtype, float* m, float* v,
                         uint16_t* p_bf16_out, size_t row_len, size_t n_rows_total,
                         const int32_t* rows, size_t n_rows, int64_t step,
                         const slide_adamw_hp* hp, int n_threads);
/* slide_cpu_adamw on listed rows whose gradients arrive packed: row k of g_packed (n_rows rows
 * of row_len elements, g_dtype) is the gradient of row rows[k] of p, m, v (n_rows_total rows;
 * for an embedding, only the rows the batch selected leave the GPU). For a 16-bit g_dtype the
 * new row's 16-bit copy (the gradient's type) is written to row rows[k] of out_full and to row
 * k of out_packed (either may be NULL; out_packed may be g_packed itself, each row is consumed
 * before it is overwritten), so the packed rows can go back to the device as they are. For
 * SLIDE_F32 out_full must be NULL and out_packed receives the new fp32 rows. rows: distinct
 * indices in [0, n_rows_total), else SLIDE_E_ARG. Same bits as slide_cpu_adamw_rows. */
int slide_cpu_adamw_rows_packed(float* p, float* m, float* v, size_t row_len,
                                size_t n_rows_total, const int32_t* rows, size_t n_rows,
                                const void* g_packed, int g_dtype, void* out_full,
                                void* out_packed, int64_t step, const slide_adamw_hp* hp,
                                int n_threads);

/* The same AdamW step on the GPU, for training whose optimizer state stays in HBM (the
 * non-offloaded baseline of the paper page's abstract, which compares the layer-sliding method
 * with training that keeps everything on the GPU). p, m, v: device float [n]; g: device [n] of
 * g_dtype; p_bf16_out: optional device uint16 [n], which may alias g for a bf16 g. Same
 * operation order and rounding as slide_cpu_adamw, so the results are equal bit for bit.
 * Asynchronous on `stream`; argument errors as slide_cpu_adamw. */
int slide_gpu_adamw(float* p, const void* g, int g_dtype, float* m, float* v,
                    uint16_t* p_bf16_out, size_t n, int64_t step, const slide_adamw_hp* hp,
                    void* stream);

/* fp32 -> 16-bit conversion on the host, n_threads threads: dst [n] in dst_dtype (SLIDE_BF16 or
 * SLIDE_F16), rounded to nearest-even, NaN kept as a quiet NaN; the 16-bit compute copy of
 * fp32 master weights (summary, section 2B: FP32 -> BF16/FP16 conversion in the shared host
 * buffers). SLIDE_E_ARG for a null pointer or another dtype. Blocks until done. */
int slide_cpu_convert_f32(const float* src, void* dst, int dst_dtype, size_t n, int n_threads);
/* The same conversion on the GPU, for 16-bit copies of fp32 weights that already live in HBM
 * (the optimizer-resident baseline): src fp32 [n] and dst [n] in dst_dtype (SLIDE_BF16 or
 * SLIDE_F16) device memory, rounded to nearest-even (the bits of slide_cpu_convert_f32 for every
 * non-NaN input; NaN stays NaN). Asynchronous on `stream`; SLIDE_E_ARG for a null pointer with
 * n > 0 or another dtype. */
int slide_convert_f32(const float* src, void* dst, int dst_dtype, size_t n, void* stream);

/* The host-DRAM roofline of the CPU optimizer (summary, section 2B: the optimizer state lives
 * in host memory, so the update of a layer is bound by host memory bandwidth): a STREAM triad
 * a = b + s*c over three float arrays of n elements that the call maps (transparent huge pages)
 * and unmaps itself, on n_threads threads (<= 0: the available cores) with the same contiguous
 * per-thread ranges as slide_cpu_adamw, 64-byte loads and streaming stores (so no written line
 * is read first and the counted bytes are the bytes moved). 12 bytes per element per
 * repetition; *gbs_best (and *gbs_median, nullable) receive GB/s over `reps` repetitions.
 * SLIDE_E_ARG for n < 16, reps < 1 or a failed mapping. Blocks until done. */
int slide_host_triad(size_t n, int n_threads, int reps, double* gbs_best, double* gbs_median);

/* The scalar (non-vector) code path of slide_cpu_adamw on one thread; same contract. Exposed so
 * that tests can check both code paths give identical bits. */
int slide_cpu_adamw_scalar_for_test(float* p, const void* g, int g_dtype, float* m, float* v,
                                    uint16_t* p_bf16_out, size_t n, int64_t step,
                                    const slide_adamw_hp* hp);

/* ------------------------------------------------------------------------------------------
 * Disk tier of the optimizer state (the method's CPU optimizer keeps its state in host memory
 * and can move it to NVMe: summary, section 2B, "Layer-Adam"; for models larger than host memory
 * the optimizer state goes to NVMe first: summary, section 3, and the paper page's "Analysis of
 * NVMe Offloading").
 * A tier is one file of capacity_bytes holding fp32 arrays at offsets that are multiples of 4096.
 * The caller places the arrays; an array of n floats takes slide_tier_region_bytes(n) bytes (n*4
 * rounded up to 4096). Every transfer goes through the tier's page-aligned bounce buffers
 * (3 sets x 3 arrays x chunk_elems floats, owned by the tier) in 1 MiB requests served by
 * n_io_threads threads (<= 0: 8).
 * flags: SLIDE_TIER_DIRECT opens the file with O_DIRECT (the page cache is bypassed, so the
 *   bytes reach the device); where the file system refuses O_DIRECT the file is opened buffered
 *   and slide_tier_info reports direct = 0. SLIDE_TIER_UNLINK removes the file's name right
 *   after it is created, so its space is returned when the tier is destroyed or the process ends.
 * The file is created (or truncated) and sized to capacity_bytes; it reads as zeros until
 * written. Calls on one tier are serialized by the tier. File errors return SLIDE_E_IO;
 * offsets that are not page multiples or regions past the capacity return SLIDE_E_ARG.
 * ------------------------------------------------------------------------------------------ */
enum { SLIDE_TIER_DIRECT = 1, SLIDE_TIER_UNLINK = 2 };
typedef struct slide_tier slide_tier;
size_t slide_tier_region_bytes(size_t n_floats);
int slide_tier_create(slide_tier** out, const char* path, uint64_t capacity_bytes,
                      size_t chunk_elems /* 0: 4Mi; rounded up to a multiple of 1024 */,
                      int n_io_threads, int flags);
int slide_tier_destroy(slide_tier* t);
int slide_tier_info(slide_tier* t, int* direct, uint64_t* capacity_bytes, size_t* chunk_elems);
/* Totals since creation: bytes moved to and from the file, seconds spent inside tier calls and
 * seconds of those spent waiting for I/O. */
int slide_tier_stats(slide_tier* t, uint64_t* bytes_read, uint64_t* bytes_written,
                     double* busy_s, double* stall_s);
/* Blocking copies between host memory and the tier. src == NULL writes zeros. Whole pages are
 * written: the bytes from off + bytes up to the next multiple of 4096 become zero. */
int slide_tier_write(slide_tier* t, uint64_t off, const void* src, size_t bytes);
int slide_tier_read(slide_tier* t, uint64_t off, void* dst, size_t bytes);
/* slide_cpu_adamw on one parameter block whose p, m and v each live either in host memory (a
 * non-NULL pointer; the offset is ignored) or in the tier at the given offset (a NULL pointer).
 * The block is streamed in chunks of chunk_elems: while chunk k is updated, chunk k+1's tier
 * arrays are read and chunk k-1's written back. Every element gets exactly slide_cpu_adamw's
 * operations, so the results are bit-identical to that call with the arrays in memory. g and
 * p_bf16_out are host memory as for slide_cpu_adamw (p_bf16_out may alias a bf16 g). Blocks. */
int slide_tier_adamw(slide_tier* t, float* p, uint64_t p_off, float* m, uint64_t m_off, float* v,
                     uint64_t v_off, const void* g, int g_dtype, uint16_t* p_bf16_out, size_t n,
                     int64_t step, const slide_adamw_hp* hp, int n_threads);

/* ------------------------------------------------------------------------------------------
 * Kernel timing: when enabled, every kernel the library launches is bracketed by HIP events
 * on its own stream; slide_prof_read synchronizes them and returns, per kernel name, the
 * launch count and total milliseconds since the last reset.
 * ------------------------------------------------------------------------------------------ */
int slide_prof_enable(int on);
int slide_prof_reset(void);
/* Writes up to max_entries records; *n_out = number written. name buffers are 64 bytes. */
int slide_prof_read(char (*names)[64], int64_t* counts, double* total_ms, int max_entries,
                    int* n_out);

#ifdef __cplusplus
}
#endif
#endif /* SLIDE_H */
