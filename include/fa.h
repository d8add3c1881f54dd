/*
 * fa.h -- C ABI of an exact-attention (FlashAttention-2) library for AMD
 * MI355X (gfx950, CDNA4).
 *
 * The library computes exact scaled-dot-product attention and its gradient
 * without ever forming the N x N score matrix, as the pages define it:
 *   - "FlashAttention-2 from PyTorch to Triton": the forward pass (the
 *     online-softmax recurrence, one program per query tile, the per-row
 *     log-sum-exp L = m + log l saved for the backward, the kernel signature
 *     with per-tensor strides, N_QUERIES, N_KEYS and scale), its test file's
 *     causal convention (a lower-triangular ``tril`` mask: key j is visible
 *     to query i iff j <= i) and its backward outline (L, D = rowsum(dO o O)
 *     and a loop over query tiles per key tile);
 *   - "Triton FlashAttention" (architjain.me): the backward split into a
 *     rowsum(dO.O) kernel, a dK/dV kernel and a dQ kernel with no atomics,
 *     probabilities rebuilt from the saved log-sum-exp, fp16 and fp32 inputs,
 *     head dims 16-128, non-contiguous inputs and 64-bit offsets.
 *
 * Tensor convention.  Every tensor argument is a logical [B, H, S, D] array
 * given by a base pointer and four int64 ELEMENT strides in that order
 * ({stride_b, stride_h, stride_s, stride_d}); any non-negative strides are
 * accepted, so [B, S, H, D] storage is passed as a strided view.  q, k, v,
 * o, dO, dq, dk, dv all have the element type `dtype`.  lse and the delta
 * workspace are float32, contiguous [B, H, Sq].  Offsets are computed in
 * 64-bit arithmetic.  All device pointers must be device memory of the GPU
 * that is current when the call is made.
 *
 * Causal masking (argument `causal`): 0 = none; 1 = top-left aligned, query
 * row i sees keys 0..i (clipped to Sk), the pages' ``tril`` convention, so
 * with Sk >= 1 every row sees key 0; 2 = bottom-right aligned, query row i
 * sees keys 0..i + (Sk - Sq), the same as 1 when Sq == Sk.  Under 2 with
 * Sq > Sk the first Sq - Sk rows see no key: their output row is 0, their
 * lse is -inf and they contribute no gradient (the pages leave such rows
 * open; this is the reading taken).  Other values are FA_ERR_CAUSAL.
 *
 * Ownership.  The caller owns every buffer.  The library allocates no device
 * memory and keeps no state other than read-only tables.  Outputs are fully
 * overwritten; outputs must not alias inputs or each other (identical base
 * pointers are rejected with FA_ERR_ALIAS; partial overlap is undefined).
 *
 * Execution.  Calls enqueue kernels on `stream` (a hipStream_t; NULL is the
 * default stream) and return without synchronising.  Argument validation
 * happens before any HIP call, so a rejected call touches no device state.
 * Device faults surface at the next synchronisation, as usual in HIP.  Calls
 * are reentrant; results are bitwise deterministic (no atomics).
 *
 * Return values: FA_OK (0) or a negative fa_status.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_F16 = 0, /* IEEE binary16 storage, fp16 MFMA with fp32 accumulation */
  FA_F32 = 1, /* IEEE binary32 storage, full-precision fp32 MFMA (no reduced-precision xf32) */
  FA_BF16 = 2 /* bfloat16 storage, bf16 MFMA with fp32 accumulation; P and dS are rounded to
                 bfloat16 (nearest even) before their products, as P is for fp16 */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,   /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,  /* B, H, Sq or Sk negative, Sk == 0 with B*H*Sq > 0, D not in {16,32,64,128},
                         or a size beyond 2^31-1 rows */
  FA_ERR_DTYPE = -3,  /* dtype is not a fa_dtype value */
  FA_ERR_STRIDE = -4, /* a negative stride */
  FA_ERR_ALIAS = -5,  /* an output base pointer equals an input's or another output's */
  FA_ERR_HIP = -6,    /* the HIP runtime reported an error at launch */
  FA_ERR_TILE = -7,   /* a forced tile id is out of range for this pass, dtype and D */
  FA_ERR_CAUSAL = -8, /* causal is not 0, 1 or 2 */
  FA_ERR_SCALE = -9,  /* scale is not a finite number > 0 (the kernels take the softmax over
                         scale * q.k in base 2 with the running max raised, never lowered, which
                         needs a positive scale; masked scores are -inf, so scale = 0 would give
                         0 * inf) */
  FA_ERR_WORKSPACE = -10 /* fa_bwd_noalloc: B*H*Sq is larger than its fixed scratch (2^22 rows) */
} fa_status;

/* Pass ids for the tile-table queries. */
typedef enum { FA_PASS_FWD = 0, FA_PASS_BWD_DKDV = 1, FA_PASS_BWD_DQ = 2 } fa_pass;

/*
 * fa_fwd -- forward attention ("FlashAttention-2 from PyTorch to Triton",
 * the forward kernel and its online-softmax recurrence; "Triton
 * FlashAttention", the forward kernel description).
 *
 *   O[b,h,i,:] = sum_j softmax_j(scale * q_i . k_j) v_j   (j <= i + c when causal:
 *                                                          c = 0, or Sk - Sq when causal = 2)
 *   lse[b,h,i] = log sum_j exp(scale * q_i . k_j)         (natural log, fp32)
 *
 * q: [B,H,Sq,D], k and v: [B,H,Sk,D], out: [B,H,Sq,D] (dtype), lse: [B,H,Sq]
 * contiguous float32.  `scale` is applied to the fp32 scores (typically
 * 1/sqrt(D)); it must be finite and > 0 (else FA_ERR_SCALE).  B*H*Sq == 0 is a
 * successful no-op.
 */
int fa_fwd(const void* q, const int64_t q_strides[4],
           const void* k, const int64_t k_strides[4],
           const void* v, const int64_t v_strides[4],
           int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
           int causal, float scale, int dtype,
           void* out, const int64_t out_strides[4], float* lse,
           void* stream);

/*
 * fa_bwd -- gradient of <dO, O> with respect to q, k, v ("Triton
 * FlashAttention": the rowsum(dO.O) kernel, then the dK/dV kernel over
 * query blocks per key block and the dQ kernel over key blocks per query
 * block, both rebuilding P = exp(S - L) from the saved log-sum-exp, no
 * atomics; "FlashAttention-2 from PyTorch to Triton", the backward outline).
 *
 *   delta_i = sum_d dO_id O_id           (written to delta_ws)
 *   dS_ij = P_ij (dO_i . v_j - delta_i)
 *   dq = scale * dS k,  dk = scale * dS^T q,  dv = P^T dO
 *
 * q, k, v, o (= fa_fwd's out), dO and lse (= fa_fwd's lse for the same
 * inputs) are read; delta_ws is a caller-owned float32 [B,H,Sq] workspace
 * that is overwritten (it holds delta afterwards); dq [B,H,Sq,D], dk and dv
 * [B,H,Sk,D] are overwritten.  `scale` must be the forward's (finite, > 0,
 * else FA_ERR_SCALE).  The kernels run in order on `stream`: the
 * rowsum, the dQ kernel, the dK/dV kernel; where the dQ kernel can form delta
 * from the query rows it holds (16-bit, D = 128 or 64, 16-byte-aligned rows)
 * there is no separate rowsum launch and the dQ kernel writes delta_ws.
 */
int fa_bwd(const void* q, const int64_t q_strides[4],
           const void* k, const int64_t k_strides[4],
           const void* v, const int64_t v_strides[4],
           const void* o, const int64_t o_strides[4],
           const void* dout, const int64_t dout_strides[4],
           const float* lse,
           int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
           int causal, float scale, int dtype,
           float* delta_ws,
           void* dq, const int64_t dq_strides[4],
           void* dk, const int64_t dk_strides[4],
           void* dv, const int64_t dv_strides[4],
           void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and kernels as fa_bwd, without the
 * delta_ws argument: delta = rowsum(dO o O) goes to a fixed scratch array
 * of 2^22 floats (16 MiB) that the library holds in its own device globals,
 * one per GPU, for the life of the process.  The call allocates nothing and
 * frees nothing.  B*H*Sq above 2^22 is FA_ERR_WORKSPACE (checked before any
 * HIP call, like every other argument).  The first call on a device looks up
 * that device's scratch address once.  Nothing in the scratch needs to
 * start at zero (delta is written before it is read, on `stream`), but the
 * array is shared by every call on that GPU: calls that overlap on one GPU
 * (different streams, or host threads) race on it and must be serialised by
 * the caller.
 */
int fa_bwd_noalloc(const void* q, const int64_t q_strides[4],
                   const void* k, const int64_t k_strides[4],
                   const void* v, const int64_t v_strides[4],
                   const void* o, const int64_t o_strides[4],
                   const void* dout, const int64_t dout_strides[4],
                   const float* lse,
                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                   int causal, float scale, int dtype,
                   void* dq, const int64_t dq_strides[4],
                   void* dk, const int64_t dk_strides[4],
                   void* dv, const int64_t dv_strides[4],
                   void* stream);

/*
 * Tile table ("Triton FlashAttention": block sizes tuned per power-of-two
 * length bucket with configurations that do not fit on-chip memory pruned,
 * and every configuration tested directly, including unequal query and key
 * block sizes).
 *
 * fa_tile_count returns how many tile configurations exist for a pass,
 * dtype and head dim (0 for unsupported arguments).  fa_tile_info writes
 * {block_m, block_n, waves, lds_bytes} of configuration `tile_id` into
 * info[4] and returns FA_OK or FA_ERR_TILE.  fa_tile_default returns the
 * id that fa_fwd / fa_bwd choose for the given problem (or a negative
 * fa_status: FA_ERR_DTYPE, FA_ERR_SHAPE for an unsupported D or a negative
 * length, FA_ERR_CAUSAL, FA_ERR_TILE for an unknown pass): the configuration
 * measured fastest on MI355X for the pass, dtype, head dim, causal flag
 * (bottom-right counts as causal) and the power-of-two bucket of
 * max(Sq, Sk), clamped to 128..16384 (a compiled-in table written by the
 * offline sweep exact_attention_88_amd/tile_sweep.py).
 */
int fa_tile_count(int pass, int dtype, int64_t D);
int fa_tile_info(int pass, int dtype, int64_t D, int tile_id, int64_t info[4]);
int fa_tile_default(int pass, int dtype, int64_t D, int64_t Sq, int64_t Sk, int causal);

/*
 * fa_fwd_tile / fa_bwd_tile -- fa_fwd / fa_bwd with the tile configuration
 * forced instead of looked up (tile ids from fa_tile_count; -1 keeps the
 * default).  For testing every table entry and for sweeps.
 */
int fa_fwd_tile(int tile_id,
                const void* q, const int64_t q_strides[4],
                const void* k, const int64_t k_strides[4],
                const void* v, const int64_t v_strides[4],
                int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                int causal, float scale, int dtype,
                void* out, const int64_t out_strides[4], float* lse,
                void* stream);
int fa_bwd_tile(int dkdv_tile_id, int dq_tile_id,
                const void* q, const int64_t q_strides[4],
                const void* k, const int64_t k_strides[4],
                const void* v, const int64_t v_strides[4],
                const void* o, const int64_t o_strides[4],
                const void* dout, const int64_t dout_strides[4],
                const float* lse,
                int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                int causal, float scale, int dtype,
                float* delta_ws,
                void* dq, const int64_t dq_strides[4],
                void* dk, const int64_t dk_strides[4],
                void* dv, const int64_t dv_strides[4],
                void* stream);

/*
 * fa_bwd_stage -- one of the backward kernels alone, with the same
 * arguments as fa_bwd_tile: stage 0 = the rowsum(dO.O) preprocess (writes
 * delta_ws; `tile_id` is the dQ tile stage 2 will run, -1 for the default),
 * 2 = the dQ kernel (writes dq), 1 = the dK/dV
 * kernel (reads delta_ws, writes dk, dv; q/o/dout/lse/dq may be NULL when
 * Sq == 0).  Where the chosen dQ kernel can form delta from the rows it
 * holds (16-bit, D = 128 or 64, 16-byte-aligned rows: the default there), stage 0
 * launches nothing and stage 2 writes delta_ws itself; otherwise stage 2
 * reads it.  Running stages 0, 2, 1 in that order on one stream is exactly
 * fa_bwd_tile.  For per-kernel timing and profiling.
 */
int fa_bwd_stage(int stage, int tile_id,
                 const void* q, const int64_t q_strides[4],
                 const void* k, const int64_t k_strides[4],
                 const void* v, const int64_t v_strides[4],
                 const void* o, const int64_t o_strides[4],
                 const void* dout, const int64_t dout_strides[4],
                 const float* lse,
                 int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                 int causal, float scale, int dtype,
                 float* delta_ws,
                 void* dq, const int64_t dq_strides[4],
                 void* dk, const int64_t dk_strides[4],
                 void* dv, const int64_t dv_strides[4],
                 void* stream);

/* Human-readable name of a fa_status code (static storage). */
const char* fa_status_string(int status);

/* Text of the HIP runtime error behind the calling thread's most recent
 * FA_ERR_HIP (hipGetErrorName: hipGetErrorString), or "" if none occurred. */
const char* fa_last_hip_error(void);

/* Library version string: name, version and target, then the HIP version and
 * the compiler that built it, e.g. "fa-mi355x 0.2 gfx950; HIP 7.2.x; AMD
 * clang version ...". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
