/*
 * g2attn — Gemma 2 attention layer (prefill and decode) for AMD MI355X (gfx950).
 *
 * The operation (Gemma 2 model card on wikillm, "Method" section, one-layer
 * attention pseudocode; aifetchly "Gemma 2 Guide", section 1 soft-cap formula):
 *
 *   for batch b, query row t, query head h, with g = h / (H / KVH) and query
 *   position p = t + S - T:
 *     x_j   = query_scale * <q[b,t,h,:], k[b,j,g,:]>
 *     s_j   = softcap * tanh(x_j / softcap)        (identity if softcap <= 0)
 *     key j is visible iff j <= p and, on a local layer, j > p - window
 *     w     = softmax over visible keys of s
 *     out[b,t,h,:] = sum_j w_j * v[b,j,g,:]
 *
 *   The cap acts on the scaled logits before the mask (card, "Paper vs code").
 *   Every two query heads share one key/value head in all three model sizes
 *   (card, "Method" item 4 and "Pitfalls", GQA naming); the library accepts
 *   H / KVH of 1 or 2.  The 27B model's query_scale is 144^-0.5, not
 *   head_dim^-0.5 (card, "Pitfalls"): the caller passes query_scale, the
 *   library never derives it.  Local layers use window 4096, global layers see
 *   the whole causal prefix (card, "Method" item 1).
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers (hipMalloc'd or equivalent) on the current
 *     device, 16-byte aligned.  The caller owns all buffers; the library never
 *     allocates device memory and keeps no state between calls.
 *   - Tensors are dense row-major: q and out (B, T, H, d); k and v (B, S, KVH, d).
 *   - dtype: G2_BF16 (bf16 storage, fp32 accumulation; bf16 output rounded to
 *     nearest even) or G2_F32 (fp32 storage and arithmetic).  All tensors of
 *     one call share the dtype.
 *   - Calls only enqueue work on `stream` (0 = the null stream) and return; no
 *     host synchronisation.  `out` must not alias any input.
 *   - Return value: G2_OK or a negative g2_status; no call aborts or throws.
 *     Argument errors are detected on the host before anything is enqueued.
 *
 * Supported shapes: d in {64, 128, 256}; H / KVH in {1, 2}.
 */
#ifndef G2ATTN_H
#define G2ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { G2_BF16 = 0, G2_F32 = 1 } g2_dtype;

typedef enum {
  G2_OK = 0,
  G2_ERR_ARG = -1,         /* null pointer, non-positive size, H % KVH != 0,
                              T > S, window < 1 on a local layer, T != 1 for
                              decode, unknown dtype */
  G2_ERR_UNSUPPORTED = -2, /* d not in {64,128,256} or H/KVH not in {1,2} */
  G2_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  G2_ERR_WORKSPACE = -4,   /* decode workspace missing or too small */
  G2_ERR_LAUNCH = -5       /* the HIP runtime reported a launch error */
} g2_status;

/*
 * Prefill: causal (local: sliding-window) soft-capped GQA attention of T query
 * rows against S keys/values.
 *   q, out : (B, T, H, d)       k, v : (B, S, KVH, d)
 *   query row t sits at position t + S - T (the mask is aligned bottom-right,
 *   so T = S is ordinary prefill and T < S a chunk continuing a prefix).
 *   query_scale : multiplies the logits (1/sqrt(d) for 2B/9B, 1/12 for 27B).
 *   softcap     : cap of cap*tanh(x/cap); <= 0 or +inf disables the cap.
 *   window      : sliding-window length W of a local layer (key j visible to
 *                 position p iff p - W < j <= p); ignored when is_local == 0.
 *   is_local    : 1 for a sliding-window (local) layer, 0 for a global layer.
 * Work is proportional to the visible (query, key) pairs: tiles wholly outside
 * the causal / window band are skipped.
 * Range: for caps up to about 55 the bf16 kernel uses one constant softmax
 * offset, so an unnormalised weight can reach 2^50; the fp32 accumulators stay
 * finite while (visible keys of a row) * max|v| < 2^77.  Other caps keep a
 * running maximum (weights <= 2^8).
 * Performance: G2_BF16 is the performance path (MFMA, K/V tiles staged in LDS
 * and shared by the query heads of a group).  G2_F32 is a correctness path
 * for small inputs such as a 256-token fp32 layer: one wave per (row, head)
 * reads every visible K/V row from global memory with plain fp32 arithmetic,
 * no MFMA and no LDS staging, so its cost grows with T * (visible keys) * H
 * memory reads; do not use it for long sequences where speed matters.
 */
int g2attn_prefill(const void* q, const void* k, const void* v, void* out,
                   int B, int T, int S, int H, int KVH, int d,
                   float query_scale, float softcap, int window, int is_local,
                   int dtype, hipStream_t stream);

/*
 * Prefill that also returns each row's log-sum-exp, the statistic a backward
 * pass keeps from the forward (Gemma 2 Guide, "Deep Dive" item 1: the cap is
 * differentiated in training).  Arguments as for g2attn_prefill, plus
 *   lse : device float32 (B, H, T), 4-byte aligned; lse[b][h][t] is the
 *         natural-log log-sum-exp over the visible keys of the capped logits
 *         s_j of row (b, t, h), so the softmax weights are exp(s_j - lse).
 */
int g2attn_prefill_lse(const void* q, const void* k, const void* v, void* out,
                       float* lse, int B, int T, int S, int H, int KVH, int d,
                       float query_scale, float softcap, int window,
                       int is_local, int dtype, hipStream_t stream);

/*
 * Backward pass of the prefill (Gemma 2 Guide, "Deep Dive" item 1: the cap's
 * derivative is 1 - tanh^2(x / cap)).  For an upstream gradient dout of the
 * output it writes
 *   dq (B,T,H,d), dk and dv (B,S,KVH,d): the gradients of the loss with
 *   respect to q, k and v, summed over the query heads sharing a K/V head and
 *   over every row that sees a key.
 * q, k, v and the scalars are those of the forward call; out and lse are its
 * results (g2attn_prefill_lse).  bf16 only (fp32: G2_ERR_UNSUPPORTED).
 * workspace: device scratch of g2attn_prefill_backward_workspace_bytes(B,T,S,H)
 * bytes, 16-byte aligned: one float per row and, for each (batch, head,
 * 32-row tile, 16-key block), 1 KiB of bf16 dS = p (<dO, v> - D) (1 - tanh^2)
 * that the dK/dV kernel stores and the dQ kernel reads, about 2 B T S H bytes
 * in all (4.3 GB for B = 2, T = S = 8192, H = 16).  Buffers may not alias
 * each other.  G2_ERR_WORKSPACE if the workspace is missing or too small.
 * To bound the workspace on long contexts, call it per chunk of query rows:
 * rows [t0, t1) passed as q, out, dout and lse sliced to those rows against
 * the first t1 keys (S = t1) sit at their own positions, and give those
 * rows' dq and their rows' share of dk and dv (for keys below t1); the shares
 * summed over the chunks are the layer's dk and dv.
 */
int g2attn_prefill_backward(const void* q, const void* k, const void* v,
                            const void* out, const void* dout, const float* lse,
                            void* dq, void* dk, void* dv, int B, int T, int S,
                            int H, int KVH, int d, float query_scale,
                            float softcap, int window, int is_local, int dtype,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Bytes of backward workspace for these sizes (0 for invalid sizes). */
size_t g2attn_prefill_backward_workspace_bytes(int B, int T, int S, int H);

/*
 * Decode: one new query token per sequence against a KV cache of capacity S
 * (model card, "Method"; Guide section 2 on local layers keeping only the last
 * 4096 tokens).
 *   q, out          : (B, 1, H, d)
 *   k_cache, v_cache: (B, S, KVH, d); token position j of sequence b lives in
 *                     slot j mod S, so a local layer's cache of S = window
 *                     slots is a ring and a global layer's cache is linear.
 *   kv_lens         : device int32[B]; kv_lens[b] = L_b >= 1 tokens, the
 *                     newest (already written) at position L_b - 1, which is
 *                     also the query's position.  Visible positions are those
 *                     the prefill mask allows; they must fit the cache:
 *                     L_b <= S for a global layer, min(L_b, window) <= S for a
 *                     local one.  A sequence whose L_b breaks this rule gets
 *                     NaN outputs; nothing outside the cache is read.
 *   T               : must be 1.
 *   workspace       : device scratch of at least
 *                     g2attn_decode_workspace_bytes(B, H, d, S) bytes, used for
 *                     split-K partial results; owned by the caller, may be
 *                     reused between calls on the same stream.
 */
int g2attn_decode(const void* q, const void* k_cache, const void* v_cache,
                  void* out, const int32_t* kv_lens,
                  int B, int T, int S, int H, int KVH, int d,
                  float query_scale, float softcap, int window, int is_local,
                  int dtype, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* Bytes of decode workspace needed for these sizes (0 for invalid sizes). */
size_t g2attn_decode_workspace_bytes(int B, int H, int d, int S);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, behaviour and results as g2attn_decode, but
 * without the workspace: the split-K scratch is a device array of
 * G2ATTN_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 * until the process ends.  The call allocates nothing.
 *   Limit: g2attn_decode_workspace_bytes(B, H, d, S) must not exceed
 *   G2ATTN_NOALLOC_SCRATCH_BYTES (32 MiB: the 9B-shaped decode at S = 8192
 *   fits up to B = 127), else G2_ERR_WORKSPACE is returned before any launch.
 *   All calls on one GPU share its scratch array: calls that overlap in time
 *   on one GPU (different streams, or different host threads) race and must
 *   be serialised by the caller.  The first call on a device looks up the
 *   array's device address (a host-side query, no allocation).
 */
#define G2ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int g2attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                          void* out, const int32_t* kv_lens,
                          int B, int T, int S, int H, int KVH, int d,
                          float query_scale, float softcap, int window, int is_local,
                          int dtype, hipStream_t stream);

/*
 * Decode against a paged KV cache (Gemma 2 Guide, "Deep Dive" item 2: serving
 * runtimes keep KV memory in fixed-size blocks, and local layers drop the
 * blocks older than the window).
 *   q, out          : (B, 1, H, d)
 *   k_pool, v_pool  : (num_blocks, block_size, KVH, d), the caller's block pool.
 *   block_table     : device int32[B * max_blocks]; entry [b][i] is the pool
 *                     block holding positions i*block_size .. (i+1)*block_size-1
 *                     of sequence b.  Only entries of blocks that hold a
 *                     position the query sees are read, so entries of unused
 *                     or dropped blocks may hold anything (e.g. -1).
 *   kv_lens         : device int32[B]; L_b tokens, the newest (already
 *                     written) at position L_b - 1, the query's position;
 *                     1 <= L_b <= max_blocks * block_size.  The visible
 *                     positions are those the prefill mask allows.
 *   block_size      : a power of two, 1 .. 65536.
 *   workspace       : device scratch of at least
 *                     g2attn_decode_paged_workspace_bytes(B, H, d, max_blocks,
 *                     block_size) bytes; owned by the caller.
 * A sequence whose L_b is out of range, or whose visible positions need a
 * table entry outside [0, num_blocks), gets NaN outputs; nothing outside the
 * pool is read.  Other errors as for g2attn_decode.
 */
int g2attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                        void* out, const int32_t* block_table, int max_blocks,
                        const int32_t* kv_lens, int B, int H, int KVH, int d,
                        int block_size, int num_blocks, float query_scale,
                        float softcap, int window, int is_local, int dtype,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Bytes of paged-decode workspace for these sizes (0 for invalid sizes). */
size_t g2attn_decode_paged_workspace_bytes(int B, int H, int d, int max_blocks,
                                           int block_size);

/*
 * Host-only validation of the scalar arguments of g2attn_decode_paged,
 * returning the status the call would return for non-null, aligned pointers.
 */
int g2attn_check_paged_args(int B, int H, int KVH, int d, int block_size,
                            int max_blocks, int num_blocks, int window,
                            int is_local, int dtype);

/*
 * Rotary position embedding of Q or K, in place (wikillm model card, "Method"
 * item 5: Gemma 2 keeps Gemma 1's rotary embeddings; the pages give no
 * formula, so the pair layout and base are this library's reading).
 *   x         : (B, T, NH, d) device tensor of dtype; NH is H for queries and
 *               KVH for keys.  Pair i < d/2 of every head vector is
 *               (x[i], x[i + d/2]), rotated by the angle pos * base^(-2i/d):
 *               (a, b) -> (a cos - b sin, b cos + a sin).
 *   positions : device int32 (B, T), the absolute position of each token
 *               (for a chunk of T tokens ending a cache of S: t + S - T).
 *   base      : > 1 (10000 for the rotary embeddings of the Gemma family).
 *   d         : 64, 128 or 256 (G2_ERR_UNSUPPORTED otherwise).
 * x must be 16-byte aligned, positions 4-byte aligned.
 */
int g2attn_rope(void* x, const int32_t* positions, int B, int T, int NH, int d,
                float base, int dtype, hipStream_t stream);

/*
 * Final-logit soft-cap in place: x[i] = cap * tanh(x[i] / cap) for the n
 * elements of x (Gemma 2 Guide, section 1, second formula: the vocabulary
 * logits are capped at 30).  cap <= 0 or +inf leaves x unchanged; n = 0 is a
 * no-op.  x must be 16-byte aligned.
 */
int g2attn_softcap(void* x, size_t n, float cap, int dtype, hipStream_t stream);

/*
 * Host-only validation of the scalar arguments of either entry point
 * (decode = 1 for decode), returning the status the call would return for
 * non-null, aligned pointers.  Touches no GPU.
 */
int g2attn_check_args(int B, int T, int S, int H, int KVH, int d, int window,
                      int is_local, int dtype, int decode);

/* Static, human-readable name of a status code. */
const char* g2attn_status_string(int status);

/*
 * Static string: the sha256 (64 hex digits) of the sources this library was
 * built from (its kernel sources, this header and the compiler flags), or
 * "unknown" for a build that did not set it.  Lets a caller check that the
 * binary it loaded matches the sources it measures or tests.
 */
const char* g2attn_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* G2ATTN_H */
