// C-ABI entry points of libg2attn (declared in include/g2attn.h).
//
// Host side only: argument validation (the same checks g2attn_check_args
// exposes to CPU-only callers), dispatch on (dtype, head dim, heads per K/V
// head) and launch on the caller's stream.  No allocation, no global state.
#include <stdint.h>

#include "g2_kernels.h"
#include "g2attn.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_scalars(int B, int T, int S, int H, int KVH, int d, int window, int is_local,
                  int dtype, int decode) {
  if (B <= 0 || T <= 0 || S <= 0 || H <= 0 || KVH <= 0 || d <= 0) return G2_ERR_ARG;
  if (dtype != G2_BF16 && dtype != G2_F32) return G2_ERR_ARG;
  if (H % KVH != 0) return G2_ERR_ARG;
  if (T > S) return G2_ERR_ARG;
  if (is_local != 0 && is_local != 1) return G2_ERR_ARG;
  if (is_local && window < 1) return G2_ERR_ARG;
  if (decode && T != 1) return G2_ERR_ARG;
  if (d != 64 && d != 128 && d != 256) return G2_ERR_UNSUPPORTED;
  const int G = H / KVH;
  if (G != 1 && G != 2) return G2_ERR_UNSUPPORTED;
  // Index arithmetic inside the kernels is 32-bit per (batch, head) slice.
  if ((long long)S * KVH * d >= (1LL << 31) || (long long)T * H * d >= (1LL << 31)) return G2_ERR_UNSUPPORTED;
  return G2_OK;
}

int check_paged_scalars(int B, int H, int KVH, int d, int block_size, int max_blocks,
                        int num_blocks, int window, int is_local, int dtype) {
  if (B <= 0 || H <= 0 || KVH <= 0 || d <= 0) return G2_ERR_ARG;
  if (block_size <= 0 || max_blocks <= 0 || num_blocks <= 0) return G2_ERR_ARG;
  if ((block_size & (block_size - 1)) != 0 || block_size > 65536) return G2_ERR_ARG;
  if ((long long)max_blocks * block_size >= (1LL << 31)) return G2_ERR_ARG;
  if (dtype != G2_BF16 && dtype != G2_F32) return G2_ERR_ARG;
  if (H % KVH != 0) return G2_ERR_ARG;
  if (is_local != 0 && is_local != 1) return G2_ERR_ARG;
  if (is_local && window < 1) return G2_ERR_ARG;
  if (d != 64 && d != 128 && d != 256) return G2_ERR_UNSUPPORTED;
  const int G = H / KVH;
  if (G != 1 && G != 2) return G2_ERR_UNSUPPORTED;
  return G2_OK;
}

size_t paged_workspace_bytes(int B, int H, int d, int max_blocks, int block_size) {
  const long long cap = (long long)max_blocks * block_size;
  const size_t splits = (size_t)((cap + g2::kDecodeChunk - 1) / g2::kDecodeChunk);
  return (size_t)B * H * splits * (2 + (size_t)d) * sizeof(float);
}

}  // namespace

// The sha256 of the sources this library was built from, set by the build
// script; the tag lets a reader find it in the binary without loading it.
#ifndef G2ATTN_BUILD_ID
#define G2ATTN_BUILD_ID "unknown"
#endif
static const char kBuildIdRecord[] = "g2attn-build-id:" G2ATTN_BUILD_ID;

extern "C" {

const char* g2attn_build_id(void) { return kBuildIdRecord + sizeof("g2attn-build-id:") - 1; }

int g2attn_check_args(int B, int T, int S, int H, int KVH, int d, int window, int is_local,
                      int dtype, int decode) {
  return check_scalars(B, T, S, H, KVH, d, window, is_local, dtype, decode);
}

const char* g2attn_status_string(int status) {
  switch (status) {
    case G2_OK: return "ok";
    case G2_ERR_ARG: return "invalid argument";
    case G2_ERR_UNSUPPORTED: return "unsupported shape (d must be 64, 128 or 256; H/KVH 1 or 2)";
    case G2_ERR_ALIGN: return "pointer not 16-byte aligned";
    case G2_ERR_WORKSPACE: return "decode workspace missing or too small";
    case G2_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t g2attn_decode_workspace_bytes(int B, int H, int d, int S) {
  if (B <= 0 || H <= 0 || d <= 0 || S <= 0) return 0;
  return g2::decode_workspace_bytes(B, H, d, S);
}

int g2attn_prefill(const void* q, const void* k, const void* v, void* out, int B, int T, int S,
                   int H, int KVH, int d, float query_scale, float softcap, int window,
                   int is_local, int dtype, hipStream_t stream) {
  int st = check_scalars(B, T, S, H, KVH, d, window, is_local, dtype, 0);
  if (st != G2_OK) return st;
  if (!q || !k || !v || !out) return G2_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return G2_ERR_ALIGN;
  g2::PrefillLaunch L{q, k, v, out, B, T, S, H, KVH, d, query_scale, softcap, window, is_local};
  const hipError_t e = dtype == G2_BF16 ? g2::launch_prefill_bf16(L, stream)
                                        : g2::launch_prefill_f32(L, stream);
  return e == hipSuccess ? G2_OK : G2_ERR_LAUNCH;
}

int g2attn_prefill_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int T, int S, int H, int KVH, int d, float query_scale,
                       float softcap, int window, int is_local, int dtype, hipStream_t stream) {
  int st = check_scalars(B, T, S, H, KVH, d, window, is_local, dtype, 0);
  if (st != G2_OK) return st;
  if (!q || !k || !v || !out || !lse) return G2_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return G2_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return G2_ERR_ALIGN;
  g2::PrefillLaunch L{q, k, v, out, B, T, S, H, KVH, d, query_scale, softcap, window, is_local};
  L.lse = lse;
  const hipError_t e = dtype == G2_BF16 ? g2::launch_prefill_bf16(L, stream)
                                        : g2::launch_prefill_f32(L, stream);
  return e == hipSuccess ? G2_OK : G2_ERR_LAUNCH;
}

int g2attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                  const int32_t* kv_lens, int B, int T, int S, int H, int KVH, int d,
                  float query_scale, float softcap, int window, int is_local, int dtype,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_scalars(B, T, S, H, KVH, d, window, is_local, dtype, 1);
  if (st != G2_OK) return st;
  if (!q || !k_cache || !v_cache || !out || !kv_lens) return G2_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return G2_ERR_ALIGN;
  if (!workspace || workspace_bytes < g2::decode_workspace_bytes(B, H, d, S)) return G2_ERR_WORKSPACE;
  if (!aligned16(workspace)) return G2_ERR_ALIGN;
  g2::DecodeLaunch L{q, k_cache, v_cache, out, kv_lens, B, S, H, KVH, d,
                     query_scale, softcap, window, is_local, workspace};
  const hipError_t e = g2::launch_decode(L, dtype, stream);
  return e == hipSuccess ? G2_OK : G2_ERR_LAUNCH;
}

int g2attn_check_paged_args(int B, int H, int KVH, int d, int block_size, int max_blocks,
                            int num_blocks, int window, int is_local, int dtype) {
  return check_paged_scalars(B, H, KVH, d, block_size, max_blocks, num_blocks, window, is_local,
                             dtype);
}

size_t g2attn_decode_paged_workspace_bytes(int B, int H, int d, int max_blocks, int block_size) {
  if (B <= 0 || H <= 0 || d <= 0 || max_blocks <= 0 || block_size <= 0) return 0;
  if ((long long)max_blocks * block_size >= (1LL << 31)) return 0;
  return paged_workspace_bytes(B, H, d, max_blocks, block_size);
}

int g2attn_decode_paged(const void* q, const void* k_pool, const void* v_pool, void* out,
                        const int32_t* block_table, int max_blocks, const int32_t* kv_lens,
                        int B, int H, int KVH, int d, int block_size, int num_blocks,
                        float query_scale, float softcap, int window, int is_local, int dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_paged_scalars(B, H, KVH, d, block_size, max_blocks, num_blocks, window,
                               is_local, dtype);
  if (st != G2_OK) return st;
  if (!q || !k_pool || !v_pool || !out || !block_table || !kv_lens) return G2_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return G2_ERR_ALIGN;
  g2::DecodeLaunch L{q, k_pool, v_pool, out, kv_lens, B, 1, H, KVH, d,
                     query_scale, softcap, window, is_local, workspace};
  L.block_table = block_table;
  L.max_blocks = max_blocks;
  L.block_size = block_size;
  L.num_blocks = num_blocks;
  const size_t need = (size_t)B * H * g2::decode_call_splits(L) * (2 + (size_t)d) * sizeof(float);
  if (!workspace || workspace_bytes < need) return G2_ERR_WORKSPACE;
  if (!aligned16(workspace)) return G2_ERR_ALIGN;
  const hipError_t e = g2::launch_decode(L, dtype, stream);
  return e == hipSuccess ? G2_OK : G2_ERR_LAUNCH;
}

int g2attn_rope(void* x, const int32_t* positions, int B, int T, int NH, int d, float base,
                int dtype, hipStream_t stream) {
  if (B <= 0 || T <= 0 || NH <= 0) return G2_ERR_ARG;
  if (!(base > 1.0f) || __builtin_isinf(base)) return G2_ERR_ARG;
  if (dtype != G2_BF16 && dtype != G2_F32) return G2_ERR_ARG;
  if (d != 64 && d != 128 && d != 256) return G2_ERR_UNSUPPORTED;
  if (!x || !positions) return G2_ERR_ARG;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(positions) & 3u) != 0) return G2_ERR_ALIGN;
  g2::RopeLaunch L{x, positions, B, T, NH, d, base, dtype};
  return g2::launch_rope(L, stream) == hipSuccess ? G2_OK : G2_ERR_LAUNCH;
}

int g2attn_softcap(void* x, size_t n, float cap, int dtype, hipStream_t stream) {
  if (dtype != G2_BF16 && dtype != G2_F32) return G2_ERR_ARG;
  if (n == 0 || !(cap > 0.0f) || __builtin_isinf(cap)) return G2_OK;  // nothing to do
  if (!x) return G2_ERR_ARG;
  if (!aligned16(x)) return G2_ERR_ALIGN;
  return g2::launch_softcap(x, n, cap, dtype, stream) == hipSuccess ? G2_OK : G2_ERR_LAUNCH;
}

size_t g2attn_prefill_backward_workspace_bytes(int B, int T, int S, int H) {
  if (B <= 0 || T <= 0 || S < T || H <= 0) return 0;
  return g2::backward_workspace_bytes(B, T, S, H);
}

int g2attn_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            int B, int T, int S, int H, int KVH, int d, float query_scale,
                            float softcap, int window, int is_local, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  int st = check_scalars(B, T, S, H, KVH, d, window, is_local, dtype, 0);
  if (st != G2_OK) return st;
  if (dtype != G2_BF16) return G2_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return G2_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return G2_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return G2_ERR_ALIGN;
  if (!workspace || workspace_bytes < g2::backward_workspace_bytes(B, T, S, H)) return G2_ERR_WORKSPACE;
  if (!aligned16(workspace)) return G2_ERR_ALIGN;
  g2::BackwardLaunch L{q, k, v, out, dout, lse, dq, dk, dv, B, T, S, H, KVH, d,
                       query_scale, softcap, window, is_local, workspace};
  return g2::launch_prefill_backward(L, stream) == hipSuccess ? G2_OK : G2_ERR_LAUNCH;
}

}  // extern "C"
