// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace g2 {

struct PrefillLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int B, T, S, H, KVH, d;
  float query_scale, softcap;
  int window, is_local;
  float* lse = nullptr;  // optional (B, H, T) natural-log log-sum-exp of each row
};

struct DecodeLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* kv_lens;
  int B, S, H, KVH, d;
  float query_scale, softcap;
  int window, is_local;
  void* workspace;
  // Paged mode when block_table is non-null: k/v are (num_blocks,
  // block_size, KVH, d) pools and S is unused.
  const int32_t* block_table = nullptr;
  int max_blocks = 0, block_size = 0, num_blocks = 0;
};

// Keys handled by one split-K workgroup of the decode kernel.
constexpr int kDecodeChunk = 512;

inline int decode_splits(int S) { return (S + kDecodeChunk - 1) / kDecodeChunk; }

// Workspace layout: float m[B*H*splits], l[B*H*splits], acc[B*H*splits*d].
inline size_t decode_workspace_bytes(int B, int H, int d, int S) {
  const size_t n = (size_t)B * H * decode_splits(S);
  return n * (2 + (size_t)d) * sizeof(float);
}

// Splits of a decode call: enough 512-position chunks for the most positions
// one query can see.
inline int decode_call_splits(const DecodeLaunch& L) {
  if (!L.block_table) return decode_splits(L.S);
  const long long cap = (long long)L.max_blocks * L.block_size;
  const long long seen = L.is_local && L.window < cap ? L.window : cap;
  return (int)((seen + kDecodeChunk - 1) / kDecodeChunk);
}

struct BackwardLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;  // (B, H, T) natural-log log-sum-exp from the forward
  void* dq;
  void* dk;
  void* dv;
  int B, T, S, H, KVH, d;
  float query_scale, softcap;
  int window, is_local;
  void* workspace;   // backward_workspace_bytes(B, T, S, H) bytes, layout below
};

// Backward workspace: D = <dO, out> per row, float (B, H, T), then, from a
// 256-byte boundary, the dS blocks: for each (b, h, 32-row tile, 16-key
// block) 1 KiB holding dS^T of the block as 16 key rows of 32 bf16 (one per
// query row), in that order.
inline size_t backward_ds_offset(int B, int T, int H) {
  return ((size_t)B * H * T * sizeof(float) + 255) & ~(size_t)255;
}
inline size_t backward_ds_blocks(int B, int T, int S, int H) {
  return (size_t)B * H * (size_t)((T + 31) / 32) * (size_t)((S + 15) / 16);
}
inline size_t backward_workspace_bytes(int B, int T, int S, int H) {
  return backward_ds_offset(B, T, H) + backward_ds_blocks(B, T, S, H) * 1024;
}

hipError_t launch_prefill_backward(const BackwardLaunch& L, hipStream_t stream);

struct RopeLaunch {
  void* x;                  // (B, T, NH, d), rotated in place
  const int32_t* positions;  // (B, T)
  int B, T, NH, d;
  float base;
  int dtype;
};

hipError_t launch_rope(const RopeLaunch& L, hipStream_t stream);
hipError_t launch_softcap(void* x, size_t n, float cap, int dtype, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillLaunch& L, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillLaunch& L, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& L, int dtype, hipStream_t stream);

}  // namespace g2
