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
};

// Keys handled by one split-K workgroup of the decode kernel.
constexpr int kDecodeChunk = 512;

inline int decode_splits(int S) { return (S + kDecodeChunk - 1) / kDecodeChunk; }

// Workspace layout: float m[B*H*splits], l[B*H*splits], acc[B*H*splits*d].
inline size_t decode_workspace_bytes(int B, int H, int d, int S) {
  const size_t n = (size_t)B * H * decode_splits(S);
  return n * (2 + (size_t)d) * sizeof(float);
}

hipError_t launch_prefill_bf16(const PrefillLaunch& L, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillLaunch& L, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& L, int dtype, hipStream_t stream);

}  // namespace g2
