// Allocation-free decode: g2attn_decode with its split-K scratch in a
// file-scope device array instead of a caller-supplied workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array lives in the library's code object: every GPU the library runs on
// holds one copy of G2ATTN_NOALLOC_SCRATCH_BYTES bytes until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory, so its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) on the first call on that device and kept; only that address
// is ever handed to the kernels.  All calls on one GPU share its array, so
// calls that overlap in time on one GPU race (serialise them, e.g. on one
// stream).  The decode kernels write every scratch entry they read (each split
// stores its max and sum, even when empty), so nothing must start at zero.
#include <mutex>

#include "g2_kernels.h"
#include "g2attn.h"

static __device__ __align__(256) unsigned char scratch[G2ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's scratch array (looked up once).
int current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return G2_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return G2_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return G2_OK;
}

}  // namespace

extern "C" int g2attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     void* out, const int32_t* kv_lens, int B, int T, int S,
                                     int H, int KVH, int d, float query_scale, float softcap,
                                     int window, int is_local, int dtype, hipStream_t stream) {
  const int st = g2attn_check_args(B, T, S, H, KVH, d, window, is_local, dtype, 1);
  if (st != G2_OK) return st;
  if (g2::decode_workspace_bytes(B, H, d, S) > (size_t)G2ATTN_NOALLOC_SCRATCH_BYTES)
    return G2_ERR_WORKSPACE;
  void* ws = nullptr;
  const int sst = current_scratch(&ws);
  if (sst != G2_OK) return sst;
  return g2attn_decode(q, k_cache, v_cache, out, kv_lens, B, T, S, H, KVH, d, query_scale,
                       softcap, window, is_local, dtype, ws,
                       (size_t)G2ATTN_NOALLOC_SCRATCH_BYTES, stream);
}
