// Steps on either side of the attention call, both elementwise and HBM-bound.
//
// Rotary embedding (wikillm model card "Method" item 5: Gemma 2 keeps the
// rotary embeddings of Gemma 1; the pages give no formula).  Pair i of a head
// vector is (x[i], x[i + d/2]), i < d/2, rotated by pos * base^(-2i/d), the
// rotary embedding of Su et al. in its half-split layout.  One thread owns 16
// bytes of each half of a (batch, position) row (8 bf16 or 4 fp32 pairs),
// computes those pairs' angles once and applies them to every head of the
// row, so sin/cos cost is amortised over the heads and every access is a
// coalesced 16-byte load or store.  The angle is formed and reduced to
// [-pi, pi] in fp64 (positions reach thousands of radians), then sin/cos are
// evaluated in fp32.
//
// Final-logit soft-cap (Gemma 2 Guide, section 1, second formula): the
// vocabulary logits become cap * tanh(x / cap) with cap = 30, in place.
//
// The logits are streamed once (non-temporal loads and stores); Q and K are
// usually still in the caches from the projection that produced them, so the
// rotary embedding uses ordinary accesses.
#include "g2_device.h"
#include "g2_kernels.h"

namespace g2 {

template <typename E>
struct Lanes16;
template <>
struct Lanes16<bf16> {
  static constexpr int N = 8;
  template <bool NT>
  __device__ static void load(const bf16* p, float (&v)[8]) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    const u32x4 w = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo_to_f32(w[e]);
      v[2 * e + 1] = bf16_hi_to_f32(w[e]);
    }
  }
  template <bool NT>
  __device__ static void store(bf16* p, const float (&v)[8]) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    if (NT) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = w;
  }
};
template <>
struct Lanes16<float> {
  static constexpr int N = 4;
  template <bool NT>
  __device__ static void load(const float* p, float (&v)[4]) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    const f32x4 w = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = w[e];
  }
  template <bool NT>
  __device__ static void store(float* p, const float (&v)[4]) {
    const f32x4 w = {v[0], v[1], v[2], v[3]};
    if (NT) __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = w;
  }
};

template <typename E, int D>
__global__ __launch_bounds__(256) void rope_kernel(E* x, const int32_t* positions, long rows, int NH,
                                                   double log2_base) {
  constexpr int N = Lanes16<E>::N;
  constexpr int HALF = D / 2;
  constexpr int GROUPS = HALF / N;  // threads per (batch, position) row
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long r = gid / GROUPS;
  if (r >= rows) return;
  const int i0 = (int)(gid % GROUPS) * N;
  const double pos = (double)positions[r];
  constexpr double kTwoPi = 6.283185307179586476925;
  float c[N], s[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const double theta = pos * exp2(-(2.0 * (i0 + j) / D) * log2_base);
    const double turns = rint(theta * (1.0 / kTwoPi));
    const float red = (float)fma(-turns, kTwoPi, theta);
    sincosf(red, &s[j], &c[j]);
  }
  E* row = x + (size_t)r * NH * D + i0;
  for (int h = 0; h < NH; ++h, row += D) {
    float a[N], b[N];
    Lanes16<E>::template load<false>(row, a);
    Lanes16<E>::template load<false>(row + HALF, b);
    float ya[N], yb[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      ya[j] = a[j] * c[j] - b[j] * s[j];
      yb[j] = b[j] * c[j] + a[j] * s[j];
    }
    Lanes16<E>::template store<false>(row, ya);
    Lanes16<E>::template store<false>(row + HALF, yb);
  }
}

template <typename E>
__global__ __launch_bounds__(256) void softcap_kernel(E* x, size_t n, float cap, float inv_cap) {
  constexpr int N = Lanes16<E>::N;
  const size_t nvec = n / N;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
    float v[N];
    Lanes16<E>::template load<true>(x + i * N, v);
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = cap * tanhf(v[e] * inv_cap);
    Lanes16<E>::template store<true>(x + i * N, v);
  }
  // tail: the last n % N elements, one thread each
  const size_t t = nvec * N + (size_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && t < n) x[t] = (E)(cap * tanhf((float)x[t] * inv_cap));
}

template <typename E, int D>
static void launch_rope_t(E* x, const RopeLaunch& L, long rows, double l2b, hipStream_t stream) {
  constexpr long kGroups = D / 2 / Lanes16<E>::N;
  const unsigned grid = (unsigned)((rows * kGroups + 255) / 256);
  hipLaunchKernelGGL((rope_kernel<E, D>), dim3(grid), dim3(256), 0, stream, x, L.positions, rows, L.NH, l2b);
}

template <typename E>
static hipError_t launch_rope_e(E* x, const RopeLaunch& L, hipStream_t stream) {
  const long rows = (long)L.B * L.T;
  const double l2b = log2((double)L.base);
  switch (L.d) {
    case 64: launch_rope_t<E, 64>(x, L, rows, l2b, stream); break;
    case 128: launch_rope_t<E, 128>(x, L, rows, l2b, stream); break;
    case 256: launch_rope_t<E, 256>(x, L, rows, l2b, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rope(const RopeLaunch& L, hipStream_t stream) {
  return L.dtype == 0 ? launch_rope_e(static_cast<bf16*>(L.x), L, stream)
                      : launch_rope_e(static_cast<float*>(L.x), L, stream);
}

hipError_t launch_softcap(void* x, size_t n, float cap, int dtype, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t per = dtype == 0 ? 8 : 4;
  const size_t nvec = n / per;
  size_t blocks = (nvec + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond this
  if (blocks == 0) blocks = 1;
  if (dtype == 0)
    hipLaunchKernelGGL(softcap_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<bf16*>(x), n, cap, 1.0f / cap);
  else
    hipLaunchKernelGGL(softcap_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<float*>(x), n, cap, 1.0f / cap);
  return hipGetLastError();
}

}  // namespace g2
