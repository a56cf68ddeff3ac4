// Prefill for fp32 storage: fp32 arithmetic throughout, with the device
// library's tanhf / expf so the soft-cap is accurate to a few ulp (the fp32
// path is held to 1e-4 absolute against the fp64 definition).
//
// One wave per (batch, query row, head).  Lanes split the head dimension; each
// visible key's logit is reduced across the wave, soft-capped
// (cap*tanh(x/cap), Gemma 2 model card "Method"), and folded into an online
// softmax.  Only the keys the causal / sliding-window mask allows are visited.
#include "g2_device.h"
#include "g2_kernels.h"

namespace g2 {

struct PrefillF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* out;
  float* lse;  // optional (B, H, T), natural log
  int B, T, S, H, KVH, G;
  float query_scale, softcap;
  int use_cap, window, is_local;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillF32Args a) {
  constexpr int E = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, t, h) flat
  const long rows = (long)a.B * a.T * a.H;
  if (row >= rows) return;
  const int h = (int)(row % a.H);
  const int t = (int)((row / a.H) % a.T);
  const int b = (int)(row / ((long)a.H * a.T));
  const int g = h / a.G;
  const int p = t + a.S - a.T;
  const int lo = a.is_local ? max(0, p - a.window + 1) : 0;

  float qv[E], acc[E];
  const float* qrow = a.q + row * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = qrow[lane + 64 * e] * a.query_scale;
    acc[e] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  const size_t stride = (size_t)a.KVH * D;
  const float* kb = a.k + ((size_t)b * a.S * a.KVH + g) * D;
  const float* vb = a.v + ((size_t)b * a.S * a.KVH + g) * D;
  for (int j = lo; j <= p; ++j) {
    const float* kr = kb + (size_t)j * stride;
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) x = __builtin_fmaf(qv[e], kr[lane + 64 * e], x);
    x = wave_sum(x);
    const float s = a.use_cap ? a.softcap * tanhf(x / a.softcap) : x;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);  // m = -inf on the first key: 0
    const float w = expf(s - m_new);
    l = l * alpha + w;
    const float* vr = vb + (size_t)j * stride;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(w, vr[lane + 64 * e], acc[e] * alpha);
    m = m_new;
  }
  float* orow = a.out + row * D;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[lane + 64 * e] = acc[e] / l;
  if (a.lse && lane == 0) a.lse[((size_t)b * a.H + h) * a.T + t] = m + logf(l);
}

hipError_t launch_prefill_f32(const PrefillLaunch& L, hipStream_t stream) {
  PrefillF32Args a;
  a.q = static_cast<const float*>(L.q);
  a.k = static_cast<const float*>(L.k);
  a.v = static_cast<const float*>(L.v);
  a.out = static_cast<float*>(L.out);
  a.lse = L.lse;
  a.B = L.B;
  a.T = L.T;
  a.S = L.S;
  a.H = L.H;
  a.KVH = L.KVH;
  a.G = L.H / L.KVH;
  a.query_scale = L.query_scale;
  a.softcap = L.softcap;
  a.use_cap = (L.softcap > 0.0f && !__builtin_isinf(L.softcap)) ? 1 : 0;
  a.window = L.window;
  a.is_local = L.is_local;
  const long rows = (long)L.B * L.T * L.H;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  switch (L.d) {
    case 64: hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3(grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3(grid), dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(prefill_f32_kernel<256>, dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace g2
