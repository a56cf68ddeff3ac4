// Device-side helpers shared by the g2attn HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// v_exp_f32: 2^x (exact -inf -> 0, +inf -> inf).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// v_rcp_f32: 1/x to about 1 ulp.
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// Soft-cap modes, picked on the host from the cap value.
enum CapMode : int { kCapNone = 0, kCapFast = 1, kCapAccurate = 2 };
// Caps up to this value use the fast form below; larger ones the accurate form.
constexpr float kFastCapLimit = 256.0f;

struct CapConsts {
  int mode;
  float k_in;   // fast: 2*log2(e)*qs/cap; accurate: qs/cap; none: qs*log2(e)
  float c_out;  // cap*log2(e) (unused by kCapNone)
};

inline CapConsts make_cap_consts(float query_scale, float softcap) {
  CapConsts c;
  if (!(softcap > 0.0f) || __builtin_isinf(softcap)) {
    c.mode = kCapNone;
    c.k_in = query_scale * kLog2e;
    c.c_out = 0.0f;
  } else if (softcap <= kFastCapLimit) {
    c.mode = kCapFast;
    c.k_in = 2.0f * kLog2e * query_scale / softcap;
    c.c_out = softcap * kLog2e;
  } else {
    c.mode = kCapAccurate;
    c.k_in = query_scale / softcap;
    c.c_out = softcap * kLog2e;
  }
  return c;
}

// Soft-capped logit in log2 units, cap*log2(e)*tanh(qs*x/cap), fast form:
//   tanh(y) = 1 - 2 / (1 + e^{2y}),  e^{2y} = 2^{x*k_in}.
// Saturates cleanly (e^{2y} -> inf gives +c_out, -> 0 gives -c_out).  The
// subtraction 1 - 2r cancels near y = 0, so the absolute error is a few
// ulp(1) times c_out: about 1e-5 (log2 units) at cap 50 and at most ~1e-4 for
// caps up to kFastCapLimit, far below the bf16 rounding of the weights.
__device__ __forceinline__ float capped_log2_fast(float x, float k_in, float c_out) {
  const float e = exp2_fast(x * k_in);
  const float r = rcp_fast(1.0f + e);
  return __builtin_fmaf(-2.0f * c_out, r, c_out);
}

// Accurate form for large caps, where tanh works near 0 and the fast form's
// absolute error (proportional to the cap) would show: y = qs*x/cap;
//   |y| < 1/4: odd Taylor polynomial through y^9 (next term < 3e-9 relative);
//   else:      sign(y) * (1 - e) / (1 + e),  e = e^{-2|y|} <= 0.61 (no cancellation).
__device__ __forceinline__ float capped_log2_accurate(float x, float k_in, float c_out) {
  const float y = x * k_in;
  const float a = __builtin_fabsf(y);
  const float y2 = y * y;
  float poly = __builtin_fmaf(y2, 62.0f / 2835.0f, -17.0f / 315.0f);
  poly = __builtin_fmaf(y2, poly, 2.0f / 15.0f);
  poly = __builtin_fmaf(y2, poly, -1.0f / 3.0f);
  const float t_small = __builtin_fmaf(y * y2, poly, y);
  const float e = exp2_fast(-2.0f * kLog2e * a);
  const float t_big = __builtin_copysignf((1.0f - e) * rcp_fast(1.0f + e), y);
  return c_out * (a < 0.25f ? t_small : t_big);
}

__device__ __forceinline__ float capped_log2(int mode, float x, float k_in, float c_out) {
  if (mode == kCapFast) return capped_log2_fast(x, k_in, c_out);
  if (mode == kCapAccurate) return capped_log2_accurate(x, k_in, c_out);
  return x * k_in;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16x2 (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (bf16)lo;
  r[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// All-reduce over the lane pairs (l, l^16) and (l, l^32) of a wave64 using the
// gfx950 row / half-wave swaps (plain VALU, no LDS round trip).  After
// v_permlane16_swap(x, x) the two results hold, in every lane, x of the lane
// itself and of lane l^16 (in some order); likewise v_permlane32_swap for
// l^32.  Applying a commutative op to the pair therefore reduces over both.
// The second operand goes through an empty asm so the compiler cannot treat
// the two inputs as one value (it would then fold the pair to one result).
__device__ __forceinline__ unsigned opaque_copy(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}
template <typename Op>
__device__ __forceinline__ float reduce_xor16_32(float v, Op op) {
  unsigned u = __builtin_bit_cast(unsigned, v);
  auto a = __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false);
  v = op(__builtin_bit_cast(float, (unsigned)a[0]), __builtin_bit_cast(float, (unsigned)a[1]));
  u = __builtin_bit_cast(unsigned, v);
  auto b = __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
  return op(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}
__device__ __forceinline__ float max_xor16_32(float v) {
  return reduce_xor16_32(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float min_xor16_32(float v) {
  return reduce_xor16_32(v, [](float x, float y) { return fminf(x, y); });
}
// Min over the same lanes for values that are all >= +0 (or +inf): such floats
// order like their bit patterns, so an unsigned min replaces the float min
// and needs none of the NaN-quieting a float min of lane-swapped values gets.
__device__ __forceinline__ float min_xor16_32_nonneg(float v) {
  unsigned u = __builtin_bit_cast(unsigned, v);
  auto a = __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false);
  u = min((unsigned)a[0], (unsigned)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
  return __builtin_bit_cast(float, min((unsigned)b[0], (unsigned)b[1]));
}
__device__ __forceinline__ float sum_xor16_32(float v) {
  return reduce_xor16_32(v, [](float x, float y) { return x + y; });
}

// All-reduce (sum) over aligned groups of N lanes (N = 1..64, power of two),
// built from DPP lane swizzles and the gfx950 row / half-wave swaps, all plain
// VALU: xor 1 and xor 2 within a quad (quad_perm), then the 8-lane half-row
// mirror (pairs quad 0 with quad 1), the 16-lane row mirror (pairs the two
// halves of a row), then the 16- and 32-lane swaps.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  if constexpr (N >= 4) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  if constexpr (N >= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  if constexpr (N >= 16) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  if constexpr (N >= 32) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    auto a = __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false);
    v = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
  }
  if constexpr (N >= 64) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    auto b = __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
    v = __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
  }
  return v;
}

// Lane exchange within a wave64 (ds_bpermute based).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  int src = lane ^ mask;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

}  // namespace g2
