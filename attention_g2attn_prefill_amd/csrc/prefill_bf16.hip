// Fused prefill kernel for Gemma 2 attention, bf16 storage, fp32 accumulation,
// on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// What one layer computes (Gemma 2 model card, "Method", one-layer attention
// pseudocode): scaled logits of each query head against the key/value head its
// group shares, soft-cap cap*tanh(x/cap), causal mask (local layers: also a
// sliding window), softmax over keys, weighted sum of values.
//
// Design (MI355X-first):
//  * One workgroup = 4 waves = 128 query rows that all read the same K/V head:
//    with two query heads per K/V head (the card's "Method" item 4) that is 64
//    positions x 2 heads, so every K/V tile staged in LDS serves both heads.
//  * Transposed scores: each wave computes S^T = K * Q^T (keys x queries) with
//    K from LDS as the A operand and its 32 queries' Q^T kept in registers as
//    the B operand.  The accumulator layout then gives every lane whole
//    columns (queries), so the softmax row statistics are per-lane values and
//    P^T feeds the P*V product (O^T = V^T * P^T) straight from registers.
//  * V is transposed once on its way into LDS (4 keys x 8 dims per thread,
//    repacked in registers), so V^T operands are plain 8-byte LDS reads.
//  * Soft-cap, mask and online softmax run in fp32 in base 2 (log2(e) is folded
//    into the constants).  The running max is rescaled lazily: only when a
//    row's max grows by more than 8 (log2 units) are O and l multiplied down.
//  * Tiles wholly outside the causal / sliding-window band are skipped; the
//    mask is evaluated only on tiles that cross the band's edges.
//  * Work order: heaviest query blocks first (causal rows near the end see the
//    most keys); consecutive workgroups take different (batch, kv-head) pairs,
//    which the dispatcher spreads over the 8 XCDs, so each XCD's L2 keeps
//    serving the same K/V heads.
#include "g2_device.h"
#include "g2_kernels.h"

namespace g2 {

template <int D, int G, int BN>
struct PrefillShape {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQPW = 32;                 // query rows per wave
  static constexpr int kWPH = kWaves / G;         // waves per query head
  static constexpr int kBMP = kQPW * kWPH;        // positions per workgroup
  static constexpr int kKK = D / 32;              // MFMA k-steps over d
  static constexpr int kDB = D / 16;              // 16-row blocks of O^T
  static constexpr int kNB = BN / 16;             // 16-key blocks per tile
  static constexpr int kKS = BN / 32;             // 32-key steps of P*V
  static constexpr int kKStr = D + 8;             // K row stride in LDS (elements)
  static constexpr int kVStr = BN + 4;            // V^T row stride in LDS (elements)
  static constexpr int kLdsBytes = (BN * kKStr + D * kVStr) * 2;
  static_assert(BN % 32 == 0, "tile must hold whole 32-key steps");
  static_assert(G == 1 || G == 2, "one or two query heads per K/V head");
};

struct PrefillArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* out;
  int T, S, H, KVH;
  CapConsts cap;
  int window;
  int is_local;
  int n_mblocks;
};

template <int D, int G, int BN>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a) {
  using P = PrefillShape<D, G, BN>;
  constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
  __shared__ __attribute__((aligned(16))) bf16 k_lds[BN * P::kKStr];
  __shared__ __attribute__((aligned(16))) bf16 vt_lds[D * P::kVStr];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lq = lane >> 4;  // 0..3

  const int nbg = gridDim.x / a.n_mblocks;  // B*KVH
  const int bid = blockIdx.x;
  const int mb = a.n_mblocks - 1 - bid / nbg;  // heaviest first
  const int bg = bid % nbg;
  const int b = bg / a.KVH;
  const int g = bg % a.KVH;
  const int h = g * G + wave / P::kWPH;
  const int T = a.T, S = a.S, H = a.H, KVH = a.KVH;
  const int off = S - T;
  const int t0 = mb * P::kBMP + (wave % P::kWPH) * P::kQPW;  // first row of this wave

  // ---- Q^T fragments (B operand): lane holds query 16*qb + l16, dims 32*kk + 8*lq .. +7
  bf16x8 qf[2][P::kKK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = t0 + qb * 16 + l16;
    const bf16* qrow = a.q + (((size_t)b * T + (t < T ? t : 0)) * H + h) * D + lq * 8;
#pragma unroll
    for (int kk = 0; kk < P::kKK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (t < T) w = *reinterpret_cast<const u32x4*>(qrow + kk * 32);
      qf[qb][kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- key range of the workgroup and of this wave
  const int wg_t_last = min(mb * P::kBMP + P::kBMP, T) - 1;
  const int wg_p_first = mb * P::kBMP + off;
  const int wg_p_last = wg_t_last + off;
  const int j_lo = a.is_local ? max(0, wg_p_first - a.window + 1) : 0;
  const int j_hi = wg_p_last;  // inclusive, <= S-1
  const int n_start = (j_lo / BN) * BN;

  const bool wave_active = t0 < T;
  const int w_p_first = t0 + off;
  const int w_p_last = min(t0 + P::kQPW - 1, T - 1) + off;
  const int w_j_lo = a.is_local ? max(0, w_p_first - a.window + 1) : 0;
  const int w_j_lo_last = a.is_local ? max(0, w_p_last - a.window + 1) : 0;

  f32x4 o[P::kDB][2];
#pragma unroll
  for (int db = 0; db < P::kDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {kNegInf, kNegInf};
  float l_run[2] = {0.f, 0.f};

  const size_t kv_row_stride = (size_t)KVH * D;
  const bf16* kbase = a.k + ((size_t)b * S * KVH + g) * D;
  const bf16* vbase = a.v + ((size_t)b * S * KVH + g) * D;

  for (int n0 = n_start; n0 <= j_hi; n0 += BN) {
    // ---- stage K (row-major) and V^T (dim-major) tiles in LDS
    constexpr int kKCh = D / 8;           // 16-byte chunks per K row
    constexpr int kKU = BN * kKCh;        // K chunks per tile
    constexpr int kNKG = BN / 4;          // 4-key groups
    constexpr int kVU = kNKG * (D / 8);   // V transpose units (4 keys x 8 dims)
    constexpr int kKIt = (kKU + P::kThreads - 1) / P::kThreads;
    constexpr int kVIt = (kVU + P::kThreads - 1) / P::kThreads;
    __syncthreads();  // previous tile fully consumed
    {
      u32x4 kreg[kKIt];
#pragma unroll
      for (int it = 0; it < kKIt; ++it) {
        const int u = tid + it * P::kThreads;
        const int row = u / kKCh, c = u % kKCh;
        const int j = n0 + row;
        kreg[it] = u32x4{0u, 0u, 0u, 0u};
        if (u < kKU && j < S) kreg[it] = *reinterpret_cast<const u32x4*>(kbase + j * kv_row_stride + c * 8);
      }
#pragma unroll
      for (int it = 0; it < kKIt; ++it) {
        const int u = tid + it * P::kThreads;
        const int row = u / kKCh, c = u % kKCh;
        if (u < kKU) *reinterpret_cast<u32x4*>(&k_lds[row * P::kKStr + c * 8]) = kreg[it];
      }
    }
#pragma unroll
    for (int it = 0; it < kVIt; ++it) {
      const int u = tid + it * P::kThreads;
      const int kg = u % kNKG, dg = u / kNKG;
      u32x4 vreg[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = n0 + kg * 4 + r;
        vreg[r] = u32x4{0u, 0u, 0u, 0u};
        if (u < kVU && j < S) vreg[r] = *reinterpret_cast<const u32x4*>(vbase + j * kv_row_stride + dg * 8);
      }
      if (u < kVU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dword e of each key row holds dims (8dg+2e, 8dg+2e+1)
          const uint32_t r0 = vreg[0][e], r1 = vreg[1][e];
          const uint32_t r2 = vreg[2][e], r3 = vreg[3][e];
          u32x2 lo, hi;
          lo[0] = (r0 & 0xffffu) | (r1 << 16);
          lo[1] = (r2 & 0xffffu) | (r3 << 16);
          hi[0] = (r0 >> 16) | (r1 & 0xffff0000u);
          hi[1] = (r2 >> 16) | (r3 & 0xffff0000u);
          const int d0 = dg * 8 + 2 * e;
          *reinterpret_cast<u32x2*>(&vt_lds[d0 * P::kVStr + kg * 4]) = lo;
          *reinterpret_cast<u32x2*>(&vt_lds[(d0 + 1) * P::kVStr + kg * 4]) = hi;
        }
      }
    }
    __syncthreads();

    // ---- does this wave see any key of the tile?
    if (!wave_active || n0 > w_p_last || n0 + BN - 1 < w_j_lo) continue;
    const bool need_mask = (n0 + BN - 1 > w_p_first) || (n0 + BN > S) ||
                           (a.is_local && n0 < w_j_lo_last);

    // ---- S^T = K * Q^T
    f32x4 st[P::kNB][2];
#pragma unroll
    for (int kb = 0; kb < P::kNB; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) st[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < P::kKK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < P::kNB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&k_lds[(kb * 16 + l16) * P::kKStr + kk * 32 + lq * 8]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          st[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][kk], st[kb][qb], 0, 0, 0);
      }
    }

    // ---- soft-cap (log2 units) and mask; the cap form is uniform per launch
    auto cap_and_mask = [&](auto capfn) {
#pragma unroll
      for (int kb = 0; kb < P::kNB; ++kb) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float s2 = capfn(st[kb][qb][i]);
            if (need_mask) {
              const int j = n0 + kb * 16 + lq * 4 + i;
              const int p = t0 + qb * 16 + l16 + off;
              const bool vis = (j <= p) && (j < S) && (!a.is_local || j > p - a.window);
              s2 = vis ? s2 : kNegInf;
            }
            st[kb][qb][i] = s2;
          }
        }
      }
    };
    const float k_in = a.cap.k_in, c_out = a.cap.c_out;
    if (a.cap.mode == kCapFast)
      cap_and_mask([&](float x) { return capped_log2_fast(x, k_in, c_out); });
    else if (a.cap.mode == kCapAccurate)
      cap_and_mask([&](float x) { return capped_log2_accurate(x, k_in, c_out); });
    else
      cap_and_mask([&](float x) { return x * k_in; });

    // ---- online softmax (per lane: two query columns)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < P::kNB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, st[kb][qb][i]);
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const bool grow = mt > m_run[qb] + kTau;  // true also for the first visible keys
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mt : m_run[qb];
        const float alpha = grow ? exp2_fast(m_run[qb] - m_new) : 1.0f;
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < P::kDB; ++db) o[db][qb] *= alpha;
      }
      const float m_use = (m_run[qb] == kNegInf) ? 0.0f : m_run[qb];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < P::kNB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_fast(st[kb][qb][i] - m_use);
          st[kb][qb][i] = p;
          ls += p;
        }
      l_run[qb] += ls;
    }

    // ---- O^T += V^T * P^T
#pragma unroll
    for (int ks = 0; ks < P::kKS; ++ks) {
      bf16x8 pf[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        u32x4 w;
        w[0] = pack_bf16x2(st[2 * ks][qb][0], st[2 * ks][qb][1]);
        w[1] = pack_bf16x2(st[2 * ks][qb][2], st[2 * ks][qb][3]);
        w[2] = pack_bf16x2(st[2 * ks + 1][qb][0], st[2 * ks + 1][qb][1]);
        w[3] = pack_bf16x2(st[2 * ks + 1][qb][2], st[2 * ks + 1][qb][3]);
        pf[qb] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int db = 0; db < P::kDB; ++db) {
        const bf16* vrow = &vt_lds[(db * 16 + l16) * P::kVStr + ks * 32 + lq * 4];
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(vrow + 16);
        const u32x4 aw = {a0[0], a0[1], a1[0], a1[1]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, aw);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], o[db][qb], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
  // ---- epilogue: O = O^T / l, bf16, store 4 consecutive dims per lane and block
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l_run[qb];
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    const int t = t0 + qb * 16 + l16;
    if (t < T) {
      bf16* orow = a.out + (((size_t)b * T + t) * H + h) * D + lq * 4;
#pragma unroll
      for (int db = 0; db < P::kDB; ++db) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][qb][0] * inv, o[db][qb][1] * inv);
        w[1] = pack_bf16x2(o[db][qb][2] * inv, o[db][qb][3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 16) = w;
      }
    }
  }
}

template <int D, int G, int BN>
static hipError_t launch_prefill_bf16_t(const PrefillLaunch& L, hipStream_t stream) {
  using P = PrefillShape<D, G, BN>;
  PrefillArgs a;
  a.q = static_cast<const bf16*>(L.q);
  a.k = static_cast<const bf16*>(L.k);
  a.v = static_cast<const bf16*>(L.v);
  a.out = static_cast<bf16*>(L.out);
  a.T = L.T;
  a.S = L.S;
  a.H = L.H;
  a.KVH = L.KVH;
  a.cap = make_cap_consts(L.query_scale, L.softcap);
  a.window = L.window;
  a.is_local = L.is_local;
  a.n_mblocks = (L.T + P::kBMP - 1) / P::kBMP;
  const unsigned grid = (unsigned)a.n_mblocks * (unsigned)(L.B * L.KVH);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G, BN>), dim3(grid), dim3(P::kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillLaunch& L, hipStream_t stream) {
  const int G = L.H / L.KVH;
  switch (L.d) {
    case 64:
      return G == 2 ? launch_prefill_bf16_t<64, 2, 64>(L, stream) : launch_prefill_bf16_t<64, 1, 64>(L, stream);
    case 128:
      return G == 2 ? launch_prefill_bf16_t<128, 2, 64>(L, stream) : launch_prefill_bf16_t<128, 1, 64>(L, stream);
    case 256:
      return G == 2 ? launch_prefill_bf16_t<256, 2, 32>(L, stream) : launch_prefill_bf16_t<256, 1, 32>(L, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace g2
