// Decode: one new query token per sequence against a KV cache, split over the
// keys (split-K) and merged with a log-sum-exp combine.
//
// Gemma 2 keeps only the last 4096 tokens on local layers (Guide, section 2;
// model card "Method" item 1).  Position j of a sequence lives in cache slot
// j mod S, so a local cache of S = 4096 slots is a ring and a global cache is
// linear; the query of a sequence holding L tokens sits at position L - 1.
//
// The work is HBM-bound (each visible key costs 4*d bytes of K and V for
// 8*d flops per query-head pair), so the kernel is built around the loads:
//  * a workgroup (4 waves) owns kDecodeChunk consecutive positions of one
//    (sequence, K/V head); both query heads of the pair reuse every K/V byte;
//  * a key row is read by a group of d/8 lanes with 16-byte loads (d=256:
//    half a wave per 512-byte row), so every load instruction is coalesced;
//  * K/V rows are read once, with non-temporal loads, so the stream does not
//    evict what other workgroups reuse from the caches;
//  * each lane group keeps 4 keys' loads in flight and its own online-softmax
//    state; logits are reduced across the group with lane shuffles;
//  * groups, then waves (through LDS), are merged at the end, and each split
//    writes (max, sum, unnormalised accumulator) to the workspace;
//  * a second kernel merges the splits of every (sequence, head).
//
// Paged mode (Gemma 2 Guide, "Deep Dive" item 2: block-managed KV memory,
// local layers dropping blocks older than the window): K and V live in a pool
// of fixed-size blocks and a per-sequence table maps logical block i to a
// pool block.  Each split stages the table entries of the blocks it covers in
// LDS once and checks them; the loads then address pool rows through them.
#include "g2_device.h"
#include "g2_kernels.h"

namespace g2 {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* kv_lens;
  int B, S, H, KVH;
  CapConsts cap;
  int window, is_local, nsplit;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  // paged mode
  const int32_t* table;
  int max_blocks, bs_log2, num_blocks;
};

// 16-byte vector of the storage type, kept raw until used.
template <typename E>
struct Vec16;
template <>
struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ static float get(const u32x4& w, int e) {
    return (e & 1) ? bf16_hi_to_f32(w[e >> 1]) : bf16_lo_to_f32(w[e >> 1]);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static float get(const u32x4& w, int e) {
    const f32x4 f = __builtin_bit_cast(f32x4, w);
    return f[e];
  }
};

__device__ __forceinline__ bool decode_len_ok(int L, int S, int window, int is_local) {
  if (L < 1) return false;
  const int seen = is_local ? min(L, window) : L;
  return seen <= S;
}

// Length check of either cache form (paged: the table's capacity).
template <bool PAGED>
__device__ __forceinline__ bool decode_len_ok_any(const DecodeArgs& a, int L) {
  if constexpr (PAGED) return L >= 1 && (long long)L <= ((long long)a.max_blocks << a.bs_log2);
  else return decode_len_ok(L, a.S, a.window, a.is_local);
}

template <typename E, int D, int G, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int VEC = Vec16<E>::N;
  constexpr int LPK = D / VEC;   // lanes per key row (16-byte loads)
  constexpr int KPI = 64 / LPK;  // keys per wave per load instruction
  constexpr int UNR = 4;         // keys per lane group per batch
  static_assert(LPK <= 64 && 64 % LPK == 0, "key row must fit a wave");

  __shared__ float sm_m[4][G], sm_l[4][G];
  __shared__ float sm_acc[4][G][D];
  __shared__ int sm_blk[PAGED ? kDecodeChunk + 1 : 1];  // pool blocks of this split

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane / LPK, sub = lane % LPK;
  const int split = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.KVH, g = bg % a.KVH;
  const int S = a.S;
  const int L = a.kv_lens[b];
  const bool ok = decode_len_ok_any<PAGED>(a, L);
  const int lo = a.is_local ? max(0, L - a.window) : 0;
  const int c0 = lo + split * kDecodeChunk;
  const int c1 = min(c0 + kDecodeChunk, L);
  const size_t part0 = ((size_t)b * a.H + (size_t)g * G) * a.nsplit + split;  // head g*G
  if (!ok || c0 >= c1) {
    if (tid < G) {
      a.ws_m[part0 + (size_t)tid * a.nsplit] = kNegInf;
      a.ws_l[part0 + (size_t)tid * a.nsplit] = 0.f;
    }
    return;
  }
  const int bs_log2 = a.bs_log2;
  const int fb = c0 >> bs_log2;  // first logical block of the split (paged)
  if constexpr (PAGED) {
    const int nb = ((c1 - 1) >> bs_log2) - fb + 1;
    int bad = 0;
    for (int i = tid; i < nb; i += 256) {
      const int e = a.table[(size_t)b * a.max_blocks + fb + i];
      bad |= (e < 0) | (e >= a.num_blocks);
      sm_blk[i] = e;
    }
    if (__syncthreads_or(bad)) {  // a visible position has no pool block: NaN result
      if (tid < G) {
        a.ws_m[part0 + (size_t)tid * a.nsplit] = kNegInf;
        a.ws_l[part0 + (size_t)tid * a.nsplit] = __builtin_nanf("");
      }
      return;
    }
  }

  const E* qbase = static_cast<const E*>(a.q) + ((size_t)b * a.H + (size_t)g * G) * D + sub * VEC;
  float qv[G][VEC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qbase + hh * D);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[hh][e] = Vec16<E>::get(w, e);
  }

  const size_t row_stride = (size_t)a.KVH * D;
  const size_t seq_rows = PAGED ? 0 : (size_t)b * S;  // pools are shared by all sequences
  const E* kb = static_cast<const E*>(a.k) + (seq_rows * a.KVH + g) * D + sub * VEC;
  const E* vb = static_cast<const E*>(a.v) + (seq_rows * a.KVH + g) * D + sub * VEC;

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = kNegInf;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[hh][e] = 0.f;
  }

  const int c0_slot = PAGED ? 0 : c0 % S;
  constexpr int kWaveStep = KPI * UNR;      // positions per wave per batch
  constexpr int kStep = 4 * kWaveStep;      // positions per workgroup per batch
  u32x4 kraw[2][UNR], vraw[2][UNR];

  // Loads of one batch (positions base + u*KPI + grp); positions past c1 load nothing.
  auto load_batch = [&](u32x4 (&kr)[UNR], u32x4 (&vr)[UNR], int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int pos = base + u * KPI + grp;
      size_t slot;  // row of the cache (ring / linear) or of the pool (paged)
      if constexpr (PAGED) {
        slot = 0;
        if (pos < c1)
          slot = ((size_t)sm_blk[(pos >> bs_log2) - fb] << bs_log2) | (size_t)(pos & ((1 << bs_log2) - 1));
      } else {
        int sl = c0_slot + (pos - c0);
        if (sl >= S) sl -= S;
        slot = (size_t)sl;
      }
      if (pos < c1) {
        kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (size_t)slot * row_stride));
        vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (size_t)slot * row_stride));
      } else {
        kr[u] = u32x4{0u, 0u, 0u, 0u};
        vr[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // Logits, soft-cap, online softmax and value accumulation of one batch.
  auto compute_batch = [&](const u32x4 (&kr)[UNR], const u32x4 (&vr)[UNR], int base) __attribute__((always_inline)) {
    float s2[UNR][G];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const bool in = base + u * KPI + grp < c1;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = __builtin_fmaf(qv[hh][e], Vec16<E>::get(kr[u], e), d);
        d = group_sum<LPK>(d);
        const float s = capped_log2(a.cap.mode, d, a.cap.k_in, a.cap.c_out);
        s2[u][hh] = in ? s : kNegInf;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mb = s2[0][hh];
#pragma unroll
      for (int u = 1; u < UNR; ++u) mb = fmaxf(mb, s2[u][hh]);
      const float m_new = fmaxf(m[hh], mb);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m[hh] - m_use);
      float p[UNR];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        p[u] = exp2_fast(s2[u][hh] - m_use);
        ps += p[u];
      }
      l[hh] = l[hh] * alpha + ps;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float x = acc[hh][e] * alpha;
#pragma unroll
        for (int u = 0; u < UNR; ++u) x = __builtin_fmaf(p[u], Vec16<E>::get(vr[u], e), x);
        acc[hh][e] = x;
      }
      m[hh] = m_new;
    }
  };

  // Software pipeline: batch i+1's loads are in flight while batch i is computed.
  int base = c0 + wave * kWaveStep;
  if (base < c1) load_batch(kraw[0], vraw[0], base);
  while (base < c1) {
    if (base + kStep < c1) load_batch(kraw[1], vraw[1], base + kStep);
    compute_batch(kraw[0], vraw[0], base);
    base += kStep;
    if (base >= c1) break;
    if (base + kStep < c1) load_batch(kraw[0], vraw[0], base + kStep);
    compute_batch(kraw[1], vraw[1], base);
    base += kStep;
  }

  // ---- merge the KPI lane groups of this wave
#pragma unroll
  for (int step = LPK; step < 64; step <<= 1) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mo = shfl_xor(m[hh], step);
      const float lo_ = shfl_xor(l[hh], step);
      const float mn = fmaxf(m[hh], mo);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float fa = exp2_fast(m[hh] - mu), fb = exp2_fast(mo - mu);
      l[hh] = l[hh] * fa + lo_ * fb;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = shfl_xor(acc[hh][e], step);
        acc[hh][e] = acc[hh][e] * fa + ao * fb;
      }
      m[hh] = mn;
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (sub == 0) {
        sm_m[wave][hh] = m[hh];
        sm_l[wave][hh] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[wave][hh][sub * VEC + e] = acc[hh][e];
    }
  }
  __syncthreads();
  // ---- merge the 4 waves and write this split's partial result
  for (int i = tid; i < G * D; i += 256) {
    const int hh = i / D, dd = i % D;
    float mn = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) mn = fmaxf(mn, sm_m[w][hh]);
    const float mu = (mn == kNegInf) ? 0.f : mn;
    float ls = 0.f, as = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2_fast(sm_m[w][hh] - mu);
      ls += sm_l[w][hh] * f;
      as += sm_acc[w][hh][dd] * f;
    }
    const size_t pi = part0 + (size_t)hh * a.nsplit;
    a.ws_acc[pi * D + dd] = as;
    if (dd == 0) {
      a.ws_m[pi] = mn;
      a.ws_l[pi] = ls;
    }
  }
}

// One workgroup per (sequence, head): merge the splits and write the output.
template <typename E, int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int L = a.kv_lens[b];
  bool ok = decode_len_ok_any<PAGED>(a, L);
  const size_t p0 = (size_t)bh * a.nsplit;
  // The loops are unrolled so that each issues several splits' loads before
  // it waits on any of them.
  float mx = kNegInf;
#pragma unroll 8
  for (int s = 0; s < a.nsplit; ++s) {
    const float ls = a.ws_l[p0 + s];
    if (ls != ls) ok = false;  // a split that could not read its keys
    if (ls > 0.f) mx = fmaxf(mx, a.ws_m[p0 + s]);
  }
  float lsum = 0.f;
#pragma unroll 8
  for (int s = 0; s < a.nsplit; ++s) {
    const float ls = a.ws_l[p0 + s];
    if (ls > 0.f) lsum += ls * exp2_fast(a.ws_m[p0 + s] - mx);
  }
  const float inv = ok ? 1.0f / lsum : __builtin_nanf("");
  E* orow = static_cast<E*>(a.out) + (size_t)bh * D;
  for (int dd = threadIdx.x; dd < D; dd += blockDim.x) {
    float x = 0.f;
#pragma unroll 8
    for (int s = 0; s < a.nsplit; ++s) {
      const float ls = a.ws_l[p0 + s];
      if (ls > 0.f) x += a.ws_acc[(p0 + s) * D + dd] * exp2_fast(a.ws_m[p0 + s] - mx);
    }
    orow[dd] = (E)(x * inv);
  }
}

template <typename E, int D, int G, bool PAGED>
static hipError_t launch_decode_p(DecodeArgs a, int B, int KVH, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<E, D, G, PAGED>), dim3(a.nsplit, B * KVH), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<E, D, PAGED>), dim3(B * a.H), dim3(D < 256 ? D : 256), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int D, int G>
static hipError_t launch_decode_t(DecodeArgs a, int B, int KVH, hipStream_t stream) {
  return a.table ? launch_decode_p<E, D, G, true>(a, B, KVH, stream)
                 : launch_decode_p<E, D, G, false>(a, B, KVH, stream);
}

template <typename E>
static hipError_t launch_decode_e(const DecodeArgs& a, int d, int G, int B, int KVH, hipStream_t stream) {
  switch (d) {
    case 64: return G == 2 ? launch_decode_t<E, 64, 2>(a, B, KVH, stream) : launch_decode_t<E, 64, 1>(a, B, KVH, stream);
    case 128: return G == 2 ? launch_decode_t<E, 128, 2>(a, B, KVH, stream) : launch_decode_t<E, 128, 1>(a, B, KVH, stream);
    case 256: return G == 2 ? launch_decode_t<E, 256, 2>(a, B, KVH, stream) : launch_decode_t<E, 256, 1>(a, B, KVH, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeLaunch& L, int dtype, hipStream_t stream) {
  DecodeArgs a;
  a.q = L.q;
  a.k = L.k;
  a.v = L.v;
  a.out = L.out;
  a.kv_lens = L.kv_lens;
  a.B = L.B;
  a.S = L.S;
  a.H = L.H;
  a.KVH = L.KVH;
  a.cap = make_cap_consts(L.query_scale, L.softcap);
  a.window = L.window;
  a.is_local = L.is_local;
  a.nsplit = decode_call_splits(L);
  a.table = L.block_table;
  a.max_blocks = L.max_blocks;
  a.num_blocks = L.num_blocks;
  a.bs_log2 = 0;
  while (L.block_size > (1 << a.bs_log2)) ++a.bs_log2;
  const size_t n = (size_t)L.B * L.H * a.nsplit;
  float* ws = static_cast<float*>(L.workspace);
  a.ws_m = ws;
  a.ws_l = ws + n;
  a.ws_acc = ws + 2 * n;
  const int G = L.H / L.KVH;
  return dtype == 0 ? launch_decode_e<bf16>(a, L.d, G, L.B, L.KVH, stream)
                    : launch_decode_e<float>(a, L.d, G, L.B, L.KVH, stream);
}

}  // namespace g2
