// Backward pass of the prefill, bf16 storage, fp32 accumulation, on gfx950
// MFMA (v_mfma_f32_16x16x32_bf16).
//
// What it differentiates (Gemma 2 Guide, "Deep Dive" item 1, the cap's
// derivative 1 - tanh^2(x/cap); wikillm model card "Method" for the layer):
// for a row with capped logits s_j = cap tanh(x_j / cap), x_j = qs <q, k_j>,
// weights w_j = exp(s_j - lse) and upstream gradient dO,
//   dv_j += w_j dO,  D = <dO, out>,  ds_j = w_j (<dO, v_j> - D),
//   dx_j = ds_j (1 - tanh^2),  dq = qs sum_j dx_j k_j,  dk_j += qs dx_j q.
// lse is the forward's log-sum-exp (g2attn_prefill_lse), so nothing of the
// forward is stored but the output and lse.
//
// Three kernels:
//  * prep: D per row (B, H, T) into the workspace;
//  * dK/dV, key-stationary: a workgroup owns 64 keys of one K/V head (16 per
//    wave).  Each wave keeps its keys' K and V fragments and its dK^T, dV^T
//    accumulators in registers and streams 32-row tiles of Q and dO (both
//    heads of the GQA pair) through double-buffered LDS.  Per tile:
//    S = Q K^T and dP = dO V^T with the tile as A operand (ds_read_b128) and
//    the stationary fragments as B; each lane then holds one key column and
//    eight query rows, so P and dS are formed in registers and feed
//    dV^T += dO^T P and dK^T += Q^T dS with the tile's transpose (the LDS
//    transpose read) as A operand.  The bf16 dS of the tile (the operand of
//    dK) is also stored to the workspace, 1 KiB per wave, as 16 key rows of
//    32 query columns;
//  * dQ, query-stationary: dQ = dS K needs no recomputation of S and dP.  A
//    workgroup owns BMP positions of the heads of one K/V head and streams
//    32-key tiles of K and the matching stored dS blocks through
//    double-buffered LDS; a wave holds dQ^T for 64 rows of one head and up to
//    128 dims and forms dQ^T += K^T dS^T with both operands from transpose
//    reads.
// Every tile uses one 16-byte-chunk swizzle, byte (c/4)*R*64 + r*64 +
// 16*((c%4) ^ sw(r)) for chunk c of row r of an R-row tile, with
// sw(r) = (r/2) % 4.  With it neither the row reads (ds_read_b128) nor the
// transpose reads (ds_read_b64_tr_b16) of a tile meet a bank conflict, so
// one layout serves both uses of Q, dO, K and dS.  The stored dS blocks are
// not swizzled; the dQ kernel's copies apply the swizzle.
#include "g2_device.h"
#include "g2_kernels.h"
#define G2_TILES_FN __host__ __device__ inline
#include "g2_tiles.h"

#include <type_traits>

namespace g2 {

typedef short s16x4_b __attribute__((ext_vector_type(4)));
typedef short s16x8_b __attribute__((ext_vector_type(8)));
#define G2B_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define G2B_LDS_S16X4(p) ((__attribute__((address_space(3))) s16x4_b*)(p))

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* out;
  const bf16* dout;
  const float* lse;  // (B, H, T), natural log
  float* dsum;       // (B, H, T): D = <dO, out>, written by the prep kernel
  char* ds;          // dS blocks, 1 KiB per (b, h, 32-row tile, 16-key block)
  int n_tt, n_kb;    // 32-row tiles and 16-key blocks per (b, h)
  float dq_scale;    // dQ = dq_scale * dS K
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int B, T, S, H, KVH;
  CapConsts cap;
  float query_scale;
  int window, is_local;
};

__device__ __forceinline__ int swz_rows(int r) { return (r >> 1) & 3; }

// Transpose-read lane offset inside an R-row tile for column block parity
// `par`: lane reads row 4*lq + l16/4 at dims 16*db + 4*(l16%4) (rows 16 and
// 32 further down share that row's swizzle).
__device__ __forceinline__ int tr_lane_off(int l16, int lq, int par) {
  const int r = 4 * lq + (l16 >> 2);
  return r * 64 + 16 * (((2 * par) + ((l16 & 3) >> 1)) ^ swz_rows(r)) + 8 * (l16 & 1);
}

// A-operand fragment of rows (tile rows 32*ks + 4*lq + j and + 16) x dims
// 16*db + l16, through two transpose reads.
template <int R>
__device__ __forceinline__ bf16x8 read_tr(const char* tile, int db, int ks, const int (&tr)[2]) {
  const char* p = tile + (db >> 1) * (R * 64) + (32 * ks) * 64 + tr[db & 1];
  const s16x4_b a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G2B_LDS_S16X4(p));
  const s16x4_b b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(G2B_LDS_S16X4(p + 16 * 64));
  const s16x8_b v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The two per-score factors of the backward for raw score x = <q, k>:
//   p = exp(s - lse) = 2^(s2 - l2), s2 the capped logit in log2 units;
//   g = the cap's derivative 1 - tanh^2 up to a constant, so that
//   dx = p (<dO, v> - D) * g * grad_scale<CAP>(qs).
// Fast form: s2 = C (1 - 2r) with r = 1/(1 + e^{2y}), so tanh = 1 - 2r and
// 1 - tanh^2 = 4 r (1 - r): g = r (1 - r) in one fma, and 4 qs is applied
// to the accumulated gradient.  row is C - l2 for the fast form, -l2 else.
template <int CAP>
__device__ __forceinline__ float2 score_terms(float x, float k_in, float c_out, float inv_cout, float row) {
  if constexpr (CAP == kCapFast) {
    const float r = rcp_fast(1.0f + exp2_fast(x * k_in));
    return float2{exp2_fast(__builtin_fmaf(r, -2.0f * c_out, row)), __builtin_fmaf(-r, r, r)};
  } else if constexpr (CAP == kCapAccurate) {
    const float s2 = capped_log2_accurate(x, k_in, c_out);
    const float t = s2 * inv_cout;
    return float2{exp2_fast(s2 + row), __builtin_fmaf(-t, t, 1.0f)};
  } else {
    return float2{exp2_fast(__builtin_fmaf(x, k_in, row)), 1.0f};
  }
}

template <int CAP>
__host__ __device__ inline float grad_scale(float qs) { return CAP == kCapFast ? 4.0f * qs : qs; }

template <int CAP>
__device__ __forceinline__ float row_term(float lse, float c_out) {
  constexpr float kLog2eF = 1.4426950408889634f;
  return CAP == kCapFast ? c_out - lse * kLog2eF : -lse * kLog2eF;
}

// ---------------------------------------------------------------- prep
// D[b, h, t] = <dO[b, t, h, :], out[b, t, h, :]>; a group of D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;
  const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;  // (b, t, h) flat
  const int sub = threadIdx.x % LPR;
  const long rows = (long)a.B * a.T * a.H;
  const bool live = row < rows;
  float s = 0.f;
  if (live) {
    const u32x4 go = *reinterpret_cast<const u32x4*>(a.dout + row * D + sub * 8);
    const u32x4 oo = *reinterpret_cast<const u32x4*>(a.out + row * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = __builtin_fmaf(bf16_lo_to_f32(go[e]), bf16_lo_to_f32(oo[e]), s);
      s = __builtin_fmaf(bf16_hi_to_f32(go[e]), bf16_hi_to_f32(oo[e]), s);
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) s += shfl_xor(s, m);
  if (live && sub == 0) {
    const int h = (int)(row % a.H);
    const int t = (int)((row / a.H) % a.T);
    const int b = (int)(row / ((long)a.H * a.T));
    a.dsum[((size_t)b * a.H + h) * a.T + t] = s;
  }
}

// ---------------------------------------------------------------- dK, dV
template <int D, int G, int CAP>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int QT = 32;               // query rows per tile
  constexpr int KB = 64;               // keys per workgroup
  constexpr int KK = D / 32;           // k-steps over d
  constexpr int DB = D / 16;           // 16-row blocks of dK^T, dV^T
  constexpr int TILE = QT * D * 2;     // bytes of a Q or dO tile
  constexpr int CPW = TILE / 1024 / 4; // wave-wide 1 KiB copies per wave and tile
  constexpr int RG = QT / 16;          // 16-row groups per tile
  static_assert(CPW >= 1, "tile copies split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char lds[2][2][TILE];  // [stage][Q | dO]
  __shared__ __attribute__((aligned(16))) float stat_lds[2][2 * QT];  // [stage][lse | D] of the tile's rows
  static_assert(2 * QT == 64, "one wave-wide 4-byte copy stages a tile's lse and D");
  static_assert(QT == kDsRows && KB / 4 == kDsKeys, "a wave's tile is one stored dS block");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const int T = a.T, S = a.S, H = a.H, KVH = a.KVH;
  const int nbg = a.B * KVH;
  const int kb_i = blockIdx.x / nbg;  // key block: the first ones are seen by the most rows
  const int bg = blockIdx.x % nbg;
  const int b = bg / KVH, g = bg % KVH;
  const int j0 = kb_i * KB;
  const int jw = j0 + 16 * wave;      // this wave's first key
  const int off = S - T;
  const int win = a.window;

  // stationary B operands: key jw + l16, dims 32*kk + 8*lq .. +7
  const size_t kv_row = (size_t)KVH * D;
  bf16x8 kfr[KK], vfr[KK];
  {
    const int j = jw + l16;
    const bf16* kr = a.k + ((size_t)b * S * KVH + g) * D + (size_t)(j < S ? j : 0) * kv_row + lq * 8;
    const bf16* vr = a.v + ((size_t)b * S * KVH + g) * D + (size_t)(j < S ? j : 0) * kv_row + lq * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 wk = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};
      if (j < S) {
        wk = *reinterpret_cast<const u32x4*>(kr + kk * 32);
        wv = *reinterpret_cast<const u32x4*>(vr + kk * 32);
      }
      kfr[kk] = __builtin_bit_cast(bf16x8, wk);
      vfr[kk] = __builtin_bit_cast(bf16x8, wv);
    }
  }
  f32x4 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // query rows that see any of the workgroup's keys, in QT-row tiles per
  // head (none: the keys' gradients are zero)
  const RowTiles rows = rows_seeing_keys(j0, KB, T, S, win, a.is_local, QT);
  const int t_lo = rows.t_lo;
  const int n_pos = rows.n_pos;
  const int n_tiles = G * n_pos;

  // tile copies (rows t of head h; lanes past T copy nothing)
  const unsigned q_row_bytes = (unsigned)H * D * 2u;
  const unsigned dma_rl = lane >> 2;
  const unsigned dma_lane = dma_rl * q_row_bytes + (((lane & 3) ^ swz_rows(dma_rl)) * 16u);
  auto issue = [&](char (*__restrict__ dst)[TILE], float* __restrict__ sdst, int i) __attribute__((always_inline)) {
    const int hh = i / n_pos;
    const int t0 = t_lo + (i % n_pos) * QT;
    const int h = g * G + hh;
    if (wave == 0) {  // the rows' lse (lanes 0..31) and D (lanes 32..63), clamped to row T-1
      const int tl = t0 + (lane & (QT - 1));
      const float* src = (lane < QT ? a.lse : a.dsum) + ((size_t)b * H + h) * T + (tl < T ? tl : T - 1);
      __builtin_amdgcn_global_load_lds(src, G2B_LDS(sdst), 4, 0, 0);
    }
    const char* qb = reinterpret_cast<const char*>(a.q + ((size_t)b * T * H + h) * D);
    const char* ob = reinterpret_cast<const char*>(a.dout + ((size_t)b * T * H + h) * D);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int n = wave + c * 4;
      const int cg = n / RG, r0 = 16 * (n % RG);
      const size_t uni = (size_t)(t0 + r0) * q_row_bytes + 64u * cg;
      const char* rq = qb + uni;
      const char* ro = ob + uni;
      unsigned lo = dma_lane;
      asm volatile("" : "+s"(rq));
      asm volatile("" : "+s"(ro));
      asm volatile("" : "+v"(lo));
      if (t0 + r0 + (int)dma_rl < T) {
        __builtin_amdgcn_global_load_lds(rq + lo, G2B_LDS(&dst[0][n * 1024]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(ro + lo, G2B_LDS(&dst[1][n * 1024]), 16, 0, 0);
      }
    }
  };

  const int k_lane = l16 * 64 + ((lq ^ swz_rows(l16)) << 4);
  const int tr[2] = {tr_lane_off(l16, lq, 0), tr_lane_off(l16, lq, 1)};
  const float k_in = a.cap.k_in, c_out = a.cap.c_out;
  const float inv_cout = c_out > 0.f ? 1.0f / c_out : 0.f;
  auto compute = [&](const char (*__restrict__ buf)[TILE], const float* __restrict__ sbuf, int i) __attribute__((always_inline)) {
    const int t0 = t_lo + (i % n_pos) * QT;
    const RowBand band = row_band(t0, min(t0 + QT - 1, T - 1), T, S, win, a.is_local);
    if (jw >= S || keys_unseen(band, jw, 16)) return;
    const bool need_mask = keys_need_mask(band, jw, 16, S, a.is_local) || (t0 + QT > T);
    const char* qt = buf[0];
    const char* ot = buf[1];
    // S = Q K^T and dP = dO V^T: rows = queries (A from the tile), cols = keys;
    // the tile fragments of k-step kk + 1 are read before the MFMAs of kk
    f32x4 sc[2], dp[2];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 qa[2][2], oa[2][2];  // [stage][16-row block]
    auto load_a = [&](int sg, int kk) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        qa[sg][qb] = *reinterpret_cast<const bf16x8*>(qt + kk * (QT * 64) + qb * 1024 + k_lane);
        oa[sg][qb] = *reinterpret_cast<const bf16x8*>(ot + kk * (QT * 64) + qb * 1024 + k_lane);
      }
    };
    load_a(0, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) load_a((kk + 1) & 1, kk + 1);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk & 1][qb], kfr[kk], kk == 0 ? zero4 : sc[qb], 0, 0, 0);
        dp[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[kk & 1][qb], vfr[kk], kk == 0 ? zero4 : dp[qb], 0, 0, 0);
      }
    }
    // P and dS for this lane's key column and its 8 query rows
    const int j = jw + l16;
    float pv[2][4], dsv[2][4];
    // the mask test is compiled only into the edge-tile copy of this loop
    auto scores = [&](auto mask_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // the 4 rows' log-sum-exp and D, staged in LDS with the tile
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sbuf + 16 * qb + 4 * lq);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sbuf + QT + 16 * qb + 4 * lq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 pg = score_terms<CAP>(sc[qb][e], k_in, c_out, inv_cout, row_term<CAP>(l4[e], c_out));
          float p = pg.x;
          float ds = p * (dp[qb][e] - d4[e]) * pg.y;
          if constexpr (decltype(mask_tag)::value) {
            const int t = t0 + 16 * qb + 4 * lq + e;
            const int p_ = t + off;
            const bool vis = (t < T) & (j < S) & (j <= p_) & ((j > p_ - win) | !a.is_local);
            p = vis ? p : 0.f;
            ds = vis ? ds : 0.f;
          }
          pv[qb][e] = p;
          dsv[qb][e] = ds;
        }
      }
    };
    if (need_mask) scores(std::true_type());
    else scores(std::false_type());
    u32x4 wp, wd;
    wp[0] = pack_bf16x2(pv[0][0], pv[0][1]);
    wp[1] = pack_bf16x2(pv[0][2], pv[0][3]);
    wp[2] = pack_bf16x2(pv[1][0], pv[1][1]);
    wp[3] = pack_bf16x2(pv[1][2], pv[1][3]);
    wd[0] = pack_bf16x2(dsv[0][0], dsv[0][1]);
    wd[1] = pack_bf16x2(dsv[0][2], dsv[0][3]);
    wd[2] = pack_bf16x2(dsv[1][0], dsv[1][1]);
    wd[3] = pack_bf16x2(dsv[1][2], dsv[1][3]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, wp);
    const bf16x8 sb = __builtin_bit_cast(bf16x8, wd);
    {  // dS^T of the block for the dQ kernel: key row l16, query columns 4*lq.. and 16 + 4*lq..
       // Non-temporal (the dQ kernel reads it, this kernel never does), and
       // issued here rather than sunk to the tile's end, a tile's dK/dV
       // MFMAs ahead of the wait that ends the tile.
      const int h = g * G + i / n_pos;
      char* blk = a.ds + ((((size_t)b * H + h) * a.n_tt + t0 / kDsRows) * a.n_kb + jw / kDsKeys) * 1024;
      __builtin_nontemporal_store(u32x2{wd[0], wd[1]}, reinterpret_cast<u32x2*>(blk + l16 * 64 + 8 * lq));
      __builtin_nontemporal_store(u32x2{wd[2], wd[3]}, reinterpret_cast<u32x2*>(blk + l16 * 64 + 32 + 8 * lq));
      asm volatile("" ::: "memory");
    }
    // dV^T += dO^T P, dK^T += Q^T dS (k = the tile's 32 query rows)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 oT = read_tr<QT>(ot, db, 0, tr);
      const bf16x8 qT = read_tr<QT>(qt, db, 0, tr);
      dv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oT, pb, dv[db], 0, 0, 0);
      dk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qT, sb, dk[db], 0, 0, 0);
    }
  };

  {
    u32x4* z = reinterpret_cast<u32x4*>(&lds[0][0][0]);
    for (int i = tid; i < (int)(sizeof(lds) / 16); i += 256) z[i] = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  auto step = [&](const char (*__restrict__ cur)[TILE], char (*__restrict__ nxt)[TILE], const float* __restrict__ scur,
                  float* __restrict__ snxt, int i) __attribute__((always_inline)) {
    if (i + 1 < n_tiles) issue(nxt, snxt, i + 1);
    compute(cur, scur, i);
  };
  if (n_tiles > 0) issue(lds[0], stat_lds[0], 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = 0; i < n_tiles; i += 2) {
    step(lds[0], lds[1], stat_lds[0], stat_lds[1], i);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (i + 1 < n_tiles) {
      step(lds[1], lds[0], stat_lds[1], stat_lds[0], i + 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // dK, dV rows: key jw + l16, dims 16*db + 4*lq .. +3
  const int j = jw + l16;
  const float gs = grad_scale<CAP>(a.query_scale);
  if (j < S) {
    bf16* kr = a.dk + (((size_t)b * S + j) * KVH + g) * D + 4 * lq;
    bf16* vr = a.dv + (((size_t)b * S + j) * KVH + g) * D + 4 * lq;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dk[db][0] * gs, dk[db][1] * gs);
      wk[1] = pack_bf16x2(dk[db][2] * gs, dk[db][3] * gs);
      wv[0] = pack_bf16x2(dv[db][0], dv[db][1]);
      wv[1] = pack_bf16x2(dv[db][2], dv[db][3]);
      *reinterpret_cast<u32x2*>(kr + db * 16) = wk;
      *reinterpret_cast<u32x2*>(vr + db * 16) = wv;
    }
  }
}

// ---------------------------------------------------------------- dQ
template <int D, int G>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = 32;                 // keys per tile
  constexpr int DW = D < 128 ? D : 128;  // dims per wave
  constexpr int ND = D / DW;             // waves per (head, 64 rows)
  constexpr int NQ = 4 / (G * ND);       // 64-row blocks per head
  constexpr int BMP = 64 * NQ;           // positions per workgroup
  constexpr int DBW = DW / 16;           // 16-dim blocks per wave
  constexpr int KTILE = BN * D * 2;      // bytes of a K tile
  constexpr int TPH = BMP / kDsRows;     // dS row tiles per head
  constexpr int DSB = G * TPH * 2;       // 1 KiB dS blocks per key tile
  constexpr int NK = KTILE / 1024;       // 1 KiB copies of K per key tile
  constexpr int NC = (NK + DSB) / 4;     // 1 KiB copies per wave and key tile
  static_assert(G * ND * NQ == 4 && NK % 4 == 0 && DSB % 4 == 0, "copies split evenly over the waves");
  static_assert(BN == 2 * kDsKeys, "a key tile holds two dS key blocks");
  __shared__ __attribute__((aligned(1024))) char lds[2][KTILE + DSB * 1024];  // [stage][K | dS blocks]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const int T = a.T, S = a.S, H = a.H, KVH = a.KVH;
  const int win = a.window, is_local = a.is_local;
  const int nbg = a.B * KVH;
  const int n_mb = (T + BMP - 1) / BMP;
  const int mb = n_mb - 1 - (int)(blockIdx.x / nbg);  // heaviest first
  const int bg = blockIdx.x % nbg;
  const int b = bg / KVH, g = bg % KVH;
  const int hh = wave / (ND * NQ);     // head of the K/V head's group
  const int qi = (wave / ND) % NQ;     // 64-row block of the workgroup
  const int dp = wave % ND;            // dims [DW * dp, DW * dp + DW)
  const int h = g * G + hh;
  const int m0 = mb * BMP;
  const int tw = m0 + 64 * qi;         // this wave's first row
  const int tt0 = m0 / kDsRows;        // the workgroup's first dS row tile

  const RowBand wg_band = row_band(m0, min(m0 + BMP, T) - 1, T, S, win, is_local);
  const KeyTiles wg_tiles = key_tiles(wg_band, BN);
  const int n_start = wg_tiles.n_start;
  const int n_tiles = wg_tiles.n_tiles;
  const bool wave_active = tw < T;
  const RowBand w_band = row_band(tw, min(tw + 63, T - 1), T, S, win, is_local);

  // copies: K rows past S and dS blocks no row sees are not copied (the
  // fragments of such blocks are zeroed in compute)
  const unsigned kv_row_bytes = (unsigned)KVH * D * 2u;
  const char* kbase = reinterpret_cast<const char*>(a.k + ((size_t)b * S * KVH + g) * D);
  const size_t head_blocks = (size_t)a.n_tt * a.n_kb;
  const char* dsbase = a.ds + ((size_t)b * H + (size_t)g * G) * head_blocks * 1024;
  const unsigned dma_rl = lane >> 2;
  const unsigned k_src = dma_rl * kv_row_bytes + (((lane & 3) ^ swz_rows(dma_rl)) * 16u);
  const unsigned ds_src = dma_rl * 64u + (((lane & 3) ^ swz_rows(dma_rl)) * 16u);
  auto issue = [&](char* __restrict__ dst, int n0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int n = wave + 4 * c;
      if (4 * c < NK) {  // K rows n0 + 16 * (n % 2) .., dims 32 * (n / 2) ..
        const int r0 = 16 * (n & 1);
        const char* rk = kbase + (size_t)(n0 + r0) * kv_row_bytes + 64u * (n >> 1);
        unsigned lo = k_src;
        asm volatile("" : "+s"(rk));
        asm volatile("" : "+v"(lo));
        if (n0 + r0 + (int)dma_rl < S)
          __builtin_amdgcn_global_load_lds(rk + lo, G2B_LDS(dst + n * 1024), 16, 0, 0);
      } else {  // dS block (head hx, row tile tt0 + tl, key block n0/16 + kl)
        const int m = n - NK;
        const int hx = m / (2 * TPH), tl = (m >> 1) % TPH, kl = m & 1;
        const int tt = tt0 + tl, kb = n0 / kDsKeys + kl;
        if (ds_block_seen(tt, kb, T, S, win, is_local)) {
          const char* rd = dsbase + (((size_t)hx * a.n_tt + tt) * a.n_kb + kb) * 1024;
          unsigned lo = ds_src;
          asm volatile("" : "+s"(rd));
          asm volatile("" : "+v"(lo));
          __builtin_amdgcn_global_load_lds(rd + lo, G2B_LDS(dst + n * 1024), 16, 0, 0);
        }
      }
    }
  };

  const int tr[2] = {tr_lane_off(l16, lq, 0), tr_lane_off(l16, lq, 1)};
  f32x4 acc[DBW][4];
#pragma unroll
  for (int i = 0; i < DBW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const char* __restrict__ buf, int n0) __attribute__((always_inline)) {
    if (!wave_active || keys_unseen(w_band, n0, BN)) return;
    // B = dS^T of the wave's 16-row blocks r: rows = the tile's keys; the
    // halves of a fragment (keys 4*lq.. and 16 + 4*lq..) come from the two
    // key blocks and are zero where no row of the block's row tile sees them
    const char* dst = buf + KTILE + (hh * TPH + 2 * qi) * 2048;
    bf16x8 bq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = tt0 + 2 * qi + (r >> 1);
      u32x4 w = __builtin_bit_cast(u32x4, read_tr<32>(dst + (r >> 1) * 2048, r & 1, 0, tr));
      if (!ds_block_seen(tt, n0 / kDsKeys, T, S, win, is_local)) w[0] = w[1] = 0u;
      if (!ds_block_seen(tt, n0 / kDsKeys + 1, T, S, win, is_local)) w[2] = w[3] = 0u;
      bq[r] = __builtin_bit_cast(bf16x8, w);
    }
    // dQ^T += K^T dS^T (k = the tile's 32 keys)
#pragma unroll
    for (int i = 0; i < DBW; ++i) {
      const bf16x8 kT = read_tr<BN>(buf, dp * DBW + i, 0, tr);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kT, bq[r], acc[i][r], 0, 0, 0);
    }
  };

  {
    u32x4* z = reinterpret_cast<u32x4*>(&lds[0][0]);
    for (int i = tid; i < (int)(sizeof(lds) / 16); i += 256) z[i] = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  issue(lds[0], n_start);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; it += 2) {
    const int n0 = n_start + it * BN;
    if (it + 1 < n_tiles) issue(lds[1], n0 + BN);
    compute(lds[0], n0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < n_tiles) {
      if (it + 2 < n_tiles) issue(lds[0], n0 + 2 * BN);
      compute(lds[1], n0 + BN);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  if (!wave_active) return;
  const float gs = a.dq_scale;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = tw + 16 * r + l16;
    if (t >= T) continue;
    bf16* qr = a.dq + (((size_t)b * T + t) * H + h) * D + DW * dp + 4 * lq;
#pragma unroll
    for (int i = 0; i < DBW; ++i) {
      u32x2 w2;
      w2[0] = pack_bf16x2(acc[i][r][0] * gs, acc[i][r][1] * gs);
      w2[1] = pack_bf16x2(acc[i][r][2] * gs, acc[i][r][3] * gs);
      *reinterpret_cast<u32x2*>(qr + i * 16) = w2;
    }
  }
}

template <int D, int G, int CAP>
static hipError_t launch_bwd_t(BwdArgs a, hipStream_t stream) {
  a.dq_scale = grad_scale<CAP>(a.query_scale);
  const long rows = (long)a.B * a.T * a.H;
  const unsigned gp = (unsigned)((rows * (D / 8) + 255) / 256);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(gp), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nbg = (unsigned)(a.B * a.KVH);
  const unsigned gk = (unsigned)((a.S + 63) / 64) * nbg;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, G, CAP>), dim3(gk), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int ND = D > 128 ? D / 128 : 1;
  constexpr int BMP = 64 * (4 / (G * ND));  // the dQ kernel's positions per workgroup
  const unsigned gq = (unsigned)((a.T + BMP - 1) / BMP) * nbg;
  hipLaunchKernelGGL((bwd_dq_kernel<D, G>), dim3(gq), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_bwd_dg(const BwdArgs& a, hipStream_t stream) {
  switch (a.cap.mode) {
    case kCapFast: return launch_bwd_t<D, G, kCapFast>(a, stream);
    case kCapAccurate: return launch_bwd_t<D, G, kCapAccurate>(a, stream);
    default: return launch_bwd_t<D, G, kCapNone>(a, stream);
  }
}

hipError_t launch_prefill_backward(const BackwardLaunch& L, hipStream_t stream) {
  BwdArgs a;
  a.q = static_cast<const bf16*>(L.q);
  a.k = static_cast<const bf16*>(L.k);
  a.v = static_cast<const bf16*>(L.v);
  a.out = static_cast<const bf16*>(L.out);
  a.dout = static_cast<const bf16*>(L.dout);
  a.lse = L.lse;
  a.dsum = static_cast<float*>(L.workspace);
  a.ds = static_cast<char*>(L.workspace) + backward_ds_offset(L.B, L.T, L.H);
  a.n_tt = (L.T + kDsRows - 1) / kDsRows;
  a.n_kb = (L.S + kDsKeys - 1) / kDsKeys;
  a.dq = static_cast<bf16*>(L.dq);
  a.dk = static_cast<bf16*>(L.dk);
  a.dv = static_cast<bf16*>(L.dv);
  a.B = L.B;
  a.T = L.T;
  a.S = L.S;
  a.H = L.H;
  a.KVH = L.KVH;
  a.cap = make_cap_consts(L.query_scale, L.softcap);
  a.query_scale = L.query_scale;
  a.window = L.window;
  a.is_local = L.is_local;
  const int G = L.H / L.KVH;
  switch (L.d) {
    case 64: return G == 2 ? launch_bwd_dg<64, 2>(a, stream) : launch_bwd_dg<64, 1>(a, stream);
    case 128: return G == 2 ? launch_bwd_dg<128, 2>(a, stream) : launch_bwd_dg<128, 1>(a, stream);
    case 256: return G == 2 ? launch_bwd_dg<256, 2>(a, stream) : launch_bwd_dg<256, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace g2
