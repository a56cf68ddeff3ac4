/*
 * CPU fp64 oracle for the Gemma 2 attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file, and everything under oracle/, is the
 * slow and obviously-correct definition that the GPU kernels are checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it.  It shares no code, header, table or helper with the HIP
 * library, and it includes nothing from it.
 *
 * What it computes (Gemma 2 model card, wikillm "Gemma 2: Improving Open
 * Language Models at a Practical Size", section "Method", the one-layer
 * attention pseudocode; cross-checked with the aifetchly "Gemma 2 Guide",
 * section 1 "Logit Soft-Capping" formula and its PyTorch layer):
 *
 *   queries are multiplied by query_scale;
 *   each group of H/KVH consecutive query heads shares one key/value head
 *     (head h reads K/V head g = h / (H/KVH));
 *   logits x_j = <scaled q, k_j> for every key j;
 *   logits are soft-capped, s_j = cap * tanh(x_j / cap), BEFORE masking
 *     (card, "Paper vs code": the cap acts on the raw scores, then the mask);
 *   a causal mask keeps key j for query position p iff j <= p; on a local
 *     layer the key must also satisfy j > p - window (card "Paper vs code",
 *     sliding-window bounds; the Guide's layer builds the same set of W keys
 *     with a lower-triangular -inf band at offset -W);
 *   masked logits become -inf, a softmax over keys gives the weights, and the
 *     output is the weighted sum of the value rows of head g.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - query row t of a (T, S) call sits at absolute position p = t + S - T
 *     (causal mask aligned bottom-right, so decode is the last prefill row);
 *   - cap <= 0 or cap = +inf means "no soft-cap" (the identity), the limit of
 *     cap * tanh(x / cap) as cap grows;
 *   - decode reads key position j from cache slot j mod S, which makes a
 *     local-layer cache of S = window slots a ring.
 *
 * Arithmetic: inputs arrive as float32 (bf16 values are exact in float32);
 * every step runs in double with libm tanh/exp.  Each output row is computed
 * with two plain passes over its keys: logits, cap and max first; then the
 * exponentials, their sum and the weighted value sum.  No tiling, no online
 * softmax, no reordering beyond that.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define G2O_OK 0
#define G2O_ERR_ARG (-1)

/* sha256 of this source and its compiler flags, set by oracle/build.py. */
#ifndef G2O_BUILD_ID
#define G2O_BUILD_ID "unknown"
#endif
const char g2o_build_id_record[] = "g2oracle-build-id:" G2O_BUILD_ID;

/* Soft-cap of one logit: cap * tanh(x / cap); the identity when the cap is
 * disabled (cap <= 0 or infinite).  Guide section 1, first formula. */
double g2o_softcap(double x, double cap) {
  if (!(cap > 0.0) || isinf(cap)) return x;
  return cap * tanh(x / cap);
}

/* Mask predicate: may query position p see key position j?
 * Causal for every layer; local layers also require j > p - window. */
int g2o_allowed(int64_t p, int64_t j, int window, int is_local) {
  if (j < 0 || j > p) return 0;
  if (is_local && !(j > p - (int64_t)window)) return 0;
  return 1;
}

static int check_shapes(int B, int T, int S, int H, int KVH, int d, int window,
                        int is_local) {
  if (B <= 0 || T <= 0 || S <= 0 || H <= 0 || KVH <= 0 || d <= 0) return 0;
  if (H % KVH != 0) return 0;
  if (T > S) return 0;
  if (is_local && window < 1) return 0;
  return 1;
}

/* Capped logits of one query row against key rows k_rows[0..n-1] (each d
 * floats, already the rows of the shared K/V head), with the mask given as a
 * list of allowed flags.  s[j] = -inf where the key is masked. */
static void row_logits(const float* qrow, const float* const* k_rows,
                       const unsigned char* allowed, int64_t n, int d,
                       double query_scale, double cap, double* s) {
  double* qs = (double*)malloc(sizeof(double) * (size_t)d);
  for (int e = 0; e < d; ++e) qs[e] = (double)qrow[e] * query_scale;
  for (int64_t j = 0; j < n; ++j) {
    if (!allowed[j]) {
      s[j] = -INFINITY;
      continue;
    }
    const float* kr = k_rows[j];
    double x = 0.0;
    for (int e = 0; e < d; ++e) x += qs[e] * (double)kr[e];
    s[j] = g2o_softcap(x, cap);
  }
  free(qs);
}

/* Softmax over the logits of one row (masked entries are -inf and get 0). */
static void row_softmax(const double* s, int64_t n, double* w) {
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j)
    if (s[j] > m) m = s[j];
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    w[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
    z += w[j];
  }
  for (int64_t j = 0; j < n; ++j) w[j] /= z;
}

/* Gather, for prefill row (b, t, h), the key rows and allowed flags. */
static void prefill_row_setup(const float* k, int T, int S, int H, int KVH,
                              int d, int window, int is_local, int b, int t,
                              int h, const float** k_rows,
                              unsigned char* allowed) {
  const int group = H / KVH;
  const int g = h / group;
  const int64_t p = (int64_t)t + S - T;
  for (int64_t j = 0; j < S; ++j) {
    k_rows[j] = k + (((int64_t)b * S + j) * KVH + g) * d;
    allowed[j] = (unsigned char)g2o_allowed(p, j, window, is_local);
  }
}

/* One output row: weights then weighted sum of value rows. */
static void row_output(const float* const* v_rows, const double* w, int64_t n,
                       int d, double* out) {
  for (int e = 0; e < d; ++e) out[e] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    if (w[j] == 0.0) continue;
    const float* vr = v_rows[j];
    for (int e = 0; e < d; ++e) out[e] += w[j] * (double)vr[e];
  }
}

/* Capped, masked logits s[0..S-1] of prefill row (b, t, h).
 * q: (B,T,H,d), k: (B,S,KVH,d), row-major float32. */
int g2o_prefill_row_logits(const float* q, const float* k, int B, int T, int S,
                           int H, int KVH, int d, double query_scale,
                           double softcap, int window, int is_local, int b,
                           int t, int h, double* s) {
  if (!check_shapes(B, T, S, H, KVH, d, window, is_local)) return G2O_ERR_ARG;
  if (b < 0 || b >= B || t < 0 || t >= T || h < 0 || h >= H) return G2O_ERR_ARG;
  const float** k_rows = (const float**)malloc(sizeof(float*) * (size_t)S);
  unsigned char* allowed = (unsigned char*)malloc((size_t)S);
  prefill_row_setup(k, T, S, H, KVH, d, window, is_local, b, t, h, k_rows,
                    allowed);
  const float* qrow = q + (((int64_t)b * T + t) * H + h) * d;
  row_logits(qrow, k_rows, allowed, S, d, query_scale, softcap, s);
  free(k_rows);
  free(allowed);
  return G2O_OK;
}

/* Attention weights w[0..S-1] of prefill row (b, t, h). */
int g2o_prefill_row_weights(const float* q, const float* k, int B, int T,
                            int S, int H, int KVH, int d, double query_scale,
                            double softcap, int window, int is_local, int b,
                            int t, int h, double* w) {
  double* s = (double*)malloc(sizeof(double) * (size_t)S);
  int st = g2o_prefill_row_logits(q, k, B, T, S, H, KVH, d, query_scale,
                                  softcap, window, is_local, b, t, h, s);
  if (st == G2O_OK) row_softmax(s, S, w);
  free(s);
  return st;
}

/* Prefill.  q,out: (B,T,H,d); k,v: (B,S,KVH,d).
 * rows == NULL: every row, out is (B,T,H,d) in double.
 * rows != NULL: nrows flat row ids r = (b*T + t)*H + h, out is (nrows, d). */
int g2o_prefill(const float* q, const float* k, const float* v, double* out,
                int B, int T, int S, int H, int KVH, int d, double query_scale,
                double softcap, int window, int is_local, const int64_t* rows,
                int64_t nrows) {
  if (!check_shapes(B, T, S, H, KVH, d, window, is_local)) return G2O_ERR_ARG;
  const int64_t total = (int64_t)B * T * H;
  const int64_t n = rows ? nrows : total;
  if (rows) {
    for (int64_t i = 0; i < n; ++i)
      if (rows[i] < 0 || rows[i] >= total) return G2O_ERR_ARG;
  }
#pragma omp parallel
  {
    const float** k_rows = (const float**)malloc(sizeof(float*) * (size_t)S);
    const float** v_rows = (const float**)malloc(sizeof(float*) * (size_t)S);
    unsigned char* allowed = (unsigned char*)malloc((size_t)S);
    double* s = (double*)malloc(sizeof(double) * (size_t)S);
    double* w = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
      const int64_t r = rows ? rows[i] : i;
      const int h = (int)(r % H);
      const int t = (int)((r / H) % T);
      const int b = (int)(r / ((int64_t)H * T));
      prefill_row_setup(k, T, S, H, KVH, d, window, is_local, b, t, h, k_rows,
                        allowed);
      const int g = h / (H / KVH);
      for (int64_t j = 0; j < S; ++j)
        v_rows[j] = v + (((int64_t)b * S + j) * KVH + g) * d;
      const float* qrow = q + r * d;
      row_logits(qrow, k_rows, allowed, S, d, query_scale, softcap, s);
      row_softmax(s, S, w);
      row_output(v_rows, w, S, d, out + i * d);
    }
    free(k_rows);
    free(v_rows);
    free(allowed);
    free(s);
    free(w);
  }
  return G2O_OK;
}

/* Log-sum-exp of the capped, masked logits of prefill rows (natural log):
 * lse = log sum_j exp(s_j) over the keys row (b, t, h) sees.  It is what a
 * backward pass saves from the forward (Gemma 2 Guide, "Deep Dive" item 1
 * differentiates the cap; the softmax weights are exp(s_j - lse)).
 * rows == NULL: every row, lse is (B,T,H); else rows r = (b*T + t)*H + h. */
int g2o_prefill_lse(const float* q, const float* k, double* lse, int B, int T,
                    int S, int H, int KVH, int d, double query_scale,
                    double softcap, int window, int is_local,
                    const int64_t* rows, int64_t nrows) {
  if (!check_shapes(B, T, S, H, KVH, d, window, is_local)) return G2O_ERR_ARG;
  const int64_t total = (int64_t)B * T * H;
  const int64_t n = rows ? nrows : total;
  if (rows) {
    for (int64_t i = 0; i < n; ++i)
      if (rows[i] < 0 || rows[i] >= total) return G2O_ERR_ARG;
  }
#pragma omp parallel
  {
    const float** k_rows = (const float**)malloc(sizeof(float*) * (size_t)S);
    unsigned char* allowed = (unsigned char*)malloc((size_t)S);
    double* s = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
      const int64_t r = rows ? rows[i] : i;
      const int h = (int)(r % H);
      const int t = (int)((r / H) % T);
      const int b = (int)(r / ((int64_t)H * T));
      prefill_row_setup(k, T, S, H, KVH, d, window, is_local, b, t, h, k_rows,
                        allowed);
      row_logits(q + r * d, k_rows, allowed, S, d, query_scale, softcap, s);
      double m = -INFINITY;
      for (int64_t j = 0; j < S; ++j)
        if (s[j] > m) m = s[j];
      double z = 0.0;
      for (int64_t j = 0; j < S; ++j)
        if (s[j] != -INFINITY) z += exp(s[j] - m);
      lse[i] = m + log(z);
    }
    free(k_rows);
    free(allowed);
    free(s);
  }
  return G2O_OK;
}

/* Decode of one new token per sequence against a KV cache.
 * q,out: (B,1,H,d); k_cache, v_cache: (B,S,KVH,d); kv_lens[b] = L_b >= 1 is
 * the number of tokens the sequence holds, the newest one (already written)
 * at position L_b - 1.  Key position j lives in slot j mod S.  The query sits
 * at position p = L_b - 1 and sees the keys the prefill mask allows.  The
 * positions it sees must occupy distinct slots: L_b <= S for a global layer,
 * min(L_b, window) <= S for a local one.
 * rows == NULL: every (b, h), out is (B,1,H,d); else rows r = b*H + h. */
int g2o_decode(const float* q, const float* k_cache, const float* v_cache,
               const int32_t* kv_lens, double* out, int B, int S, int H,
               int KVH, int d, double query_scale, double softcap, int window,
               int is_local, const int64_t* rows, int64_t nrows) {
  if (!check_shapes(B, 1, S, H, KVH, d, window, is_local)) return G2O_ERR_ARG;
  for (int b = 0; b < B; ++b) {
    const int64_t L = kv_lens[b];
    if (L < 1) return G2O_ERR_ARG;
    const int64_t seen = is_local ? (L < window ? L : window) : L;
    if (seen > S) return G2O_ERR_ARG;
  }
  const int64_t total = (int64_t)B * H;
  const int64_t n = rows ? nrows : total;
  if (rows) {
    for (int64_t i = 0; i < n; ++i)
      if (rows[i] < 0 || rows[i] >= total) return G2O_ERR_ARG;
  }
  int64_t maxL = 0;
  for (int b = 0; b < B; ++b)
    if (kv_lens[b] > maxL) maxL = kv_lens[b];
#pragma omp parallel
  {
    const float** k_rows = (const float**)malloc(sizeof(float*) * (size_t)maxL);
    const float** v_rows = (const float**)malloc(sizeof(float*) * (size_t)maxL);
    unsigned char* allowed = (unsigned char*)malloc((size_t)maxL);
    double* s = (double*)malloc(sizeof(double) * (size_t)maxL);
    double* w = (double*)malloc(sizeof(double) * (size_t)maxL);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
      const int64_t r = rows ? rows[i] : i;
      const int h = (int)(r % H);
      const int b = (int)(r / H);
      const int g = h / (H / KVH);
      const int64_t L = kv_lens[b];
      const int64_t p = L - 1;
      for (int64_t j = 0; j < L; ++j) {
        const int64_t slot = j % S;
        k_rows[j] = k_cache + (((int64_t)b * S + slot) * KVH + g) * d;
        v_rows[j] = v_cache + (((int64_t)b * S + slot) * KVH + g) * d;
        allowed[j] = (unsigned char)g2o_allowed(p, j, window, is_local);
      }
      const float* qrow = q + r * d;
      row_logits(qrow, k_rows, allowed, L, d, query_scale, softcap, s);
      row_softmax(s, L, w);
      row_output(v_rows, w, L, d, out + i * d);
    }
    free(k_rows);
    free(v_rows);
    free(allowed);
    free(s);
    free(w);
  }
  return G2O_OK;
}

/* Decode against a paged KV cache (Gemma 2 Guide, "Deep Dive" item 2: KV
 * memory managed in discrete blocks; local layers drop blocks older than the
 * window).  k_pool, v_pool: (num_blocks, block_size, KVH, d); block_table:
 * (B, max_blocks) int32, entry [b][i] = physical block holding positions
 * i*block_size .. (i+1)*block_size - 1 of sequence b.  The query of sequence
 * b sits at position L_b - 1 and sees the keys the prefill mask allows; only
 * those positions are looked up, so table entries of other blocks (evicted or
 * unused) are never read.  1 <= L_b <= max_blocks * block_size.  A needed
 * entry outside [0, num_blocks) makes that row's output NaN.
 * rows == NULL: every (b, h), out is (B,1,H,d); else rows r = b*H + h. */
int g2o_decode_paged(const float* q, const float* k_pool, const float* v_pool,
                     const int32_t* block_table, int max_blocks,
                     const int32_t* kv_lens, double* out, int B, int H, int KVH,
                     int d, int block_size, int num_blocks, double query_scale,
                     double softcap, int window, int is_local,
                     const int64_t* rows, int64_t nrows) {
  if (B <= 0 || H <= 0 || KVH <= 0 || d <= 0 || H % KVH != 0) return G2O_ERR_ARG;
  if (block_size <= 0 || max_blocks <= 0 || num_blocks <= 0) return G2O_ERR_ARG;
  if (is_local && window < 1) return G2O_ERR_ARG;
  const int64_t cap_len = (int64_t)max_blocks * block_size;
  int64_t maxL = 0;
  for (int b = 0; b < B; ++b) {
    if (kv_lens[b] < 1 || kv_lens[b] > cap_len) return G2O_ERR_ARG;
    if (kv_lens[b] > maxL) maxL = kv_lens[b];
  }
  const int64_t total = (int64_t)B * H;
  const int64_t n = rows ? nrows : total;
  if (rows) {
    for (int64_t i = 0; i < n; ++i)
      if (rows[i] < 0 || rows[i] >= total) return G2O_ERR_ARG;
  }
#pragma omp parallel
  {
    const float** k_rows = (const float**)malloc(sizeof(float*) * (size_t)maxL);
    const float** v_rows = (const float**)malloc(sizeof(float*) * (size_t)maxL);
    unsigned char* allowed = (unsigned char*)malloc((size_t)maxL);
    double* s = (double*)malloc(sizeof(double) * (size_t)maxL);
    double* w = (double*)malloc(sizeof(double) * (size_t)maxL);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
      const int64_t r = rows ? rows[i] : i;
      const int h = (int)(r % H);
      const int b = (int)(r / H);
      const int g = h / (H / KVH);
      const int64_t L = kv_lens[b];
      const int64_t p = L - 1;
      int bad = 0;
      for (int64_t j = 0; j < L; ++j) {
        allowed[j] = (unsigned char)g2o_allowed(p, j, window, is_local);
        k_rows[j] = v_rows[j] = NULL;
        if (!allowed[j]) continue;
        const int64_t blk = block_table[(int64_t)b * max_blocks + j / block_size];
        if (blk < 0 || blk >= num_blocks) {
          bad = 1;
          break;
        }
        const int64_t row = (blk * block_size + j % block_size) * KVH + g;
        k_rows[j] = k_pool + row * d;
        v_rows[j] = v_pool + row * d;
      }
      if (bad) {
        for (int e = 0; e < d; ++e) out[i * d + e] = NAN;
        continue;
      }
      const float* qrow = q + r * d;
      row_logits(qrow, k_rows, allowed, L, d, query_scale, softcap, s);
      row_softmax(s, L, w);
      row_output(v_rows, w, L, d, out + i * d);
    }
    free(k_rows);
    free(v_rows);
    free(allowed);
    free(s);
    free(w);
  }
  return G2O_OK;
}

/* Backward pass of the prefill (Gemma 2 Guide, "Deep Dive" item 1: the cap's
 * derivative is 1 - tanh^2(x / cap)).  With y_j = x_j / cap, s_j = cap tanh y_j
 * and the softmax weights w_j of a row, for an upstream gradient dO of the
 * output row:
 *   dv_j += w_j dO,   D = <dO, out>,   ds_j = w_j (<dO, v_j> - D),
 *   dx_j = ds_j (1 - tanh^2 y_j)   (dx_j = ds_j when the cap is disabled),
 *   dq   = query_scale * sum_j dx_j k_j,   dk_j += query_scale * dx_j q.
 * q, dout, dq: (B,T,H,d); k, v, dk, dv: (B,S,KVH,d).  dk and dv sum over the
 * query heads of a group and over every row that sees the key.  The rows of one
 * (batch, K/V head) group run in order, so every sum has a fixed order. */
int g2o_prefill_backward(const float* q, const float* k, const float* v,
                         const float* dout, double* dq, double* dk, double* dv,
                         int B, int T, int S, int H, int KVH, int d,
                         double query_scale, double softcap, int window,
                         int is_local) {
  if (!check_shapes(B, T, S, H, KVH, d, window, is_local)) return G2O_ERR_ARG;
  const int G = H / KVH;
  const int use_cap = (softcap > 0.0) && !isinf(softcap);
  memset(dk, 0, sizeof(double) * (size_t)B * S * KVH * d);
  memset(dv, 0, sizeof(double) * (size_t)B * S * KVH * d);
#pragma omp parallel
  {
    const float** k_rows = (const float**)malloc(sizeof(float*) * (size_t)S);
    const float** v_rows = (const float**)malloc(sizeof(float*) * (size_t)S);
    unsigned char* allowed = (unsigned char*)malloc((size_t)S);
    double* sc = (double*)malloc(sizeof(double) * (size_t)S);
    double* w = (double*)malloc(sizeof(double) * (size_t)S);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < (int64_t)B * KVH; ++bg) {
      const int b = (int)(bg / KVH), g = (int)(bg % KVH);
      for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        for (int t = 0; t < T; ++t) {
          prefill_row_setup(k, T, S, H, KVH, d, window, is_local, b, t, h, k_rows,
                            allowed);
          for (int64_t j = 0; j < S; ++j)
            v_rows[j] = v + (((int64_t)b * S + j) * KVH + g) * d;
          const int64_t r = ((int64_t)b * T + t) * H + h;
          const float* qrow = q + r * d;
          const float* gout = dout + r * d;
          row_logits(qrow, k_rows, allowed, S, d, query_scale, softcap, sc);
          row_softmax(sc, S, w);
          row_output(v_rows, w, S, d, o);
          double D = 0.0;
          for (int e = 0; e < d; ++e) D += (double)gout[e] * o[e];
          double* dqr = dq + r * d;
          for (int e = 0; e < d; ++e) dqr[e] = 0.0;
          for (int64_t j = 0; j < S; ++j) {
            if (w[j] == 0.0) continue;
            const float* vr = v_rows[j];
            const float* kr = k_rows[j];
            double dw = 0.0;
            for (int e = 0; e < d; ++e) dw += (double)gout[e] * (double)vr[e];
            const double ds = w[j] * (dw - D);
            const double th = use_cap ? sc[j] / softcap : 0.0;
            const double dx = use_cap ? ds * (1.0 - th * th) : ds;
            double* dkr = dk + (((int64_t)b * S + j) * KVH + g) * d;
            double* dvr = dv + (((int64_t)b * S + j) * KVH + g) * d;
            for (int e = 0; e < d; ++e) {
              dqr[e] += query_scale * dx * (double)kr[e];
              dkr[e] += query_scale * dx * (double)qrow[e];
              dvr[e] += w[j] * (double)gout[e];
            }
          }
        }
      }
    }
    free(k_rows);
    free(v_rows);
    free(allowed);
    free(sc);
    free(w);
    free(o);
  }
  return G2O_OK;
}

/* Rotary position embedding (wikillm model card, "Method" item 5: rotary
 * embeddings carried over from Gemma 1; the pages give no formula).  Reading:
 * the rotary embedding of Su et al. with pair i of a head vector formed by
 * elements i and i + d/2 (i < d/2), rotated by the angle
 * pos * base^(-2i/d):  (a, b) -> (a cos - b sin, b cos + a sin).
 * x, out: (B, T, NH, d); positions: (B, T) int32.  d must be even. */
int g2o_rope(const float* x, const int32_t* positions, double* out, int B,
             int T, int NH, int d, double base) {
  if (B <= 0 || T <= 0 || NH <= 0 || d <= 0 || (d & 1) || !(base > 1.0))
    return G2O_ERR_ARG;
  const int half = d / 2;
  const int64_t rows = (int64_t)B * T;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double pos = (double)positions[r];
    for (int i = 0; i < half; ++i) {
      const double theta = pos * pow(base, -2.0 * i / d);
      const double c = cos(theta), sn = sin(theta);
      for (int h = 0; h < NH; ++h) {
        const int64_t o = (r * NH + h) * d;
        const double a = x[o + i], b = x[o + i + half];
        out[o + i] = a * c - b * sn;
        out[o + i + half] = b * c + a * sn;
      }
    }
  }
  return G2O_OK;
}

/* Final-logit soft-cap over an array (Guide section 1, second formula: the
 * vocabulary logits are capped at 30 with the same tanh form). */
void g2o_softcap_array(const float* x, double* out, int64_t n, double cap) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = g2o_softcap((double)x[i], cap);
}

/* Number of threads the parallel loops above use (OpenMP's default team). */
#ifdef _OPENMP
#include <omp.h>
#endif
int g2o_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
