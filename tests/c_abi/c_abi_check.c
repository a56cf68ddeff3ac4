/*
 * The C ABI used from plain C, with no Python or PyTorch in the process:
 * device buffers from the HIP runtime, every compute entry point of the
 * library on them (prefill, prefill with log-sum-exp, backward, decode, paged
 * decode, rotary embedding, final cap), results checked against the CPU fp64
 * oracle (test infrastructure, linked only into this checker), and the
 * documented error statuses.
 *
 * Inputs are seeded normal draws rounded to bf16; the oracle reads the same
 * values widened to float.  Tolerances: attention outputs max |diff| <= 2e-2,
 * mean <= 2e-3; lse 2e-3; gradients 2e-2 of the largest and 1e-2 of the mean
 * magnitude; fp32 rotary embedding 2e-5; the bf16 final cap one bf16 ulp.
 * Prints "c_abi_check ok" and exits 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "g2attn.h"

/* the oracle's entry points (oracle/g2_oracle.c) */
int g2o_prefill(const float* q, const float* k, const float* v, double* out, int B, int T,
                int S, int H, int KVH, int d, double query_scale, double softcap, int window,
                int is_local, const int64_t* rows, int64_t nrows);
int g2o_decode(const float* q, const float* k_cache, const float* v_cache,
               const int32_t* kv_lens, double* out, int B, int S, int H, int KVH, int d,
               double query_scale, double softcap, int window, int is_local,
               const int64_t* rows, int64_t nrows);

int g2o_prefill_lse(const float* q, const float* k, double* lse, int B, int T, int S, int H,
                    int KVH, int d, double query_scale, double softcap, int window, int is_local,
                    const int64_t* rows, int64_t nrows);
int g2o_prefill_backward(const float* q, const float* k, const float* v, const float* dout,
                         double* dq, double* dk, double* dv, int B, int T, int S, int H, int KVH,
                         int d, double query_scale, double softcap, int window, int is_local);
int g2o_decode_paged(const float* q, const float* k_pool, const float* v_pool,
                     const int32_t* block_table, int max_blocks, const int32_t* kv_lens,
                     double* out, int B, int H, int KVH, int d, int block_size, int num_blocks,
                     double query_scale, double softcap, int window, int is_local,
                     const int64_t* rows, int64_t nrows);
int g2o_rope(const float* x, const int32_t* positions, double* out, int B, int T, int NH, int d,
             double base);
void g2o_softcap_array(const float* x, double* out, int64_t n, double cap);

static int failures = 0;
#define EXPECT(cond, ...)                      \
  do {                                         \
    if (!(cond)) {                             \
      printf("FAIL: " __VA_ARGS__);            \
      printf("\n");                            \
      ++failures;                              \
    }                                          \
  } while (0)
#define HIP_OK(x)                                                                   \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);        \
      exit(2);                                                                      \
    }                                                                               \
  } while (0)

/* splitmix64 and Box-Muller: seeded normal draws */
static uint64_t rng_state;
static uint64_t splitmix64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double uniform01(void) { return ((splitmix64() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
static double normal(void) {
  const double u = uniform01(), w = uniform01();
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * w);
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* n seeded draws times mul, as bf16 bits and as the floats they hold */
static void draw(size_t n, uint64_t seed, double mul, uint16_t* bits, float* vals) {
  rng_state = seed;
  for (size_t i = 0; i < n; ++i) {
    bits[i] = to_bf16((float)(normal() * mul));
    vals[i] = from_bf16(bits[i]);
  }
}

static void* to_device(const void* host, size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes));
  HIP_OK(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
  return p;
}

static void compare(const uint16_t* got_bits, const double* ref, size_t n, const char* what) {
  double mx = 0.0, sum = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double g = from_bf16(got_bits[i]);
    const double e = fabs(g - ref[i]);
    if (!(e == e)) { mx = INFINITY; break; }
    if (e > mx) mx = e;
    sum += e;
  }
  printf("%s: max|d| %.3e mean|d| %.3e\n", what, mx, sum / (double)n);
  EXPECT(mx <= 2e-2 && sum / (double)n <= 2e-3, "%s outside tolerance", what);
}

/* gradients: max|d| <= 2e-2 max|ref| + 1e-4 and mean|d| <= 1e-2 mean|ref| + 1e-4 */
static void compare_rel(const uint16_t* got_bits, const double* ref, size_t n, const char* what) {
  double mx = 0.0, sum = 0.0, rmax = 0.0, rsum = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double e = fabs((double)from_bf16(got_bits[i]) - ref[i]);
    if (!(e == e)) { mx = INFINITY; break; }
    if (e > mx) mx = e;
    sum += e;
    if (fabs(ref[i]) > rmax) rmax = fabs(ref[i]);
    rsum += fabs(ref[i]);
  }
  printf("%s: max|d|/max|ref| %.3e mean|d|/mean|ref| %.3e\n", what, mx / (rmax + 1e-30),
         sum / (rsum + 1e-30));
  EXPECT(mx <= 2e-2 * rmax + 1e-4 && sum / (double)n <= 1e-2 * rsum / (double)n + 1e-4,
         "%s outside tolerance", what);
}

/* elementwise results stored as bf16: within one bf16 ulp of the exact value */
static void compare_ulp(const uint16_t* got_bits, const double* ref, size_t n, const char* what) {
  size_t bad = 0;
  for (size_t i = 0; i < n; ++i) {
    const double a = fabs(ref[i]) > 1e-30 ? fabs(ref[i]) : 1e-30;
    const double ulp = ldexp(1.0, (int)floor(log2(a)) - 7);
    const double e = fabs((double)from_bf16(got_bits[i]) - ref[i]);
    if (!(e <= ulp)) ++bad;
  }
  printf("%s: %zu of %zu elements beyond one bf16 ulp\n", what, bad, n);
  EXPECT(bad == 0, "%s outside tolerance", what);
}

int main(void) {
  /* ---- prefill, local and global layer */
  const int B = 1, T = 333, S = 333, H = 4, KVH = 2, d = 128, W = 100;
  const float qs = 0.0883883476f, cap = 50.0f; /* 1/sqrt(128) */
  const size_t nq = (size_t)B * T * H * d, nk = (size_t)B * S * KVH * d;
  uint16_t *qb = malloc(nq * 2), *kb = malloc(nk * 2), *vb = malloc(nk * 2), *ob = malloc(nq * 2);
  float *qf = malloc(nq * 4), *kf = malloc(nk * 4), *vf = malloc(nk * 4);
  double* ref = malloc(nq * 8);
  draw(nq, 11, 3.0, qb, qf);
  draw(nk, 12, 3.0, kb, kf);
  draw(nk, 13, 1.0, vb, vf);
  void *dq = to_device(qb, nq * 2), *dk = to_device(kb, nk * 2), *dv = to_device(vb, nk * 2);
  void* dout = NULL;
  HIP_OK(hipMalloc(&dout, nq * 2));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  for (int is_local = 1; is_local >= 0; --is_local) {
    const int st = g2attn_prefill(dq, dk, dv, dout, B, T, S, H, KVH, d, qs, cap, W, is_local,
                                  G2_BF16, stream);
    EXPECT(st == G2_OK, "prefill status %d (%s)", st, g2attn_status_string(st));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(ob, dout, nq * 2, hipMemcpyDeviceToHost));
    EXPECT(g2o_prefill(qf, kf, vf, ref, B, T, S, H, KVH, d, qs, cap, W, is_local, NULL, 0) == 0,
           "oracle prefill");
    compare(ob, ref, nq, is_local ? "prefill local" : "prefill global");
  }

  /* ---- decode: three sequences against a linear 500-position cache */
  const int DB = 3, DS = 500;
  const int32_t lens[3] = {500, 123, 1};
  const size_t dnq = (size_t)DB * H * d, dnk = (size_t)DB * DS * KVH * d;
  uint16_t *dqb = malloc(dnq * 2), *dkb = malloc(dnk * 2), *dvb = malloc(dnk * 2), *dob = malloc(dnq * 2);
  float *dqf = malloc(dnq * 4), *dkf = malloc(dnk * 4), *dvf = malloc(dnk * 4);
  double* dref = malloc(dnq * 8);
  draw(dnq, 21, 3.0, dqb, dqf);
  draw(dnk, 22, 1.0, dkb, dkf);
  draw(dnk, 23, 1.0, dvb, dvf);
  void *ddq = to_device(dqb, dnq * 2), *ddk = to_device(dkb, dnk * 2), *ddv = to_device(dvb, dnk * 2);
  void* dlens = to_device(lens, sizeof(lens));
  void* ddo = NULL;
  HIP_OK(hipMalloc(&ddo, dnq * 2));
  const size_t wsb = g2attn_decode_workspace_bytes(DB, H, d, DS);
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, wsb));
  int st = g2attn_decode(ddq, ddk, ddv, ddo, (const int32_t*)dlens, DB, 1, DS, H, KVH, d, qs, cap,
                         W, 0, G2_BF16, ws, wsb, stream);
  EXPECT(st == G2_OK, "decode status %d (%s)", st, g2attn_status_string(st));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(dob, ddo, dnq * 2, hipMemcpyDeviceToHost));
  EXPECT(g2o_decode(dqf, dkf, dvf, lens, dref, DB, DS, H, KVH, d, qs, cap, W, 0, NULL, 0) == 0,
         "oracle decode");
  compare(dob, dref, dnq, "decode global");

  /* ---- prefill with log-sum-exp (local layer): out as above, lse within 2e-3 */
  {
    float* dlse = NULL;
    const size_t nl = (size_t)B * H * T;
    HIP_OK(hipMalloc((void**)&dlse, nl * sizeof(float)));
    st = g2attn_prefill_lse(dq, dk, dv, dout, dlse, B, T, S, H, KVH, d, qs, cap, W, 1, G2_BF16,
                            stream);
    EXPECT(st == G2_OK, "prefill_lse status %d (%s)", st, g2attn_status_string(st));
    HIP_OK(hipStreamSynchronize(stream));
    float* lse = malloc(nl * sizeof(float));
    double* lref = malloc(nl * sizeof(double));
    HIP_OK(hipMemcpy(ob, dout, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, dlse, nl * sizeof(float), hipMemcpyDeviceToHost));
    EXPECT(g2o_prefill(qf, kf, vf, ref, B, T, S, H, KVH, d, qs, cap, W, 1, NULL, 0) == 0,
           "oracle prefill");
    compare(ob, ref, nq, "prefill_lse out");
    EXPECT(g2o_prefill_lse(qf, kf, lref, B, T, S, H, KVH, d, qs, cap, W, 1, NULL, 0) == 0,
           "oracle lse");
    double lmx = 0.0; /* the library's lse is (B, H, T), the oracle's (B, T, H) */
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int t = 0; t < T; ++t) {
          const double e = fabs((double)lse[((size_t)b * H + h) * T + t] -
                                lref[((size_t)b * T + t) * H + h]);
          if (!(e <= lmx)) lmx = e;
        }
    printf("prefill_lse lse: max|d| %.3e\n", lmx);
    EXPECT(lmx <= 2e-3, "lse outside tolerance");

    /* ---- backward (keys of unit scale, so rows are not one-hot): forward with
       lse, then dq, dk, dv against the oracle's gradients */
    uint16_t *gob = malloc(nq * 2), *k2b = malloc(nk * 2);
    float *gof = malloc(nq * 4), *k2f = malloc(nk * 4);
    draw(nq, 14, 1.0, gob, gof);
    draw(nk, 15, 1.0, k2b, k2f);
    void *dgo = to_device(gob, nq * 2), *dk2 = to_device(k2b, nk * 2);
    st = g2attn_prefill_lse(dq, dk2, dv, dout, dlse, B, T, S, H, KVH, d, qs, cap, W, 1, G2_BF16,
                            stream);
    EXPECT(st == G2_OK, "prefill_lse status %d (%s)", st, g2attn_status_string(st));
    void *gdq = NULL, *gdk = NULL, *gdv = NULL, *bws = NULL;
    HIP_OK(hipMalloc(&gdq, nq * 2));
    HIP_OK(hipMalloc(&gdk, nk * 2));
    HIP_OK(hipMalloc(&gdv, nk * 2));
    const size_t bwsb = g2attn_prefill_backward_workspace_bytes(B, T, S, H);
    HIP_OK(hipMalloc(&bws, bwsb));
    st = g2attn_prefill_backward(dq, dk2, dv, dout, dgo, dlse, gdq, gdk, gdv, B, T, S, H, KVH, d, qs,
                                 cap, W, 1, G2_BF16, bws, bwsb, stream);
    EXPECT(st == G2_OK, "backward status %d (%s)", st, g2attn_status_string(st));
    HIP_OK(hipStreamSynchronize(stream));
    uint16_t *gq = malloc(nq * 2), *gk = malloc(nk * 2), *gv = malloc(nk * 2);
    HIP_OK(hipMemcpy(gq, gdq, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gk, gdk, nk * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gv, gdv, nk * 2, hipMemcpyDeviceToHost));
    double *rq = malloc(nq * 8), *rk = malloc(nk * 8), *rv = malloc(nk * 8);
    EXPECT(g2o_prefill_backward(qf, k2f, vf, gof, rq, rk, rv, B, T, S, H, KVH, d, qs, cap, W, 1) == 0,
           "oracle backward");
    compare_rel(gq, rq, nq, "backward dq");
    compare_rel(gk, rk, nk, "backward dk");
    compare_rel(gv, rv, nk, "backward dv");
    hipFree(dlse); hipFree(dgo); hipFree(dk2); hipFree(gdq); hipFree(gdk); hipFree(gdv); hipFree(bws);
    free(lse); free(lref); free(gob); free(gof); free(k2b); free(k2f); free(gq); free(gk); free(gv);
    free(rq); free(rk); free(rv);
  }

  /* ---- paged decode: the linear caches above cut into 16-position blocks,
     placed in the pool in a scrambled order (local layer, window W) */
  {
    const int bs = 16, MB = (DS + bs - 1) / bs, NB = DB * MB;
    const size_t row = (size_t)KVH * d, nb_elems = (size_t)NB * bs * row;
    uint16_t *pk = calloc(nb_elems, 2), *pv = calloc(nb_elems, 2);
    float *pkf = calloc(nb_elems, 4), *pvf = calloc(nb_elems, 4);
    int32_t* table = malloc(sizeof(int32_t) * (size_t)DB * MB);
    for (int b = 0; b < DB; ++b)
      for (int i = 0; i < MB; ++i) {
        const int blk = (int)(((long)(b * MB + i) * 37 + 11) % NB); /* 37 is prime to NB = 96 */
        table[b * MB + i] = blk;
        for (int r = 0; r < bs; ++r) {
          const int pos = i * bs + r;
          if (pos >= DS) break;
          const size_t src = ((size_t)b * DS + pos) * row, dst = ((size_t)blk * bs + r) * row;
          memcpy(pk + dst, dkb + src, row * 2);
          memcpy(pv + dst, dvb + src, row * 2);
          memcpy(pkf + dst, dkf + src, row * 4);
          memcpy(pvf + dst, dvf + src, row * 4);
        }
      }
    void *dpk = to_device(pk, nb_elems * 2), *dpv = to_device(pv, nb_elems * 2);
    void* dtab = to_device(table, sizeof(int32_t) * (size_t)DB * MB);
    const size_t pwsb = g2attn_decode_paged_workspace_bytes(DB, H, d, MB, bs);
    void* pws = NULL;
    HIP_OK(hipMalloc(&pws, pwsb));
    st = g2attn_decode_paged(ddq, dpk, dpv, ddo, (const int32_t*)dtab, MB, (const int32_t*)dlens, DB,
                             H, KVH, d, bs, NB, qs, cap, W, 1, G2_BF16, pws, pwsb, stream);
    EXPECT(st == G2_OK, "decode_paged status %d (%s)", st, g2attn_status_string(st));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(dob, ddo, dnq * 2, hipMemcpyDeviceToHost));
    EXPECT(g2o_decode_paged(dqf, pkf, pvf, table, MB, lens, dref, DB, H, KVH, d, bs, NB, qs, cap, W,
                            1, NULL, 0) == 0,
           "oracle decode_paged");
    compare(dob, dref, dnq, "decode_paged local");
    hipFree(dpk); hipFree(dpv); hipFree(dtab); hipFree(pws);
    free(pk); free(pv); free(pkf); free(pvf); free(table);
  }

  /* ---- rotary embedding (fp32, positions up to 4000) and the final cap (bf16) */
  {
    const int RB = 2, RT = 37, NH = 4, Rd = 128;
    const size_t nr = (size_t)RB * RT * NH * Rd;
    float* rx = malloc(nr * 4);
    double* rref = malloc(nr * 8);
    int32_t* pos = malloc(sizeof(int32_t) * (size_t)RB * RT);
    rng_state = 31;
    for (size_t i = 0; i < nr; ++i) rx[i] = (float)normal();
    for (int i = 0; i < RB * RT; ++i) pos[i] = (int32_t)(splitmix64() % 4001);
    void *drx = to_device(rx, nr * 4), *dpos = to_device(pos, sizeof(int32_t) * (size_t)RB * RT);
    st = g2attn_rope(drx, (const int32_t*)dpos, RB, RT, NH, Rd, 10000.0f, G2_F32, stream);
    EXPECT(st == G2_OK, "rope status %d (%s)", st, g2attn_status_string(st));
    HIP_OK(hipStreamSynchronize(stream));
    float* rgot = malloc(nr * 4);
    HIP_OK(hipMemcpy(rgot, drx, nr * 4, hipMemcpyDeviceToHost));
    EXPECT(g2o_rope(rx, pos, rref, RB, RT, NH, Rd, 10000.0) == 0, "oracle rope");
    double rmx = 0.0;
    for (size_t i = 0; i < nr; ++i) {
      const double e = fabs((double)rgot[i] - rref[i]);
      if (!(e <= rmx)) rmx = e;
    }
    printf("rope f32: max|d| %.3e\n", rmx);
    EXPECT(rmx <= 2e-5, "rope outside tolerance");

    const size_t ncap = 100003; /* not a multiple of the 8-element vectors */
    uint16_t* cb = malloc(ncap * 2);
    float* cf = malloc(ncap * 4);
    double* cref = malloc(ncap * 8);
    draw(ncap, 41, 40.0, cb, cf);
    void* dcx = to_device(cb, ncap * 2);
    st = g2attn_softcap(dcx, ncap, 30.0f, G2_BF16, stream);
    EXPECT(st == G2_OK, "softcap status %d (%s)", st, g2attn_status_string(st));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(cb, dcx, ncap * 2, hipMemcpyDeviceToHost));
    g2o_softcap_array(cf, cref, (int64_t)ncap, 30.0);
    compare_ulp(cb, cref, ncap, "final cap 30 bf16");
    hipFree(drx); hipFree(dpos); hipFree(dcx);
    free(rx); free(rref); free(pos); free(rgot); free(cb); free(cf); free(cref);
  }

  /* ---- documented error statuses (host-side checks; nothing is launched) */
  st = g2attn_prefill(NULL, dk, dv, dout, B, T, S, H, KVH, d, qs, cap, W, 1, G2_BF16, stream);
  EXPECT(st == G2_ERR_ARG, "null q gave %d", st);
  st = g2attn_prefill((const char*)dq + 2, dk, dv, dout, B, T, S, H, KVH, d, qs, cap, W, 1, G2_BF16,
                      stream);
  EXPECT(st == G2_ERR_ALIGN, "misaligned q gave %d", st);
  st = g2attn_prefill(dq, dk, dv, dout, B, T, S, H, KVH, 96, qs, cap, W, 1, G2_BF16, stream);
  EXPECT(st == G2_ERR_UNSUPPORTED, "d = 96 gave %d", st);
  st = g2attn_prefill(dq, dk, dv, dout, B, S + 1, S, H, KVH, d, qs, cap, W, 1, G2_BF16, stream);
  EXPECT(st == G2_ERR_ARG, "T > S gave %d", st);
  st = g2attn_decode(ddq, ddk, ddv, ddo, (const int32_t*)dlens, DB, 1, DS, H, KVH, d, qs, cap, W, 0,
                     G2_BF16, ws, wsb - 4, stream);
  EXPECT(st == G2_ERR_WORKSPACE, "short workspace gave %d", st);
  EXPECT(g2attn_status_string(G2_ERR_LAUNCH) != NULL, "status string");

  HIP_OK(hipStreamDestroy(stream));
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dout);
  hipFree(ddq); hipFree(ddk); hipFree(ddv); hipFree(ddo); hipFree(dlens); hipFree(ws);
  free(qb); free(kb); free(vb); free(ob); free(qf); free(kf); free(vf); free(ref);
  free(dqb); free(dkb); free(dvb); free(dob); free(dqf); free(dkf); free(dvf); free(dref);
  if (failures) {
    printf("c_abi_check: %d failure(s)\n", failures);
    return 1;
  }
  printf("c_abi_check ok\n");
  return 0;
}
