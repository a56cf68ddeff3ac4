/*
 * The C ABI used from plain C, with no Python or PyTorch in the process:
 * device buffers from the HIP runtime, the library's prefill and decode on
 * them, results checked against the CPU fp64 oracle (test infrastructure,
 * linked only into this checker), and the documented error statuses.
 *
 * Inputs are seeded normal draws rounded to bf16; the oracle reads the same
 * values widened to float.  Tolerances: max |diff| <= 2e-2, mean <= 2e-3.
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
