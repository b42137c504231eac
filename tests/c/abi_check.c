/*
 * abi_check.c -- libattnres used from plain C, as a C caller would: device
 * buffers from the HIP runtime, attnres_init / attnres_fwd / attnres_fwd_path
 * / attnres_validate / attnres_strerror, every kernel path, checked against
 * the fp64 C oracle (oracle/attnres_oracle.c, linked as liboracle_attnres).
 * Test infrastructure: built by build(), run by tests/test_gpu_c_abi.py.
 *
 * Bar (as everywhere in the tests): out within 1e-2 + 1.6e-2 |oracle| of the
 * oracle rounded to bf16; prefix and the whole bank bit-exact.
 * Exit status 0 when every case passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attnres.h"

/* The oracle's entry point (oracle/attnres_oracle.c). */
int oracle_attnres_fwd(int64_t T, int64_t H, uint16_t *prefix, const uint16_t *delta,
                       uint16_t *blocks, int64_t token_stride, int64_t slot_stride, int cap,
                       int nb, const uint16_t *res_w, const uint16_t *rms_w, double rms_eps,
                       const uint16_t *onw, double out_eps, int widx, double *out_f64,
                       uint16_t *out_bf16, double *logits, double *probs);

#define H 7168
#define CAP 8

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, uniform in [0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
/* An input value as bf16 bits: a float cut to its top 16 bits (inputs only
 * need to be bf16 values, not any particular rounding of a draw). */
static uint16_t to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static double widen(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

#define HIP_OK(x)                                                               \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                  \
    }                                                                           \
  } while (0)

static void *to_device(const void *h, size_t bytes) {
  void *d = NULL;
  HIP_OK(hipMalloc(&d, bytes));
  HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

/* One call on one path against the oracle; returns 1 on pass. */
static int run_case(const char *name, int T, int nb, int has_delta, int has_onorm, int widx,
                    int path) {
  const int64_t ts = (int64_t)CAP * H, ss = H;
  const size_t row = (size_t)H * 2, mat = (size_t)T * row, bank_bytes = (size_t)T * ts * 2;
  uint16_t *prefix = malloc(mat), *delta = malloc(mat), *bank = malloc(bank_bytes);
  uint16_t *res_w = malloc(row), *rms_w = malloc(row), *onw = malloc(row), *out = malloc(mat);
  for (int64_t i = 0; i < (int64_t)T * H; ++i) {
    prefix[i] = to_bf16_bits((float)(4.0 * uniform() - 2.0));
    delta[i] = to_bf16_bits((float)(4.0 * uniform() - 2.0));
  }
  for (int64_t i = 0; i < (int64_t)T * ts; ++i) bank[i] = to_bf16_bits((float)(4.0 * uniform() - 2.0));
  for (int h = 0; h < H; ++h) {
    res_w[h] = to_bf16_bits((float)(1.0 + 0.2 * (uniform() - 0.5)));
    rms_w[h] = to_bf16_bits((float)(1.0 + 0.2 * (uniform() - 0.5)));
    onw[h] = to_bf16_bits((float)(1.0 + 0.2 * (uniform() - 0.5)));
  }
  memset(out, 0xFF, mat);

  /* GPU */
  uint16_t *d_prefix = to_device(prefix, mat), *d_delta = to_device(delta, mat);
  uint16_t *d_bank = to_device(bank, bank_bytes), *d_out = to_device(out, mat);
  uint16_t *d_res = to_device(res_w, row), *d_rms = to_device(rms_w, row), *d_onw = to_device(onw, row);
  int rc = attnres_fwd_path(d_prefix, has_delta ? d_delta : NULL, d_bank, ts, ss, CAP, nb, d_res,
                            d_rms, 1e-6f, has_onorm ? d_onw : NULL, 1e-6f, widx, d_out, T, H,
                            NULL, path);
  if (rc != ATTNRES_OK) {
    printf("FAIL %s path %d: %s\n", name, path, attnres_strerror(rc));
    return 0;
  }
  HIP_OK(hipDeviceSynchronize());
  uint16_t *g_out = malloc(mat), *g_prefix = malloc(mat), *g_bank = malloc(bank_bytes);
  HIP_OK(hipMemcpy(g_out, d_out, mat, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(g_prefix, d_prefix, mat, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(g_bank, d_bank, bank_bytes, hipMemcpyDeviceToHost));

  /* oracle, on host copies */
  double *o64 = malloc((size_t)T * H * 8), *logits = malloc((size_t)T * (nb + 1) * 8);
  double *probs = malloc((size_t)T * (nb + 1) * 8);
  uint16_t *obf = malloc(mat);
  rc = oracle_attnres_fwd(T, H, prefix, has_delta ? delta : NULL, bank, ts, ss, CAP, nb, res_w,
                          rms_w, 1e-6, has_onorm ? onw : NULL, 1e-6, widx, o64, obf, logits, probs);
  int ok = rc == 0;
  double worst = 0.0;
  for (int64_t i = 0; ok && i < (int64_t)T * H; ++i) {
    const double g = widen(g_out[i]), o = widen(obf[i]);
    const double err = fabs(g - o);
    if (!(err <= 1e-2 + 1.6e-2 * fabs(o))) ok = 0;
    if (err > worst) worst = err;
  }
  if (ok && memcmp(g_prefix, prefix, mat) != 0) ok = 0;
  if (ok && memcmp(g_bank, bank, bank_bytes) != 0) ok = 0;
  printf("%s %s path %d: T=%d nb=%d delta=%d norm=%d widx=%d, max |gpu - oracle| = %.3e\n",
         ok ? "PASS" : "FAIL", name, path, T, nb, has_delta, has_onorm, widx, worst);

  HIP_OK(hipFree(d_prefix)); HIP_OK(hipFree(d_delta)); HIP_OK(hipFree(d_bank));
  HIP_OK(hipFree(d_out)); HIP_OK(hipFree(d_res)); HIP_OK(hipFree(d_rms)); HIP_OK(hipFree(d_onw));
  free(prefix); free(delta); free(bank); free(res_w); free(rms_w); free(onw); free(out);
  free(g_out); free(g_prefix); free(g_bank); free(o64); free(logits); free(probs); free(obf);
  return ok;
}

int main(void) {
  int device_count = 0;
  HIP_OK(hipGetDeviceCount(&device_count));
  if (device_count < 1) {
    fprintf(stderr, "no GPU\n");
    return 2;
  }
  if (attnres_init(0) != ATTNRES_OK) {
    fprintf(stderr, "attnres_init failed\n");
    return 2;
  }
  int pass = 1;
  const int paths[] = {ATTNRES_PATH_AUTO, ATTNRES_PATH_ROW, ATTNRES_PATH_SPLIT, ATTNRES_PATH_ANY_H};
  for (int k = 0; k < 4; ++k) {
    pass &= run_case("mixed", 7, 5, 1, 1, 2, paths[k]);
    pass &= run_case("plain", 3, 0, 0, 0, -1, paths[k]);
    pass &= run_case("full", 2, 8, 1, 0, 7, paths[k]);
  }
  /* a rejected call: out aliasing prefix, checked on the host only */
  const int rc = attnres_validate((void *)0x10000000, NULL, NULL, 0, 0, 0, 0, (void *)0x20000000,
                                  (void *)0x30000000, 1e-6f, NULL, 0.f, -1, (void *)0x10000000, 4, H);
  const int alias_ok = rc == ATTNRES_E_ALIAS;
  printf("%s rejected call: %s\n", alias_ok ? "PASS" : "FAIL", attnres_strerror(rc));
  pass &= alias_ok;
  pass &= attnres_device_status(0) == ATTNRES_OK;
  attnres_shutdown();
  printf("%s\n", pass ? "ALL PASS" : "SOME FAILED");
  return pass ? 0 : 1;
}
