/*
 * Oracle driver for the sanitizer build (AddressSanitizer +
 * UndefinedBehaviorSanitizer, gcc, no OpenMP): runs every entry point of the
 * oracle on small seeded inputs -- direct, folded and split modes, selected
 * rows, per-chunk partials, bf16 and e4m3 KV, ragged batches, chunk counts
 * with empty last chunks -- and checks the relations the oracle's definition
 * fixes (folded == direct bitwise, split + merge == direct to 1e-12, rows ==
 * the full decode bitwise), so that an out-of-bounds access or undefined
 * behaviour anywhere in it surfaces under the sanitizers.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_mla_decode(int batch, int H, const int* q_len, const int* kv_len, const uint16_t* q_bits,
                      const void* kv, int kv_is_fp8, double kv_scale, double sm_scale, int mode,
                      const int* splits, int granule, double* o, double* lse);
int oracle_mla_decode_rows(int batch, int H, const int* q_len, const int* kv_len,
                           const uint16_t* q_bits, const void* kv, int kv_is_fp8, double kv_scale,
                           double sm_scale, long nrows, const long* rows, double* o, double* lse);
int oracle_mla_partial(int batch, int H, const int* q_len, const int* kv_len,
                       const uint16_t* q_bits, const void* kv, int kv_is_fp8, double kv_scale,
                       double sm_scale, int b, int i, int h, long lo, long hi, double* o,
                       double* lse);
int oracle_fold_factor(int H, int q);
void oracle_split_layout(long n, int S, int G, long* L_out, int* S_eff_out);

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);  \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

static unsigned g_state = 987654321u;
static unsigned next_u(void) {
  g_state = g_state * 1664525u + 1013904223u;
  return g_state >> 8;
}
/* a bf16 bit pattern of a value in [-0.25, 0.25) (exponent well inside range) */
static uint16_t rand_bf16(void) {
  float x = ((float)(next_u() % 65536u) / 65536.0f - 0.5f) * 0.5f;
  union { float f; uint32_t u; } c;
  c.f = x;
  return (uint16_t)(c.u >> 16);
}
/* an e4m3 code that is never NaN (0x7F / 0xFF) */
static uint8_t rand_e4m3(void) {
  uint8_t v;
  do v = (uint8_t)(next_u() & 0xFF); while ((v & 0x7F) == 0x7F);
  return v;
}

static void run_case(int batch, int H, const int* q_len, const int* kv_len, int fp8) {
  long sq = 0, sn = 0, rows, r, k;
  int b, S, mode;
  uint16_t* q;
  void* kv;
  double *o0, *l0, *o1, *l1;
  for (b = 0; b < batch; ++b) {
    sq += q_len[b];
    sn += kv_len[b];
  }
  rows = sq * H;
  q = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(rows * 576));
  for (k = 0; k < rows * 576; ++k) q[k] = rand_bf16();
  if (fp8) {
    uint8_t* kv8 = (uint8_t*)malloc((size_t)(sn * 576));
    for (k = 0; k < sn * 576; ++k) kv8[k] = rand_e4m3();
    kv = kv8;
  } else {
    uint16_t* kv16 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(sn * 576));
    for (k = 0; k < sn * 576; ++k) kv16[k] = rand_bf16();
    kv = kv16;
  }
  o0 = (double*)malloc(sizeof(double) * (size_t)(rows * 512));
  o1 = (double*)malloc(sizeof(double) * (size_t)(rows * 512));
  l0 = (double*)malloc(sizeof(double) * (size_t)rows);
  l1 = (double*)malloc(sizeof(double) * (size_t)rows);
  const double kvs = fp8 ? 1.0 / 448.0 : 1.0, sm = 1.0 / 24.0;
  CHECK(oracle_mla_decode(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, 0, NULL, 64, o0, l0) == 0);
  /* folded: bitwise equal */
  CHECK(oracle_mla_decode(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, 1, NULL, 64, o1, l1) == 0);
  for (r = 0; r < rows; ++r) CHECK(l0[r] == l1[r]);
  for (k = 0; k < rows * 512; ++k) CHECK(o0[k] == o1[k]);
  /* split + merge == direct, several chunk counts (empty last chunks included) */
  for (S = 1; S <= 9; S += 4) {
    int* splits = (int*)malloc(sizeof(int) * (size_t)batch);
    for (b = 0; b < batch; ++b) splits[b] = S + b % 3;
    for (mode = 2; mode <= 2; ++mode)
      CHECK(oracle_mla_decode(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, mode, splits, 64, o1,
                              l1) == 0);
    for (r = 0; r < rows; ++r) CHECK(fabs(l0[r] - l1[r]) <= 1e-12 * (1.0 + fabs(l0[r])));
    for (k = 0; k < rows * 512; ++k) CHECK(fabs(o0[k] - o1[k]) <= 1e-12);
    free(splits);
  }
  /* selected rows == the full decode, bitwise */
  {
    long sel[3] = {0, rows / 2, rows - 1};
    double os[3 * 512], ls[3];
    CHECK(oracle_mla_decode_rows(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, 3, sel, os, ls) == 0);
    for (r = 0; r < 3; ++r) {
      CHECK(ls[r] == l0[sel[r]]);
      for (k = 0; k < 512; ++k) CHECK(os[r * 512 + k] == o0[sel[r] * 512 + k]);
    }
    sel[1] = rows; /* out of range: rejected */
    CHECK(oracle_mla_decode_rows(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, 3, sel, os, ls) != 0);
  }
  /* partials over the whole visible range == the full decode; empty ranges */
  {
    double op[512], lp;
    const int bl = batch - 1, il = q_len[bl] - 1;
    long tok = sq - 1;
    CHECK(oracle_mla_partial(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, bl, il, H - 1, -5,
                             kv_len[bl] + 100, op, &lp) == 0);
    CHECK(fabs(lp - l0[tok * H + H - 1]) <= 1e-12 * (1.0 + fabs(lp)));
    CHECK(oracle_mla_partial(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, 0, 0, 0, 7, 7, op, &lp) == 0);
    CHECK(isinf(lp) && lp < 0);
    CHECK(oracle_mla_partial(batch, H, q_len, kv_len, q, kv, fp8, kvs, sm, batch, 0, 0, 0, 1, op,
                             &lp) != 0);
  }
  free(q);
  free(kv);
  free(o0);
  free(o1);
  free(l0);
  free(l1);
}

int main(void) {
  int H, qq;
  long n;
  int cases = 0;
  for (H = 1; H <= 130; ++H)
    for (qq = 1; qq <= 16; ++qq) {
      const int F = oracle_fold_factor(H, qq);
      CHECK(H > 128 ? F == 0 : (F >= 1 && qq % F == 0 && H * F <= 128));
    }
  for (n = 1; n <= 700; n += 37) {
    int S;
    for (S = 1; S <= 12; ++S) {
      long L;
      int Se;
      oracle_split_layout(n, S, 64, &L, &Se);
      CHECK(L % 64 == 0 && L * Se >= n && L * (Se - 1) < n && Se <= S);
    }
  }
  {
    const int q1[1] = {2}, n1[1] = {70};
    run_case(1, 12, q1, n1, 0);
    run_case(1, 12, q1, n1, 1);
    const int q2[3] = {1, 4, 3}, n2[3] = {9, 130, 3};
    run_case(3, 5, q2, n2, 0);
    run_case(3, 5, q2, n2, 1);
    const int q3[2] = {8, 1}, n3[2] = {200, 1};
    run_case(2, 16, q3, n3, 0);
    cases = 5;
  }
  /* invalid arguments are rejected */
  {
    const int qb[1] = {3}, nb[1] = {2};
    uint16_t dummy_q[3 * 576] = {0};
    uint16_t dummy_kv[2 * 576] = {0};
    double o[3 * 512], l[3];
    CHECK(oracle_mla_decode(1, 1, qb, nb, dummy_q, dummy_kv, 0, 1.0, 0.1, 0, NULL, 64, o, l) != 0);
  }
  printf("oracle driver: %d cases ok\n", cases);
  return 0;
}
