/*
 * mla_oracle.c -- fp64 CPU oracle for MLA speculative-verify decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file.  It is used by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark, and by nothing else.  It shares no code,
 * header, table or constant with the HIP library: the fold factor, the split
 * bounds and the value decoders below are written here from the pages, on
 * their own.
 *
 * What it computes (plain definition, no blocking, no fusion, no reordering
 * beyond what the definition states):
 *
 *   For sequence b with q_b verify tokens and n_b cached keys (the q_b tokens
 *   are the last q_b of the n_b positions), token i in [0, q_b), head h:
 *     visible keys   j in [0, n_b - q_b + i]          (causal among the tail)
 *     logit          s_j = sm_scale * sum_{d<576} Q[b,i,h,d] * KV[b,j,d]
 *     m = max_j s_j,  l = sum_j exp(s_j - m)
 *     O[b,i,h,c]   = sum_j exp(s_j - m) * KV[b,j,c] / l      c in [0, 512)
 *     LSE[b,i,h]   = m + ln(l)                               (natural log)
 *
 * Sources (cited by page title and section):
 *  - "[Kimi-K3] Allow DSPARK verify on cutedsl_mla (fold_sq)" (sglang PR
 *    #33650): the verify width (block_size 7 + 1 = 8 tokens per sequence,
 *    opening paragraphs); one shared KV head (MQA) for all H query heads and
 *    the H-per-rank values, section "Which decode backend?"; the 576-wide
 *    query/key ("HQk576" in the kernel name, section "GPU timeline");
 *    the fold rule F = largest divisor of q with H*F <= 128 and the fact
 *    that the folded kernel streams each KV byte once per tile, section
 *    "Decision rule", paragraph "Why"; the split-KV reduction that follows
 *    the folded kernel at long context, section "GPU timeline".
 *  - The same PR's prhub report, section "实现拆解" item 3, restates the F rule.
 *  - "bench(cake_mla_varq_dcp_decode): ..." (flashinfer PR #5588), table
 *    "What was measured", row "split rows": partial results of a split item
 *    are merged by a separate reduce kernel.
 *  - The 512 latent + 64 rope split of the 576 columns, V = the first 512
 *    columns of the same latent row, the causal tail and the softmax scale are
 *    the workload's problem statement for absorbed MLA decode; they are not
 *    printed on the pages, and every such reading is listed with the design
 *    notes.
 *
 * Pins (what checks this oracle against something other than itself) live in
 * tests/test_oracle_pins.py: closed forms (one key, two keys, identical keys),
 * invariants (shift, permutation, causal truncation, folded == direct bitwise,
 * split+merge == unsplit), brute force against scipy's logsumexp/softmax on
 * tiny inputs, planted-key probes with exact answers, and the decoders against
 * torch's bfloat16 / float8_e4m3fn and the fixed points of the OCP format.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_DQK 576   /* query/key width: 512 latent + 64 rope */
#define ORC_DV 512    /* value width: the first 512 columns of the latent row */
#define ORC_MAX_ROWS 128 /* H * F must not exceed this (fold rule) */

/* ---------------------------------------------------------------- decoders */

/* bfloat16 bits -> exact double: the 16 bits are the top half of an IEEE
 * binary32 value. */
double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3FN code -> exact double.  Sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the codes with
 * all exponent and mantissa bits set (0x7F, 0xFF) are NaN; there is no
 * infinity, so the largest finite magnitude is 1.75 * 2^8 = 448 (the value
 * the workload's per-tensor scale maps the KV amax to). */
double oracle_e4m3_to_double(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* -------------------------------------------------------- spec index math */

/* Fold factor: the largest divisor F of q with H * F <= 128 ("Decision rule",
 * paragraph "Why").  Returns 0 when no divisor qualifies (H > 128). */
int oracle_fold_factor(int H, int q) {
  int d;
  if (H < 1 || q < 1) return 0;
  for (d = q; d >= 1; --d)
    if (q % d == 0 && (long)H * d <= ORC_MAX_ROWS) return d;
  return 0;
}

/* Split layout for one sequence of n keys cut into S requested chunks whose
 * length is a multiple of the granule G:
 *   L     = G * ceil(ceil(n / S) / G)
 *   S_eff = ceil(n / L)
 *   chunk s covers keys [s * L, min((s + 1) * L, n)).
 * The pages give no boundary rule; this is the plain reading (equal chunks,
 * rounded up to whole granules, last chunk short). */
void oracle_split_layout(long n, int S, int G, long* L_out, int* S_eff_out) {
  long per, L;
  if (n < 1 || S < 1 || G < 1) {
    *L_out = 0;
    *S_eff_out = 0;
    return;
  }
  per = (n + S - 1) / S;
  L = ((per + G - 1) / G) * G;
  *L_out = L;
  *S_eff_out = (int)((n + L - 1) / L);
}

/* ----------------------------------------------------------- one attention row */

typedef struct {
  const void* kv;   /* [sum n, 576] bf16 bits (uint16) or e4m3 codes (uint8) */
  int kv_is_fp8;
  double kv_scale;  /* fp8: value = decoded code * kv_scale; bf16: 1 */
  double e4m3_lut[256];
} kv_view;

static double kv_at(const kv_view* v, long row, int col) {
  if (v->kv_is_fp8)
    return v->e4m3_lut[((const uint8_t*)v->kv)[row * ORC_DQK + col]] * v->kv_scale;
  return oracle_bf16_to_double(((const uint16_t*)v->kv)[row * ORC_DQK + col]);
}

/* Attention of one query row q[576] over the keys [lo, hi) of the sequence
 * whose first KV row is kv_base.  Two-pass safe softmax.  An empty range gives
 * lse = -inf and o = 0 (the merge gives such a chunk weight 0).
 * scratch must hold hi - lo doubles. */
static void attend_range(const double* q, const kv_view* v, long kv_base, long lo, long hi,
                         double sm_scale, double* o, double* lse, double* scratch) {
  long j;
  int c, d;
  double m = -INFINITY, l = 0.0;
  for (c = 0; c < ORC_DV; ++c) o[c] = 0.0;
  if (hi <= lo) {
    *lse = -INFINITY;
    return;
  }
  for (j = lo; j < hi; ++j) {
    double s = 0.0;
    for (d = 0; d < ORC_DQK; ++d) s += q[d] * kv_at(v, kv_base + j, d);
    s *= sm_scale;
    scratch[j - lo] = s;
    if (s > m) m = s;
  }
  for (j = lo; j < hi; ++j) {
    double w = exp(scratch[j - lo] - m);
    l += w;
    for (c = 0; c < ORC_DV; ++c) o[c] += w * kv_at(v, kv_base + j, c);
  }
  for (c = 0; c < ORC_DV; ++c) o[c] /= l;
  *lse = m + log(l);
}

/* Merge of per-chunk partials (normalised O_s, lse_s), in ascending s:
 *   M = max_s lse_s,  w_s = exp(lse_s - M),
 *   lse = M + ln(sum_s w_s),  O = sum_s w_s * O_s / sum_s w_s.
 * Chunks with lse_s = -inf get weight 0.  At least one chunk is non-empty. */
static void merge_partials(int S, const double* Os, const double* lses, double* o, double* lse) {
  int s, c;
  double M = -INFINITY, W = 0.0;
  for (s = 0; s < S; ++s)
    if (lses[s] > M) M = lses[s];
  for (c = 0; c < ORC_DV; ++c) o[c] = 0.0;
  for (s = 0; s < S; ++s) {
    double w;
    if (lses[s] == -INFINITY) continue;
    w = exp(lses[s] - M);
    W += w;
    for (c = 0; c < ORC_DV; ++c) o[c] += w * Os[(long)s * ORC_DV + c];
  }
  for (c = 0; c < ORC_DV; ++c) o[c] /= W;
  *lse = M + log(W);
}

/* ------------------------------------------------------------- batch driver */

enum { ORACLE_DIRECT = 0, ORACLE_FOLDED = 1, ORACLE_SPLIT = 2 };

/* Output row (token-major, then head) of a global query row: index
 * (q_off_b + i) * H + h into O [sum q, H, 512] and LSE [sum q, H]. */

typedef struct {
  int b, i, h;
} row_id;

static void build_view(kv_view* v, const void* kv, int kv_is_fp8, double kv_scale) {
  int c;
  v->kv = kv;
  v->kv_is_fp8 = kv_is_fp8;
  v->kv_scale = kv_is_fp8 ? kv_scale : 1.0;
  for (c = 0; c < 256; ++c) v->e4m3_lut[c] = oracle_e4m3_to_double((uint8_t)c);
}

/* Compute one output row (b, i, h) in the given mode. */
static void compute_row(int mode, int b, int i, int h, int H, const int* q_len, const long* q_off,
                        const int* kv_len, const long* kv_off, const uint16_t* q_bits,
                        const kv_view* v, double sm_scale, const int* splits, int granule,
                        double* o, double* lse) {
  double q[ORC_DQK];
  long n = kv_len[b];
  long visible = n - q_len[b] + i + 1; /* keys [0, visible) */
  long qrow = (q_off[b] + i) * (long)H + h;
  int d;
  double* scratch;
  for (d = 0; d < ORC_DQK; ++d) q[d] = oracle_bf16_to_double(q_bits[qrow * ORC_DQK + d]);
  scratch = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  if (mode != ORACLE_SPLIT) {
    attend_range(q, v, kv_off[b], 0, visible, sm_scale, o, lse, scratch);
  } else {
    long L;
    int S_eff, s;
    double *Os, *lses;
    oracle_split_layout(n, splits[b], granule, &L, &S_eff);
    Os = (double*)malloc(sizeof(double) * (size_t)S_eff * ORC_DV);
    lses = (double*)malloc(sizeof(double) * (size_t)S_eff);
    for (s = 0; s < S_eff; ++s) {
      long lo = (long)s * L;
      long hi = lo + L < n ? lo + L : n;
      if (hi > visible) hi = visible;
      attend_range(q, v, kv_off[b], lo, hi, sm_scale, Os + (long)s * ORC_DV, lses + s, scratch);
    }
    merge_partials(S_eff, Os, lses, o, lse);
    free(Os);
    free(lses);
  }
  free(scratch);
}

/*
 * Full decode.  mode: 0 direct loop over (b, i, h); 1 folded loop over tiles
 * and tile rows (row r of tile t is token t*F + r/H, head r%H, F from the fold
 * rule); 2 split-then-merge with splits[b] requested chunks of granule keys.
 * q_bits: bf16 bits [sum q, H, 576].  kv: [sum n, 576] bf16 bits or e4m3 codes.
 * o: [sum q, H, 512] doubles; lse: [sum q, H] doubles.
 * Returns 0 on success, -1 on invalid arguments (kv_len < q_len, H*1 > 128 ...).
 */
int oracle_mla_decode(int batch, int H, const int* q_len, const int* kv_len, const uint16_t* q_bits,
                      const void* kv, int kv_is_fp8, double kv_scale, double sm_scale, int mode,
                      const int* splits, int granule, double* o, double* lse) {
  long *q_off, *kv_off;
  long total_rows = 0;
  int b;
  kv_view* v;
  if (batch < 1 || H < 1) return -1;
  for (b = 0; b < batch; ++b) {
    if (q_len[b] < 1 || kv_len[b] < q_len[b]) return -1;
    if (oracle_fold_factor(H, q_len[b]) == 0) return -1;
    if (mode == ORACLE_SPLIT && (splits == NULL || splits[b] < 1 || granule < 1)) return -1;
  }
  q_off = (long*)malloc(sizeof(long) * (size_t)batch);
  kv_off = (long*)malloc(sizeof(long) * (size_t)batch);
  for (b = 0; b < batch; ++b) {
    q_off[b] = b == 0 ? 0 : q_off[b - 1] + q_len[b - 1];
    kv_off[b] = b == 0 ? 0 : kv_off[b - 1] + kv_len[b - 1];
    total_rows += (long)q_len[b] * H;
  }
  v = (kv_view*)malloc(sizeof(kv_view));
  build_view(v, kv, kv_is_fp8, kv_scale);

  if (mode == ORACLE_FOLDED) {
    /* Enumerate (b, t, r) and map each tile row to its (token, head). */
    long n_units = 0, u;
    row_id* ids;
    for (b = 0; b < batch; ++b) n_units += (long)q_len[b] * H;
    ids = (row_id*)malloc(sizeof(row_id) * (size_t)n_units);
    u = 0;
    for (b = 0; b < batch; ++b) {
      int F = oracle_fold_factor(H, q_len[b]);
      int T = q_len[b] / F, R = H * F, t, r;
      for (t = 0; t < T; ++t)
        for (r = 0; r < R; ++r) {
          ids[u].b = b;
          ids[u].i = t * F + r / H;
          ids[u].h = r % H;
          ++u;
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (u = 0; u < n_units; ++u) {
      row_id id = ids[u];
      long orow = (q_off[id.b] + id.i) * (long)H + id.h;
      compute_row(mode, id.b, id.i, id.h, H, q_len, q_off, kv_len, kv_off, q_bits, v, sm_scale,
                  splits, granule, o + orow * ORC_DV, lse + orow);
    }
    free(ids);
  } else {
    long rrow;
#pragma omp parallel for schedule(dynamic, 1)
    for (rrow = 0; rrow < total_rows; ++rrow) {
      /* rrow is the output row index (token-major, head-minor). */
      long tok = rrow / H;
      int h = (int)(rrow % H), bb = 0;
      while (tok >= q_off[bb] + q_len[bb]) ++bb;
      compute_row(mode, bb, (int)(tok - q_off[bb]), h, H, q_len, q_off, kv_len, kv_off, q_bits, v,
                  sm_scale, splits, granule, o + rrow * ORC_DV, lse + rrow);
    }
  }
  free(v);
  free(q_off);
  free(kv_off);
  (void)total_rows;
  return 0;
}

/*
 * Selected rows only (for full-size configurations): rows[k] is an output row
 * index (token-major, head-minor, as above).  o: [nrows, 512], lse: [nrows].
 * Direct mode.
 */
int oracle_mla_decode_rows(int batch, int H, const int* q_len, const int* kv_len,
                           const uint16_t* q_bits, const void* kv, int kv_is_fp8, double kv_scale,
                           double sm_scale, long nrows, const long* rows, double* o, double* lse) {
  long *q_off, *kv_off, k, total = 0;
  int b;
  kv_view* v;
  if (batch < 1 || H < 1) return -1;
  for (b = 0; b < batch; ++b) {
    if (q_len[b] < 1 || kv_len[b] < q_len[b]) return -1;
    total += (long)q_len[b] * H;
  }
  for (k = 0; k < nrows; ++k)
    if (rows[k] < 0 || rows[k] >= total) return -1;
  q_off = (long*)malloc(sizeof(long) * (size_t)batch);
  kv_off = (long*)malloc(sizeof(long) * (size_t)batch);
  for (b = 0; b < batch; ++b) {
    q_off[b] = b == 0 ? 0 : q_off[b - 1] + q_len[b - 1];
    kv_off[b] = b == 0 ? 0 : kv_off[b - 1] + kv_len[b - 1];
  }
  v = (kv_view*)malloc(sizeof(kv_view));
  build_view(v, kv, kv_is_fp8, kv_scale);
#pragma omp parallel for schedule(dynamic, 1)
  for (k = 0; k < nrows; ++k) {
    long tok = rows[k] / H;
    int h = (int)(rows[k] % H), bb = 0;
    while (tok >= q_off[bb] + q_len[bb]) ++bb;
    compute_row(ORACLE_DIRECT, bb, (int)(tok - q_off[bb]), h, H, q_len, q_off, kv_len, kv_off,
                q_bits, v, sm_scale, NULL, 0, o + k * ORC_DV, lse + k);
  }
  free(v);
  free(q_off);
  free(kv_off);
  return 0;
}

/* Per-chunk partial of one row (for checking split workspaces): keys
 * [lo, hi) of sequence b seen by token i, head h.  o: [512], lse: scalar. */
int oracle_mla_partial(int batch, int H, const int* q_len, const int* kv_len,
                       const uint16_t* q_bits, const void* kv, int kv_is_fp8, double kv_scale,
                       double sm_scale, int b, int i, int h, long lo, long hi, double* o,
                       double* lse) {
  long q_off = 0, kv_off = 0, n, visible, qrow;
  int bb, d;
  double q[ORC_DQK];
  double* scratch;
  kv_view* v;
  if (b < 0 || b >= batch || i < 0 || i >= q_len[b] || h < 0 || h >= H) return -1;
  for (bb = 0; bb < b; ++bb) {
    q_off += q_len[bb];
    kv_off += kv_len[bb];
  }
  n = kv_len[b];
  visible = n - q_len[b] + i + 1;
  if (lo < 0) lo = 0;
  if (hi > n) hi = n;
  if (hi > visible) hi = visible;
  qrow = (q_off + i) * (long)H + h;
  for (d = 0; d < ORC_DQK; ++d) q[d] = oracle_bf16_to_double(q_bits[qrow * ORC_DQK + d]);
  v = (kv_view*)malloc(sizeof(kv_view));
  build_view(v, kv, kv_is_fp8, kv_scale);
  scratch = (double*)malloc(sizeof(double) * (size_t)(hi > lo ? hi - lo : 1));
  attend_range(q, v, kv_off, lo, hi, sm_scale, o, lse, scratch);
  free(scratch);
  free(v);
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count for the following calls (timing runs: a single-thread run
 * beside the all-core one).  n < 1 is ignored. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
