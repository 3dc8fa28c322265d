// Host plan: fold factor, split-KV chunking, work-unit layout and workspace
// size.  Pure host code; the only device interaction is an optional CU-count
// query (done by the caller in api.cpp).
//
// Fold rule: "[Kimi-K3] Allow DSPARK verify on cutedsl_mla (fold_sq)" (sglang
// PR #33650), section "Decision rule", paragraph "Why": F = the largest divisor
// of q with H * F <= 128, so the F tokens' H heads share one tile and the KV
// is streamed once per tile.
// Split-KV chunking plus a reduction at long context: same PR, section "GPU
// timeline".  The pages do not give a split rule; the plan's cost model below
// is this library's own (the pages' Cake planner chooses splits from
// host-known scalars only, "bench(cake_mla_varq_dcp_decode): ..." (flashinfer
// PR #5588), table "What was measured", row "host plan" -- so does this one).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>

#include "plan.hpp"

namespace mla {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

const char* last_error() { return g_err; }

// Largest divisor d of q with H * d <= kMaxRows and d <= cap (cap <= 0: none).
int fold_factor(int H, int q, int cap) {
  for (int d = q; d >= 1; --d) {
    if (q % d) continue;
    if (static_cast<int64_t>(H) * d > kMaxRows) continue;
    if (cap > 0 && d > cap) continue;
    return d;
  }
  return 0;
}

// L = G * ceil(ceil(n / S) / G), S_eff = ceil(n / L).
void split_layout(int64_t n, int S, int G, int32_t* L, int32_t* S_eff) {
  int64_t per = (n + S - 1) / S;
  int64_t l = (per + G - 1) / G * G;
  *L = static_cast<int32_t>(l);
  *S_eff = static_cast<int32_t>((n + l - 1) / l);
}

namespace {

// Cost of one chunk length L (keys, a granule multiple) used for every
// sequence: the main kernel runs ceil(units / CUs) waves of workgroups (one
// workgroup per CU), each wave as long as its longest unit; a unit costs its
// KV bytes plus a fixed start-up equivalent plus, when split, writing and
// re-reading its partial rows.  Modelled in bytes of HBM traffic per CU.
double plan_cost(const std::vector<int32_t>& q_len, const std::vector<int32_t>& kv_len,
                 const std::vector<int32_t>& F, int H, int num_cus, int64_t row_bytes, int32_t L,
                 int64_t* units_out) {
  int64_t units = 0;
  double longest = 0.0;
  for (size_t b = 0; b < q_len.size(); ++b) {
    const int64_t n = kv_len[b];
    const int32_t T = q_len[b] / F[b];
    const int32_t R = H * F[b];
    const int32_t NRB = (R + kMaxUnitRows - 1) / kMaxUnitRows;
    const int64_t S = (n + L - 1) / L;
    units += static_cast<int64_t>(T) * NRB * S;
    const double part = S > 1 ? static_cast<double>(R) * 2.0 * (kDv * 2 + 4) : 0.0;
    const double unit = static_cast<double>(std::min<int64_t>(L, n)) * row_bytes + part + 65536.0;
    longest = std::max(longest, unit);
  }
  *units_out = units;
  const int64_t waves = (units + num_cus - 1) / num_cus;
  return static_cast<double>(waves) * longest;
}

}  // namespace

mla_status build_plan(int32_t batch, int32_t H, const int32_t* q_len, const int32_t* kv_len,
                      const int32_t* causal_end, mla_kv_dtype dtype,
                      const mla_plan_options* opts, mla_plan* plan) {
  if (batch < 1) {
    set_error("batch must be >= 1 (got %d)", batch);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (H < 1) {
    set_error("num_heads must be >= 1 (got %d)", H);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (H > kMaxRows) {
    set_error("num_heads %d > %d: no fold factor F satisfies H*F <= %d", H, kMaxRows, kMaxRows);
    return MLA_ERR_UNSUPPORTED;
  }
  if (!q_len || !kv_len) {
    set_error("q_len and kv_len must be non-null host arrays");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (dtype != MLA_KV_BF16 && dtype != MLA_KV_FP8_E4M3) {
    set_error("unknown kv dtype %d", static_cast<int>(dtype));
    return MLA_ERR_UNSUPPORTED;
  }
  const int force_fold = opts ? opts->force_fold : 0;
  const int force_splits = opts ? opts->force_splits : 0;
  const int num_cus = opts ? opts->num_cus : 0;
  if (force_fold < 0 || force_splits < 0 || num_cus < 0) {
    set_error("plan options must be >= 0");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (num_cus < 1) {
    set_error("num_cus must be resolved before build_plan");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  int64_t sum_q = 0, sum_kv = 0;
  for (int b = 0; b < batch; ++b) {
    if (!causal_end && (q_len[b] < 1 || kv_len[b] < q_len[b])) {
      set_error("sequence %d: need 1 <= q_len <= kv_len (got q_len=%d kv_len=%d)", b, q_len[b],
                kv_len[b]);
      return MLA_ERR_INVALID_ARGUMENT;
    }
    if (causal_end && (q_len[b] < 1 || kv_len[b] < 1 || causal_end[b] < 1)) {
      set_error("sequence %d: need q_len >= 1, kv_len >= 1 and causal_end >= 1 (got %d, %d, %d)", b,
                q_len[b], kv_len[b], causal_end[b]);
      return MLA_ERR_INVALID_ARGUMENT;
    }
    sum_q += q_len[b];
    sum_kv += kv_len[b];
  }
  if (sum_q * H > std::numeric_limits<int32_t>::max() || sum_kv > std::numeric_limits<int32_t>::max()) {
    set_error("too many rows for one call (sum q_len * H = %lld, sum kv_len = %lld)",
              static_cast<long long>(sum_q * H), static_cast<long long>(sum_kv));
    return MLA_ERR_INVALID_ARGUMENT;
  }

  plan->batch = batch;
  plan->H = H;
  plan->dtype = dtype;
  plan->num_cus = num_cus;
  const int64_t row_bytes = dtype == MLA_KV_BF16 ? 2 * kDqk : kDqk;

  std::vector<int32_t> ql(q_len, q_len + batch), kl(kv_len, kv_len + batch), F(batch);
  for (int b = 0; b < batch; ++b) {
    F[b] = fold_factor(H, ql[b], force_fold);
    if (F[b] < 1) {  // cannot happen for H <= 128 (d = 1 always qualifies)
      set_error("sequence %d: no fold factor", b);
      return MLA_ERR_UNSUPPORTED;
    }
  }

  // Chunk length: forced, or the cost model's choice over granule multiples.
  std::vector<int32_t> Sreq(batch);
  if (force_splits > 0) {
    std::fill(Sreq.begin(), Sreq.end(), force_splits);
  } else {
    const int64_t nmax = *std::max_element(kl.begin(), kl.end());
    double best = std::numeric_limits<double>::infinity();
    int32_t bestL = static_cast<int32_t>((nmax + kGranule - 1) / kGranule * kGranule);
    // Candidates: every granule multiple up to 4096 keys, then ~3% steps.
    int64_t L = kGranule;
    while (true) {
      int64_t units = 0;
      const double c = plan_cost(ql, kl, F, H, num_cus, row_bytes, static_cast<int32_t>(L), &units);
      if (c < best * (1.0 - 1e-9)) {
        best = c;
        bestL = static_cast<int32_t>(L);
      }
      if (L >= nmax) break;
      int64_t step = L < 4096 ? kGranule : std::max<int64_t>(kGranule, L / 32 / kGranule * kGranule);
      L += step;
    }
    for (int b = 0; b < batch; ++b)
      Sreq[b] = static_cast<int32_t>((static_cast<int64_t>(kl[b]) + bestL - 1) / bestL);
  }

  plan->seqs.resize(batch);
  int64_t q_row = 0, kv_row = 0, part_row = 0;
  int32_t split_tiles = 0;
  for (int b = 0; b < batch; ++b) {
    SeqDesc& d = plan->seqs[b];
    d.q_row0 = static_cast<int32_t>(q_row);
    d.kv_row0 = static_cast<int32_t>(kv_row);
    d.n = kl[b];
    d.ce = causal_end ? causal_end[b] : kl[b];
    d.qlen = ql[b];
    d.F = F[b];
    d.T = ql[b] / F[b];
    d.R = H * F[b];
    d.NRB = (d.R + kMaxUnitRows - 1) / kMaxUnitRows;
    d.RBS = d.NRB == 1 ? d.R : (((d.R + d.NRB - 1) / d.NRB + 15) / 16) * 16;
    split_layout(d.n, Sreq[b], kGranule, &d.L, &d.S);
    if (d.S > 1) {
      d.part_row0 = static_cast<int32_t>(part_row);
      part_row += static_cast<int64_t>(d.T) * d.S * d.R;
      split_tiles += d.T;
      if (part_row > std::numeric_limits<int32_t>::max()) {
        set_error("split workspace too large (%lld partial rows)", static_cast<long long>(part_row));
        return MLA_ERR_INVALID_ARGUMENT;
      }
    } else {
      d.part_row0 = -1;
    }
    q_row += static_cast<int64_t>(ql[b]) * H;
    kv_row += kl[b];
  }

  // Launch slices: up to kMaxSeqPerLaunch sequences each.
  plan->launches.clear();
  plan->num_units = 0;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    Launch ln{};
    ln.seq_begin = b0;
    ln.seq_end = std::min(batch, b0 + kMaxSeqPerLaunch);
    int64_t units = 0;
    int maxRU = 0, split_rows = 0;
    for (int b = ln.seq_begin; b < ln.seq_end; ++b) {
      SeqDesc& d = plan->seqs[b];
      d.unit0 = static_cast<int32_t>(units);
      units += static_cast<int64_t>(d.T) * d.NRB * d.S;
      maxRU = std::max(maxRU, std::min(d.RBS, d.R));
      if (d.S > 1) split_rows += d.T * d.R;
    }
    if (units > std::numeric_limits<int32_t>::max() / 2) {
      set_error("too many work units (%lld)", static_cast<long long>(units));
      return MLA_ERR_INVALID_ARGUMENT;
    }
    ln.num_units = static_cast<int>(units);
    ln.nrt = ((maxRU + 1) / 2 + 15) / 16;
    ln.num_split_rows = split_rows;
    plan->num_units += ln.num_units;
    plan->launches.push_back(ln);
  }

  plan->total_part_rows = part_row;
  plan->num_split_tiles = split_tiles;
  if (part_row > 0) {
    const size_t lse_bytes = static_cast<size_t>(part_row) * sizeof(float);
    plan->part_o_offset = (lse_bytes + 255) / 256 * 256;
    plan->workspace_bytes = plan->part_o_offset + static_cast<size_t>(part_row) * kDv * sizeof(uint16_t);
  } else {
    plan->part_o_offset = 0;
    plan->workspace_bytes = 0;
  }
  return MLA_OK;
}

}  // namespace mla
