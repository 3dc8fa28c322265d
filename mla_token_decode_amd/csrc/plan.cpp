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
#include <functional>
#include <limits>
#include <numeric>
#include <queue>

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

// Per-sequence chunking (plan_mode MLA_PLAN_AUTO).  A unit of sequence b
// (one tile, or row block of a tile, against one chunk) is modelled in
// microseconds of the one CU it occupies: streaming its KV rows or running
// its MFMAs, whichever is longer, plus a fixed start-up and, when b is split,
// writing its partial rows.  The rates are the kernels' measured ones on the
// MI355X (HBM streaming shared by 256 CUs; MFMA throughput as the kernels
// achieve it, per padded row), so the model ranks plans, it does not predict
// times to the microsecond.
constexpr double kCuBytesPerUs = 6.0e12 / 256 / 1e6;     // ~23.4 KB/us per CU
constexpr double kFlopsPerKeyRow = 2.0 * (kDqk + kDv);     // QK^T and PV
constexpr double kCuFlopsPerUsBf16 = 4.0e6;                // bf16 KV kernel
constexpr double kCuFlopsPerUsFp8 = 8.0e6;                 // fp8 KV kernel
constexpr double kUnitFixedUs = 4.0;                       // Q set-up, first tile, epilogue
constexpr double kMergeFixedUs = 6.0;                      // launch and ramp of the merge
constexpr double kMergeBytesPerUs = 5.0e12 / 1e6;          // merge: partial rows read back

struct SeqModel {
  int64_t n;
  int64_t units_per_chunk;  // T * NRB
  double per_key;           // us per key of one unit
  double part;              // us per unit to write its partial rows (split sequences)
  double part_bytes;        // partial bytes per unit
};

double unit_us(const SeqModel& m, int64_t keys, bool split) {
  return kUnitFixedUs + static_cast<double>(keys) * m.per_key + (split ? m.part : 0.0);
}

// Chunk length of sequence m for a target unit time tau: the longest granule
// multiple whose unit fits tau (at least one granule), then balanced over the
// resulting chunk count by the split rule.
void chunking_for(const SeqModel& m, double tau, int32_t* L, int32_t* S) {
  if (unit_us(m, m.n, false) <= tau) {  // the whole sequence fits one unit
    split_layout(m.n, 1, kGranule, L, S);
    return;
  }
  const double keys = (tau - kUnitFixedUs - m.part) / m.per_key;
  const int64_t l = keys <= kGranule ? kGranule : static_cast<int64_t>(keys) / kGranule * kGranule;
  split_layout(m.n, static_cast<int>((m.n + l - 1) / l), kGranule, L, S);
}

// Predicted main-kernel makespan plus merge time of per-sequence chunkings
// (L[b], S[b]): units taken in `order` (sequence by sequence, every unit of
// a chunk together), each started on the CU that frees first.
double schedule_us(const std::vector<SeqModel>& m, const std::vector<int32_t>& L,
                   const std::vector<int32_t>& S, const std::vector<int>& order, int num_cus) {
  double makespan = 0.0, part_bytes = 0.0;
  int64_t units = 0;
  for (size_t b = 0; b < m.size(); ++b) units += m[b].units_per_chunk * S[b];
  if (units <= num_cus) {  // one wave: every unit starts at once
    for (size_t b = 0; b < m.size(); ++b) {
      makespan = std::max(makespan, unit_us(m[b], std::min<int64_t>(L[b], m[b].n), S[b] > 1));
      if (S[b] > 1) part_bytes += m[b].part_bytes * m[b].units_per_chunk * S[b];
    }
    return makespan + (part_bytes > 0.0 ? kMergeFixedUs + part_bytes / kMergeBytesPerUs : 0.0);
  }
  std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
  for (int i = 0; i < num_cus; ++i) cu.push(0.0);
  for (int b : order) {
    const bool split = S[b] > 1;
    for (int32_t s = 0; s < S[b]; ++s) {
      const int64_t keys = std::min<int64_t>(L[b], m[b].n - static_cast<int64_t>(s) * L[b]);
      const double t = unit_us(m[b], keys, split);
      for (int64_t u = 0; u < m[b].units_per_chunk; ++u) {
        const double start = cu.top();
        cu.pop();
        cu.push(start + t);
        makespan = std::max(makespan, start + t);
      }
    }
    if (split) part_bytes += m[b].part_bytes * m[b].units_per_chunk * S[b];
  }
  return makespan + (part_bytes > 0.0 ? kMergeFixedUs + part_bytes / kMergeBytesPerUs : 0.0);
}

// Sequences by decreasing unit time (ties: the caller's order).
std::vector<int> longest_first(const std::vector<SeqModel>& m, const std::vector<int32_t>& L,
                               const std::vector<int32_t>& S) {
  std::vector<int> order(m.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return unit_us(m[a], std::min<int64_t>(L[a], m[a].n), S[a] > 1) >
           unit_us(m[b], std::min<int64_t>(L[b], m[b].n), S[b] > 1);
  });
  return order;
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
  const int plan_mode = opts ? opts->plan_mode : MLA_PLAN_AUTO;
  const int merge_mode = opts ? opts->merge_mode : MLA_MERGE_AUTO;
  if (force_fold < 0 || force_splits < 0 || num_cus < 0) {
    set_error("plan options must be >= 0");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (plan_mode != MLA_PLAN_AUTO && plan_mode != MLA_PLAN_UNIFORM) {
    set_error("unknown plan_mode %d", plan_mode);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (merge_mode != MLA_MERGE_AUTO && merge_mode != MLA_MERGE_REDUCE &&
      merge_mode != MLA_MERGE_LAST_ARRIVER && merge_mode != MLA_MERGE_GRID) {
    set_error("unknown merge_mode %d", merge_mode);
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

  // Chunking: forced, one chunk length for all (MLA_PLAN_UNIFORM), or per
  // sequence (MLA_PLAN_AUTO).
  std::vector<int32_t> Lb(batch), Sb(batch);
  std::vector<int> order(batch);
  std::iota(order.begin(), order.end(), 0);
  if (force_splits > 0) {
    for (int b = 0; b < batch; ++b) split_layout(kl[b], force_splits, kGranule, &Lb[b], &Sb[b]);
  } else if (plan_mode == MLA_PLAN_UNIFORM) {
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
      split_layout(kl[b], static_cast<int>((static_cast<int64_t>(kl[b]) + bestL - 1) / bestL),
                   kGranule, &Lb[b], &Sb[b]);
  } else {
    std::vector<SeqModel> m(batch);
    const double flops = dtype == MLA_KV_BF16 ? kCuFlopsPerUsBf16 : kCuFlopsPerUsFp8;
    double tau_hi = 0.0;
    for (int b = 0; b < batch; ++b) {
      const int32_t T = ql[b] / F[b], R = H * F[b];
      const int32_t NRB = (R + kMaxUnitRows - 1) / kMaxUnitRows;
      const int32_t RBS = NRB == 1 ? R : (((R + NRB - 1) / NRB + 15) / 16) * 16;
      const int32_t rows_pad = (std::min(RBS, R) + 31) / 32 * 32;  // the kernels' row tiles
      m[b].n = kl[b];
      m[b].units_per_chunk = static_cast<int64_t>(T) * NRB;
      m[b].per_key = std::max(static_cast<double>(row_bytes) / kCuBytesPerUs,
                              rows_pad * kFlopsPerKeyRow / flops);
      m[b].part_bytes = static_cast<double>(std::min(RBS, R)) * (kDv * 2 + 4);
      m[b].part = m[b].part_bytes / kCuBytesPerUs;
      tau_hi = std::max(tau_hi, unit_us(m[b], kl[b], false));
    }
    // Candidate unit times come from the chunk counts of the sequence with
    // the most work: a ~3% geometric sweep of its chunk count, plus the counts
    // that fill whole waves of CUs (1..16 waves, less a few units for the
    // other sequences); each candidate's unit time then sets every
    // sequence's chunking.  Chunkings needing more than 16 waves only add
    // fixed costs and are skipped; "every sequence whole" always counts.
    int dom = 0;
    for (int b = 1; b < batch; ++b)
      if (m[b].n * m[b].per_key * m[b].units_per_chunk >
          m[dom].n * m[dom].per_key * m[dom].units_per_chunk)
        dom = b;
    const int64_t max_units = 16 * static_cast<int64_t>(num_cus);
    const int64_t s_max = std::max<int64_t>(
        1, std::min<int64_t>((m[dom].n + kGranule - 1) / kGranule, max_units / m[dom].units_per_chunk));
    std::vector<int64_t> counts;
    for (double x = 1.0; x <= static_cast<double>(s_max); x *= 1.03) counts.push_back(static_cast<int64_t>(x));
    counts.push_back(s_max);
    for (int64_t w = 1; w <= 16; ++w)
      for (int64_t k = 0; k < 4; ++k)
        counts.push_back((w * num_cus - k) / m[dom].units_per_chunk);
    std::sort(counts.begin(), counts.end());
    counts.erase(std::unique(counts.begin(), counts.end()), counts.end());
    std::vector<double> taus;
    for (int64_t c : counts) {
      if (c < 1 || c > s_max) continue;
      int32_t Ld, Sd;
      split_layout(m[dom].n, static_cast<int>(c), kGranule, &Ld, &Sd);
      taus.push_back(unit_us(m[dom], std::min<int64_t>(Ld, m[dom].n), Sd > 1) + 1e-9);
    }
    taus.push_back(tau_hi * (1.0 + 1e-9));  // every sequence whole
    double best = std::numeric_limits<double>::infinity();
    std::vector<int32_t> L(batch), S(batch), prevS;
    for (size_t i = 0; i < taus.size(); ++i) {
      const bool last = i + 1 == taus.size();
      int64_t units = 0;
      for (int b = 0; b < batch; ++b) {
        chunking_for(m[b], taus[i], &L[b], &S[b]);
        units += m[b].units_per_chunk * S[b];
      }
      if ((units > max_units && !last) || S == prevS) continue;
      prevS = S;
      const std::vector<int> ord = longest_first(m, L, S);
      const double c = schedule_us(m, L, S, ord, num_cus);
      if (c < best * (1.0 - 1e-9)) {
        best = c;
        Lb = L;
        Sb = S;
        order = ord;
      }
    }
  }

  // Rows of each sequence in the caller's layout.
  std::vector<int64_t> q_row0(batch), kv_row0(batch);
  {
    int64_t q_row = 0, kv_row = 0;
    for (int b = 0; b < batch; ++b) {
      q_row0[b] = q_row;
      kv_row0[b] = kv_row;
      q_row += static_cast<int64_t>(ql[b]) * H;
      kv_row += kl[b];
    }
  }
  plan->seqs.resize(batch);
  plan->pos.resize(batch);
  int64_t part_row = 0;
  int32_t split_tiles = 0;
  for (int i = 0; i < batch; ++i) {
    const int b = order[i];
    plan->pos[b] = i;
    SeqDesc& d = plan->seqs[i];
    d.src = b;
    d.q_row0 = static_cast<int32_t>(q_row0[b]);
    d.kv_row0 = static_cast<int32_t>(kv_row0[b]);
    d.n = kl[b];
    d.ce = causal_end ? causal_end[b] : kl[b];
    d.qlen = ql[b];
    d.F = F[b];
    d.T = ql[b] / F[b];
    d.R = H * F[b];
    d.NRB = (d.R + kMaxUnitRows - 1) / kMaxUnitRows;
    d.RBS = d.NRB == 1 ? d.R : (((d.R + d.NRB - 1) / d.NRB + 15) / 16) * 16;
    d.L = Lb[b];
    d.S = Sb[b];
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
  }

  // One launch: its sequence descriptors travel in the kernel arguments (up
  // to kMaxSeqPerLaunch) or, for larger batches, in a table in the workspace.
  plan->launches.clear();
  plan->num_units = 0;
  plan->seq_table = batch > kMaxSeqPerLaunch;
  {
    Launch ln{};
    ln.seq_begin = 0;
    ln.seq_end = batch;
    int64_t units = 0;
    int maxRU = 0, split_rows = 0, max_s = 0;
    bool shared_chunks = false;  // some chunk is read by more than one unit (tiles or row blocks)
    for (int b = ln.seq_begin; b < ln.seq_end; ++b) {
      SeqDesc& d = plan->seqs[b];
      d.unit0 = static_cast<int32_t>(units);
      units += static_cast<int64_t>(d.T) * d.NRB * d.S;
      maxRU = std::max(maxRU, std::min(d.RBS, d.R));
      shared_chunks = shared_chunks || d.T * d.NRB > 1;
      if (d.S > 1) {
        split_rows += d.T * d.R;
        max_s = std::max(max_s, d.S);
      }
    }
    // The grid merge needs every workgroup of the launch resident at once:
    // at most one per compute unit (the main kernels hold one workgroup per
    // CU).  A mode that cannot serve a launch falls back to the reduce kernel.
    const int64_t grid = (units + kNumXcd - 1) / kNumXcd * kNumXcd;
    const bool grid_fits = grid <= num_cus && grid <= kMaxArrivals;
    if (split_rows == 0)
      ln.merge = kMergeReduce;  // nothing to merge
    else if (merge_mode == MLA_MERGE_LAST_ARRIVER && max_s <= kMaxArrivals)
      ln.merge = kMergeLastArriver;
    else if (merge_mode == MLA_MERGE_GRID && grid_fits)
      ln.merge = kMergeGrid;
    else
      ln.merge = kMergeReduce;  // AUTO: on the MI355X both in-kernel merges measured slower
    if (units > std::numeric_limits<int32_t>::max() / 2) {
      set_error("too many work units (%lld)", static_cast<long long>(units));
      return MLA_ERR_INVALID_ARGUMENT;
    }
    // The non-temporal hint keeps KV lines out of the caches: right when every
    // chunk is read once; where the tiles of a sequence share chunks (one
    // XCD's L2 serves the rereads) it would send each reread to HBM.
    ln.kv_nt = !shared_chunks;
    ln.num_units = static_cast<int>(units);
    ln.nrt = ((maxRU + 1) / 2 + 15) / 16;
    ln.num_split_rows = split_rows;
    plan->num_units += ln.num_units;
    plan->launches.push_back(ln);
  }

  plan->total_part_rows = part_row;
  plan->num_split_tiles = split_tiles;
  plan->arrivals_offset = 0;
  plan->grid_words_offset = 0;
  if (part_row > 0) {
    const size_t lse_bytes = static_cast<size_t>(part_row) * sizeof(float);
    plan->part_o_offset = (lse_bytes + 255) / 256 * 256;
    plan->workspace_bytes = plan->part_o_offset + static_cast<size_t>(part_row) * kDv * sizeof(uint16_t);
    bool any_last = false, any_grid = false;
    for (const Launch& ln : plan->launches) {
      any_last = any_last || ln.merge == kMergeLastArriver;
      any_grid = any_grid || ln.merge == kMergeGrid;
    }
    if (any_last) {  // one 64-bit arrival word per partial row
      plan->arrivals_offset = (plan->workspace_bytes + 255) / 256 * 256;
      plan->workspace_bytes = plan->arrivals_offset + static_cast<size_t>(part_row) * 8;
    }
    if (any_grid) {  // one 64-bit counter per launch
      plan->grid_words_offset = (plan->workspace_bytes + 255) / 256 * 256;
      plan->workspace_bytes = plan->grid_words_offset + plan->launches.size() * 8;
    }
  } else {
    plan->part_o_offset = 0;
    plan->workspace_bytes = 0;
  }
  plan->table_offset = plan->reduce_table_offset = plan->row0_table_offset = 0;
  plan->reduce_seqs = 0;
  plan->table_blob.clear();
  if (plan->seq_table) {
    std::vector<SeqDesc> red;
    std::vector<int32_t> row0;
    int64_t rows = 0;
    for (const SeqDesc& d : plan->seqs) {
      if (d.S <= 1) continue;
      red.push_back(d);
      row0.push_back(static_cast<int32_t>(rows));
      rows += static_cast<int64_t>(d.T) * d.R;
    }
    plan->reduce_seqs = static_cast<int32_t>(red.size());
    const size_t main_bytes = plan->seqs.size() * sizeof(SeqDesc);
    plan->reduce_table_offset = (main_bytes + 255) / 256 * 256;
    plan->row0_table_offset =
        (plan->reduce_table_offset + red.size() * sizeof(SeqDesc) + 255) / 256 * 256;
    plan->table_blob.assign(plan->row0_table_offset + row0.size() * sizeof(int32_t), 0);
    std::memcpy(plan->table_blob.data(), plan->seqs.data(), main_bytes);
    if (!red.empty()) {
      std::memcpy(plan->table_blob.data() + plan->reduce_table_offset, red.data(),
                  red.size() * sizeof(SeqDesc));
      std::memcpy(plan->table_blob.data() + plan->row0_table_offset, row0.data(),
                  row0.size() * sizeof(int32_t));
    }
    plan->table_offset = (plan->workspace_bytes + 255) / 256 * 256;
    plan->workspace_bytes = plan->table_offset + plan->table_blob.size();
  }
  return MLA_OK;
}

}  // namespace mla
