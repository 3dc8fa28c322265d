// Host-plan driver for the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer, g++ only, no device code): builds plans over a
// sweep of head counts, verify widths, context lengths, ragged batches and
// forced options, both plan modes and every merge mode, and checks the plan's own invariants --
// the sequence order (a permutation of the caller's, with the caller's row
// offsets), the fold rule (largest divisor of q with H * F <= 128), the split
// rule (chunks of whole 64-key granules covering [0, n)), the unit and
// partial-row counts, each launch's merge kind, the workspace size -- so that any out-of-bounds access,
// overflow or uninitialised read in the planner surfaces under the
// sanitizers.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "plan.hpp"

#define CHECK(c)                                                                   \
  do {                                                                             \
    if (!(c)) {                                                                    \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);  \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

static unsigned g_state = 12345u;
static int next_int(int lo, int hi) {  // [lo, hi]
  g_state = g_state * 1664525u + 1013904223u;
  return lo + static_cast<int>((g_state >> 8) % static_cast<unsigned>(hi - lo + 1));
}

static void check_plan(const mla_plan& p, const std::vector<int32_t>& q, const std::vector<int32_t>& n,
                       int H, const int32_t* ce, int fold_cap, int num_cus, int merge_mode) {
  int64_t part_rows = 0, units = 0;
  const int batch = static_cast<int>(q.size());
  CHECK(static_cast<int>(p.seqs.size()) == batch && static_cast<int>(p.pos.size()) == batch);
  std::vector<int64_t> q_row0(batch), kv_row0(batch);
  for (int b = 0, qr = 0, kr = 0; b < batch; ++b) {
    q_row0[b] = qr;
    kv_row0[b] = kr;
    qr += q[b] * H;
    kr += n[b];
  }
  std::vector<int> seen(batch, 0);
  for (int i = 0; i < batch; ++i) {
    const mla::SeqDesc& d = p.seqs[i];
    CHECK(d.src >= 0 && d.src < batch && !seen[d.src]);
    seen[d.src] = 1;
    const int b = d.src;
    CHECK(p.pos[b] == i);
    CHECK(d.q_row0 == q_row0[b] && d.kv_row0 == kv_row0[b]);
    CHECK(d.F >= 1 && q[b] % d.F == 0 && H * d.F <= 128);
    for (int f = d.F + 1; f <= q[b]; ++f)  // the largest such divisor (up to the forced cap)
      CHECK(q[b] % f != 0 || H * f > 128 || (fold_cap > 0 && f > fold_cap));
    CHECK(d.T == q[b] / d.F && d.R == H * d.F);
    CHECK(d.L % 64 == 0 && d.L >= 64);
    CHECK(static_cast<int64_t>(d.S) * d.L >= n[b] && static_cast<int64_t>(d.S - 1) * d.L < n[b]);
    CHECK(d.n == n[b] && d.qlen == q[b]);
    CHECK(d.ce == (ce ? ce[b] : n[b]));
    CHECK(d.NRB >= 1 && d.RBS * d.NRB >= d.R && d.RBS <= 96);
    if (d.S > 1) {
      CHECK(d.part_row0 == part_rows);
      part_rows += static_cast<int64_t>(d.T) * d.S * d.R;
    } else {
      CHECK(d.part_row0 == -1);
    }
    units += static_cast<int64_t>(d.T) * d.NRB * d.S;
  }
  CHECK(p.total_part_rows == part_rows);
  CHECK(p.num_units == units);
  if (part_rows > 0) {
    CHECK(p.part_o_offset % 256 == 0 && p.part_o_offset >= static_cast<size_t>(part_rows) * 4);
    const size_t o_end = p.part_o_offset + static_cast<size_t>(part_rows) * 512 * 2;
    bool any_last = false, any_grid = false;
    for (const mla::Launch& ln : p.launches) {
      any_last = any_last || ln.merge == mla::kMergeLastArriver;
      any_grid = any_grid || ln.merge == mla::kMergeGrid;
    }
    size_t end = o_end;
    if (any_last) {
      CHECK(p.arrivals_offset % 256 == 0 && p.arrivals_offset >= end);
      end = p.arrivals_offset + static_cast<size_t>(part_rows) * 8;
    } else {
      CHECK(p.arrivals_offset == 0);
    }
    if (any_grid) {
      CHECK(p.grid_words_offset % 256 == 0 && p.grid_words_offset >= end);
      end = p.grid_words_offset + p.launches.size() * 8;
    } else {
      CHECK(p.grid_words_offset == 0);
    }
    if (!p.seq_table) CHECK(p.workspace_bytes == end);
  } else if (!p.seq_table) {
    CHECK(p.workspace_bytes == 0);
  }
  // more than kMaxSeqPerLaunch sequences: one launch, descriptor tables last
  // in the workspace (all sequences, the split ones, their first reduce rows)
  CHECK(p.seq_table == (batch > mla::kMaxSeqPerLaunch));
  CHECK(static_cast<int>(p.launches.size()) == 1);
  if (p.seq_table) {
    CHECK(p.table_offset % 256 == 0 && p.workspace_bytes == p.table_offset + p.table_blob.size());
    const mla::SeqDesc* all = reinterpret_cast<const mla::SeqDesc*>(p.table_blob.data());
    for (int i = 0; i < batch; ++i) CHECK(std::memcmp(&all[i], &p.seqs[i], sizeof(mla::SeqDesc)) == 0);
    const mla::SeqDesc* red =
        reinterpret_cast<const mla::SeqDesc*>(p.table_blob.data() + p.reduce_table_offset);
    const int32_t* row0 = reinterpret_cast<const int32_t*>(p.table_blob.data() + p.row0_table_offset);
    int k = 0;
    int64_t rows = 0;
    for (int i = 0; i < batch; ++i) {
      if (p.seqs[i].S <= 1) continue;
      CHECK(std::memcmp(&red[k], &p.seqs[i], sizeof(mla::SeqDesc)) == 0);
      CHECK(row0[k] == rows);
      rows += static_cast<int64_t>(p.seqs[i].T) * p.seqs[i].R;
      ++k;
    }
    CHECK(k == p.reduce_seqs);
    CHECK(p.row0_table_offset + sizeof(int32_t) * k == p.table_blob.size());
  }
  int covered = 0;
  for (const mla::Launch& ln : p.launches) {
    // merge kind: the requested one where it applies, else the reduce kernel
    const int64_t grid = (ln.num_units + 7) / 8 * 8;
    int max_s = 0;
    for (int i = ln.seq_begin; i < ln.seq_end; ++i) max_s = p.seqs[i].S > max_s ? p.seqs[i].S : max_s;
    int want = mla::kMergeReduce;
    if (ln.num_split_rows > 0) {
      if (merge_mode == MLA_MERGE_LAST_ARRIVER && max_s <= mla::kMaxArrivals)
        want = mla::kMergeLastArriver;
      else if (merge_mode == MLA_MERGE_GRID && grid <= num_cus)
        want = mla::kMergeGrid;
    }
    CHECK(ln.merge == want);
    bool shared = false;  // a chunk read by two units: no non-temporal KV hint
    for (int i = ln.seq_begin; i < ln.seq_end; ++i) shared = shared || p.seqs[i].T * p.seqs[i].NRB > 1;
    CHECK(ln.kv_nt == !shared);
    CHECK(ln.seq_begin == covered && ln.seq_end > ln.seq_begin);
    CHECK(p.seq_table || ln.seq_end - ln.seq_begin <= mla::kMaxSeqPerLaunch);
    CHECK(ln.nrt >= 1 && ln.nrt <= 3);
    covered = ln.seq_end;
  }
  CHECK(covered == static_cast<int>(q.size()));
}

int main() {
  int plans = 0;
  // single sequences: every H and q of the fold table, contexts around granules
  const int ctxs[] = {1, 2, 31, 63, 64, 65, 127, 4096, 4097, 125000, 131072, 1048576};
  for (int H = 1; H <= 128; H += (H < 16 ? 1 : 7)) {
    for (int qq = 1; qq <= 16; ++qq) {
      for (int c : ctxs) {
        if (c < qq) continue;
        for (int fs : {0, 1, 3, 256}) {
          std::vector<int32_t> q{qq}, n{c};
          mla_plan_options o{0, fs, 256, MLA_PLAN_AUTO, MLA_MERGE_AUTO};
          mla_plan p;
          CHECK(mla::build_plan(1, H, q.data(), n.data(), nullptr, MLA_KV_BF16, &o, &p) == MLA_OK);
          check_plan(p, q, n, H, nullptr, 0, 256, MLA_MERGE_AUTO);
          ++plans;
        }
      }
    }
  }
  // ragged batches, both dtypes, forced folds, more sequences than one launch holds
  for (int rep = 0; rep < 200; ++rep) {
    const int batch = next_int(1, 150);
    const int H = next_int(1, 128);
    std::vector<int32_t> q(batch), n(batch), ce(batch);
    for (int b = 0; b < batch; ++b) {
      q[b] = next_int(1, 16);
      n[b] = next_int(q[b], rep % 3 == 0 ? 40000 : 3000);
      ce[b] = next_int(1, n[b] + 5000);
    }
    mla_plan_options o{next_int(0, 4), next_int(0, 1) ? 0 : next_int(1, 70), next_int(1, 512),
                       next_int(0, 1), next_int(0, 3)};
    mla_plan p;
    const bool shard = rep % 4 == 1;
    CHECK(mla::build_plan(batch, H, q.data(), n.data(), shard ? ce.data() : nullptr,
                          rep % 2 ? MLA_KV_FP8_E4M3 : MLA_KV_BF16, &o, &p) == MLA_OK);
    check_plan(p, q, n, H, shard ? ce.data() : nullptr, o.force_fold, o.num_cus, o.merge_mode);
    ++plans;
  }
  // rejected shapes leave no trace
  {
    std::vector<int32_t> q{5}, n{4};
    mla_plan_options o{0, 0, 256};
    mla_plan p;
    CHECK(mla::build_plan(1, 12, q.data(), n.data(), nullptr, MLA_KV_BF16, &o, &p) ==
          MLA_ERR_INVALID_ARGUMENT);
    CHECK(mla::build_plan(1, 129, q.data(), n.data(), nullptr, MLA_KV_BF16, &o, &p) ==
          MLA_ERR_UNSUPPORTED);
  }
  std::printf("plan driver: %d plans ok\n", plans);
  return 0;
}
