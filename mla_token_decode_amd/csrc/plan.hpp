// Internal plan structures shared by the host plan and the kernel launchers.
// Not part of the public ABI (include/mla_decode.h is).
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <vector>

#include "mla_decode.h"

namespace mla {

constexpr int kDqk = MLA_DQK;            // 576 = 512 latent + 64 rope
constexpr int kDv = MLA_DV;              // 512
constexpr int kMaxRows = MLA_MAX_TILE_ROWS;  // 128
constexpr int kGranule = MLA_KV_GRANULE;     // 64 keys
constexpr int kMaxSeqPerLaunch = 60;     // sequence descriptors that travel in kernel arguments
constexpr int kMaxUnitRows = 96;         // rows one workgroup processes (2 groups x 3 MFMA tiles)
constexpr int kNumXcd = 8;               // MI355X: 8 XCDs, workgroups dealt round-robin
// Largest workspace mla_decode_run_static serves from its per-device array.
constexpr size_t kStaticScratchBytes = MLA_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevicesStatic = 64;

// One sequence as the kernels see it.  All counts fit int32 for any cache that
// fits in one GPU's HBM (row counts, not bytes); byte offsets are formed in
// 64-bit inside the kernels.
struct SeqDesc {
  int32_t q_row0;     // first Q/O/LSE row of the sequence: (sum of earlier q_len) * H
  int32_t kv_row0;    // first KV row of the sequence
  int32_t part_row0;  // first partial row in the workspace (-1 when the sequence is unsplit)
  int32_t n;          // kv_len
  int32_t qlen;       // q_len
  int32_t F;          // fold factor
  int32_t T;          // tiles = qlen / F
  int32_t R;          // rows per tile = H * F
  int32_t S;          // effective split count
  int32_t L;          // chunk length (keys, multiple of kGranule)
  int32_t NRB;        // row blocks per tile (tiles of more than 96 rows are cut)
  int32_t RBS;        // rows per row block (multiple of 16 unless NRB == 1)
  int32_t unit0;      // first work unit of the sequence within its launch
  int32_t ce;         // causal end: token i sees the keys j <= ce - qlen + i (ce = n normally)
  int32_t src;        // the caller's index of the sequence (its page-table row)
};

struct MainArgs {
  const uint16_t* q;
  const uint8_t* kv;
  uint16_t* o;
  float* lse;
  float* part_lse;     // [total partial rows]
  uint16_t* part_o;    // [total partial rows][512] bf16 (normalised partial O)
  float scale_log2;    // sm_scale * kv_scale * log2(e)
  float o_scale;       // kv_scale (fp8) or 1 (bf16)
  const int32_t* page_table;  // paged KV: [batch][pt_stride] page indices; null: contiguous KV
  int32_t pt_stride;
  int32_t page_shift;  // page size = 2^page_shift keys (paged only)
  int32_t num_pages;   // pages in the pool (entries are clamped to it)
  int32_t H;
  int32_t num_seqs;
  int32_t num_units;
  int32_t units_per_xcd;
  // merge_kind: a MergeKind; arrivals (last-arriver merge): one 64-bit word
  // per partial row (the counter of a split row block is the word of its
  // chunk 0, row 0); grid_word (grid merge): the launch's counter; epoch: this
  // call's tag in the high half of those words (never 0 or ~0);
  // num_split_rows: the launch's split output rows (grid merge)
  int32_t merge_kind;
  uint32_t epoch;
  unsigned long long* arrivals;
  unsigned long long* grid_word;
  int32_t num_split_rows;
  // plans of more than kMaxSeqPerLaunch sequences: the descriptors of all
  // num_seqs sequences in device memory (seqs[] unused); null otherwise
  const SeqDesc* seq_table;
  SeqDesc seqs[kMaxSeqPerLaunch];
};

struct ReduceArgs {
  const float* part_lse;
  const uint16_t* part_o;
  uint16_t* o;
  float* lse;
  int32_t H;
  int32_t num_seqs;
  int32_t num_rows;    // split rows covered by this launch
  int32_t max_splits;  // largest S among the launch's sequences (picks the merge layout)
  SeqDesc seqs[kMaxSeqPerLaunch];
  int32_t row0[kMaxSeqPerLaunch];  // first reduce row of each sequence in this launch
  // more than kMaxSeqPerLaunch split sequences: seqs and row0 in device memory
  // (the arrays above unused); null otherwise
  const SeqDesc* seq_table;
  const int32_t* row0_table;
};

struct MergeArgs {
  const uint16_t* o_shards;   // bf16 [num_shards][num_rows][512]
  const float* lse_shards;    // fp32 [num_shards][num_rows]
  uint16_t* o;                // bf16 [num_rows][512]
  float* lse;                 // fp32 [num_rows]
  int32_t num_rows;
  int32_t num_shards;
};

struct Launch {
  int seq_begin, seq_end;  // [begin, end) global sequence indices
  int num_units;
  int nrt;                 // 16-row MFMA tiles per row group (1..3), from the widest unit
  int num_split_rows;      // rows merged for this slice (by the reduce or in the kernel)
  int merge;               // MergeKind of this slice's split rows
  bool kv_nt;              // no KV chunk is read by two units: load KV with the non-temporal hint
};

// Who merges a launch's split rows: the reduce kernel (mla_decode_reduce),
// the last unit of each split row block to finish, or the whole grid of the
// main kernel after its last unit (MLA_MERGE_REDUCE / LAST_ARRIVER / GRID).
enum MergeKind : int32_t { kMergeReduce = 0, kMergeLastArriver = 1, kMergeGrid = 2 };

// Largest count an arrival word holds (its low 16 bits).
constexpr int kMaxArrivals = 65535;

}  // namespace mla

struct mla_plan {
  int32_t batch = 0;
  int32_t H = 0;
  mla_kv_dtype dtype = MLA_KV_BF16;
  int32_t num_cus = 0;
  std::vector<mla::SeqDesc> seqs;  // plan order; unit0 is relative to the sequence's launch
  std::vector<int32_t> pos;        // caller's sequence index -> index in seqs
  std::vector<mla::Launch> launches;
  int64_t total_part_rows = 0;
  int32_t num_units = 0;
  int32_t num_split_tiles = 0;
  size_t workspace_bytes = 0;
  size_t part_o_offset = 0;  // byte offset of partial O inside the workspace
  size_t arrivals_offset = 0;  // byte offset of the last-arriver merge's arrival words (0: none)
  size_t grid_words_offset = 0;  // byte offset of the grid merge's counters, one per launch (0: none)
  // More than kMaxSeqPerLaunch sequences: one launch, its descriptor tables in
  // the workspace at table_offset (mla_decode_run uploads table_blob there):
  // all sequences (plan order), then the split ones at reduce_table_offset,
  // then their first reduce rows at row0_table_offset (offsets in the blob).
  bool seq_table = false;
  size_t table_offset = 0;
  size_t reduce_table_offset = 0;
  size_t row0_table_offset = 0;
  int32_t reduce_seqs = 0;
  std::vector<uint8_t> table_blob;
  // a pinned host copy of table_blob, made by the first mla_decode_run that
  // needs it (so that the upload is an asynchronous copy) and freed with the
  // plan
  mutable std::mutex pinned_mu;
  mutable void* pinned_blob = nullptr;
};

namespace mla {
// Implemented in plan.cpp.
mla_status build_plan(int32_t batch, int32_t H, const int32_t* q_len, const int32_t* kv_len,
                      const int32_t* causal_end, mla_kv_dtype dtype,
                      const mla_plan_options* opts, mla_plan* plan);
void set_error(const char* fmt, ...);
int fold_factor(int H, int q, int cap);
void split_layout(int64_t n, int S, int G, int32_t* L, int32_t* S_eff);
}  // namespace mla
