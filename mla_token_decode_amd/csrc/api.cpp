// C ABI of libmla_decode.so: argument validation, device checks and kernel
// launches.  See include/mla_decode.h for the contract of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <random>

#include "plan.hpp"

namespace mla {
const char* last_error();
// nt: load the KV with the non-temporal hint (Launch::kv_nt)
hipError_t launch_main_contiguous(const MainArgs& a, int nrt, bool nt, hipStream_t stream);  // bf16 KV
hipError_t launch_main_paged(const MainArgs& a, int nrt, bool nt, hipStream_t stream);       // bf16 KV
hipError_t launch_fp8_contiguous(const MainArgs& a, int nrt, bool nt, hipStream_t stream);
hipError_t launch_fp8_paged(const MainArgs& a, int nrt, bool nt, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t static_scratch(void** ptr);

namespace {

constexpr int kMaxDevices = 64;

// Tags of the in-kernel merge's arrival words: one per main-kernel call,
// never 0 or 0xffffffff, so that a zeroed or 0xff-filled workspace (or the
// words another call left) holds no arrival of this call.  The sequence
// starts at a random point in each process.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{static_cast<uint32_t>(std::random_device{}())};
  uint32_t e;
  do {
    e = counter.fetch_add(1, std::memory_order_relaxed) + 1u;
  } while (e == 0u || e == 0xffffffffu);
  return e;
}

std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
int g_dev_cus[kMaxDevices];

// Checks that the current device is a gfx950 and returns its CU count.
mla_status current_device(int* cus) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    set_error("hipGetDevice failed: %s", hipGetErrorString(e));
    return MLA_ERR_DEVICE;
  }
  if (dev >= kMaxDevices) {
    set_error("device index %d out of range", dev);
    return MLA_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      set_error("hipGetDeviceProperties failed: %s", hipGetErrorString(e));
      return MLA_ERR_DEVICE;
    }
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_cus[dev] = prop.multiProcessorCount;
  }
  if (g_dev_state[dev] != 1) {
    set_error("device %d is not gfx950; this library only carries gfx950 code", dev);
    return MLA_ERR_UNSUPPORTED;
  }
  if (cus) *cus = g_dev_cus[dev];
  return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The pinned host copy of a large plan's descriptor tables, the source of the
// upload that every run enqueues.  Made once under the plan's lock: by plan
// creation, or, when that could not make it, by the first run allowed to
// allocate.  A failed allocation leaves HIP's error state clear, so that it
// is not reported by a later launch check.
hipError_t pinned_tables(const mla_plan* p, bool may_allocate, const void** out) {
  std::lock_guard<std::mutex> lk(p->pinned_mu);
  if (!p->pinned_blob && may_allocate) {
    void* ptr = nullptr;
    const hipError_t e = hipHostMalloc(&ptr, p->table_blob.size(), hipHostMallocDefault);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e;
    }
    std::memcpy(ptr, p->table_blob.data(), p->table_blob.size());
    p->pinned_blob = ptr;
  }
  *out = p->pinned_blob;
  return hipSuccess;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

static mla_status plan_common(int32_t batch, int32_t num_heads, const int32_t* q_len,
                              const int32_t* kv_len, const int32_t* causal_end,
                              mla_kv_dtype kv_dtype, const mla_plan_options* opts,
                              mla_plan** plan_out, size_t* workspace_bytes_out) {
  if (!plan_out) {
    set_error("plan_out must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  *plan_out = nullptr;
  mla_plan_options o{};
  if (opts) o = *opts;
  if (o.num_cus == 0) {
    int cus = 0;
    mla_status st = current_device(&cus);
    if (st != MLA_OK) return st;
    o.num_cus = cus;
  }
  mla_plan* p = new (std::nothrow) mla_plan();
  if (!p) {
    set_error("out of host memory");
    return MLA_ERR_OUT_OF_MEMORY;
  }
  mla_status st;
  try {  // the plan's tables are host vectors: no exception may leave the C ABI
    st = build_plan(batch, num_heads, q_len, kv_len, causal_end, kv_dtype, &o, p);
  } catch (const std::bad_alloc&) {
    set_error("out of host memory building the plan");
    st = MLA_ERR_OUT_OF_MEMORY;
  }
  if (st != MLA_OK) {
    delete p;
    return st;
  }
  if (p->seq_table) {  // made here when possible, so that no run needs to allocate
    const void* unused = nullptr;
    (void)pinned_tables(p, true, &unused);
  }
  *plan_out = p;
  if (workspace_bytes_out) *workspace_bytes_out = p->workspace_bytes;
  return MLA_OK;
}

mla_status mla_decode_plan(int32_t batch, int32_t num_heads, const int32_t* q_len,
                           const int32_t* kv_len, mla_kv_dtype kv_dtype,
                           const mla_plan_options* opts, mla_plan** plan_out,
                           size_t* workspace_bytes_out) {
  return plan_common(batch, num_heads, q_len, kv_len, nullptr, kv_dtype, opts, plan_out,
                     workspace_bytes_out);
}

mla_status mla_decode_plan_shard(int32_t batch, int32_t num_heads, const int32_t* q_len,
                                 const int32_t* kv_len, const int32_t* causal_end,
                                 mla_kv_dtype kv_dtype, const mla_plan_options* opts,
                                 mla_plan** plan_out, size_t* workspace_bytes_out) {
  if (!causal_end) {
    if (plan_out) *plan_out = nullptr;
    set_error("causal_end must be a non-null host array");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  return plan_common(batch, num_heads, q_len, kv_len, causal_end, kv_dtype, opts, plan_out,
                     workspace_bytes_out);
}

void mla_plan_destroy(mla_plan* plan) {
  if (plan && plan->pinned_blob) (void)hipHostFree(plan->pinned_blob);
  delete plan;
}

const char* mla_last_error(void) { return mla::last_error(); }

mla_status mla_plan_order(const mla_plan* plan, int32_t* order) {
  if (!plan || !order) {
    set_error("plan and order must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  for (int32_t i = 0; i < plan->batch; ++i) order[i] = plan->seqs[i].src;
  return MLA_OK;
}

mla_status mla_plan_query(const mla_plan* plan, int32_t seq, int32_t* fold, int32_t* tiles,
                          int32_t* splits, int32_t* chunk_len) {
  if (!plan) {
    set_error("plan must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (seq < 0 || seq >= plan->batch) {
    set_error("sequence index %d out of range [0, %d)", seq, plan->batch);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  const SeqDesc& d = plan->seqs[plan->pos[seq]];
  if (fold) *fold = d.F;
  if (tiles) *tiles = d.T;
  if (splits) *splits = d.S;
  if (chunk_len) *chunk_len = d.L;
  return MLA_OK;
}

mla_status mla_plan_info(const mla_plan* plan, int32_t* num_units, int32_t* num_split_tiles,
                         int32_t* num_launches, size_t* workspace_bytes) {
  if (!plan) {
    set_error("plan must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (num_units) *num_units = plan->num_units;
  if (num_split_tiles) *num_split_tiles = plan->num_split_tiles;
  if (num_launches) *num_launches = static_cast<int32_t>(plan->launches.size());
  if (workspace_bytes) *workspace_bytes = plan->workspace_bytes;
  return MLA_OK;
}

mla_status mla_plan_launch_info(const mla_plan* plan, int32_t launch, int32_t* num_units,
                                int32_t* merge_mode) {
  if (!plan || launch < 0 || launch >= static_cast<int32_t>(plan->launches.size())) {
    set_error("need a plan and 0 <= launch < its launch count (got %d)", launch);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  const Launch& ln = plan->launches[launch];
  if (num_units) *num_units = ln.num_units;
  if (merge_mode) {
    *merge_mode = ln.num_split_rows == 0          ? 0
                  : ln.merge == kMergeGrid        ? MLA_MERGE_GRID
                  : ln.merge == kMergeLastArriver ? MLA_MERGE_LAST_ARRIVER
                                                  : MLA_MERGE_REDUCE;
  }
  return MLA_OK;
}

namespace {

mla_status reduce_launch(const mla_plan* plan, const Launch& ln, const void* workspace, void* o,
                         float* lse, void* stream);

// Shared by the contiguous and the paged entry points: `kv` is the KV array or
// the page pool; `page_table` is null for contiguous KV.
// may_allocate: whether a large plan without its pinned tables may make them
// here (not for mla_decode_run_static).
mla_status run_common(const mla_plan* plan, const void* q, const void* kv, const int32_t* page_table,
                      int32_t pt_stride, int32_t page_shift, int32_t num_pages, float sm_scale,
                      float kv_scale, void* o, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream, bool may_allocate) {
  if (!plan) {
    set_error("plan must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!q || !kv || !o || !lse) {
    set_error("q, kv, o and lse must be non-null device pointers");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o) || !aligned16(lse)) {
    set_error("q, kv, o and lse must be 16-byte aligned");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) {
    set_error("sm_scale must be finite and > 0 (got %g)", static_cast<double>(sm_scale));
    return MLA_ERR_INVALID_ARGUMENT;
  }
  const bool fp8 = plan->dtype == MLA_KV_FP8_E4M3;
  if (fp8 && (!(kv_scale > 0.0f) || !std::isfinite(kv_scale))) {
    set_error("fp8 kv_scale must be finite and > 0 (got %g)", static_cast<double>(kv_scale));
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!fp8 && kv_scale != 1.0f) {
    set_error("bf16 KV takes kv_scale == 1 (got %g)", static_cast<double>(kv_scale));
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < plan->workspace_bytes) {
    set_error("workspace of %zu bytes is smaller than the planned %zu", workspace_bytes,
              plan->workspace_bytes);
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  if (plan->workspace_bytes > 0 && (!workspace || !aligned16(workspace))) {
    set_error("this plan needs a 16-byte aligned workspace of %zu bytes", plan->workspace_bytes);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  int dev_cus = 0;
  mla_status st = current_device(&dev_cus);
  if (st != MLA_OK) return st;

  MainArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.part_lse = plan->total_part_rows ? static_cast<float*>(workspace) : nullptr;
  a.part_o = plan->total_part_rows
                 ? reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + plan->part_o_offset)
                 : nullptr;
  const double log2e = 1.4426950408889634;
  a.scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * (fp8 ? kv_scale : 1.0) * log2e);
  a.o_scale = fp8 ? kv_scale : 1.0f;
  a.pt_stride = pt_stride;
  a.page_shift = page_shift;
  a.num_pages = num_pages;
  a.H = plan->H;
  a.epoch = next_epoch();
  a.arrivals = plan->arrivals_offset
                   ? reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) +
                                                           plan->arrivals_offset)
                   : nullptr;
  unsigned long long* grid_words =
      plan->grid_words_offset
          ? reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + plan->grid_words_offset)
          : nullptr;
  if (plan->seq_table) {  // the descriptor tables of a large plan, into the workspace
    const void* src = nullptr;
    const hipError_t pe = pinned_tables(plan, may_allocate, &src);
    if (pe != hipSuccess) {
      set_error("pinned host buffer for the descriptor tables failed: %s", hipGetErrorString(pe));
      return MLA_ERR_DEVICE;
    }
    if (!src) {
      set_error("the plan has no pinned host buffer for its descriptor tables (its creation could "
                "not make one) and mla_decode_run_static allocates nothing; run the plan once with "
                "mla_decode_run first");
      return MLA_ERR_DEVICE;
    }
    char* tab = static_cast<char*>(workspace) + plan->table_offset;
    hipError_t e = hipMemcpyAsync(tab, src, plan->table_blob.size(), hipMemcpyHostToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
      set_error("descriptor table upload failed: %s", hipGetErrorString(e));
      return MLA_ERR_DEVICE;
    }
    a.seq_table = reinterpret_cast<const SeqDesc*>(tab);
  }
  for (size_t li = 0; li < plan->launches.size(); ++li) {
    const Launch& ln = plan->launches[li];
    // The grid merge needs the launch's workgroups resident at once; on a
    // device with fewer CUs than the plan assumed, the reduce kernel merges
    // this launch's split rows right after it instead.
    const int grid = (ln.num_units + kNumXcd - 1) / kNumXcd * kNumXcd;
    const bool reduce_here = ln.merge == kMergeGrid && grid > dev_cus;
    a.merge_kind = reduce_here ? kMergeReduce : ln.merge;
    a.grid_word = ln.merge == kMergeGrid ? grid_words + li : nullptr;
    a.num_split_rows = ln.num_split_rows;
    a.num_seqs = ln.seq_end - ln.seq_begin;
    a.num_units = ln.num_units;
    a.units_per_xcd = (ln.num_units + kNumXcd - 1) / kNumXcd;
    a.page_table = page_table;  // a sequence's row is its SeqDesc::src (the caller's index)
    if (!plan->seq_table)
      for (int b = ln.seq_begin; b < ln.seq_end; ++b) a.seqs[b - ln.seq_begin] = plan->seqs[b];
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool nt = ln.kv_nt;
    hipError_t e = fp8 ? (page_table ? launch_fp8_paged(a, ln.nrt, nt, s)
                                     : launch_fp8_contiguous(a, ln.nrt, nt, s))
                       : (page_table ? launch_main_paged(a, ln.nrt, nt, s)
                                     : launch_main_contiguous(a, ln.nrt, nt, s));
    if (e != hipSuccess) {
      set_error("main kernel launch failed: %s", hipGetErrorString(e));
      return MLA_ERR_DEVICE;
    }
    if (reduce_here) {
      st = reduce_launch(plan, ln, workspace, o, lse, stream);
      if (st != MLA_OK) return st;
    }
  }
  return MLA_OK;
}

}  // namespace

mla_status mla_decode_run(const mla_plan* plan, const void* q, const void* kv, float sm_scale,
                          float kv_scale, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return run_common(plan, q, kv, nullptr, 0, 0, 0, sm_scale, kv_scale, o, lse, workspace,
                    workspace_bytes, stream, true);
}

mla_status mla_decode_run_paged(const mla_plan* plan, const void* q, const void* kv_pages,
                                int32_t num_pages, int32_t page_size, const int32_t* page_table,
                                int32_t page_table_stride, float sm_scale, float kv_scale, void* o,
                                float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!plan) {
    set_error("plan must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (page_size < MLA_MIN_PAGE_SIZE || page_size > MLA_MAX_PAGE_SIZE ||
      (page_size & (page_size - 1)) != 0) {
    set_error("page_size %d is not supported: pages hold a power of two from %d to %d keys",
              page_size, MLA_MIN_PAGE_SIZE, MLA_MAX_PAGE_SIZE);
    return MLA_ERR_UNSUPPORTED;
  }
  if (num_pages < 1) {
    set_error("num_pages must be >= 1 (got %d)", num_pages);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!page_table || reinterpret_cast<uintptr_t>(page_table) % 4 != 0) {
    set_error("page_table must be a non-null, 4-byte aligned device pointer");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  int64_t need = 1;
  for (const SeqDesc& d : plan->seqs) need = std::max<int64_t>(need, (d.n + page_size - 1) / page_size);
  if (page_table_stride < need) {
    set_error("page_table_stride %d is smaller than the %lld pages of the longest sequence",
              page_table_stride, static_cast<long long>(need));
    return MLA_ERR_INVALID_ARGUMENT;
  }
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  return run_common(plan, q, kv_pages, page_table, page_table_stride, shift, num_pages, sm_scale,
                    kv_scale, o, lse, workspace, workspace_bytes, stream, true);
}

namespace {

// The reduce kernel over one launch's split rows.
mla_status reduce_launch(const mla_plan* plan, const Launch& ln, const void* workspace, void* o,
                         float* lse, void* stream) {
  ReduceArgs a;
  std::memset(&a, 0, sizeof a);
  a.part_lse = static_cast<const float*>(workspace);
  a.part_o =
      reinterpret_cast<const uint16_t*>(static_cast<const char*>(workspace) + plan->part_o_offset);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.H = plan->H;
  int ns = 0, rows = 0, smax = 0;
  for (int b = ln.seq_begin; b < ln.seq_end; ++b) {
    const SeqDesc& d = plan->seqs[b];
    if (d.S <= 1) continue;
    if (!plan->seq_table) {
      a.seqs[ns] = d;
      a.row0[ns] = rows;
    }
    rows += d.T * d.R;
    smax = d.S > smax ? d.S : smax;
    ++ns;
  }
  if (plan->seq_table) {  // uploaded by mla_decode_run into the same workspace
    const char* tab = static_cast<const char*>(workspace) + plan->table_offset;
    a.seq_table = reinterpret_cast<const SeqDesc*>(tab + plan->reduce_table_offset);
    a.row0_table = reinterpret_cast<const int32_t*>(tab + plan->row0_table_offset);
  }
  a.num_seqs = ns;
  a.num_rows = rows;
  a.max_splits = smax;
  hipError_t e = launch_reduce(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_error("reduce kernel launch failed: %s", hipGetErrorString(e));
    return MLA_ERR_DEVICE;
  }
  return MLA_OK;
}

// The reduce kernel over every launch whose split rows the main kernel left
// to it.
mla_status reduce_common(const mla_plan* plan, const void* workspace, void* o, float* lse,
                         void* stream) {
  for (const Launch& ln : plan->launches) {
    if (ln.num_split_rows == 0 || ln.merge != kMergeReduce) continue;  // nothing left to merge
    mla_status st = reduce_launch(plan, ln, workspace, o, lse, stream);
    if (st != MLA_OK) return st;
  }
  return MLA_OK;
}

}  // namespace

mla_status mla_decode_reduce(const mla_plan* plan, const void* workspace, void* o, float* lse,
                             void* stream) {
  if (!plan) {
    set_error("plan must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (plan->total_part_rows == 0) return MLA_OK;
  if (!workspace || !o || !lse) {
    set_error("workspace, o and lse must be non-null device pointers");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(workspace) || !aligned16(o) || !aligned16(lse)) {
    set_error("workspace, o and lse must be 16-byte aligned");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  mla_status st = current_device(nullptr);
  if (st != MLA_OK) return st;
  return reduce_common(plan, workspace, o, lse, stream);
}

mla_status mla_decode_run_static(const mla_plan* plan, const void* q, const void* kv,
                                 float sm_scale, float kv_scale, void* o, float* lse,
                                 void* stream) {
  if (!plan) {
    set_error("plan must be non-null");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (plan->workspace_bytes > kStaticScratchBytes) {
    set_error("plan needs a %zu-byte workspace; mla_decode_run_static holds %zu bytes (use "
              "mla_decode_run with a caller workspace, or fewer split chunks)",
              plan->workspace_bytes, static_cast<size_t>(kStaticScratchBytes));
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  mla_status st = current_device(nullptr);
  if (st != MLA_OK) return st;
  void* ws = nullptr;
  if (plan->workspace_bytes > 0) {
    hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) {
      set_error("static workspace lookup failed: %s", hipGetErrorString(e));
      return MLA_ERR_DEVICE;
    }
  }
  st = run_common(plan, q, kv, nullptr, 0, 0, 0, sm_scale, kv_scale, o, lse, ws,
                  plan->workspace_bytes, stream, false);
  if (st != MLA_OK || plan->total_part_rows == 0) return st;
  return reduce_common(plan, ws, o, lse, stream);
}

mla_status mla_merge_shards(int32_t num_rows, int32_t num_shards, const void* o_shards,
                            const float* lse_shards, void* o, float* lse, void* stream) {
  if (num_rows < 1 || num_shards < 1 || num_shards > MLA_MAX_SHARDS) {
    set_error("need num_rows >= 1 and 1 <= num_shards <= %d (got %d, %d)", MLA_MAX_SHARDS,
              num_rows, num_shards);
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!o_shards || !lse_shards || !o || !lse) {
    set_error("o_shards, lse_shards, o and lse must be non-null device pointers");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(o_shards) || !aligned16(lse_shards) || !aligned16(o) || !aligned16(lse)) {
    set_error("o_shards, lse_shards, o and lse must be 16-byte aligned");
    return MLA_ERR_INVALID_ARGUMENT;
  }
  mla_status st = current_device(nullptr);
  if (st != MLA_OK) return st;
  MergeArgs a;
  a.o_shards = static_cast<const uint16_t*>(o_shards);
  a.lse_shards = lse_shards;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.num_rows = num_rows;
  a.num_shards = num_shards;
  hipError_t e = launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_error("merge kernel launch failed: %s", hipGetErrorString(e));
    return MLA_ERR_DEVICE;
  }
  return MLA_OK;
}

}  // extern "C"
