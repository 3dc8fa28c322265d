// Device helpers shared by the decode kernels (bf16 / fp8 KV main kernels and
// the merges): vector types, buffer descriptors, wave reductions, the fp8 Q
// scale rule and the work-unit decoding of the launch arguments.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "plan.hpp"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr unsigned kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer: range-checked, zero on OOB

// fp8 Q: a row's largest |q| maps to the e4m3 maximum 448.  The fp32
// rounding of 448 / M and of q * (448 / M) can put a value up to 2 ulps above
// 448; the gfx950 conversion rounds to nearest before it saturates (inputs up
// to 463 give 448, checked on the MI355X), so no clamp is needed there.
constexpr float kQ8Top = 448.0f;

// 1 / s for a row whose largest |q| (the scale rule's M) is M, s = M / 448.
// Below 2^-100 (a zero row, or values near the bottom of the fp32 range, where
// 448 / M would overflow to +inf and turn the row into NaN) 1 / s stays at
// 448 * 2^100: q / s is then finite and far inside the e4m3 range, and the
// row's scores (all below 2^-100 in size) give a near-uniform softmax.  The
// row's softmax constant is scale_log2 / inv_s in both cases.
__device__ __forceinline__ float q8_inv_scale(float M) {
  return M > 0x1p-100f ? kQ8Top / M : kQ8Top * 0x1p100f;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}

// A pointer every lane agrees on, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// Workgroup barrier that orders LDS traffic only (global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with
// the gfx950 lane-swap instructions: permlane16_swap exchanges the odd 16-lane
// rows of one operand with the even rows of the other, permlane32_swap the
// upper half with the lower half; feeding the same value to both operands and
// combining the two results gives every lane the value of its partner.
// Maxima of values that are never NaN, as plain instructions: fmaxf would
// first quiet possible signalling NaNs of operands the compiler cannot see the
// origin of (inline-assembly results), one extra instruction per operand.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float wave_max_across_groups(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = max2(__builtin_bit_cast(float, (unsigned)r16[0]), __builtin_bit_cast(float, (unsigned)r16[1]));
  const unsigned w = __builtin_bit_cast(unsigned, v);
  auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return max2(__builtin_bit_cast(float, (unsigned)r32[0]), __builtin_bit_cast(float, (unsigned)r32[1]));
}

__device__ __forceinline__ float wave_sum_across_groups(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (unsigned)r16[0]) + __builtin_bit_cast(float, (unsigned)r16[1]);
  const unsigned w = __builtin_bit_cast(unsigned, v);
  auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_bit_cast(float, (unsigned)r32[0]) + __builtin_bit_cast(float, (unsigned)r32[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  uint16_t xu = __builtin_bit_cast(uint16_t, x), yu = __builtin_bit_cast(uint16_t, y);
  return (uint32_t)xu | ((uint32_t)yu << 16);
}

// Compile-time loop helper.
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

struct UnitCtx {
  int lo, nkeys, ntiles, min_lim;
};

// Everything a unit needs, copied out of the launch arguments (all fields are
// workgroup-uniform).
struct UnitSetup {
  UnitCtx uc;
  int t, s, R, H, S, rowb0, RU, row0, tail0, hi_eff, part_row0;
  float scale_log2, o_scale;
  const uint16_t* q;
  const uint8_t* kv_unit;  // contiguous KV: first row of the unit's chunk; paged: the pool
  const int32_t* pt_row;   // paged KV: the sequence's page-table row (null: contiguous)
  int page_shift, last_page_idx, num_pages;
  uint16_t* o;
  float* lse;
  float* part_lse;
  uint16_t* part_o;
};

// Entry b (wave-uniform) of a descriptor table in device memory, moved to
// scalar registers (its fields feed buffer descriptors and scalar loops).
__device__ __forceinline__ SeqDesc uniform_desc(const SeqDesc* table, int b) {
  SeqDesc d = table[b];
  static_assert(sizeof(SeqDesc) % 4 == 0, "SeqDesc is made of 32-bit fields");
  int* w = reinterpret_cast<int*>(&d);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(SeqDesc) / 4); ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
  return d;
}

// The last index i in [0, n) with key(i) <= x, for keys that ascend with
// key(0) <= x: a binary search (x wave-uniform, so every probe is one scalar
// load).
template <class Key>
__device__ __forceinline__ int last_at_or_below(int n, int x, Key key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (key(mid) <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Descriptor of sequence b (wave-uniform) of the launch: from the kernel
// arguments, or from the device table of a large plan.
__device__ __forceinline__ SeqDesc seq_desc(const MainArgs& args, int b) {
  if (!args.seq_table) return args.seqs[b];
  return uniform_desc(args.seq_table, b);
}

// The sequence that holds work unit u (wave-uniform): the last one whose
// first unit is <= u (first units ascend in plan order; every sequence has at
// least one unit).
__device__ __forceinline__ int seq_of_unit(const MainArgs& args, int u) {
  if (args.seq_table)
    return last_at_or_below(args.num_seqs, u, [&](int i) {
      return __builtin_amdgcn_readfirstlane(args.seq_table[i].unit0);
    });
  return last_at_or_below(args.num_seqs, u, [&](int i) { return args.seqs[i].unit0; });
}

// ROW_BYTES: bytes of one KV row in memory (1152 bf16, 576 fp8); TILE_KEYS:
// keys per compute tile of the kernel (uc.ntiles counts those).
template <int ROW_BYTES, int TILE_KEYS>
__device__ __forceinline__ bool unit_setup(const MainArgs& args, UnitSetup& us) {
  const int p = blockIdx.x;
  const int u = (p % kNumXcd) * args.units_per_xcd + p / kNumXcd;  // XCD-aware order
  if (u >= args.num_units) return false;
  const SeqDesc sd = seq_desc(args, seq_of_unit(args, u));
  const int v = u - sd.unit0;
  const int per_chunk = sd.T * sd.NRB;  // units sharing one KV chunk are consecutive
  us.s = v / per_chunk;
  us.t = (v % per_chunk) / sd.NRB;
  const int rb = v % sd.NRB;
  us.R = sd.R;
  us.H = args.H;
  us.S = sd.S;
  us.part_row0 = sd.part_row0;
  us.scale_log2 = args.scale_log2;
  us.o_scale = args.o_scale;
  us.q = args.q;
  us.o = args.o;
  us.lse = args.lse;
  us.part_lse = args.part_lse;
  us.part_o = args.part_o;
  us.rowb0 = rb * sd.RBS;                          // first tile row of this unit
  us.RU = min(sd.RBS, us.R - us.rowb0);            // rows of this unit
  us.row0 = sd.q_row0 + us.t * us.R + us.rowb0;    // first Q/O row of this unit
  us.uc.lo = us.s * sd.L;
  const int hi = min(us.uc.lo + sd.L, sd.n);
  us.tail0 = sd.ce - sd.qlen + us.t * sd.F;        // tile row r sees keys <= tail0 + r / H
  const int vis_lo = us.tail0 + us.rowb0 / us.H;   // every unit row sees keys <= vis_lo
  const int vis_hi = us.tail0 + (us.rowb0 + us.RU - 1) / us.H;
  us.hi_eff = min(hi, vis_hi + 1);                 // no unit row sees keys >= hi_eff
  us.uc.nkeys = us.hi_eff - us.uc.lo;              // may be <= 0 (chunk hidden from every row)
  us.uc.ntiles = us.uc.nkeys > 0 ? (us.uc.nkeys + TILE_KEYS - 1) / TILE_KEYS : 0;
  us.uc.min_lim = min(us.hi_eff - 1, vis_lo) - us.uc.lo;  // every row sees keys <= this
  if (args.page_table == nullptr) {
    us.pt_row = nullptr;
    us.kv_unit = args.kv + ((int64_t)sd.kv_row0 + us.uc.lo) * ROW_BYTES;
  } else {
    us.pt_row = args.page_table + (int64_t)sd.src * args.pt_stride;
    us.kv_unit = args.kv;
    us.page_shift = args.page_shift;
    us.last_page_idx = (sd.n - 1) >> args.page_shift;
    us.num_pages = args.num_pages;
  }
  return true;
}

// Arrival counter of an in-kernel merge: one 64-bit word per counted group,
// holding the call's epoch (bits 63..32, never 0 or ~0), a generation (31..16)
// and the arrivals of the current generation (15..0).  A word that holds
// another epoch belongs to an earlier call (or is the workspace's prior
// contents): the first arrival of this call claims it (compare-and-swap to
// generation 0 with one arrival); every other arrival is one fetch-and-add,
// so arrivals that come together do not retry against each other.  The
// arrival that brings the count to `expected` (<= 65535) swaps in the next
// generation with a zero count, so a replay with the same epoch (a captured
// graph launches with the same arguments) counts again from zero.  Returns
// the generation this arrival belongs to; *last says whether it completed it.
// Every update is a read-modify-write, so the chain of them carries each
// arrival's release to whoever reads the word later.
__device__ __forceinline__ unsigned arrive(unsigned long long* w, uint32_t epoch, unsigned expected,
                                           bool* last) {
  const unsigned long long tag = (unsigned long long)epoch << 32;
  unsigned long long old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool claimed = false;
  while ((uint32_t)(old >> 32) != epoch) {  // ends: a failed swap means the word changed
    const unsigned long long prev = atomicCAS(w, old, tag | 1ull);
    if (prev == old) {
      claimed = true;
      break;
    }
    old = prev;
  }
  if (claimed)
    old = tag;  // this arrival is the call's first: generation 0, none before it
  else
    old = __hip_atomic_fetch_add(w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned gen = (unsigned)(old >> 16) & 0xffffu;
  const unsigned cnt = (unsigned)old & 0xffffu;
  *last = cnt + 1u >= expected;
  if (*last)
    __hip_atomic_exchange(w, tag | ((unsigned long long)((gen + 1u) & 0xffffu) << 16), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  return gen;
}

// Split-KV fold of one split output row over its S chunks, for one block of
// its 512 value columns, by 256 threads in P chunk phases x G = 256 / P column
// groups (P = 4, 8, 16 or 32; the block holds C = 8 G columns): thread
// (part p = tid / G, group cg = tid % G) owns columns 8 cg .. 8 cg + 7 of the
// block (one 16-byte load per chunk) and folds chunks p, p + P, ... in
// ascending order, eight at a time with their loads in flight together,
// against the running maximum of the LSEs it has read (its sums are rescaled
// when that maximum moves).  The P per-part results are combined in a fixed
// order (a butterfly over the parts that one wave holds, then the four waves
// in wave order through LDS), so the result does not depend on timing.  A chunk that
// shows the row no key has LSE = -inf and weight 0; a row no chunk shows a key
// gets O = 0, LSE = -inf.  Partial row of chunk s: pbase + s * R.  Every thread
// of the block calls it; it ends with the LDS free again.
constexpr int kFoldThreads = 256;
constexpr int kFoldBatch = 8;  // chunk loads in flight per thread

// Chunk phases for a launch whose sequences have at most smax chunks: the
// fewest that keep every thread within one batch of loads (up to 256 chunks).
// P = 1 is its own layout (fold_cols8: four rows per block, no LDS).
__host__ __device__ constexpr int fold_parts(int smax) {
  return smax <= kFoldBatch ? 1 : smax <= 32 ? 4 : smax <= 64 ? 8 : smax <= 128 ? 16 : 32;
}
template <int P>
constexpr int fold_cols() { return 8 * (kFoldThreads / P); }  // value columns per block (P >= 4)
constexpr int kFoldRowsP1 = kFoldThreads / (kDv / 8);         // rows per block with P = 1

constexpr int kFoldWaves = kFoldThreads / 64;
struct FoldLds {
  f32x4 acc[kFoldWaves][64][2];  // per wave: the sums of each column group
  float w[kFoldWaves], m[kFoldWaves];
};

__device__ __forceinline__ float merge_weight(float ls, float M) {
  return ls == -INFINITY ? 0.0f : __expf(ls - M);
}

// Folds (mo, Wo, b0, b1) into (m, W, a0, a1): two folds of the same columns,
// each a running maximum, its weight sum and its weighted sums, rescaled to
// their common maximum.
__device__ __forceinline__ void fold_pair(float& m, float& W, f32x4& a0, f32x4& a1, float mo,
                                          float Wo, const f32x4& b0, const f32x4& b1) {
  const float M = fmaxf(m, mo);
  const float f = merge_weight(m, M), g = merge_weight(mo, M);
  a0 = f * a0 + g * b0;
  a1 = f * a1 + g * b1;
  W = f * W + g * Wo;
  m = M;
}

// 4 bf16 (two dwords, element 0 in the low half of the first) -> fp32, exact.
__device__ __forceinline__ f32x4 bf16x4_to_f32(uint2 pk) {
  return f32x4{__builtin_bit_cast(float, pk.x << 16), __builtin_bit_cast(float, pk.x & 0xffff0000u),
               __builtin_bit_cast(float, pk.y << 16), __builtin_bit_cast(float, pk.y & 0xffff0000u)};
}

// 8 bf16 (one 16-byte load) -> two fp32 quads, exact.
__device__ __forceinline__ void bf16x8_to_f32(const u32x4& pk, f32x4& lo, f32x4& hi) {
  lo = bf16x4_to_f32(uint2{pk[0], pk[1]});
  hi = bf16x4_to_f32(uint2{pk[2], pk[3]});
}

template <int P>
__device__ __forceinline__ void fold_split_row(const float* part_lse, const uint16_t* part_o,
                                               int64_t pbase, int S, int R, int cb,
                                               uint16_t* o_row, float* lse_out, FoldLds& lds) {
  constexpr int G = kFoldThreads / P, C = fold_cols<P>();
  const int part = threadIdx.x / G;
  const int cg = threadIdx.x % G;
  float m = -INFINITY, W = 0.0f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* po = part_o + C * cb + 8 * cg;
  for (int s0 = part; s0 < S; s0 += kFoldBatch * P) {
    float ls[kFoldBatch];
    u32x4 v[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      const int s = s0 + i * P;
      if (s < S) {
        const int64_t prow = pbase + (int64_t)s * R;
        ls[i] = part_lse[prow];
        v[i] = *(const u32x4*)(po + prow * kDv);
      } else {
        ls[i] = -INFINITY;
        v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float mn = m;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) mn = fmaxf(mn, ls[i]);
    // sums so far are 0 while m = -inf; exp(-inf) = 0 covers a first finite mn
    const float sc = mn == -INFINITY ? 1.0f : __expf(m - mn);
    a0 *= sc;
    a1 *= sc;
    W *= sc;
    m = mn;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      const float w = merge_weight(ls[i], m);
      f32x4 lo, hi;
      bf16x8_to_f32(v[i], lo, hi);
      W += w;
      a0 += w * lo;
      a1 += w * hi;
    }
  }
  // The P folds of each column group are combined in two fixed stages: the
  // P / 4 parts within a wave by a butterfly over the lanes (lane l and lane
  // l ^ d hold the same columns for d >= G), then the 4 waves in wave order
  // through LDS.
  static_assert(G <= 64 && 64 % G == 0, "a wave holds whole parts");
#pragma unroll
  for (int d = G; d < 64; d <<= 1) {
    f32x4 b0, b1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      b0[k] = __shfl_xor(a0[k], d);
      b1[k] = __shfl_xor(a1[k], d);
    }
    const float mo = __shfl_xor(m, d), Wo = __shfl_xor(W, d);
    fold_pair(m, W, a0, a1, mo, Wo, b0, b1);
  }
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane < G) {  // part 0 of the wave: cg == lane
    lds.acc[wave][lane][0] = a0;
    lds.acc[wave][lane][1] = a1;
    if (lane == 0) {
      lds.w[wave] = W;
      lds.m[wave] = m;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kFoldWaves; ++k) M = fmaxf(M, lds.m[k]);
    f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
    float Wt = 0.0f;
#pragma unroll
    for (int k = 0; k < kFoldWaves; ++k) {
      const float f = merge_weight(lds.m[k], M);
      t0 += f * lds.acc[k][cg][0];
      t1 += f * lds.acc[k][cg][1];
      Wt += f * lds.w[k];
    }
    const bool empty = !(Wt > 0.0f);  // no chunk shows this row a key
    const float inv = empty ? 0.0f : 1.0f / Wt;
    u32x4 pk;
    pk[0] = pack_bf16x2(t0[0] * inv, t0[1] * inv);
    pk[1] = pack_bf16x2(t0[2] * inv, t0[3] * inv);
    pk[2] = pack_bf16x2(t1[0] * inv, t1[1] * inv);
    pk[3] = pack_bf16x2(t1[2] * inv, t1[3] * inv);
    *(u32x4*)(o_row + C * cb + 8 * cg) = pk;
    if (lse_out && cg == 0) *lse_out = empty ? -INFINITY : M + __logf(Wt);
  }
  __syncthreads();
}

// P = 1: one thread folds all S chunks of 8 columns (c8) of one split row in
// ascending order, eight at a time with their loads in flight together, with
// the same running-maximum arithmetic as one part above, and writes them.
__device__ __forceinline__ void fold_cols8(const float* part_lse, const uint16_t* part_o,
                                           int64_t pbase, int S, int R, int c8, uint16_t* o_row,
                                           float* lse_out) {
  float m = -INFINITY, W = 0.0f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* po = part_o + 8 * c8;
  for (int s0 = 0; s0 < S; s0 += kFoldBatch) {
    float ls[kFoldBatch];
    u32x4 v[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      const int s = s0 + i;
      if (s < S) {
        const int64_t prow = pbase + (int64_t)s * R;
        ls[i] = part_lse[prow];
        v[i] = *(const u32x4*)(po + prow * kDv);
      } else {
        ls[i] = -INFINITY;
        v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float mn = m;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) mn = fmaxf(mn, ls[i]);
    const float sc = mn == -INFINITY ? 1.0f : __expf(m - mn);
    a0 *= sc;
    a1 *= sc;
    W *= sc;
    m = mn;
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      const float w = merge_weight(ls[i], m);
      f32x4 lo, hi;
      bf16x8_to_f32(v[i], lo, hi);
      W += w;
      a0 += w * lo;
      a1 += w * hi;
    }
  }
  const bool empty = !(W > 0.0f);  // no chunk shows this row a key
  const float inv = empty ? 0.0f : 1.0f / W;
  u32x4 pk;
  pk[0] = pack_bf16x2(a0[0] * inv, a0[1] * inv);
  pk[1] = pack_bf16x2(a0[2] * inv, a0[3] * inv);
  pk[2] = pack_bf16x2(a1[0] * inv, a1[1] * inv);
  pk[3] = pack_bf16x2(a1[2] * inv, a1[3] * inv);
  *(u32x4*)(o_row + 8 * c8) = pk;
  if (lse_out) *lse_out = empty ? -INFINITY : m + __logf(W);
}

// fold_split_row with the chunk phases chosen at run time (uniform).
__device__ __forceinline__ void fold_split_row_p(int P, const float* part_lse, const uint16_t* part_o,
                                                 int64_t pbase, int S, int R, int cb, uint16_t* o_row,
                                                 float* lse_out, FoldLds& lds) {
  if (P == 4)
    fold_split_row<4>(part_lse, part_o, pbase, S, R, cb, o_row, lse_out, lds);
  else if (P == 8)
    fold_split_row<8>(part_lse, part_o, pbase, S, R, cb, o_row, lse_out, lds);
  else if (P == 16)
    fold_split_row<16>(part_lse, part_o, pbase, S, R, cb, o_row, lse_out, lds);
  else
    fold_split_row<32>(part_lse, part_o, pbase, S, R, cb, o_row, lse_out, lds);
}

// In-kernel split-KV merge by the last unit of a split row block to finish
// ("bench(cake_mla_varq_dcp_decode): ..." (flashinfer PR #5588), table "What
// was measured", row "split rows").  Every workgroup calls it after its unit,
// with every wave (all of them reach this point).  A unit of a split tile
// makes its partial rows visible device-wide and arrives on its row block's
// counter (the word of the block's chunk 0, row 0); the unit that arrives
// S-th folds the S partial rows of each of its rows into O and LSE: ascending
// chunk order, each thread 4 (row, 8-column) items at a time against the
// running maximum of the LSEs it has read.
__device__ __forceinline__ void merge_if_last(const MainArgs& args, unsigned char* smem) {
  if (args.merge_kind != kMergeLastArriver) return;
  UnitSetup us;  // the unit's indices only (the key layout is not used here)
  if (!unit_setup<2 * kDqk, 64>(args, us) || us.S <= 1) return;
  // release only (an L2 write-back, no invalidation: the units still running
  // on this XCD keep their cached KV rows)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();  // every wave's partial rows are written and released
  volatile unsigned* flag = reinterpret_cast<volatile unsigned*>(smem);
  if (threadIdx.x == 0) {
    unsigned long long* w =
        args.arrivals + ((int64_t)us.part_row0 + (int64_t)us.t * us.S * us.R + us.rowb0);
    bool last = false;
    arrive(w, args.epoch, (unsigned)us.S, &last);
    *flag = last ? 1u : 0u;
  }
  __syncthreads();
  if (*flag == 0u) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the row block's partial rows
  const int S = us.S, RU = us.RU;
  const int64_t p0 = (int64_t)us.part_row0 + (int64_t)us.t * S * us.R + us.rowb0;  // chunk 0, row 0
  constexpr int kItems = 4;   // (row, 8-column) items per thread at a time
  constexpr int kBatch = 4;   // chunks in flight per item
  for (int it0 = threadIdx.x * kItems; it0 < RU * 64; it0 += blockDim.x * kItems) {
    float m[kItems], W[kItems];
    f32x4 a0[kItems], a1[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      m[j] = -INFINITY;
      W[j] = 0.0f;
      a0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      a1[j] = a0[j];
    }
    for (int s0 = 0; s0 < S; s0 += kBatch) {
      float ls[kItems][kBatch];
      u32x4 v[kItems][kBatch];
#pragma unroll
      for (int j = 0; j < kItems; ++j)
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int item = it0 + j, s = s0 + i;
          if (item < RU * 64 && s < S) {
            const int64_t prow = p0 + (int64_t)s * us.R + (item >> 6);
            ls[j][i] = us.part_lse[prow];
            v[j][i] = *(const u32x4*)(us.part_o + prow * kDv + 8 * (item & 63));
          } else {
            ls[j][i] = -INFINITY;
            v[j][i] = u32x4{0u, 0u, 0u, 0u};
          }
        }
#pragma unroll
      for (int j = 0; j < kItems; ++j) {
        float mn = m[j];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) mn = fmaxf(mn, ls[j][i]);
        const float sc = mn == -INFINITY ? 1.0f : __expf(m[j] - mn);
        a0[j] *= sc;
        a1[j] *= sc;
        W[j] *= sc;
        m[j] = mn;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const float w = ls[j][i] == -INFINITY ? 0.0f : __expf(ls[j][i] - mn);
          const u32x4 x = v[j][i];
          W[j] += w;
          a0[j] += w * f32x4{__builtin_bit_cast(float, x[0] << 16), __builtin_bit_cast(float, x[0] & 0xffff0000u),
                             __builtin_bit_cast(float, x[1] << 16), __builtin_bit_cast(float, x[1] & 0xffff0000u)};
          a1[j] += w * f32x4{__builtin_bit_cast(float, x[2] << 16), __builtin_bit_cast(float, x[2] & 0xffff0000u),
                             __builtin_bit_cast(float, x[3] << 16), __builtin_bit_cast(float, x[3] & 0xffff0000u)};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int item = it0 + j;
      if (item >= RU * 64) break;
      const int r = item >> 6, c = item & 63;
      const bool empty = !(W[j] > 0.0f);  // no chunk shows this row a key
      const float inv = empty ? 0.0f : 1.0f / W[j];
      u32x4 pk;
      pk[0] = pack_bf16x2(a0[j][0] * inv, a0[j][1] * inv);
      pk[1] = pack_bf16x2(a0[j][2] * inv, a0[j][3] * inv);
      pk[2] = pack_bf16x2(a1[j][0] * inv, a1[j][1] * inv);
      pk[3] = pack_bf16x2(a1[j][2] * inv, a1[j][3] * inv);
      const int64_t orow = (int64_t)us.row0 + r;
      *(u32x4*)(us.o + orow * kDv + 8 * c) = pk;
      if (c == 0) us.lse[orow] = empty ? -INFINITY : m[j] + __logf(W[j]);
    }
  }
}


// In-kernel split-KV merge by the whole grid, for launches whose workgroups
// are all resident at once (at most one per compute unit; the host only asks
// for it then).  Every workgroup calls it after its unit, with every wave:
// it makes its partial rows visible device-wide, arrives on the launch's
// counter and waits for the last arrival; then the workgroups fold the
// launch's split rows together, workgroup g taking the (split row, column
// block) items g, g + grid, ... with the fold and layout of the reduce kernel
// (the same arithmetic in the same order, so the results are the reduce
// kernel's bit for bit).  The wait is bounded (about a second by the wall clock): a
// workgroup that gives up writes NaN into the O and LSE of its items instead
// of folding them, so such a failure shows in the outputs.
constexpr long long kGridWaitTicks = 100000000;  // wall-clock ticks (100 MHz): 1 s

__device__ __forceinline__ void merge_grid(const MainArgs& args, unsigned char* smem) {
  if (args.merge_kind != kMergeGrid) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();  // every wave's partial rows are written and released
  volatile unsigned* flag = reinterpret_cast<volatile unsigned*>(smem);
  if (threadIdx.x == 0) {
    bool last = false;
    const unsigned gen = arrive(args.grid_word, args.epoch, gridDim.x, &last);
    unsigned ok = 1u;
    if (!last) {
      const long long t0 = wall_clock64();
      while (true) {
        const unsigned long long w =
            __hip_atomic_load(args.grid_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) != args.epoch || (((unsigned)(w >> 16)) & 0xffffu) != gen) break;
        if (wall_clock64() - t0 > kGridWaitTicks) {
          ok = 0u;
          break;
        }
        __builtin_amdgcn_s_sleep(8);  // ~512 clocks between polls
      }
    }
    *flag = ok;
  }
  __syncthreads();
  const bool ok = *flag != 0u;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every unit's partial rows
  FoldLds& lds = *reinterpret_cast<FoldLds*>(smem + 256);
  int smax = 0;  // the reduce kernel's layout rule: chunk phases from the launch's largest S
  for (int b = 0; b < args.num_seqs; ++b) {
    const int sb = seq_desc(args, b).S;
    smax = max(smax, sb > 1 ? sb : 0);
  }
  const int P = fold_parts(smax);
  // items: (split row, column block) for P >= 4; groups of kFoldRowsP1 rows
  // (64 threads per row) for P = 1
  const int C = P == 1 ? kDv : 8 * (kFoldThreads / P), nb = kDv / C;
  const int items = P == 1 ? (args.num_split_rows + kFoldRowsP1 - 1) / kFoldRowsP1
                           : args.num_split_rows * nb;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int gr = P == 1 ? kFoldRowsP1 * item + (int)threadIdx.x / (kDv / 8) : item / nb;
    const int cb = P == 1 ? 0 : item % nb;
    if (P == 1 && gr >= args.num_split_rows) continue;  // per thread: no barrier below for P = 1
    int b = 0, row0 = 0;  // the split sequence that holds split row gr
    for (; b < args.num_seqs; ++b) {
      const SeqDesc d = seq_desc(args, b);
      if (d.S <= 1) continue;
      if (gr < row0 + d.T * d.R) break;
      row0 += d.T * d.R;
    }
    if (b == args.num_seqs) break;  // not reached: items cover the split rows exactly
    const SeqDesc sd = seq_desc(args, b);
    const int local = gr - row0;
    const int t = local / sd.R, r = local % sd.R;
    const int64_t orow = (int64_t)sd.q_row0 + (int64_t)t * sd.R + r;
    uint16_t* o_row = args.o + orow * kDv;
    float* lse_out = cb == 0 ? args.lse + orow : nullptr;
    const int64_t pbase = (int64_t)sd.part_row0 + (int64_t)t * sd.S * sd.R + r;
    if (P == 1) {
      const int c8 = (int)threadIdx.x % (kDv / 8);
      float* lse1 = c8 == 0 ? args.lse + orow : nullptr;
      if (ok) {
        fold_cols8(args.part_lse, args.part_o, pbase, sd.S, sd.R, c8, o_row, lse1);
      } else {
        *(u32x4*)(o_row + 8 * c8) = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
        if (lse1) *lse1 = __builtin_nanf("");
      }
    } else if (ok) {
      fold_split_row_p(P, args.part_lse, args.part_o, pbase, sd.S, sd.R, cb, o_row, lse_out, lds);
    } else if (threadIdx.x < C / 8) {
      *(u32x4*)(o_row + C * cb + 8 * threadIdx.x) = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
      if (lse_out && threadIdx.x == 0) *lse_out = __builtin_nanf("");
    }
  }
}

}  // namespace mla
