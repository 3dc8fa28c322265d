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

// ROW_BYTES: bytes of one KV row in memory (1152 bf16, 576 fp8); TILE_KEYS:
// keys per compute tile of the kernel (uc.ntiles counts those).
template <int ROW_BYTES, int TILE_KEYS>
__device__ __forceinline__ bool unit_setup(const MainArgs& args, UnitSetup& us) {
  const int p = blockIdx.x;
  const int u = (p % kNumXcd) * args.units_per_xcd + p / kNumXcd;  // XCD-aware order
  if (u >= args.num_units) return false;
  int b = 0;
  while (b + 1 < args.num_seqs && args.seqs[b + 1].unit0 <= u) ++b;
  const SeqDesc& sd = args.seqs[b];
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

// In-kernel split-KV merge by the last unit of a split row block to finish
// ("bench(cake_mla_varq_dcp_decode): ..." (flashinfer PR #5588), table "What
// was measured", row "split rows").  Every workgroup calls it after its unit,
// with every wave (all of them reach this point).  A unit of a split tile
// makes its partial rows visible device-wide and arrives on its row block's
// counter; the unit that arrives S-th folds the S partial rows of each of its
// rows into O and LSE: ascending chunk order, each thread 4 (row, 8-column)
// items at a time against the running maximum of the LSEs it has read (the
// arithmetic of the reduce kernel).  The counter word holds the call's epoch
// in its high half (never 0 or ~0) and that call's arrivals in the low half;
// a word that holds another epoch counts as no arrival, so the workspace's
// prior contents do not matter.
__device__ __forceinline__ void merge_if_last(const MainArgs& args, unsigned char* smem) {
  if (!args.merge_in_kernel) return;
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
    const unsigned long long tag = (unsigned long long)args.epoch << 32;
    unsigned long long old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long nw;
    while (true) {  // ends: each failed swap means another unit's arrival went in
      nw = (old >> 32) == (unsigned long long)args.epoch ? old + 1ull : tag | 1ull;
      const unsigned long long prev = atomicCAS(w, old, nw);
      if (prev == old) break;
      old = prev;
    }
    *flag = (unsigned)(nw & 0xffffffffull) == (unsigned)us.S ? 1u : 0u;
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

}  // namespace mla
