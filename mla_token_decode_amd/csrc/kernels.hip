// MLA speculative-verify decode kernels for gfx950 (MI355X, CDNA4).
//
// Main kernel: one workgroup (4 waves, 256 threads) per work unit = one
// folded tile (R = H*F rows: F verify tokens x H heads, contiguous in Q) and
// one split-KV chunk of its sequence.  The KV chunk is streamed once from HBM
// into LDS and shared by all R rows -- the fold_sq idea of "[Kimi-K3] Allow
// DSPARK verify on cutedsl_mla (fold_sq)" (sglang PR #33650), section
// "Decision rule", paragraph "Why".  Split chunks write normalised partials
// that the reduce kernel merges (same PR, section "GPU timeline").
//
// Work split inside a workgroup (4 waves, one per SIMD): wave w = (row group
// rg = w / 2, half dh = w % 2).  A row group is up to 48 rows (NRT 16-row
// MFMA tiles); the wave pair of a group splits the 576 score columns and the
// 512 value columns in halves:
//   S^T[key][row] partial = K[:, 288dh:288dh+288] . Q^T  (bf16 MFMA 16x16x32;
//                  A = K from LDS, B = the wave's Q half held in VGPRs)
//   the pair sums its two partials through LDS (fp32 a+b == b+a, so both
//   waves hold bitwise-identical scores, max, P and row sums)
//   online softmax: a lane holds 4 keys of ONE row (two cross-lane steps for
//   the row max; per-lane running state)
//   O^T[256dh + col][row] += V^T . P^T  (A = V^T fragments read with the
//                  gfx950 transposing LDS loads, B = P in VGPRs, O in AGPRs)
// fp8 KV is converted to bf16 in registers (exact) after the LDS read; the
// per-tensor scale is folded into the logit scale and the O epilogue.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "plan.hpp"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kTK = 32;        // keys per KV tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = 4;
constexpr unsigned kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer: range-checked, zero on OOB
constexpr float kLazyOctaves = 16.0f;          // softmax reference slack (log2 units)

template <bool FP8>
struct KvCfg;

// bf16 KV: 1152-byte rows = 72 chunks of 16 B.  Physical chunk = logical chunk
// XOR swz(key) inside aligned groups of 8 chunks, so the 16 keys one MFMA
// operand read touches land in distinct 16-B bank slots.
template <>
struct KvCfg<false> {
  static constexpr int kRowBytes = 2 * kDqk;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kTileBytes = kTK * kRowBytes;  // 36864
  static constexpr int kStages = 3;
  static constexpr int kInstr = kTileBytes / 1024;    // 16 B x 64 lanes per load
  static constexpr int kLoaderWaves = 4;
  static constexpr int kInstrPerWave = kInstr / kLoaderWaves;  // 9
  __device__ static int swz(int key) { return (key & 7) ^ ((key >> 3) & 1); }
};

// fp8 KV: 576-byte rows = 36 chunks; XOR inside aligned groups of 4 chunks.
template <>
struct KvCfg<true> {
  static constexpr int kRowBytes = kDqk;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kTileBytes = kTK * kRowBytes;  // 18432
  static constexpr int kStages = 4;
  static constexpr int kInstr = kTileBytes / 1024;    // 18
  static constexpr int kLoaderWaves = 2;
  static constexpr int kInstrPerWave = kInstr / kLoaderWaves;  // 9
  __device__ static int swz(int key) { return (key >> 2) & 3; }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with
// the gfx950 lane-swap instructions: permlane16_swap exchanges the odd 16-lane
// rows of one operand with the even rows of the other, permlane32_swap the
// upper half with the lower half; feeding the same value to both operands and
// combining the two results gives every lane the value of its partner.
__device__ __forceinline__ float wave_max_across_groups(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, (unsigned)r16[0]), __builtin_bit_cast(float, (unsigned)r16[1]));
  const unsigned w = __builtin_bit_cast(unsigned, v);
  auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r32[0]), __builtin_bit_cast(float, (unsigned)r32[1]));
}

__device__ __forceinline__ float wave_sum_across_groups(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (unsigned)r16[0]) + __builtin_bit_cast(float, (unsigned)r16[1]);
  const unsigned w = __builtin_bit_cast(unsigned, v);
  auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_bit_cast(float, (unsigned)r32[0]) + __builtin_bit_cast(float, (unsigned)r32[1]);
}

// 8 fp8 codes (two dwords) -> 8 bf16, exact (OCP E4M3FN -> bf16 never rounds).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// O accumulation: an MFMA whose accumulator is constrained to the AGPR file, so
// the register allocator never copies O between register files.  The compiler
// cannot see hazards inside inline assembly: the leading s_nop covers a VALU
// write of the A/B operands just before (the V conversion), and the code
// around the O uses adds margins for the MFMA-result reads (rescale,
// epilogue).
template <bool OA>
__device__ __forceinline__ void mfma_o(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (OA)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Score MFMA: S^T (VGPRs, read by the softmax) += K . Q^T.  QA places the Q
// operand in the AGPR file (when it fits next to O) so VGPRs stay free for the
// softmax; otherwise in VGPRs.  ZERO starts the accumulation from 0.
template <bool QA, bool ZERO>
__device__ __forceinline__ void mfma_s(f32x4& acc, const bf16x8& k, const bf16x8& q) {
  if constexpr (ZERO) {
    if constexpr (QA)
      asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "a"(q));
    else
      asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "v"(q));
  } else {
    if constexpr (QA)
      asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "a"(q));
    else
      asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "v"(q));
  }
}

// Multiply one accumulator element in place without leaving the AGPR file, so
// the loop-carried O accumulators stay AGPR values on every control path.
__device__ __forceinline__ float scale_agpr(float a, float alpha) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32 %1, %1, %2\n\t"
      "v_accvgpr_write_b32 %0, %1"
      : "+a"(a), "=&v"(t)
      : "v"(alpha));
  return a;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  uint16_t xu = __builtin_bit_cast(uint16_t, x), yu = __builtin_bit_cast(uint16_t, y);
  return (uint32_t)xu | ((uint32_t)yu << 16);
}

// Issue the DMA of one KV tile (keys [k0, k0 + 32) of a unit, clipped to
// `valid` keys; rows past it read as zero) into an LDS stage.
template <bool FP8>
__device__ __forceinline__ void issue_tile(const uint8_t* kv_seq, int k0, int valid, lds_u8* stage,
                                           const int* src_off, int wave) {
  using C = KvCfg<FP8>;
  if (wave >= C::kLoaderWaves) return;
  const int rows = valid < kTK ? valid : kTK;
  __amdgpu_buffer_rsrc_t r =
      make_rsrc(kv_seq + (int64_t)k0 * C::kRowBytes, (uint32_t)(rows * C::kRowBytes));
#pragma unroll
  for (int m = 0; m < C::kInstrPerWave; ++m) {
    const int j = wave + C::kLoaderWaves * m;  // which 1-KB block of the tile
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(stage + j * 1024),
                                             16, src_off[m], 0, 0, 0);
  }
}

// Per-lane LDS byte offsets of the K and V fragments inside a tile.  The XOR
// swizzle only touches the low bits of the chunk index, so every read is
// `lane base (chosen by a few low bits of the step) + compile-time offset`:
//  bf16 K, step ks = 2a + r:  chunk (4 ks + g) ^ sw = 8a + ((4r + g) ^ sw)
//  bf16 V, tile ct = 4a + c:  chunk (2 ct + h) ^ sw = 8a + ((2c + h) ^ sw)
//  fp8  K, step ks = 2a + r:  chunk (2 ks + g/2) ^ sw = 4a + ((2r + g/2) ^ sw)
//  fp8  V, tile ct = 4a + c:  chunk ct ^ sw = 4a + (c ^ sw)
template <bool FP8>
struct FragBases {
  int k[2][2];   // [kt][r]
  int va[4];     // [c]  (bf16: key 4g + i/4, the key 16 + 4g + i/4 is 16 rows
                 //       further with the same swizzle;  fp8: the single tr8 row)
};

template <bool FP8>
__device__ __forceinline__ FragBases<FP8> frag_bases(int l16, int g) {
  using C = KvCfg<FP8>;
  FragBases<FP8> fb;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = 16 * kt + l16;
    const int sw = C::swz(key);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if constexpr (!FP8)
        fb.k[kt][r] = key * C::kRowBytes + 16 * ((4 * r + g) ^ sw);
      else
        fb.k[kt][r] = key * C::kRowBytes + 16 * ((2 * r + (g >> 1)) ^ sw) + 8 * (g & 1);
    }
  }
  const int i = l16;
  if constexpr (!FP8) {
    const int ka = 4 * g + (i >> 2);
    const int h = (i & 3) >> 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) fb.va[c] = ka * C::kRowBytes + 16 * ((2 * c + h) ^ C::swz(ka)) + 8 * (i & 1);
  } else {
    const int kk = i >> 1;
    const int key = kk < 4 ? 4 * g + kk : 16 + 4 * g + (kk - 4);
#pragma unroll
    for (int c = 0; c < 4; ++c) fb.va[c] = key * C::kRowBytes + 16 * (c ^ C::swz(key)) + 8 * (i & 1);
  }
  return fb;
}

// K fragment (A operand of S^T = K Q^T): key 16 kt + l16, d = 32 ks + 8 g .. +8.
template <bool FP8, int KT, int KS>
__device__ __forceinline__ bf16x8 read_k(lds_u8* tile, const FragBases<FP8>& fb) {
  if constexpr (!FP8) {
    return *(const bf16x8*)(tile + fb.k[KT][KS & 1] + 128 * (KS >> 1));
  } else {
    const i32x2 w = *(const i32x2*)(tile + fb.k[KT][KS & 1] + 64 * (KS >> 1));
    return fp8x8_to_bf16(w);
  }
}

// V^T fragment (A operand of O^T = V^T P^T) for column tile CT: lane (g, i)
// gets column 16 CT + i; element e is key 4 g + e (e < 4) or 16 + 4 g + e - 4.
// The gfx950 transposing reads deliver it: in each 16-lane group, lane i
// points at a 4 (bf16) or 8 (fp8) element piece of one key row, and lane j
// receives element j of every row of the group's block.
// The transposing-read builtins do not fold constant offsets, which makes the
// compiler keep one address register per column tile; these wrappers emit the
// instruction with its immediate offset.  Their results are not tracked by the
// compiler's LDS wait counting: use them only through wait_lds<N>(), which
// waits until at most N of the LDS reads issued after the needed one are
// outstanding (LDS reads complete in order) and ties the data to that wait.
template <int OFF>
__device__ __forceinline__ i32x2 ds_read_tr16_b64(const lds_u8* addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  i32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ i32x2 ds_read_tr8_b64(const lds_u8* addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  i32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void wait_lds(i32x2& a, i32x2& b) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}

// Raw (unconverted) V^T fragment for column tile CT: bf16 -> two tr16 pieces,
// fp8 -> one tr8 piece.  Lane (g, i) gets column 16 CT + i; element e is key
// 4 g + e (e < 4) or 16 + 4 g + e - 4.  In each 16-lane group of a
// transposing read, lane i points at a 4 (bf16) or 8 (fp8) element piece of
// one key row and lane j receives element j of every row of the block.
template <bool FP8>
struct VRaw {
  i32x2 a, b;
};

template <bool FP8, int CT>
__device__ __forceinline__ void issue_v(VRaw<FP8>& r, lds_u8* tile, const FragBases<FP8>& fb) {
  if constexpr (!FP8) {
    // keys 16 apart share the swizzle, so the second piece is 16 rows further
    r.a = ds_read_tr16_b64<128 * (CT >> 2)>(tile + fb.va[CT & 3]);
    r.b = ds_read_tr16_b64<128 * (CT >> 2) + 16 * KvCfg<FP8>::kRowBytes>(tile + fb.va[CT & 3]);
  } else {
    r.a = ds_read_tr8_b64<64 * (CT >> 2)>(tile + fb.va[CT & 3]);
  }
}

// LDS reads issued per V fragment.
template <bool FP8>
constexpr int kVReads = FP8 ? 1 : 2;

template <bool FP8>
__device__ __forceinline__ bf16x8 finish_v(const VRaw<FP8>& r) {
  if constexpr (!FP8) {
    const i32x4 w = {r.a[0], r.a[1], r.b[0], r.b[1]};
    return __builtin_bit_cast(bf16x8, w);
  } else {
    return fp8x8_to_bf16(r.a);
  }
}

// Compile-time loop helper.
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// One KV tile of compute for a wave of half DH (templated so every LDS
// offset is a compile-time immediate on top of a few lane bases).
template <bool FP8, int NRT, int DH>
__device__ __forceinline__ void tile_compute(lds_u8* tile, float* xs_mine, const float* xs_peer,
                                             const FragBases<FP8>& fb,
                                             const bf16x8 (&qf)[NRT][9], f32x4 (&oacc)[16][NRT],
                                             float (&m_run)[NRT], float (&l_run)[NRT],
                                             const int (&lim)[NRT], int k0, bool edge,
                                             float scale_log2, int g, int lane) {
  // ---- partial S^T over this wave's 288 columns, K fragments one step ahead ----
  // register files: NRT <= 2 keeps O (16 NRT f32x4) in VGPRs and Q in AGPRs;
  // NRT = 3 needs O in AGPRs and Q in VGPRs
  constexpr bool kQinAgpr = NRT <= 2;
  constexpr bool kOinAgpr = !kQinAgpr;
  f32x4 sacc[2][NRT];
  bf16x8 kf[2][2];
  kf[0][0] = read_k<FP8, 0, 9 * DH>(tile, fb);
  kf[0][1] = read_k<FP8, 1, 9 * DH>(tile, fb);
  static_for<9>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int cur = j & 1;
    if constexpr (j + 1 < 9) {
      kf[cur ^ 1][0] = read_k<FP8, 0, 9 * DH + j + 1>(tile, fb);
      kf[cur ^ 1][1] = read_k<FP8, 1, 9 * DH + j + 1>(tile, fb);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) mfma_s<kQinAgpr, j == 0>(sacc[kt][rt], kf[cur][kt], qf[rt][j]);
    __builtin_amdgcn_sched_barrier(0);
  });
  // the score MFMAs retire before their results are read below
  asm volatile("s_nop 15\n\ts_nop 7" ::: "memory");

  // ---- exchange partials with the other half of the row group ----
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      *(f32x4*)(xs_mine + ((rt * 2 + kt) * 64 + lane) * 4) = sacc[kt][rt];
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      sacc[kt][rt] += *(const f32x4*)(xs_peer + ((rt * 2 + kt) * 64 + lane) * 4);

  VRaw<FP8> vr[2];
  issue_v<FP8, 16 * DH>(vr[0], tile, fb);

  // ---- online softmax (base 2) with a lazy per-row reference m_ref:
  //      P = 2^(x - m_ref); m_ref moves (and O, l are rescaled) only when a
  //      row's tile max exceeds it by more than kLazyOctaves, so P <= 2^16 and
  //      the exact result is unchanged ----
  bf16x8 pf[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    float x[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float val = sacc[kt][rt][i] * scale_log2;
        if (edge) {
          const int key = k0 + 16 * kt + 4 * g + i;
          val = key <= lim[rt] ? val : -INFINITY;
        }
        x[kt * 4 + i] = val;
      }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = wave_max_across_groups(mx);
    const bool need = mx > m_run[rt] + kLazyOctaves;
    if (__any(need)) {
      const bool rescale = need && m_run[rt] != -INFINITY;
      const float m_new = need ? mx : m_run[rt];
      if (__any(rescale)) {
        const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run[rt] - m_new) : 1.0f;
        l_run[rt] *= alpha;
        // the last MFMA that wrote O retired long ago (a whole QK phase ran
        // since); the nops are a margin for the accumulator read hazard
        asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
        if constexpr (kOinAgpr) {
#pragma unroll
          for (int ct = 0; ct < 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[ct][rt][e] = scale_agpr(oacc[ct][rt][e], alpha);
        } else {
#pragma unroll
          for (int ct = 0; ct < 16; ++ct) oacc[ct][rt] *= alpha;
        }
        asm volatile("s_nop 7" ::: "memory");
      }
      m_run[rt] = m_new;
    }
    const float mu = m_run[rt] == -INFINITY ? 0.0f : m_run[rt];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(x[e] - mu);  // v_exp_f32; tiny results flush to 0
      psum += pe;
      pf[rt][e] = (__bf16)pe;
    }
    l_run[rt] += psum;
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- O^T[256 DH + ...] += V^T P^T, V fragments one column tile ahead ----
  static_for<16>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    constexpr int cur = c & 1;
    if constexpr (c + 1 < 16) {
      issue_v<FP8, 16 * DH + c + 1>(vr[cur ^ 1], tile, fb);
      wait_lds<kVReads<FP8>>(vr[cur].a, vr[cur].b);
    } else {
      wait_lds<0>(vr[cur].a, vr[cur].b);
    }
    const bf16x8 vf = finish_v<FP8>(vr[cur]);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
      mfma_o<kOinAgpr>(oacc[c][rt], vf, pf[rt]);
    __builtin_amdgcn_sched_barrier(0);
  });
}

template <bool FP8, int NRT, int DH>
__device__ __forceinline__ void unit_body(const MainArgs& args, unsigned char* smem) {
  using C = KvCfg<FP8>;
  lds_u8* lds = (lds_u8*)smem;

  // ---- work unit: XCD-aware order (consecutive units share an XCD's L2) ----
  const int p = blockIdx.x;
  const int u = (p % kNumXcd) * args.units_per_xcd + p / kNumXcd;
  if (u >= args.num_units) return;
  int b = 0;
  while (b + 1 < args.num_seqs && args.seqs[b + 1].unit0 <= u) ++b;
  const SeqDesc sd = args.seqs[b];
  const int v = u - sd.unit0;
  const int per_chunk = sd.T * sd.NRB;  // units sharing one KV chunk are consecutive
  const int s = v / per_chunk;
  const int t = (v % per_chunk) / sd.NRB;
  const int rb = v % sd.NRB;
  const int R = sd.R;
  const int H = args.H;
  const int rowb0 = rb * sd.RBS;                 // first tile row of this unit
  const int RU = min(sd.RBS, R - rowb0);         // rows of this unit
  const int row0 = sd.q_row0 + t * R + rowb0;    // first Q/O row of this unit
  const int lo = s * sd.L;
  const int hi = min(lo + sd.L, sd.n);
  const int tail0 = sd.n - sd.qlen + t * sd.F;   // tile row r sees keys <= tail0 + r / H
  const int vis_lo = tail0 + rowb0 / H;          // every unit row sees keys <= vis_lo
  const int vis_hi = tail0 + (rowb0 + RU - 1) / H;
  const int hi_eff = min(hi, vis_hi + 1);        // no unit row sees keys >= hi_eff
  const int nkeys = hi_eff - lo;                 // may be <= 0 (chunk hidden from every row)
  const int ntiles = nkeys > 0 ? (nkeys + kTK - 1) / kTK : 0;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int rg = wave >> 1;
  constexpr int dh = DH;
  const int grow0 = rg * 16 * NRT;  // first unit row of this wave's group
  const bool wave_active = grow0 < RU;

  // ---- Q fragments (B operand): row grow0 + 16 rt + l16, d = 288 dh + 32 j + 8 g ----
  bf16x8 qf[NRT][9];
  {
    __amdgpu_buffer_rsrc_t qr = make_rsrc(args.q + (int64_t)row0 * kDqk, (uint32_t)(RU * kDqk * 2));
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int row = grow0 + 16 * rt + l16;
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            qr, row * (kDqk * 2) + dh * 576 + j * 64 + g * 16, 0, 0);
        qf[rt][j] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  // ---- loader offsets: instruction m of this wave fills LDS block j; lane
  //      `lane` of it writes physical chunk 64 j + lane, which holds the
  //      logical chunk (row, pc ^ swz(row)) of the tile ----
  int src_off[C::kInstrPerWave];
#pragma unroll
  for (int m = 0; m < C::kInstrPerWave; ++m) {
    const int j = (wave < C::kLoaderWaves ? wave : 0) + C::kLoaderWaves * m;
    const int cidx = j * 64 + lane;
    const int row = cidx / C::kChunks;
    const int pc = cidx % C::kChunks;
    src_off[m] = row * C::kRowBytes + ((pc ^ C::swz(row)) * 16);
  }

  const uint8_t* kv_seq = args.kv + ((int64_t)sd.kv_row0 + lo) * C::kRowBytes;

  // ---- per-lane softmax state (lane owns unit row grow0 + 16 rt + l16) ----
  float m_run[NRT], l_run[NRT];
  int lim[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.0f;
    const int row = grow0 + 16 * rt + l16;
    const int rv = row < RU ? row : RU - 1;
    lim[rt] = min(hi_eff - 1, tail0 + (rowb0 + rv) / H) - lo;  // last visible key, unit-relative
  }
  const int min_lim = min(hi_eff - 1, vis_lo) - lo;  // every row sees keys <= this

  f32x4 oacc[16][NRT];
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) oacc[c][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: tiles 0 .. kStages-2 in flight ----
#pragma unroll
  for (int st = 0; st < C::kStages - 1; ++st)
    if (st < ntiles)
      issue_tile<FP8>(kv_seq, st * kTK, nkeys - st * kTK, lds + st * C::kTileBytes, src_off, wave);

  const FragBases<FP8> fb = frag_bases<FP8>(l16, g);
  float* xs = (float*)(smem + C::kStages * C::kTileBytes);
  float* xs_mine = xs + wave * NRT * 2 * 256;
  const float* xs_peer = xs + (wave ^ 1) * NRT * 2 * 256;
  const float scale_log2 = args.scale_log2;

  for (int it = 0; it < ntiles; ++it) {
    // tile `it` landed (this wave's part); later tiles may still be in flight
    const int ahead = min(C::kStages - 2, ntiles - 1 - it);
    if constexpr (C::kStages == 3) {
      if (ahead >= 1) wait_vmcnt<C::kInstrPerWave>(); else wait_vmcnt<0>();
    } else {
      if (ahead >= 2) wait_vmcnt<2 * C::kInstrPerWave>();
      else if (ahead == 1) wait_vmcnt<C::kInstrPerWave>();
      else wait_vmcnt<0>();
    }
    __syncthreads();  // tile `it` visible to all; the stage of tile it-1 is free
    if (it + C::kStages - 1 < ntiles) {
      const int nt = it + C::kStages - 1;
      issue_tile<FP8>(kv_seq, nt * kTK, nkeys - nt * kTK,
                      lds + (nt % C::kStages) * C::kTileBytes, src_off, wave);
    }
    lds_u8* tile = lds + (it % C::kStages) * C::kTileBytes;
    const int k0 = it * kTK;  // unit-relative first key of the tile
    const bool edge = k0 + kTK - 1 > min_lim;
    if (wave_active) {
      tile_compute<FP8, NRT, DH>(tile, xs_mine, xs_peer, fb, qf, oacc, m_run, l_run, lim, k0, edge,
                                 scale_log2, g, lane);
    } else {
      __syncthreads();  // matches the pair exchange barrier of active waves
    }
  }

  if (!wave_active) return;
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // last O MFMA retired before reads

  // ---- epilogue: this wave's rows x columns [256 dh, 256 dh + 256) ----
  const float ln2 = 0.69314718055994530942f;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float lt = wave_sum_across_groups(l_run[rt]);
    const int row = grow0 + 16 * rt + l16;
    const bool valid = row < RU;
    if (sd.S == 1) {
      const float inv = args.o_scale / lt;
      const int64_t orow = (int64_t)row0 + row;
      if (valid) {
        uint16_t* op = args.o + orow * kDv + 256 * dh + 4 * g;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const f32x4 o4 = oacc[c][rt] * inv;
          uint2 pk;
          pk.x = pack_bf16x2(o4[0], o4[1]);
          pk.y = pack_bf16x2(o4[2], o4[3]);
          *(uint2*)(op + 16 * c) = pk;
        }
        if (g == 0 && dh == 0) args.lse[orow] = (m_run[rt] + log2f(lt)) * ln2;
      }
    } else {
      const int64_t prow = (int64_t)sd.part_row0 + ((int64_t)t * sd.S + s) * R + rowb0 + row;
      const bool empty = !(lt > 0.0f);
      const float inv = empty ? 0.0f : args.o_scale / lt;
      if (valid) {
        float* pp = args.part_o + prow * kDv + 256 * dh + 4 * g;
#pragma unroll
        for (int c = 0; c < 16; ++c) *(f32x4*)(pp + 16 * c) = oacc[c][rt] * inv;
        if (g == 0 && dh == 0) args.part_lse[prow] = empty ? -INFINITY : (m_run[rt] + log2f(lt)) * ln2;
      }
    }
  }
}

template <bool FP8, int NRT>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_main(const MainArgs args) {
  using C = KvCfg<FP8>;
  constexpr int kXsBytes = kWaves * NRT * 2 * 1024;  // score partials exchanged by wave pairs
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::kStages * C::kTileBytes + kXsBytes];
  if ((threadIdx.x >> 6) & 1)
    unit_body<FP8, NRT, 1>(args, smem);
  else
    unit_body<FP8, NRT, 0>(args, smem);
}

// Split-KV merge.  One 512-thread block per (split output row, column half):
// wave w folds chunks s = w, w + 8, ... (lane c owns columns 4c .. 4c+3 of the
// half), then the 8 waves' sums are added in wave order through LDS.  Every
// sum has a fixed order, so replays are bitwise identical.
constexpr int kRedThreads = 512;
constexpr int kRedWaves = kRedThreads / 64;

__device__ __forceinline__ float wave_max64(float v) {
  v = wave_max_across_groups(v);          // lanes l, l^16, l^32, l^48
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

__global__ __launch_bounds__(kRedThreads) void mla_decode_reduce_kernel(const ReduceArgs args) {
  __shared__ f32x4 red_acc[kRedWaves][64];
  __shared__ float red_w[kRedWaves];
  const int gr = blockIdx.x >> 1;
  const int half = blockIdx.x & 1;
  if (gr >= args.num_rows) return;
  int b = 0;
  while (b + 1 < args.num_seqs && args.row0[b + 1] <= gr) ++b;
  const SeqDesc& sd = args.seqs[b];
  const int local = gr - args.row0[b];
  const int R = sd.R;
  const int t = local / R;
  const int r = local % R;
  const int S = sd.S;
  const int64_t pbase = (int64_t)sd.part_row0 + (int64_t)t * S * R + r;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, args.part_lse[pbase + (int64_t)s * R]);
  M = wave_max64(M);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.0f;
  const float* po = args.part_o + 256 * half + 4 * lane;
#pragma unroll 4
  for (int s = wave; s < S; s += kRedWaves) {
    const int64_t prow = pbase + (int64_t)s * R;
    const float ls = args.part_lse[prow];
    if (ls == -INFINITY) continue;  // a chunk this row cannot see: weight 0
    const float w = __expf(ls - M);
    W += w;
    acc += w * *(const f32x4*)(po + prow * kDv);
  }
  red_acc[wave][lane] = acc;
  if (lane == 0) red_w[wave] = W;
  __syncthreads();
  if (wave != 0) return;
  f32x4 tot = red_acc[0][lane];
  float Wt = red_w[0];
#pragma unroll
  for (int w2 = 1; w2 < kRedWaves; ++w2) {
    tot += red_acc[w2][lane];
    Wt += red_w[w2];
  }
  const float inv = 1.0f / Wt;
  const int64_t orow = (int64_t)sd.q_row0 + (int64_t)t * R + r;
  uint2 pk;
  pk.x = pack_bf16x2(tot[0] * inv, tot[1] * inv);
  pk.y = pack_bf16x2(tot[2] * inv, tot[3] * inv);
  *(uint2*)(args.o + orow * kDv + 256 * half + 4 * lane) = pk;
  if (half == 0 && lane == 0) args.lse[orow] = M + __logf(Wt);
}

// ------------------------------------------------------------- launchers

template <bool FP8>
static void launch_main_t(const MainArgs& a, int nrt, int grid, hipStream_t stream) {
  if (nrt <= 1)
    hipLaunchKernelGGL((mla_decode_main<FP8, 1>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((mla_decode_main<FP8, 2>), dim3(grid), dim3(kThreads), 0, stream, a);
}

hipError_t launch_main(const MainArgs& a, bool fp8, int nrt, hipStream_t stream) {
  const int grid = ((a.num_units + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid == 0) return hipSuccess;
  if (nrt < 1 || nrt > 2) return hipErrorInvalidValue;
  if (fp8)
    launch_main_t<true>(a, nrt, grid, stream);
  else
    launch_main_t<false>(a, nrt, grid, stream);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream) {
  const int grid = 2 * a.num_rows;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_decode_reduce_kernel, dim3(grid), dim3(kRedThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
