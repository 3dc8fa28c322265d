// MLA speculative-verify decode kernels for gfx950 (MI355X, CDNA4).
//
// Main kernel: one workgroup (4 waves, 256 threads) per work unit = up to 96
// rows of one folded tile (F verify tokens x H heads, contiguous in Q) and one
// split-KV chunk of its sequence.  The chunk is streamed once from HBM and
// shared by all rows of the unit -- the fold_sq idea of "[Kimi-K3] Allow DSPARK
// verify on cutedsl_mla (fold_sq)" (sglang PR #33650), section "Decision rule",
// paragraph "Why".  Split chunks write normalised partials that the reduce
// kernel merges (same PR, section "GPU timeline").
//
// Loader: every thread keeps one to three 32-key KV tiles in flight in
// registers (inline-assembly buffer loads with explicit vmcnt waits), then
// writes each tile into an LDS ring of three slots (four for the fp8
// key-split kernels below): bf16 KV as bf16 rows; fp8-e4m3
// KV with the 512 latent columns kept as e4m3 codes and the 64 rope columns
// converted (exactly) to bf16.  The per-tensor fp8 scale is folded into the
// logit scale and the O epilogue.
//
// Work split inside a workgroup: wave w = (row group rg = w / 2, half
// dh = w % 2).  A row group is up to 48 rows (NRT 16-row MFMA tiles); the
// wave pair splits the 512 value columns in halves and, except in the fp8
// key-split kernels (unit_pipeline8k), the 576 score columns too:
//   S^T[key][row] partial = K[:, 288dh:+288] . Q^T   (bf16 KV: bf16 MFMA
//                  16x16x32; fp8 KV: fp8 MFMA 16x16x128 on the latent part
//                  with Q quantised per row, bf16 MFMA on the rope part;
//                  A = K from LDS, B = the wave's Q half in registers)
//   the pair sums its two partials through LDS (fp32 a+b == b+a, so both
//   waves hold bitwise-identical scores, reference, P and row sums)
//   online softmax: a lane holds 4 keys of ONE row; per-lane running state;
//                  the base-2 reference moves only for large jumps
//   O^T[256dh + col][row] += V^T . P^T  (A = V^T fragments read with the
//                  gfx950 transposing LDS loads, B = P in VGPRs, O in AGPRs;
//                  bf16 P and V with bf16 KV, e4m3 P and V with fp8 KV)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "plan.hpp"

namespace mla {


constexpr int kTK = 32;        // keys per compute tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = 4;
// Softmax reference slack in log2 units: P = 2^(x - m_ref) may reach 2^60
// with bf16 P (bf16 P and fp32 sums have the range) and 2^8 with e4m3 P (fp8
// KV: its largest finite value is 448); a larger jump moves the reference and
// rescales O and l.
template <bool FP8P>
constexpr float lazy_octaves() { return FP8P ? 8.0f : 60.0f; }


// LDS holds every KV tile as bf16 rows: 1152 bytes = 72 chunks of 16 B,
// physical chunk = logical chunk XOR swz(key) inside aligned groups of 8
// chunks, so the 16 keys an MFMA operand read touches hit distinct bank slots.
constexpr int kRowBytes = 2 * kDqk;
constexpr int kChunks = kRowBytes / 16;        // 72
constexpr int kTileBytes = kTK * kRowBytes;    // 36864
__device__ __forceinline__ int swz(int key) { return (key & 7) ^ ((key >> 3) & 1); }

// fp8 KV tiles stay fp8 in LDS for the latent part (QK^T runs on fp8 MFMAs and
// V is converted when read): 512-byte latent rows, then the 64 rope columns
// of every key as bf16 (128-byte rows; the rope part of QK^T stays bf16).
// Latent rows XOR their 16-byte chunk index with swz8(key): the 16 keys of a
// K fragment read (keys 16 kt + m) and the 8 keys of a transposing V read
// (keys 4 g + i and 16 + 4 g + i) all land in distinct 16-byte bank slots.
constexpr int kLatBytes8 = 512;
constexpr int kRopeOff8 = kTK * kLatBytes8;       // 16384
constexpr int kTileBytes8 = kRopeOff8 + kTK * 128;  // 20480
template <bool FP8>
constexpr int tile_bytes() { return FP8 ? kTileBytes8 : kTileBytes; }
__device__ __forceinline__ int swz8(int key) { return (key & 15) ^ ((key & 16) >> 1); }
__device__ __forceinline__ int rope_swz(int key) { return (key >> 1) & 7; }

// One staged KV tile per thread: 2304 pieces of the tile (16 B of bf16 or 8 B
// of fp8, i.e. 8 elements each), piece li = tid + 256 m, m = 0..8.
constexpr int kPieces = kTK * kChunks / kThreads;  // 9

template <bool FP8>
struct Stage {
  using piece_t = typename std::conditional<FP8, u32x2, u32x4>::type;
  static constexpr int kGlobalRowBytes = FP8 ? kDqk : 2 * kDqk;
  piece_t p[kPieces];
};

// Staging sets (tiles in flight per thread): as many as the register budget
// of each row-tile count allows; with 3 row tiles a bf16 set is 36 VGPRs and
// one set, issued one iteration ahead of its LDS store, is what fits.
template <bool FP8, int NRT>
constexpr int stage_sets() { return FP8 ? (NRT == 1 ? 3 : 2) : (NRT == 3 ? 1 : 2); }


// 8 fp8 codes (two dwords) -> 8 bf16, exact (OCP E4M3FN -> bf16 never rounds).
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return u32x4{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
               __builtin_bit_cast(unsigned, c), __builtin_bit_cast(unsigned, d)};
}


// ------------------------------------------------------------------ loader


// Descriptor of compute tile `t` of the unit (keys [32 t, 32 t + 32)): rows
// past `nkeys` read as zero, tiles past the end read nothing.  (readfirstlane:
// the clamp may be selected as a vector instruction, and the descriptor must
// live in scalar registers.)
template <bool FP8>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* kv_unit, int t, int nkeys) {
  constexpr int RB = Stage<FP8>::kGlobalRowBytes;
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kTK, nkeys - t * kTK)));
  return make_rsrc(kv_unit + (int64_t)t * kTK * RB, (uint32_t)(rows * RB));
}

// Issue the global load of piece M of a compute tile (descriptor r) into a
// staging set.  The loads are inline assembly so that their completion is
// waited for explicitly (wait_stage): the compiler's own counting drains every
// set in flight at the loop head.
// fp8: pieces 0..7 are latent (key tid/64 + 4 M, bytes 8 (tid % 64) ..), piece 8
// is rope (key tid/8, bytes 512 + 8 (tid % 8) ..).  bf16: piece M is the 16
// bytes at 16 tid + 4096 M of the tile.
// NT: the non-temporal hint (bf16 KV), for launches in which no KV chunk is
// read by two units: each byte is read once, and a cold streaming read
// measured faster with it.  Where several units read one chunk (the tiles of
// one sequence on one XCD) the hint would make each re-read HBM.
template <bool FP8, int M, bool NT = false>
__device__ __forceinline__ void stage_load_piece(Stage<FP8>& st, __amdgpu_buffer_rsrc_t r, int tid) {
  constexpr int PB = FP8 ? 8 : 16;  // bytes per piece
  const int off = !FP8 ? tid * PB
                  : M < 8 ? (tid >> 6) * kDqk + 8 * (tid & 63)
                          : (tid >> 3) * kDqk + 512 + 8 * (tid & 7);
  const int soff = !FP8 ? kThreads * PB * M : M < 8 ? 4 * kDqk * M : 0;
  if constexpr (FP8)
    asm volatile("buffer_load_dwordx2 %0, %1, %2, %3 offen"
                 : "=&v"(st.p[M]) : "v"(off), "s"(r), "s"(soff) : "memory");
  else if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen nt"
                 : "=&v"(st.p[M]) : "v"(off), "s"(r), "s"(soff) : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen"
                 : "=&v"(st.p[M]) : "v"(off), "s"(r), "s"(soff) : "memory");
}

template <bool FP8, bool NT = false>
__device__ __forceinline__ void stage_load(Stage<FP8>& st, __amdgpu_buffer_rsrc_t r, int tid) {
  static_for<kPieces>([&](auto mc) { stage_load_piece<FP8, decltype(mc)::value, NT>(st, r, tid); });
}

// Where a unit's KV tiles live: one contiguous run of rows, or the pages of a
// pool listed in a page table (pages hold 2^shift >= 32 keys and tiles start
// at multiples of 32 keys, so a tile never crosses a page).
template <bool FP8, bool PAGED>
struct KvSource {
  static constexpr int RB = Stage<FP8>::kGlobalRowBytes;
  const uint8_t* base;    // contiguous: first row of the chunk; paged: the pool
  const int32_t* pt_row;  // paged: the sequence's page-table row
  int lo;                 // first key of the chunk (sequence-relative)
  int nkeys, shift, last_idx;
  unsigned max_page;

  // Page-table entry of tile t (tiles past the end reuse the last entry).
  __device__ __forceinline__ int page_idx(int t) const {
    return min((lo + kTK * t) >> shift, last_idx);
  }
  // First pool row of a page-table entry's page (entries are clamped to the pool).
  __device__ __forceinline__ int64_t page_row(int entry) const {
    return (int64_t)min((unsigned)entry, max_page) << shift;
  }
  // Page row of tile t, waited for here (prologue only).
  __device__ __forceinline__ int64_t page_row_now(int t) const {
    int e;
    asm volatile("s_load_dword %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                 : "=s"(e) : "s"(pt_row), "s"(4 * page_idx(t)) : "memory");
    return page_row(e);
  }
  // The tile barrier (LDS traffic drained, then s_barrier) with the page row of
  // tile t fetched under the same wait.
  __device__ __forceinline__ int64_t barrier_and_page_row(int t) const {
    int e;
    asm volatile("s_load_dword %0, %1, %2\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                 : "=s"(e) : "s"(pt_row), "s"(4 * page_idx(t)) : "memory");
    return page_row(e);
  }
  // Descriptor of tile t (keys [lo + 32 t, lo + 32 t + 32) of the sequence):
  // rows past the chunk read as zero, tiles past the end read nothing.
  // `prow` is the page row of tile t (paged only).
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int t, int64_t prow) const {
    if constexpr (!PAGED) {
      return tile_rsrc<FP8>(base, t, nkeys);
    } else {
      const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kTK, nkeys - t * kTK)));
      const int64_t row = prow + ((lo + kTK * t) & ((1 << shift) - 1));
      return make_rsrc(base + row * RB, (uint32_t)(rows * RB));
    }
  }
};

// Wait until at most N global loads issued after this set's are outstanding
// (vector memory loads complete in order); the set's registers are tied to the
// wait so that no use moves above it.
template <int N, bool FP8>
__device__ __forceinline__ void wait_stage(Stage<FP8>& st) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%9)"
               : "+v"(st.p[0]), "+v"(st.p[1]), "+v"(st.p[2]), "+v"(st.p[3]), "+v"(st.p[4]),
                 "+v"(st.p[5]), "+v"(st.p[6]), "+v"(st.p[7]), "+v"(st.p[8])
               : "n"(N)
               : "memory");
}

// Which bf16 kernels move KV tiles by LDS DMA: those of 48-row row groups.
// With three ring slots a DMA is issued one iteration ahead of its tile, the
// lead that one register staging set gives, and 48-row groups only have room
// for one set; DMA frees those registers and the LDS stores (same process:
// h96_125k main 218 -> 212 us, ragged 557-562 -> 544, bf16 1M q = 8 246 ->
// 236).  Narrower row groups keep two staging sets, two tiles ahead, which
// the HBM-bound rows need (bf16 1M q = 1 with DMA: 195-197 -> 202 us).
template <bool FP8, int NRT>
constexpr bool tile_dma_path() { return !FP8 && NRT == 3; }

// bf16 KV tiles reach their LDS slot by DMA (buffer_load_dwordx4 ... lds, no
// staging registers): the 36 KB of a 32-key tile as 36 blocks of 1 KB, wave w
// issuing blocks J = 4 j + w (j = 0..8).  Lane i of block J fills LDS chunk
// P = 64 J + i of the slot: key P / 72, physical chunk P % 72, which holds
// logical chunk (P % 72) ^ swz(key) (the layout stage_store_piece writes; the
// XOR stays inside each group of 8 chunks), read from the tile's global
// offset 1152 key + 16 logical.  Keys past the tile's rows read as zero.
struct TileDma {
  int off[kPieces];  // per-lane global offsets of blocks 4 j + w, j = 0..8, within a tile
};
__device__ __forceinline__ TileDma tile_dma(int wave, int lane) {
  TileDma d;
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int P = 64 * (4 * j + wave) + lane;
    const int key = P / kChunks, ph = P - key * kChunks;
    d.off[j] = key * kRowBytes + 16 * (ph ^ swz(key));
  }
  return d;
}
// Block 4 j + w of a tile into `slot`; counted by vmcnt (every wait for it is
// explicit).  NT: the non-temporal hint (see stage_load_piece).
template <bool NT>
__device__ __forceinline__ void tile_dma_piece(lds_u8* slot, int j, int wave, int off,
                                               __amdgpu_buffer_rsrc_t r) {
  const unsigned m0v =
      __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(slot + 1024 * (4 * j + wave)));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(m0v), "v"(off), "s"(r) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0v), "v"(off), "s"(r) : "memory");
}
template <bool NT>
__device__ __forceinline__ void tile_dma_all(lds_u8* slot, int wave, const TileDma& d,
                                             __amdgpu_buffer_rsrc_t r) {
  static_for<kPieces>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    tile_dma_piece<NT>(slot, j, wave, d.off[j], r);
  });
}

// Write piece M of a staged tile into an LDS slot.  bf16: swizzled bf16 rows.
// fp8: latent pieces as they are (key k0 + 4 M with k0 = tid / 64, whose
// swizzle is k0 ^ f(M): the address is one XOR with a constant away from a
// per-thread base), the rope piece converted to bf16.
template <bool FP8, int M>
__device__ __forceinline__ void stage_store_piece(const Stage<FP8>& st, lds_u8* slot, int tid) {
  if constexpr (!FP8) {
    const int li = tid + kThreads * M;
    const int key = li / kChunks, c = li % kChunks;
    *(u32x4*)(slot + key * kRowBytes + 16 * (c ^ swz(key))) = st.p[M];
  } else if constexpr (M < 8) {
    const int k0 = tid >> 6, c8 = tid & 63;
    const int base = k0 * kLatBytes8 + 16 * ((c8 >> 1) ^ k0) + 8 * (c8 & 1);
    constexpr int f = (4 * (M & 3)) ^ (8 * (M >> 2));  // swz8(k0 + 4 M) = k0 ^ f
    *(u32x2*)(slot + ((base ^ (16 * f)) + 4 * kLatBytes8 * M)) = st.p[M];
  } else {
    const int key = tid >> 3, c = tid & 7;
    *(u32x4*)(slot + kRopeOff8 + key * 128 + 16 * (c ^ rope_swz(key))) = fp8x8_to_bf16(st.p[M]);
  }
}

template <bool FP8>
__device__ __forceinline__ void stage_store(const Stage<FP8>& st, lds_u8* slot, int tid) {
  static_for<kPieces>([&](auto mc) { stage_store_piece<FP8, decltype(mc)::value>(st, slot, tid); });
}

// ------------------------------------------------------------- fragments

// Per-lane LDS byte offsets of the K and V fragments inside a tile.  The XOR
// swizzle only touches the low bits of the chunk index, so every read is
// `lane base (chosen by a few low bits of the step) + compile-time offset`:
//  K, step ks = 2a + r:  chunk (4 ks + g) ^ sw = 8a + ((4r + g) ^ sw)
//  V, tile ct = 4a + c:  chunk (2 ct + h) ^ sw = 8a + ((2c + h) ^ sw)
struct FragBases {
  int k[2][2];  // [kt][r]
  int va[4];    // [c]: key 4g + i/4; key 16 + 4g + i/4 is 16 rows further, same swizzle
};

__device__ __forceinline__ FragBases frag_bases(int l16, int g) {
  FragBases fb;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = 16 * kt + l16;
    const int sw = swz(key);
#pragma unroll
    for (int r = 0; r < 2; ++r) fb.k[kt][r] = key * kRowBytes + 16 * ((4 * r + g) ^ sw);
  }
  const int i = l16;
  const int ka = 4 * g + (i >> 2);
  const int h = (i & 3) >> 1;
#pragma unroll
  for (int c = 0; c < 4; ++c) fb.va[c] = ka * kRowBytes + 16 * ((2 * c + h) ^ swz(ka)) + 8 * (i & 1);
  return fb;
}

// K fragment (A operand of S^T = K Q^T): key 16 KT + l16, d = 32 KS + 8 g .. +8.
template <int KT, int KS>
__device__ __forceinline__ bf16x8 read_k(lds_u8* tile, const FragBases& fb) {
  return *(const bf16x8*)(tile + fb.k[KT][KS & 1] + 128 * (KS >> 1));
}

// The transposing-read builtin does not fold constant offsets, which makes the
// compiler keep one address register per column tile; this wrapper emits the
// instruction with its immediate offset.  Its result is not tracked by the
// compiler's LDS wait counting: use it only through wait_lds<N>(), which waits
// until at most N of the LDS reads issued after the needed one are outstanding
// (LDS reads complete in order) and ties the data to that wait.
template <int OFF>
__device__ __forceinline__ i32x2 ds_read_tr16_b64(const lds_u8* addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  i32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void wait_lds(i32x2& a, i32x2& b) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}

// V^T fragment for column tile CT as two tr16 pieces: lane (g, i) gets column
// 16 CT + i; element e is key 4 g + e (e < 4) or 16 + 4 g + e - 4.  In each
// 16-lane group of a transposing read, lane i points at a 4-element piece of
// one key row and lane j receives element j of every row of the block.
struct VRaw {
  i32x2 a, b;
};
template <int CT>
__device__ __forceinline__ void issue_v(VRaw& r, lds_u8* tile, const FragBases& fb) {
  r.a = ds_read_tr16_b64<128 * (CT >> 2)>(tile + fb.va[CT & 3]);
  r.b = ds_read_tr16_b64<128 * (CT >> 2) + 16 * kRowBytes>(tile + fb.va[CT & 3]);
}
__device__ __forceinline__ bf16x8 finish_v(const VRaw& r) {
  const i32x4 w = {r.a[0], r.a[1], r.b[0], r.b[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// ---- fp8 tiles (latent fp8, rope bf16)
//
// K fragment of the fp8 MFMA (A operand of S^T = K Q^T, 16 x 16 x 128): lane
// (g, m) holds key 16 kt + m, latent columns 128 b + 32 g .. +32 of block b,
// read as two 16-byte chunks.  Rope fragment (bf16 MFMA): key 16 kt + m,
// rope columns 32 DH + 8 g .. +8.  V^T fragment (8 keys x 1 column, one
// transposing 8-bit read): lane (g, i) gets column 16 ct + i, element e is key
// 4 g + e (e < 4) or 16 + 4 g + e - 4, as in the bf16 layout; in each 16-lane
// group lane 2 j + h points at key j's columns 16 ct + 8 h .. +8 and lane i
// receives byte i mod 8 of the lanes 2 j + i / 8.
struct FragBases8 {
  int k[2][2][2];  // [kt][block b of the wave's half][16-byte half s]
  int kr[2];       // [kt] rope
  int v;           // V: key row + 8 h + 16 swz8(key); column tile ct adds ^ (16 ct)
};

template <int DH>
__device__ __forceinline__ FragBases8 frag_bases8(int l16, int g) {
  FragBases8 fb;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = 16 * kt + l16;
    const int sw = swz8(key);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        fb.k[kt][b][h] = key * kLatBytes8 + 256 * DH + 16 * ((8 * b + 2 * g + h) ^ sw);
    fb.kr[kt] = kRopeOff8 + key * 128 + 16 * ((4 * DH + g) ^ rope_swz(key));
  }
  const int j = l16 >> 1, h = l16 & 1;
  const int kv = 16 * (j >> 2) + 4 * g + (j & 3);
  fb.v = kv * kLatBytes8 + 8 * h + 16 * swz8(kv);
  return fb;
}

template <int KT, int B>
__device__ __forceinline__ i32x8 read_k8(lds_u8* tile, const FragBases8& fb) {
  const i32x4 a = *(const i32x4*)(tile + fb.k[KT][B][0]);
  const i32x4 b = *(const i32x4*)(tile + fb.k[KT][B][1]);
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <int KT>
__device__ __forceinline__ bf16x8 read_kr(lds_u8* tile, const FragBases8& fb) {
  return *(const bf16x8*)(tile + fb.kr[KT]);
}

// V^T fragment of column tile 16 DH + CT (fp8 codes; see wait_lds1).
template <int DH, int CT>
__device__ __forceinline__ void issue_v8(i32x2& r, lds_u8* vbase) {
  lds_u8* a = (lds_u8*)((size_t)vbase ^ (size_t)(16 * CT));
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(256 * DH));
}
template <int N>
__device__ __forceinline__ void wait_lds1(i32x2& a) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N) : "memory");
}

// MFMAs through inline assembly with explicit register files: the compiler's
// own choice kept moving accumulators between register files every
// iteration.  Score MFMA: S^T (VGPRs, read by the softmax) += K . Q^T with Q
// in AGPRs.  O MFMA: O^T (AGPRs) += V^T . P^T.  Operands come from LDS reads
// (no VALU producer) except P, whose last VALU write is separated from its
// first use by an explicit s_nop in the caller; MFMA-result reads by VALU are
// preceded by s_nop margins.
template <bool ZERO, bool QA>
__device__ __forceinline__ void mfma_s(f32x4& acc, const bf16x8& k, const bf16x8& q) {
  if constexpr (ZERO && QA)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "a"(q));
  else if constexpr (ZERO)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "v"(q));
  else if constexpr (QA)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "a"(q));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "v"(q));
}
// Q fragment (rt, j) of a wave lives in AGPRs while they last: O takes
// 64 NRT AGPRs of the 256, Q fragments fill the rest in order, the remaining
// ones (only with NRT = 3) live in VGPRs.
template <int NRT>
constexpr bool q_in_agpr(int rt, int j) {
  return 64 * NRT + 4 * (rt * 9 + j + 1) <= 256;
}
// fp8 score MFMA, Q (fp8, per-row scaled) in VGPRs: it is computed by VALU
// instructions, and a VALU-defined operand in AGPRs became a copy per MFMA.
template <bool ZERO, bool QA = false>
__device__ __forceinline__ void mfma_s8(f32x4& acc, const i32x8& k, const i32x8& q) {
  if constexpr (ZERO && QA)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "a"(q));
  else if constexpr (ZERO)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "v"(q));
  else if constexpr (QA)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "a"(q));
  else
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mfma_o(f32x4& acc, const bf16x8& v, const bf16x8& p) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}
// fp8 KV: O^T += V^T . P^T with V as the cache's e4m3 codes and P as e4m3;
// both operands hold 8 keys per lane in the same order as the bf16 form.
__device__ __forceinline__ void mfma_o8(f32x4& acc, const i32x2& v, const i32x2& p) {
  asm volatile("v_mfma_f32_16x16x32_fp8_fp8 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}
// O = 0, defined in the AGPR file (an MFMA of zeros), so that no definition of
// O lives in VGPRs.  The zero operand is written by VALU moves just before:
// an MFMA must not read a VGPR within 2 wait states of its VALU write, and
// the compiler does not pad around inline assembly, hence the s_nop.
__device__ __forceinline__ void zero_o(f32x4& acc) {
  const bf16x8 z = {};
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=&a"(acc) : "v"(z));
}

// O *= f (rare: a softmax reference move), with whole-tuple accesses only so
// that O keeps its AGPR home: the tuple goes to a per-wave LDS area straight
// from its AGPRs, is scaled in VGPRs, and comes back into the same tuple.
// Each lane touches only its own 16 bytes.
__device__ __forceinline__ void scale_o(f32x4& acc, float f, lds_u8* spill) {
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(spill), "a"(acc) : "memory");
  typedef volatile __attribute__((address_space(3))) f32x4 lds_f32x4;
  const f32x4 t = *(lds_f32x4*)spill;
  *(lds_f32x4*)spill = t * f;
  asm volatile("s_waitcnt lgkmcnt(0)\n\tds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
               : "=a"(acc)
               : "v"(spill)
               : "memory");
}

// ---------------------------------------------------------- main kernel
//
// Per workgroup: a ring of 3 LDS tile slots and, per tile, one barrier.
// Iteration t of a unit (tile t's full scores are already in registers):
//   score phase   S^T MFMAs of tile t+1 (K from its slot), interleaved one by
//                 one with the softmax of tile t (VALU work runs while the
//                 MFMAs execute);
//   PV phase      O MFMAs of tile t (V from its slot), interleaved with the
//                 exchange write of tile t+1's partial scores and with the
//                 staging of tile t+2 (LDS store of a staged set, next loads);
//   barrier       partials and the new slot become visible, tile t's slot
//                 frees;
//   exchange read tile t+1's full scores = own partial + peer partial.
// The last iteration computes the scores of a tile past the end (stale slot
// contents, discarded).

// The fp8 kernels of 32- and 48-row row groups split each tile's keys between
// the two waves of a pair (unit_pipeline8k below) and keep four tiles in the
// ring.
template <bool FP8, int NRT>
constexpr bool key_split() { return FP8 && NRT >= 2; }
template <bool FP8, int NRT>
constexpr int ring_slots() { return key_split<FP8, NRT>() ? 4 : 3; }
// Bytes of the exchange area after the ring: two buffers of partial scores
// (16 NRT KB), or the key-split records and Q set-up slots (48 KB).
template <bool FP8, int NRT>
constexpr int exchange_bytes() { return key_split<FP8, NRT>() ? 49152 : 2 * kWaves * NRT * 2 * 1024; }
// Where the staging of tile t + 2 runs: bf16 KV between the score MFMAs
// (its PV phase already carries two transposing reads per column tile); fp8
// KV between the PV MFMAs (48 of them with one read per column tile and no
// VALU work, against 6 NRT score MFMAs that carry the softmax).
template <bool FP8>
constexpr bool stage_with_scores() { return !FP8; }


template <bool FP8, bool PAGED>
__device__ __forceinline__ KvSource<FP8, PAGED> kv_source(const UnitSetup& us) {
  KvSource<FP8, PAGED> src;
  src.base = us.kv_unit;
  src.pt_row = us.pt_row;
  src.lo = us.uc.lo;
  src.nkeys = us.uc.nkeys;
  src.shift = PAGED ? us.page_shift : 0;
  src.last_idx = PAGED ? us.last_page_idx : 0;
  src.max_page = PAGED ? (unsigned)(us.num_pages - 1) : 0u;
  return src;
}

// One Q fragment (MFMA B operand) straight from memory into its register file.
template <bool QA>
__device__ __forceinline__ void load_q_frag(bf16x8& dst, int off, __amdgpu_buffer_rsrc_t r) {
  if constexpr (QA)
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=a"(dst) : "v"(off), "s"(r));
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(dst) : "v"(off), "s"(r));
}

// Q fragments: row grow0 + 16 rt + l16, d = 288 DH + 32 j + 8 g.  Rows past the
// unit read as zero (range-checked descriptor).
template <int NRT, int DH>
__device__ __forceinline__ void load_q(const UnitSetup& us, int grow0, int l16, int g,
                                       bf16x8 (&qf)[NRT][9]) {
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(us.q + (int64_t)us.row0 * kDqk, (uint32_t)(us.RU * kDqk * 2));
  static_for<NRT>([&](auto rc) {
    constexpr int rt = decltype(rc)::value;
    const int row = grow0 + 16 * rt + l16;
    static_for<9>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      load_q_frag<q_in_agpr<NRT>(rt, j)>(qf[rt][j], row * (kDqk * 2) + DH * 576 + j * 64 + g * 16,
                                          qr);
    });
  });
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// l_run: per-lane partial row sums (summed across the lane groups here), or
// with TOTAL the rows' whole sums already.
template <int NRT, int DH, bool TOTAL = false>
__device__ __forceinline__ void epilogue(const UnitSetup& us, int grow0,
                                         int l16, int g, f32x4 (&oacc)[16][NRT],
                                         const float (&m_run)[NRT], const float (&l_run)[NRT]) {
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // last O MFMA retired before reads
  const float ln2 = 0.69314718055994530942f;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float lt = TOTAL ? l_run[rt] : wave_sum_across_groups(l_run[rt]);
    const int row = grow0 + 16 * rt + l16;
    const bool valid = row < us.RU;
    if (us.S == 1) {
      // a row that sees no key (only possible for a key shard): O = 0, LSE = -inf
      const bool empty = !(lt > 0.0f);
      const float inv = empty ? 0.0f : us.o_scale / lt;
      const int64_t orow = (int64_t)us.row0 + row;
      if (valid) {
        uint16_t* op = us.o + orow * kDv + 256 * DH + 4 * g;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const f32x4 o4 = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : oacc[c][rt] * inv;
          uint2 pk;
          pk.x = pack_bf16x2(o4[0], o4[1]);
          pk.y = pack_bf16x2(o4[2], o4[3]);
          *(uint2*)(op + 16 * c) = pk;
        }
        if (g == 0 && DH == 0)
          us.lse[orow] = empty ? -INFINITY : (m_run[rt] + log2f(lt)) * ln2;
      }
    } else {
      const int64_t prow =
          (int64_t)us.part_row0 + ((int64_t)us.t * us.S + us.s) * us.R + us.rowb0 + row;
      const bool empty = !(lt > 0.0f);
      const float inv = empty ? 0.0f : us.o_scale / lt;
      if (valid) {
        uint16_t* pp = us.part_o + prow * kDv + 256 * DH + 4 * g;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const f32x4 o4 = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : oacc[c][rt] * inv;
          uint2 pk;
          pk.x = pack_bf16x2(o4[0], o4[1]);
          pk.y = pack_bf16x2(o4[2], o4[3]);
          *(uint2*)(pp + 16 * c) = pk;
        }
        if (g == 0 && DH == 0)
          us.part_lse[prow] = empty ? -INFINITY : (m_run[rt] + log2f(lt)) * ln2;
      }
    }
  }
}

// Call f(i) for the slices i of a phase that go after MFMA number `pos` when
// `nslices` slices are spread over `nmfma` MFMAs.
template <int NSLICES, int NMFMA, int POS, typename F>
__device__ __forceinline__ void slices_at(F&& f) {
  static_for<NSLICES>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int at = (s * NMFMA) / NSLICES;
    if constexpr (at == POS) f(sc);
  });
}

// LDS read-ahead: K steps and V column tiles in flight ahead of the MFMA that
// needs them, as deep as the register budget of each row-tile count allows
// (one step is 2 NRT MFMAs, one column tile NRT MFMAs).
template <int NRT, bool FP8>
constexpr int k_ahead() { return NRT == 1 ? 4 : NRT == 2 ? 2 : 1; }
template <int NRT, bool FP8>
constexpr int v_ahead() { return NRT == 1 ? 7 : FP8 ? (NRT == 2 ? 6 : 2) : (NRT == 2 ? 4 : 2); }

// Score phase: S^T partial (this wave's 288 columns) of one tile; K fragments
// DK steps ahead; pre(i) runs before MFMA i and slice(i) after it.
template <int NRT, int DH, int DK, typename P, typename W>
__device__ __forceinline__ void score_phase(lds_u8* tile, const FragBases& fb,
                                            const bf16x8 (&qf)[NRT][9], f32x4 (&sacc)[2][NRT],
                                            P&& pre, W&& slice) {
  bf16x8 kf[DK + 1][2];
  static_for<DK>([&](auto sc) {
    constexpr int j = decltype(sc)::value;
    kf[j][0] = read_k<0, 9 * DH + j>(tile, fb);
    kf[j][1] = read_k<1, 9 * DH + j>(tile, fb);
  });
  static_for<9>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int cur = j % (DK + 1);
    if constexpr (j + DK < 9) {
      kf[(j + DK) % (DK + 1)][0] = read_k<0, 9 * DH + j + DK>(tile, fb);
      kf[(j + DK) % (DK + 1)][1] = read_k<1, 9 * DH + j + DK>(tile, fb);
    }
    static_for<2 * NRT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int kt = i / NRT, rt = i % NRT;
      pre(std::integral_constant<int, j * 2 * NRT + i>{});
      mfma_s<j == 0, q_in_agpr<NRT>(rt, j)>(sacc[kt][rt], kf[cur][kt], qf[rt][j]);
      slice(std::integral_constant<int, j * 2 * NRT + i>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// Issue the V reads of column tiles 0 .. DV-1 (of this wave's half).
template <int DH, int DV>
__device__ __forceinline__ void issue_v_head(VRaw (&vr)[DV + 1], lds_u8* tile, const FragBases& fb) {
  static_for<DV>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    issue_v<16 * DH + c>(vr[c], tile, fb);
  });
}

// PV phase: O^T[256 DH + ...] += V^T P^T of one tile; V fragments DV column
// tiles ahead (the first DV issued by the caller); slice(i) runs after MFMA i.
template <int NRT, int DH, int DV, typename W>
__device__ __forceinline__ void pv_phase(lds_u8* tile, const FragBases& fb,
                                         const bf16x8 (&pf)[NRT], f32x4 (&oacc)[16][NRT],
                                         VRaw (&vr)[DV + 1], W&& slice) {
  static_assert(DV >= 1 && 2 * DV < 16, "read-ahead depth");
  asm volatile("s_nop 1" ::: "memory");  // last VALU write of P before the first O MFMA
  static_for<16>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    constexpr int cur = c % (DV + 1);
    if constexpr (c + DV < 16) {
      issue_v<16 * DH + c + DV>(vr[(c + DV) % (DV + 1)], tile, fb);
      wait_lds<2 * DV>(vr[cur].a, vr[cur].b);
    } else {
      wait_lds<2 * (15 - c)>(vr[cur].a, vr[cur].b);
    }
    const bf16x8 vf = finish_v(vr[cur]);
    static_for<NRT>([&](auto rc) {
      constexpr int rt = decltype(rc)::value;
      mfma_o(oacc[c][rt], vf, pf[rt]);
      slice(std::integral_constant<int, c * NRT + rt>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// fp8 score phase: S^T partial of one tile from this wave's two 128-column
// latent blocks (fp8 MFMAs, 2 NRT each) and its 32 rope columns (bf16 MFMAs,
// accumulated last: at least one independent MFMA separates each from the fp8
// MFMA that wrote its accumulator); pre(i) runs before MFMA i, slice(i) after.
template <int NRT>
struct QFrag8 {
  i32x8 lat[NRT][2];  // fp8 codes of Q / s_row, latent block 2 DH + b
  bf16x8 rope[NRT];   // bf16 of Q / s_row, rope columns 32 DH + 8 g .. +8 (AGPRs)
};

template <int NRT, int DH, typename P, typename W>
__device__ __forceinline__ void score_phase8(lds_u8* tile, const FragBases8& fb, const QFrag8<NRT>& q8,
                                             f32x4 (&sacc)[2][NRT], P&& pre, W&& slice) {
  i32x8 kl[2][2];  // [block][kt]
  bf16x8 kr[2];
  kl[0][0] = read_k8<0, 0>(tile, fb);
  kl[0][1] = read_k8<1, 0>(tile, fb);
  static_for<3>([&](auto sc) {
    constexpr int st = decltype(sc)::value;
    if constexpr (st == 0) {
      kl[1][0] = read_k8<0, 1>(tile, fb);
      kl[1][1] = read_k8<1, 1>(tile, fb);
    } else if constexpr (st == 1) {
      kr[0] = read_kr<0>(tile, fb);
      kr[1] = read_kr<1>(tile, fb);
    }
    static_for<2 * NRT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int kt = i / NRT, rt = i % NRT;
      pre(std::integral_constant<int, st * 2 * NRT + i>{});
      if constexpr (st < 2)
        mfma_s8<st == 0>(sacc[kt][rt], kl[st][kt], q8.lat[rt][st]);
      else
        mfma_s<false, true>(sacc[kt][rt], kr[kt], q8.rope[rt]);
      slice(std::integral_constant<int, st * 2 * NRT + i>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

template <int DH, int DV, int NSL>
__device__ __forceinline__ void issue_v_head8(i32x2 (&vr)[NSL], lds_u8* vbase) {
  static_for<DV>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    issue_v8<DH, c>(vr[c], vbase);
  });
}

// fp8 PV phase: as pv_phase, with one 8-bit transposing read per V fragment
// feeding the fp8 MFMA directly (P is e4m3 too).  The read ring has DV + 2
// slots, so a read never targets the registers of the column tile whose
// MFMAs were issued just before it.
template <int DV>
constexpr int v8_slots() { return DV + 2; }

template <int NRT, int DH, int DV, typename W>
__device__ __forceinline__ void pv_phase8(lds_u8* vbase, const i32x2 (&pf)[NRT],
                                          f32x4 (&oacc)[16][NRT], i32x2 (&vr)[v8_slots<DV>()],
                                          W&& slice) {
  static_assert(DV >= 1 && DV < 15, "read-ahead depth");
  constexpr int NSL = v8_slots<DV>();
  asm volatile("s_nop 1" ::: "memory");  // last VALU write of P before the first O MFMA
  static_for<16>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    constexpr int cur = c % NSL;
    if constexpr (c + DV < 16) {  // reads 0 .. DV-1 were issued before the score phase
      issue_v8<DH, c + DV>(vr[(c + DV) % NSL], vbase);
      wait_lds1<DV>(vr[cur]);
    } else {
      wait_lds1<15 - c>(vr[cur]);
    }
    static_for<NRT>([&](auto rc) {
      constexpr int rt = decltype(rc)::value;
      mfma_o8(oacc[c][rt], vr[cur], pf[rt]);
      slice(std::integral_constant<int, c * NRT + rt>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// Online softmax of one tile (base 2) with a lazy per-row reference m_run:
// P = 2^(c s - m_run) with c = sm_scale * kv_scale * log2(e) > 0 (fp8: times the
// row's Q scale, c is per row); the first
// tile that shows a row a key sets its reference, which moves only when a
// tile maximum exceeds it by more than lazy_octaves (then O and l are
// rescaled: rare).  Whether any row of the wave needs that is decided from
// each lane's own maximum over its 8 keys (a row's maximum exceeds a bound
// exactly when one of its lanes' does), so the cross-lane row maximum is only
// formed on that rare path (and on a row's first tile).  The work is cut into
// small slices that run between the MFMAs of the other phase: the edge mask,
// one lane-maximum slice per row tile, the wave vote, 4 slices of 2 keys per
// row tile for P, and the row sums.  The maximum is taken on raw scores
// (c > 0 keeps the order) and c is folded into one FMA per key.
template <int NRT>
constexpr int soft_slices() { return 5 * NRT + 3; }

template <int NRT>
struct SoftTile {
  float mx[NRT], nmu[NRT], psum[NRT];
  bool jump;
};

template <int NRT, int PH, typename PT>
__device__ __forceinline__ void softmax_slice(SoftTile<NRT>& w, f32x4 (&sfull)[2][NRT],
                                              PT (&pf)[NRT], float (&m_run)[NRT],
                                              float (&l_run)[NRT], f32x4 (&oacc)[16][NRT],
                                              const int (&lim)[NRT], int k0, bool edge,
                                              const float (&c)[NRT], int g, lds_u8* spill) {
  constexpr bool kFp8P = std::is_same<PT, i32x2>::value;
  constexpr float kLazy = lazy_octaves<kFp8P>();
  if constexpr (PH == 0) {  // keys past a row's causal limit (last tiles of a chunk only)
    w.jump = false;
    if (edge) {
      asm volatile("" ::: "memory");  // keep this a branch: interior tiles skip it
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 16 * kt + 4 * g + i;
            sfull[kt][rt][i] = key <= lim[rt] ? sfull[kt][rt][i] : -INFINITY;
          }
    }
  } else if constexpr (PH <= NRT) {  // lane maximum over its 8 keys; does it pass the bound?
    constexpr int rt = PH - 1;
    const f32x4 a = sfull[0][rt], b = sfull[1][rt];
    w.mx[rt] = max2(max3(a[0], a[1], a[2]), max3(a[3], b[0], max3(b[1], b[2], b[3])));
    w.jump = w.jump || w.mx[rt] * c[rt] > m_run[rt] + kLazy;
  } else if constexpr (PH == NRT + 1) {  // wave vote; rare: row maxima, references, rescale
    if (__builtin_amdgcn_ballot_w64(w.jump) != 0) {  // wave-uniform
      asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // O MFMAs retired
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float mx = wave_max_across_groups(w.mx[rt]) * c[rt];
        const bool first = m_run[rt] == -INFINITY;  // O and l are still 0
        const bool jump = !first && mx > m_run[rt] + kLazy;
        if (__builtin_amdgcn_ballot_w64(jump) != 0) {
          const float f = jump ? __builtin_amdgcn_exp2f(m_run[rt] - mx) : 1.0f;
          l_run[rt] *= f;
#pragma unroll
          for (int cc = 0; cc < 16; ++cc) scale_o(oacc[cc][rt], f, spill);
        }
        m_run[rt] = (first && mx > -INFINITY) || jump ? mx : m_run[rt];
        w.nmu[rt] = m_run[rt] == -INFINITY ? 0.0f : -m_run[rt];
        // settle both here: merged after the branch they would be selected on
        // every tile
        asm volatile("" : "+v"(m_run[rt]), "+v"(w.nmu[rt]));
      }
    }
  } else if constexpr (PH < 5 * NRT + 2) {  // P of 2 keys of one row tile: c s - m <= kLazy
    constexpr int j = PH - (NRT + 2);
    constexpr int rt = j / 4, kt = (j / 2) % 2, h = j % 2;
    // v_exp_f32: results below the fp32 normal range flush to 0
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sfull[kt][rt][2 * h], c[rt], w.nmu[rt]));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sfull[kt][rt][2 * h + 1], c[rt], w.nmu[rt]));
    w.psum[rt] = (j % 4 == 0) ? p0 + p1 : w.psum[rt] + (p0 + p1);
    if constexpr (kFp8P)  // keys 16 kt + 4 g + 2 h, +1 -> bytes 2 h, 2 h + 1 of dword kt
      pf[rt][kt] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[rt][kt], h != 0);
    else {
      pf[rt][4 * kt + 2 * h] = (__bf16)p0;
      pf[rt][4 * kt + 2 * h + 1] = (__bf16)p1;
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) l_run[rt] += w.psum[rt];
  }
}

// A row group with no row of the unit only takes its share of the staging
// (same loads, stores and barriers as unit_pipeline, no LDS reads, no MFMAs).
// It is a separate loop, so its staged registers never meet the other's.
// Page rows of tiles 0 .. N-1 (paged KV; prologue).
template <int N, bool FP8, bool PAGED>
__device__ __forceinline__ void prologue_page_rows(const KvSource<FP8, PAGED>& src, int64_t (&pr)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) pr[k] = PAGED ? src.page_row_now(k) : 0;
}

template <bool FP8, int NRT, bool PAGED, bool NT>
__device__ __forceinline__ void unit_staging_only_regs(const UnitSetup& us, lds_u8* lds, int tid) {
  constexpr int NS = stage_sets<FP8, NRT>();
  constexpr int kAhead = (NS - 1) * kPieces;
  const UnitCtx u = us.uc;
  const KvSource<FP8, PAGED> src = kv_source<FP8, PAGED>(us);
  if (u.ntiles <= 0) return;
  int64_t pr[NS + 3];
  prologue_page_rows(src, pr);
  Stage<FP8> st[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) stage_load<FP8, NT>(st[k], src.rsrc(k, pr[k]), tid);
  static_for<2>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    wait_stage<kAhead, FP8>(st[j % NS]);
    stage_store<FP8>(st[j % NS], lds + j * tile_bytes<FP8>(), tid);
    stage_load<FP8, NT>(st[j % NS], src.rsrc(j + NS, pr[j + NS]), tid);
  });
  lds_barrier();
  lds_barrier();  // the exchange of tile 0's scores
  int64_t prow_next = pr[NS + 2];  // page row of the first tile the loop loads
  for (int base = 0; base < u.ntiles; base += NS) {
    static_for<NS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ks = (k + 2) % NS;
      const int t = base + k;
      if (t < u.ntiles) {
        wait_stage<kAhead, FP8>(st[ks]);
        stage_store<FP8>(st[ks], lds + ((t + 2) % ring_slots<FP8, NRT>()) * tile_bytes<FP8>(), tid);
        stage_load<FP8, NT>(st[ks], src.rsrc(t + 2 + NS, prow_next), tid);
        if constexpr (PAGED)
          prow_next = src.barrier_and_page_row(t + 3 + NS);
        else
          lds_barrier();
      }
    });
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads issued past the end
}

template <bool FP8, int NRT, bool PAGED, bool NT>
__device__ __forceinline__ void unit_staging_only(const UnitSetup& us, lds_u8* lds, int tid) {
  if constexpr (tile_dma_path<FP8, NRT>()) {  // LDS DMA: this wave's share of every tile, same waits and barriers
    const UnitCtx u = us.uc;
    const KvSource<FP8, PAGED> src = kv_source<FP8, PAGED>(us);
    if (u.ntiles <= 0) return;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const TileDma dm = tile_dma(wave, tid & 63);
    int64_t pr[3];
    prologue_page_rows(src, pr);
    tile_dma_all<NT>(lds, wave, dm, src.rsrc(0, pr[0]));
    tile_dma_all<NT>(lds + kTileBytes, wave, dm, src.rsrc(1, pr[1]));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    lds_barrier();  // the exchange of tile 0's scores
    int64_t prow_next = pr[2];  // page row of tile 2, the first the loop loads
    for (int t = 0; t < u.ntiles; ++t) {
      tile_dma_all<NT>(lds + ((t + 2) % 3) * kTileBytes, wave, dm, src.rsrc(t + 2, prow_next));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (PAGED)
        prow_next = src.barrier_and_page_row(t + 3);
      else
        lds_barrier();
    }
  } else {
    unit_staging_only_regs<FP8, NRT, PAGED, NT>(us, lds, tid);
  }
}

// The whole KV chunk of a unit, software-pipelined as described above.  The
// tile loop is unrolled by the number of staging sets so that set k always
// holds tiles = k mod NS; every global load and wait is unconditional (tiles
// past the end load nothing), so the staged registers never need a copy while
// their loads are in flight (the compiler does not know that an
// inline-assembly load completes later).
template <bool FP8, int NRT, int DH, bool PAGED, bool NT, typename FB, typename QT>
__device__ __forceinline__ void unit_pipeline(const UnitSetup& us, lds_u8* lds, float* xs,
                                              int wave, const FB& fb, const QT& qf,
                                              const float (&c)[NRT], f32x4 (&oacc)[16][NRT],
                                              float (&m_run)[NRT], float (&l_run)[NRT],
                                              const int (&lim)[NRT], int tid, int g, int lane) {
  constexpr bool kDma = tile_dma_path<FP8, NRT>();
  constexpr int NS = kDma ? 1 : stage_sets<FP8, NRT>();
  constexpr int kAhead = (NS - 1) * kPieces;  // loads issued after a set's own
  constexpr int kXsWave = NRT * 2 * 256;      // floats of one wave's partial scores
  constexpr int DK = k_ahead<NRT, FP8>(), DV = v_ahead<NRT, FP8>();
  constexpr int TB = tile_bytes<FP8>();
  const UnitCtx u = us.uc;
  const KvSource<FP8, PAGED> src = kv_source<FP8, PAGED>(us);
  if (u.ntiles <= 0) return;

  // prologue: tiles 0 and 1 into their slots (register staging: tile k always
  // travels in set k % NS)
  int64_t pr[NS + 3];
  prologue_page_rows(src, pr);
  Stage<FP8> st[NS];
  TileDma dm;
  int64_t prow_next;  // page row of the first tile the loop loads
  if constexpr (kDma) {
    dm = tile_dma(wave, lane);
    tile_dma_all<NT>(lds, wave, dm, src.rsrc(0, pr[0]));
    tile_dma_all<NT>(lds + TB, wave, dm, src.rsrc(1, pr[1]));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    prow_next = pr[2];
  } else {
#pragma unroll
    for (int k = 0; k < NS; ++k) stage_load<FP8, NT>(st[k], src.rsrc(k, pr[k]), tid);
    static_for<2>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      wait_stage<kAhead, FP8>(st[j % NS]);
      stage_store<FP8>(st[j % NS], lds + j * TB, tid);
      stage_load<FP8, NT>(st[j % NS], src.rsrc(j + NS, pr[j + NS]), tid);
    });
    lds_barrier();
    prow_next = pr[NS + 2];
  }

  f32x4 sacc[2][NRT], sfull[2][NRT];
  auto scores = [&](lds_u8* tile, auto&& pre, auto&& slice) {
    if constexpr (FP8)
      score_phase8<NRT, DH>(tile, fb, qf, sacc, pre, slice);
    else
      score_phase<NRT, DH, DK>(tile, fb, qf, sacc, pre, slice);
  };

  // full scores of tile 0
  scores(lds, [](auto) {}, [](auto) {});
  asm volatile("s_nop 15\n\ts_nop 7" ::: "memory");  // score MFMAs retire before the reads
  {
    float* mine = xs + wave * kXsWave;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        *(f32x4*)(mine + ((rt * 2 + kt) * 64 + lane) * 4) = sacc[kt][rt];
  }
  lds_barrier();
  {  // the partner's half of the scores; this wave's half is added in the loop
    const float* peer = xs + (wave ^ 1) * kXsWave;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        sfull[kt][rt] = *(const f32x4*)(peer + ((rt * 2 + kt) * 64 + lane) * 4);
  }

  typename std::conditional<FP8, i32x2, VRaw>::type vr[FP8 ? v8_slots<DV>() : DV + 1];
  typename std::conditional<FP8, i32x2, bf16x8>::type pf[NRT];  // P^T: e4m3 with fp8 KV
  SoftTile<NRT> sw;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) sw.nmu[rt] = 0.0f;  // references not set yet (m_run = -inf)
  for (int base = 0; base < u.ntiles; base += NS) {
    static_for<NS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ks = (k + 2) % NS;  // staging set of tile t + 2
      const int t = base + k;
      if (t < u.ntiles) {
        const int par = (t + 1) & 1;  // exchange buffer of tile t + 1
        float* mine = xs + (par * kWaves + wave) * kXsWave;
        const float* peer = xs + (par * kWaves + (wave ^ 1)) * kXsWave;
        lds_u8* spill = (lds_u8*)mine + lane * 16;  // free until the exchange write below
        constexpr int RING = ring_slots<FP8, NRT>();
        lds_u8* slot_t = lds + (t % RING) * TB;
        lds_u8* slot_n = lds + ((t + 1) % RING) * TB;
        lds_u8* slot_s = lds + ((t + 2) % RING) * TB;
        const int k0 = t * kTK;
        const bool edge = k0 + kTK - 1 > u.min_lim;
        // DMA: tile t + 2 into the slot of tile t - 1; staging: loads of tile t + 2 + NS
        const __amdgpu_buffer_rsrc_t rs_next = src.rsrc(kDma ? t + 2 : t + 2 + NS, prow_next);
        lds_u8* vbase = nullptr;  // fp8: V reads of tile t (column tile ct adds ^ 16 ct)
        if constexpr (FP8) {
          vbase = slot_t + fb.v;
          issue_v_head8<DH, DV>(vr, vbase);
        } else {
          issue_v_head<DH, DV>(vr, slot_t, fb);
        }

        // tile t + 2 into its slot: the 9 DMA loads of this wave, or (register
        // staging) wait for its loads, LDS store, next loads
        constexpr int kStageSlices = kDma ? kPieces : 1 + 2 * kPieces;
        auto stage_slice = [&](auto sc) {
          constexpr int s = decltype(sc)::value;
          if constexpr (kDma) {
            tile_dma_piece<NT>(slot_s, s, wave, dm.off[s], rs_next);
          } else if constexpr (s == 0) {
            wait_stage<kAhead, FP8>(st[ks]);
          } else if constexpr (s < 1 + kPieces) {
            stage_store_piece<FP8, s - 1>(st[ks], slot_s, tid);
          } else {
            stage_load_piece<FP8, s - 1 - kPieces, NT>(st[ks], rs_next, tid);
          }
        };

        // scores of tile t + 1  ||  softmax of tile t (and the staging); before
        // the first MFMAs overwrite this wave's half of tile t's scores, it is
        // added to the partner's half read after the last barrier
        constexpr int kScoreMfma = (FP8 ? 6 : 18) * NRT;
        constexpr int kAdd = 2 * NRT;  // MFMAs of the first step
        auto add_own = [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i < kAdd) sfull[i / NRT][i % NRT] += sacc[i / NRT][i % NRT];
        };
        scores(slot_n, add_own, [&](auto ic) {
          constexpr int i = decltype(ic)::value;  // slices start once tile t's scores are whole
          slices_at<soft_slices<NRT>(), kScoreMfma - kAdd + 1, i - kAdd + 1>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            softmax_slice<NRT, s>(sw, sfull, pf, m_run, l_run, oacc, lim, k0, edge, c, g, spill);
          });
          if constexpr (stage_with_scores<FP8>()) slices_at<kStageSlices, kScoreMfma, i>(stage_slice);
        });

        // O of tile t  ||  exchange write of tile t + 1 (and the staging)
        constexpr int kPvMfma = 16 * NRT;
        auto pv_slice = [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          slices_at<NRT, kPvMfma, i>([&](auto sc) {  // partial scores of tile t + 1
            constexpr int s = decltype(sc)::value;
            if constexpr (s == 0) asm volatile("s_nop 15" ::: "memory");
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
              *(f32x4*)(mine + ((s * 2 + kt) * 64 + lane) * 4) = sacc[kt][s];
          });
          if constexpr (!stage_with_scores<FP8>()) slices_at<kStageSlices, kPvMfma, i>(stage_slice);
        };
        if constexpr (FP8)
          pv_phase8<NRT, DH, DV>(vbase, pf, oacc, vr, pv_slice);
        else
          pv_phase<NRT, DH, DV>(slot_t, fb, pf, oacc, vr, pv_slice);

        if constexpr (kDma) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t + 2 landed
        if constexpr (PAGED)
          prow_next = src.barrier_and_page_row(kDma ? t + 3 : t + 3 + NS);
        else
          lds_barrier();
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            sfull[kt][rt] = *(const f32x4*)(peer + ((rt * 2 + kt) * 64 + lane) * 4);
      }
    });
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads issued past the end
}

// fp8 Q: per row, the latent columns are quantised to e4m3 with the scale
// s = max(max |q latent|, 2^-64 max |q rope|) / 448 (round to nearest even; the
// row's scores then carry the factor s, folded into the row's softmax
// constant c = c0 s), the rope columns become bf16 of q / s (the rope term of
// the scale keeps q / s finite when the latent part is vanishingly small).  The two waves of a pair hold halves of each
// row and agree on s through LDS (one barrier, taken by every wave of the
// workgroup).  Rows past the unit read row RU - 1 (their outputs are never
// written).
template <int NRT, int DH>
__device__ __forceinline__ void load_q8(const UnitSetup& us, int grow0, int l16, int g, int wave,
                                        float* xs, QFrag8<NRT>& q8, float (&c)[NRT]) {
  u32x4 lat[NRT][2][4], rope[NRT];
  float half_max[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = min(grow0 + 16 * rt + l16, us.RU - 1);
    const uint16_t* qrow = us.q + ((int64_t)us.row0 + row) * kDqk;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lat[rt][b][i] = *(const u32x4*)(qrow + 256 * DH + 128 * b + 32 * g + 8 * i);
    rope[rt] = *(const u32x4*)(qrow + 512 + 32 * DH + 8 * g);
  }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    float m = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned x = lat[rt][b][i][w];
          m = fmaxf(m, fmaxf(fabsf(__builtin_bit_cast(float, x << 16)),
                             fabsf(__builtin_bit_cast(float, x & 0xffff0000u))));
        }
    float mr = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned x = rope[rt][w];
      mr = fmaxf(mr, fmaxf(fabsf(__builtin_bit_cast(float, x << 16)),
                           fabsf(__builtin_bit_cast(float, x & 0xffff0000u))));
    }
    m = fmaxf(m, mr * 0x1p-64f);
    half_max[rt] = wave_max_across_groups(m);
    if (g == 0) xs[(wave * NRT + rt) * 16 + l16] = half_max[rt];
  }
  lds_barrier();
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float M = fmaxf(half_max[rt], xs[((wave ^ 1) * NRT + rt) * 16 + l16]);
    const float inv = q8_inv_scale(M);
    c[rt] = us.scale_log2 / inv;
    auto q = [&](unsigned bits) {  // bf16 bits -> q / s, inside the e4m3 range
      return __builtin_bit_cast(float, bits) * inv;
    };
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // dword k: elements 4 k .. 4 k + 3 of the lane's 32
        const unsigned x0 = lat[rt][b][k >> 1][2 * (k & 1)], x1 = lat[rt][b][k >> 1][2 * (k & 1) + 1];
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q(x0 << 16), q(x0 & 0xffff0000u), 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q(x1 << 16), q(x1 & 0xffff0000u), v, true);
        q8.lat[rt][b][k] = v;
      }
    bf16x8 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned x = rope[rt][w];
      r[2 * w] = (__bf16)(__builtin_bit_cast(float, x << 16) * inv);
      r[2 * w + 1] = (__bf16)(__builtin_bit_cast(float, x & 0xffff0000u) * inv);
    }
    // the rope fragment moves to its AGPR home through LDS (a lane-private
    // 16-byte slot in the second half of the 16 NRT KB exchange area, past the
    // scale exchange), so no VGPR copy of it stays live
    static_assert(8192 * NRT + kWaves * NRT * 64 * 16 <= 2 * kWaves * NRT * 2 * 1024, "exchange area");
    lds_u8* slot = (lds_u8*)xs + 8192 * NRT + ((wave * NRT + rt) * 64 + (threadIdx.x & 63)) * 16;
    *(bf16x8*)slot = r;
    asm volatile("s_waitcnt lgkmcnt(0)\n\tds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=a"(q8.rope[rt]) : "v"(slot) : "memory");
  }
}

// ------------------------------------------------ fp8 KV, 48-row row groups
//
// The two waves of a pair split each tile's 32 keys instead of the score
// columns: wave dh computes the full 576-column scores of keys 16 dh .. +15,
// so no fp32 score exchange is needed and each wave forms the softmax of its
// own 16 keys only.  Per row tile and lane the pair exchanges one lane maximum
// (both waves then take the same reference decisions) and one dword of e4m3
// P (the partner's half of the PV operand: byte e of lane group g is key
// 4 g + e of the kt = 0 half for e < 4 and of the kt = 1 half otherwise).
// The PV of tile t runs in iteration t + 1, after the barrier that publishes
// the partner's P(t); a four-slot ring keeps tile t's V meanwhile.  A
// reference move found by the softmax of tile t rescales O after the PV of
// tile t - 1, whose P was formed against the old reference (the deferred O
// rescale of the r52 kernel in "bench(cake_mla_varq_dcp_decode): drop the
// package README and add a query-pattern benchmark option" (flashinfer PR
// #5588), embedded follow-up, section "Summary").

// K fragments of the wave's own 16 keys at full depth: latent block b (fp8
// MFMA A operand, columns 128 b + 32 g .. +32 as two 16-byte chunks) and rope
// half h (bf16 MFMA, rope columns 32 h + 8 g .. +8); V as FragBases8.
struct FragBases8K {
  int k[4][2];
  int kr[2];
  int v;
};

template <int DH>
__device__ __forceinline__ FragBases8K frag_bases8k(int l16, int g) {
  FragBases8K fb;
  const int key = 16 * DH + l16;
  const int sw = swz8(key);
  // the swizzle touches the low 4 bits of the chunk index only, so blocks 2
  // and 3 sit 256 bytes past blocks 0 and 1 (an immediate offset)
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      fb.k[b][h] = key * kLatBytes8 + 16 * ((8 * b + 2 * g + h) ^ sw);
      fb.k[b + 2][h] = fb.k[b][h] + 256;
    }
#pragma unroll
  for (int h = 0; h < 2; ++h) fb.kr[h] = kRopeOff8 + key * 128 + 16 * ((4 * h + g) ^ rope_swz(key));
  const int j = l16 >> 1, h = l16 & 1;
  const int kv = 16 * (j >> 2) + 4 * g + (j & 3);
  fb.v = kv * kLatBytes8 + 8 * h + 16 * swz8(kv);
  return fb;
}

template <int B>
__device__ __forceinline__ i32x8 read_k8k(lds_u8* tile, const FragBases8K& fb) {
  const i32x4 a = *(const i32x4*)(tile + fb.k[B][0]);
  const i32x4 b = *(const i32x4*)(tile + fb.k[B][1]);
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <int H>
__device__ __forceinline__ bf16x8 read_kr8k(lds_u8* tile, const FragBases8K& fb) {
  return *(const bf16x8*)(tile + fb.kr[H]);
}

// Latent blocks 0..2 in VGPRs, block 3 in AGPRs (with the 192 AGPRs of O and
// the rope fragments, what the register files hold).
template <int NRT>
struct QFrag8K {
  i32x8 lat[NRT][4];    // e4m3 codes of Q / s_row, latent block b (b = 3: AGPRs)
  bf16x8 rope[NRT][2];  // bf16 of Q / s_row, rope columns 32 h + 8 g .. +8 (AGPRs)
};
template <int B>
constexpr bool lat_in_agpr() { return B == 3; }

// LDS records of the key-split pipeline inside the exchange area (16 bytes
// per lane): lane maxima [2 parities][waves][64], e4m3 P [2][waves][64], the
// row sums at the end [waves][64] and a per-wave spill slot for the O rescale.
constexpr int kXmOff = 0;
constexpr int kXpOff = 2 * kWaves * 64 * 16;
constexpr int kXlOff = kXpOff + 2 * kWaves * 64 * 16;
constexpr int kSpillOff = kXlOff + kWaves * 64 * 16;
static_assert(kSpillOff + kWaves * 64 * 16 <= 49152, "key-split records fit the exchange area");

// fp8 Q at full depth, quantised once per pair: wave dh quantises latent
// blocks 2 dh, 2 dh + 1 and rope half dh of its rows (the scale rule of
// load_q8, from the whole row: the pair first exchanges its half maxima) and
// the two halves are swapped through LDS.  The exchange lives in the tile
// ring, which no wave writes before the pipeline's prologue; the last barrier
// here keeps the staging of tiles 0 and 1 behind every wave's reads.
constexpr int kQxMaxBytes = 4096;  // half maxima [waves][NRT][64] fp32
constexpr int kQxRec = 80;         // per lane and row tile: 2 latent blocks + rope half

template <int NRT, int DH>
__device__ __forceinline__ void load_q8k(const UnitSetup& us, int grow0, int l16, int g, int wave,
                                         lds_u8* ring, QFrag8K<NRT>& q8, float (&c)[NRT]) {
  static_assert(kWaves * NRT * 64 * 4 <= kQxMaxBytes, "half maxima");
  static_assert(kQxMaxBytes + kWaves * NRT * 64 * kQxRec <= 4 * kTileBytes8, "Q exchange in the ring");
  const int lane = threadIdx.x & 63;
  typedef __attribute__((address_space(3))) float lds_f32;
  lds_f32* xmax = (lds_f32*)ring;
  auto rec = [&](int w, int rt) { return ring + kQxMaxBytes + ((w * NRT + rt) * 64 + lane) * kQxRec; };
  u32x4 lat[NRT][2][4], rope[NRT];
  float hm[NRT];
  auto amax2 = [](float m, unsigned x) {
    return fmaxf(m, fmaxf(fabsf(__builtin_bit_cast(float, x << 16)),
                          fabsf(__builtin_bit_cast(float, x & 0xffff0000u))));
  };
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = min(grow0 + 16 * rt + l16, us.RU - 1);
    const uint16_t* qrow = us.q + ((int64_t)us.row0 + row) * kDqk;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lat[rt][bb][i] = *(const u32x4*)(qrow + 128 * (2 * DH + bb) + 32 * g + 8 * i);
    rope[rt] = *(const u32x4*)(qrow + 512 + 32 * DH + 8 * g);
  }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    float m = 0.0f, mr = 0.0f;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) m = amax2(m, lat[rt][bb][i][w]);
#pragma unroll
    for (int w = 0; w < 4; ++w) mr = amax2(mr, rope[rt][w]);
    hm[rt] = wave_max_across_groups(fmaxf(m, mr * 0x1p-64f));
    xmax[(wave * NRT + rt) * 64 + lane] = hm[rt];
  }
  lds_barrier();
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float M = fmaxf(hm[rt], xmax[((wave ^ 1) * NRT + rt) * 64 + lane]);
    const float inv = q8_inv_scale(M);
    c[rt] = us.scale_log2 / inv;
    auto q = [&](unsigned bits) {  // bf16 bits -> q / s, inside the e4m3 range
      return __builtin_bit_cast(float, bits) * inv;
    };
    lds_u8* mine = rec(wave, rt);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      i32x8 v8;
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // dword k: elements 4 k .. 4 k + 3 of the lane's 32
        const unsigned x0 = lat[rt][bb][k >> 1][2 * (k & 1)];
        const unsigned x1 = lat[rt][bb][k >> 1][2 * (k & 1) + 1];
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q(x0 << 16), q(x0 & 0xffff0000u), 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q(x1 << 16), q(x1 & 0xffff0000u), v, true);
        v8[k] = v;
      }
      q8.lat[rt][2 * DH + bb] = v8;
      *(i32x4*)(mine + 32 * bb) = i32x4{v8[0], v8[1], v8[2], v8[3]};
      *(i32x4*)(mine + 32 * bb + 16) = i32x4{v8[4], v8[5], v8[6], v8[7]};
    }
    bf16x8 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned x = rope[rt][w];
      r[2 * w] = (__bf16)(__builtin_bit_cast(float, x << 16) * inv);
      r[2 * w + 1] = (__bf16)(__builtin_bit_cast(float, x & 0xffff0000u) * inv);
    }
    *(bf16x8*)(mine + 64) = r;
  }
  lds_barrier();
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    lds_u8* peer = rec(wave ^ 1, rt);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const i32x4 a = *(const i32x4*)(peer + 32 * bb);
      const i32x4 b = *(const i32x4*)(peer + 32 * bb + 16);
      q8.lat[rt][2 * (1 - DH) + bb] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    // block 3 moves to the AGPR file once, here (an empty statement whose
    // output lives in AGPRs; the MFMAs read it from there)
    asm volatile("" : "=a"(q8.lat[rt][3]) : "0"(q8.lat[rt][3]));
    // both rope halves go straight from LDS to their AGPR home
    asm volatile("ds_read_b128 %0, %1 offset:64\n\ts_waitcnt lgkmcnt(0)"
                 : "=a"(q8.rope[rt][DH]) : "v"(rec(wave, rt)) : "memory");
    asm volatile("ds_read_b128 %0, %1 offset:64\n\ts_waitcnt lgkmcnt(0)"
                 : "=a"(q8.rope[rt][1 - DH]) : "v"(peer) : "memory");
  }
  lds_barrier();  // every wave's reads are done before the ring takes tiles
}

// Score phase of the key-split path: S^T of the wave's 16 keys, per row tile
// 4 fp8 MFMAs (latent blocks) then 2 bf16 MFMAs (rope halves), row tiles
// innermost so that NRT - 1 independent MFMAs separate each pair on one
// accumulator; pre(i) runs before MFMA i and slice(i) after it.
template <int NRT, typename P, typename W>
__device__ __forceinline__ void score_phase8k(lds_u8* tile, const FragBases8K& fb,
                                              const QFrag8K<NRT>& q8, f32x4 (&sacc)[NRT], P&& pre,
                                              W&& slice) {
  static_assert(NRT >= 2, "dependent MFMAs need an independent one between them");
  i32x8 kl[3];  // latent block b in kl[b % 3]: a block is read two steps ahead
  bf16x8 kr[2];
  kl[0] = read_k8k<0>(tile, fb);
  kl[1] = read_k8k<1>(tile, fb);
  static_for<6>([&](auto sc) {
    constexpr int st = decltype(sc)::value;
    if constexpr (st == 0) {
      kl[2] = read_k8k<2>(tile, fb);
    } else if constexpr (st == 1) {
      kl[0] = read_k8k<3>(tile, fb);  // block 0's MFMAs were issued in step 0
    } else if constexpr (st == 2) {
      kr[0] = read_kr8k<0>(tile, fb);
      kr[1] = read_kr8k<1>(tile, fb);
    }
    static_for<NRT>([&](auto rc) {
      constexpr int rt = decltype(rc)::value;
      constexpr int i = st * NRT + rt;
      pre(std::integral_constant<int, i>{});
      if constexpr (st < 4)
        mfma_s8<st == 0, lat_in_agpr<st>()>(sacc[rt], kl[st % 3], q8.lat[rt][st]);
      else
        mfma_s<false, true>(sacc[rt], kr[st - 4], q8.rope[rt][st - 4]);
      slice(std::integral_constant<int, i>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// Softmax of one tile in the key-split path, by slices: 0 combines the lane
// maxima of both halves and checks them against the references; 1 is the
// wave vote (rare: row maxima, references, l rescale, the O rescale left
// pending); then P of 2 keys of one row tile per slice; the last adds the row
// sums and publishes this wave's P.
template <int NRT>
constexpr int soft_slices_k() { return 2 * NRT + 3; }

template <int NRT>
struct SoftTileK {
  float mxc[NRT], nmu[NRT], psum[NRT], pend[NRT];
  bool jump, pending;
};

template <int NRT, int PH>
__device__ __forceinline__ void softmax_slice_k(SoftTileK<NRT>& w, const f32x4 (&sfull)[NRT],
                                                const float (&own_mx)[NRT], const f32x4& peer_mx,
                                                int (&pnew)[NRT], float (&m_run)[NRT],
                                                float (&l_run)[NRT], const float (&c)[NRT],
                                                i32x4* p_out) {
  constexpr float kLazy = lazy_octaves<true>();
  if constexpr (PH == 0) {
    w.jump = false;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      w.mxc[rt] = max2(own_mx[rt], peer_mx[rt]);
      w.jump = w.jump || w.mxc[rt] * c[rt] > m_run[rt] + kLazy;
    }
  } else if constexpr (PH == 1) {
    w.pending = false;
    if (__builtin_amdgcn_ballot_w64(w.jump) != 0) {  // wave-uniform
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float mx = wave_max_across_groups(w.mxc[rt]) * c[rt];
        const bool first = m_run[rt] == -INFINITY;  // O and l are still 0
        const bool jump = !first && mx > m_run[rt] + kLazy;
        const float f = jump ? __builtin_amdgcn_exp2f(m_run[rt] - mx) : 1.0f;
        l_run[rt] *= f;
        w.pend[rt] = f;
        w.pending = w.pending || __builtin_amdgcn_ballot_w64(jump) != 0;
        m_run[rt] = (first && mx > -INFINITY) || jump ? mx : m_run[rt];
        w.nmu[rt] = m_run[rt] == -INFINITY ? 0.0f : -m_run[rt];
        asm volatile("" : "+v"(m_run[rt]), "+v"(w.nmu[rt]));
      }
    }
  } else if constexpr (PH < 2 + 2 * NRT) {  // P of keys 4 g + 2 h, +1: bytes 2 h, 2 h + 1
    constexpr int j = PH - 2;
    constexpr int rt = j / 2, h = j % 2;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sfull[rt][2 * h], c[rt], w.nmu[rt]));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sfull[rt][2 * h + 1], c[rt], w.nmu[rt]));
    w.psum[rt] = h == 0 ? p0 + p1 : w.psum[rt] + (p0 + p1);
    pnew[rt] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pnew[rt], h != 0);
  } else {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) l_run[rt] += w.psum[rt];
    i32x4 rec = {0, 0, 0, 0};
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) rec[rt] = pnew[rt];
    *p_out = rec;
  }
}

// 2 wait states between the VALU writes of the PV operand P and the first
// MFMA that reads it (the asm consumes and redefines P, so it stays between).
template <int NRT>
__device__ __forceinline__ void pad_p_writes(i32x2 (&pf)[NRT]) {
  if constexpr (NRT == 2)
    asm volatile("s_nop 1" : "+v"(pf[0]), "+v"(pf[1]));
  else
    asm volatile("s_nop 1" : "+v"(pf[0]), "+v"(pf[1]), "+v"(pf[2]));
}

// The whole KV chunk of a unit in the key-split path (see above).  Same
// staging, barriers and tile-loop unrolling as unit_pipeline; the exchange
// records replace the score exchange.
template <int NRT, int DH, bool PAGED>
__device__ __forceinline__ void unit_pipeline8k(const UnitSetup& us, lds_u8* lds, float* xs,
                                                int wave, const FragBases8K& fb,
                                                const QFrag8K<NRT>& qf, const float (&c)[NRT],
                                                f32x4 (&oacc)[16][NRT], float (&m_run)[NRT],
                                                float (&l_run)[NRT], const int (&lim)[NRT], int tid,
                                                int g, int lane) {
  constexpr bool FP8 = true;
  static_assert(NRT >= 2 && NRT <= 3, "exchange records hold one dword per row tile, at most 3");
  constexpr int NS = stage_sets<FP8, NRT>();
  constexpr int kAhead = (NS - 1) * kPieces;
  constexpr int DV = v_ahead<NRT, FP8>();
  constexpr int TB = tile_bytes<FP8>();
  constexpr int RING = ring_slots<FP8, NRT>();
  static_assert(RING == 4, "tile t - 1 (V), t, t + 1 (K) and t + 2 (staged) are live together");
  const UnitCtx u = us.uc;
  const KvSource<FP8, PAGED> src = kv_source<FP8, PAGED>(us);
  auto zero_all_o = [&] {
#pragma unroll
    for (int cc = 0; cc < 16; ++cc)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) zero_o(oacc[cc][rt]);
  };
  if (u.ntiles <= 0) {
    zero_all_o();
    return;
  }
  unsigned char* xb = (unsigned char*)xs;
  auto xm_at = [&](int par, int w) { return (f32x4*)(xb + kXmOff + (par * kWaves + w) * 1024) + lane; };
  auto xp_at = [&](int par, int w) { return (i32x4*)(xb + kXpOff + (par * kWaves + w) * 1024) + lane; };
  lds_u8* spill = (lds_u8*)(xb + kSpillOff + wave * 1024 + lane * 16);

  // prologue: tiles 0 and 1 into their slots; tile k always travels in set k % NS
  int64_t pr[NS + 3];
  prologue_page_rows(src, pr);
  Stage<FP8> st[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) stage_load<FP8>(st[k], src.rsrc(k, pr[k]), tid);
  static_for<2>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    wait_stage<kAhead, FP8>(st[j % NS]);
    stage_store<FP8>(st[j % NS], lds + j * TB, tid);
    stage_load<FP8>(st[j % NS], src.rsrc(j + NS, pr[j + NS]), tid);
  });
  lds_barrier();
  int64_t prow_next = pr[NS + 2];  // page row of the first tile the loop loads

  // scores of tile t in sc[t % 2] (the loop is unrolled by NS = 2, so the
  // score MFMAs of tile t + 1 and the softmax of tile t use fixed registers)
  static_assert(NS % 2 == 0, "tile parity must be static");
  f32x4 sc[2][NRT];
  float own_mx[NRT];
  // scores of tile t1 in sc[t1 % 2]: causal mask (last tiles of a chunk), lane
  // maxima, published for the partner
  auto lane_max = [&](auto parc, int t1) {
    constexpr int par = decltype(parc)::value;
    f32x4 (&sacc)[NRT] = sc[par];
    const int k0 = t1 * kTK;
    if (k0 + kTK - 1 > u.min_lim) {
      asm volatile("" ::: "memory");  // keep this a branch: interior tiles skip it
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 16 * DH + 4 * g + i;
          sacc[rt][i] = key <= lim[rt] ? sacc[rt][i] : -INFINITY;
        }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
      own_mx[rt] = max2(max2(sacc[rt][0], sacc[rt][1]), max2(sacc[rt][2], sacc[rt][3]));
    f32x4 rec = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) rec[rt] = own_mx[rt];
    *xm_at(t1 & 1, wave) = rec;
  };

  score_phase8k<NRT>(lds, fb, qf, sc[0], [](auto) {}, [](auto) {});
  asm volatile("s_nop 15\n\ts_nop 7" ::: "memory");  // score MFMAs retire before the reads
  lane_max(std::integral_constant<int, 0>{}, 0);
  *xp_at(1, wave) = i32x4{0, 0, 0, 0};  // P of "tile -1", read by the partner at t = 0
  lds_barrier();
  // the partner's records, read at the start of each iteration's score phase
  // (after its K reads are issued, so no iteration starts with a wait on them)
  f32x4 peer_mx;
  i32x4 peer_p;

  zero_all_o();  // here rather than before the prologue: fewer values live across it
  i32x2 vr[v8_slots<DV>()];
  i32x2 pf[NRT];
  int pnew[NRT];
  SoftTileK<NRT> sw;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    pf[rt] = i32x2{0, 0};  // P of "tile -1": the first PV adds nothing
    pnew[rt] = 0;
    sw.nmu[rt] = 0.0f;  // references not set yet (m_run = -inf)
  }
  for (int base = 0; base < u.ntiles; base += NS) {
    static_for<NS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ks = (k + 2) % NS;  // staging set of tile t + 2
      const int t = base + k;
      if (t < u.ntiles) {
        // V of tile t - 1 (tile 0's slot at t = 0, where P is 0)
        lds_u8* vbase = lds + ((t == 0 ? 0 : t - 1) % RING) * TB + fb.v;
        lds_u8* slot_n = lds + ((t + 1) % RING) * TB;
        lds_u8* slot_s = lds + ((t + 2) % RING) * TB;
        const __amdgpu_buffer_rsrc_t rs_next = src.rsrc(t + 2 + NS, prow_next);
        issue_v_head8<DH, DV>(vr, vbase);

        constexpr int kStageSlices = 1 + 2 * kPieces;
        auto stage_slice = [&](auto sc) {
          constexpr int s = decltype(sc)::value;
          if constexpr (s == 0) {
            wait_stage<kAhead, FP8>(st[ks]);
          } else if constexpr (s < 1 + kPieces) {
            stage_store_piece<FP8, s - 1>(st[ks], slot_s, tid);
          } else {
            stage_load_piece<FP8, s - 1 - kPieces>(st[ks], rs_next, tid);
          }
        };

        // scores of tile t + 1 (into sc[(k + 1) % 2]) || softmax of tile t (sc[k])
        constexpr int kScoreMfma = 6 * NRT;
        i32x4* p_out = xp_at(t & 1, wave);
        auto read_peer = [&](auto ic) {
          if constexpr (decltype(ic)::value == 0) {
            peer_p = *xp_at((t + 1) & 1, wave ^ 1);  // P(t - 1)
            peer_mx = *xm_at(t & 1, wave ^ 1);       // lane maxima of tile t
          }
        };
        score_phase8k<NRT>(slot_n, fb, qf, sc[(k + 1) % 2], read_peer, [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          slices_at<soft_slices_k<NRT>(), kScoreMfma, i>([&](auto slc) {
            constexpr int s = decltype(slc)::value;
            softmax_slice_k<NRT, s>(sw, sc[k], own_mx, peer_mx, pnew, m_run, l_run, c, p_out);
          });
        });

        // the partner's half of P(t - 1) joins the PV operand (VALU writes: at
        // least 2 wait states before the first MFMA reads them)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) pf[rt][1 - DH] = peer_p[rt];
        pad_p_writes(pf);

        // O of tile t - 1  ||  lane maxima of tile t + 1, staging of tile t + 2
        constexpr int kPvMfma = 16 * NRT;
        auto pv_slice = [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i == 2) {
            asm volatile("s_nop 15" ::: "memory");  // the score MFMAs have retired
            lane_max(std::integral_constant<int, (k + 1) % 2>{}, t + 1);
          }
          slices_at<kStageSlices, kPvMfma, i>(stage_slice);
        };
        pv_phase8<NRT, DH, DV>(vbase, pf, oacc, vr, pv_slice);

        if (sw.pending) {  // rare, wave-uniform: a reference moved at tile t
          asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // O MFMAs retired
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            if (__builtin_amdgcn_ballot_w64(sw.pend[rt] != 1.0f) != 0) {
#pragma unroll
              for (int cc = 0; cc < 16; ++cc) scale_o(oacc[cc][rt], sw.pend[rt], spill);
            }
        }

        if constexpr (PAGED)
          prow_next = src.barrier_and_page_row(t + 3 + NS);
        else
          lds_barrier();
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) pf[rt][DH] = pnew[rt];
      }
    });
  }
  // PV of the last tile
  {
    lds_u8* vbase = lds + ((u.ntiles - 1) % RING) * TB + fb.v;
    issue_v_head8<DH, DV>(vr, vbase);
    peer_p = *xp_at((u.ntiles - 1) & 1, wave ^ 1);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) pf[rt][1 - DH] = peer_p[rt];
    pad_p_writes(pf);
    pv_phase8<NRT, DH, DV>(vbase, pf, oacc, vr, [](auto) {});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads issued past the end
}

// Row sums of the key-split path: each wave of a pair summed its own keys;
// both waves add the two totals (in either order: the same fp32 result).
template <int NRT>
__device__ __forceinline__ void total_row_sums(float* xs, int wave, float (&l_run)[NRT]) {
  const int lane = threadIdx.x & 63;
  unsigned char* xb = (unsigned char*)xs;
  f32x4 own = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) own[rt] = wave_sum_across_groups(l_run[rt]);
  *((f32x4*)(xb + kXlOff + wave * 1024) + lane) = own;
  lds_barrier();
  const f32x4 peer = *((const f32x4*)(xb + kXlOff + (wave ^ 1) * 1024) + lane);
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) l_run[rt] = own[rt] + peer[rt];
}

template <bool FP8, int NRT, int DH, bool PAGED, bool NT>
__device__ __forceinline__ void unit_body(const MainArgs& args, unsigned char* smem) {
  UnitSetup us;
  if (!unit_setup<Stage<FP8>::kGlobalRowBytes, kTK>(args, us)) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int grow0 = (wave >> 1) * 16 * NRT;  // first unit row of this wave's row group
  const bool wave_active = grow0 < us.RU;     // the row group holds a row of the unit
  int lim[NRT];  // last key (chunk-relative) the lane's row may see
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int row = grow0 + 16 * rt + l16;
    const int rv = row < us.RU ? row : us.RU - 1;
    lim[rt] = min(us.hi_eff - 1, us.tail0 + (us.rowb0 + rv) / us.H) - us.uc.lo;
  }
  lds_u8* lds = (lds_u8*)smem;
  float* xs = (float*)(smem + ring_slots<FP8, NRT>() * tile_bytes<FP8>());

  // per-lane softmax state: lane owns unit row grow0 + 16 rt + l16
  float m_run[NRT], l_run[NRT];
  f32x4 oacc[16][NRT];
  auto run = [&](const auto& fb, const auto& qf, const float (&c)[NRT]) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      m_run[rt] = -INFINITY;
      l_run[rt] = 0.0f;
    }
    if constexpr (!key_split<FP8, NRT>()) {  // the key-split pipeline zeroes O itself
#pragma unroll
      for (int cc = 0; cc < 16; ++cc)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) zero_o(oacc[cc][rt]);
    }
    if (!wave_active) {  // a row group with no row of the unit only stages
      unit_staging_only<FP8, NRT, PAGED, NT>(us, lds, tid);
      if constexpr (key_split<FP8, NRT>()) lds_barrier();  // the other pair's row-sum exchange
      return;
    }
    if constexpr (key_split<FP8, NRT>()) {
      unit_pipeline8k<NRT, DH, PAGED>(us, lds, xs, wave, fb, qf, c, oacc, m_run, l_run, lim, tid,
                                      g, lane);
      total_row_sums<NRT>(xs, wave, l_run);
      epilogue<NRT, DH, true>(us, grow0, l16, g, oacc, m_run, l_run);
    } else {
      unit_pipeline<FP8, NRT, DH, PAGED, NT>(us, lds, xs, wave, fb, qf, c, oacc, m_run, l_run, lim,
                                             tid, g, lane);
      epilogue<NRT, DH>(us, grow0, l16, g, oacc, m_run, l_run);
    }
  };
  if constexpr (key_split<FP8, NRT>()) {
    QFrag8K<NRT> q8;
    float c[NRT];
    load_q8k<NRT, DH>(us, grow0, l16, g, wave, lds, q8, c);
    run(frag_bases8k<DH>(l16, g), q8, c);
  } else if constexpr (FP8) {
    QFrag8<NRT> q8;
    float c[NRT];
    load_q8<NRT, DH>(us, grow0, l16, g, wave, xs, q8, c);
    run(frag_bases8<DH>(l16, g), q8, c);
  } else {
    // Rows past the unit hold zero Q (their outputs are never written).
    bf16x8 qf[NRT][9];
    load_q<NRT, DH>(us, grow0, l16, g, qf);
    float c[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) c[rt] = us.scale_log2;
    run(frag_bases(l16, g), qf, c);
  }
}

template <bool FP8, int NRT>
constexpr int main_lds_bytes() {
  // tile ring + 2 exchange buffers
  return ring_slots<FP8, NRT>() * tile_bytes<FP8>() + exchange_bytes<FP8, NRT>();
}

// One kernel per (KV dtype, row tiles per row group, KV layout, KV cache
// hint): a kernel holds a single pipeline, so that the register allocation of
// one layout never constrains the other.
template <bool FP8, int NRT, bool PAGED, bool NT>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_main(const MainArgs args) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[main_lds_bytes<FP8, NRT>()];
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1)
    unit_body<FP8, NRT, 1, PAGED, NT>(args, smem);
  else
    unit_body<FP8, NRT, 0, PAGED, NT>(args, smem);
  merge_if_last(args, smem);
  merge_grid(args, smem);
}

#ifndef MLA_PAGED_KV  // the merges are built once, with the contiguous-KV kernels

// The split sequence that holds reduce row gr (wave-uniform; first rows
// ascend and every split sequence has at least one row) and the row's index
// inside it, found by binary search over a large plan's tables in the
// workspace (TABLE) or over the kernel arguments.  Each kernel reads one of
// the two sources only: a kernel that could read a descriptor from either
// would have its arguments copied to scratch memory.
struct RedRow {
  SeqDesc sd;
  int local;
};
template <bool TABLE>
__device__ __forceinline__ RedRow red_row(const ReduceArgs& args, int gr) {
  RedRow rr;
  if constexpr (TABLE) {
    const int b = last_at_or_below(args.num_seqs, gr, [&](int i) {
      return __builtin_amdgcn_readfirstlane(args.row0_table[i]);
    });
    rr.sd = uniform_desc(args.seq_table, b);
    rr.local = gr - __builtin_amdgcn_readfirstlane(args.row0_table[b]);
  } else {
    const int b = last_at_or_below(args.num_seqs, gr, [&](int i) { return args.row0[i]; });
    rr.sd = args.seqs[b];
    rr.local = gr - args.row0[b];
  }
  return rr;
}

// Split-KV merge: one 256-thread block per (split output row, block of
// fold_cols<P>() value columns), folded by fold_split_row<P> (the fold the
// grid merge of the main kernels also runs, with the same layout rule, so
// that the two give the same bits).  P = fold_parts(largest S of the launch).
template <int P, bool TABLE>
__global__ __launch_bounds__(kFoldThreads) void mla_decode_reduce_kernel(const ReduceArgs args) {
  __shared__ FoldLds lds;
  constexpr int kBlocksPerRow = kDv / fold_cols<P>();
  const int gr = blockIdx.x / kBlocksPerRow;
  const int cb = blockIdx.x % kBlocksPerRow;
  if (gr >= args.num_rows) return;
  const RedRow rr = red_row<TABLE>(args, gr);
  const SeqDesc& sd = rr.sd;
  const int local = rr.local;
  const int R = sd.R;
  const int t = local / R;
  const int r = local % R;
  const int64_t pbase = (int64_t)sd.part_row0 + (int64_t)t * sd.S * R + r;
  const int64_t orow = (int64_t)sd.q_row0 + (int64_t)t * R + r;
  fold_split_row<P>(args.part_lse, args.part_o, pbase, sd.S, R, cb, args.o + orow * kDv,
                    cb == 0 ? args.lse + orow : nullptr, lds);
}

// Split-KV merge of launches whose sequences have at most 8 chunks (P = 1):
// kFoldRowsP1 split rows per block, 64 threads per row, each thread folding
// all chunks of 8 columns (fold_cols8).
template <bool TABLE>
__global__ __launch_bounds__(kFoldThreads) void mla_decode_reduce_rows_kernel(const ReduceArgs args) {
  // one row per wave: the row index is wave-uniform
  static_assert(kDv / 8 == 64, "a row's 8-column groups fill one wave");
  const int gr = blockIdx.x * kFoldRowsP1 + __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int c8 = (int)threadIdx.x % 64;
  if (gr >= args.num_rows) return;
  const RedRow rr = red_row<TABLE>(args, gr);
  const SeqDesc& sd = rr.sd;
  const int local = rr.local;
  const int R = sd.R;
  const int t = local / R;
  const int r = local % R;
  const int64_t pbase = (int64_t)sd.part_row0 + (int64_t)t * sd.S * R + r;
  const int64_t orow = (int64_t)sd.q_row0 + (int64_t)t * R + r;
  fold_cols8(args.part_lse, args.part_o, pbase, sd.S, R, c8, args.o + orow * kDv,
             c8 == 0 ? args.lse + orow : nullptr);
}

// Merge layout of the shard merge below: one 256-thread block per (output
// row, 64 of the 512 value columns); thread (part p, column group cg) owns
// columns 4 cg .. 4 cg + 3 of the block and folds inputs s = 16 i + p in
// ascending order; the 16 partial sums are then added in a fixed order
// through LDS, so replays are bitwise identical.
constexpr int kRedThreads = 256;
constexpr int kRedCols = 64;                         // value columns per block
constexpr int kRedGroups = kRedCols / 4;             // 4-column groups
constexpr int kRedParts = kRedThreads / kRedGroups;  // partial sums per block

__device__ __forceinline__ float wave_max64(float v) {
  v = wave_max_across_groups(v);          // lanes l, l^16, l^32, l^48
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

// Sums of the per-part folds in part order; writes 4 bf16 columns and the LSE.
__device__ __forceinline__ void merge_finish(f32x4 (&red_acc)[kRedParts][kRedGroups],
                                             float (&red_w)[kRedParts], int cg, float M,
                                             uint16_t* o_row, float* lse_row, bool lse_writer) {
  f32x4 tot = red_acc[0][cg];
  float Wt = red_w[0];
#pragma unroll
  for (int k = 1; k < kRedParts; ++k) {
    tot += red_acc[k][cg];
    Wt += red_w[k];
  }
  const bool empty = !(Wt > 0.0f);  // no chunk or shard shows this row a key
  const float inv = empty ? 0.0f : 1.0f / Wt;
  uint2 pk;
  pk.x = pack_bf16x2(tot[0] * inv, tot[1] * inv);
  pk.y = pack_bf16x2(tot[2] * inv, tot[3] * inv);
  *(uint2*)(o_row + 4 * cg) = pk;
  if (lse_writer) *lse_row = empty ? -INFINITY : M + __logf(Wt);
}

__global__ __launch_bounds__(kRedThreads) void mla_merge_shards_kernel(const MergeArgs args) {
  __shared__ f32x4 red_acc[kRedParts][kRedGroups];
  __shared__ float red_w[kRedParts];
  constexpr int kBlocksPerRow = kDv / kRedCols;
  const int row = blockIdx.x / kBlocksPerRow;
  const int cb = blockIdx.x % kBlocksPerRow;
  if (row >= args.num_rows) return;
  const int W = args.num_shards;
  const int64_t rows = args.num_rows;
  const int lane = threadIdx.x & 63;
  const int part = threadIdx.x / kRedGroups;
  const int cg = threadIdx.x % kRedGroups;

  float M = -INFINITY;
  for (int s = lane; s < W; s += 64) M = fmaxf(M, args.lse_shards[s * rows + row]);
  M = wave_max64(M);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Wsum = 0.0f;
  const uint16_t* po = args.o_shards + kRedCols * cb + 4 * cg;
  for (int s = part; s < W; s += kRedParts) {
    const float ls = args.lse_shards[s * rows + row];
    if (ls == -INFINITY) continue;  // a shard that shows the row no key: its O is not read
    const f32x4 v = bf16x4_to_f32(*(const uint2*)(po + (s * rows + row) * kDv));
    const float w = __expf(ls - M);
    Wsum += w;
    acc += w * v;
  }
  red_acc[part][cg] = acc;
  if (cg == 0) red_w[part] = Wsum;
  __syncthreads();
  if (threadIdx.x >= kRedGroups) return;
  merge_finish(red_acc, red_w, cg, M, args.o + (int64_t)row * kDv + kRedCols * cb, args.lse + row,
               cb == 0 && cg == 0);
}

#endif  // !MLA_PAGED_KV

// ------------------------------------------------------------- launchers

template <bool FP8, bool PAGED, bool NT>
static void launch_main_t(const MainArgs& a, int nrt, int grid, hipStream_t stream) {
  if (nrt <= 1)
    hipLaunchKernelGGL((mla_decode_main<FP8, 1, PAGED, NT>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (nrt == 2)
    hipLaunchKernelGGL((mla_decode_main<FP8, 2, PAGED, NT>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((mla_decode_main<FP8, 3, PAGED, NT>), dim3(grid), dim3(kThreads), 0, stream, a);
}

// This file is compiled twice: once for contiguous KV (with the merges) and
// once, with MLA_PAGED_KV defined (kernels_paged.hip), for paged KV, so that
// the two sets of main kernels build in parallel.
// bf16 KV only: fp8 KV runs the kernel of fp8_decode.hip (this file's fp8
// template branches are the earlier fp8 kernels, no longer instantiated).
#ifdef MLA_PAGED_KV
hipError_t launch_main_paged(const MainArgs& a, int nrt, bool nt, hipStream_t stream) {
  constexpr bool kPaged = true;
#else
hipError_t launch_main_contiguous(const MainArgs& a, int nrt, bool nt, hipStream_t stream) {
  constexpr bool kPaged = false;
#endif
  const int grid = ((a.num_units + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid == 0) return hipSuccess;
  if (nrt < 1 || nrt > 3) return hipErrorInvalidValue;
  if (nt)
    launch_main_t<false, kPaged, true>(a, nrt, grid, stream);
  else
    launch_main_t<false, kPaged, false>(a, nrt, grid, stream);
  return hipGetLastError();
}

#ifndef MLA_PAGED_KV
template <bool TABLE>
static void launch_reduce_t(const ReduceArgs& a, hipStream_t stream) {
  switch (fold_parts(a.max_splits)) {
    case 1:
      hipLaunchKernelGGL(mla_decode_reduce_rows_kernel<TABLE>,
                         dim3((a.num_rows + kFoldRowsP1 - 1) / kFoldRowsP1), dim3(kFoldThreads), 0,
                         stream, a);
      break;
    case 4:
      hipLaunchKernelGGL((mla_decode_reduce_kernel<4, TABLE>), dim3((kDv / fold_cols<4>()) * a.num_rows),
                         dim3(kFoldThreads), 0, stream, a);
      break;
    case 8:
      hipLaunchKernelGGL((mla_decode_reduce_kernel<8, TABLE>), dim3((kDv / fold_cols<8>()) * a.num_rows),
                         dim3(kFoldThreads), 0, stream, a);
      break;
    case 16:
      hipLaunchKernelGGL((mla_decode_reduce_kernel<16, TABLE>),
                         dim3((kDv / fold_cols<16>()) * a.num_rows), dim3(kFoldThreads), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((mla_decode_reduce_kernel<32, TABLE>),
                         dim3((kDv / fold_cols<32>()) * a.num_rows), dim3(kFoldThreads), 0, stream, a);
      break;
  }
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  if (a.seq_table)
    launch_reduce_t<true>(a, stream);
  else
    launch_reduce_t<false>(a, stream);
  return hipGetLastError();
}

// Workspace for callers that cannot allocate (mla_decode_run_static): one
// array per device, held for the life of the process.  Host code never uses
// the array's name as an address (on the host it is only a stand-in for the
// symbol): its device address comes from hipGetSymbolAddress, looked up once
// per device with that device current and kept here.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevicesStatic];
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevicesStatic) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int grid = (kDv / kRedCols) * a.num_rows;
  hipLaunchKernelGGL(mla_merge_shards_kernel, dim3(grid), dim3(kRedThreads), 0, stream, a);
  return hipGetLastError();
}

#endif  // !MLA_PAGED_KV

}  // namespace mla
