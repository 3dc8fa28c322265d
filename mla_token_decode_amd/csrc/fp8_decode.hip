// MLA speculative-verify decode over an fp8 (OCP E4M3FN) KV cache, gfx950.
//
// One workgroup (4 waves) per work unit: up to 96 folded rows (F verify tokens
// x H heads, one contiguous slab of Q) against one split-KV chunk of their
// sequence, which is streamed from HBM once and shared by all rows -- the
// fold_sq decode of "[Kimi-K3] Allow DSPARK verify on cutedsl_mla (fold_sq)"
// (sglang PR #33650), section "Decision rule", paragraph "Why"; split chunks
// leave normalised partials for the merge kernel (same PR, section "GPU
// timeline").
//
// KV stream.  64-key tiles go from HBM straight into a 4-slot LDS ring with
// buffer_load_dwordx4 ... lds (no staging registers): the latent part as
// 64 rows of 512 e4m3 bytes, the rope part as 64 rows of 64 e4m3 bytes, both
// with their 16-byte chunks XOR-swizzled by the key so that the fragment reads
// below are free of bank conflicts.  Two tiles are in flight while one is
// computed.  The per-tensor fp8 scale is folded into the softmax constant and
// the epilogue.
//
// Work of one tile.  Wave w has two roles:
//   scores  (key half kh = w & 1, row half rh = w >> 1): S^T for keys
//           32 kh .. 32 kh + 31 of the tile and 16 N rows of the unit, over
//           all 576 columns: v_mfma_f32_16x16x128_f8f6f4 with K (A operand)
//           from LDS and Q (B operand) quantised per row to e4m3 in
//           registers -- 4 latent blocks of 128 columns and the 64 rope
//           columns zero-padded to 128; then the softmax of those scores into
//           e4m3 P, written to a P buffer in LDS;
//   values  (column quarter w): O^T[128 w .. 128 w + 127][all rows] +=
//           V^T P^T with v_mfma_f32_32x32x64_f8f6f4: V^T from LDS through
//           the transposing 8-bit reads, P^T from the P buffer.
// The PV of tile t runs in the iteration after its scores, once the barrier
// has published every wave's P.
//
// Softmax.  Base-2 logits with a lazy per-row reference m: P = 2^(c s - m),
// c = sm_scale * kv_scale * log2(e) * s_q (the row's Q scale).  The reference
// only moves when a row's scores pass it by more than 8 octaves (so P <= 2^8
// stays inside e4m3, whose largest value is 448), as in the pages' own fp8
// kernel ("bench(cake_mla_varq_dcp_decode): ..." (flashinfer PR #5588),
// embedded follow-up, section "Summary": a lazy E4M3 reference and a deferred
// O rescale).  Each wave checks its own scores against the reference and
// publishes one flag with its P; when any flag of a tile is set, every wave
// takes the rare path after the barrier: the two waves of each row exchange
// row maxima, move the references, recompute that tile's P, and all waves
// rescale the O rows and row sums formed against the old reference.  The
// first tile of a unit takes that path to set the references.
#include "device_common.hpp"
#include "fp8_agpr.hpp"

namespace mla {
namespace fp8k {

constexpr int kThreads = 256;
constexpr int kKeys = 64;                    // keys per tile
constexpr int kLatB = 512;                   // latent bytes of a key
constexpr int kRopeB = 64;                   // rope bytes of a key
constexpr int kRowB = kLatB + kRopeB;        // 576: one KV row in memory
constexpr int kTileB = kKeys * kRowB;        // 36864: one LDS slot
constexpr int kRopeOff = kKeys * kLatB;      // 32768: rope rows inside a slot
constexpr int kSlots = 4;
constexpr int kPOff = kSlots * kTileB;       // 147456: two P buffers
constexpr int kPBuf = kMaxUnitRows * kKeys;  // 6144: rows x 64 e4m3
constexpr int kMisc = kPOff + 2 * kPBuf;     // 159744
constexpr int kFlagOff = kMisc;              // [2 parities][4 waves] u32
constexpr int kRowMaxOff = kMisc + 64;       // [2 key halves][96 rows] f32
constexpr int kFactorOff = kRowMaxOff + 768; // [96 rows] f32
constexpr int kLsumOff = kFactorOff + 384;   // [2 key halves][96 rows] f32
constexpr int kMrefOff = kLsumOff + 768;     // [96 rows] f32
constexpr int kLdsBytes = kMisc + 4096;      // 163840: all of a CU's LDS
static_assert(kMrefOff + 384 <= kLdsBytes, "misc area");
static_assert(kMaxUnitRows == 96, "P buffer and misc arrays hold 96 rows");
constexpr float kLazy = 8.0f;  // octaves a score may pass the reference by

// --------------------------------------------------------------- KV stream

// Where a unit's tiles live: a contiguous run of rows, or the pages of a pool
// (pages of 2^shift >= 32 keys; a tile's two 32-key halves each lie in one
// page).  Chunk-relative key k is sequence key lo + k.
template <bool PAGED>
struct Src {
  const uint8_t* base;    // contiguous: row `lo` of the sequence; paged: the pool
  const int32_t* pt_row;  // paged: the sequence's page-table row
  int lo, nkeys, shift, last_idx;
  unsigned max_page;

  __device__ __forceinline__ int entry_idx(int t, int h) const {
    return min((lo + kKeys * t + 32 * h) >> shift, last_idx);
  }
  // First row (of the pool, or of the chunk) of half h of tile t, given the
  // page-table entry of that half (paged only).
  __device__ __forceinline__ const uint8_t* half_base(int t, int h, int entry) const {
    if constexpr (!PAGED) {
      return base + (int64_t)(kKeys * t + 32 * h) * kRowB;
    } else {
      const int64_t prow = ((int64_t)min((unsigned)entry, max_page) << shift) +
                           ((lo + kKeys * t + 32 * h) & ((1 << shift) - 1));
      return base + prow * kRowB;
    }
  }
  // Keys of half h of tile t that exist (0..32): the rest read as zero.
  __device__ __forceinline__ int half_rows(int t, int h) const {
    return max(0, min(32, nkeys - kKeys * t - 32 * h));
  }
};

// Page-table entries of the two halves of tile t, fetched by scalar loads
// waited for together with the LDS traffic in front of the tile barrier (no
// scalar load is ever outstanding while the loop's LDS waits run).
template <bool PAGED>
__device__ __forceinline__ void barrier_fetch(const Src<PAGED>& src, int t, int (&e)[2]) {
  if constexpr (PAGED) {
    asm volatile("s_load_dword %0, %2, %3\n\ts_load_dword %1, %2, %4\n\ts_waitcnt lgkmcnt(0)\n\t"
                 "s_barrier"
                 : "=&s"(e[0]), "=&s"(e[1])
                 : "s"(src.pt_row), "s"(4 * src.entry_idx(t, 0)), "s"(4 * src.entry_idx(t, 1))
                 : "memory");
  } else {
    e[0] = e[1] = 0;
    lds_barrier();
  }
}
template <bool PAGED>
__device__ __forceinline__ void fetch_now(const Src<PAGED>& src, int t, int (&e)[2]) {
  if constexpr (PAGED) {
    asm volatile("s_load_dword %0, %2, %3\n\ts_load_dword %1, %2, %4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(e[0]), "=&s"(e[1])
                 : "s"(src.pt_row), "s"(4 * src.entry_idx(t, 0)), "s"(4 * src.entry_idx(t, 1))
                 : "memory");
  } else {
    e[0] = e[1] = 0;
  }
}

// One 16-byte-per-lane load of global memory straight into LDS: the wave's 64
// lanes fill the 1 KB at `dst` (lane i at dst + 16 i) from their own offsets
// into the descriptor's range (bytes past the range read as zero).  Counted
// by vmcnt; the compiler does not see it, so every wait for it is explicit.
// NT: the non-temporal hint, for the KV tiles of launches in which no KV
// chunk is read by two units (each byte is then read once; a cold streaming
// read measured 8-15 % faster with it; where several units read one chunk the
// hint would make each re-read HBM); Q rows, which every CU reads, keep the
// default policy.
template <bool NT = false>
__device__ __forceinline__ void dma16(const lds_u8* dst, int voff, __amdgpu_buffer_rsrc_t r) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(m0v), "v"(voff), "s"(r) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0v), "v"(voff), "s"(r) : "memory");
}

// Per-lane global offsets of the 9 loads of a tile (8 latent, 1 rope).  Load
// k < 8 fills LDS chunks 256 k + tid of the latent rows: key 8 k + tid / 32,
// physical chunk tid % 32 = logical chunk ^ (key & 7) (the XOR is an
// involution; key & 7 = tid / 32).  Load 8 fills rope chunk tid: key tid / 4,
// physical chunk tid % 4 = logical ^ ((key >> 1) & 3).
// lat[sub]: offset of load k (sub = k % 4) from the base of its 32-key half.
struct DmaLanes {
  int lat[4], rope;
};
__device__ __forceinline__ DmaLanes dma_lanes(int tid) {
  DmaLanes d;
  const int lat = (tid >> 5) * kRowB + 16 * ((tid & 31) ^ (tid >> 5));
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) d.lat[sub] = lat + 8 * sub * kRowB;
  d.rope = ((tid >> 2) & 31) * kRowB + kLatB + 16 * ((tid & 3) ^ ((tid >> 3) & 3));
  return d;
}

// The 9 loads of tile t into `slot` (tiles past the chunk load nothing but
// still count): issue<j>() issues the j-th of them (order below), so that the
// loop can spread them between its MFMAs.  One descriptor per 32-key half, its range the half's
// rows in the chunk (the range check on the lane offsets zero-fills the
// rest).  e: page-table entries of the tile's halves (paged).
template <bool PAGED, bool NT>
struct TileLoads {
  __amdgpu_buffer_rsrc_t r[2];
  lds_u8* slot;
  __device__ __forceinline__ TileLoads(const Src<PAGED>& src, int t, const int (&e)[2],
                                       lds_u8* slot_)
      : slot(slot_) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rows = __builtin_amdgcn_readfirstlane(src.half_rows(t, h));
      r[h] = make_rsrc(uniform_ptr(src.half_base(t, h, e[h])), (uint32_t)(rows * kRowB));
    }
  }
  // Issue J (0..8) is load K = (J + 8) % 9: the rope load first, with the
  // default cache policy.  A 576-byte KV row is not a whole number of
  // 128-byte lines, so the line holding a row's rope also holds the start of
  // the next row's latent part: fetched and kept by the rope load, the line
  // then serves that latent load too, which a non-temporal latent load first
  // would not leave behind (measured 4 % more HBM reads and a slower stream).
  template <int J>
  __device__ __forceinline__ void issue(const DmaLanes& dl, int wave) const {
    constexpr int K = (J + 8) % 9;
    if constexpr (K < 8) {  // keys 8 (K % 4) .. + 7 of half K / 4
      dma16<NT>(slot + 4096 * K + 1024 * wave, dl.lat[K & 3], r[K >> 2]);
    } else {  // rope keys of this wave: 16 wave .. 16 wave + 15
      dma16<false>(slot + kRopeOff + 1024 * wave, dl.rope, wave >= 2 ? r[1] : r[0]);
    }
  }
};
template <bool PAGED, bool NT>
__device__ __forceinline__ void issue_tile(const Src<PAGED>& src, int t, const int (&e)[2],
                                           lds_u8* slot, const DmaLanes& dl, int wave) {
  const TileLoads<PAGED, NT> tl(src, t, e, slot);
  static_for<9>([&](auto kc) { tl.template issue<decltype(kc)::value>(dl, wave); });
}

template <int N>
__device__ __forceinline__ void wait_tiles_behind() {
  static_assert(N == 9 || N == 18, "9 loads per tile");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ------------------------------------------------------------------ MFMAs
//
// Inline assembly with explicit register files (the compiler pads no hazards
// around it: the callers keep >= 2 wait states between a VALU write and an
// MFMA read of the same VGPRs, and >= 19 between an MFMA result and its first
// VALU or LDS read).

// S^T (16 keys x 16 rows) += K (A, 16 x 128 e4m3) . Q^T (B, 128 x 16 e4m3).
template <bool ZERO, bool QA>
__device__ __forceinline__ void mfma_qk(f32x4& acc, const i32x8& k, const i32x8& q) {
  if constexpr (ZERO && QA)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "a"(q));
  else if constexpr (ZERO)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "v"(q));
  else if constexpr (QA)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "a"(q));
  else
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "v"(q));
}
// O^T (32 value columns x 32 rows) += V^T (A, 32 x 64) . P^T (B, 64 x 32):
// OAcc<b>::pv, with O block b = cb N + pbk in fixed AGPRs (fp8_agpr.hpp).

// ------------------------------------------------------------ fragments

// K fragment (A operand) of key block kb (16 keys), column block db (0..3
// latent, 4 rope): lane 16 g + m holds key 32 kh + 16 kb + m, columns
// 128 db + 32 g .. + 31 (rope: rope columns 32 (g & 1) .. + 31; lanes g >= 2
// meet zero Q columns).  Two 16-byte reads from per-lane bases that carry the
// swizzle; kb and db are immediate offsets.
struct KBase {
  int lat[2], rope[2];
};
__device__ __forceinline__ KBase k_base(int kh, int l16, int g) {
  KBase b;
  const int key = 32 * kh + l16;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    b.lat[x] = key * kLatB + 16 * ((2 * g + x) ^ (l16 & 7));
    b.rope[x] = kRopeOff + key * kRopeB + 16 * ((2 * (g & 1) + x) ^ ((l16 >> 1) & 3));
  }
  return b;
}
template <int KB, int DB>
__device__ __forceinline__ i32x8 read_k(const lds_u8* slot, const KBase& b) {
  i32x4 a, c;
  if constexpr (DB < 4) {
    a = *(const i32x4*)(slot + b.lat[0] + 8192 * KB + 128 * DB);
    c = *(const i32x4*)(slot + b.lat[1] + 8192 * KB + 128 * DB);
  } else {
    a = *(const i32x4*)(slot + b.rope[0] + 1024 * KB);
    c = *(const i32x4*)(slot + b.rope[1] + 1024 * KB);
  }
  return i32x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
}

// V^T fragment (A operand of the PV MFMA) of value columns 128 cq + 32 cb ..
// + 31: lane l holds column l % 32, keys 32 (l / 32) .. + 31, from four
// transposing reads of 8 keys each.  In a 16-lane group q of one read, lane
// 2 j + h points at key 32 (q >> 1) + 8 i + j, columns 16 (q & 1) + 8 h .. + 7
// of the block, and lane n receives column n of the 8 keys (in key order).
struct VBase {
  int cb[4];
};
__device__ __forceinline__ VBase v_base(int cq, int lane) {
  VBase b;
  const int q = lane >> 4, idx = lane & 15, j = idx >> 1, h = idx & 1;
  const int key = 32 * (q >> 1) + j;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    b.cb[cb] = key * kLatB + 16 * (8 * cq + ((2 * cb + (q & 1)) ^ j)) + 8 * h;
  return b;
}
template <int CB>
__device__ __forceinline__ i32x8 read_v(const lds_u8* slot, const VBase& b) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const lds_u8* p = slot + b.cb[CB];
  const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 4096));
  const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 8192));
  const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 12288));
  return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// P buffer: row r holds the tile's 64 e4m3 P values of unit row r in key
// order, its four 16-byte chunks XOR-swizzled by (r >> 1) & 3.  PV fragment
// (B operand) of row block pb: lane l holds row 32 pb + l % 32, keys
// 32 (l / 32) .. + 31.
struct PBase {
  int rd[2];   // PV reads: chunk 2 G + x of row l % 32
  int wr[2];   // score-side writes, key block kb: chunk 2 kh + kb of row l16, byte 4 g
};
__device__ __forceinline__ PBase p_base(int kh, int rh, int N, int lane) {
  PBase b;
  const int l32 = lane & 31, G = lane >> 5, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int x = 0; x < 2; ++x) b.rd[x] = l32 * 64 + 16 * ((2 * G + x) ^ ((l32 >> 1) & 3));
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    b.wr[kb] = (16 * N * rh + l16) * 64 + 16 * ((2 * kh + kb) ^ ((l16 >> 1) & 3)) + 4 * g;
  return b;
}
template <int PB>
__device__ __forceinline__ i32x8 read_p(const lds_u8* pbuf, const PBase& b) {
  const i32x4 a = *(const i32x4*)(pbuf + b.rd[0] + 2048 * PB);
  const i32x4 c = *(const i32x4*)(pbuf + b.rd[1] + 2048 * PB);
  return i32x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
}

// ------------------------------------------------------------------ Q

// e4m3 Q of this wave's 16 N rows: [rb][db], db 0..3 latent, 4 rope (zero in
// lanes g >= 2).  With N = 3, row block 2 and the rope blocks of row blocks 0
// and 1 live in the AGPR groups after O (QAcc 0..6), the rest in VGPRs.
template <int N>
constexpr int q_group(int rb, int db) {
  return N != 3 ? -1 : rb == 2 ? db : db == 4 ? 5 + rb : -1;
}
template <int N>
struct QFrag {
  i32x8 q[N][5];
};

// Raw bf16 Q of one row block: lane (l16, g) holds row `row` (clamped to the
// unit), columns 128 db + 32 g .. + 31 and rope columns 32 g .. + 31 (g < 2;
// zero otherwise).  Inline-assembly buffer loads, waited for explicitly with
// wait_q (the tile loads issued after them may stay in flight meanwhile).
struct QRaw {
  u32x4 v[5][4];
};
__device__ __forceinline__ void load_q_raw(QRaw& r, __amdgpu_buffer_rsrc_t qr, int row, int g) {
#pragma unroll
  for (int db = 0; db < 5; ++db) {
    const int col = db < 4 ? 128 * db + 32 * g : 512 + 32 * (g & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen"
                   : "=&v"(r.v[db][i]) : "v"(row * (2 * kDqk) + 2 * (col + 8 * i)), "s"(qr) : "memory");
  }
}
// Wait until at most N vector-memory loads issued after r's are outstanding;
// r's registers are tied to the wait so that no use (or copy) moves above it.
template <int N>
__device__ __forceinline__ void wait_q(QRaw& r) {
#pragma unroll
  for (int db = 0; db < 5; ++db)
    asm volatile("s_waitcnt vmcnt(%4)"
                 : "+v"(r.v[db][0]), "+v"(r.v[db][1]), "+v"(r.v[db][2]), "+v"(r.v[db][3])
                 : "n"(N) : "memory");
}

// Raw bf16 Q of row blocks 1 .. N - 1 of both row halves (32 (N - 1) rows)
// is copied into LDS slots 2 (and 3) by LDS DMA when a unit starts, so that
// the tile loads issued after it need not land before those rows are
// quantised.  LDS row lr holds unit row 16 N h + 16 + j (h = lr / (16 (N - 1)),
// j = lr % (16 (N - 1))) as 72 16-byte chunks, chunk c at position
// c ^ (lr & 7): the 8 lanes of one 16-byte read (8 rows, one chunk) then
// meet 8 different bank groups.  Rows past the unit read as zero.
constexpr int kQOff = 2 * kTileB;
constexpr int kQChunks = 2 * kDqk / 16;  // 72 chunks of one bf16 row
template <int N>
constexpr int q_dma_loads() { return 9 * (N - 1); }  // per wave: 36 (N - 1) KB in all
static_assert(kQOff + 4 * q_dma_loads<3>() * 1024 <= kPOff, "Q rows fit slots 2 and 3");
template <int N>
__device__ __forceinline__ void q_to_lds(__amdgpu_buffer_rsrc_t qr, lds_u8* lds, int wave,
                                         int lane) {
  constexpr int kRowsHalf = 16 * (N - 1);
#pragma unroll
  for (int j = 0; j < q_dma_loads<N>(); ++j) {
    const int J = 4 * j + wave;      // 1 KB block of the LDS rows
    const int C = 64 * J + lane;     // the lane's chunk position
    const int lr = C / kQChunks, cl = C - lr * kQChunks;
    const int h = lr >= kRowsHalf ? 1 : 0;
    const int urow = 16 * N * h + 16 + (lr - h * kRowsHalf);
    dma16(lds + kQOff + 1024 * J, urow * (2 * kDqk) + 16 * (cl ^ (lr & 7)), qr);
  }
}
// Row block RB (>= 1) of row half rh from the LDS rows into the QRaw layout.
template <int N, int RB>
__device__ __forceinline__ void q_from_lds(QRaw& r, const lds_u8* lds, int rh, int l16, int g) {
  const int lr = 16 * (N - 1) * rh + 16 * (RB - 1) + l16;
  const lds_u8* row = lds + kQOff + lr * (2 * kDqk);
  const int x = lr & 7;
#pragma unroll
  for (int db = 0; db < 5; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = db < 4 ? 16 * db + 4 * g + i : 64 + 4 * (g & 1) + i;
      r.v[db][i] = *(const u32x4*)(row + 16 * (c ^ x));
    }
}

// Quantise one row block to e4m3: one scale per row over all 576 columns
// (the rope and latent parts feed one accumulator), a power of two s = 2^k,
// the smallest with max |q| / s <= 448 (so max |q| / s lies in (224, 448]
// exactly), at least 2^-108 (a zero row, or one below 2^-100 in size, then
// stays far inside e4m3 and gives a near-uniform softmax); c = scale_log2 * s.
// With a power-of-two scale, gfx950's packed bf16 -> e4m3 conversion (which
// divides by the power of two of its scale operand, round to nearest even)
// quantises two columns per instruction.
typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float q8_pow2_scale(float M) {
  const float r = M * (1.0f / kQ8Top);
  float sc = __builtin_bit_cast(float, (__builtin_bit_cast(unsigned, r) + 0x007fffffu) & 0x7f800000u);
  sc = M > kQ8Top * sc ? 2.0f * sc : sc;  // r rounded below M / 448 onto a power of two
  return fmaxf(sc, 0x1p-108f);
}
template <int N, int RB>
__device__ __forceinline__ void quantise_q(const UnitSetup& us, QRaw& raw, int g, QFrag<N>& qf,
                                           float& c) {
  if (g >= 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw.v[4][i] = u32x4{0u, 0u, 0u, 0u};
  }
  // max |q| on the packed bf16 bits: with the sign bits cleared, the order of
  // the 16-bit patterns is the order of the magnitudes (no unpacked copies)
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mb = {0, 0};
#pragma unroll
  for (int db = 0; db < 5; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, raw.v[db][i][w] & 0x7fff7fffu));
  const unsigned top = (unsigned)(mb[0] > mb[1] ? mb[0] : mb[1]) << 16;
  const float M = wave_max_across_groups(__builtin_bit_cast(float, top));
  const float sc = q8_pow2_scale(M);
  c = us.scale_log2 * sc;
  static_for<5>([&](auto dc) {
    constexpr int db = decltype(dc)::value;
    i32x8 v8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // dword k: columns 4 k .. 4 k + 3 of the lane's 32
      const unsigned x0 = raw.v[db][k >> 1][2 * (k & 1)], x1 = raw.v[db][k >> 1][2 * (k & 1) + 1];
      v2i16 v = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2i16{0, 0}, __builtin_bit_cast(v2bf16, x0),
                                                          sc, false);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v, __builtin_bit_cast(v2bf16, x1), sc, true);
      v8[k] = __builtin_bit_cast(int, v);
    }
    if constexpr (q_group<N>(RB, db) >= 0)
      QAcc<q_group<N>(RB, db)>::set(v8);
    else
      qf.q[RB][db] = v8;
  });
}

// ------------------------------------------------------------------ softmax

// Per-lane softmax state of the lane's rows (one per row block rb).
template <int N>
struct Soft {
  float m[N];     // reference (base-2 logit units); -inf until the row sees a key
  float nmu[N];   // -m, or 0 while m = -inf
  float l[N];     // row sum (this lane's keys), tiles up to the last confirmed one
  float ps[N];    // row sum of the tile whose P was formed last (not yet confirmed)
  float c[N];     // logit scale of the row
  int lim[N];     // last chunk-relative key the row may see
};

// P of score block (kb, rb) of a tile, in two halves (keys 4 g + 0, 1, then
// 4 g + 2, 3 of the lane's row): on the chunk's last tiles (EDGE) the first
// masks the block in place (keys past the row's causal limit get -inf), then
// P = 2^(c s - m) (v_exp_f32 flushes results below the fp32 normal range to
// 0), packed to e4m3 (keys 4 g .. 4 g + 3 -> bytes 0..3 of one dword) and
// stored into the P buffer by the second half, which also adds the block's
// row sum to ps.  The reference must move when a P value passes 2^8 (a score
// more than kLazy octaves above it); as P >= 0, every P of a row is at most
// the lane's row sum ps, so the loop tests ps > 2^8 instead of every P (a
// rare false alarm only sends the tile down the rare path, which finds no
// reference to move and forms the same P again).
struct HalfTmp {
  int pk;
  float sum;
};
template <int N, int KB, int RB, int HALF, bool EDGE>
__device__ __forceinline__ void softmax_half(f32x4 (&S)[2][N], Soft<N>& sm, int k0,
                                             lds_u8* pbuf, const PBase& pb, HalfTmp& ht) {
  f32x4& s = S[KB][RB];
  if constexpr (HALF == 0) {
    if constexpr (EDGE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = k0 + 16 * KB + i <= sm.lim[RB] ? s[i] : -INFINITY;
    }
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0], sm.c[RB], sm.nmu[RB]));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1], sm.c[RB], sm.nmu[RB]));
    ht.sum = p0 + p1;
    ht.pk = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __builtin_bit_cast(int, p1), false);
  } else {
    const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2], sm.c[RB], sm.nmu[RB]));
    const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[3], sm.c[RB], sm.nmu[RB]));
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, ht.pk, true);
    sm.ps[RB] += ht.sum + (p2 + p3);
    *(int*)(pbuf + pb.wr[KB] + 1024 * RB) = pk;
  }
}

// The whole softmax of a tile (rare path).
template <int N, bool EDGE>
__device__ __forceinline__ void softmax_tile_as(f32x4 (&S)[2][N], Soft<N>& sm, int k0,
                                                lds_u8* pbuf, const PBase& pb) {
#pragma unroll
  for (int rb = 0; rb < N; ++rb) sm.ps[rb] = 0.0f;
  static_for<2 * N>([&](auto bc) {
    constexpr int kb = decltype(bc)::value % 2, rb = decltype(bc)::value / 2;
    HalfTmp ht;
    softmax_half<N, kb, rb, 0, EDGE>(S, sm, k0, pbuf, pb, ht);
    softmax_half<N, kb, rb, 1, EDGE>(S, sm, k0, pbuf, pb, ht);
  });
}
template <int N>
__device__ __forceinline__ void softmax_tile(f32x4 (&S)[2][N], Soft<N>& sm, int k0, bool edge,
                                             lds_u8* pbuf, const PBase& pb) {
  if (edge)
    softmax_tile_as<N, true>(S, sm, k0, pbuf, pb);
  else
    softmax_tile_as<N, false>(S, sm, k0, pbuf, pb);
}

// Rare path for tile t (its scores S still in registers): the references of
// the rows whose scores passed them move to the row maxima, the tile's P is
// formed again, and every O row and row sum formed against an old reference
// is rescaled.  Every wave of the workgroup calls it (two barriers).
template <int N>
__device__ __forceinline__ void move_references(f32x4 (&S)[2][N], Soft<N>& sm, int k0,
                                                bool edge, bool o_zero, lds_u8* lds, lds_u8* pbuf,
                                                const PBase& pb, int kh, int rh, int lane) {
  const int l16 = lane & 15, g = lane >> 4, l32 = lane & 31;
  typedef __attribute__((address_space(3))) float lds_f32;
  lds_f32* rowmax = (lds_f32*)(lds + kRowMaxOff);
  lds_f32* factor = (lds_f32*)(lds + kFactorOff);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // MFMA results settled
#pragma unroll
  for (int rb = 0; rb < N; ++rb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = !edge || k0 + 16 * kb + i <= sm.lim[rb] ? S[kb][rb][i] : -INFINITY;
        mx = fmaxf(mx, s);
      }
    mx = wave_max_across_groups(mx);
    if (g == 0) rowmax[kh * kMaxUnitRows + 16 * N * rh + 16 * rb + l16] = mx;
  }
  lds_barrier();
#pragma unroll
  for (int rb = 0; rb < N; ++rb) {
    const int row = 16 * N * rh + 16 * rb + l16;
    const float M = fmaxf(rowmax[row], rowmax[kMaxUnitRows + row]) * sm.c[rb];
    const bool first = sm.m[rb] == -INFINITY;
    const bool move = M > sm.m[rb] + kLazy;  // false for M = -inf
    const float mn = move ? M : sm.m[rb];
    const float f = !move ? 1.0f : first ? 0.0f : __builtin_amdgcn_exp2f(sm.m[rb] - mn);
    sm.l[rb] *= f;
    sm.m[rb] = mn;
    sm.nmu[rb] = mn == -INFINITY ? 0.0f : -mn;
    if (kh == 0 && g == 0) factor[row] = f;
  }
  softmax_tile<N>(S, sm, k0, edge, pbuf, pb);
#pragma unroll
  for (int rb = 0; rb < N; ++rb) sm.l[rb] += sm.ps[rb];
  lds_barrier();
  // O rows of row block pbk: every lane scales its row (rare: the AGPRs are
  // read, scaled and written back in place); nothing to scale while O is
  // still zero (the first tile, which sets the references)
  if (o_zero) return;
  static_for<N>([&](auto pc) {
    constexpr int pbk = decltype(pc)::value;
    const float f = factor[32 * pbk + l32];
    if (__builtin_amdgcn_ballot_w64(f != 1.0f) != 0) {
      static_for<4>([&](auto cc) { OAcc<decltype(cc)::value * N + pbk>::scale(f); });
    }
  });
}

// ------------------------------------------------------------------ unit

template <int N, bool PAGED, bool NT>
__device__ __forceinline__ void unit_fp8(const MainArgs& args, unsigned char* smem) {
  UnitSetup us;
  if (!unit_setup<kRowB, kKeys>(args, us)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave & 1, rh = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4, l32 = lane & 31, G = lane >> 5;
  lds_u8* lds = (lds_u8*)smem;
  const int T = us.uc.ntiles;

  Src<PAGED> src;
  src.base = us.kv_unit;
  src.pt_row = us.pt_row;
  src.lo = us.uc.lo;
  src.nkeys = us.uc.nkeys;
  src.shift = PAGED ? us.page_shift : 0;
  src.last_idx = PAGED ? us.last_page_idx : 0;
  src.max_page = PAGED ? (unsigned)(us.num_pages - 1) : 0u;
  const DmaLanes dl = dma_lanes(tid);

  // Q loads of the first row block, then tiles 0, 1, 2 start streaming into
  // slots 0, 1, 2, then Q is quantised (row block by row block) while the
  // tiles land.
  Soft<N> sm;
  QFrag<N> qf;
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(uniform_ptr(us.q + (int64_t)us.row0 * kDqk), (uint32_t)(us.RU * kDqk * 2));
  auto q_row = [&](int rb) { return min(16 * N * rh + 16 * rb + l16, us.RU - 1); };
  static_for<N>([&](auto rc) {
    constexpr int rb = decltype(rc)::value;
    const int rv = q_row(rb);
    sm.lim[rb] = min(us.hi_eff - 1, us.tail0 + (us.rowb0 + rv) / us.H) - us.uc.lo;
    sm.m[rb] = -INFINITY;
    sm.nmu[rb] = 0.0f;
    sm.l[rb] = 0.0f;
    sm.ps[rb] = 0.0f;
  });
  // Q of row block 0 into registers and (N >= 2) the other row blocks into
  // LDS slots 2..3, then tiles 0 and 1 start streaming while Q is quantised;
  // tile 2 follows once slot 2 is free again.
  {
    QRaw raw;
    load_q_raw(raw, qr, q_row(0), g);
    if constexpr (N >= 2) q_to_lds<N>(qr, lds, wave, lane);
    int e[2];
    constexpr int kEarly = N == 1 ? 3 : 2;  // tiles issued before the quantisation
#pragma unroll
    for (int k = 0; k < kEarly; ++k) {
      fetch_now(src, k, e);
      issue_tile<PAGED, NT>(src, k, e, lds + k * kTileB, dl, wave);
    }
    wait_q<q_dma_loads<N>() + 9 * kEarly>(raw);
    quantise_q<N, 0>(us, raw, g, qf, sm.c[0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (N >= 2) {
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");  // this wave's Q rows landed
      lds_barrier();                                      // and every other wave's
      static_for<N - 1>([&](auto rc) {
        constexpr int rb = decltype(rc)::value + 1;
        q_from_lds<N, rb>(raw, lds, rh, l16, g);
        quantise_q<N, rb>(us, raw, g, qf, sm.c[rb]);
        __builtin_amdgcn_sched_barrier(0);
      });
      lds_barrier();  // the Q rows are read before tile 2 overwrites slot 2
      fetch_now(src, 2, e);
      issue_tile<PAGED, NT>(src, 2, e, lds + 2 * kTileB, dl, wave);
    }
  }
  {
    const i32x8 z = {};
    static_for<4 * N>([&](auto bc) { OAcc<decltype(bc)::value>::zero(z); });
  }

  const KBase kb_ = k_base(kh, l16, g);
  const VBase vb = v_base(wave, lane);
  const PBase pb = p_base(kh, rh, N, lane);
  lds_u8* pbuf0 = lds + kPOff;

  f32x4 S[2][N];
  // Score MFMAs of one step (key block kb, column block db) into S[kb][.].
  auto qk_step = [&](auto kbc, auto dbc, const i32x8& kf) {
    constexpr int kb = decltype(kbc)::value, db = decltype(dbc)::value;
    static_for<N>([&](auto rc) {
      constexpr int rb = decltype(rc)::value;
      if constexpr (q_group<N>(rb, db) >= 0)
        QAcc<q_group<N>(rb, db)>::template qk<db == 0>(S[kb][rb], kf);
      else
        mfma_qk<db == 0, false>(S[kb][rb], kf, qf.q[rb][db]);
    });
  };
  // Scores of tile t (slot t % 4) into S, K fragments one step ahead of their
  // MFMAs (the first one, k0, read by the caller); hook(st) runs after the
  // MFMAs of step st (0..9).  N >= 2: key
  // block 0 first (N independent accumulators per step), so that the softmax
  // of key block 0 can run under the MFMAs of key block 1 (steps 5..9); N = 1:
  // the two key blocks alternate (their accumulators are the independent
  // MFMAs between dependent ones).
  constexpr bool kMajor = N >= 2;
  auto scores = [&](int t, const i32x8& k0, auto&& hook) {
    const lds_u8* slot = lds + (t % kSlots) * kTileB;
    i32x8 kf[2];
    kf[0] = k0;
    static_for<10>([&](auto sc) {
      constexpr int st = decltype(sc)::value;
      constexpr int kb = kMajor ? st / 5 : st % 2, db = kMajor ? st % 5 : st / 2;
      if constexpr (st + 1 < 10)
        kf[(st + 1) % 2] = read_k<(kMajor ? (st + 1) / 5 : (st + 1) % 2),
                                  (kMajor ? (st + 1) % 5 : (st + 1) / 2)>(slot, kb_);
      qk_step(std::integral_constant<int, kb>{}, std::integral_constant<int, db>{}, kf[st % 2]);
      if constexpr (kMajor && st == 4)
        asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");  // key block 0 retired before its softmax
      hook(sc);
      __builtin_amdgcn_sched_barrier(0);
    });
    asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");  // score MFMAs retired before VALU reads
  };

  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  typedef __attribute__((address_space(3))) unsigned lds_u32;
  if (T > 0) {
    wait_tiles_behind<18>();  // tile 0 landed (tiles 1 and 2 may still be in flight)
    lds_barrier();
    scores(0, read_k<0, 0>(lds, kb_), [](auto) {});
    // tile 0 sets the references: its flags force the rare path in the loop
    if (lane == 0) *(lds_u32*)(lds + kFlagOff + 4 * wave) = 1u;
  }

  // Iteration t: PV of tile t; with MORE (t + 1 < T) also the scores and P of
  // tile t + 1, masked when EDGE (tile t + 1 reaches past the smallest causal
  // limit of the unit's rows), and the 9 loads of tile t + 3.  Each variant is
  // straight-line code: no branch inside the MFMA stream.
  auto iteration = [&](int t, auto edge_c, auto more_c) {
    constexpr bool EDGE = decltype(edge_c)::value, MORE = decltype(more_c)::value;
    // tile t + 1 landed (tile t + 2 may still be in flight); the barrier
    // publishes it, P(t) and the flags of tile t
    wait_tiles_behind<9>();
    int e[2];
    barrier_fetch(src, t + 3, e);
    lds_u8* pbuf_t = pbuf0 + (t & 1) * kPBuf;
    const u32x4 fl = *(const lds_u32x4*)(lds + kFlagOff + (t & 1) * 16);
    // the first K fragment of tile t + 1 is read together with the flags
    // (its LDS latency overlaps theirs; the rare path leaves it alone)
    i32x8 k0;
    if constexpr (MORE) k0 = read_k<0, 0>(lds + ((t + 1) % kSlots) * kTileB, kb_);
    // tile t + 3 goes into the slot of tile t - 1 (read by the last PV)
    const TileLoads<PAGED, NT> tl(src, t + 3, e, lds + ((t + 3) % kSlots) * kTileB);
    if (__builtin_amdgcn_readfirstlane((fl[0] | fl[1]) | (fl[2] | fl[3])) != 0) {
      move_references<N>(S, sm, kKeys * t + 32 * kh + 4 * g, kKeys * t + kKeys - 1 > us.uc.min_lim,
                         t == 0, lds, pbuf_t, pb, kh, rh, lane);
    } else {
#pragma unroll
      for (int rb = 0; rb < N; ++rb) sm.l[rb] += sm.ps[rb];
    }

    const lds_u8* slot_t = lds + (t % kSlots) * kTileB;
    const int kq = kKeys * (t + 1) + 32 * kh + 4 * g;  // lane's first key of tile t + 1
    lds_u8* pbuf_n = pbuf0 + ((t + 1) & 1) * kPBuf;
#pragma unroll
    for (int rb = 0; rb < N; ++rb) sm.ps[rb] = 0.0f;
    HalfTmp ht;
    // half-slice h of the softmax of tile t + 1 over key block KB: row block
    // h / 2, half h % 2
    auto soft_half = [&](auto kbc, auto hc) {
      constexpr int kb = decltype(kbc)::value, h = decltype(hc)::value;
      softmax_half<N, kb, h / 2, h % 2, EDGE>(S, sm, kq, pbuf_n, pb, ht);
    };
    // P(t) and the first V fragments are read ahead of the PV MFMAs
    i32x8 P[N];
    i32x8 V[2];
    if constexpr (MORE) {
      scores(t + 1, k0, [&](auto sc) {
        constexpr int st = decltype(sc)::value;
        if constexpr (st < 9) tl.template issue<st>(dl, wave);  // load st of tile t + 3
        if constexpr (kMajor && st >= 5) {  // key block 0's softmax under key block 1's MFMAs
          constexpr int i = st - 5;
          static_for<2 * N>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            if constexpr ((h * 5) / (2 * N) == i) soft_half(std::integral_constant<int, 0>{}, hc);
          });
        }
      });
    }
    static_for<N>([&](auto pc) {
      constexpr int pbk = decltype(pc)::value;
      P[pbk] = read_p<pbk>(pbuf_t, pb);
    });
    V[0] = read_v<0>(slot_t, vb);
    __builtin_amdgcn_sched_barrier(0);
    // PV of tile t; the rest of the softmax of tile t + 1 between its MFMAs
    // (key block 1; with N = 1 both key blocks)
    constexpr int kHalves = N >= 2 ? 2 * N : 4 * N;
    static_for<4>([&](auto cc) {
      constexpr int cb = decltype(cc)::value;
      if constexpr (cb + 1 < 4) V[(cb + 1) % 2] = read_v<cb + 1>(slot_t, vb);
      static_for<N>([&](auto pc) {
        constexpr int pbk = decltype(pc)::value;
        OAcc<cb * N + pbk>::pv(V[cb % 2], P[pbk]);
        constexpr int mi = cb * N + pbk;  // MFMA index 0 .. 4 N - 1
        if constexpr (MORE) {
          static_for<kHalves>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            if constexpr ((h * 4 * N) / kHalves == mi) {
              if constexpr (N >= 2)
                soft_half(std::integral_constant<int, 1>{}, hc);
              else  // N = 1: halves 0..3 = key block 0 (h 0, 1), key block 1 (h 2, 3)
                soft_half(std::integral_constant<int, h / 2>{}, std::integral_constant<int, h % 2>{});
            }
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    if constexpr (MORE) {
      float psmax = sm.ps[0];
#pragma unroll
      for (int rb = 1; rb < N; ++rb) psmax = fmaxf(psmax, sm.ps[rb]);
      const unsigned any = __builtin_amdgcn_ballot_w64(psmax > 0x1p8f) != 0 ? 1u : 0u;
      if (lane == 0) *(lds_u32*)(lds + kFlagOff + ((t + 1) & 1) * 16 + 4 * wave) = any;
    }
  };

  // first tile that reaches past the smallest causal limit of the unit's rows
  const int min_lim = us.uc.min_lim;
  const int e0 = min_lim >= kKeys - 1 ? (min_lim - (kKeys - 1)) / kKeys + 1 : 0;
  const int t_plain = min(max(e0 - 1, 0), T - 1);
  const std::integral_constant<bool, false> no;
  const std::integral_constant<bool, true> yes;
  int t = 0;
  for (; t < t_plain; ++t) iteration(t, no, yes);
  for (; t < T - 1; ++t) iteration(t, yes, yes);
  if (T > 0) iteration(T - 1, no, no);  // the last tile's PV (its loads past the end are not issued)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads issued past the end

  // ---- epilogue: row sums, then O / l through LDS in full rows
  typedef __attribute__((address_space(3))) float lds_f32;
  lds_f32* lsum = (lds_f32*)(lds + kLsumOff);
  lds_f32* mref = (lds_f32*)(lds + kMrefOff);
#pragma unroll
  for (int rb = 0; rb < N; ++rb) {
    const float lt = wave_sum_across_groups(sm.l[rb]);
    const int row = 16 * N * rh + 16 * rb + l16;
    if (g == 0) {
      lsum[kh * kMaxUnitRows + row] = lt;
      if (kh == 0) mref[row] = sm.m[rb];
    }
  }
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // last PV MFMAs retired
  lds_barrier();
  const bool split = us.S > 1;
  lds_u8* stage = lds + wave * (kMaxUnitRows * 256);  // this wave's 96 rows x 128 bf16 columns
  float inv[N];
#pragma unroll
  for (int pbk = 0; pbk < N; ++pbk) {
    const int row = 32 * pbk + l32;
    const float l = lsum[row] + lsum[kMaxUnitRows + row];
    inv[pbk] = l > 0.0f ? us.o_scale / l : 0.0f;
    if (wave == 0 && G == 0 && row < us.RU) {
      const float lse = l > 0.0f ? (mref[row] + log2f(l)) * 0.69314718055994530942f : -INFINITY;
      if (split)
        us.part_lse[(int64_t)us.part_row0 + ((int64_t)us.t * us.S + us.s) * us.R + us.rowb0 + row] = lse;
      else
        us.lse[(int64_t)us.row0 + row] = lse;
    }
  }
  static_for<4>([&](auto cc) {
    constexpr int cb = decltype(cc)::value;
    static_for<N>([&](auto pc) {
      constexpr int pbk = decltype(pc)::value;
      const int row = 32 * pbk + l32;
      const f32x16 o = OAcc<cb * N + pbk>::read();  // one block through VGPRs at a time
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 pk;
        pk.x = pack_bf16x2(o[4 * a] * inv[pbk], o[4 * a + 1] * inv[pbk]);
        pk.y = pack_bf16x2(o[4 * a + 2] * inv[pbk], o[4 * a + 3] * inv[pbk]);
        const int lc = 4 * cb + a;  // 8-column chunk of the wave's 128 columns
        *(uint2*)(stage + row * 256 + 16 * (lc ^ (row & 15)) + 8 * G) = pk;
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  });
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  uint16_t* out = split ? us.part_o + ((int64_t)us.part_row0 + ((int64_t)us.t * us.S + us.s) * us.R +
                                       us.rowb0) * kDv
                        : us.o + (int64_t)us.row0 * kDv;
#pragma unroll
  for (int i = 0; i < 8 * N; ++i) {
    const int row = 4 * i + (lane >> 4), lc = lane & 15;
    if (row < us.RU) {
      const u32x4 v = *(const u32x4*)(stage + row * 256 + 16 * (lc ^ (row & 15)));
      *(u32x4*)(out + (int64_t)row * kDv + 128 * wave + 8 * lc) = v;
    }
  }
}

template <int N, bool PAGED, bool NT>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_fp8(const MainArgs args) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsBytes];
  unit_fp8<N, PAGED, NT>(args, smem);
  merge_if_last(args, smem);
  merge_grid(args, smem);
}

}  // namespace fp8k

// Launch of the fp8-KV main kernel over a launch's units; nrt = 16-row blocks
// per row half of the widest unit (1..3); nt: the non-temporal KV hint.
template <bool PAGED, bool NT>
static hipError_t launch_fp8_t(const MainArgs& a, int nrt, int grid, hipStream_t stream) {
  if (nrt == 1)
    hipLaunchKernelGGL((fp8k::mla_decode_fp8<1, PAGED, NT>), dim3(grid), dim3(fp8k::kThreads), 0, stream, a);
  else if (nrt == 2)
    hipLaunchKernelGGL((fp8k::mla_decode_fp8<2, PAGED, NT>), dim3(grid), dim3(fp8k::kThreads), 0, stream, a);
  else if (nrt == 3)
    hipLaunchKernelGGL((fp8k::mla_decode_fp8<3, PAGED, NT>), dim3(grid), dim3(fp8k::kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

#ifdef MLA_PAGED_KV
hipError_t launch_fp8_paged(const MainArgs& a, int nrt, bool nt, hipStream_t stream) {
  constexpr bool kPaged = true;
#else
hipError_t launch_fp8_contiguous(const MainArgs& a, int nrt, bool nt, hipStream_t stream) {
  constexpr bool kPaged = false;
#endif
  const int grid = ((a.num_units + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid == 0) return hipSuccess;
  return nt ? launch_fp8_t<kPaged, true>(a, nrt, grid, stream)
            : launch_fp8_t<kPaged, false>(a, nrt, grid, stream);
}

}  // namespace mla
