"""Seeded synthetic inputs for MLA speculative-verify decode.

This module draws and encodes inputs only; it holds none of the attention
arithmetic, and both the HIP path's tests and the CPU oracle consume what it
makes.  Every array is a deterministic function of its seed.

Encodings:
  * bf16: round-to-nearest-even of an fp32 value (integer bit arithmetic).
  * fp8: OCP E4M3FN, per-tensor scale s = fp32(amax|x| / 448); the code is the
    round-to-nearest-even, saturating (to +-448) encoding of fp32(x / s).

Workloads (shapes and value distributions of the decode problem: one shared
576-wide latent KV head, q verify tokens per sequence, all values drawn as
N(0,1) * 0.1 in fp32 before encoding, softmax scale 1/sqrt(576)):
  small     H=12, q=2,  ctx=4096, bf16                       seed 1
  h12_131k  H=12, q=8,  ctx=131072, bf16                     seed 2
  h96_125k  H=96, q=8,  ctx=125000, bf16                     seed 3
  h12_1m_fp8 H=12, q=8, ctx=1048576, fp8 KV, bf16 Q           seed 4
  ragged    32 sequences, H=96, q_b uniform in {1..4}, ctx=32768 each, bf16  seed 5
Random streams: Q <- PCG64 seeded [seed, 0]; KV row block k (65536 rows) <-
[seed, 1, k]; ragged q lengths <- [seed, 2].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DQK = 576
DV = 512
KV_BLOCK_ROWS = 65536
E4M3_MAX = 448.0
SM_SCALE = float(np.float32(1.0 / math.sqrt(576.0)))  # exactly 1/24 rounded to fp32


# --------------------------------------------------------------------- codecs

def bf16_bits_from_f32(x) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(bits) -> np.ndarray:
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3_codes_from_f32(y) -> np.ndarray:
    """OCP E4M3FN round-to-nearest-even, saturating at +-448 (never emits NaN)."""
    import torch  # CPU-only use: the dtype's cast is RNE but not saturating

    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(y).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


# ------------------------------------------------------------------ workloads

@dataclass
class Workload:
    name: str
    H: int
    q_len: list
    kv_len: list
    kv_fp8: bool
    seed: int
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.q_len)

    @property
    def sum_q(self) -> int:
        return int(sum(self.q_len))

    @property
    def sum_kv(self) -> int:
        return int(sum(self.kv_len))

    def kv_bytes(self) -> int:
        return self.sum_kv * DQK * (1 if self.kv_fp8 else 2)


def ragged_q_lens(seed: int, batch: int = 32) -> list:
    rng = np.random.default_rng([seed, 2])
    return [int(v) for v in rng.integers(1, 5, size=batch)]


def workload(name: str) -> Workload:
    if name == "small":
        return Workload(name, 12, [2], [4096], False, 1,
                        "bf16, batch 1, H=12, q=2, ctx=4096")
    if name == "h12_131k":
        return Workload(name, 12, [8], [131072], False, 2,
                        "bf16, batch 1, H=12, q=8 (F=8, 96 rows), ctx=131072")
    if name == "h96_125k":
        return Workload(name, 96, [8], [125000], False, 3,
                        "bf16, batch 1, H=96, q=8 (F=1, 8 tiles of 96 rows), ctx=125000")
    if name == "h12_1m_fp8":
        return Workload(name, 12, [8], [1048576], True, 4,
                        "fp8-e4m3 KV (per-tensor scale, amax->448), bf16 Q, batch 1, H=12, q=8, ctx=1048576")
    if name == "ragged":
        ql = ragged_q_lens(5, 32)
        return Workload(name, 96, ql, [32768] * 32, False, 5,
                        "bf16, 32 sequences, H=96, q_b uniform {1..4}, ctx=32768 each")
    if name in ("batch150", "batch150_fp8"):  # more sequences than the kernel arguments hold
        rng = np.random.default_rng([6, 3])
        kl = [int(v) for v in rng.integers(2048, 4097, size=150)]
        fp8 = name.endswith("fp8")
        return Workload(name, 12, [2] * 150, kl, fp8, 6,
                        f"{'fp8-e4m3' if fp8 else 'bf16'} KV, 150 sequences, H=12, q=2, "
                        "ctx uniform in [2048, 4096]")
    raise KeyError(name)


WORKLOADS = ["small", "h12_131k", "h96_125k", "h12_1m_fp8", "ragged"]


# ------------------------------------------------------------------ generators

def _normal_f32(rng, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(0.1)


def gen_q_bits(seed: int, sum_q: int, H: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 0])
    return bf16_bits_from_f32(_normal_f32(rng, (sum_q, H, DQK)))


def _kv_block_f32(seed: int, block: int, rows: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 1, block])
    return _normal_f32(rng, (rows, DQK))


def gen_kv(seed: int, rows: int, fp8: bool):
    """Returns (kv array, kv_scale).  bf16: uint16 bits and scale 1.0.
    fp8: uint8 codes and the fp32 per-tensor scale (amax -> 448)."""
    nblk = (rows + KV_BLOCK_ROWS - 1) // KV_BLOCK_ROWS
    sizes = [min(KV_BLOCK_ROWS, rows - k * KV_BLOCK_ROWS) for k in range(nblk)]
    if not fp8:
        out = np.empty((rows, DQK), dtype=np.uint16)
        for k, r in enumerate(sizes):
            out[k * KV_BLOCK_ROWS:k * KV_BLOCK_ROWS + r] = bf16_bits_from_f32(_kv_block_f32(seed, k, r))
        return out, 1.0
    amax = np.float32(0.0)
    for k, r in enumerate(sizes):
        amax = max(amax, np.float32(np.max(np.abs(_kv_block_f32(seed, k, r)))))
    scale = np.float32(amax / np.float32(E4M3_MAX))
    out = np.empty((rows, DQK), dtype=np.uint8)
    for k, r in enumerate(sizes):
        x = _kv_block_f32(seed, k, r)
        out[k * KV_BLOCK_ROWS:k * KV_BLOCK_ROWS + r] = e4m3_codes_from_f32(x / scale)
    return out, float(scale)


@dataclass
class Inputs:
    H: int
    q_len: np.ndarray
    kv_len: np.ndarray
    q_bits: np.ndarray      # uint16 [sum q, H, 576]
    kv: np.ndarray          # uint16 bf16 bits or uint8 e4m3 codes [sum n, 576]
    kv_fp8: bool
    kv_scale: float
    sm_scale: float = SM_SCALE

    @property
    def batch(self) -> int:
        return len(self.q_len)


def gen_workload_inputs(w: Workload) -> Inputs:
    q = gen_q_bits(w.seed, w.sum_q, w.H)
    kv, scale = gen_kv(w.seed, w.sum_kv, w.kv_fp8)
    return Inputs(w.H, np.asarray(w.q_len, np.int32), np.asarray(w.kv_len, np.int32), q, kv,
                  w.kv_fp8, scale)


def random_inputs(H: int, q_len, kv_len, fp8: bool, seed: int) -> Inputs:
    """Small random case with the workloads' distribution (tests)."""
    q_len = np.asarray(q_len, np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    q = gen_q_bits(seed, int(q_len.sum()), H)
    kv, scale = gen_kv(seed, int(kv_len.sum()), fp8)
    return Inputs(H, q_len, kv_len, q, kv, fp8, scale)


def peaked_inputs(base: Inputs, beta: float = 10.0, seed: int = 0) -> Inputs:
    """Same KV; each query row becomes beta * sign(KV row j*) for a seeded
    random key j* the row can see (sign taken from the stored bit pattern), so
    that row's softmax concentrates on j* and |O| is far above the tolerances.
    Needs no attention arithmetic: only sign bits and integer index draws."""
    rng = np.random.default_rng([seed, 7])
    H = base.H
    q = np.empty_like(base.q_bits)
    q_off = np.concatenate([[0], np.cumsum(base.q_len)]).astype(np.int64)
    kv_off = np.concatenate([[0], np.cumsum(base.kv_len)]).astype(np.int64)
    sign_shift = 7 if base.kv_fp8 else 15
    plus = bf16_bits_from_f32(np.float32(beta))
    minus = bf16_bits_from_f32(np.float32(-beta))
    for b in range(base.batch):
        n, qb = int(base.kv_len[b]), int(base.q_len[b])
        for i in range(qb):
            visible = n - qb + i + 1
            targets = rng.integers(0, visible, size=H)
            rows = base.kv[kv_off[b] + targets]                      # [H, 576]
            neg = ((rows.astype(np.uint32) >> sign_shift) & 1).astype(bool)
            q[q_off[b] + i] = np.where(neg, minus, plus)
    return Inputs(H, base.q_len.copy(), base.kv_len.copy(), q, base.kv, base.kv_fp8, base.kv_scale)


def planted_inputs(H: int, q_len, kv_len, marker_positions, fp8: bool = False,
                   amp: float = 32.0) -> Inputs:
    """Planted-key probe.  All keys are zero except marker rows.  Query row
    (token i, head h) of sequence b is amp * e_{512 + d}, d = (i * H + h) % 64,
    i.e. it looks only at one rope column.  Marker m at position p of sequence
    b carries amp in rope column 512 + dir and a value code in columns 0..511
    (column (p % 512) holds (p % 251 + 1) / 8, column ((p + 7) % 512) holds
    -(b + 1) / 8), all exactly representable.  marker_positions: list over
    sequences of lists of (position, dir).  A row whose direction matches a
    visible marker scores amp^2/24 there and 0 elsewhere."""
    q_len = np.asarray(q_len, np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    sum_q, sum_n = int(q_len.sum()), int(kv_len.sum())
    qf = np.zeros((sum_q, H, DQK), np.float32)
    q_off = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int64)
    kv_off = np.concatenate([[0], np.cumsum(kv_len)]).astype(np.int64)
    for b in range(len(q_len)):
        for i in range(int(q_len[b])):
            for h in range(H):
                qf[q_off[b] + i, h, DV + (i * H + h) % 64] = amp
    kvf = np.zeros((sum_n, DQK), np.float32)
    for b, marks in enumerate(marker_positions):
        for (p, d) in marks:
            r = kv_off[b] + p
            kvf[r, DV + d] = amp
            kvf[r, p % DV] = (p % 251 + 1) / 8.0
            kvf[r, (p + 7) % DV] = -(b + 1) / 8.0
    q_bits = bf16_bits_from_f32(qf)
    if fp8:
        amax = np.float32(np.max(np.abs(kvf)))
        scale = np.float32(amax / np.float32(E4M3_MAX))
        # amp / scale = 448 exactly when amax == amp; value codes stay exact
        # when scale is a power of two, which the default amp=32 ensures only
        # approximately; tests use the decoded values, so exactness is not needed.
        kv = e4m3_codes_from_f32(kvf / scale)
        return Inputs(H, q_len, kv_len, q_bits, kv, True, float(scale))
    return Inputs(H, q_len, kv_len, q_bits, bf16_bits_from_f32(kvf), False, 1.0)


def escalating_inputs(H: int, q_len, kv_len, targets, fp8: bool = False, seed: int = 0) -> Inputs:
    """Stress input for the running softmax reference.  Query rows are random
    +-1 sign vectors; keys are N(0,1)*0.1 except planted ones.  targets: list of
    (sequence b, token i, head h, [p_1, p_2, ...]); the 64 rope columns of key
    p_j of sequence b are set to 2^(j+4) times the rope signs of query row
    (i, h) of b (its 512 value columns stay random, so |O| stays small).  With
    the softmax scale 1/24 that row's score at p_j is 64 * 2^(j+4) / 24 *
    log2(e), i.e. about 123 * 2^(j-1) octaves: every planted key lifts the row's
    running maximum by more than 60 octaves."""
    q_len = np.asarray(q_len, np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    sum_q, sum_n = int(q_len.sum()), int(kv_len.sum())
    rng = np.random.default_rng([seed, 7])
    qf = np.where(rng.random((sum_q, H, DQK)) < 0.5, -1.0, 1.0).astype(np.float32)
    kvf = (rng.standard_normal((sum_n, DQK)) * 0.1).astype(np.float32)
    q_off = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int64)
    kv_off = np.concatenate([[0], np.cumsum(kv_len)]).astype(np.int64)
    for (b, i, h, positions) in targets:
        for j, p in enumerate(positions, start=1):
            kvf[kv_off[b] + p, DV:] = np.float32(2.0 ** (j + 4)) * qf[q_off[b] + i, h, DV:]
    q_bits = bf16_bits_from_f32(qf)
    if fp8:
        amax = np.float32(np.max(np.abs(kvf)))
        scale = np.float32(amax / np.float32(E4M3_MAX))
        return Inputs(H, q_len, kv_len, q_bits, e4m3_codes_from_f32(kvf / scale), True,
                      float(scale))
    return Inputs(H, q_len, kv_len, q_bits, bf16_bits_from_f32(kvf), False, 1.0)


def identical_key_inputs(H: int, q_len, kv_len, seed: int) -> Inputs:
    """Every KV row of a sequence equals one random row: each query row's
    output is that row's first 512 columns and its LSE is s + ln(visible)."""
    q_len = np.asarray(q_len, np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    q = gen_q_bits(seed, int(q_len.sum()), H)
    rng = np.random.default_rng([seed, 9])
    rows = []
    for b in range(len(q_len)):
        r = bf16_bits_from_f32(_normal_f32(rng, (1, DQK)))
        rows.append(np.repeat(r, int(kv_len[b]), axis=0))
    return Inputs(H, q_len, kv_len, q, np.concatenate(rows, axis=0), False, 1.0)
