"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle.

Small shapes are compared element by element; the full-size workloads are
compared on sampled rows the oracle computes one by one.  Extra gates beyond
the graded tolerances: planted-key probes (exact answers), peaked queries (|O|
far above the tolerance), folded == unfolded, split invariance, bitwise replay
determinism, NaN-poisoned workspace."""
import numpy as np
import pytest

from mla_token_decode_amd import binding as mb
from mla_token_decode_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


SMALL_CASES = [
    # (H, q_len, kv_len, fp8)
    (12, [2], [4096], False),
    (12, [8], [700], False),
    (12, [8], [700], True),
    (96, [8], [300], False),
    (96, [3], [257], True),
    (24, [8], [129], False),
    (1, [1], [1], False),
    (6, [16], [16], False),
    (7, [20], [90], False),
    (40, [6], [200], True),
    (64, [2], [65], False),
    (128, [1], [130], False),
    (128, [2], [64], False),
    (12, [1, 2, 3, 4, 8], [33, 64, 65, 500, 8], False),
    (96, [1, 2, 3, 4], [100, 40, 9, 4], True),
    # fp8 KV at every row-group width of the key-split kernels: 128-row tiles
    # cut into 64-row units, 70- and 96-row tiles, kv_len == q_len
    (128, [1], [130], True),
    (64, [2], [65], True),
    (7, [20], [90], True),
    (6, [16], [16], True),
]


@pytest.mark.parametrize("H,q_len,kv_len,fp8", SMALL_CASES)
@pytest.mark.parametrize("peaked", [False, True])
def test_small_shapes_vs_oracle(H, q_len, kv_len, fp8, peaked):
    gu.log(f"case H={H} q={q_len} n={kv_len} fp8={fp8} peaked={peaked}")
    inp = gen.random_inputs(H, q_len, kv_len, fp8, seed=hash((H, len(q_len), kv_len[0])) % 1000)
    if peaked:
        inp = gen.peaked_inputs(inp, beta=10.0, seed=3)
    ro, rl = gu.oracle_full(inp)
    for splits in (0, 1, 3):
        o, lse, plan = gu.run_gpu(inp, force_splits=splits)
        gu.compare(o, lse, ro, rl, fp8, f"splits={splits} units={plan.num_units}")


@pytest.mark.parametrize("fp8", [False, True])
def test_planted_probe(fp8):
    H, q_len, kv_len = 12, [8, 3], [600, 200]
    markers = [[(0, 0), (63, 1), (64, 13), (600 - 8, 0), (600 - 7, 12), (599, 31), (150, 5),
                (191, 24), (192, 36), (255, 48), (256, 60)],
               [(0, 2), (199, 6), (198, 5), (197, 4), (63, 3), (64, 15), (127, 27)]]
    inp = gen.planted_inputs(H, q_len, kv_len, markers, fp8=fp8)
    ro, rl = gu.oracle_full(inp)
    # the same attention over |V| (sign bits of the 512 value columns cleared):
    # it bounds sum_s w_s |O_s| / sum_s w_s over the chunks of a split row
    kv_abs = inp.kv.copy()
    kv_abs[:, :512] &= 0x7F if fp8 else 0x7FFF
    ra, _ = gu.oracle_full(gen.Inputs(H, inp.q_len, inp.kv_len, inp.q_bits, kv_abs, fp8, inp.kv_scale))
    for splits in (1, 2, 5, 9):
        o, lse, plan = gu.run_gpu(inp, force_splits=splits)
        gu.log(f"planted fp8={fp8} splits={splits}")
        # bf16 rounding (unit roundoff 2^-8) is the only expected error on these
        # exact inputs: of the output, and for a split row also of each chunk's
        # normalised partial O (bf16 in the workspace) before the merge
        split = plan.query(0)[2] > 1 or plan.query(1)[2] > 1
        err = np.abs(o - ro) - 2.0 ** -8 * np.abs(ro) - (2.0 ** -8 * 1.01 * ra if split else 0.0)
        assert err.max() <= 1e-6, f"max excess {err.max()}"
        assert np.abs(lse - rl).max() <= 1e-3


@pytest.mark.parametrize("fp8", [False, True])
def test_folded_equals_unfolded(fp8):
    """Folding changes which rows share a tile, not a row's arithmetic: O and
    LSE match the unfolded run bitwise, except that with fp8 KV the 96-row
    tiles split each KV tile's keys between two waves, so a row's sum of P
    adds its two halves last (LSE within 2 fp32 ulps; O within 1 bf16 ulp)."""
    inp = gen.peaked_inputs(gen.random_inputs(12, [8, 4], [1000, 333], fp8, seed=5), beta=10.0)
    for splits in (1, 4):
        o1, l1, p1 = gu.run_gpu(inp, force_splits=splits)
        o2, l2, p2 = gu.run_gpu(inp, force_splits=splits, force_fold=1)
        assert p1.query(0)[0] == 8 and p2.query(0)[0] == 1
        same = np.array_equal(o1, o2) and np.array_equal(l1, l2)
        gu.log(f"folded vs unfolded splits={splits}: bitwise={same} "
               f"max|dO|={np.abs(o1 - o2).max():.3e} max|dLSE|={np.abs(l1 - l2).max():.3e}")
        if not fp8:
            assert same
        else:
            assert np.all(np.abs(o1 - o2) <= 2.0 ** -7 * np.abs(o2))
            assert np.all(np.abs(l1 - l2) <= 2 * np.spacing(np.abs(l2).astype(np.float32)))


def test_split_counts_agree():
    inp = gen.peaked_inputs(gen.random_inputs(12, [8], [5000], False, seed=7), beta=10.0)
    ro, rl = gu.oracle_full(inp)
    for splits in (1, 2, 7, 40, 79):
        o, lse, _ = gu.run_gpu(inp, force_splits=splits)
        gu.compare(o, lse, ro, rl, False, f"splits={splits}")


@pytest.mark.parametrize("fp8", [False, True])
def test_replay_is_bitwise_deterministic(fp8):
    inp = gen.random_inputs(96, [8], [3000], fp8, seed=9)
    dev = gu.to_device(inp)
    o1, l1, _ = gu.run_gpu(inp, dev)
    o2, l2, _ = gu.run_gpu(inp, dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fp8", [False, True])
def test_every_merge_layout_vs_oracle(fp8):
    """The split-KV merge folds a launch's rows in P = 1, 4, 8, 16 or 32 chunk
    phases (the fewest that keep each thread within one batch of 8 loads up to
    256 chunks; past that each thread loops): chunk counts on both sides of
    each switch and one past 256 (64-key chunks: kv_len = 64 S), then a launch
    that mixes a short and a long sequence (the longest sets the layout)."""
    for S in (2, 8, 9, 32, 33, 64, 65, 128, 129, 300):
        gu.log(f"merge layout S={S} fp8={fp8}")
        inp = gen.random_inputs(4, [2], [64 * S], fp8, seed=41 + S)
        ro, rl = gu.oracle_full(inp)
        o, lse, plan = gu.run_gpu(inp, force_splits=S)
        assert plan.query(0)[2] == S
        gu.compare(o, lse, ro, rl, fp8, f"S={S}")
    inp = gen.random_inputs(24, [1, 4, 2], [320, 70, 12800], fp8, seed=43)
    ro, rl = gu.oracle_full(inp)
    o, lse, plan = gu.run_gpu(inp, force_splits=200)
    assert [plan.query(b)[2] for b in range(3)] == [5, 2, 200]
    gu.compare(o, lse, ro, rl, fp8, "mixed chunk counts 5, 2, 200")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("batch,mode", [(130, mb.MLA_MERGE_REDUCE), (70, mb.MLA_MERGE_LAST_ARRIVER),
                                        (70, mb.MLA_MERGE_GRID)])
def test_large_batch_is_one_launch(fp8, batch, mode):
    """More than 60 sequences run as one launch whose descriptor tables sit in
    the workspace (uploaded by mla_decode_run, searched by the kernels): mixed
    q_len and lengths, split into up to 3 chunks, every merge, vs the oracle."""
    gu.log(f"large batch B={batch} merge={mode} fp8={fp8}")
    rng = np.random.default_rng(batch + 7 * mode)
    ql = rng.integers(1, 5, batch).tolist()
    kl = rng.integers(64, 700, batch).tolist()
    inp = gen.random_inputs(8, ql, kl, fp8, seed=batch + mode)
    ro, rl = gu.oracle_full(inp)
    o, lse, plan = gu.run_gpu(inp, force_splits=3, merge_mode=mode, poison_workspace=True)
    assert plan.num_launches == 1 and plan.num_split_tiles > 0
    assert plan.launch(0)[1] == mode, "the case must take the merge it names"
    gu.compare(o, lse, ro, rl, fp8, f"B={batch} merge={mode}")


@pytest.mark.parametrize("splits,fp8,mode", [
    (20, False, mb.MLA_MERGE_REDUCE),        # 4 chunk phases
    (40, False, mb.MLA_MERGE_REDUCE),        # 8
    (40, True, mb.MLA_MERGE_LAST_ARRIVER),
    (100, True, mb.MLA_MERGE_REDUCE),        # 16
    (150, True, mb.MLA_MERGE_REDUCE),        # 32
])
def test_large_batch_every_fold_layout(splits, fp8, mode):
    """More than 60 sequences with enough chunks that the merge reads the
    workspace tables in every fold layout (4 to 32 chunk phases): sequence b
    holds 64 splits - r_b keys (r_b < 64), so every sequence has exactly
    `splits` chunks and a ragged last one."""
    batch = 70
    gu.log(f"large batch B={batch} splits={splits} fp8={fp8} merge={mode}")
    rng = np.random.default_rng(splits + 3 * mode)
    kl = (64 * splits - rng.integers(0, 64, batch)).tolist()
    inp = gen.random_inputs(2, [1] * batch, kl, fp8, seed=splits)
    ro, rl = gu.oracle_full(inp)
    o, lse, plan = gu.run_gpu(inp, force_splits=splits, merge_mode=mode, poison_workspace=True)
    assert plan.num_launches == 1
    assert all(plan.query(b)[2] == splits for b in range(batch))
    assert plan.launch(0)[1] == mode
    gu.compare(o, lse, ro, rl, fp8, f"B={batch} splits={splits} merge={mode}")


@pytest.mark.parametrize("fp8", [False, True])
def test_large_mixed_batch_auto_plan(fp8):
    """80 sequences, about a third of them long: the automatic plan splits
    only those (and reorders the batch, longest first), so the merge's table
    of split sequences is a reordered subset of the descriptor table."""
    batch = 80
    rng = np.random.default_rng(1)
    kl = np.where(rng.random(batch) < 0.3, rng.integers(3000, 12000, batch),
                  rng.integers(16, 400, batch)).tolist()
    ql = rng.integers(1, 5, batch).tolist()
    gu.log(f"large mixed batch B={batch} fp8={fp8}")
    inp = gen.random_inputs(4, ql, kl, fp8, seed=88)
    ro, rl = gu.oracle_full(inp)
    o, lse, plan = gu.run_gpu(inp, poison_workspace=True)
    splits = [plan.query(b)[2] for b in range(batch)]
    assert plan.num_launches == 1
    assert 0 < sum(s > 1 for s in splits) < batch and max(splits) > 8
    gu.compare(o, lse, ro, rl, fp8, f"B={batch} auto plan, {sum(s > 1 for s in splits)} split")


@pytest.mark.parametrize("beta", [1.0, 2.0, 3.0])
def test_moderate_peaks_fp8(beta):
    """Dominant keys a few octaves above the rest, below the reference-move
    threshold of the fp8 kernels, so P reaches values that e4m3 rounds (up to
    2^8): O stays within the fp8 tolerance and LSE (from fp32 sums) within
    the LSE tolerance."""
    inp = gen.peaked_inputs(gen.random_inputs(12, [8, 3], [2000, 700], True, seed=47), beta=beta,
                            seed=8)
    ro, rl = gu.oracle_full(inp)
    for splits in (1, 4):
        o, lse, _ = gu.run_gpu(inp, force_splits=splits)
        gu.compare(o, lse, ro, rl, True, f"beta={beta} splits={splits}")


@pytest.mark.parametrize("fp8", [False, True])
def test_large_logit_jumps_move_the_reference(fp8):
    """Rows whose running maximum rises by more than 60 octaves after their
    first tile, several times, in and across split chunks: the kernel moves
    its softmax reference and rescales O and l in place."""
    H, q_len, kv_len = 12, [4, 2], [1000, 3000]
    targets = [(0, 0, 0, [100, 300, 700, 990]),    # four jumps inside one sequence
               (0, 3, 11, [31, 32, 600]),          # last key of tile 0, first of tile 1
               (0, 2, 6, [0, 64, 65, 500]),
               (1, 1, 5, [5, 1500, 2999]),         # 2999: the last key this row sees
               (1, 0, 0, [2000, 2500])]
    inp = gen.escalating_inputs(H, q_len, kv_len, targets, fp8=fp8, seed=23)
    # the input is discriminating: each planted key lifts its row's running
    # maximum (base-2 logits) by more than 60 octaves
    import oracle
    q = gen.f32_from_bf16_bits(inp.q_bits).astype(np.float64)
    if fp8:
        table = np.array([oracle.e4m3_to_double(c) for c in range(256)])
        kvd = table[inp.kv] * inp.kv_scale
    else:
        kvd = gen.f32_from_bf16_bits(inp.kv).astype(np.float64)
    q_off, kv_off = np.concatenate([[0], np.cumsum(q_len)]), np.concatenate([[0], np.cumsum(kv_len)])
    for (b, i, h, pos) in targets:
        n = kv_len[b]
        lim = n - q_len[b] + i
        x = kvd[kv_off[b]:kv_off[b] + lim + 1] @ q[q_off[b] + i, h] * inp.sm_scale / np.log(2.0)
        for p in pos:
            before = x[:p].max() if p > 0 else -np.inf
            assert x[p] > before + 60.0 or p == 0, (b, i, h, p, x[p], before)
    ro, rl = gu.oracle_full(inp)
    for splits in (1, 3, 7):
        o, lse, plan = gu.run_gpu(inp, force_splits=splits)
        gu.compare(o, lse, ro, rl, fp8, f"escalating splits={splits} units={plan.num_units}")


@pytest.mark.parametrize("fp8", [False, True])
def test_reference_moves_in_96_row_tiles(fp8):
    """Reference moves in the 96-row tiles of H=12, q=8 (with fp8 KV the
    key-split pipeline: a move found at tile t rescales O after the PV of
    tile t - 1): jumps on either half of a tile's keys, on the first and the
    last tile, and at chunk boundaries."""
    H, q_len, kv_len = 12, [8], [1500]
    targets = [(0, 7, 0, [3, 17, 40, 1499]),     # keys of both halves of tiles 0 and 1; last key
               (0, 0, 11, [15, 16, 700]),        # the two halves of tile 0
               (0, 4, 5, [31, 32, 33, 1200]),    # last key of tile 0, first keys of tile 1
               (0, 6, 9, [63, 64, 1024])]        # chunk boundaries of 64-key chunks
    inp = gen.escalating_inputs(H, q_len, kv_len, targets, fp8=fp8, seed=29)
    ro, rl = gu.oracle_full(inp)
    for splits in (1, 5, 24):
        o, lse, plan = gu.run_gpu(inp, force_splits=splits)
        gu.compare(o, lse, ro, rl, fp8, f"96-row escalating splits={splits} units={plan.num_units}")


def test_poisoned_workspace_is_never_read_unwritten():
    inp = gen.random_inputs(12, [8, 2], [3000, 77], False, seed=13)
    ro, rl = gu.oracle_full(inp)
    o, lse, _ = gu.run_gpu(inp, poison_workspace=True, force_splits=6)
    gu.compare(o, lse, ro, rl, False, "poisoned workspace")


def test_outputs_outside_the_rows_are_untouched():
    import torch
    from mla_token_decode_amd import binding as mb
    inp = gen.random_inputs(12, [4], [900], False, seed=17)
    plan = mb.Plan(12, inp.q_len, inp.kv_len, False, force_splits=3)
    q, kv = gu.to_device(inp)
    rows = 4 * 12
    guard = 4096
    o_big = torch.full((rows * 512 + 2 * guard,), -7.0, dtype=torch.bfloat16, device="cuda")
    l_big = torch.full((rows + 2 * guard,), -7.0, dtype=torch.float32, device="cuda")
    o = o_big[guard:guard + rows * 512]
    lse = l_big[guard:guard + rows]
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    mb.mla_decode_run(plan, q, kv, inp.sm_scale, 1.0, o, lse, ws, ws.numel())
    mb.mla_decode_reduce(plan, ws, o, lse)
    torch.cuda.synchronize()
    ob, lb = o_big.float().cpu().numpy(), l_big.cpu().numpy()
    assert np.all(ob[:guard] == -7.0) and np.all(ob[guard + rows * 512:] == -7.0)
    assert np.all(lb[:guard] == -7.0) and np.all(lb[guard + rows:] == -7.0)
    ro, rl = gu.oracle_full(inp)
    gu.compare(o.double().cpu().numpy().reshape(4, 12, 512), lse.double().cpu().numpy().reshape(4, 12),
               ro, rl, False, "guarded")


def test_identical_keys_give_the_value_row():
    inp = gen.identical_key_inputs(12, [8, 1], [40, 1000], seed=19)
    o, lse, _ = gu.run_gpu(inp, force_splits=3)
    kv = gen.f32_from_bf16_bits(inp.kv).astype(np.float64)
    np.testing.assert_allclose(o[:8], np.broadcast_to(kv[0, :512], (8, 12, 512)), rtol=2 ** -7, atol=1e-6)
    np.testing.assert_allclose(o[8:], np.broadcast_to(kv[40, :512], (1, 12, 512)), rtol=2 ** -7, atol=1e-6)
    ro, rl = gu.oracle_full(inp)
    assert np.abs(lse - rl).max() <= 1e-3


def _check_covers_every_sequence(inp, rows):
    q_off = np.concatenate([[0], np.cumsum(inp.q_len)]) * inp.H
    for b in range(inp.batch):
        assert np.any((rows >= q_off[b]) & (rows < q_off[b + 1])), f"sequence {b} not sampled"
        assert q_off[b] in rows and q_off[b + 1] - 1 in rows


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_workload_sampled_rows(name):
    gu.log(f"workload {name}")
    inp = gu.workload_inputs(name)
    o, lse, plan = gu.run_gpu(inp)
    gu.log(f"  plan: units={plan.num_units} split_tiles={plan.num_split_tiles} "
           f"fold/tiles/splits/L of seq0={plan.query(0)}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rows = gu.sample_rows(inp, 24 if name != "small" else 48)
    _check_covers_every_sequence(inp, rows)
    gu.log(f"  {len(rows)} rows compared")
    ro, rl = gu.oracle_rows(inp, rows)
    gu.compare(o.reshape(-1, 512)[rows], lse.reshape(-1)[rows], ro, rl, inp.kv_fp8, name)


@pytest.mark.parametrize("name", ["h12_131k", "h96_125k", "h12_1m_fp8", "ragged"])
def test_workload_peaked_sampled_rows(name):
    gu.log(f"peaked workload {name}")
    inp = gen.peaked_inputs(gu.workload_inputs(name), beta=10.0, seed=1)
    o, lse, _ = gu.run_gpu(inp)
    rows = gu.sample_rows(inp, 16, seed=2)
    _check_covers_every_sequence(inp, rows)
    ro, rl = gu.oracle_rows(inp, rows)
    do, dl, mo = gu.compare(o.reshape(-1, 512)[rows], lse.reshape(-1)[rows], ro, rl, inp.kv_fp8,
                            f"{name} peaked")
    assert mo > 5 * gu.TOL_O[inp.kv_fp8]  # the check is discriminating
    # every sampled row is discriminating, not only the largest one
    per_row = np.abs(ro).max(axis=1)
    assert np.all(per_row > gu.TOL_O[inp.kv_fp8]), f"rows with small |O|: {np.sum(per_row <= gu.TOL_O[inp.kv_fp8])}"


@pytest.mark.parametrize("fp8", [False, True])
def test_query_rows_of_very_different_magnitudes(fp8):
    """Query rows scaled by powers of two from 2^-16 to 2^4, all-zero rows, and
    rows whose latent part is vanishingly small next to their rope part: the
    fp8 path quantises Q per row, so each row's scale must follow its own
    magnitude (and stay finite)."""
    H, q_len, kv_len = 12, [8, 3], [2000, 700]
    inp = gen.peaked_inputs(gen.random_inputs(H, q_len, kv_len, fp8, seed=29), beta=10.0, seed=6)
    q = gen.f32_from_bf16_bits(inp.q_bits).astype(np.float32)
    rows = q.shape[0] * H
    qr = q.reshape(rows, gen.DQK)
    k = np.arange(rows) % 21 - 16  # 2^-16 .. 2^4, exact in bf16
    qr *= np.float32(2.0) ** k[:, None].astype(np.float32)
    qr[5] = 0.0
    qr[40] = 0.0
    qr[17, :gen.DV] *= np.float32(2.0 ** -100)  # latent ~1e-31 next to an O(1) rope part
    qr[63, :gen.DV] = 0.0                          # rope part only
    # rows whose largest |q| is below 448 / FLT_MAX: 448 / max|q| overflows fp32,
    # so the per-row fp8 scale must be bounded (bf16 subnormals and zeros)
    qr[70] *= np.float32(2.0 ** -130)
    qr[71] *= np.float32(2.0 ** -140)
    qr[72, :gen.DV] = np.float32(2.0 ** -133)      # one subnormal step, latent part only
    qr[72, gen.DV:] = 0.0
    # rows whose entries, scaled so that the largest maps to 448, sit just
    # under e4m3 rounding midpoints of several binades (and the largest a hair
    # below the top code, so q * 448 / max|q| rounds across it)
    mids = np.array([0.5 * (a + b) for a, b in [(256, 288), (112, 120), (28, 30), (3.5, 3.75),
                                                 (0.4375, 0.46875), (2 ** -7, 1.5 * 2 ** -7)]])
    vals = (mids * (1 - 2 ** -7) / 448.0).astype(np.float32)
    for r, scale in ((73, 1.0), (74, 3.0), (75, 2.0 ** -20)):
        row = np.resize(vals, gen.DQK).astype(np.float32) * np.float32(scale)
        row[::7] *= -1
        row[5] = np.float32(scale * (1 - 2 ** -9))
        qr[r] = row
    inp = gen.Inputs(H, inp.q_len, inp.kv_len, gen.bf16_bits_from_f32(q), inp.kv, inp.kv_fp8,
                     inp.kv_scale)
    ro, rl = gu.oracle_full(inp)
    for splits in (1, 4):
        o, lse, plan = gu.run_gpu(inp, force_splits=splits)
        gu.compare(o, lse, ro, rl, fp8, f"row magnitudes splits={splits}")


def test_binding_rejects_tensors_that_do_not_match_the_plan():
    """Short, strided or wrongly typed device tensors are refused by the
    binding (ValueError) before any kernel is launched."""
    import torch
    from mla_token_decode_amd import binding as mb
    inp = gen.random_inputs(12, [4], [300], False, seed=31)
    plan = mb.Plan(12, inp.q_len, inp.kv_len, False, force_splits=2)
    q, kv = gu.to_device(inp)
    o, lse, ws = mb.alloc_outputs(plan, q.device)
    bad = [
        dict(kv=kv[:299]),                                   # fewer KV rows than the plan
        dict(q=q[:3]),                                       # fewer Q rows
        dict(o=o.view(-1)[: o.numel() - 512]),               # short O
        dict(lse=lse.view(-1)[:-1]),                         # short LSE
        dict(kv=kv.view(torch.int16)),                       # wrong dtype
        dict(q=q.transpose(1, 2).contiguous().transpose(1, 2)),  # strided
        dict(lse=lse.to(torch.float64)),
    ]
    for c in bad:
        kw = dict(q=q, kv=kv, o=o, lse=lse)
        kw.update(c)
        with pytest.raises(ValueError):
            mb.mla_decode_run(plan, kw["q"], kw["kv"], inp.sm_scale, 1.0, kw["o"], kw["lse"], ws)
    fp8 = gen.random_inputs(12, [4], [300], True, seed=31)
    p8 = mb.Plan(12, fp8.q_len, fp8.kv_len, True)
    with pytest.raises(ValueError):  # bf16 KV given to an fp8 plan
        mb.mla_decode_run(p8, q, kv, inp.sm_scale, 0.01, o, lse, ws)
