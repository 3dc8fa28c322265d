"""C-ABI library: loads, exports every symbol include/mla_decode.h declares,
and its host plan agrees with the oracle's independent fold / split code.
CPU only: no compute call touches a GPU here (num_cus is passed explicitly)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from mla_token_decode_amd import binding as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = mb.lib()
    names = declared_functions()
    assert set(names) == set(mb.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_status_codes_match_the_header():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    enum = {k: int(v) for k, v in re.findall(r"\b(MLA_(?:OK|ERR_[A-Z_]+))\s*=\s*(\d+)", text)}
    assert "MLA_ERR_OUT_OF_MEMORY" in enum
    binding = {n: getattr(mb, n) for n in dir(mb) if n == "MLA_OK" or n.startswith("MLA_ERR_")}
    assert enum == binding


def plan(H, q_len, kv_len, fp8=False, **kw):
    kw.setdefault("num_cus", 256)
    return mb.Plan(H, q_len, kv_len, fp8, **kw)


@pytest.mark.parametrize("H", [1, 6, 7, 12, 24, 40, 48, 64, 96, 128])
def test_fold_matches_oracle(H):
    for q in range(1, 17):
        p = plan(H, [q], [max(q, 100)])
        F, T, S, L = p.query(0)
        assert F == oracle.fold_factor(H, q), (H, q)
        assert T == q // F


def test_force_fold_caps_fold():
    p = plan(12, [8, 6, 4], [50, 50, 50], force_fold=1)
    assert [p.query(b)[0] for b in range(3)] == [1, 1, 1]
    p = plan(12, [8, 6, 4], [50, 50, 50], force_fold=3)
    assert [p.query(b)[0] for b in range(3)] == [2, 3, 2]


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 100, 127, 128, 129, 4096, 125000, 131072, 1048576])
@pytest.mark.parametrize("S", [1, 2, 3, 7, 16, 100, 257])
def test_forced_split_layout_bit_exact(n, S):
    q = 1
    p = plan(12, [q], [n], force_splits=S)
    _, _, S_eff, L = p.query(0)
    assert (L, S_eff) == oracle.split_layout(n, S, mb.KV_GRANULE)


def test_auto_plan_shapes_of_the_workloads():
    # bf16 H=12 q=8 ctx 131072: one 96-row tile, split so every CU has work
    p = plan(12, [8], [131072])
    F, T, S, L = p.query(0)
    assert (F, T) == (8, 1) and S > 1 and L % 64 == 0
    assert p.workspace_bytes > 0
    # H=96 q=8: F=1, eight tiles
    p = plan(96, [8], [125000])
    assert p.query(0)[:2] == (1, 8)
    # ragged
    ql = [1, 2, 3, 4] * 8
    p = plan(96, ql, [32768] * 32)
    for b in range(32):
        assert p.query(b)[:2] == (1, ql[b])
    # short context: a single chunk needs no workspace when forced
    p = plan(12, [2], [4096], force_splits=1)
    assert p.query(0)[2] == 1 and p.workspace_bytes == 0


def test_workspace_size_formula():
    H, ql, kl = 12, [8, 3, 1], [5000, 700, 64]
    p = plan(H, ql, kl, force_splits=4, merge_mode=mb.MLA_MERGE_REDUCE)
    rows = 0
    for b in range(3):
        F, T, S, L = p.query(b)
        if S > 1:
            rows += T * S * H * F
    lse_bytes = -(-rows * 4 // 256) * 256
    assert p.workspace_bytes == lse_bytes + rows * 512 * 2  # fp32 LSE, then bf16 O per partial row
    # the in-kernel merge adds one 64-bit arrival word per partial row (256-byte aligned)
    q = plan(H, ql, kl, force_splits=4, merge_mode=mb.MLA_MERGE_LAST_ARRIVER)
    base = -(-(lse_bytes + rows * 512 * 2) // 256) * 256
    assert q.workspace_bytes == base + rows * 8
    # the grid merge adds one 64-bit counter per launch (256-byte aligned)
    g = plan(H, ql, kl, force_splits=4, merge_mode=mb.MLA_MERGE_GRID)
    assert g.launch(0)[1] == mb.MLA_MERGE_GRID
    assert g.workspace_bytes == base + g.num_launches * 8


def test_merge_mode_choice():
    # AUTO: the reduce kernel; GRID: where a launch's units fit the CUs at once
    # (units rounded up to a multiple of 8 <= num_cus)
    head = plan(12, [8], [1048576], True)
    units, mode = head.launch(0)
    assert (units + 7) // 8 * 8 <= 256 and mode == mb.MLA_MERGE_REDUCE
    for mm, want in ((mb.MLA_MERGE_REDUCE, mb.MLA_MERGE_REDUCE),
                     (mb.MLA_MERGE_LAST_ARRIVER, mb.MLA_MERGE_LAST_ARRIVER),
                     (mb.MLA_MERGE_GRID, mb.MLA_MERGE_GRID)):
        assert plan(12, [8], [1048576], True, merge_mode=mm).launch(0)[1] == want
    # more units than CUs: no grid merge even when asked for
    for mm in (mb.MLA_MERGE_AUTO, mb.MLA_MERGE_GRID):
        p = plan(12, [8], [1048576], True, force_splits=300, merge_mode=mm)
        assert p.launch(0)[0] > 256 and p.launch(0)[1] == mb.MLA_MERGE_REDUCE
        assert p.workspace_bytes == plan(12, [8], [1048576], True, force_splits=300,
                                         merge_mode=mb.MLA_MERGE_REDUCE).workspace_bytes
    # the same plan for a device with fewer CUs
    p = plan(12, [8], [1048576], True, num_cus=128, merge_mode=mb.MLA_MERGE_GRID)
    assert p.launch(0)[1] == (mb.MLA_MERGE_GRID if p.launch(0)[0] <= 128 else mb.MLA_MERGE_REDUCE)
    # an arrival word counts to 65535: a sequence of more chunks is left to the reduce kernel
    p = plan(1, [1], [64 * 70000], merge_mode=mb.MLA_MERGE_LAST_ARRIVER, force_splits=70000)
    assert p.query(0)[2] == 70000 and p.launch(0)[1] == mb.MLA_MERGE_REDUCE
    # a launch with no split rows reports 0
    assert plan(12, [2], [4096], force_splits=1).launch(0)[1] == 0
    for bad in (4, -1):
        with pytest.raises(mb.MlaError):
            plan(12, [1], [100], merge_mode=bad)
    with pytest.raises(mb.MlaError):
        head.launch(1)


def test_many_sequences_run_as_one_launch_with_a_descriptor_table():
    # up to 60 sequence descriptors travel in the kernel arguments; a larger
    # batch is still one launch, its descriptors in the workspace
    small = plan(8, [1] * 60, [300] * 60, force_splits=1)
    assert small.num_launches == 1 and small.workspace_bytes == 0
    big = plan(8, [1] * 150, [300] * 150, force_splits=1)
    assert big.num_launches == 1 and big.launch(0)[0] == big.num_units
    desc = 60  # bytes of one sequence descriptor
    assert 150 * desc <= big.workspace_bytes < 150 * desc + 1024  # no split: the table alone
    split = plan(8, [1] * 150, [3000] * 150, force_splits=3)
    assert split.num_launches == 1 and split.num_split_tiles == 150


@pytest.mark.parametrize("args,status", [
    ((12, [0], [10]), mb.MLA_ERR_INVALID_ARGUMENT),
    ((12, [5], [4]), mb.MLA_ERR_INVALID_ARGUMENT),
    ((0, [1], [4]), mb.MLA_ERR_INVALID_ARGUMENT),
    ((129, [1], [4]), mb.MLA_ERR_UNSUPPORTED),
    ((12, [], []), mb.MLA_ERR_INVALID_ARGUMENT),
])
def test_plan_rejects(args, status):
    with pytest.raises(mb.MlaError) as e:
        plan(*args)
    assert e.value.status == status
    assert e.value.message


def test_run_rejects_bad_arguments_before_touching_a_device():
    p = plan(12, [2], [100], force_splits=2)
    good = 1 << 20
    cases = [
        dict(q=None), dict(q=good + 8), dict(sm_scale=0.0), dict(sm_scale=float("nan")),
        dict(kv_scale=2.0), dict(workspace_bytes=p.workspace_bytes - 1),
    ]
    for c in cases:
        kw = dict(q=good, kv=good, sm_scale=0.04, kv_scale=1.0, o=good, lse=good, workspace=good,
                  workspace_bytes=p.workspace_bytes, stream=0)
        kw.update(c)
        with pytest.raises(mb.MlaError) as e:
            mb.mla_decode_run(p, **kw)
        assert e.value.status in (mb.MLA_ERR_INVALID_ARGUMENT, mb.MLA_ERR_WORKSPACE_TOO_SMALL)
    pf = plan(12, [2], [100], fp8=True)
    with pytest.raises(mb.MlaError):
        mb.mla_decode_run(pf, good, good, 0.04, 0.0, good, good, good, pf.workspace_bytes, 0)


def test_query_out_of_range():
    p = plan(4, [1, 1], [3, 3])
    with pytest.raises(mb.MlaError):
        p.query(2)


def test_shard_plan_validation():
    # a shard may hold fewer keys than verify tokens
    p = mb.Plan(12, [8], [5], False, causal_end=[5], num_cus=256)
    assert p.query(0)[0] == 8
    for bad in ([0], [-3]):
        with pytest.raises(mb.MlaError) as e:
            mb.Plan(12, [8], [100], False, causal_end=bad, num_cus=256)
        assert e.value.status == mb.MLA_ERR_INVALID_ARGUMENT
    with pytest.raises(mb.MlaError) as e:
        mb.Plan(12, [8], [0], False, causal_end=[10], num_cus=256)
    assert e.value.status == mb.MLA_ERR_INVALID_ARGUMENT
    # a whole-sequence plan still needs kv_len >= q_len
    with pytest.raises(mb.MlaError):
        mb.Plan(12, [8], [5], False, num_cus=256)


def test_shard_plan_without_causal_end_is_rejected():
    L = mb.lib()
    qa = (ctypes.c_int32 * 1)(8)
    ka = (ctypes.c_int32 * 1)(100)
    opts = mb._Options(0, 0, 256)
    h = ctypes.c_void_p()
    st = L.mla_decode_plan_shard(1, 12, qa, ka, None, mb.MLA_KV_BF16, ctypes.byref(opts),
                                 ctypes.byref(h), None)
    assert st == mb.MLA_ERR_INVALID_ARGUMENT and not h.value


def test_merge_shards_argument_checks():
    L = mb.lib()
    fake = 1 << 20  # aligned, never dereferenced: the checks reject before any device work
    for rows, shards in ((0, 2), (4, 0), (4, mb.MAX_SHARDS + 1)):
        assert L.mla_merge_shards(rows, shards, fake, fake, fake, fake, None) == mb.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_merge_shards(4, 2, None, fake, fake, fake, None) == mb.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_merge_shards(4, 2, fake + 4, fake, fake, fake, None) == mb.MLA_ERR_INVALID_ARGUMENT


def test_paged_run_argument_checks():
    """mla_decode_run_paged rejects page sizes that are not powers of two in
    [32, 2^20] as unsupported, and an empty pool, a null or misaligned page
    table or a stride shorter than the longest sequence as invalid, before
    any device work."""
    L = mb.lib()
    p = plan(12, [8], [3000])
    fake = 1 << 20  # aligned, never dereferenced

    def call(num_pages=64, page=64, table=fake, stride=64):
        return L.mla_decode_run_paged(p.handle, fake, fake, num_pages, page, table, stride, 0.04,
                                      1.0, fake, fake, fake, 1 << 30, None)

    for page in (0, -64, 1, 16, 48, 96, 1 << 21):
        assert call(page=page) == mb.MLA_ERR_UNSUPPORTED, page
    assert call(num_pages=0) == mb.MLA_ERR_INVALID_ARGUMENT
    assert call(table=None) == mb.MLA_ERR_INVALID_ARGUMENT
    assert call(table=fake + 2) == mb.MLA_ERR_INVALID_ARGUMENT
    assert call(page=64, stride=46) == mb.MLA_ERR_INVALID_ARGUMENT  # 3000 keys need 47 pages
    assert call(page=32, stride=93) == mb.MLA_ERR_INVALID_ARGUMENT  # ... or 94
    assert "page" in mb.lib().mla_last_error().decode()


def test_binding_rejects_host_tensors_before_the_library_call():
    """The binding checks torch tensors against the plan before their pointers
    reach the kernels: a host tensor is refused with ValueError (the
    device-side size, dtype and contiguity checks are in the GPU suite)."""
    import torch
    p = plan(12, [2], [100], force_splits=2)
    q = torch.zeros((2, 12, mb.DQK), dtype=torch.bfloat16)
    kv = torch.zeros((100, mb.DQK), dtype=torch.bfloat16)
    o = torch.zeros((2, 12, mb.DV), dtype=torch.bfloat16)
    lse = torch.zeros((2, 12), dtype=torch.float32)
    ws = torch.zeros((p.workspace_bytes,), dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):
        mb.mla_decode_run(p, q, kv, 0.04, 1.0, o, lse, ws, stream=0)
    with pytest.raises(ValueError, match="device"):
        mb.mla_decode_reduce(p, ws, o, lse, stream=0)
