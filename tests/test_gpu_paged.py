"""GPU parity of paged KV (mla_decode_run_paged): the KV rows of every
sequence are scattered over the pages of a pool in a seeded random order,
with poison values in every page slot and page tail that holds no key.  The
paged run must give exactly the O and LSE of mla_decode_run on the
contiguous KV with the same plan (the same arithmetic; only the row
addresses differ), match the oracle, and give the same result again when the
pool is re-permuted under a new page table with the same plan."""
import numpy as np
import pytest

from mla_token_decode_amd import binding as mb
from mla_token_decode_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # (H, q_len, kv_len, page_size, force_splits)
    (12, [8], [3000], 32, 0),
    (12, [8], [3000], 64, 3),
    (96, [2], [700], 64, 0),
    (12, [1, 3, 2, 4], [100, 2048, 513, 1200], 256, 0),
    (16, [4, 1], [4097, 64], 4096, 2),
    # more than 60 sequences: one launch, its descriptor tables in the workspace
    (8, ([1, 2, 3, 4] * 18)[:70], [65 + (97 * i) % 640 for i in range(70)], 64, 3),
]


def paginate(inp, page_size, seed):
    """(pool [num_pages, page_size, 576], page table int32 [batch, stride])
    holding the rows of inp.kv; unused slots and page tails are poison."""
    rng = np.random.default_rng(seed)
    counts = [(int(n) + page_size - 1) // page_size for n in inp.kv_len]
    num_pages = sum(counts) + 3  # pages no sequence uses
    slots = rng.permutation(num_pages)
    stride = max(counts) + 2
    table = rng.integers(0, num_pages, size=(len(counts), stride), dtype=np.int32)  # never read
    kv = np.asarray(inp.kv)
    poison = np.uint8(0x7E) if inp.kv_fp8 else np.uint16(0x7F7F)  # 448 / 3.4e38
    pool = np.full((num_pages, page_size, kv.shape[1]), poison, dtype=kv.dtype)
    row0, k = 0, 0
    for b, n in enumerate(int(x) for x in inp.kv_len):
        for p in range(counts[b]):
            slot = int(slots[k])
            k += 1
            table[b, p] = slot
            rows = kv[row0 + p * page_size: row0 + min((p + 1) * page_size, n)]
            pool[slot, :len(rows)] = rows
        row0 += n
    return pool, table


def pool_to_device(pool, fp8):
    import torch
    if fp8:
        return torch.from_numpy(pool).cuda()
    return torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).cuda()


def run(plan, inp, q, kv=None, paged=None):
    import torch
    o, lse, ws = mb.alloc_outputs(plan, q.device)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    if paged is None:
        mb.mla_decode_run(plan, q, kv, inp.sm_scale, inp.kv_scale, o, lse, ws, ws.numel())
    else:
        pool, table = paged
        mb.mla_decode_run_paged(plan, q, pool, table, inp.sm_scale, inp.kv_scale, o, lse, ws,
                                ws.numel())
    mb.mla_decode_reduce(plan, ws, o, lse)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy(), lse.cpu().numpy(), o.double().cpu().numpy()


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("H,q_len,kv_len,page,splits", CASES)
def test_paged_equals_contiguous(H, q_len, kv_len, page, splits, fp8):
    import torch
    gu.log(f"paged H={H} q={q_len} kv={kv_len} page={page} splits={splits} fp8={fp8}")
    inp = gen.peaked_inputs(gen.random_inputs(H, q_len, kv_len, fp8, seed=7 + H), beta=10.0, seed=3)
    q, kv = gu.to_device(inp)
    plan = mb.Plan(H, q_len, kv_len, fp8, force_splits=splits, num_cus=0)
    ob, lb, od = run(plan, inp, q, kv=kv)
    for rep in range(2):  # the second run: the pool re-permuted, a new table, the same plan
        pool, table = paginate(inp, page, seed=100 * rep + page)
        pb, pl, _ = run(plan, inp, q, paged=(pool_to_device(pool, fp8),
                                             torch.from_numpy(table).cuda()))
        assert np.array_equal(pb, ob), f"O differs from the contiguous run (table {rep})"
        assert np.array_equal(pl, lb), f"LSE differs from the contiguous run (table {rep})"
    ro, rl = gu.oracle_full(inp)
    gu.compare(od, lb.astype(np.float64), ro, rl, fp8, "paged vs oracle")


def test_paged_many_sequences_span_launches():
    """70 sequences need two launches (60 sequence descriptors per launch): the
    second launch must index the page table from its own first sequence."""
    import torch
    rng = np.random.default_rng(11)
    kv_len = [int(x) for x in rng.integers(40, 300, size=70)]
    q_len = [1 + int(x) for x in rng.integers(0, 2, size=70)]
    inp = gen.peaked_inputs(gen.random_inputs(12, q_len, kv_len, False, seed=12), beta=10.0, seed=4)
    q, kv = gu.to_device(inp)
    plan = mb.Plan(12, q_len, kv_len, False, num_cus=0)
    ob, lb, od = run(plan, inp, q, kv=kv)
    pool, table = paginate(inp, 32, seed=5)
    pb, pl, _ = run(plan, inp, q, paged=(pool_to_device(pool, False), torch.from_numpy(table).cuda()))
    assert np.array_equal(pb, ob) and np.array_equal(pl, lb)
    ro, rl = gu.oracle_full(inp)
    gu.compare(od, lb.astype(np.float64), ro, rl, False, "paged, 70 sequences")
