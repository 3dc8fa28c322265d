"""GPU: mla_decode_run_static (the entry point for callers that cannot
allocate) against mla_decode_run + mla_decode_reduce with a caller workspace,
through the C ABI: bitwise equal outputs (the same kernels and arithmetic),
on calls in a row that reuse the library's static workspace, the second and
third with smaller plans; plans that need more than the static workspace are
rejected; plans with no split work need none."""
import numpy as np
import pytest

from mla_token_decode_amd import binding as mb
from mla_token_decode_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _static(inp, dev, **plan_opts):
    import torch
    plan = mb.Plan(inp.H, inp.q_len, inp.kv_len, inp.kv_fp8, **plan_opts)
    q, kv = dev
    o, lse, _ = mb.alloc_outputs(plan, q.device)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    mb.mla_decode_run_static(plan, q, kv, inp.sm_scale, inp.kv_scale, o, lse)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), plan


@pytest.mark.parametrize("fp8", [False, True])
def test_static_workspace_matches_caller_workspace(fp8):
    cases = [  # (H, q_len, kv_len, force_splits): large first, then smaller
        (12, [8], [20000], 40),
        (12, [8, 2], [3000, 500], 6),
        (96, [1, 3], [900, 100], 2),
    ]
    for H, q_len, kv_len, splits in cases:
        gu.log(f"static workspace fp8={fp8} H={H} q={q_len} n={kv_len} splits={splits}")
        inp = gen.peaked_inputs(gen.random_inputs(H, q_len, kv_len, fp8, seed=71), beta=10.0, seed=2)
        dev = gu.to_device(inp)
        o1, l1, p1 = gu.run_gpu(inp, dev, poison_workspace=True, force_splits=splits)
        o2, l2, p2 = _static(inp, dev, force_splits=splits)
        assert p2.workspace_bytes > 0
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), \
            f"max|dO|={np.abs(o1 - o2).max()} max|dLSE|={np.abs(l1 - l2).max()}"
        ro, rl = gu.oracle_full(inp)
        gu.compare(o2, l2, ro, rl, fp8, "static workspace vs oracle")


def test_static_workspace_full_size_headline_and_limit():
    """The headline workload's plan (about 25 MB of partials) fits the static
    workspace and matches the caller-workspace run bitwise; a plan above
    32 MiB is rejected with WORKSPACE_TOO_SMALL and launches nothing."""
    import torch
    inp = gu.workload_inputs("h12_1m_fp8")
    dev = gu.to_device(inp)
    o1, l1, p1 = gu.run_gpu(inp, dev)
    assert 0 < p1.workspace_bytes <= mb.STATIC_WORKSPACE_BYTES
    o2, l2, _ = _static(inp, dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # then a smaller call again
    small = gen.random_inputs(12, [2], [4096], False, seed=3)
    sdev = gu.to_device(small)
    o3, l3, _ = gu.run_gpu(small, sdev)
    o4, l4, _ = _static(small, sdev)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
    big = mb.Plan(96, [8] * 8, [300000] * 8, False, force_splits=64)
    assert big.workspace_bytes > mb.STATIC_WORKSPACE_BYTES
    q = torch.zeros((64, 96, mb.DQK), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((8 * 300000, mb.DQK), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((64, 96, mb.DV), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((64, 96), dtype=torch.float32, device="cuda")
    with pytest.raises(mb.MlaError) as e:
        mb.mla_decode_run_static(big, q, kv, 1 / 24, 1.0, o, lse)
    assert e.value.status == mb.MLA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0  # nothing was launched


def test_static_entry_point_first_run_of_a_large_plan():
    """A plan of more than 60 sequences uploads its descriptor tables from the
    pinned host buffer made when the plan was created: the static entry
    point, as the plan's first run, allocates nothing and matches the
    caller-workspace run bitwise."""
    rng = np.random.default_rng(9)
    batch = 70
    gu.log(f"static entry point, first run of a {batch}-sequence plan")
    inp = gen.random_inputs(8, rng.integers(1, 5, batch).tolist(), rng.integers(64, 700, batch).tolist(),
                            False, seed=9)
    dev = gu.to_device(inp)
    o2, l2, p2 = _static(inp, dev, force_splits=3)
    assert p2.num_launches == 1 and p2.num_split_tiles > 0
    assert 0 < p2.workspace_bytes <= mb.STATIC_WORKSPACE_BYTES
    o1, l1, _ = gu.run_gpu(inp, dev, poison_workspace=True, force_splits=3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_static_entry_point_without_split_work():
    inp = gen.random_inputs(12, [4], [200], False, seed=5)
    dev = gu.to_device(inp)
    o1, l1, _ = gu.run_gpu(inp, dev, force_splits=1)
    o2, l2, p = _static(inp, dev, force_splits=1)
    assert p.workspace_bytes == 0
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
