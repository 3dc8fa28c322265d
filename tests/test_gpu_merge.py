"""GPU: the split-KV merges -- in the main kernel (by the last unit of a split
row block to finish, or by the whole grid once the last unit is done) and the
reduce kernel -- each checked against the oracle on the same inputs
("bench(cake_mla_varq_dcp_decode): ..." (flashinfer PR #5588), table "What
was measured", row "split rows", where an in-kernel merge replaced the reduce
kernel).  The in-kernel merges count arrivals in workspace words tagged with
each call's epoch and a generation, so the tests also run them on a zeroed,
a 0xff-filled and a reused workspace, and replay them from a captured graph
(the same epoch every replay); all must give the same bits."""
import numpy as np
import pytest

from mla_token_decode_amd import binding as mb
from mla_token_decode_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

IN_KERNEL = [mb.MLA_MERGE_LAST_ARRIVER, mb.MLA_MERGE_GRID]

CASES = [
    # (H, q_len, kv_len, fp8, force_splits)
    (96, [1, 2, 3, 4], [3000, 2000, 2500, 1300], False, 0),
    (96, [1, 2, 3, 4], [3000, 2000, 2500, 1300], True, 3),
    (12, [8], [5000], True, 3),
    (12, [8, 1, 3], [2000, 700, 4096], False, 4),
    (24, [2, 4], [130, 64], True, 2),
    (12, [8], [20000], True, 40),     # 8 chunk phases
    (16, [2, 5], [9000, 6000], False, 24),
    (12, [8], [64 * 150], False, 150),  # 32 chunk phases
]


def _run(inp, dev, ws_fill, merge_mode, force_splits, ws=None, plan=None):
    import torch
    if plan is None:
        plan = mb.Plan(inp.H, inp.q_len, inp.kv_len, inp.kv_fp8, merge_mode=merge_mode,
                       force_splits=force_splits)
    q, kv = dev
    o, lse, ws_new = mb.alloc_outputs(plan, q.device)
    if ws is None:
        ws = ws_new
        if ws_fill is not None:
            ws.fill_(ws_fill)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    mb.mla_decode_run(plan, q, kv, inp.sm_scale, inp.kv_scale, o, lse, ws, ws.numel())
    mb.mla_decode_reduce(plan, ws, o, lse)
    torch.cuda.synchronize()
    return o.cpu().clone(), lse.cpu().clone(), ws, plan


@pytest.mark.parametrize("mode", IN_KERNEL)
@pytest.mark.parametrize("H,ql,kl,fp8,fs", CASES)
def test_in_kernel_merge_vs_reduce_kernel(H, ql, kl, fp8, fs, mode):
    gu.log(f"merge mode={mode} H={H} q={ql} n={kl} fp8={fp8} splits={fs}")
    inp = gen.peaked_inputs(gen.random_inputs(H, ql, kl, fp8, seed=60 + H), beta=10.0, seed=3)
    dev = gu.to_device(inp)
    ro, rl = gu.oracle_full(inp)
    o_k, l_k, ws, plan_k = _run(inp, dev, None, mode, fs)
    assert plan_k.num_split_tiles > 0, "the case must have split tiles"
    assert plan_k.launch(0)[1] == mode, "the case must take the in-kernel merge"
    o_r, l_r, _, _ = _run(inp, dev, None, mb.MLA_MERGE_REDUCE, fs)
    gu.compare(o_k.double().numpy(), l_k.double().numpy(), ro, rl, fp8, f"in-kernel merge {mode}")
    gu.compare(o_r.double().numpy(), l_r.double().numpy(), ro, rl, fp8, "reduce kernel")
    # the same partial rows, folded in the same chunk order: within 1 bf16 ulp
    d = np.abs(o_k.double().numpy() - o_r.double().numpy())
    assert np.all(d <= 2.0 ** -7 * np.abs(o_r.double().numpy()) + 1e-30), float(d.max())
    if mode == mb.MLA_MERGE_GRID:  # the reduce kernel's own fold and layout: the same bits
        assert torch_equal(o_k, o_r) and torch_equal(l_k, l_r)


@pytest.mark.parametrize("mode", IN_KERNEL)
@pytest.mark.parametrize("fp8", [False, True])
def test_in_kernel_merge_ignores_prior_workspace_contents(fp8, mode):
    H, ql, kl = 96, [2, 3], [2600, 1900]
    gu.log(f"workspace contents mode={mode} fp8={fp8}")
    inp = gen.random_inputs(H, ql, kl, fp8, seed=77)
    dev = gu.to_device(inp)
    ref_o, ref_l, ws, plan = _run(inp, dev, 0, mode, 3)
    assert plan.launch(0)[1] == mode
    for fill in (0xFF, 0, 0x5A):
        o, l, _, _ = _run(inp, dev, fill, mode, 3)
        assert torch_equal(o, ref_o) and torch_equal(l, ref_l), f"workspace filled with {fill:#x}"
    for rep in range(3):  # the same workspace again: new epochs, the words of the last call
        o, l, _, _ = _run(inp, dev, None, mode, 3, ws=ws, plan=plan)
        assert torch_equal(o, ref_o) and torch_equal(l, ref_l), f"reuse {rep}"


@pytest.mark.parametrize("mode", IN_KERNEL)
def test_in_kernel_merge_of_rows_that_see_no_key(mode):
    # a key shard whose last keys are hidden from the first verify tokens
    import torch
    gu.log(f"rows that see no key mode={mode}")
    H, q, n = 12, 8, 3000
    inp = gen.random_inputs(H, [q], [n], True, seed=81)
    a, b = 2100, 3000
    sh = gen.Inputs(H, inp.q_len.copy(), np.array([b - a], np.int32), inp.q_bits,
                    np.ascontiguousarray(inp.kv[a:b]), True, inp.kv_scale)
    qd, kvd = gu.to_device(sh)
    outs = []
    for mm in (mode, mb.MLA_MERGE_REDUCE):
        plan = mb.Plan(H, [q], [b - a], True, causal_end=[n - a - 895], force_splits=3,
                       merge_mode=mm)
        assert plan.launch(0)[1] == mm
        o, lse, ws = mb.alloc_outputs(plan, qd.device)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        mb.mla_decode_run(plan, qd, kvd, sh.sm_scale, sh.kv_scale, o, lse, ws, ws.numel())
        mb.mla_decode_reduce(plan, ws, o, lse)
        torch.cuda.synchronize()
        outs.append((o.double().cpu().numpy(), lse.double().cpu().numpy()))
    (ok, lk), (orr, lr) = outs
    empty = np.isneginf(lr)
    assert empty.any() and (~empty).any()
    assert np.array_equal(np.isneginf(lk), empty)
    assert np.all(ok[empty] == 0.0)
    assert np.all(np.abs(ok[~empty] - orr[~empty]) <= 2.0 ** -7 * np.abs(orr[~empty]) + 1e-30)


@pytest.mark.parametrize("mode", IN_KERNEL + [mb.MLA_MERGE_REDUCE])
def test_graph_replays_match_the_eager_call(mode):
    """A captured graph launches with the arguments of capture time (one
    epoch for every replay): each replay must still merge, and give the bits
    of the eager call.  Eager calls with other inputs run on the same
    workspace between the replays."""
    import torch
    gu.log(f"graph replay mode={mode}")
    H, ql, kl, fp8 = 12, [8], [20000], True
    inp = gen.random_inputs(H, ql, kl, fp8, seed=91)
    other = gen.random_inputs(H, ql, kl, fp8, seed=92)
    q, kv = gu.to_device(inp)
    q2, kv2 = gu.to_device(other)
    plan = mb.Plan(H, ql, kl, fp8, merge_mode=mode, force_splits=40)
    assert plan.launch(0)[1] == mode
    o, lse, ws = mb.alloc_outputs(plan, q.device)
    o2, lse2, _ = mb.alloc_outputs(plan, q.device)

    def call(qq, kk, oo, ll):
        mb.mla_decode_run(plan, qq, kk, inp.sm_scale, inp.kv_scale, oo, ll, ws, ws.numel())
        mb.mla_decode_reduce(plan, ws, oo, ll)

    call(q, kv, o, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    call(q2, kv2, o2, lse2)
    torch.cuda.synchronize()
    ref_o2, ref_l2 = o2.clone(), lse2.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(q, kv, o, lse)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch_equal(o.cpu(), ref_o.cpu()) and torch_equal(lse.cpu(), ref_l.cpu()), f"replay {rep}"
        call(q2, kv2, o2, lse2)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        assert torch_equal(o2.cpu(), ref_o2.cpu()) and torch_equal(lse2.cpu(), ref_l2.cpu()), f"eager {rep}"


def test_graph_replays_of_a_large_plan():
    """A plan of more than 60 sequences copies its descriptor tables into the
    workspace on every run (an asynchronous copy from the plan's pinned host
    buffer, which a captured graph holds as a copy node).  Eager runs of
    another large plan overwrite those tables between the replays; every
    replay must still give the bits of the eager call."""
    import torch
    gu.log("graph replay of a 70-sequence plan, 90-sequence plan between replays")
    rng = np.random.default_rng(5)

    def make(batch, seed):
        return gen.random_inputs(8, rng.integers(1, 5, batch).tolist(),
                                 rng.integers(64, 700, batch).tolist(), False, seed=seed)

    inp, other = make(70, 11), make(90, 12)
    q, kv = gu.to_device(inp)
    q2, kv2 = gu.to_device(other)
    plan = mb.Plan(inp.H, inp.q_len, inp.kv_len, False, force_splits=3)
    plan2 = mb.Plan(other.H, other.q_len, other.kv_len, False, force_splits=3)
    assert plan.num_launches == 1 and plan2.num_launches == 1
    assert plan.num_split_tiles > 0 and plan2.num_split_tiles > 0
    o, lse, ws = mb.alloc_outputs(plan, q.device)
    o2, lse2, ws2 = mb.alloc_outputs(plan2, q.device)
    ws = ws if ws.numel() >= ws2.numel() else ws2  # one workspace for both plans

    def call(pl, qq, kk, oo, ll, src):
        mb.mla_decode_run(pl, qq, kk, src.sm_scale, src.kv_scale, oo, ll, ws, ws.numel())
        mb.mla_decode_reduce(pl, ws, oo, ll)

    call(plan, q, kv, o, lse, inp)
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    call(plan2, q2, kv2, o2, lse2, other)
    torch.cuda.synchronize()
    ref_o2, ref_l2 = o2.clone(), lse2.clone()
    ro, rl = gu.oracle_full(inp)
    gu.compare(o.cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, False, "eager, 70 sequences")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(plan, q, kv, o, lse, inp)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch_equal(o.cpu(), ref_o.cpu()) and torch_equal(lse.cpu(), ref_l.cpu()), f"replay {rep}"
        call(plan2, q2, kv2, o2, lse2, other)  # the other plan's tables into the same workspace
        torch.cuda.synchronize()
        assert torch_equal(o2.cpu(), ref_o2.cpu()) and torch_equal(lse2.cpu(), ref_l2.cpu()), f"eager {rep}"


def torch_equal(a, b):
    import torch
    return bool(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                            b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)))
