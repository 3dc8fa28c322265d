"""GPU parity of key-shard decoding (decode context parallelism on one GPU):
one sequence's keys are cut into contiguous shards, each shard is decoded
with its causal end through mla_decode_plan_shard, every shard's (O, LSE)
is checked against the oracle's partial over the same keys (under the whole
sequence's causal rule), and mla_merge_shards of the shard results is checked
against the oracle on the whole sequence."""
import numpy as np
import pytest

import oracle
from mla_token_decode_amd import binding as mb
from mla_token_decode_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # (H, q, n, shard cut points); the last shard of the first case holds
    # fewer keys than there are verify tokens, so some rows see none of it
    (12, 8, 3000, [0, 1000, 2100, 2995]),
    (96, 8, 700, [0, 350, 696]),
    (12, 4, 5000, [0, 2500]),
    (24, 2, 130, [0, 64, 65, 128, 129]),
]


def shard_inputs(inp, a, b):
    """Inputs holding keys [a, b) of the single sequence of `inp`."""
    return gen.Inputs(inp.H, inp.q_len.copy(), np.array([b - a], np.int32), inp.q_bits,
                      np.ascontiguousarray(inp.kv[a:b]), inp.kv_fp8, inp.kv_scale)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("H,q,n,cuts", CASES)
def test_key_shards(H, q, n, cuts, fp8):
    import torch
    gu.log(f"shards H={H} q={q} n={n} cuts={cuts} fp8={fp8}")
    inp = gen.peaked_inputs(gen.random_inputs(H, [q], [n], fp8, seed=41 + H), beta=10.0, seed=5)
    bounds = list(zip(cuts, cuts[1:] + [n]))
    q_dev = gu.to_device(inp)[0]
    o_shards, lse_shards = [], []
    for a, b in bounds:
        sh = shard_inputs(inp, a, b)
        kv_dev = gu.to_device(sh)[1]
        ro = np.empty((q, H, mb.DV))
        rl = np.empty((q, H))
        for i in range(q):
            for h in range(H):
                ro[i, h], rl[i, h] = oracle.mla_partial(
                    inp.q_bits, inp.kv, inp.q_len, inp.kv_len, H, 0, i, h, a, b,
                    kv_is_fp8=fp8, kv_scale=inp.kv_scale, sm_scale=inp.sm_scale)
        empty = np.isneginf(rl)
        for splits in (0, 3):
            plan = mb.Plan(H, [q], [b - a], fp8, causal_end=[n - a], force_splits=splits,
                           num_cus=0)
            o, lse, ws = mb.alloc_outputs(plan, q_dev.device)
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            mb.mla_decode_run(plan, q_dev, kv_dev, sh.sm_scale, sh.kv_scale, o, lse, ws, ws.numel())
            mb.mla_decode_reduce(plan, ws, o, lse)
            torch.cuda.synchronize()
            go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
            assert np.all(np.isneginf(gl[empty])), "rows that see no key need LSE = -inf"
            assert np.all(go[empty] == 0.0), "rows that see no key need O = 0"
            if (~empty).any():
                gu.compare(go[~empty], gl[~empty], ro[~empty], rl[~empty], fp8,
                           f"shard [{a},{b}) splits={splits} empty_rows={int(empty.sum())}")
        o_shards.append(o)
        lse_shards.append(lse)
    # combine the shards (each shard's last result) and compare with the whole sequence
    o_all = torch.stack(o_shards).contiguous()
    lse_all = torch.stack(lse_shards).contiguous()
    om = torch.empty_like(o_shards[0])
    lm = torch.empty_like(lse_shards[0])
    mb.mla_merge_shards(o_all, lse_all, om, lm)
    torch.cuda.synchronize()
    ro, rl = gu.oracle_full(inp)
    gu.compare(om.double().cpu().numpy(), lm.double().cpu().numpy(), ro, rl, fp8,
               f"merged {len(bounds)} shards")


@pytest.mark.parametrize("fp8", [False, True])
def test_key_shards_of_a_large_batch(fp8):
    """70 sequences, each decoded over its own key shard [a_b, n_b) with its
    causal end (the plan's descriptors then live in the workspace tables):
    every row against the oracle's partial over the same keys."""
    import torch
    batch, H = 70, 8
    rng = np.random.default_rng(83)
    ql = rng.integers(1, 5, batch)
    kl = rng.integers(200, 900, batch)
    cut = np.array([rng.integers(0, n - 1) for n in kl])  # shard [cut, n): at least 2 keys
    gu.log(f"shards of a {batch}-sequence batch fp8={fp8}")
    inp = gen.peaked_inputs(gen.random_inputs(H, ql.tolist(), kl.tolist(), fp8, seed=84), beta=10.0,
                            seed=6)
    off = np.concatenate([[0], np.cumsum(kl)])
    kv_sh = np.concatenate([inp.kv[off[b] + cut[b]:off[b + 1]] for b in range(batch)])
    sh = gen.Inputs(H, inp.q_len.copy(), (kl - cut).astype(np.int32), inp.q_bits,
                    np.ascontiguousarray(kv_sh), fp8, inp.kv_scale)
    q_dev, kv_dev = gu.to_device(sh)
    plan = mb.Plan(H, ql.tolist(), (kl - cut).tolist(), fp8, causal_end=(kl - cut).tolist(),
                   force_splits=3)
    assert plan.num_launches == 1 and plan.num_split_tiles > 0
    o, lse, ws = mb.alloc_outputs(plan, q_dev.device)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ws.fill_(0xFF)
    mb.mla_decode_run(plan, q_dev, kv_dev, sh.sm_scale, sh.kv_scale, o, lse, ws, ws.numel())
    mb.mla_decode_reduce(plan, ws, o, lse)
    torch.cuda.synchronize()
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    rows = int(ql.sum())
    ro = np.empty((rows, H, mb.DV))
    rl = np.empty((rows, H))
    r = 0
    for b in range(batch):
        for i in range(int(ql[b])):
            for h in range(H):
                ro[r, h], rl[r, h] = oracle.mla_partial(
                    inp.q_bits, inp.kv, inp.q_len, inp.kv_len, H, b, i, h, int(cut[b]), int(kl[b]),
                    kv_is_fp8=fp8, kv_scale=inp.kv_scale, sm_scale=inp.sm_scale)
            r += 1
    empty = np.isneginf(rl)
    assert np.all(np.isneginf(gl[empty])) and np.all(go[empty] == 0.0)
    gu.compare(go[~empty], gl[~empty], ro[~empty], rl[~empty], fp8,
               f"{batch} shards, empty rows {int(empty.sum())}")


def test_merge_of_one_shard_is_the_identity_up_to_rounding():
    import torch
    rows = 37
    o = (torch.randn(1, rows, mb.DV, device="cuda") * 0.3).to(torch.bfloat16)
    lse = torch.randn(1, rows, device="cuda", dtype=torch.float32) * 3
    lse[0, 5] = float("-inf")
    om = torch.empty(rows, mb.DV, dtype=torch.bfloat16, device="cuda")
    lm = torch.empty(rows, dtype=torch.float32, device="cuda")
    mb.mla_merge_shards(o, lse, om, lm)
    torch.cuda.synchronize()
    keep = torch.ones(rows, dtype=torch.bool)
    keep[5] = False
    assert torch.equal(om[keep.cuda()], o[0][keep.cuda()])
    assert torch.allclose(lm[keep.cuda()], lse[0][keep.cuda()], atol=1e-6, rtol=0)
    assert torch.isneginf(lm[5]) and torch.all(om[5] == 0)
