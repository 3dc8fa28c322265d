"""GPU: the split-KV workspace itself, checked against the oracle.

After mla_decode_run (and before the merge) the workspace holds, for every
split tile row and chunk, the normalised partial O (bf16) and the partial LSE
(fp32) of that chunk's keys.  Each (chunk, row) record is compared with the
oracle's partial over the same keys (oracle.mla_partial), so a wrong chunk
bound, a wrong row of a folded tile or a misplaced record fails here even if
the merge happened to hide it.  The record layout (partial LSE [P] fp32, then
at the next 256-byte boundary partial O [P, 512] bf16; record of sequence b,
tile t, chunk s, tile row r at part_row0(b) + (t S + s) R + r, sequences in
the plan's run order -- the caller's order under forced splits -- unsplit
ones taking no records) is recomputed here from the plan's per-sequence
facts.  The plans merge with the reduce kernel, so the workspace holds the
partial records and nothing else."""
import numpy as np
import pytest

import oracle
from mla_token_decode_amd import binding as mb
from mla_token_decode_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _layout(plan, H):
    recs, row0 = [], 0
    for b in range(len(plan.q_len)):
        F, T, S, L = plan.query(b)
        if S > 1:
            recs.append((b, F, T, S, L, row0))
            row0 += T * S * H * F
        else:
            recs.append(None)
    return recs, row0


@pytest.mark.parametrize("case", [
    (12, [8], [1500], False, 5),
    (12, [8], [1500], True, 5),
    (96, [2, 3], [700, 300], False, 3),
    (24, [1, 4, 2], [400, 90, 1000], True, 4),
])
@pytest.mark.parametrize("peaked", [False, True])
def test_split_workspace_matches_oracle_partials(case, peaked):
    import torch
    H, q_len, kv_len, fp8, splits = case
    gu.log(f"partials H={H} q={q_len} n={kv_len} fp8={fp8} splits={splits} peaked={peaked}")
    inp = gen.random_inputs(H, q_len, kv_len, fp8, seed=61)
    if peaked:
        inp = gen.peaked_inputs(inp, beta=10.0, seed=4)
    plan = mb.Plan(H, inp.q_len, inp.kv_len, fp8, force_splits=splits,
                   merge_mode=mb.MLA_MERGE_REDUCE)
    recs, P = _layout(plan, H)
    assert P > 0
    q, kv = gu.to_device(inp)
    o, lse, ws = mb.alloc_outputs(plan, q.device)
    ws.fill_(0xFF)  # NaN everywhere the kernel does not write
    mb.mla_decode_run(plan, q, kv, inp.sm_scale, inp.kv_scale, o, lse, ws, ws.numel())
    torch.cuda.synchronize()
    off = (P * 4 + 255) // 256 * 256
    assert plan.workspace_bytes == off + P * 512 * 2
    raw = ws.cpu().numpy()
    plse = raw[:P * 4].view(np.float32).astype(np.float64)
    po = gen.f32_from_bf16_bits(raw[off:off + P * 1024].view(np.uint16)).reshape(P, 512).astype(np.float64)
    worst_o = worst_l = 0.0
    q_off = np.concatenate([[0], np.cumsum(inp.q_len)])
    for rec in recs:
        if rec is None:
            continue
        b, F, T, S, L, row0 = rec
        R = H * F
        n = int(inp.kv_len[b])
        for t in range(T):
            for s in range(S):
                for r in range(R):
                    i, h = t * F + r // H, r % H
                    pr = row0 + (t * S + s) * R + r
                    ro, rl = oracle.mla_partial(inp.q_bits, inp.kv, inp.q_len, inp.kv_len, H, b, i, h,
                                                s * L, min((s + 1) * L, n), kv_is_fp8=fp8,
                                                kv_scale=inp.kv_scale, sm_scale=inp.sm_scale)
                    if np.isneginf(rl):  # the chunk shows this row no key
                        assert np.isneginf(plse[pr]), (b, t, s, r, plse[pr])
                        assert np.all(po[pr] == 0.0), (b, t, s, r)
                        continue
                    assert np.isfinite(plse[pr]) and np.all(np.isfinite(po[pr])), (b, t, s, r)
                    worst_l = max(worst_l, abs(plse[pr] - rl))
                    worst_o = max(worst_o, float(np.abs(po[pr] - ro).max()))
    gu.log(f"  max|dO_s|={worst_o:.3e} max|dLSE_s|={worst_l:.3e} over {P} records")
    assert worst_l <= gu.TOL_LSE
    assert worst_o <= gu.TOL_O[fp8]
    del q_off
