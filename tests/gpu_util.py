"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
from mla_token_decode_amd import binding as mb
from mla_token_decode_amd import inputs as gen

# Tolerances of the decode problem statement: max |O - O_ref| <= 1e-2 and
# max |LSE - LSE_ref| <= 1e-3 for bf16 KV; max |O - O_ref| <= 3e-2 for fp8 KV.
# fp8 LSE: the library decodes e4m3 exactly to bf16 before any arithmetic, so
# its LSE carries the same error sources as the bf16 path: 1e-3 is used.
TOL_O = {False: 1e-2, True: 3e-2}
TOL_LSE = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(inp.q_bits).view(np.int16)).view(torch.bfloat16).cuda()
    if inp.kv_fp8:
        kv = torch.from_numpy(np.ascontiguousarray(inp.kv)).cuda()
    else:
        kv = torch.from_numpy(np.ascontiguousarray(inp.kv).view(np.int16)).view(torch.bfloat16).cuda()
    return q, kv


def run_gpu(inp, dev=None, *, poison_workspace=False, **plan_opts):
    """Returns (O float64 [sum q, H, 512], LSE float64 [sum q, H], plan)."""
    import torch
    plan_opts.setdefault("num_cus", 0)
    plan = mb.Plan(inp.H, inp.q_len, inp.kv_len, inp.kv_fp8, **plan_opts)
    q, kv = dev if dev is not None else to_device(inp)
    o, lse, ws = mb.alloc_outputs(plan, q.device)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    if poison_workspace:
        ws.fill_(0xFF)  # every partial reads as NaN unless the kernel wrote it
    mb.mla_decode_run(plan, q, kv, inp.sm_scale, inp.kv_scale, o, lse, ws, ws.numel())
    mb.mla_decode_reduce(plan, ws, o, lse)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), plan


def oracle_full(inp):
    return oracle.mla_decode(inp.q_bits, inp.kv, inp.q_len, inp.kv_len, inp.H,
                             kv_is_fp8=inp.kv_fp8, kv_scale=inp.kv_scale, sm_scale=inp.sm_scale)


def oracle_rows(inp, rows):
    return oracle.mla_decode_rows(inp.q_bits, inp.kv, inp.q_len, inp.kv_len, inp.H, rows,
                                  kv_is_fp8=inp.kv_fp8, kv_scale=inp.kv_scale,
                                  sm_scale=inp.sm_scale)


def compare(o, lse, ro, rl, fp8, what=""):
    """Assert the graded tolerances; return (max|dO|, max|dLSE|, max|O_ref|)."""
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite LSE"
    do = float(np.max(np.abs(o - ro)))
    dl = float(np.max(np.abs(lse - rl)))
    mo = float(np.max(np.abs(ro)))
    rel = do / mo if mo > 0 else float("inf")
    log(f"  {what}: max|dO|={do:.3e} (max|O_ref|={mo:.3e}, ratio {rel:.3e}) max|dLSE|={dl:.3e}")
    assert do <= TOL_O[fp8], f"{what}: max|dO| {do} > {TOL_O[fp8]}"
    assert dl <= TOL_LSE, f"{what}: max|dLSE| {dl} > {TOL_LSE}"
    return do, dl, mo


def sample_rows(inp, count, seed=0):
    """Row indices (token * H + head): for every token of every sequence the
    first, a middle and the last head (so every sequence, every folded tile
    and every tile of a wide-head workload is compared), then seeded random
    rows until `count` rows are chosen (never fewer than the per-token rows)."""
    H = inp.H
    total = int(np.sum(inp.q_len)) * H
    rows = set()
    for tok in range(int(np.sum(inp.q_len))):
        rows.update([tok * H, tok * H + H // 2, tok * H + H - 1])
    rng = np.random.default_rng([seed, 11])
    count = min(max(count, len(rows)), total)
    while len(rows) < count:
        rows.add(int(rng.integers(0, total)))
    return np.array(sorted(rows), dtype=np.int64)


@functools.lru_cache(maxsize=2)
def workload_inputs(name):
    return gen.gen_workload_inputs(gen.workload(name))
