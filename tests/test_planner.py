"""Host-only checks of the planner's rules (no GPU): per-sequence chunking
under MLA_PLAN_AUTO, the longest-first unit order, filling the last wave of
CUs, and MLA_PLAN_UNIFORM as the single-chunk-length control.  The rules
follow "bench(cake_mla_varq_dcp_decode): ..." (flashinfer PR #5588), table
"What was measured", row "host plan": the plan is chosen from host-known
scalars only."""
import pytest

from mla_token_decode_amd import binding as mb

CUS = 256


def plan(H, q_len, kv_len, fp8=False, **kw):
    kw.setdefault("num_cus", CUS)
    return mb.Plan(H, q_len, kv_len, fp8, **kw)


def facts(p):
    return [p.query(b) for b in range(len(p.q_len))]


def test_order_is_a_permutation_and_uniform_mode_keeps_the_callers_order():
    ql, kl = [1, 8, 3, 2, 8], [5000, 300000, 70000, 64, 1200]
    a = plan(12, ql, kl)
    assert sorted(a.order()) == list(range(5))
    u = plan(12, ql, kl, plan_mode=mb.MLA_PLAN_UNIFORM)
    assert u.order() == list(range(5))
    f = plan(12, ql, kl, force_splits=3)
    assert f.order() == list(range(5))


def test_uniform_mode_uses_one_chunk_length():
    # one target length L* for all; each sequence then balances its
    # ceil(n / L*) chunks by the split rule
    ql, kl = [8, 8, 8], [1048576, 300000, 200000]
    u = plan(12, ql, kl, plan_mode=mb.MLA_PLAN_UNIFORM)
    fs = facts(u)
    Lstar = max(L for F, T, S, L in fs)
    assert all(S == -(-n // Lstar) for (F, T, S, L), n in zip(fs, kl))


def test_longest_units_run_first():
    # equal rows per unit: a unit's time grows with its keys, so along the
    # run order keys per unit do not increase (up to the partial-row write a
    # split unit adds, worth less than one granule of keys here)
    ql = [1] * 40
    kl = [64 * (1 + (7 * b) % 40) for b in range(40)]
    p = plan(12, ql, kl)
    keys = []
    for b in p.order():
        F, T, S, L = p.query(b)
        keys.append(min(L, kl[b]))
    assert all(keys[i] + 64 >= keys[i + 1] for i in range(len(keys) - 1)), keys


def test_single_long_sequence_fills_the_machine():
    for fp8 in (False, True):
        p = plan(12, [8], [1048576], fp8)
        F, T, S, L = p.query(0)
        assert (F, T) == (8, 1) and L % 64 == 0
        assert p.num_units >= CUS and p.num_units % CUS <= CUS // 8 or p.num_units % CUS == 0


def test_tail_wave_is_filled_by_splitting():
    # 300 unsplit sequences would be 300 units: one full wave and a tail of
    # 44 units; splitting them fills whole waves instead
    p = plan(12, [1] * 300, [4096] * 300)
    assert p.num_units > 300
    tail = p.num_units % CUS
    assert tail == 0 or tail > CUS // 2, p.num_units


def test_short_sequences_stay_whole_next_to_a_long_one():
    p = plan(12, [8, 8, 8], [1048576, 512, 640])
    assert p.query(0)[2] > 1
    assert p.query(1)[2] == 1 and p.query(2)[2] == 1
    assert p.order()[0] == 0 or p.query(0)[3] <= 640


def test_plans_are_deterministic():
    ql, kl = [1, 4, 2, 3] * 8, [32768] * 32
    a, b = plan(96, ql, kl), plan(96, ql, kl)
    assert facts(a) == facts(b) and a.order() == b.order()
    assert a.num_units == b.num_units and a.workspace_bytes == b.workspace_bytes


def test_unknown_plan_mode_is_rejected():
    with pytest.raises(mb.MlaError) as e:
        plan(12, [1], [100], plan_mode=7)
    assert e.value.status == mb.MLA_ERR_INVALID_ARGUMENT


def test_every_mode_covers_each_sequence_with_whole_granules():
    ql = [1, 2, 3, 4, 8, 16, 5]
    kl = [64, 65, 4095, 131072, 777, 5000, 30000]
    for mode in (mb.MLA_PLAN_AUTO, mb.MLA_PLAN_UNIFORM):
        p = plan(24, ql, kl, plan_mode=mode)
        for b in range(len(ql)):
            F, T, S, L = p.query(b)
            assert L % 64 == 0 and S * L >= kl[b] and (S - 1) * L < kl[b]
