"""bench.py's host-side helpers, on the CPU: the measurement-validity checks
(the shader clock read around each timed workload against the loaded-clock
gate, and the headline measured twice against the repeat gate)."""
import bench


def _clk(before, after):
    return {"clocks_before": {"sclk_mhz": before}, "clocks_after": {"sclk_mhz": after}}


def test_clock_gate_takes_the_lowest_reading_of_any_workload():
    per = {"h": _clk(2400, 2392), "small": _clk(2396, 1600), "ratio": 1.3}
    v = bench.validity_checks(per, 136.0, 136.5)
    assert v["sclk_min_frac"] == round(1600 / 2400, 4)
    assert v["clock_gate_passed"] is False and v["clock_gate_failed"] == ["small"]
    v = bench.validity_checks({"h": _clk(2400, 1700)}, 136.0, None)
    assert v["clock_gate_passed"] is True and v["clock_gate_failed"] == []  # 1700 / 2400 >= 0.70


def test_repeat_gate():
    per = {"h": _clk(2400, 2400)}
    v = bench.validity_checks(per, 100.0, 101.9)
    assert v["repeat_disagreement"] == 0.019 and v["repeat_gate_passed"] is True
    v = bench.validity_checks(per, 100.0, 97.5)
    assert v["repeat_disagreement"] == 0.025 and v["repeat_gate_passed"] is False
    v = bench.validity_checks(per, 100.0, None)  # --quick: no repeat
    assert v["repeat_gate_passed"] is None and v["headline_repeat_us"] is None


def test_missing_clock_readings_leave_the_gate_undecided():
    v = bench.validity_checks({"h": {"clocks_before": {"error": "rocm-smi"}, "clocks_after": None}},
                              100.0, 100.0)
    assert v["sclk_min_frac"] is None and v["clock_gate_passed"] is None
