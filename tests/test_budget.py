"""Verify-budget scheduling (DSpark, "Hardware-aware prefix scheduler"): the
oracle against brute force and closed forms, then the library's host function
against the oracle.  Host code only: runs on the CPU."""
import itertools

import numpy as np
import pytest

from oracle import budget
from speculative_decoding_verification_attn_amd import ops


def _theta(cond, sel, sps_rows, sps_value):
    """Theta of verifying the prefixes sel[i] (independent of the greedy order)."""
    n = len(cond)
    tau = float(n)
    for i, k in enumerate(sel):
        s = 1.0
        for m in range(k):
            s *= float(cond[i][m])
            tau += s
    return tau * budget.sps_at(sps_rows, sps_value, n + sum(sel))


def _random_instance(rng, n_req, gmax):
    gam = [int(rng.integers(0, gmax + 1)) for _ in range(n_req)]
    cond = [rng.uniform(0.0, 1.0, g).round(3).astype(np.float32) for g in gam]
    npt = int(rng.integers(1, 5))
    rows = np.sort(rng.choice(np.arange(1, 3 * (n_req * (gmax + 1)) + 6), npt, replace=False)).astype(np.float32)
    val = rng.uniform(1.0, 100.0, npt).astype(np.float32)
    return cond, gam, rows, val


def test_oracle_matches_brute_force_over_prefix_batches():
    """Every prefix-closed batch of tiny instances: the oracle's Theta is the largest
    and its batch is the smallest that reaches it."""
    rng = np.random.default_rng(5)
    for _ in range(400):
        cond, gam, rows, val = _random_instance(rng, int(rng.integers(1, 4)), 3)
        verify, brows, th = budget.verify_budget(cond, gam, rows, val)
        best = max(_theta(cond, sel, rows, val) for sel in itertools.product(*[range(g + 1) for g in gam]))
        assert th == pytest.approx(best, rel=1e-12, abs=1e-12)
        assert _theta(cond, verify, rows, val) == pytest.approx(th, rel=1e-12, abs=1e-12)
        smallest = min(len(gam) + sum(sel) for sel in itertools.product(*[range(g + 1) for g in gam])
                       if _theta(cond, sel, rows, val) >= best * (1 - 1e-12))
        assert brows == smallest == len(gam) + sum(verify)


def test_sps_interpolation_hand_values():
    """Linear interpolation between unequal table values, worked by hand, and
    clamping at both ends of the table."""
    rows, val = [2.0, 6.0, 10.0], [10.0, 30.0, 20.0]
    cases = {1.0: 10.0, 2.0: 10.0, 3.0: 15.0, 5.0: 25.0, 6.0: 30.0, 7.0: 27.5, 8.0: 25.0, 9.5: 21.25,
             10.0: 20.0, 64.0: 20.0}
    for b, want in cases.items():
        assert budget.sps_at(rows, val, b) == pytest.approx(want, rel=0, abs=1e-12), b
    # one point: constant
    assert budget.sps_at([4.0], [7.0], 1.0) == 7.0 and budget.sps_at([4.0], [7.0], 9.0) == 7.0


def test_sps_interpolation_matches_numpy_interp():
    """Library special case: numpy.interp is piecewise-linear interpolation with
    the end values held outside the table."""
    rng = np.random.default_rng(9)
    for _ in range(300):
        n = int(rng.integers(1, 7))
        rows = np.sort(rng.choice(np.arange(1, 200), n, replace=False)).astype(np.float64)
        val = rng.uniform(0.0, 100.0, n)
        for b in rng.uniform(0.0, 210.0, 8):
            assert budget.sps_at(rows, val, b) == pytest.approx(float(np.interp(b, rows, val)), rel=1e-12,
                                                              abs=1e-12)


def _budget_pins_fail():
    try:
        test_sps_interpolation_hand_values()
        test_sps_interpolation_matches_numpy_interp()
        test_oracle_closed_forms()
        test_oracle_matches_brute_force_over_prefix_batches()
    except AssertionError:
        return True
    return False


BUDGET_MUTANTS = [
    ("wrong_interval", "t = (b - rows[j - 1]) / (float(rows[j]) - float(rows[j - 1]))",
     "t = (b - rows[j - 1]) / (float(rows[j]) - float(rows[0]))"),
    ("swapped_weight", "return float(value[j - 1]) + t * (float(value[j]) - float(value[j - 1]))",
     "return float(value[j]) + t * (float(value[j - 1]) - float(value[j]))"),
    ("first_interval_only", "while rows[j] < b:", "while j < 1:"),
    ("no_low_clamp", "if b <= rows[0]:\n        return float(value[0])", "if b < 0:\n        return float(value[0])"),
    ("tau_without_bonus", "tau = float(n)\n    best", "tau = 0.0\n    best"),
]


@pytest.mark.parametrize("name,old,new", BUDGET_MUTANTS, ids=[m[0] for m in BUDGET_MUTANTS])
def test_budget_pins_catch_planted_mistake(tmp_path, monkeypatch, name, old, new):
    import importlib.util
    src = open(budget.__file__).read()
    assert src.count(old) == 1, name
    path = tmp_path / f"budget_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"budget_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(budget, "sps_at", mod.sps_at)
    monkeypatch.setattr(budget, "verify_budget", mod.verify_budget)
    assert _budget_pins_fail(), f"no pin caught {name}"


def test_oracle_closed_forms():
    # constant SPS: every draft with survival > 0 raises tau -> all of them
    cond = [np.array([0.5, 0.5, 0.0, 0.9], np.float32), np.array([1.0, 0.2], np.float32)]
    verify, brows, th = budget.verify_budget(cond, [4, 2], [1.0], [10.0])
    assert verify == [2, 2] and brows == 6
    assert th == pytest.approx(10.0 * (2 + 0.5 + 0.25 + 1.0 + 0.2))
    # SPS collapses beyond the root rows: verify nothing
    verify, brows, th = budget.verify_budget(cond, [4, 2], [2.0, 3.0], [10.0, 0.0])
    assert verify == [0, 0] and brows == 2 and th == pytest.approx(20.0)
    # a certain draft (c = 1) is admitted before any uncertain one
    verify, _, _ = budget.verify_budget([np.array([1.0, 1.0], np.float32), np.array([0.99], np.float32)],
                                        [2, 1], [2.0, 4.0, 5.0], [10.0, 10.0, 7.0])
    assert verify == [2, 0]


@pytest.mark.parametrize("seed", range(4))
def test_library_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(150):
        cond, gam, rows, val = _random_instance(rng, int(rng.integers(0, 40)), 8)
        cu = np.zeros(len(gam) + 1, np.int32)
        cu[1:] = np.cumsum(gam)
        flat = np.concatenate(cond).astype(np.float32) if cu[-1] else np.zeros(0, np.float32)
        verify, brows, th = ops.spec_verify_budget(flat, cu, rows, val)
        ov, ob, oth = budget.verify_budget(cond, gam, rows, val)
        assert th == pytest.approx(oth, rel=1e-12, abs=1e-9)
        assert verify.tolist() == ov and brows == ob


def test_library_rejects_bad_arguments():
    cu = np.array([0, 2], np.int32)
    rows, val = np.array([1.0, 4.0], np.float32), np.array([5.0, 4.0], np.float32)
    for bad_c in (np.array([0.5, 1.5], np.float32), np.array([0.5, np.nan], np.float32)):
        with pytest.raises(ops.SpecVerifyError) as e:
            ops.spec_verify_budget(bad_c, cu, rows, val)
        assert e.value.status == ops.SV_ERR_SHAPE
    with pytest.raises(ops.SpecVerifyError):
        ops.spec_verify_budget(np.array([0.5, 0.5], np.float32), cu, np.array([4.0, 1.0], np.float32), val)
    with pytest.raises(ops.SpecVerifyError):
        ops.spec_verify_budget(np.zeros(64, np.float32), np.array([0, 64], np.int32), rows, val)
    verify, brows, th = ops.spec_verify_budget(np.zeros(0, np.float32), np.array([0], np.int32), rows, val)
    assert len(verify) == 0 and brows == 0 and th == 0.0


def _measured_sps():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                        "sps_table_llama3_70b.json")
    t = json.load(open(path))
    rows, sps = np.asarray(t["rows"], np.float32), np.asarray(t["steps_per_s"], np.float32)
    assert len(rows) >= 3 and np.all(np.diff(rows) > 0) and np.all(sps > 0)
    return rows, sps


@pytest.mark.parametrize("shape", ["b256_p075_gamma3", "ragged_beta22", "b16_mixed"])
def test_library_matches_oracle_on_measured_sps_table(shape):
    """The verify path's measured SPS(B) table (verify rows -> verify steps per
    second, 70B-shape sweep in profiles/) as the scheduler's cost table, with
    survival probabilities shaped like the workloads' acceptance: the library
    and the oracle choose the same verify lengths, and the chosen Theta is at
    least that of verifying no draft and of verifying every draft."""
    rows, sps = _measured_sps()
    rng = np.random.default_rng({"b256_p075_gamma3": 1, "ragged_beta22": 2, "b16_mixed": 3}[shape])
    if shape == "b256_p075_gamma3":
        gam = [3] * 256
        cond = [np.full(3, 0.75, np.float32) for _ in gam]
    elif shape == "ragged_beta22":
        gam = [int(g) for g in rng.integers(1, 9, 64)]
        cond = [np.full(g, rng.beta(2, 2), np.float32) for g in gam]
    else:
        gam = [int(g) for g in rng.integers(0, 9, 16)]
        cond = [rng.uniform(0.2, 1.0, g).astype(np.float32) for g in gam]
    cu = np.zeros(len(gam) + 1, np.int32)
    cu[1:] = np.cumsum(gam)
    flat = np.concatenate(cond).astype(np.float32)
    verify, brows, th = ops.spec_verify_budget(flat, cu, rows, sps)
    ov, ob, oth = budget.verify_budget(cond, gam, rows, sps)
    assert verify.tolist() == ov and brows == ob
    assert th == pytest.approx(oth, rel=1e-9)
    assert th >= _theta(cond, [0] * len(gam), rows, sps) * (1 - 1e-12)
    assert th >= _theta(cond, gam, rows, sps) * (1 - 1e-12)
    assert brows == len(gam) + int(verify.sum())
