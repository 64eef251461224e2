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
