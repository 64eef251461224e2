"""Pins of the stochastic-acceptance oracle (CPU): the target softmax against
torch's softmax and the two-logit logistic closed form; the rejection rule
keeps the target's distribution (the defining property the pages state), plus
special cases and the inverse CDF against brute force."""
import numpy as np
import pytest

from oracle import stochastic as S

GRID = 4000
MID = (np.arange(GRID) + 0.5) / GRID  # midpoints of [0, 1)


def _first_token_distribution(logits, dprobs, temperature=1.0):
    """P(first emitted token = v) for a one-draft chain, with x ~ q and u, w
    uniform, integrated on a grid of u and w (exact to ~1/GRID)."""
    V = logits.shape[1]
    q = dprobs[1]
    out = np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        draft = np.array([0, x])
        n_acc = 0
        for u in MID[::4]:  # 1000 values of u
            n, _, _ = S.accept_request(logits, dprobs, draft, np.array([0.0, u]), 0.5, 0, 2, temperature)
            n_acc += n
        pa = n_acc / len(MID[::4])
        out[x] += q[x] * pa
        # rejected: y from the residual, integrated over w
        _, _, r = S.accept_request(logits, dprobs, draft, np.array([0.0, 0.999999]), 0.5, 0, 2, temperature)
        ys = np.array([S.inverse_cdf(r, w) for w in MID])
        out += q[x] * (1 - pa) * np.bincount(ys, minlength=V) / GRID
    return out


@pytest.mark.parametrize("seed", range(4))
def test_lossless_first_token(seed):
    rng = np.random.default_rng(seed)
    V = 5
    logits = rng.standard_normal((2, V)) * 1.5
    dprobs = rng.dirichlet(np.ones(V), 2)
    temp = [1.0, 0.7, 1.3, 1.0][seed]
    got = _first_token_distribution(logits, dprobs, temp)
    want = S.target_probs(logits[0], temp)
    assert np.abs(got - want).max() < 3e-3, (got, want)


def test_target_probs_matches_torch_softmax():
    """Library special case: torch's softmax of logits / T in float64."""
    import torch
    rng = np.random.default_rng(11)
    for temp in (0.25, 0.7, 1.0, 1.9):
        for V in (1, 2, 7, 1000):
            x = rng.standard_normal(V) * 4.0
            want = torch.softmax(torch.from_numpy(x) / temp, dim=0).numpy()
            got = S.target_probs(x, temp)
            assert np.abs(got - want).max() <= 1e-14, (temp, V)


def test_target_probs_two_logit_closed_form():
    """Two logits a, b: p(a) = 1 / (1 + e^{-(a-b)/T}), the logistic function."""
    for a, b, temp in ((0.0, 0.0, 1.0), (1.0, 0.0, 1.0), (0.3, -1.2, 0.5), (-2.0, 3.0, 2.0), (5.0, 4.0, 0.1)):
        p = S.target_probs(np.array([a, b]), temp)
        want = 1.0 / (1.0 + np.exp(-(a - b) / temp))
        assert abs(p[0] - want) <= 1e-15 and abs(p[1] - (1.0 - want)) <= 1e-15, (a, b, temp)


def test_target_probs_neg_inf_logit_and_shift():
    """A -inf logit has probability 0 exactly; adding a constant to every logit
    changes nothing; the probabilities sum to 1."""
    x = np.array([0.5, -np.inf, 2.0, -1.0])
    p = S.target_probs(x, 1.0)
    assert p[1] == 0.0
    e = np.exp(np.array([0.5, 2.0, -1.0]))
    assert np.abs(p[[0, 2, 3]] - e / e.sum()).max() <= 1e-15
    assert abs(p.sum() - 1.0) <= 1e-15
    assert np.abs(S.target_probs(x + 100.0, 1.0) - p).max() <= 1e-15


def test_all_accepted_bonus_from_last_row():
    rng = np.random.default_rng(7)
    V = 6
    logits = rng.standard_normal((2, V))
    p1 = S.target_probs(logits[0], 1.0)
    dprobs = np.stack([np.full(V, 1 / V), p1])  # q == p: every draft is accepted
    counts = np.zeros(V)
    for w in MID:
        n, y, _ = S.accept_request(logits, dprobs, np.array([0, 2]), np.array([0.0, 0.9999]), w, 0, 2, 1.0)
        assert n == 1
        counts[y] += 1
    assert np.abs(counts / GRID - S.target_probs(logits[1], 1.0)).max() < 2e-3


def test_zero_target_probability_is_never_accepted():
    V = 4
    logits = np.array([[0.0, -np.inf, 1.0, 2.0], [0.0, 0.0, 0.0, 0.0]])
    dprobs = np.stack([np.full(V, 0.25), np.array([0.1, 0.7, 0.1, 0.1])])
    for u in (0.0, 0.3, 0.99):
        n, y, _ = S.accept_request(logits, dprobs, np.array([0, 1]), np.array([0.0, u]), 0.5, 0, 2, 1.0)
        assert n == 0 and y != 1


def test_temperature_scales_logits():
    rng = np.random.default_rng(3)
    V, T = 50, 5
    logits = rng.standard_normal((T, V))
    dprobs = rng.dirichlet(np.ones(V), T)
    draft = rng.integers(0, V, T)
    for _ in range(20):
        u, w = rng.random(T), rng.random(1)
        a = S.accept_stochastic(logits, dprobs, draft, u, w, [0, T], temperature=0.5)
        b = S.accept_stochastic(2.0 * logits, dprobs, draft, u, w, [0, T], temperature=1.0)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(4)
    for _ in range(200):
        wts = rng.random(int(rng.integers(1, 20))) * (rng.random() < 0.8)
        wts[rng.integers(0, len(wts))] += 0.1
        w = rng.random()
        total = wts.sum()
        acc, v = 0.0, None
        for k, x in enumerate(wts):
            acc += x
            if acc > w * total:
                v = k
                break
        assert S.inverse_cdf(wts, w) == v


def test_outputs_layout():
    rng = np.random.default_rng(5)
    V = 30
    cu = np.array([0, 4, 4, 9, 10])
    T = cu[-1]
    logits = rng.standard_normal((T, V))
    dprobs = rng.dirichlet(np.ones(V), T)
    draft = rng.integers(0, V, T)
    acc, path, toks = S.accept_stochastic(logits, dprobs, draft, rng.random(T), rng.random(4), cu)
    assert acc[1] == 0 and acc[3] == 1
    for i in range(4):
        o, q = cu[i], cu[i + 1] - cu[i]
        if q == 0:
            continue
        n = acc[i] - 1
        assert 0 <= n < q
        assert path[o:o + n + 1].tolist() == list(range(n + 1)) and np.all(path[o + n + 1:o + q] == -1)
        assert toks[o:o + n].tolist() == draft[o + 1:o + n + 1].tolist() and 0 <= toks[o + n] < V


MUTANTS = [
    ("accept_ignores_draft_prob", "if float(u[o + j]) * float(draft_probs[o + j][x]) < p[x]:",
     "if float(u[o + j]) < p[x]:"),
    ("residual_unclipped", "r = np.maximum(0.0, p - np.asarray(draft_probs[o + n + 1], np.float64))",
     "r = np.abs(p - np.asarray(draft_probs[o + n + 1], np.float64))"),
    ("target_row_shifted", "p = target_probs(logits[o + j - 1], temperature)",
     "p = target_probs(logits[o + j], temperature)"),
    ("residual_wrong_draft_row", "r = np.maximum(0.0, p - np.asarray(draft_probs[o + n + 1], np.float64))",
     "r = np.maximum(0.0, p - np.asarray(draft_probs[o + n], np.float64))"),
    ("softmax_exp2_without_log2e", "e = np.exp(x - x.max())", "e = np.exp2(x - x.max())"),
    ("softmax_missing_normaliser", "return e / e.sum()", "return e"),
    ("softmax_temperature_multiplies", "x = np.asarray(row_logits, np.float64) / float(temperature)",
     "x = np.asarray(row_logits, np.float64) * float(temperature)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, monkeypatch, name, old, new):
    import importlib.util
    src = open(S.__file__).read()
    assert src.count(old) == 1, name
    path = tmp_path / f"stochastic_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"stochastic_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(S, "accept_request", mod.accept_request)
    monkeypatch.setattr(S, "target_probs", mod.target_probs)
    failed = False
    for check in (test_target_probs_matches_torch_softmax, test_target_probs_two_logit_closed_form,
                  test_target_probs_neg_inf_logit_and_shift,
                  lambda: test_lossless_first_token(0), lambda: test_lossless_first_token(1),
                  test_all_accepted_bonus_from_last_row, test_zero_target_probability_is_never_accepted):
        try:
            check()
        except AssertionError:
            failed = True
            break
    assert failed, f"no pin caught {name}"
