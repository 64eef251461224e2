"""Pins of the stochastic-acceptance oracle (CPU): the target softmax against
torch's softmax and the two-logit logistic closed form; the rejection rule
keeps the target's distribution (the defining property the pages state), plus
special cases and the inverse CDF against brute force."""
import itertools

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


# ---------------------------------------------------------------------------
# Draft trees: multi-draft rejection sampling over the siblings of each node.
# The defining property is again that the emitted token keeps the target's
# distribution.  The pins integrate the oracle's decisions exactly: a test is
# a threshold in its uniform and a draw is monotone in w, so bisection on the
# oracle as a black box gives each branch's probability to ~1e-15.
def _bisect(pred, iters=64):
    """Measure of {t in [0, 1): pred(t)} for a predicate true on [0, a) only."""
    if not pred(0.0):
        return 0.0
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return lo


def _draw_law(y_of_w, V):
    """Law of y(w) for w uniform in [0, 1), y non-decreasing in w."""
    bounds = [0.0] + [_bisect(lambda w, v=v: y_of_w(w) < v) for v in range(1, V)] + [1.0]
    return np.diff(np.array(bounds))


def _token_law_at(node, logits, dprobs, parent, draft, u, temp):
    """Law of the token emitted right after `node` (an accepted child's draft
    or the draw at `node`), given that the walk reaches `node`, integrated over
    the children's drafts and uniforms and the draw's w."""
    V = logits.shape[1]
    q = len(parent)
    kids = [k for k in range(node + 1, q) if parent[k] == node]
    depth = 0
    a = node
    while a != 0:
        a = parent[a]
        depth += 1
    law = np.zeros(V)
    for xs in itertools.product(range(V), repeat=len(kids)):
        pr = float(np.prod([dprobs[k][x] for k, x in zip(kids, xs)]))
        if pr == 0.0:
            continue
        d = draft.copy()
        d[kids] = xs
        uu = u.copy()

        def run(w=0.5):
            return S.accept_request_tree(logits, dprobs, d, parent, uu, w, 0, q, temp)
        reach = pr
        for k, x in zip(kids, xs):
            def accepted(t, k=k):
                uu[k] = t
                pth = run()[0]
                return len(pth) > depth + 1 and pth[depth + 1] == k
            acc = _bisect(accepted)
            law[x] += reach * acc
            reach *= 1.0 - acc
            if reach == 0.0:
                break
            uu[k] = 0.5 * (acc + 1.0)  # inside the rejection region
        if reach > 0.0:
            law += reach * _draw_law(lambda w: run(w)[1], V)
    return law


def _tree_case(seed, V, parent):
    """Each draft row a perturbed copy of its parent's target row, so that the
    residuals left by rejections keep mass on several tokens."""
    rng = np.random.default_rng(seed)
    q = len(parent)
    logits = rng.standard_normal((q, V)) * 1.5
    dprobs = np.zeros((q, V))
    for k in range(1, q):
        dprobs[k] = S.target_probs(logits[parent[k]] + rng.standard_normal(V) * 0.8, 1.0)
    return logits, dprobs, np.zeros(q, np.int64), np.full(q, 0.5)


@pytest.mark.parametrize("seed,temp", [(0, 1.0), (1, 0.7), (2, 1.3)])
def test_tree_lossless_first_token(seed, temp):
    """Root with three children whose drafts come from three different q rows."""
    V = 4
    parent = np.array([-1, 0, 0, 0])
    logits, dprobs, draft, u = _tree_case(100 + seed, V, parent)
    got = _token_law_at(0, logits, dprobs, parent, draft, u, temp)
    want = S.target_probs(logits[0], temp)
    assert np.abs(got - want).max() < 1e-9, (got, want)


def test_tree_lossless_after_a_rejected_sibling():
    """parent = [-1, 0, 0, 2, 2]: node 1 rejected, node 2 accepted, then node
    2's children; the token after node 2 must follow node 2's own row (the
    residual left at the root does not carry over), for every draft of nodes 1
    and 2 that can reach node 2 this way."""
    V = 3
    parent = np.array([-1, 0, 0, 2, 2])
    logits, dprobs, draft, u = _tree_case(7, V, parent)
    dprobs[1] = [0.9, 0.05, 0.05]
    checked = 0
    for x1 in range(V):
        for x2 in range(V):
            draft[1], draft[2] = x1, x2
            uu = u.copy()
            uu[1] = 1.0 - 1e-12
            uu[2] = 0.0
            pth = S.accept_request_tree(logits, dprobs, draft, parent, uu, 0.5, 0, 5, 1.0)[0]
            if pth[:2] != [0, 2]:
                continue
            got = _token_law_at(2, logits, dprobs, parent, draft, uu, 1.0)
            assert np.abs(got - S.target_probs(logits[2], 1.0)).max() < 1e-9, (x1, x2, got)
            checked += 1
    assert checked >= 2


def test_tree_chain_equals_chain_rule():
    """A tree with one child per node is a chain: same path, same draw."""
    rng = np.random.default_rng(21)
    for _ in range(300):
        q = int(rng.integers(1, 8))
        V = int(rng.integers(2, 12))
        logits = rng.standard_normal((q, V)) * 2.0
        dprobs = rng.dirichlet(np.ones(V) * 0.5, q)
        draft = rng.integers(0, V, q)
        u, w = rng.random(q), rng.random()
        n, y, _ = S.accept_request(logits, dprobs, draft, u, w, 0, q, 0.9)
        pth, yt, _, _ = S.accept_request_tree(logits, dprobs, draft, np.arange(-1, q - 1), u, w, 0, q, 0.9)
        assert pth == list(range(n + 1)) and yt == y


def test_tree_siblings_in_index_order():
    """Two children that would both be accepted: the lower index wins."""
    V = 4
    parent = np.array([-1, 0, 0])
    logits = np.zeros((3, V))
    dprobs = np.full((3, V), 0.25)  # q == p: every test with u < 1 accepts
    draft = np.array([0, 2, 1])
    pth = S.accept_request_tree(logits, dprobs, draft, parent, np.array([0.0, 0.3, 0.3]), 0.5, 0, 3, 1.0)[0]
    assert pth == [0, 1]


def test_tree_outputs_layout():
    rng = np.random.default_rng(8)
    V = 20
    parent = np.array([-1, 0, 0, 1, 1, 3, -1, -1, 0, 1])  # requests of 6, 1 and 3 tokens
    cu = np.array([0, 6, 7, 7, 10])
    T = 10
    logits = rng.standard_normal((T, V))
    dprobs = np.tile(S.target_probs(np.zeros(V), 1.0), (T, 1))
    draft = rng.integers(0, V, T)
    for _ in range(20):
        acc, path, toks = S.accept_stochastic_tree(logits, dprobs, draft, parent, rng.random(T), rng.random(4), cu)
        assert acc[1] == 1 and acc[2] == 0 and path[6] == 0
        for i in (0, 1, 3):
            o, q = cu[i], cu[i + 1] - cu[i]
            n = acc[i] - 1
            pth = path[o:o + n + 1]
            assert pth[0] == 0 and all(parent[o + pth[t + 1]] == pth[t] for t in range(n))
            assert np.all(path[o + n + 1:o + q] == -1) and np.all(toks[o + n + 1:o + q] == -1)
            assert toks[o:o + n].tolist() == [draft[o + k] for k in pth[1:]] and 0 <= toks[o + n] < V


TREE_MUTANTS = [
    ("tree_test_against_target_not_residual", "if lhs < cur[x]:", "if lhs < p[x]:"),
    ("tree_residual_unnormalised", "cur = r / r.sum()", "cur = r"),
    ("tree_residual_from_target", "r = np.maximum(0.0, cur - qk)", "r = np.maximum(0.0, p - qk)"),
    ("tree_draw_ignores_residual", "weights = p if last is None else last", "weights = p"),
    ("tree_row_by_depth", "p = target_probs(logits[o + c], temperature)",
     "p = target_probs(logits[o + len(path) - 1], temperature)"),
    ("tree_first_sibling_draft_row", "qk = np.asarray(draft_probs[o + k], np.float64)",
     "qk = np.asarray(draft_probs[o + c + 1], np.float64)"),
    ("tree_siblings_reversed", "for k in range(c + 1, q):", "for k in reversed(range(c + 1, q)):"),
    ("tree_residual_kept_after_move", "cur, last, moved = p, None, False",
     "cur, last, moved = (p if c == 0 else cur), (None if c == 0 else last), False"),
]


@pytest.mark.parametrize("name,old,new", TREE_MUTANTS, ids=[m[0] for m in TREE_MUTANTS])
def test_tree_pins_catch_planted_mistake(tmp_path, monkeypatch, name, old, new):
    import importlib.util
    src = open(S.__file__).read()
    assert src.count(old) == 1, name
    path = tmp_path / f"stochastic_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"stochastic_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(S, "accept_request_tree", mod.accept_request_tree)
    failed = False
    for check in (lambda: test_tree_lossless_first_token(0, 1.0), test_tree_lossless_after_a_rejected_sibling,
                  test_tree_chain_equals_chain_rule, test_tree_siblings_in_index_order):
        try:
            check()
        except AssertionError:
            failed = True
            break
    assert failed, f"no pin caught {name}"
