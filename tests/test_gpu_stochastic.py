"""Lossless stochastic acceptance (speculative sampling) on the GPU, through
the C ABI, against the fp64 oracle on the same inputs and random numbers.

The GPU works in fp32, so a decision whose margin lies within fp32 rounding
may legitimately differ from the fp64 oracle: an acceptance test counts as
decided only when |u*q - p| exceeds 1e-4 of p, and a draw is checked to lie
at the oracle's inverse-CDF point within 1e-4 of the total weight.  Outside
those margins the results must be identical."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, i32, note
from oracle import stochastic as S
from speculative_decoding_verification_attn_amd import ops

pytestmark = pytest.mark.gpu


def _case(seed, B, V, qmax, temperature, sigma=2.0, noise=0.3):
    rng = np.random.default_rng(seed)
    q = rng.integers(1, qmax + 1, B)
    q[0] = 1  # a request with no draft
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(q)
    T = int(cu[-1])
    logits = (rng.standard_normal((T, V)) * sigma).astype(np.float32)
    dprobs = np.zeros((T, V), np.float32)
    draft = np.zeros(T, np.int32)
    for i in range(B):
        o = cu[i]
        for j in range(1, q[i]):
            # the drafter: a perturbed copy of the target's distribution at position j
            d = S.target_probs(logits[o + j - 1].astype(np.float64) + rng.standard_normal(V) * noise, temperature)
            dprobs[o + j] = d.astype(np.float32)
            dprobs[o + j] /= dprobs[o + j].sum(dtype=np.float64)
            draft[o + j] = rng.choice(V, p=dprobs[o + j].astype(np.float64) / dprobs[o + j].sum(dtype=np.float64))
    u = rng.random(T).astype(np.float32)
    w = rng.random(B).astype(np.float32)
    return cu, logits, dprobs, draft, u, w


def _compare(cu, logits, dprobs, draft, u, w, temperature, acc, path, toks):
    B = len(cu) - 1
    exact = borderline = 0
    for i in range(B):
        o, q = int(cu[i]), int(cu[i + 1] - cu[i])
        # oracle walk with margins
        n_ref, undecided = 0, False
        for j in range(1, q):
            p = S.target_probs(logits[o + j - 1], temperature)
            x = int(draft[o + j])
            lhs = float(u[o + j]) * float(dprobs[o + j][x])
            if abs(lhs - p[x]) <= 1e-4 * max(p[x], 1e-30):
                undecided = True
                break
            if lhs < p[x]:
                n_ref += 1
            else:
                break
        n = int(acc[i]) - 1
        assert 0 <= n < q, (i, n)
        assert path[o:o + n + 1].tolist() == list(range(n + 1)) and np.all(path[o + n + 1:o + q] == -1)
        assert toks[o:o + n].tolist() == draft[o + 1:o + n + 1].tolist() and np.all(toks[o + n + 1:o + q] == -1)
        if undecided and n != n_ref:
            borderline += 1
            continue
        assert n == n_ref, (i, n, n_ref)
        # the draw: at the oracle's inverse-CDF point, within 1e-4 of the total weight
        p = S.target_probs(logits[o + n], temperature)
        r = np.maximum(0.0, p - dprobs[o + n + 1].astype(np.float64)) if n < q - 1 else p
        if r.sum() <= 0.0:
            r = p
        c = np.cumsum(r)
        tgt = float(w[i]) * c[-1]
        y = int(toks[o + n])
        tol = 1e-4 * c[-1]
        assert 0 <= y < len(r) and r[y] > 0.0, (i, y)
        assert (c[y - 1] if y > 0 else 0.0) <= tgt + tol and c[y] >= tgt - tol, (i, y, tgt)
        exact += int(y == S.inverse_cdf(r, w[i]))
    return exact, borderline


@pytest.mark.parametrize("seed,B,V,qmax,temp", [(0, 16, 1000, 8, 1.0), (1, 32, 4099, 6, 0.7),
                                                (2, 8, 128256, 5, 1.0), (3, 4, 151936, 8, 1.3)])
def test_stochastic_acceptance_matches_oracle(seed, B, V, qmax, temp):
    cu, logits, dprobs, draft, u, w = _case(seed, B, V, qmax, temp)
    T = int(cu[-1])
    note(f"[gpu] spec_accept_stochastic seed={seed} B={B} T={T} V={V} T={temp}")
    ws = torch.empty(ops.spec_accept_stochastic_workspace_size(B, T, V), dtype=torch.uint8, device=DEV)
    acc, path, toks = ops.spec_accept_stochastic(torch.from_numpy(logits).to(DEV), torch.from_numpy(dprobs).to(DEV),
                                                 i32(draft), torch.from_numpy(u).to(DEV), torch.from_numpy(w).to(DEV),
                                                 i32(cu), temperature=temp, workspace=ws)
    torch.cuda.synchronize()
    assert ops.spec_accept_stochastic_device_status(ws) == 0
    exact, borderline = _compare(cu, logits, dprobs, draft, u, w, temp, acc.cpu().numpy(), path.cpu().numpy(),
                                 toks.cpu().numpy())
    note(f"  draws equal to the oracle's: {exact}/{B}, borderline acceptances: {borderline}")
    assert borderline <= 1 and exact >= B - 2


def test_stochastic_bad_token_sets_status():
    cu, logits, dprobs, draft, u, w = _case(5, 4, 300, 4, 1.0)
    draft[int(cu[1]) + 1] = 300 if cu[2] - cu[1] > 1 else draft[int(cu[1]) + 1]
    draft[1] = -3 if cu[1] > 1 else draft[1]
    draft[int(cu[3]) + 1] = 1000 if cu[4] - cu[3] > 1 else draft[int(cu[3]) + 1]
    ws = torch.empty(ops.spec_accept_stochastic_workspace_size(4, int(cu[-1]), 300), dtype=torch.uint8, device=DEV)
    ops.spec_accept_stochastic(torch.from_numpy(logits).to(DEV), torch.from_numpy(dprobs).to(DEV), i32(draft),
                               torch.from_numpy(u).to(DEV), torch.from_numpy(w).to(DEV), i32(cu), workspace=ws)
    torch.cuda.synchronize()
    if (cu[2] - cu[1] > 1) or (cu[4] - cu[3] > 1):
        assert ops.spec_accept_stochastic_device_status(ws) & ops.DEV_BAD_TOKEN


# ---------------------------------------------------------------------------
# Draft trees (multi-draft rejection sampling)
def _tree_parents(rng, q, shape):
    if shape == "wide":
        return [-1] + [0] * (q - 1)
    if shape == "chain":
        return list(range(-1, q - 1))
    if shape == "bushy":  # a few children per node, breadth first
        return [-1] + [(k - 1) // 3 for k in range(1, q)]
    return [-1] + [int(rng.integers(0, k)) for k in range(1, q)]


def _stoch_tree_case(seed, B, V, qmax, temperature, shape, sigma=2.0, noise=0.5):
    rng = np.random.default_rng(seed)
    q = rng.integers(1, qmax + 1, B)
    q[0] = 1
    q[-1] = qmax
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(q)
    T = int(cu[-1])
    logits = (rng.standard_normal((T, V)) * sigma).astype(np.float32)
    dprobs = np.zeros((T, V), np.float32)
    draft = np.zeros(T, np.int32)
    parent = np.zeros(T, np.int32)
    for i in range(B):
        o = int(cu[i])
        par = _tree_parents(rng, int(q[i]), shape)
        parent[o:o + q[i]] = par
        for k in range(1, q[i]):
            # each node's drafter: a perturbed copy of the target at its parent
            d = S.target_probs(logits[o + par[k]].astype(np.float64) + rng.standard_normal(V) * noise, temperature)
            dprobs[o + k] = d.astype(np.float32)
            dprobs[o + k] /= dprobs[o + k].sum(dtype=np.float64)
            draft[o + k] = rng.choice(V, p=dprobs[o + k].astype(np.float64) / dprobs[o + k].sum(dtype=np.float64))
    u = rng.random(T).astype(np.float32)
    w = rng.random(B).astype(np.float32)
    return cu, logits, dprobs, draft, parent, u, w


def _run_tree(cu, logits, dprobs, draft, parent, u, w, temp):
    B, T, V = len(cu) - 1, int(cu[-1]), logits.shape[1]
    ws = torch.empty(ops.spec_accept_stochastic_workspace_size(B, T, V), dtype=torch.uint8, device=DEV)
    out = ops.spec_accept_stochastic_tree(torch.from_numpy(logits).to(DEV), torch.from_numpy(dprobs).to(DEV),
                                          i32(draft), i32(parent), torch.from_numpy(u).to(DEV),
                                          torch.from_numpy(w).to(DEV), i32(cu), temperature=temp, workspace=ws)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in out], ops.spec_accept_stochastic_device_status(ws)


def _compare_tree(cu, logits, dprobs, draft, parent, u, w, temp, acc, path, toks):
    B = len(cu) - 1
    exact = borderline = 0
    for i in range(B):
        o, q = int(cu[i]), int(cu[i + 1] - cu[i])
        pth, y_ref, r, tests = S.accept_request_tree(logits, dprobs, draft, parent, u, w[i], o, q, temp)
        undecided = any(abs(lhs - rhs) <= 1e-4 * max(rhs, 1e-30) for lhs, rhs in tests)
        n = int(acc[i]) - 1
        assert 0 <= n < q, (i, n)
        got = path[o:o + n + 1].tolist()
        # structure: a root path of the tree, tokens of its nodes, -1 after
        assert got[0] == 0 and all(parent[o + got[t + 1]] == got[t] for t in range(n)), (i, got)
        assert np.all(path[o + n + 1:o + q] == -1) and np.all(toks[o + n + 1:o + q] == -1)
        assert toks[o:o + n].tolist() == [int(draft[o + k]) for k in got[1:]]
        if undecided and got != pth:
            borderline += 1
            continue
        assert got == pth, (i, got, pth)
        c = np.cumsum(r)
        tgt = float(w[i]) * c[-1]
        y = int(toks[o + n])
        tol = 1e-4 * c[-1]
        assert 0 <= y < len(r) and r[y] > 0.0, (i, y)
        assert (c[y - 1] if y > 0 else 0.0) <= tgt + tol and c[y] >= tgt - tol, (i, y, tgt)
        exact += int(y == y_ref)
    return exact, borderline


@pytest.mark.parametrize("seed,B,V,qmax,temp,shape", [
    (10, 16, 1000, 8, 1.0, "random"), (11, 12, 4099, 12, 0.7, "wide"), (12, 8, 128256, 10, 1.0, "bushy"),
    (13, 4, 151936, 16, 1.3, "random"), (14, 6, 2048, 64, 1.0, "random"), (15, 3, 32000, 64, 0.8, "wide")])
def test_stochastic_tree_matches_oracle(seed, B, V, qmax, temp, shape):
    cu, logits, dprobs, draft, parent, u, w = _stoch_tree_case(seed, B, V, qmax, temp, shape)
    note(f"[gpu] spec_accept_stochastic_tree seed={seed} B={B} T={int(cu[-1])} V={V} shape={shape}")
    (acc, path, toks), st = _run_tree(cu, logits, dprobs, draft, parent, u, w, temp)
    assert st == 0
    exact, borderline = _compare_tree(cu, logits, dprobs, draft, parent, u, w, temp, acc, path, toks)
    note(f"  draws equal to the oracle's: {exact}/{B}, borderline walks: {borderline}, "
         f"accepted drafts: {int(acc.sum()) - B}")
    assert borderline <= 1 and exact >= B - 2


def test_stochastic_tree_of_chains_equals_chain_call():
    """One child per node: the tree call gives the chain call's outputs bit for bit."""
    cu, logits, dprobs, draft, parent, u, w = _stoch_tree_case(16, 24, 5000, 8, 1.0, "chain")
    (acc, path, toks), st = _run_tree(cu, logits, dprobs, draft, parent, u, w, 1.0)
    B, T = len(cu) - 1, int(cu[-1])
    ws = torch.empty(ops.spec_accept_stochastic_workspace_size(B, T, 5000), dtype=torch.uint8, device=DEV)
    ref = ops.spec_accept_stochastic(torch.from_numpy(logits).to(DEV), torch.from_numpy(dprobs).to(DEV), i32(draft),
                                     torch.from_numpy(u).to(DEV), torch.from_numpy(w).to(DEV), i32(cu), workspace=ws)
    torch.cuda.synchronize()
    assert st == 0
    for x, y in zip((acc, path, toks), ref):
        assert np.array_equal(x, y.cpu().numpy())


def test_stochastic_tree_bad_parent_sets_status():
    cu, logits, dprobs, draft, parent, u, w = _stoch_tree_case(17, 6, 700, 6, 1.0, "random")
    bad = 2 if cu[3] - cu[2] > 1 else 5
    o = int(cu[bad])
    parent[o + cu[bad + 1] - cu[bad] - 1] = 9 if cu[bad + 1] - cu[bad] > 1 else 0  # forward or root != -1
    (acc, path, toks), st = _run_tree(cu, logits, dprobs, draft, parent, u, w, 1.0)
    assert st & ops.DEV_BAD_PARENT
    assert acc[bad] == 0 and np.all(path[o:cu[bad + 1]] == -1)
    keep = [i for i in range(6) if i != bad]
    for i in keep:
        o2, q2 = int(cu[i]), int(cu[i + 1] - cu[i])
        pth, _, _, _ = S.accept_request_tree(logits, dprobs, draft, parent, u, w[i], o2, q2, 1.0)
        assert path[o2:o2 + len(pth)].tolist() == pth


@pytest.mark.parametrize("shape", ["chain", "random"])
def test_stochastic_in_captured_graph(shape):
    """Both stochastic calls captured in one HIP graph: three replays, with eager
    work and synchronisation between them, each equal bit for bit to an eager
    call on the same inputs."""
    cu, logits, dprobs, draft, parent, u, w = _stoch_tree_case(18, 12, 3000, 10, 1.0, shape)
    B, T, V = len(cu) - 1, int(cu[-1]), 3000
    d = lambda x: torch.from_numpy(x).to(DEV)
    L, Q, U, W = d(logits), d(dprobs), d(u), d(w)
    dr, par, cq = i32(draft), i32(parent), i32(cu)
    ws = [torch.empty(ops.spec_accept_stochastic_workspace_size(B, T, V), dtype=torch.uint8, device=DEV)
          for _ in range(2)]
    outs = [[torch.full((n,), -7, dtype=torch.int32, device=DEV) for n in (B, T, T)] for _ in range(2)]

    def calls(stream=None):
        if shape == "chain":
            ops.spec_accept_stochastic(L, Q, dr, U, W, cq, workspace=ws[0], accept_len=outs[0][0],
                                       accepted_path=outs[0][1], out_tokens=outs[0][2], stream=stream)
        ops.spec_accept_stochastic_tree(L, Q, dr, par, U, W, cq, workspace=ws[1], accept_len=outs[1][0],
                                        accepted_path=outs[1][1], out_tokens=outs[1][2], stream=stream)
    calls()
    torch.cuda.synchronize()
    eager = [[x.clone() for x in o] for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        calls(side)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        calls(side)
    for rep in range(3):
        for o in outs:
            for x in o:
                x.fill_(-7)
        noise = torch.randn(1 << 16, device=DEV).sum()  # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        for k in (0, 1) if shape == "chain" else (1,):
            for x, y in zip(outs[k], eager[k]):
                assert torch.equal(x, y), (rep, k)
    assert ops.spec_accept_stochastic_device_status(ws[1]) == 0
