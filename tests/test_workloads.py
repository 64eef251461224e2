"""Seeded input generator: determinism, bf16 rounding, paging structure, tree
shapes, planted greedy targets and the closed-form expected acceptance."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_verification_attn_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 37,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38,
                                  1e-40, 65504.0], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_determinism():
    a = W.make_case("tiny_chain")
    b = W.make_case("tiny_chain")
    for f in ("q", "k_cache", "v_cache", "logits", "draft_tokens", "block_tables", "cu_q"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = W.make_case("tiny_chain", seed=99)
    assert not np.array_equal(a.q, c.q)


@pytest.mark.parametrize("name", ["tiny_chain", "llama31_8b_chain", "llama3_70b_tree"])
def test_paging_structure(name):
    case = W.make_case(name)
    P = case.page_size
    used = []
    for i in range(case.batch):
        n = (int(case.context_lens[i]) + int(case.q_lens[i]) + P - 1) // P
        used.extend(case.block_tables[i, :n].tolist())
        assert np.all(case.block_tables[i, n:] == case.poison_page)
    assert len(set(used)) == len(used)
    assert set(used) | {case.poison_page} == set(range(case.num_pages))
    # poison page and tail slots hold +-1e3
    pk = W.bf16_bits_to_f32(case.k_cache[case.poison_page])
    assert np.all(np.abs(pk) == 1000.0)


def test_tree_shape():
    for seed in range(20):
        rng = np.random.Generator(np.random.PCG64(seed))
        par = W.draw_tree(rng, 64, 6, 4, 4)
        assert len(par) == 64 and par[0] == -1
        assert all(0 <= par[j] < j for j in range(1, 64))
        depth = np.zeros(64, int)
        for j in range(1, 64):
            depth[j] = depth[par[j]] + 1
        assert depth.max() == 6
        fan = np.bincount(par[1:], minlength=64)
        assert fan[0] <= 4 and fan.max() <= 4
        # BFS order: depths non-decreasing
        assert np.all(np.diff(depth) >= 0)


def test_planted_target_is_unique_row_max():
    case = W.make_case("tiny_chain")
    assert np.array_equal(np.argmax(case.logits, axis=1), case.planted_target)
    rowmax = case.logits.max(axis=1)
    assert np.all((case.logits == rowmax[:, None]).sum(axis=1) == 1)
    assert np.array_equal(oracle.argmax(case.logits), case.planted_target)


def _empirical_accept(p, gamma, n_req, seed):
    case = W.build_case("stat", seed, batch=n_req, q_lens=np.full(n_req, gamma + 1),
                        context_lens=np.zeros(n_req, np.int32), tree_parents=None, hq=1, hkv=1,
                        d=8, vocab=64, logit_sigma=2.0, qkv_scale=1.0,
                        match_prob_per_req=np.full(n_req, p))
    t = oracle.argmax(case.logits)
    acc, _, _ = oracle.accept(case.draft_tokens, t, case.cu_q, None)
    return acc


@pytest.mark.parametrize("p,gamma", [(0.7, 4), (0.8, 5), (0.75, 3)])
def test_expected_accept_len_closed_form(p, gamma):
    """E[accept_len] = sum_{k=0..gamma} p^k (draft j matches with prob p independently)."""
    acc = _empirical_accept(p, gamma, 20000, seed=int(p * 100) + gamma)
    mean = acc.mean()
    expect = W.expected_chain_accept_len(p, gamma)
    se = acc.std() / np.sqrt(len(acc))
    assert abs(mean - expect) < 4 * se, (mean, expect, se)


def test_beta_ragged_expected_accept_len():
    """Config with gamma ~ U{1..8} and p ~ Beta(2,2): E = mean_gamma E_p[sum_k p^k],
    where E[p^k] for Beta(2,2) is 6/((k+2)(k+3))."""
    cfg = W.CONFIGS["qwen3_8b_ragged"]
    rng = np.random.default_rng(1)
    n = 20000
    gam = rng.integers(1, 9, size=n)
    p = rng.beta(2, 2, size=n)
    case = W.build_case("stat", 5, batch=n, q_lens=gam + 1, context_lens=np.zeros(n, np.int32),
                        tree_parents=None, hq=1, hkv=1, d=8, vocab=64, logit_sigma=3.0,
                        qkv_scale=1.0, match_prob_per_req=p)
    t = oracle.argmax(case.logits)
    acc, _, _ = oracle.accept(case.draft_tokens, t, case.cu_q, None)

    def e_beta(k):
        return 6.0 / ((k + 2) * (k + 3))
    expect = np.mean([sum(e_beta(k) for k in range(g + 1)) for g in range(1, 9)])
    se = acc.std() / np.sqrt(n)
    assert abs(acc.mean() - expect) < 4 * se, (acc.mean(), expect)
    assert cfg["match"][0] == "beta"
