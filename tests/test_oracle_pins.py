"""The oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_tree_bruteforce_seven_nodes():
    """All 720 topologically ordered 7-node trees x 64 match patterns."""
    pins.check_accept_tree_bruteforce(max_nodes=7)


def test_oracle_attention_same_at_any_thread_count():
    """The parallel loop over (request, KV head) changes no arithmetic: one
    host thread and several give bit-identical attention on a ragged tree and
    chain batch."""
    import numpy as np

    import oracle
    from speculative_decoding_verification_attn_amd import workloads as W
    trees = [W.draw_tree(np.random.Generator(np.random.PCG64(70 + i)), n, min(n - 1, 6), 4, 4)
             for i, n in enumerate([9, 33, 64])]
    cases = [W.make_custom(71, context_lens=[0, 300, 777], tree_parents=trees, hq=16, hkv=4, d=64, vocab=64),
             W.make_custom(72, context_lens=[5, 1200, 64, 0], q_lens=[4, 17, 64, 1], hq=24, hkv=8, d=128,
                           vocab=64)]
    before = oracle.set_threads(0)
    try:
        for case in cases:
            args = (case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.cu_q,
                    case.tree_parent)
            kw = dict(num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                      page_size=case.page_size, num_pages=case.num_pages)
            oracle.set_threads(1)
            one = oracle.verify_attn(*args, **kw)
            oracle.set_threads(4)
            many = oracle.verify_attn(*args, **kw)
            assert np.array_equal(one, many)
    finally:
        oracle.set_threads(before)
