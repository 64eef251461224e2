"""Content errors only the device can see (the header's contract): a request
whose metadata breaks the rules gets a status bit and unspecified outputs,
nothing outside the caches or the workspace is touched, and every other
request of the same call is still computed exactly as the oracle computes it.

Each case corrupts one request of an otherwise valid batch on the device; the
oracle runs on the uncorrupted batch, and only the untouched requests' rows are
compared."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (LAYOUT_IDS, LAYOUTS, DevCase, assert_attn_close, bf16_out_to_f64, compact_fn,
                      gpu_attn, i32, note, oracle_attn, u16_to_bf16_dev, bf16_dev_to_u16, v_from_dev, v_to_dev)
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu
layouts = pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)


def _chain_case(seed=900, q_lens=(4, 5, 3), ctx=(300, 500, 200)):
    return W.make_custom(seed, context_lens=list(ctx), q_lens=list(q_lens), hq=8, hkv=2, d=128, vocab=64)


def _rows(case, reqs):
    return np.concatenate([np.arange(case.cu_q[i], case.cu_q[i + 1]) for i in reqs]).astype(np.int64)


def _check_others(case, out, reqs, tag):
    ref = oracle_attn(case)
    rows = _rows(case, reqs)
    assert_attn_close(bf16_out_to_f64(out)[rows], ref[rows], tag)


@layouts
def test_bad_page_id(vt):
    case = _chain_case()
    dc = DevCase(case, vt)
    for bad in (case.num_pages + 7, -5):
        bt = case.block_tables.copy()
        bt[1, 2] = bad  # a page request 1 needs (its keys span 32 pages)
        dc.bt = i32(bt)
        note(f"[gpu] bad page id {bad} in request 1, vt={vt}")
        out, ws = gpu_attn(dc)
        assert ops.spec_verify_attn_device_status(ws) & ops.DEV_BAD_PAGE
        _check_others(case, out, [0, 2], f"bad page {bad}")


@layouts
def test_bad_parent(vt):
    trees = [W.draw_tree(np.random.Generator(np.random.PCG64(910 + i)), n, min(n - 1, 6), 4, 4)
             for i, n in enumerate([9, 12, 7])]
    case = W.make_custom(911, context_lens=[100, 250, 60], tree_parents=trees, hq=8, hkv=2, d=128, vocab=64)
    dc = DevCase(case, vt)
    par = case.tree_parent.copy()
    o = int(case.cu_q[1])
    par[o + 5] = 7  # a parent after its child
    dc.par = i32(par)
    note(f"[gpu] parent after child in request 1, vt={vt}")
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) & ops.DEV_BAD_PARENT
    _check_others(case, out, [0, 2], "bad parent")


@layouts
def test_negative_context_and_too_many_pages(vt):
    case = _chain_case()
    dc = DevCase(case, vt)
    ctx = case.context_lens.copy()
    ctx[1] = -3
    dc.ctx = i32(ctx)
    note(f"[gpu] negative context length in request 1, vt={vt}")
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) & ops.DEV_BAD_CONTEXT
    _check_others(case, out, [0, 2], "negative context")
    # a block table narrower than request 1 needs (32 pages), wide enough for the others
    dc.ctx = i32(case.context_lens)
    dc.bt = i32(np.ascontiguousarray(case.block_tables[:, :20]))
    note(f"[gpu] block table too narrow for request 1, vt={vt}")
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) & ops.DEV_TOO_MANY_PAGES
    _check_others(case, out, [0, 2], "too many pages")


@layouts
def test_too_many_tokens_and_bad_cu_q(vt):
    case = _chain_case(q_lens=(4, 64, 1), ctx=(300, 500, 200))
    dc = DevCase(case, vt)
    cu = case.cu_q.copy()
    cu[2] += 1  # request 1 now has 65 rows, request 2 none
    dc.cu = i32(cu)
    note(f"[gpu] 65 verify tokens in request 1, vt={vt}")
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) & ops.DEV_TOO_MANY_TOKENS
    _check_others(case, out, [0], "too many tokens")
    cu = case.cu_q.copy()
    cu[1], cu[2] = cu[2], cu[1]  # not non-decreasing
    dc.cu = i32(cu)
    note(f"[gpu] cu_q out of order, vt={vt}")
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) & ops.DEV_BAD_CU_Q


@layouts
def test_compaction_leaves_a_broken_request_untouched(vt):
    trees = [W.draw_tree(np.random.Generator(np.random.PCG64(920 + i)), n, min(n - 1, 6), 4, 4)
             for i, n in enumerate([10, 14, 9])]
    case = W.make_custom(921, context_lens=[40, 130, 75], tree_parents=trees, hq=4, hkv=2, d=64, vocab=64,
                         tree_match=(1.0, 0.0))
    t_ref = oracle.argmax(case.logits)
    acc, path, _ = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    assert np.all(acc >= 2)  # every request moves something or at least has a path to check
    o1 = int(case.cu_q[1])
    bad_path = path.copy()
    bad_path[o1 + 1] = 0  # not strictly increasing
    # the oracle: requests 0 and 2 as given, request 1 without moves
    k_ref, v_ref = case.k_cache.copy(), case.v_cache.copy()
    acc_ref = acc.copy()
    acc_ref[1] = 1
    new_ref = oracle.compact(k_ref, v_ref, case.block_tables, case.context_lens, case.cu_q, path, acc_ref,
                             num_kv_heads=2, head_dim=64, page_size=16, num_pages=case.num_pages)
    kd, vd = u16_to_bf16_dev(case.k_cache), v_to_dev(case.v_cache, vt)
    note(f"[gpu] kv_compact with a broken path in request 1, vt={vt}")
    new = compact_fn(vt)(kd, vd, i32(case.block_tables), i32(case.context_lens), i32(case.cu_q), i32(bad_path),
                         i32(acc))
    torch.cuda.synchronize()
    new = new.cpu().numpy()
    assert new[1] == -1 and new[0] == new_ref[0] and new[2] == new_ref[2]
    assert np.array_equal(bf16_dev_to_u16(kd), k_ref) and np.array_equal(v_from_dev(vd, vt), v_ref)


def test_acceptance_with_a_broken_request():
    """spec_accept: a parent after its child in one tree request, then a request of
    65 rows: the status bit is set and every other request's argmax, acceptance,
    path and tokens equal the oracle's."""
    trees = [W.draw_tree(np.random.Generator(np.random.PCG64(930 + i)), n, min(n - 1, 6), 4, 4)
             for i, n in enumerate([11, 16, 8])]
    case = W.make_custom(931, context_lens=[10, 20, 30], tree_parents=trees, hq=4, hkv=2, d=64, vocab=3000,
                         tree_match=(0.8, 0.3))
    dc = DevCase(case, False)
    t_ref = oracle.argmax(case.logits)
    acc_ref, path_ref, tok_ref = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    par = case.tree_parent.copy()
    o1 = int(case.cu_q[1])
    par[o1 + 4] = 9
    ws = torch.empty(ops.spec_accept_workspace_size(case.batch, case.total_q, case.vocab), dtype=torch.uint8,
                     device=dc.logits.device)
    note("[gpu] spec_accept with a parent after its child in request 1")
    t, acc, path, tok = [x.cpu().numpy() for x in ops.spec_accept(dc.logits, dc.draft, dc.cu, i32(par),
                                                                  workspace=ws)]
    assert ops.spec_accept_device_status(ws) & ops.DEV_BAD_PARENT
    assert np.array_equal(t, t_ref)  # the argmax of every row is still exact
    rows = _rows(case, [0, 2])
    assert acc[0] == acc_ref[0] and acc[2] == acc_ref[2]
    assert np.array_equal(path[rows], path_ref[rows]) and np.array_equal(tok[rows], tok_ref[rows])
    # a chain batch whose middle request claims 65 rows
    case = _chain_case(q_lens=(4, 64, 1), ctx=(30, 50, 20))
    dc = DevCase(case, False)
    t_ref = oracle.argmax(case.logits)
    acc_ref, path_ref, tok_ref = oracle.accept(case.draft_tokens, t_ref, case.cu_q, None)
    cu = case.cu_q.copy()
    cu[2] += 1
    ws = torch.empty(ops.spec_accept_workspace_size(case.batch, case.total_q, case.vocab), dtype=torch.uint8,
                     device=dc.logits.device)
    note("[gpu] spec_accept with 65 rows in request 1")
    t, acc, path, tok = [x.cpu().numpy() for x in ops.spec_accept(dc.logits, dc.draft, i32(cu), None,
                                                                  workspace=ws)]
    assert ops.spec_accept_device_status(ws) & ops.DEV_TOO_MANY_TOKENS
    rows = _rows(case, [0])
    assert acc[0] == acc_ref[0]
    assert np.array_equal(path[rows], path_ref[rows]) and np.array_equal(tok[rows], tok_ref[rows])
