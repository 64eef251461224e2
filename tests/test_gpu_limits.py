"""HIP path vs the CPU oracle at the edges of the supported sizes (needs an
MI355X): a batch larger than the plan keeps in LDS, a context of 131k tokens,
and 64-token chains (the most verify tokens one request may carry)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (DEV, LAYOUT_IDS, LAYOUTS, DevCase, assert_attn_close, bf16_out_to_f64, gpu_accept,
                      gpu_attn, i32, note, oracle_attn)
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu

PLAN_LDS_REQUESTS = 4096  # batches above this keep the plan's per-request data in the workspace


def _accept_all(case, dc):
    (t, acc, path, toks), ws = gpu_accept(dc)
    assert ops.spec_accept_device_status(ws) == 0
    t_ref = oracle.argmax(case.logits)
    acc_ref, path_ref, toks_ref = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    assert np.array_equal(t, t_ref)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(path, path_ref)
    assert np.array_equal(toks, toks_ref)
    return acc_ref, path_ref


def test_batch_beyond_plan_lds():
    """4100 ragged requests (contexts 0..48, 1..4 verify tokens): attention,
    acceptance and compaction against the oracle, through the plan's
    workspace-resident path."""
    rng = np.random.default_rng(11)
    B = PLAN_LDS_REQUESTS + 4
    ctx = rng.integers(0, 49, B).tolist()
    ql = rng.integers(1, 5, B).tolist()
    case = W.make_custom(41, context_lens=ctx, q_lens=ql, hq=8, hkv=2, d=64, vocab=64)
    dc = DevCase(case)
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) == 0
    assert_attn_close(bf16_out_to_f64(out), oracle_attn(case), f"B={B}")
    acc_ref, path_ref = _accept_all(case, dc)
    new = ops.kv_compact(dc.k, dc.v, dc.bt, dc.ctx, dc.cu, i32(path_ref), i32(acc_ref))
    torch.cuda.synchronize()
    assert np.array_equal(new.cpu().numpy(), case.context_lens + acc_ref)
    note(f"  B={B}: mean accept_len {acc_ref.mean():.3f}")


@pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)
def test_long_context(vt):
    """One request with a 131,072-token context beside a 40,001-token one
    (8,193 + 2,501 pages, permuted): every row against the oracle."""
    case = W.make_custom(42, context_lens=[131072, 40001], q_lens=[4, 2], hq=32, hkv=8, d=128,
                         vocab=256)
    dc = DevCase(case, vt)
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) == 0
    assert_attn_close(bf16_out_to_f64(out), oracle_attn(case), "L=131072")


@pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)
def test_chain_of_64_tokens(vt):
    """Chains of 64 and 33 verify tokens with G = 8 (512 and 264 rows: 16 and 9
    row tiles of one KV head): attention and acceptance, including an
    all-correct 64-token draft that accepts 64."""
    case = W.make_custom(43, context_lens=[5000, 100], q_lens=[64, 33], hq=32, hkv=4, d=128,
                         vocab=128, match_p=0.97)
    # the first request's drafts all equal the target's argmax at their parent
    t_ref = oracle.argmax(case.logits)
    o = int(case.cu_q[0])
    case.draft_tokens[o + 1:o + 64] = t_ref[o:o + 63]
    dc = DevCase(case, vt)
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) == 0
    assert_attn_close(bf16_out_to_f64(out), oracle_attn(case), "q=64")
    acc_ref, _ = _accept_all(case, dc)
    assert acc_ref[0] == 64
