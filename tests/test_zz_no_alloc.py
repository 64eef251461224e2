"""spec_verify_attn_noalloc: the verify attention of spec_verify_attn with its
workspace in the library's static device scratch instead of a caller buffer,
for callers that cannot allocate.  Through the C ABI, two calls in a row (the
second smaller, so it runs over what the first left in the scratch) must give
spec_verify_attn's output bit for bit, and the oracle's within the attention
tolerance; sizes past the scratch are refused before anything is launched."""
import numpy as np
import pytest
import torch

import pins
from gpu_util import DEV, DevCase, assert_attn_close, bf16_out_to_f64, i32, note, oracle_attn
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu


def _tree(seed, nodes, depth):
    return W.draw_tree(np.random.Generator(np.random.PCG64(seed)), nodes, depth, 4, 4)


def _compare(case, tag):
    dc = DevCase(case)
    out = torch.full_like(dc.q, 7.0)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    note(f"[gpu] spec_verify_attn_noalloc {tag}: B={case.batch} T={case.total_q}")
    ops.spec_verify_attn_noalloc(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, dc.par, out=out, device_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, tag
    ref = ops.spec_verify_attn(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, dc.par)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), tag
    assert_attn_close(bf16_out_to_f64(out), oracle_attn(case), tag)


def test_noalloc_equals_spec_verify_attn_twice():
    big = W.make_custom(61, context_lens=[3000, 17, 900, 0, 4500, 260],
                        tree_parents=[_tree(1, 64, 6), pins.SMALL_TREES[0], _tree(2, 30, 5),
                                      np.array([-1, 0], np.int32), _tree(3, 9, 3), _tree(4, 64, 8)],
                        hq=64, hkv=8, d=128)
    small = W.make_custom(62, context_lens=[40, 700], q_lens=[3, 6], hq=32, hkv=8, d=128)
    _compare(big, "first call")
    _compare(small, "second call, smaller")


def test_noalloc_refuses_sizes_past_the_scratch():
    """Sizes whose workspace exceeds the static scratch are refused on the host,
    with nothing launched (the output keeps its contents)."""
    case = W.make_custom(63, context_lens=[10], q_lens=[4], hq=8, hkv=2, d=64)
    dc = DevCase(case)
    B, T = 40000, 40000 * 64
    assert ops.spec_verify_attn_workspace_size(B, T, 64, 8, 128) > ops.NOALLOC_SCRATCH_BYTES
    lib = ops.load_library()
    out = torch.full_like(dc.q, 3.0)
    rc = lib.spec_verify_attn_noalloc(ops._ptr(dc.q), ops._ptr(dc.k), ops._ptr(dc.v), ops._ptr(dc.bt), 4,
                                      ops._ptr(dc.ctx), ops._ptr(dc.cu), None, ops._ptr(out), B, T, 64, 8, 128,
                                      16, case.num_pages, 0.0, None, ops._stream(None))
    torch.cuda.synchronize()
    assert rc == ops.SV_ERR_WORKSPACE
    assert b"static scratch" in lib.sv_last_error()
    assert bool((out.float() == 3.0).all())
