"""The diagnostic trace build of the library (libspecverify_trace.so): its
attention output is bit-identical to the production library's (the trace
only adds timestamps and moves two waits), and the timeline it records is
well formed: every wave of every range opens with codes 1, 2, closes with 9,
moves only along the kernel's phase transitions, and its times never run
backwards."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from gpu_util import DevCase, gpu_attn, note
from speculative_decoding_verification_attn_amd import build, ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu

ALLOWED = {(1, 2), (2, 3), (3, 4), (4, 5), (5, 6), (6, 3), (6, 7), (7, 8), (7, 9), (8, 3)}


def _trace_lib_call(fn):
    """fn() with the trace build loaded in place of the production library."""
    saved = ops._lib, ops.LIB_PATH
    try:
        ops._lib = None
        ops.LIB_PATH = build.TRACE_LIB
        ops.load_library()
        return fn()
    finally:
        ops._lib, ops.LIB_PATH = saved


@pytest.mark.parametrize("kind", ["tree", "ragged_chain"])
def test_trace_build_output_and_timeline(kind):
    if not os.path.exists(build.TRACE_LIB):
        pytest.skip("trace build absent (python -m speculative_decoding_verification_attn_amd.build --trace)")
    if kind == "tree":
        trees = [W.draw_tree(np.random.Generator(np.random.PCG64(950 + i)), n, 6, 4, 4) for i, n in enumerate([64, 40])]
        case = W.make_custom(951, context_lens=[3000, 1700], tree_parents=trees, hq=32, hkv=4, d=128, vocab=64)
    else:
        case = W.make_custom(952, context_lens=[5000, 37, 900, 12000, 0, 2500], q_lens=[4, 1, 7, 2, 3, 5],
                             hq=32, hkv=8, d=128, vocab=64)
    dc = DevCase(case, True)
    out_prod, _ = gpu_attn(dc)

    def traced():
        ops.spec_verify_attn_phase_trace(clear=True)
        note(f"[gpu] trace build: spec_verify_attn_vt {kind}")
        out, _ = gpu_attn(dc)
        return out, ops.spec_verify_attn_phase_trace(clear=True)

    out_tr, tl = _trace_lib_call(traced)
    assert torch.equal(out_prod.view(torch.int16), out_tr.view(torch.int16))
    waves = 0
    for w in range(tl.shape[0]):
        for wv in range(tl.shape[1]):
            ev = tl[w, wv]
            ev = ev[ev != 0]
            if len(ev) == 0:
                continue
            waves += 1
            t = (ev >> np.uint64(8)).astype(np.int64)
            c = (ev & np.uint64(255)).astype(np.int64).tolist()
            assert c[0] == 1 and c[1] == 2 and c[-1] == 9, (w, wv, c[:8], c[-4:])
            assert all((a, b) in ALLOWED for a, b in zip(c[:-1], c[1:])), (w, wv, c)
            assert np.all(np.diff(t) >= 0), (w, wv)
    assert waves > 0 and waves % 4 == 0
