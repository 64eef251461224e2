"""Acceptance and compaction in one launch (SwiftSpec, "Fused Latency-Optimized
Kernels") on the GPU, through the C ABI: the outputs and the whole multi-layer
caches must equal the oracle's acceptance followed by its copy-based
compaction, bit for bit, on several calls in a row on one workspace (the launch
clears its own counters), eagerly and replayed from a HIP graph."""
import numpy as np
import pytest
import torch

import oracle
import pins
from gpu_util import (DEV, LAYOUT_IDS, LAYOUTS, DevCase, accept_compact_fn, bf16_dev_to_u16, i32, note,
                      u16_to_bf16_dev, v_from_dev, v_to_dev)
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu

LAYERS = 3


def _tree(seed, nodes=64, depth=6):
    return W.draw_tree(np.random.Generator(np.random.PCG64(seed)), nodes, depth, 4, 4)


CASES = {
    "trees_d128": dict(context_lens=[5, 18, 0, 250, 40],
                       tree_parents=[pins.SMALL_TREES[0], pins.SMALL_TREES[1], np.array([-1, 0, 1, 1, 2], np.int32),
                                     _tree(5), _tree(6, 30, 5)],
                       hq=16, hkv=8, d=128, vocab=600, tree_match=(0.7, 0.6)),
    "trees_d64": dict(context_lens=[100, 3, 17], tree_parents=[_tree(7), _tree(8, 20, 4), _tree(9, 9, 3)],
                      hq=8, hkv=2, d=64, vocab=300, tree_match=(0.8, 0.7)),
    "chains_d128": dict(context_lens=[0, 47, 64, 500], q_lens=[4, 9, 1, 6], hq=32, hkv=8, d=128, vocab=700,
                        match_p=0.8),
}


def _caches(case):
    rng = np.random.default_rng(1)
    extra = lambda shp: W.f32_to_bf16_bits(rng.standard_normal(shp).astype(np.float32))
    k = np.stack([case.k_cache] + [extra(case.k_cache.shape) for _ in range(LAYERS - 1)])
    v = np.stack([case.v_cache] + [extra(case.v_cache.shape) for _ in range(LAYERS - 1)])
    return k, v


def _oracle(case, k_all, v_all):
    t_ref = oracle.argmax(case.logits)
    acc, path, toks = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    k_ref, v_ref = k_all.copy(), v_all.copy()
    new = oracle.compact(k_ref, v_ref, case.block_tables, case.context_lens, case.cu_q, path, acc,
                         num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, page_size=16,
                         num_pages=case.num_pages, num_layers=LAYERS)
    return dict(t=t_ref, acc=acc, path=path, toks=toks, new=new, k=k_ref, v=v_ref)


def _check(ref, outs, kd, vd, tag, vt):
    t, acc, path, toks, new = [x.cpu().numpy() for x in outs]
    assert np.array_equal(t, ref["t"]), tag
    assert np.array_equal(acc, ref["acc"]), tag
    assert np.array_equal(path, ref["path"]), tag
    assert np.array_equal(toks, ref["toks"]), tag
    assert np.array_equal(new, ref["new"]), tag
    assert np.array_equal(bf16_dev_to_u16(kd), ref["k"]), tag
    assert np.array_equal(v_from_dev(vd, vt), ref["v"]), tag


@pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_oracle_on_repeated_calls(name, vt):
    case = W.make_custom(400 + list(CASES).index(name), **CASES[name])
    dc = DevCase(case)
    k_all, v_all = _caches(case)
    ref = _oracle(case, k_all, v_all)
    if case.tree_parent is not None:
        assert not np.array_equal(ref["k"], k_all)  # something really moves
    ws = torch.zeros(ops.spec_accept_compact_workspace_size(case.batch, case.total_q, case.vocab),
                     dtype=torch.uint8, device=DEV)
    for rep in range(3):
        note(f"[gpu] spec_accept_compact {name} vt={vt} call {rep}")
        kd, vd = u16_to_bf16_dev(k_all), v_to_dev(v_all, vt)
        outs = accept_compact_fn(vt)(dc.logits, dc.draft, dc.cu, dc.par, kd, vd, dc.bt, dc.ctx,
                                     workspace=ws, num_layers=LAYERS)
        torch.cuda.synchronize()
        assert ops.spec_accept_device_status(ws) == 0
        _check(ref, outs, kd, vd, f"{name} call {rep}", vt)


@pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)
def test_fused_graph_replays(vt):
    """The fused call captured in a HIP graph, replayed with eager cache restores between."""
    name = "trees_d128"
    case = W.make_custom(400, **CASES[name])
    dc = DevCase(case)
    k_all, v_all = _caches(case)
    ref = _oracle(case, k_all, v_all)
    k0, v0 = u16_to_bf16_dev(k_all), v_to_dev(v_all, vt)
    kd, vd = k0.clone(), v0.clone()
    ws = torch.zeros(ops.spec_accept_compact_workspace_size(case.batch, case.total_q, case.vocab),
                     dtype=torch.uint8, device=DEV)
    B, T = case.batch, case.total_q
    outs = [torch.empty(n, dtype=torch.int32, device=DEV) for n in (T, B, T, T, B)]

    def call():
        accept_compact_fn(vt)(dc.logits, dc.draft, dc.cu, dc.par, kd, vd, dc.bt, dc.ctx, workspace=ws,
                              num_layers=LAYERS, target_argmax=outs[0], accept_len=outs[1],
                              accepted_path=outs[2], out_tokens=outs[3], new_context_lens=outs[4])

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        kd.copy_(k0)
        vd.copy_(v0)
        for o in outs:
            o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert ops.spec_accept_device_status(ws) == 0
        _check(ref, outs, kd, vd, f"replay {rep}", vt)
        note(f"[gpu] fused replay {rep} ok")


def _ragged_trees(seed, batch, total):
    """`batch` random trees (1 to 9 nodes) with `total` nodes in all."""
    rng = np.random.default_rng(seed)
    sizes = np.full(batch, total // batch)
    sizes[: total % batch] += 1
    for _ in range(4 * batch):  # reshuffle node counts, keeping the total
        a, b = rng.integers(0, batch, 2)
        if sizes[a] > 1 and sizes[b] < 9:
            sizes[a] -= 1
            sizes[b] += 1
    trees = []
    for k, n in enumerate(sizes):
        depth = int(min(n - 1, rng.integers(3, 6)))  # depth >= 3 holds 9 nodes whatever the root fan-out
        trees.append(np.array([-1], np.int32) if n == 1 else _tree(seed * 1000 + k, int(n), depth))
    ctx = rng.integers(0, 90, batch).tolist()
    return dict(context_lens=ctx, tree_parents=trees, hq=8, hkv=2, d=64, vocab=151936, tree_match=(0.8, 0.5))


def test_fused_workspace_shared_across_shapes():
    """One zero-filled workspace, sized for the largest shape, serves calls of
    different (batch, total_q): a continuous batch changes shape every step.
    Batch 64 with 300 then 290 verify rows puts the slice count per row (and so
    every offset after the slice partials) at different places; then a smaller
    batch, then the first shape again."""
    shapes = [(64, 300), (64, 290), (40, 200), (64, 300)]
    cases = [W.make_custom(470 + k, **_ragged_trees(470 + k, b, t)) for k, (b, t) in enumerate(shapes)]
    size = max(ops.spec_accept_compact_workspace_size(c.batch, c.total_q, c.vocab) for c in cases)
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    for k, case in enumerate(cases):
        assert case.total_q == shapes[k][1]
        note(f"[gpu] spec_accept_compact shared workspace call {k}: B={case.batch} T={case.total_q}")
        dc = DevCase(case)
        k_all, v_all = _caches(case)
        ref = _oracle(case, k_all, v_all)
        kd, vd = u16_to_bf16_dev(k_all), v_to_dev(v_all, False)
        outs = ops.spec_accept_compact(dc.logits, dc.draft, dc.cu, dc.par, kd, vd, dc.bt, dc.ctx,
                                       workspace=ws, num_layers=LAYERS)
        torch.cuda.synchronize()
        assert ops.spec_accept_device_status(ws) == 0, k
        _check(ref, outs, kd, vd, f"shared workspace call {k}", False)
        # everything the call wrote is zero again, apart from the status word
        rest = ws[4:].cpu().numpy()
        assert not rest.any(), (k, np.flatnonzero(rest)[:8])


def test_fused_waits_give_up_and_workspace_recovers():
    """The ticket counter is preset from the host, so every waiting work item
    draws a ticket past the last item: the launch must report
    SV_DEV_SYNC_TIMEOUT and still end (every wait is bounded), and its last
    item must leave the workspace zeroed, so the next call on the same
    workspace is exact."""
    name = "trees_d128"
    case = W.make_custom(400, **CASES[name])
    dc = DevCase(case)
    k_all, v_all = _caches(case)
    ref = _oracle(case, k_all, v_all)
    ws = torch.zeros(ops.spec_accept_compact_workspace_size(case.batch, case.total_q, case.vocab),
                     dtype=torch.uint8, device=DEV)
    ws[8:12].view(torch.int32).fill_(1 << 30)  # header word 2: the ticket counter
    torch.cuda.synchronize()
    note("[gpu] spec_accept_compact with a preset ticket counter (bounded waits give up)")
    kd, vd = u16_to_bf16_dev(k_all), v_to_dev(v_all, False)
    ops.spec_accept_compact(dc.logits, dc.draft, dc.cu, dc.par, kd, vd, dc.bt, dc.ctx, workspace=ws,
                            num_layers=LAYERS)
    torch.cuda.synchronize()
    st = ops.spec_accept_device_status(ws)
    assert st & ops.SV_DEV_SYNC_TIMEOUT, st
    assert not ws[4:].cpu().numpy().any()
    note("[gpu] next call on the same workspace")
    kd, vd = u16_to_bf16_dev(k_all), v_to_dev(v_all, False)
    outs = ops.spec_accept_compact(dc.logits, dc.draft, dc.cu, dc.par, kd, vd, dc.bt, dc.ctx, workspace=ws,
                                   num_layers=LAYERS)
    torch.cuda.synchronize()
    assert ops.spec_accept_device_status(ws) == 0
    _check(ref, outs, kd, vd, "after give-up", False)
