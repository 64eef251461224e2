"""The whole verify step captured in one HIP graph and replayed.

Graph replays must equal eager launches bit for bit, replay after replay,
with the program's own eager work and synchronisations between replays (the
library records no memset node: every piece of workspace state is written by
its own kernels).  The caches are restored eagerly before each replay because
compaction moves tree K/V in place."""
import numpy as np
import pytest
import torch

from gpu_util import (DEV, LAYOUT_IDS, LAYOUTS, DevCase, attn_run_fn, compact_fn, note, u16_to_bf16_dev,
                      v_to_dev)
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu


def _tree(seed, nodes=64, depth=6):
    return W.draw_tree(np.random.Generator(np.random.PCG64(seed)), nodes, depth, 4, 4)


@pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("kind", ["chains", "trees"])
def test_graph_replay_equals_eager(kind, vt):
    if kind == "chains":
        case = W.make_custom(21, context_lens=[300, 5, 1200, 64, 0], q_lens=[4, 9, 2, 6, 1], hq=32, hkv=8, d=128)
    else:
        case = W.make_custom(22, context_lens=[300, 0, 77], tree_parents=[_tree(1), _tree(2, 40, 9), _tree(3, 7, 3)],
                             hq=32, hkv=8, d=128, vocab=512)
    note(f"[gpu] graph replay {kind}: B={case.batch} T={case.total_q}")
    dc = DevCase(case, vt)
    B, T, layers = case.batch, case.total_q, 3
    rng = np.random.default_rng(7)
    # three layers: distinct K/V pools stacked so one compaction call covers them
    K = torch.stack([dc.k] + [u16_to_bf16_dev(W.f32_to_bf16_bits(
        rng.standard_normal(case.k_cache.shape).astype(np.float32))) for _ in range(layers - 1)])
    V = torch.stack([dc.v] + [v_to_dev(W.f32_to_bf16_bits(
        rng.standard_normal(case.v_cache.shape).astype(np.float32)), vt) for _ in range(layers - 1)])
    K0, V0 = K.clone(), V.clone()
    ws = torch.empty(ops.spec_verify_attn_workspace_size(B, T, 32, 8, 128), dtype=torch.uint8, device=DEV)
    wsa = torch.empty(ops.spec_accept_workspace_size(B, T, case.vocab), dtype=torch.uint8, device=DEV)
    outs = torch.empty((layers,) + tuple(dc.q.shape), dtype=torch.bfloat16, device=DEV)
    t_arg = torch.empty(T, dtype=torch.int32, device=DEV)
    acc = torch.empty(B, dtype=torch.int32, device=DEV)
    path = torch.empty(T, dtype=torch.int32, device=DEV)
    toks = torch.empty(T, dtype=torch.int32, device=DEV)
    new_len = torch.empty(B, dtype=torch.int32, device=DEV)

    def step():
        ops.spec_verify_attn_plan(dc.ctx, dc.cu, max_blocks_per_seq=case.max_blocks, num_q_heads=32,
                                  num_kv_heads=8, head_dim=128, num_pages=case.num_pages, total_q=T, workspace=ws)
        for layer in range(layers):
            attn_run_fn(vt)(dc.q, K[layer], V[layer], dc.bt, dc.ctx, dc.cu, dc.par, out=outs[layer],
                            workspace=ws)
        ops.spec_accept(dc.logits, dc.draft, dc.cu, dc.par, target_argmax=t_arg, accept_len=acc,
                        accepted_path=path, out_tokens=toks, workspace=wsa)
        compact_fn(vt)(K, V, dc.bt, dc.ctx, dc.cu, path, acc, num_layers=layers, new_context_lens=new_len)

    def results():
        return [x.clone() for x in (outs, t_arg, acc, path, toks, new_len, K, V)]

    def scrub():
        # eager work between replays: restore the caches, poison every output
        K.copy_(K0)
        V.copy_(V0)
        outs.fill_(float("nan"))
        for x in (t_arg, acc, path, toks, new_len):
            x.fill_(-7)
        ws.fill_(0xAB)
        wsa.fill_(0xCD)

    scrub()
    step()
    torch.cuda.synchronize()
    ref = results()
    assert ops.spec_verify_attn_device_status(ws) == 0

    g = torch.cuda.CUDAGraph()
    scrub()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        scrub()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = results()
        for name, a, b in zip(("out", "target_argmax", "accept_len", "path", "tokens", "new_len", "K", "V"),
                              ref, got):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        note(f"[gpu] replay {rep} ok")
