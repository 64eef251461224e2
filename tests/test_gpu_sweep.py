"""Randomised sweeps of the whole path against the oracle, stopping at the first
mismatch: verify attention with argmax and acceptance, compaction (plain and
fused with acceptance) with the chunked acceptance loop, and stochastic
acceptance of chains and of draft trees, over seeded random batches and both V
page layouts.

The default run is short (SV_SWEEP_BATCHES batches per sweep, default 3, in one
part); longer sweeps run the same tests with more parts and batches:

    SV_SWEEP_PARTS=40 SV_SWEEP_BATCHES=25 python -m pytest tests/test_gpu_sweep.py -m gpu -x -v

Part p draws its batches from its own seed, so every (part, batch) is a fixed
case and a failure names it."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import test_gpu_stochastic as TS
from gpu_util import (DEV, DevCase, accept_compact_fn, assert_attn_close, bf16_dev_to_u16, bf16_out_to_f64,
                      compact_fn, gpu_accept, gpu_attn, i32, note, oracle_attn, u16_to_bf16_dev, v_from_dev,
                      v_to_dev)
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu

PARTS = int(os.environ.get("SV_SWEEP_PARTS", "1"))
BATCHES = int(os.environ.get("SV_SWEEP_BATCHES", "3"))
parts = pytest.mark.parametrize("part", range(PARTS))


def _trees(rng, cs, B):
    trees = []
    for i in range(B):
        nodes = int(rng.integers(1, 65))
        depth = nodes - 1 if nodes < 8 else min(nodes - 1, int(rng.integers(6, 13)))
        trees.append(W.draw_tree(np.random.Generator(np.random.PCG64(cs * 100 + i)), nodes, depth, 4, 4))
    return trees


@parts
def test_sweep_attention_and_acceptance(part):
    """1-8 requests, contexts 0-4000 (some empty), chains of 1-64 tokens or trees
    of 1-64 nodes, 1-8 KV heads, GQA ratio 1-16, head_dim 64 or 128, either V
    layout: attention, argmax and acceptance against the oracle."""
    rng = np.random.default_rng(20_000 + part)
    for c in range(BATCHES):
        B = int(rng.integers(1, 9))
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        d = int(rng.choice([64, 128]))
        vt = bool(rng.integers(0, 2))
        ctx = [int(x) for x in rng.integers(0, 4000, B)]
        if rng.random() < 0.3:
            ctx[int(rng.integers(0, B))] = 0
        cs = 21_000 + 1000 * part + c
        if rng.random() < 0.4:
            case = W.make_custom(cs, context_lens=ctx, tree_parents=_trees(rng, cs, B), hq=g * hkv, hkv=hkv,
                                 d=d, vocab=300)
        else:
            ql = [int(x) for x in rng.integers(1, 65, B)]
            case = W.make_custom(cs, context_lens=ctx, q_lens=ql, hq=g * hkv, hkv=hkv, d=d, vocab=300)
        tag = (f"part {part} batch {c}: B={B} hkv={hkv} G={g} D={d} vt={vt} T={case.total_q} "
               f"tree={case.tree_parent is not None}")
        note(tag)
        dc = DevCase(case, vt)
        out, ws = gpu_attn(dc)
        assert ops.spec_verify_attn_device_status(ws) == 0, tag
        assert_attn_close(bf16_out_to_f64(out), oracle_attn(case), tag)
        (t, acc, path, toks), _ = gpu_accept(dc)
        t_ref = oracle.argmax(case.logits)
        acc_ref, path_ref, toks_ref = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
        assert np.array_equal(t, t_ref) and np.array_equal(acc, acc_ref), tag
        assert np.array_equal(path, path_ref) and np.array_equal(toks, toks_ref), tag


@parts
def test_sweep_compaction_and_chunked_acceptance(part):
    """Random chain and tree batches: two-layer compaction, plain and fused with
    acceptance (whole pools bit-exact against the oracle's copy-based
    compaction), in either V layout; then the chunked acceptance loop with a
    random chunk size ends with the unchunked oracle's acceptance."""
    rng = np.random.default_rng(30_000 + part)
    layers = 2
    for c in range(BATCHES):
        B = int(rng.integers(1, 7))
        hkv = int(rng.choice([1, 2, 8]))
        d = int(rng.choice([64, 128]))
        vt = bool(rng.integers(0, 2))
        vocab = int(rng.choice([50, 1000, 5000]))
        ctx = [int(x) for x in rng.integers(0, 2000, B)]
        cs = 31_000 + 1000 * part + c
        if rng.random() < 0.6:
            case = W.make_custom(cs, context_lens=ctx, tree_parents=_trees(rng, cs, B), hq=2 * hkv, hkv=hkv, d=d,
                                 vocab=vocab, tree_match=(float(rng.uniform(0.5, 1.0)), float(rng.uniform(0.2, 0.9))))
        else:
            ql = [int(x) for x in rng.integers(1, 65, B)]
            case = W.make_custom(cs, context_lens=ctx, q_lens=ql, hq=2 * hkv, hkv=hkv, d=d, vocab=vocab,
                                 match_p=float(rng.uniform(0.5, 1.0)))
        tag = (f"part {part} batch {c}: B={B} hkv={hkv} D={d} vt={vt} T={case.total_q} "
               f"tree={case.tree_parent is not None}")
        note(tag)
        dc = DevCase(case, vt)
        t_ref = oracle.argmax(case.logits)
        acc, path, toks = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
        extra = lambda shp: W.f32_to_bf16_bits(rng.standard_normal(shp).astype(np.float32))
        k_all = np.stack([case.k_cache] + [extra(case.k_cache.shape) for _ in range(layers - 1)])
        v_all = np.stack([case.v_cache] + [extra(case.v_cache.shape) for _ in range(layers - 1)])
        k_ref, v_ref = k_all.copy(), v_all.copy()
        new_ref = oracle.compact(k_ref, v_ref, case.block_tables, case.context_lens, case.cu_q, path, acc,
                                 num_kv_heads=hkv, head_dim=d, page_size=16, num_pages=case.num_pages,
                                 num_layers=layers)
        # plain compaction
        kd, vd = u16_to_bf16_dev(k_all), v_to_dev(v_all, vt)
        new = compact_fn(vt)(kd, vd, dc.bt, dc.ctx, dc.cu, i32(path), i32(acc), num_layers=layers)
        torch.cuda.synchronize()
        assert np.array_equal(new.cpu().numpy(), new_ref), tag
        assert np.array_equal(bf16_dev_to_u16(kd), k_ref) and np.array_equal(v_from_dev(vd, vt), v_ref), tag
        # acceptance and compaction in one launch
        kd, vd = u16_to_bf16_dev(k_all), v_to_dev(v_all, vt)
        ws = torch.zeros(ops.spec_accept_compact_workspace_size(case.batch, case.total_q, case.vocab),
                         dtype=torch.uint8, device=DEV)
        outs = accept_compact_fn(vt)(dc.logits, dc.draft, dc.cu, dc.par, kd, vd, dc.bt, dc.ctx, workspace=ws,
                                     num_layers=layers)
        torch.cuda.synchronize()
        assert ops.spec_accept_device_status(ws) == 0, tag
        t, a2, p2, tk, nw = [x.cpu().numpy() for x in outs]
        assert np.array_equal(t, t_ref) and np.array_equal(a2, acc) and np.array_equal(p2, path), tag
        assert np.array_equal(tk, toks) and np.array_equal(nw, new_ref), tag
        assert np.array_equal(bf16_dev_to_u16(kd), k_ref) and np.array_equal(v_from_dev(vd, vt), v_ref), tag
        # the chunked acceptance loop
        chunk = int(rng.choice([1, 2, 3, 5, 8, 64]))
        T, V = case.total_q, case.vocab
        ta = torch.full((T,), -5, dtype=torch.int32, device=DEV)
        ac = torch.full((B,), -9, dtype=torch.int32, device=DEV)
        pa = torch.full((T,), -9, dtype=torch.int32, device=DEV)
        to = torch.full((T,), -9, dtype=torch.int32, device=DEV)
        wsc = torch.empty(ops.spec_accept_chunk_workspace_size(B, T, V), dtype=torch.uint8, device=DEV)
        begin, cuc = ops.spec_chunk_start(dc.cu, chunk, total_q=T)
        nb, ncu = torch.empty_like(begin), torch.empty_like(cuc)
        # on the device throughout: as many iterations as the longest request needs, no host read
        for _ in range(-(-int(np.diff(case.cu_q).max()) // chunk)):
            ops.spec_accept_chunk(dc.logits, dc.draft, dc.cu, begin, cuc, dc.par, chunk_size=chunk,
                                  target_argmax=ta, accept_len=ac, accepted_path=pa, out_tokens=to,
                                  next_begin=nb, next_cu=ncu, workspace=wsc)
            begin, cuc, nb, ncu = nb, ncu, begin, cuc
        assert ops.spec_accept_device_status(wsc) == 0, tag
        assert cuc.cpu().numpy()[-1] == 0, (tag, chunk)
        assert np.array_equal(ac.cpu().numpy(), acc) and np.array_equal(pa.cpu().numpy(), path), (tag, chunk)
        assert np.array_equal(to.cpu().numpy(), toks), (tag, chunk)


@parts
def test_sweep_stochastic_acceptance(part):
    """Random batches of 1-32 requests, vocabularies 2-32,000, drafts of up to 12
    tokens, temperatures 0.5-2.0: acceptances and draws against the oracle
    (a decision within fp32 rounding of its threshold is not counted)."""
    rng = np.random.default_rng(40_000 + part)
    for c in range(BATCHES):
        B = int(rng.integers(1, 33))
        V = int(rng.choice([2, 7, 100, 1000, 4099, 32000]))
        qmax = int(rng.integers(1, 13))
        temp = float(rng.choice([0.5, 0.7, 1.0, 1.3, 2.0]))
        cu, logits, dprobs, draft, u, w = TS._case(41_000 + 1000 * part + c, B, V, qmax, temp)
        T = int(cu[-1])
        tag = f"part {part} batch {c}: B={B} V={V} qmax={qmax} temperature={temp} T={T}"
        note(tag)
        ws = torch.empty(ops.spec_accept_stochastic_workspace_size(B, T, V), dtype=torch.uint8, device=DEV)
        acc, path, toks = ops.spec_accept_stochastic(
            torch.from_numpy(logits).to(DEV), torch.from_numpy(dprobs).to(DEV), i32(draft),
            torch.from_numpy(u).to(DEV), torch.from_numpy(w).to(DEV), i32(cu), temperature=temp, workspace=ws)
        torch.cuda.synchronize()
        assert ops.spec_accept_stochastic_device_status(ws) == 0, tag
        exact, borderline = TS._compare(cu, logits, dprobs, draft, u, w, temp, acc.cpu().numpy(),
                                        path.cpu().numpy(), toks.cpu().numpy())
        note(f"  draws equal to the oracle's {exact}/{B}, borderline acceptances {borderline}")
        # every draw was checked against the oracle's weights inside _compare; an
        # index may differ only where the draw point lies within 1e-4 of a boundary
        assert borderline <= 1 and exact >= B - 2, (tag, exact, borderline)


@parts
def test_sweep_stochastic_tree_acceptance(part):
    """Random batches of 1-16 draft trees (random, wide, bushy and chain shapes,
    up to 24 nodes), vocabularies 2-32,000, temperatures 0.5-2.0: walks and draws
    against the oracle (a decision within fp32 rounding of its threshold is not
    counted)."""
    rng = np.random.default_rng(50_000 + part)
    for c in range(BATCHES):
        B = int(rng.integers(1, 17))
        V = int(rng.choice([2, 7, 100, 1000, 4099, 32000]))
        qmax = int(rng.integers(1, 25))
        temp = float(rng.choice([0.5, 0.7, 1.0, 1.3, 2.0]))
        shape = str(rng.choice(["random", "wide", "bushy", "chain"]))
        case = TS._stoch_tree_case(51_000 + 1000 * part + c, B, V, qmax, temp, shape)
        tag = f"part {part} batch {c}: B={B} V={V} qmax={qmax} temperature={temp} shape={shape} T={int(case[0][-1])}"
        note(tag)
        (acc, path, toks), st = TS._run_tree(*case, temp)
        assert st == 0, tag
        exact, borderline = TS._compare_tree(*case, temp, acc, path, toks)
        note(f"  draws equal to the oracle's {exact}/{B}, borderline walks {borderline}")
        assert borderline <= 1 and exact >= B - 2, (tag, exact, borderline)
