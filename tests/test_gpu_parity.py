"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Acceptance lengths, accepted paths, emitted tokens, argmaxes and the whole
compacted KV pool must be bit-exact; attention must be within max-abs 2e-2,
mean-abs 2e-3 (and relative L2 1e-2) of the fp64 oracle on unit-scale data.
Attention and compaction run with both V page layouts (token-major, and
transposed through the *_vt calls)."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import pins
from gpu_util import (DEV, LAYOUT_IDS, LAYOUTS, DevCase, assert_attn_close, attn_fn, attn_run_fn,
                      bf16_dev_to_u16, bf16_out_to_f64, compact_fn, gpu_accept, gpu_attn, i32, note,
                      oracle_attn, u16_to_bf16_dev, v_from_dev, v_to_dev)
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu
layouts = pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)


def _tree(seed, nodes=64, depth=6):
    return W.draw_tree(np.random.Generator(np.random.PCG64(seed)), nodes, depth, 4, 4)


SMALL = {
    # ragged chains: L=0, q=1, L not a multiple of 16/32, GQA 4
    "chains_d64_g4": dict(context_lens=[0, 1, 15, 16, 31, 33, 100, 257], q_lens=[1, 5, 2, 7, 3, 1, 8, 5],
                          hq=8, hkv=2, d=64),
    "chains_d128_g4": dict(context_lens=[0, 47, 64, 500, 1000], q_lens=[4, 9, 1, 6, 3], hq=32, hkv=8, d=128),
    # multi-head (G = 1) and G = 8 with 9 tokens (72 rows -> three row tiles)
    "chains_d128_g1": dict(context_lens=[5, 77], q_lens=[6, 2], hq=4, hkv=4, d=128),
    "chains_d128_g8": dict(context_lens=[130, 3, 999], q_lens=[9, 9, 4], hq=64, hkv=8, d=128),
    # trees
    "trees_small_d64": dict(context_lens=[0, 17], tree_parents=[pins.SMALL_TREES[0], pins.SMALL_TREES[1]],
                            hq=8, hkv=2, d=64),
    "trees_64_d128_g8": dict(context_lens=[300, 0], tree_parents=[_tree(1), _tree(2, nodes=40, depth=9)],
                             hq=64, hkv=8, d=128),
    "tree_chainlike_64": dict(context_lens=[33], tree_parents=[np.arange(-1, 63, dtype=np.int32)],
                              hq=16, hkv=8, d=128),
    # the widest head groups the library accepts: G = 32 and G = 64 query heads per KV head
    "chains_d128_g32": dict(context_lens=[70, 0, 517], q_lens=[9, 3, 1], hq=64, hkv=2, d=128),
    "chains_d64_g64": dict(context_lens=[31, 400], q_lens=[2, 5], hq=64, hkv=1, d=64),
    "trees_d128_g64": dict(context_lens=[129, 6], tree_parents=[_tree(3, nodes=20, depth=4), pins.SMALL_TREES[1]],
                           hq=64, hkv=1, d=128),
}


@layouts
@pytest.mark.parametrize("name", list(SMALL))
def test_attn_small_cases(name, vt):
    case = W.make_custom(100 + list(SMALL).index(name), **SMALL[name])
    dc = DevCase(case, vt)
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) == 0
    assert_attn_close(bf16_out_to_f64(out), oracle_attn(case), name)


@layouts
@pytest.mark.parametrize("name", ["tiny_chain", "llama31_8b_chain", "llama3_70b_tree"])
@pytest.mark.parametrize("unit", [True, False], ids=["unit_scale", "config_scale"])
def test_attn_config_full(name, unit, vt):
    case = W.make_case(name, unit_scale=unit)
    dc = DevCase(case, vt)
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) == 0
    got = bf16_out_to_f64(out)
    ref = oracle_attn(case)
    if unit:
        assert_attn_close(got, ref, name)
    else:
        # config-scale outputs are ~1e-2; the same relative accuracy is required
        scale = np.abs(ref).max()
        assert_attn_close(got / scale, ref / scale, name + " (normalised)")


@layouts
@pytest.mark.parametrize("name", ["qwen3_8b_ragged", "llama3_70b_b256"])
def test_attn_config_full_size_all_requests(name, vt):
    """Full-size batch in the launch configuration the benchmark times, every
    request against the oracle (which runs on all host cores).  The device-drawn
    K/V pool is copied back byte for byte."""
    case = W.make_case(name, unit_scale=True, kv_device=DEV)
    dc = DevCase(case, vt)
    out, ws = gpu_attn(dc)
    assert ops.spec_verify_attn_device_status(ws) == 0
    got = bf16_out_to_f64(out)
    del out
    case.k_cache = bf16_dev_to_u16(dc.k)
    case.v_cache = v_from_dev(dc.v, vt)
    dc.k = dc.v = case.k_cache_dev = case.v_cache_dev = None
    torch.cuda.empty_cache()
    note(f"  oracle on {case.batch} requests, {oracle.set_threads(0)} host threads")
    ref = oracle_attn(case)
    assert_attn_close(got, ref, f"{name} all {case.batch} requests")
    # and per request, so that no request hides behind the batch mean
    for i in range(case.batch):
        r = slice(int(case.cu_q[i]), int(case.cu_q[i + 1]))
        err = np.abs(got[r] - ref[r])
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (name, i, err.max(), err.mean())


@layouts
@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_attn_explicit_softmax_scale(scale, vt):
    """A caller's softmax scale instead of 1/sqrt(D), on chains and a tree."""
    case = W.make_custom(9, context_lens=[300, 17], tree_parents=[_tree(4, nodes=30, depth=5), pins.SMALL_TREES[0]],
                         hq=32, hkv=8, d=128)
    dc = DevCase(case, vt)
    out, ws = gpu_attn(dc, softmax_scale=scale)
    assert ops.spec_verify_attn_device_status(ws) == 0
    ref = oracle.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                             case.cu_q, case.tree_parent, num_q_heads=case.num_q_heads,
                             num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                             page_size=case.page_size, num_pages=case.num_pages, scale=scale)
    assert_attn_close(bf16_out_to_f64(out), ref, f"scale {scale}")
    # the default scale gives a different result here
    assert np.abs(ref - oracle_attn(case)).max() > 1e-2


@layouts
def test_attn_sharp_softmax(vt):
    """Queries scaled x4: attention concentrates on few keys, outputs are O(1)."""
    case = W.make_custom(7, context_lens=[700, 64, 5], q_lens=[4, 8, 2], hq=64, hkv=8, d=128,
                         qkv_scale=1.0)
    case.q = W.f32_to_bf16_bits(W.bf16_bits_to_f32(case.q) * 4.0)
    dc = DevCase(case, vt)
    out, _ = gpu_attn(dc)
    ref = oracle_attn(case)
    assert np.abs(ref).max() > 0.5
    assert_attn_close(bf16_out_to_f64(out), ref, "sharp")


@layouts
def test_attn_chain_equals_degenerate_tree_and_page_permutation(vt):
    """Bit-identical GPU outputs for a chain stated as a tree, and for the same
    logical cache laid out through a different page permutation."""
    case = W.make_custom(8, context_lens=[40, 600, 0], q_lens=[5, 3, 7], hq=32, hkv=8, d=128)
    dc = DevCase(case, vt)
    out1, _ = gpu_attn(dc)
    tp = np.concatenate([np.arange(-1, q - 1, dtype=np.int32) for q in case.q_lens])
    out2 = attn_fn(vt)(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, i32(tp))
    perm = np.random.default_rng(3).permutation(case.num_pages)
    k2 = np.empty_like(case.k_cache)
    v2 = np.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    out3 = attn_fn(vt)(dc.q, u16_to_bf16_dev(k2), v_to_dev(v2, vt),
                       i32(perm[case.block_tables]), dc.ctx, dc.cu, None)
    torch.cuda.synchronize()
    a, b, c = (bf16_dev_to_u16(x) for x in (out1, out2, out3))
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_attn_layouts_agree():
    """The two V page layouts give the same attention: the P.V products sum the
    same terms, only the order of the fp32 accumulation differs (8 keys per
    MFMA k-step in either case), so the outputs agree to bf16 rounding."""
    case = W.make_custom(11, context_lens=[77, 1000, 3], tree_parents=[_tree(12, nodes=40, depth=6),
                                                                       pins.SMALL_TREES[1], np.array([-1], np.int32)],
                         hq=32, hkv=8, d=128)
    a, _ = gpu_attn(DevCase(case, False))
    b, _ = gpu_attn(DevCase(case, True))
    fa, fb = bf16_out_to_f64(a), bf16_out_to_f64(b)
    assert np.abs(fa - fb).max() <= 2 * 2.0 ** -8 * max(np.abs(fa).max(), 1.0)


# ---------------------------------------------------------------------------
# acceptance
# ---------------------------------------------------------------------------
def _check_accept(case, dc=None):
    dc = dc or DevCase(case)
    (t, acc, path, toks), ws = gpu_accept(dc)
    assert ops.spec_accept_device_status(ws) == 0
    logits = case.logits if case.logits is not None else dc.logits.cpu().numpy()
    t_ref = oracle.argmax(logits)
    acc_ref, path_ref, toks_ref = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    assert np.array_equal(t, t_ref)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(path, path_ref)
    assert np.array_equal(toks, toks_ref)
    return acc_ref


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_accept_configs(name):
    dev_logits = DEV if name in ("qwen3_8b_ragged", "llama3_70b_b256") else None
    case = W.make_case(name, kv_device=DEV if dev_logits else None, logits_device=dev_logits)
    acc = _check_accept(case)
    note(f"  {name}: mean accept_len {acc.mean():.3f}")


def test_accept_tree_seeds():
    """Config-3 geometry over many seeds, so accepted depths vary."""
    depths = []
    for seed in range(30, 46):
        case = W.build_case("tree", seed, batch=4, q_lens=[64] * 4, context_lens=[1] * 4,
                            tree_parents=[_tree(seed * 10 + k) for k in range(4)], hq=1, hkv=1, d=64,
                            vocab=128256, logit_sigma=3.0, qkv_scale=1.0, tree_match=(0.8, 0.3))
        depths.extend(_check_accept(case).tolist())
    assert max(depths) >= 4 and min(depths) == 1, depths


def test_accept_exhaustive_small_trees():
    """Every tree with <= 6 nodes x every edge-match pattern, in one batch."""
    parents, drafts, targets = [], [], []
    vocab = 64
    for n in range(1, 7):
        for par in pins.all_trees(n):
            for pattern in itertools.product([0, 1], repeat=n - 1):
                tgt = (np.arange(n) * 7 + 3) % vocab
                d = np.empty(n, np.int32)
                d[0] = 0
                for j in range(1, n):
                    d[j] = tgt[par[j]] if pattern[j - 1] else (tgt[par[j]] + 1) % vocab
                parents.append(par); drafts.append(d); targets.append(tgt)
    T = sum(len(p) for p in parents)
    logits = np.random.default_rng(0).standard_normal((T, vocab)).astype(np.float32)
    tg = np.concatenate(targets)
    logits[np.arange(T), tg] = 10.0
    cu = np.zeros(len(parents) + 1, np.int32)
    cu[1:] = np.cumsum([len(p) for p in parents])
    tp = np.concatenate(parents)
    dr = np.concatenate(drafts)
    res = ops.spec_accept(torch.from_numpy(logits).to(DEV), i32(dr), i32(cu), i32(tp))
    t, acc, path, toks = (r.cpu().numpy() for r in res)
    t_ref = oracle.argmax(logits)
    acc_ref, path_ref, toks_ref = oracle.accept(dr, t_ref, cu, tp)
    assert np.array_equal(t, t_ref)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(path, path_ref)
    assert np.array_equal(toks, toks_ref)


@pytest.mark.parametrize("vocab", [1, 3, 4, 1027, 128256, 151936])
def test_argmax_ties_and_signed_zero(vocab):
    """Planted equal maxima (lowest index must win, also across slice
    boundaries), +-0 maxima, vocabularies not a multiple of 4."""
    rng = np.random.default_rng(vocab)
    T = 12
    x = rng.standard_normal((T, vocab)).astype(np.float32)
    if vocab >= 4:
        for r in range(T):
            a, b = sorted(rng.choice(vocab, size=2, replace=False))
            x[r, a] = x[r, b] = 50.0
        x[0, :] = -1.0
        x[0, vocab - 1] = 0.0
        x[0, vocab // 2] = -0.0
        x[1, :] = 2.5  # all equal -> 0
    cu = np.array([0, T], np.int32)
    dr = np.zeros(T, np.int32)
    res = ops.spec_accept(torch.from_numpy(x).to(DEV), i32(dr), i32(cu), None)
    t = res[0].cpu().numpy()
    assert np.array_equal(t, oracle.argmax(x))
    assert np.array_equal(t, np.argmax(x, axis=1))


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------
@layouts
def test_kv_compact_trees_multilayer(vt):
    """Tree paths (including overlapping moves like [0,2,3]) over 3 layers: the
    whole pool after the GPU move equals the oracle's copy-based compaction."""
    trees = [pins.SMALL_TREES[0], pins.SMALL_TREES[1], np.array([-1, 0, 1, 1, 2], np.int32), _tree(5)]
    case = W.make_custom(9, context_lens=[5, 18, 0, 250], tree_parents=trees, hq=16, hkv=8, d=128)
    paths = [[0, 2, 5], [0, 6, 7, 8], [0, 2, 3], None]
    # the fourth request's path comes from the oracle's own acceptance
    t_ref = oracle.argmax(case.logits)
    acc_o, path_o, _ = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    acc = np.zeros(case.batch, np.int32)
    ap = np.full(case.total_q, -1, np.int32)
    for i, p in enumerate(paths):
        o = case.cu_q[i]
        if p is None:
            p = path_o[o:o + acc_o[i]].tolist()
        acc[i] = len(p)
        ap[o:o + len(p)] = p
    layers = 3
    rng = np.random.default_rng(1)
    k_all = np.stack([case.k_cache] + [W.f32_to_bf16_bits(rng.standard_normal(case.k_cache.shape).astype(np.float32))
                                       for _ in range(layers - 1)])
    v_all = np.stack([case.v_cache] + [W.f32_to_bf16_bits(rng.standard_normal(case.v_cache.shape).astype(np.float32))
                                       for _ in range(layers - 1)])
    kd, vd = u16_to_bf16_dev(k_all), v_to_dev(v_all, vt)
    new = compact_fn(vt)(kd, vd, i32(case.block_tables), i32(case.context_lens), i32(case.cu_q),
                         i32(ap), i32(acc), num_layers=layers)
    torch.cuda.synchronize()
    k_ref, v_ref = k_all.copy(), v_all.copy()
    new_ref = oracle.compact(k_ref, v_ref, case.block_tables, case.context_lens, case.cu_q, ap, acc,
                             num_kv_heads=8, head_dim=128, page_size=16, num_pages=case.num_pages,
                             num_layers=layers)
    assert np.array_equal(new.cpu().numpy(), new_ref)
    assert np.array_equal(bf16_dev_to_u16(kd), k_ref)
    assert np.array_equal(v_from_dev(vd, vt), v_ref)
    assert not np.array_equal(k_ref, k_all)  # something really moved


def test_kv_compact_chain_config_is_noop():
    """Large-batch chain config: after acceptance, compaction moves nothing and
    every request's length grows by its accept length."""
    case = W.make_case("llama3_70b_b256", kv_device=DEV, logits_device=DEV)
    dc = DevCase(case)
    (t, acc, path, toks), _ = gpu_accept(dc)
    k_before = dc.k.clone()
    v_before = dc.v.clone()
    t_ref = oracle.argmax(dc.logits.cpu().numpy())
    acc_ref, path_ref, _ = oracle.accept(case.draft_tokens, t_ref, case.cu_q, None)
    new = ops.kv_compact(dc.k, dc.v, dc.bt, dc.ctx, dc.cu, i32(path_ref), i32(acc_ref))
    torch.cuda.synchronize()
    assert np.array_equal(new.cpu().numpy(), case.context_lens + acc_ref)
    assert torch.equal(dc.k.view(torch.int16), k_before.view(torch.int16))
    assert torch.equal(dc.v.view(torch.int16), v_before.view(torch.int16))


def test_empty_inputs_are_noops():
    q = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((1, 2, 64, 16), dtype=torch.bfloat16, device=DEV)  # V pages transposed
    bt = torch.zeros((0, 1), dtype=torch.int32, device=DEV)
    ctx = torch.zeros(0, dtype=torch.int32, device=DEV)
    cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    ops.spec_verify_attn_vt(q, k, v, bt, ctx, cu, None)
    ops.spec_verify_attn(q, k, k, bt, ctx, cu, None)
    # requests with no verify tokens
    cu2 = i32([0, 0, 0])
    res = ops.spec_accept(torch.zeros((0, 16), device=DEV), torch.zeros(0, dtype=torch.int32, device=DEV),
                          cu2, None)
    torch.cuda.synchronize()
    assert res[1].cpu().tolist() == [0, 0]


@layouts
def test_plan_once_run_per_layer(vt):
    """One plan serves several layers: each run equals the one-shot call bit for bit."""
    case = W.make_custom(10, context_lens=[300, 5, 1200, 64], q_lens=[4, 9, 2, 6], hq=32, hkv=8, d=128)
    dc = DevCase(case, vt)
    ws = torch.empty(ops.spec_verify_attn_workspace_size(case.batch, case.total_q, 32, 8, 128),
                     dtype=torch.uint8, device=DEV)
    ops.spec_verify_attn_plan(dc.ctx, dc.cu, max_blocks_per_seq=case.max_blocks, num_q_heads=32,
                              num_kv_heads=8, head_dim=128, num_pages=case.num_pages,
                              total_q=case.total_q, workspace=ws)
    rng = np.random.default_rng(4)
    for layer in range(3):
        q = u16_to_bf16_dev(W.f32_to_bf16_bits(rng.standard_normal(case.q.shape).astype(np.float32)))
        k = u16_to_bf16_dev(W.f32_to_bf16_bits(rng.standard_normal(case.k_cache.shape).astype(np.float32)))
        v = v_to_dev(W.f32_to_bf16_bits(rng.standard_normal(case.v_cache.shape).astype(np.float32)), vt)
        got = attn_run_fn(vt)(q, k, v, dc.bt, dc.ctx, dc.cu, None, workspace=ws)
        ref = attn_fn(vt)(q, k, v, dc.bt, dc.ctx, dc.cu, None)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), layer
    assert ops.spec_verify_attn_device_status(ws) == 0


def test_binding_rejects_mismatched_shapes():
    """The binding checks the sizes the library cannot see behind device
    pointers and raises before anything is launched."""
    case = W.make_custom(7, context_lens=[40, 9], q_lens=[3, 2], hq=8, hkv=2, d=64)
    dc = DevCase(case)
    with pytest.raises(ValueError):
        ops.spec_verify_attn(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu[:-1], None)
    with pytest.raises(ValueError):
        ops.spec_verify_attn(dc.q, dc.k, dc.v, dc.bt[:1], dc.ctx, dc.cu, None)
    with pytest.raises(ValueError):
        ops.spec_verify_attn(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, i32(np.full(3, -1, np.int32)))
    with pytest.raises(ValueError):
        ops.spec_verify_attn(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, None, num_pages=case.num_pages + 1)
    with pytest.raises(ValueError):
        ops.spec_verify_attn(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, None, out=torch.empty_like(dc.q[:-1]))
    # compaction: more layers than the caches hold would write past them
    path = i32(np.zeros(case.total_q, np.int32))
    acc = i32(np.ones(case.batch, np.int32))
    with pytest.raises(ValueError):
        ops.kv_compact(dc.k, dc.v, dc.bt, dc.ctx, dc.cu, path, acc, num_layers=2)
    with pytest.raises(ValueError):
        ops.spec_accept(dc.logits, dc.draft[:-1], dc.cu)
    # V handed over in the other layout: same size, wrong layout (D != 16 here)
    v_t = dc.v.transpose(-1, -2).contiguous()
    with pytest.raises(ValueError):
        ops.spec_verify_attn(dc.q, dc.k, v_t, dc.bt, dc.ctx, dc.cu, None)
    with pytest.raises(ValueError):
        ops.spec_verify_attn_vt(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, None)
    with pytest.raises(ValueError):
        ops.kv_compact(dc.k, v_t, dc.bt, dc.ctx, dc.cu, path, acc)
    with pytest.raises(ValueError):
        ops.kv_compact_vt(dc.k, dc.v, dc.bt, dc.ctx, dc.cu, path, acc)
    ws = torch.zeros(ops.spec_accept_compact_workspace_size(case.batch, case.total_q, case.vocab),
                     dtype=torch.uint8, device=dc.k.device)
    with pytest.raises(ValueError):
        ops.spec_accept_compact(dc.logits, dc.draft, dc.cu, None, dc.k, v_t, dc.bt, dc.ctx, workspace=ws)
    with pytest.raises(ValueError):
        ops.spec_accept_compact_vt(dc.logits, dc.draft, dc.cu, None, dc.k, dc.v, dc.bt, dc.ctx, workspace=ws)


@layouts
@pytest.mark.parametrize("seed", range(8))
def test_random_shapes(seed, vt):
    """Seeded random batches: 1-8 requests, contexts 0-1500 (some 0), chains of
    1-64 tokens or trees of 1-64 nodes, 1-8 KV heads, GQA ratio 1-16, head_dim
    64 or 128; attention, argmax and acceptance against the oracle."""
    rng = np.random.default_rng(500 + seed)
    for c in range(5):
        B = int(rng.integers(1, 9))
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        d = int(rng.choice([64, 128]))
        ctx = [int(x) for x in rng.integers(0, 1500, B)]
        if rng.random() < 0.3:
            ctx[int(rng.integers(0, B))] = 0
        cs = 3000 + 10 * seed + c
        if rng.random() < 0.4:
            trees = []
            for i in range(B):
                nodes = int(rng.integers(1, 65))
                depth = nodes - 1 if nodes < 8 else min(nodes - 1, int(rng.integers(6, 13)))
                trees.append(W.draw_tree(np.random.Generator(np.random.PCG64(cs * 100 + i)), nodes, depth, 4, 4))
            case = W.make_custom(cs, context_lens=ctx, tree_parents=trees, hq=g * hkv, hkv=hkv, d=d, vocab=300)
        else:
            ql = [int(x) for x in rng.integers(1, 65, B)]
            case = W.make_custom(cs, context_lens=ctx, q_lens=ql, hq=g * hkv, hkv=hkv, d=d, vocab=300)
        tag = f"seed {seed} case {c}: B={B} hkv={hkv} G={g} D={d} T={case.total_q} vt={vt}"
        note(tag)
        dc = DevCase(case, vt)
        out, ws = gpu_attn(dc)
        assert ops.spec_verify_attn_device_status(ws) == 0, tag
        assert_attn_close(bf16_out_to_f64(out), oracle_attn(case), tag)
        _check_accept(case, dc)
