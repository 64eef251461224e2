"""Chunked verification with early pruning (FASER, "Early Token Pruning") on the
GPU, through the C ABI, against the oracle.

Attention over a chunk's rows must give the rows of full verification (the
mask and keys of a verify token do not depend on how the tokens are chunked)
and leave every other row alone; the chunk loop of spec_chunk_start /
spec_accept_chunk must visit exactly the oracle's chunks and end with the
oracle's unchunked acceptance, bit for bit, also when it runs on the device
from start to end (a fixed number of iterations, no host reads, replayed as
one graph)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, LAYOUT_IDS, LAYOUTS, DevCase, assert_attn_close, chunk_run_fn, i32, note, oracle_attn
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd import workloads as W

pytestmark = pytest.mark.gpu


def _tree(seed, nodes=64, depth=6):
    return W.draw_tree(np.random.Generator(np.random.PCG64(seed)), nodes, depth, 4, 4)


CASES = {
    "chains_d128_g4": dict(context_lens=[0, 47, 64, 500, 1000, 3], q_lens=[4, 9, 1, 6, 3, 8], hq=32, hkv=8,
                           d=128, vocab=700, match_p=0.8),
    "chains_d64_g8": dict(context_lens=[130, 3, 999], q_lens=[9, 9, 4], hq=16, hkv=2, d=64, vocab=300,
                          match_p=0.9),
    "trees_d128_g8": dict(context_lens=[300, 0, 77], tree_parents=[_tree(1), _tree(2, 40, 9), _tree(3, 7, 3)],
                          hq=64, hkv=8, d=128, vocab=512, tree_match=(0.8, 0.3)),
}


def _chunk_rows(cu, begin, length):
    rows = [np.arange(cu[i] + begin[i], cu[i] + begin[i] + length[i]) for i in range(len(begin))]
    rows = np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)
    cu_chunk = np.zeros(len(begin) + 1, np.int32)
    cu_chunk[1:] = np.cumsum(length)
    return rows, cu_chunk


SENTINEL = -512.0  # exact in bf16; rows outside a chunk must keep it


def _attn_ws(case):
    return torch.empty(ops.spec_verify_attn_workspace_size(case.batch, case.total_q, case.num_q_heads,
                                                           case.num_kv_heads, case.head_dim),
                       dtype=torch.uint8, device=DEV)


def _chunk_attn_into(dc, b_dev, cu_dev, out, ws):
    case = dc.case
    ops.spec_verify_attn_chunk_plan(dc.ctx, dc.cu, b_dev, cu_dev, total_q=case.total_q,
                                    max_blocks_per_seq=case.block_tables.shape[1],
                                    num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                                    head_dim=case.head_dim, num_pages=case.num_pages, workspace=ws)
    chunk_run_fn(dc.vt)(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, b_dev, cu_dev, dc.par,
                        total_q=case.total_q, out=out, workspace=ws)


def _chunk_attn(dc, begin, length):
    """The chunk's rows, and out [T, Hq, D] after one chunk run (other rows: SENTINEL)."""
    rows, cu_chunk = _chunk_rows(dc.case.cu_q, begin, length)
    ws = _attn_ws(dc.case)
    out = torch.full_like(dc.q, SENTINEL)
    _chunk_attn_into(dc, i32(begin), i32(cu_chunk), out, ws)
    torch.cuda.synchronize()
    return rows, out, ws


@pytest.mark.parametrize("vt", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", list(CASES))
def test_chunk_attention_rows_equal_full_verification(name, seed, vt):
    case = W.make_custom(300 + list(CASES).index(name), **CASES[name])
    dc = DevCase(case, vt)
    ref = oracle_attn(case)
    rng = np.random.default_rng(seed)
    q = np.diff(case.cu_q)
    begin = np.array([rng.integers(0, qi + 1) for qi in q], np.int32)
    length = np.array([rng.integers(0, qi - b + 1) for qi, b in zip(q, begin)], np.int32)
    if seed == 0:  # one chunk per request, the last one: every request's tail
        begin = (q // 2).astype(np.int32)
        length = (q - begin).astype(np.int32)
    note(f"[gpu] chunk attention {name} seed {seed}: begin {begin.tolist()} len {length.tolist()}")
    rows, out, ws = _chunk_attn(dc, begin, length)
    got = out.float().cpu().numpy().astype(np.float64)
    others = np.setdiff1d(np.arange(case.total_q), rows)
    assert np.all(got[others] == SENTINEL), "a row outside the chunk was written"
    if len(rows) == 0:
        return
    assert ops.spec_verify_attn_device_status(ws) == 0
    assert_attn_close(got[rows], ref[rows], f"{name} seed {seed}")


def test_chunk_attention_bad_chunk_sets_status():
    """A chunk that does not lie inside its request is flagged, not read out of range."""
    case = W.make_custom(310, **CASES["chains_d128_g4"])
    dc = DevCase(case)
    q = np.diff(case.cu_q)
    begin = np.zeros(case.batch, np.int32)
    length = np.minimum(q, 2).astype(np.int32)
    begin[1] = q[1] - 1  # begin + length > q for request 1
    rows, out, ws = _chunk_attn(dc, begin, np.where(np.arange(case.batch) == 1, 2, length).astype(np.int32))
    assert ops.spec_verify_attn_device_status(ws) & ops.DEV_BAD_CU_Q


@pytest.mark.parametrize("chunk", [1, 2, 3, 8, 64])
@pytest.mark.parametrize("name", list(CASES))
def test_chunk_loop_ends_with_unchunked_acceptance(name, chunk):
    case = W.make_custom(320 + list(CASES).index(name), **CASES[name])
    dc = DevCase(case)
    B, T, V = case.batch, case.total_q, case.vocab
    t_ref = oracle.argmax(case.logits)
    full = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    o_acc, o_path, o_toks, steps = oracle.accept_chunked(case.draft_tokens, t_ref, case.cu_q,
                                                         case.tree_parent, chunk)
    assert np.array_equal(o_acc, full[0])
    t_arg = torch.full((T,), -5, dtype=torch.int32, device=DEV)
    acc = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    path = torch.full((T,), -9, dtype=torch.int32, device=DEV)
    toks = torch.full((T,), -9, dtype=torch.int32, device=DEV)
    ws = torch.empty(ops.spec_accept_chunk_workspace_size(B, T, V), dtype=torch.uint8, device=DEV)
    begin, cu_chunk = ops.spec_chunk_start(dc.cu, chunk, total_q=T)
    nb = torch.empty_like(begin)
    ncu = torch.empty_like(cu_chunk)
    k = 0
    verified = 0
    while True:
        b_h = begin.cpu().numpy()
        cu_h = cu_chunk.cpu().numpy()
        len_h = np.diff(cu_h)
        if k < len(steps):
            note(f"[gpu] chunk loop {name} c={chunk} step {k}: rows {int(cu_h[-1])}")
            assert np.array_equal(len_h, steps[k][1]), (k, len_h, steps[k][1])
            assert np.array_equal(b_h[len_h > 0], steps[k][0][len_h > 0]), k
        else:
            assert cu_h[-1] == 0, k
        if cu_h[-1] == 0:
            break
        rows, _ = _chunk_rows(case.cu_q, b_h, len_h)
        verified += len(rows)
        ops.spec_accept_chunk(dc.logits, dc.draft, dc.cu, begin, cu_chunk, dc.par, chunk_size=chunk,
                              target_argmax=t_arg, accept_len=acc, accepted_path=path, out_tokens=toks,
                              next_begin=nb, next_cu=ncu, workspace=ws)
        assert ops.spec_accept_device_status(ws) == 0
        begin, cu_chunk, nb, ncu = nb, ncu, begin, cu_chunk
        k += 1
        assert k <= 64
    assert k == len(steps)
    note(f"  verified {verified} of {T} rows in {k} chunks")
    assert np.array_equal(acc.cpu().numpy(), full[0])
    assert np.array_equal(path.cpu().numpy(), full[1])
    assert np.array_equal(toks.cpu().numpy(), full[2])
    seen = t_arg.cpu().numpy()
    assert np.array_equal(seen[seen != -5], t_ref[seen != -5])


@pytest.mark.parametrize("chunk", [1, 3, 8])
@pytest.mark.parametrize("name", list(CASES))
def test_device_resident_chunk_loop(name, chunk):
    """The whole step on the device: ceil(max q / C) iterations of (plan, run, accept) with no host
    read in between, eagerly and as one replayed graph; the result equals the oracle's unchunked
    acceptance, every verified token's attention row equals full verification, and the rows of
    tokens dropped by pruning are never written."""
    case = W.make_custom(330 + list(CASES).index(name), **CASES[name])
    dc = DevCase(case, True)
    B, T, V = case.batch, case.total_q, case.vocab
    ref = oracle_attn(case)
    t_ref = oracle.argmax(case.logits)
    full = oracle.accept(case.draft_tokens, t_ref, case.cu_q, case.tree_parent)
    _, _, _, steps = oracle.accept_chunked(case.draft_tokens, t_ref, case.cu_q, case.tree_parent, chunk)
    verified = np.zeros(T, bool)
    for b, ln in steps:
        for i in range(B):
            verified[case.cu_q[i] + b[i]: case.cu_q[i] + b[i] + ln[i]] = True
    n_iter = -(-int(np.diff(case.cu_q).max()) // chunk)
    ws_a = _attn_ws(case)
    ws_c = torch.empty(ops.spec_accept_chunk_workspace_size(B, T, V), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(dc.q)
    t_arg = torch.empty(T, dtype=torch.int32, device=DEV)
    acc = torch.empty(B, dtype=torch.int32, device=DEV)
    path = torch.empty(T, dtype=torch.int32, device=DEV)
    toks = torch.empty(T, dtype=torch.int32, device=DEV)
    bufs = [(torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B + 1, dtype=torch.int32, device=DEV))
            for _ in range(2)]

    def reset():
        for t, v in ((out, SENTINEL), (t_arg, -5), (acc, -9), (path, -9), (toks, -9)):
            t.fill_(v)

    def step():
        ops.spec_chunk_start(dc.cu, chunk, total_q=T, chunk_begin=bufs[0][0], cu_chunk=bufs[0][1])
        for k in range(n_iter):
            (b, cu), (nb, ncu) = bufs[k % 2], bufs[(k + 1) % 2]
            _chunk_attn_into(dc, b, cu, out, ws_a)
            ops.spec_accept_chunk(dc.logits, dc.draft, dc.cu, b, cu, dc.par, chunk_size=chunk, target_argmax=t_arg,
                                  accept_len=acc, accepted_path=path, out_tokens=toks, next_begin=nb, next_cu=ncu,
                                  workspace=ws_c)

    def check(what):
        torch.cuda.synchronize()
        assert ops.spec_verify_attn_device_status(ws_a) == 0, what
        assert ops.spec_accept_device_status(ws_c) == 0, what
        assert np.array_equal(acc.cpu().numpy(), full[0]), what
        assert np.array_equal(path.cpu().numpy(), full[1]), what
        assert np.array_equal(toks.cpu().numpy(), full[2]), what
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.all(got[~verified] == SENTINEL), what + ": a pruned token's row was written"
        assert_attn_close(got[verified], ref[verified], f"{name} c={chunk} {what}")

    note(f"[gpu] device-resident chunk loop {name} c={chunk}: {n_iter} iterations, {int(verified.sum())} of {T} rows")
    reset()
    step()
    check("eager")
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep_i in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        check(f"replay {rep_i}")
