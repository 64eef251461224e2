"""CPU oracle for the speculative-decoding verification step -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product path never does.  The arithmetic lives in the plain
C file next to this one (`oracle.c`, fp64, one function per step, each citing
the page passage it follows).  This wrapper only marshals numpy arrays.

Parity status of each function (what pins it is listed in the tests):
  verify_attn  -- pinned: closed forms, convexity, torch SDPA special case,
                  decode equivalence, brute-force walk of ancestors
  decode_attn  -- pinned: closed forms, SDPA special case
  argmax       -- pinned: numpy.argmax (first occurrence), planted ties, +-0
  accept       -- pinned: brute-force path enumeration, chain closed form
  compact      -- pinned: logical read-back, serial in-place copy, chain no-op,
                  non-idempotence on a path with moves
  accept_chunk_step -- pinned: chain closed form, brute-force alive checks
  stochastic.target_probs -- pinned: torch softmax (fp64), two-logit logistic
                  closed form, -inf logits, shift invariance
  stochastic.accept_request -- pinned: losslessness integral, special cases,
                  inverse CDF by brute force
  budget.sps_at -- pinned: hand-worked interpolation and clamping, numpy.interp
  budget.verify_budget -- pinned: brute force over prefix-closed batches,
                  closed forms
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None
_lib_override = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-fPIC", "-shared", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    LL = ctypes.c_longlong
    D = ctypes.c_double
    lib.oracle_verify_attn.argtypes = [P, P, P, P, I, P, P, P, I, I, I, I, I, I, D, I, I, P]
    lib.oracle_decode_attn.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, D, P]
    lib.oracle_argmax.argtypes = [P, LL, LL, P]
    lib.oracle_accept.argtypes = [P, P, P, P, I, P, P, P]
    lib.oracle_compact.argtypes = [P, P, LL, I, P, I, P, P, P, P, P, I, I, I, I, I]
    lib.oracle_accept_chunk_step.argtypes = [P, P, P, P, P, P, I, I, P, P, P, P, P]
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_set_threads.restype = I
    for f in (lib.oracle_verify_attn, lib.oracle_decode_attn, lib.oracle_argmax,
              lib.oracle_accept, lib.oracle_compact):
        f.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _bind(_LIB)
    return _lib


def set_threads(n: int = 0) -> int:
    """Host threads of the oracle's verify attention (0 keeps the OpenMP
    default, which follows OMP_NUM_THREADS); returns the count now in use."""
    lib = _lib_override or _load()
    return int(lib.oracle_set_threads(int(n)))


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} rejected its input (code {rc})")


def verify_attn(q, k_cache, v_cache, block_tables, context_lens, cu_q, tree_parent, *,
                num_q_heads, num_kv_heads, head_dim, page_size, num_pages, scale=None,
                req_begin=0, req_end=None, out=None):
    """fp64 verify attention; returns out [T, Hq, D] (rows outside the range are 0)."""
    lib = _lib_override or _load()
    q = _c(q, np.uint16); k_cache = _c(k_cache, np.uint16); v_cache = _c(v_cache, np.uint16)
    block_tables = _c(block_tables, np.int32); context_lens = _c(context_lens, np.int32)
    cu_q = _c(cu_q, np.int32); tree_parent = _c(tree_parent, np.int32)
    batch = len(context_lens)
    T = int(cu_q[-1])
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    if req_end is None:
        req_end = batch
    if out is None:
        out = np.zeros((T, num_q_heads, head_dim), dtype=np.float64)
    rc = lib.oracle_verify_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                block_tables.shape[1], _ptr(context_lens), _ptr(cu_q),
                                _ptr(tree_parent), batch, num_q_heads, num_kv_heads, head_dim,
                                page_size, num_pages, float(scale), req_begin, req_end, _ptr(out))
    _check(rc, "oracle_verify_attn")
    return out


def decode_attn(q_row, k_cache, v_cache, block_tables, i, h, pos, *, num_q_heads, num_kv_heads,
                head_dim, page_size, scale=None):
    """fp64 one-token decode: query (request i, head h) at position pos over keys [0, pos]."""
    lib = _lib_override or _load()
    q_row = _c(q_row, np.uint16); k_cache = _c(k_cache, np.uint16); v_cache = _c(v_cache, np.uint16)
    block_tables = _c(block_tables, np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    out = np.zeros(head_dim, dtype=np.float64)
    rc = lib.oracle_decode_attn(_ptr(q_row), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                block_tables.shape[1], i, h, pos, num_q_heads, num_kv_heads,
                                head_dim, page_size, float(scale), _ptr(out))
    _check(rc, "oracle_decode_attn")
    return out


def argmax(logits):
    """Naive row argmax of fp32 logits [T, V] (lowest index wins ties)."""
    lib = _lib_override or _load()
    logits = _c(logits, np.float32)
    rows, vocab = logits.shape
    out = np.empty(rows, dtype=np.int32)
    _check(lib.oracle_argmax(_ptr(logits), rows, vocab, _ptr(out)), "oracle_argmax")
    return out


def accept(draft_tokens, target, cu_q, tree_parent):
    """Greedy acceptance; returns (accept_len [B], accepted_path [T], out_tokens [T])."""
    lib = _lib_override or _load()
    draft_tokens = _c(draft_tokens, np.int32); target = _c(target, np.int32)
    cu_q = _c(cu_q, np.int32); tree_parent = _c(tree_parent, np.int32)
    B = len(cu_q) - 1
    T = int(cu_q[-1])
    acc = np.empty(B, dtype=np.int32)
    path = np.empty(T, dtype=np.int32)
    toks = np.empty(T, dtype=np.int32)
    _check(lib.oracle_accept(_ptr(draft_tokens), _ptr(target), _ptr(cu_q), _ptr(tree_parent), B,
                             _ptr(acc), _ptr(path), _ptr(toks)), "oracle_accept")
    return acc, path, toks


def accept_chunk_step(draft_tokens, target, cu_q, tree_parent, chunk_begin, chunk_len, chunk_size,
                      accept_len, accepted_path, out_tokens):
    """One step of chunked acceptance with early pruning (see oracle_accept_chunk_step).
    Updates accept_len / accepted_path / out_tokens in place for requests that end;
    returns (next_begin [B], next_len [B])."""
    lib = _lib_override or _load()
    draft_tokens = _c(draft_tokens, np.int32); target = _c(target, np.int32)
    cu_q = _c(cu_q, np.int32); tree_parent = _c(tree_parent, np.int32)
    chunk_begin = _c(chunk_begin, np.int32); chunk_len = _c(chunk_len, np.int32)
    for a in (accept_len, accepted_path, out_tokens):
        assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    B = len(cu_q) - 1
    nb = np.empty(B, dtype=np.int32)
    nl = np.empty(B, dtype=np.int32)
    _check(lib.oracle_accept_chunk_step(_ptr(draft_tokens), _ptr(target), _ptr(cu_q), _ptr(tree_parent),
                                        _ptr(chunk_begin), _ptr(chunk_len), B, int(chunk_size),
                                        _ptr(accept_len), _ptr(accepted_path), _ptr(out_tokens),
                                        _ptr(nb), _ptr(nl)), "oracle_accept_chunk_step")
    return nb, nl


def accept_chunked(draft_tokens, target, cu_q, tree_parent, chunk_size, *, hide_unverified=True):
    """The whole chunk loop: first chunk = tokens [0, min(chunk_size, q_i)), then
    accept_chunk_step until no request has rows left.  With hide_unverified, each
    step sees target[] only for the tokens verified so far (the rest set to -2).
    Returns (accept_len, accepted_path, out_tokens, steps) where steps lists the
    (chunk_begin, chunk_len) of every chunk."""
    cu_q = np.asarray(cu_q, dtype=np.int32)
    target = np.asarray(target, dtype=np.int32)
    B = len(cu_q) - 1
    T = int(cu_q[-1])
    q = np.diff(cu_q)
    acc = np.full(B, -9, dtype=np.int32)
    path = np.full(T, -9, dtype=np.int32)
    toks = np.full(T, -9, dtype=np.int32)
    begin = np.zeros(B, dtype=np.int32)
    length = np.minimum(q, chunk_size).astype(np.int32)
    seen = np.zeros(T, dtype=bool)
    steps = []
    while length.sum() > 0:
        if len(steps) > 64:  # every chunk verifies >= 1 new token of <= 64
            raise OracleError("chunk loop makes no progress")
        steps.append((begin.copy(), length.copy()))
        for i in range(B):
            seen[cu_q[i] + begin[i]: cu_q[i] + begin[i] + length[i]] = True
        t = np.where(seen, target, -2).astype(np.int32) if hide_unverified else target
        begin, length = accept_chunk_step(draft_tokens, t, cu_q, tree_parent, begin, length, chunk_size,
                                          acc, path, toks)
    for i in range(B):
        if q[i] == 0:
            acc[i] = 0
    return acc, path, toks, steps


def compact(k_cache, v_cache, block_tables, context_lens, cu_q, accepted_path, accept_len, *,
            num_kv_heads, head_dim, page_size, num_pages, num_layers=1, layer_stride_elems=None):
    """Copy-based compaction IN PLACE on the given uint16 arrays; returns new_context_lens.

    k_cache / v_cache hold `num_layers` pools back to back (layer stride in elements).
    """
    lib = _lib_override or _load()
    assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    block_tables = _c(block_tables, np.int32); context_lens = _c(context_lens, np.int32)
    cu_q = _c(cu_q, np.int32); accepted_path = _c(accepted_path, np.int32)
    accept_len = _c(accept_len, np.int32)
    pool = num_pages * num_kv_heads * page_size * head_dim
    if layer_stride_elems is None:
        layer_stride_elems = pool
    B = len(context_lens)
    new_lens = np.empty(B, dtype=np.int32)
    rc = lib.oracle_compact(_ptr(k_cache), _ptr(v_cache), layer_stride_elems, num_layers,
                            _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(cu_q),
                            _ptr(accepted_path), _ptr(accept_len), _ptr(new_lens), B, num_kv_heads,
                            head_dim, page_size, num_pages)
    _check(rc, "oracle_compact")
    return new_lens


class use_library:
    """Context manager: route every oracle call through another build of oracle.c.

    Used by the tests that plant a mistake in a copy of the oracle source and
    check that the pins catch it.
    """

    def __init__(self, so_path):
        self.lib = _bind(so_path)

    def __enter__(self):
        global _lib_override
        self._prev = _lib_override
        _lib_override = self.lib
        return self

    def __exit__(self, *exc):
        global _lib_override
        _lib_override = self._prev
        return False
