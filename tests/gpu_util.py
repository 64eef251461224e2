"""Shared helpers for the GPU parity tests: move a generated case to the device,
run the HIP path through the C ABI, run the oracle on the same bytes, compare.

No expected value here ever comes from the HIP path: the oracle's inputs are
the generator's arrays (or device-drawn K/V copied back byte for byte)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from speculative_decoding_verification_attn_amd import ops
from speculative_decoding_verification_attn_amd.workloads import bf16_bits_to_f32

DEV = "cuda:0"

# Attention tolerance on unit-scale data (stated bound), plus a relative L2
# bound derived from the arithmetic: bf16 rounding of P and of the output each
# contribute about 2^-9 relative error, fp32 accumulation far less.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def u16_to_bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_dev_to_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def v_to_dev(v):
    """V pages in the generator's (and the oracle's) layout, uint16 [..., page_size, D],
    to the device in the library's layout: every (page, head) block transposed,
    [..., D, page_size]."""
    return u16_to_bf16_dev(np.ascontiguousarray(np.swapaxes(v, -1, -2)))


def v_from_dev(vd):
    """The inverse of v_to_dev: device V [..., D, page_size] as uint16 [..., page_size, D]."""
    return np.ascontiguousarray(np.swapaxes(bf16_dev_to_u16(vd), -1, -2))


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


class DevCase:
    """Device copies of a case's arrays."""

    def __init__(self, case):
        self.case = case
        self.q = u16_to_bf16_dev(case.q)
        if case.k_cache_dev is not None:
            self.k = case.k_cache_dev
            self.v = case.v_cache_dev
        else:
            self.k = u16_to_bf16_dev(case.k_cache)
            self.v = v_to_dev(case.v_cache)
        self.bt = i32(case.block_tables)
        self.ctx = i32(case.context_lens)
        self.cu = i32(case.cu_q)
        self.par = None if case.tree_parent is None else i32(case.tree_parent)
        if case.logits_dev is not None:
            self.logits = case.logits_dev
        else:
            self.logits = torch.from_numpy(case.logits).to(DEV) if case.logits is not None else None
        self.draft = i32(case.draft_tokens)


def gpu_attn(dc, **kw):
    note(f"[gpu] spec_verify_attn {dc.case.name} B={dc.case.batch} T={dc.case.total_q}")
    ws = torch.empty(ops.spec_verify_attn_workspace_size(dc.case.batch, dc.case.total_q,
                                                         dc.case.num_q_heads, dc.case.num_kv_heads,
                                                         dc.case.head_dim),
                     dtype=torch.uint8, device=DEV)
    out = ops.spec_verify_attn(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, dc.par, workspace=ws, **kw)
    torch.cuda.synchronize()
    return out, ws


def gpu_accept(dc):
    note(f"[gpu] spec_accept {dc.case.name} B={dc.case.batch} T={dc.case.total_q} V={dc.case.vocab}")
    ws = torch.empty(ops.spec_accept_workspace_size(dc.case.batch, dc.case.total_q, dc.case.vocab),
                     dtype=torch.uint8, device=DEV)
    res = ops.spec_accept(dc.logits, dc.draft, dc.cu, dc.par, workspace=ws)
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in res], ws


def oracle_attn(case, req_begin=0, req_end=None):
    return oracle.verify_attn(case.q, case.k_cache, case.v_cache, case.block_tables,
                              case.context_lens, case.cu_q, case.tree_parent,
                              num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                              head_dim=case.head_dim, page_size=case.page_size,
                              num_pages=case.num_pages, req_begin=req_begin, req_end=req_end)


def assert_attn_close(got, ref, tag=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    note(f"  {tag} max_abs={err.max():.3e} mean_abs={err.mean():.3e} rel_l2={rel:.3e} "
         f"ref_absmax={np.abs(ref).max():.3e}")
    assert np.all(np.isfinite(got)), tag
    assert err.max() <= MAX_ABS, (tag, err.max())
    assert err.mean() <= MEAN_ABS, (tag, err.mean())
    assert rel <= REL_L2, (tag, rel)


def subcase_from_device(dc, reqs):
    """Host copy of a few requests of a case whose K/V live on the device: their
    pages are copied back byte for byte and the block tables renumbered."""
    case = dc.case
    P = case.page_size
    reqs = list(reqs)
    pages = []
    bt_rows = []
    for i in reqs:
        n = (int(case.context_lens[i]) + int(case.q_lens[i]) + P - 1) // P
        row = list(range(len(pages), len(pages) + n))
        pages.extend(int(p) for p in case.block_tables[i, :n])
        bt_rows.append(row)
    idx = torch.tensor(pages, dtype=torch.long, device=DEV)
    k = bf16_dev_to_u16(dc.k.index_select(0, idx))
    v = v_from_dev(dc.v.index_select(0, idx))
    mb = max(len(r) for r in bt_rows)
    bt = np.zeros((len(reqs), mb), np.int32)
    for r, row in enumerate(bt_rows):
        bt[r, :len(row)] = row
    q_lens = case.q_lens[reqs]
    cu = np.zeros(len(reqs) + 1, np.int32)
    cu[1:] = np.cumsum(q_lens)
    rows = np.concatenate([np.arange(case.cu_q[i], case.cu_q[i + 1]) for i in reqs])
    sub = dict(q=case.q[rows], k_cache=k, v_cache=v, block_tables=bt,
               context_lens=case.context_lens[reqs], cu_q=cu,
               tree_parent=None if case.tree_parent is None else case.tree_parent[rows],
               num_pages=len(pages), rows=rows)
    return sub


def oracle_attn_sub(case, sub):
    return oracle.verify_attn(sub["q"], sub["k_cache"], sub["v_cache"], sub["block_tables"],
                              sub["context_lens"], sub["cu_q"], sub["tree_parent"],
                              num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                              head_dim=case.head_dim, page_size=case.page_size,
                              num_pages=sub["num_pages"])


def bf16_out_to_f64(out):
    return bf16_bits_to_f32(bf16_dev_to_u16(out)).astype(np.float64)
