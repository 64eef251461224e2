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


# The two V page layouts of the library: token-major [..., page_size, D] (the
# generator's and the oracle's layout, taken by the plain calls) and transposed
# [..., D, page_size] (the *_vt calls).
LAYOUTS = [False, True]
LAYOUT_IDS = ["v_token_major", "v_transposed"]


def v_to_dev(v, vt):
    """V pages in the generator's (and the oracle's) layout, uint16 [..., page_size, D],
    to the device in the layout of the calls used: as they are, or (vt) with every
    (page, head) block transposed, [..., D, page_size]."""
    return u16_to_bf16_dev(np.ascontiguousarray(np.swapaxes(v, -1, -2)) if vt else v)


def v_from_dev(vd, vt):
    """The inverse of v_to_dev: device V as uint16 [..., page_size, D]."""
    u = bf16_dev_to_u16(vd)
    return np.ascontiguousarray(np.swapaxes(u, -1, -2)) if vt else u


def attn_fn(vt):
    return ops.spec_verify_attn_vt if vt else ops.spec_verify_attn


def attn_run_fn(vt):
    return ops.spec_verify_attn_run_vt if vt else ops.spec_verify_attn_run


def compact_fn(vt):
    return ops.kv_compact_vt if vt else ops.kv_compact


def accept_compact_fn(vt):
    return ops.spec_accept_compact_vt if vt else ops.spec_accept_compact


def chunk_run_fn(vt):
    return ops.spec_verify_attn_chunk_run_vt if vt else ops.spec_verify_attn_chunk_run


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


class DevCase:
    """Device copies of a case's arrays, V in the layout of the calls used (vt:
    the *_vt calls, V page blocks transposed)."""

    def __init__(self, case, vt=False):
        self.case = case
        self.vt = vt
        self.q = u16_to_bf16_dev(case.q)
        if case.k_cache_dev is not None:
            self.k = case.k_cache_dev
            self.v = case.v_cache_dev.transpose(-1, -2).contiguous() if vt else case.v_cache_dev
        else:
            self.k = u16_to_bf16_dev(case.k_cache)
            self.v = v_to_dev(case.v_cache, vt)
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
    note(f"[gpu] spec_verify_attn{'_vt' if dc.vt else ''} {dc.case.name} B={dc.case.batch} T={dc.case.total_q}")
    ws = torch.empty(ops.spec_verify_attn_workspace_size(dc.case.batch, dc.case.total_q,
                                                         dc.case.num_q_heads, dc.case.num_kv_heads,
                                                         dc.case.head_dim),
                     dtype=torch.uint8, device=DEV)
    out = attn_fn(dc.vt)(dc.q, dc.k, dc.v, dc.bt, dc.ctx, dc.cu, dc.par, workspace=ws, **kw)
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


def bf16_out_to_f64(out):
    return bf16_bits_to_f32(bf16_dev_to_u16(out)).astype(np.float64)
