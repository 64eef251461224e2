"""Thin Python binding of libspecverify.so (ctypes).

Argument marshalling only: every step of the verification path runs in the
HIP kernels behind the C ABI declared in include/spec_verify.h.  torch is used
for device memory and streams.  There is no fallback: if the library is
missing or no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK = 0
SV_ERR_NULL = 1
SV_ERR_SHAPE = 2
SV_ERR_UNSUPPORTED = 3
SV_ERR_WORKSPACE = 4
SV_ERR_ALIAS = 5
SV_ERR_HIP = 6

# device status bits (the *_device_status calls)
SV_DEV_BAD_CU_Q = 0x1
SV_DEV_BAD_CONTEXT = 0x2
SV_DEV_TOO_MANY_TOKENS = 0x4
SV_DEV_BAD_PARENT = 0x8
SV_DEV_BAD_PAGE = 0x10
SV_DEV_TOO_MANY_PAGES = 0x20
SV_DEV_SYNC_TIMEOUT = 0x40
SV_DEV_BAD_TOKEN = 0x80

DEV_BAD_CU_Q = 0x1
DEV_BAD_CONTEXT = 0x2
DEV_TOO_MANY_TOKENS = 0x4
DEV_BAD_PARENT = 0x8
DEV_BAD_PAGE = 0x10
DEV_TOO_MANY_PAGES = 0x20
DEV_SYNC_TIMEOUT = 0x40
DEV_BAD_TOKEN = 0x80

EXPORTED = ["spec_verify_attn_workspace_size", "spec_verify_attn", "spec_verify_attn_vt", "spec_verify_attn_plan",
            "spec_verify_attn_run", "spec_verify_attn_run_vt", "spec_verify_attn_device_status",
            "spec_accept_workspace_size", "spec_accept", "spec_accept_device_status",
            "kv_compact", "kv_compact_vt", "sv_status_string", "sv_last_error",
            "spec_verify_attn_chunk_plan", "spec_verify_attn_chunk_run", "spec_verify_attn_chunk_run_vt",
            "spec_chunk_start", "spec_accept_chunk_workspace_size", "spec_accept_chunk", "spec_verify_budget",
            "spec_accept_compact_workspace_size", "spec_accept_compact", "spec_accept_compact_vt",
            "spec_accept_stochastic_workspace_size", "spec_accept_stochastic", "spec_accept_stochastic_tree",
            "spec_accept_stochastic_device_status", "spec_hbm_read_probe", "spec_verify_attn_noalloc",
            "spec_verify_attn_phase_trace"]

NOALLOC_SCRATCH_BYTES = 40 << 20  # SV_NOALLOC_SCRATCH_BYTES

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status


def load_library():
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or `python -m speculative_decoding_verification_attn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, SZ, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64
    lib.spec_verify_attn_workspace_size.argtypes = [I, I, I, I, I]
    lib.spec_verify_attn_workspace_size.restype = SZ
    for fn in ("spec_verify_attn", "spec_verify_attn_vt", "spec_verify_attn_run", "spec_verify_attn_run_vt"):
        getattr(lib, fn).argtypes = [P, P, P, P, I, P, P, P, P, I, I, I, I, I, I, I, F, P, SZ, P]
        getattr(lib, fn).restype = I
    lib.spec_verify_attn_plan.argtypes = [P, P, I, I, I, I, I, I, I, P, SZ, P]
    lib.spec_verify_attn_plan.restype = I
    lib.spec_verify_attn_device_status.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.spec_verify_attn_device_status.restype = I
    lib.spec_verify_attn_phase_trace.argtypes = [P, SZ, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.spec_verify_attn_phase_trace.restype = I
    lib.spec_accept_workspace_size.argtypes = [I, I, I]
    lib.spec_accept_workspace_size.restype = SZ
    lib.spec_accept.argtypes = [P, I, P, P, P, I, I, P, P, P, P, P, SZ, P]
    lib.spec_accept.restype = I
    lib.spec_accept_device_status.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.spec_accept_device_status.restype = I
    for fn in ("kv_compact", "kv_compact_vt"):
        getattr(lib, fn).argtypes = [P, P, I64, I, P, I, P, P, P, P, P, I, I, I, I, I, I, P]
        getattr(lib, fn).restype = I
    lib.spec_verify_attn_chunk_plan.argtypes = [P, P, I, P, P, I, I, I, I, I, I, P, SZ, P]
    lib.spec_verify_attn_chunk_plan.restype = I
    for fn in ("spec_verify_attn_chunk_run", "spec_verify_attn_chunk_run_vt"):
        getattr(lib, fn).argtypes = [P, P, P, P, I, P, P, I, P, P, P, P, I, I, I, I, I, I, F, P, SZ, P]
        getattr(lib, fn).restype = I
    lib.spec_chunk_start.argtypes = [P, I, I, I, P, P, P]
    lib.spec_chunk_start.restype = I
    lib.spec_accept_chunk_workspace_size.argtypes = [I, I, I]
    lib.spec_accept_chunk_workspace_size.restype = SZ
    lib.spec_accept_chunk.argtypes = [P, I, P, P, P, P, P, I, I, I, P, P, P, P, P, P, P, SZ, P]
    lib.spec_accept_chunk.restype = I
    lib.spec_verify_budget.argtypes = [P, P, I, P, P, I, P, P, ctypes.POINTER(ctypes.c_double)]
    lib.spec_verify_budget.restype = I
    lib.spec_accept_compact_workspace_size.argtypes = [I, I, I]
    lib.spec_accept_compact_workspace_size.restype = SZ
    for fn in ("spec_accept_compact", "spec_accept_compact_vt"):
        getattr(lib, fn).argtypes = [P, I, P, P, P, I, I, P, P, P, P, P, P, I64, I, P, I, P, P, I, I, I, I, P, SZ, P]
        getattr(lib, fn).restype = I
    lib.spec_accept_stochastic_workspace_size.argtypes = [I, I, I]
    lib.spec_accept_stochastic_workspace_size.restype = SZ
    lib.spec_accept_stochastic.argtypes = [P, P, I, F, P, P, P, P, I, I, P, P, P, P, SZ, P]
    lib.spec_accept_stochastic.restype = I
    lib.spec_accept_stochastic_tree.argtypes = [P, P, I, F, P, P, P, P, P, I, I, P, P, P, P, SZ, P]
    lib.spec_accept_stochastic_tree.restype = I
    lib.spec_accept_stochastic_device_status.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.spec_accept_stochastic_device_status.restype = I
    lib.spec_verify_attn_noalloc.argtypes = [P, P, P, P, I, P, P, P, P, I, I, I, I, I, I, I, F, P, P]
    lib.spec_verify_attn_noalloc.restype = I
    lib.spec_hbm_read_probe.argtypes = [P, P, P, I64, I, I64, P, I64, P]
    lib.spec_hbm_read_probe.restype = I
    lib.sv_status_string.argtypes = [I]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_last_error.argtypes = []
    lib.sv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != SV_OK:
        lib = load_library()
        raise SpecVerifyError(rc, lib.sv_last_error().decode() or lib.sv_status_string(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ----------------------------------------------------------------------------
def spec_verify_attn_workspace_size(batch, total_q, num_q_heads, num_kv_heads, head_dim) -> int:
    return int(load_library().spec_verify_attn_workspace_size(batch, total_q, num_q_heads,
                                                              num_kv_heads, head_dim))


def _v_shape(k_shape, vt):
    """V cache shape matching a K cache shape [..., pages, Hkv, 16, D]: the same
    (token-major pages), or each page's block transposed, [..., pages, Hkv, D, 16]
    (the *_vt calls)."""
    k_shape = tuple(k_shape)
    return k_shape[:-2] + (k_shape[-1], k_shape[-2]) if vt else k_shape


def _attn_call(fn, q, k_cache, v_cache, block_tables, context_lens, cu_q, tree_parent, out,
               softmax_scale, workspace, num_pages, stream):
    vt = fn.endswith("_vt")
    lib = load_library()
    _dev(q, torch.bfloat16, "q")
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    _dev(block_tables, torch.int32, "block_tables")
    _dev(context_lens, torch.int32, "context_lens")
    _dev(cu_q, torch.int32, "cu_q")
    _dev(tree_parent, torch.int32, "tree_parent")
    T, Hq, D = q.shape
    pages, Hkv, P, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != _v_shape(k_cache.shape, vt):
        raise ValueError("caches must be K [pages, Hkv, 16, D] and V [pages, Hkv, %s] matching q"
                         % ("D, 16" if vt else "16, D"))
    B = context_lens.shape[0]
    # sizes the library cannot see behind device pointers
    if cu_q.numel() != B + 1 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("cu_q must hold batch+1 entries and block_tables batch rows")
    if tree_parent is not None and tree_parent.numel() != T:
        raise ValueError("tree_parent must hold one entry per verify token")
    if num_pages is not None and not 0 < num_pages <= pages:
        raise ValueError(f"num_pages {num_pages} exceeds the {pages} pages of the caches")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    if workspace is not None and (workspace.device != q.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    if workspace is None:
        workspace = torch.empty(spec_verify_attn_workspace_size(B, T, Hq, Hkv, D),
                                dtype=torch.uint8, device=q.device)
    _check(getattr(lib, fn)(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                            block_tables.shape[1], _ptr(context_lens), _ptr(cu_q), _ptr(tree_parent),
                            _ptr(out), B, T, Hq, Hkv, D, P, pages if num_pages is None else num_pages,
                            float(softmax_scale), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def spec_verify_attn(q, k_cache, v_cache, block_tables, context_lens, cu_q, tree_parent=None,
                     out=None, softmax_scale=0.0, workspace=None, num_pages=None, stream=None):
    """q [T,Hq,D] bf16; k_cache and v_cache [pages,Hkv,16,D] bf16; returns out [T,Hq,D]
    bf16 (plan + run)."""
    return _attn_call("spec_verify_attn", q, k_cache, v_cache, block_tables, context_lens, cu_q,
                      tree_parent, out, softmax_scale, workspace, num_pages, stream)


def spec_verify_attn_vt(q, k_cache, v_cache, block_tables, context_lens, cu_q, tree_parent=None,
                        out=None, softmax_scale=0.0, workspace=None, num_pages=None, stream=None):
    """spec_verify_attn with v_cache [pages,Hkv,D,16] (each page's V block transposed)."""
    return _attn_call("spec_verify_attn_vt", q, k_cache, v_cache, block_tables, context_lens, cu_q,
                      tree_parent, out, softmax_scale, workspace, num_pages, stream)


def spec_verify_attn_run(q, k_cache, v_cache, block_tables, context_lens, cu_q, tree_parent=None,
                         out=None, softmax_scale=0.0, workspace=None, num_pages=None, stream=None):
    """Verify attention with the plan already in `workspace` (see spec_verify_attn_plan)."""
    if workspace is None:
        raise ValueError("spec_verify_attn_run needs the workspace holding the plan")
    return _attn_call("spec_verify_attn_run", q, k_cache, v_cache, block_tables, context_lens, cu_q,
                      tree_parent, out, softmax_scale, workspace, num_pages, stream)


def spec_verify_attn_run_vt(q, k_cache, v_cache, block_tables, context_lens, cu_q, tree_parent=None,
                            out=None, softmax_scale=0.0, workspace=None, num_pages=None, stream=None):
    """spec_verify_attn_run with v_cache [pages,Hkv,D,16] (each page's V block transposed)."""
    if workspace is None:
        raise ValueError("spec_verify_attn_run_vt needs the workspace holding the plan")
    return _attn_call("spec_verify_attn_run_vt", q, k_cache, v_cache, block_tables, context_lens, cu_q,
                      tree_parent, out, softmax_scale, workspace, num_pages, stream)


def spec_verify_attn_noalloc(q, k_cache, v_cache, block_tables, context_lens, cu_q, tree_parent=None, *,
                             out, softmax_scale=0.0, device_status=None, num_pages=None, stream=None):
    """spec_verify_attn on the library's static scratch: no workspace, nothing allocated
    (out, and device_status if wanted, are the caller's).  Returns out."""
    lib = load_library()
    for t, dt, nm in ((q, torch.bfloat16, "q"), (k_cache, torch.bfloat16, "k_cache"),
                      (v_cache, torch.bfloat16, "v_cache"), (out, torch.bfloat16, "out"),
                      (block_tables, torch.int32, "block_tables"), (context_lens, torch.int32, "context_lens"),
                      (cu_q, torch.int32, "cu_q"), (tree_parent, torch.int32, "tree_parent"),
                      (device_status, torch.int32, "device_status")):
        _dev(t, dt, nm)
    T, Hq, D = q.shape
    pages, Hkv, P, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != _v_shape(k_cache.shape, False):
        raise ValueError("caches must be K and V [pages, Hkv, 16, D] matching q")
    B = context_lens.shape[0]
    if cu_q.numel() != B + 1 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("cu_q must hold batch+1 entries and block_tables batch rows")
    if tree_parent is not None and tree_parent.numel() != T:
        raise ValueError("tree_parent must hold one entry per verify token")
    if num_pages is not None and not 0 < num_pages <= pages:
        raise ValueError(f"num_pages {num_pages} exceeds the {pages} pages of the caches")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    if device_status is not None and device_status.numel() < 1:
        raise ValueError("device_status must hold one word")
    _check(lib.spec_verify_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                        block_tables.shape[1], _ptr(context_lens), _ptr(cu_q), _ptr(tree_parent),
                                        _ptr(out), B, T, Hq, Hkv, D, P, pages if num_pages is None else num_pages,
                                        float(softmax_scale), _ptr(device_status), _stream(stream)))
    return out


def spec_verify_attn_plan(context_lens, cu_q, *, max_blocks_per_seq, num_q_heads, num_kv_heads,
                          head_dim, num_pages, total_q, workspace, stream=None):
    """Build the verify-attention plan for this batch into `workspace`."""
    lib = load_library()
    _dev(context_lens, torch.int32, "context_lens")
    _dev(cu_q, torch.int32, "cu_q")
    B = context_lens.shape[0]
    _check(lib.spec_verify_attn_plan(_ptr(context_lens), _ptr(cu_q), int(max_blocks_per_seq), B,
                                     int(total_q), int(num_q_heads), int(num_kv_heads), int(head_dim),
                                     int(num_pages), _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


def spec_verify_attn_device_status(workspace, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(load_library().spec_verify_attn_device_status(_ptr(workspace), ctypes.byref(flags),
                                                         _stream(stream)))
    return int(flags.value)


def spec_verify_attn_phase_trace(clear: bool = True):
    """The attention kernel's phase timeline from the trace build of the
    library (libspecverify_trace.so): a uint64 numpy array of
    [512 ranges, 4 waves, 2048 events], each event (shader-clock time << 8 | code);
    zeroed afterwards if `clear`.  SV_ERR_UNSUPPORTED from the production build."""
    import numpy as np
    lib = load_library()
    total = ctypes.c_size_t(0)
    _check(lib.spec_verify_attn_phase_trace(None, 0, 0, ctypes.byref(total)))
    buf = np.zeros(total.value // 8, dtype=np.uint64)
    _check(lib.spec_verify_attn_phase_trace(buf.ctypes.data, total.value, int(clear), ctypes.byref(total)))
    return buf.reshape(-1, 4, 2048)


def spec_accept_workspace_size(batch, total_q, vocab) -> int:
    return int(load_library().spec_accept_workspace_size(batch, total_q, vocab))


def spec_accept(logits, draft_tokens, cu_q, tree_parent=None, *, target_argmax=None,
                accept_len=None, accepted_path=None, out_tokens=None, workspace=None, stream=None):
    """logits [T,V] fp32 -> (target_argmax [T], accept_len [B], accepted_path [T], out_tokens [T])."""
    lib = load_library()
    _dev(logits, torch.float32, "logits")
    _dev(draft_tokens, torch.int32, "draft_tokens")
    _dev(cu_q, torch.int32, "cu_q")
    _dev(tree_parent, torch.int32, "tree_parent")
    T, V = logits.shape
    B = cu_q.shape[0] - 1
    dev = logits.device
    if draft_tokens.numel() != T or (tree_parent is not None and tree_parent.numel() != T):
        raise ValueError("draft_tokens (and tree_parent) must hold one entry per logits row")
    if target_argmax is None:
        target_argmax = torch.empty(T, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if accepted_path is None:
        accepted_path = torch.empty(T, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(T, dtype=torch.int32, device=dev)
    for t, nm, n in ((target_argmax, "target_argmax", T), (accept_len, "accept_len", B),
                     (accepted_path, "accepted_path", T), (out_tokens, "out_tokens", T)):
        _dev(t, torch.int32, nm)
        if t.numel() != n:
            raise ValueError(f"{nm} must hold {n} entries")
    if workspace is None:
        workspace = torch.empty(spec_accept_workspace_size(B, T, V), dtype=torch.uint8, device=dev)
    _check(lib.spec_accept(_ptr(logits), V, _ptr(draft_tokens), _ptr(cu_q), _ptr(tree_parent), B, T,
                           _ptr(target_argmax), _ptr(accept_len), _ptr(accepted_path),
                           _ptr(out_tokens), _ptr(workspace), workspace.numel(), _stream(stream)))
    return target_argmax, accept_len, accepted_path, out_tokens


def spec_accept_device_status(workspace, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(load_library().spec_accept_device_status(_ptr(workspace), ctypes.byref(flags),
                                                    _stream(stream)))
    return int(flags.value)


def _check_cache_pair(k_cache, v_cache, vt):
    """K pages [..., pages, Hkv, 16, D] and V pages of the same shape, or (vt)
    [..., pages, Hkv, D, 16]: a V tensor in the other layout has the same size
    and would be moved with the wrong strides, so the shapes are compared, not
    only the sizes."""
    ks = tuple(k_cache.shape)
    if len(ks) < 4 or tuple(v_cache.shape) != _v_shape(ks, vt):
        raise ValueError("caches must be K [..., pages, Hkv, 16, D] and V [..., pages, Hkv, %s]"
                         % ("D, 16" if vt else "16, D"))


def kv_compact(k_cache, v_cache, block_tables, context_lens, cu_q, accepted_path, accept_len, *,
               num_layers=1, layer_stride_elems=None, num_kv_heads=None, head_dim=None,
               num_pages=None, new_context_lens=None, stream=None):
    """In-place compaction of every layer.  With num_layers > 1, k_cache and v_cache are
    [layers, pages, Hkv, 16, D] (or flat pools `layer_stride_elems` apart).
    Returns new_context_lens [B]."""
    return _kv_compact_call("kv_compact", k_cache, v_cache, block_tables, context_lens, cu_q, accepted_path,
                            accept_len, num_layers, layer_stride_elems, num_kv_heads, head_dim, num_pages,
                            new_context_lens, stream)


def kv_compact_vt(k_cache, v_cache, block_tables, context_lens, cu_q, accepted_path, accept_len, *,
                  num_layers=1, layer_stride_elems=None, num_kv_heads=None, head_dim=None,
                  num_pages=None, new_context_lens=None, stream=None):
    """kv_compact with v_cache [(layers,) pages, Hkv, D, 16] (each page's V block transposed)."""
    return _kv_compact_call("kv_compact_vt", k_cache, v_cache, block_tables, context_lens, cu_q, accepted_path,
                            accept_len, num_layers, layer_stride_elems, num_kv_heads, head_dim, num_pages,
                            new_context_lens, stream)


def _kv_compact_call(fn, k_cache, v_cache, block_tables, context_lens, cu_q, accepted_path, accept_len,
                     num_layers, layer_stride_elems, num_kv_heads, head_dim, num_pages, new_context_lens, stream):
    lib = load_library()
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    for t, nm in ((block_tables, "block_tables"), (context_lens, "context_lens"), (cu_q, "cu_q"),
                  (accepted_path, "accepted_path"), (accept_len, "accept_len")):
        _dev(t, torch.int32, nm)
    shp = k_cache.shape
    if num_kv_heads is None:
        _check_cache_pair(k_cache, v_cache, fn.endswith("_vt"))
        num_kv_heads, head_dim = shp[-3], shp[-1]
        num_pages = shp[-4]
    elif head_dim is None or num_pages is None:
        raise ValueError("with num_kv_heads given, head_dim and num_pages are needed too")
    if layer_stride_elems is None:
        layer_stride_elems = num_pages * num_kv_heads * 16 * head_dim
    B = context_lens.shape[0]
    T = accepted_path.shape[0]
    # the kernel writes every layer in place: all of them must lie inside both tensors
    need = (int(num_layers) - 1) * int(layer_stride_elems) + int(num_pages) * num_kv_heads * 16 * head_dim
    if num_layers > 0 and (need > k_cache.numel() or v_cache.numel() != k_cache.numel()):
        raise ValueError(f"{num_layers} layers {layer_stride_elems} elements apart do not fit the caches")
    if cu_q.numel() != B + 1 or accept_len.numel() != B or block_tables.dim() != 2 \
            or block_tables.shape[0] != B:
        raise ValueError("cu_q, accept_len and block_tables must match the batch of context_lens")
    if new_context_lens is None:
        new_context_lens = torch.empty(B, dtype=torch.int32, device=k_cache.device)
    _dev(new_context_lens, torch.int32, "new_context_lens")
    _check(getattr(lib, fn)(_ptr(k_cache), _ptr(v_cache), int(layer_stride_elems), int(num_layers),
                          _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(cu_q),
                          _ptr(accepted_path), _ptr(accept_len), _ptr(new_context_lens), B, T,
                          num_kv_heads, head_dim, 16, num_pages, _stream(stream)))
    return new_context_lens


# ----------------------------------------------------------------------------
# Chunked verification with early pruning
def spec_chunk_start(cu_q, chunk_size, *, total_q, chunk_begin=None, cu_chunk=None, stream=None):
    """First chunk of a verify step: chunk_begin [B] = 0, cu_chunk [B+1] packs
    min(chunk_size, q_i) rows per request.  Returns (chunk_begin, cu_chunk)."""
    lib = load_library()
    _dev(cu_q, torch.int32, "cu_q")
    B = cu_q.shape[0] - 1
    dev = cu_q.device
    if chunk_begin is None:
        chunk_begin = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    if cu_chunk is None:
        cu_chunk = torch.empty(B + 1, dtype=torch.int32, device=dev)
    _dev(chunk_begin, torch.int32, "chunk_begin")
    _dev(cu_chunk, torch.int32, "cu_chunk")
    _check(lib.spec_chunk_start(_ptr(cu_q), B, int(total_q), int(chunk_size), _ptr(chunk_begin), _ptr(cu_chunk),
                                _stream(stream)))
    return chunk_begin, cu_chunk


def spec_verify_attn_chunk_plan(context_lens, cu_q, chunk_begin, cu_chunk, *, total_q,
                                max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, num_pages,
                                workspace, stream=None):
    """Plan of verify attention over one chunk's rows into `workspace` (sized for total_q rows);
    the chunk's row count is read on the device."""
    lib = load_library()
    for t, nm in ((context_lens, "context_lens"), (cu_q, "cu_q"), (chunk_begin, "chunk_begin"),
                  (cu_chunk, "cu_chunk")):
        _dev(t, torch.int32, nm)
    B = context_lens.shape[0]
    _check(lib.spec_verify_attn_chunk_plan(_ptr(context_lens), _ptr(cu_q), int(total_q), _ptr(chunk_begin),
                                           _ptr(cu_chunk), int(max_blocks_per_seq), B,
                                           int(num_q_heads), int(num_kv_heads), int(head_dim),
                                           int(num_pages), _ptr(workspace), workspace.numel(),
                                           _stream(stream)))
    return workspace


def spec_verify_attn_chunk_run(q, k_cache, v_cache, block_tables, context_lens, cu_q, chunk_begin,
                               cu_chunk, tree_parent=None, *, total_q, out=None, softmax_scale=0.0,
                               workspace, num_pages=None, stream=None):
    """q, out [T,Hq,D] bf16, one row per verify token of the step: the chunk's rows are read and
    written in place; the plan must be in `workspace` (spec_verify_attn_chunk_plan).  k_cache and
    v_cache [pages,Hkv,16,D]."""
    return _chunk_run_call("spec_verify_attn_chunk_run", q, k_cache, v_cache, block_tables, context_lens, cu_q,
                           chunk_begin, cu_chunk, tree_parent, total_q, out, softmax_scale, workspace, num_pages,
                           stream)


def spec_verify_attn_chunk_run_vt(q, k_cache, v_cache, block_tables, context_lens, cu_q, chunk_begin,
                                  cu_chunk, tree_parent=None, *, total_q, out=None, softmax_scale=0.0,
                                  workspace, num_pages=None, stream=None):
    """spec_verify_attn_chunk_run with v_cache [pages,Hkv,D,16] (each page's V block transposed)."""
    return _chunk_run_call("spec_verify_attn_chunk_run_vt", q, k_cache, v_cache, block_tables, context_lens,
                           cu_q, chunk_begin, cu_chunk, tree_parent, total_q, out, softmax_scale, workspace,
                           num_pages, stream)


def _chunk_run_call(fn, q, k_cache, v_cache, block_tables, context_lens, cu_q, chunk_begin, cu_chunk,
                    tree_parent, total_q, out, softmax_scale, workspace, num_pages, stream):
    lib = load_library()
    vt = fn.endswith("_vt")
    _dev(q, torch.bfloat16, "q")
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    for t, nm in ((block_tables, "block_tables"), (context_lens, "context_lens"), (cu_q, "cu_q"),
                  (chunk_begin, "chunk_begin"), (cu_chunk, "cu_chunk"), (tree_parent, "tree_parent")):
        _dev(t, torch.int32, nm)
    T, Hq, D = q.shape
    if T != total_q:
        raise ValueError("q and out hold one row per verify token of the step (total_q rows)")
    pages, Hkv, P, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != _v_shape(k_cache.shape, vt):
        raise ValueError("caches must be K [pages, Hkv, 16, D] and V [pages, Hkv, %s] matching q"
                         % ("D, 16" if vt else "16, D"))
    B = context_lens.shape[0]
    if cu_q.numel() != B + 1 or cu_chunk.numel() != B + 1 or chunk_begin.numel() < B \
            or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("cu_q, cu_chunk, chunk_begin and block_tables must match the batch of context_lens")
    if tree_parent is not None and tree_parent.numel() != total_q:
        raise ValueError("tree_parent must hold one entry per verify token of the step")
    if num_pages is not None and not 0 < num_pages <= pages:
        raise ValueError(f"num_pages {num_pages} exceeds the {pages} pages of the caches")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    _check(getattr(lib, fn)(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                          block_tables.shape[1], _ptr(context_lens), _ptr(cu_q), int(total_q),
                                          _ptr(chunk_begin), _ptr(cu_chunk), _ptr(tree_parent), _ptr(out),
                                          B, Hq, Hkv, D, P, pages if num_pages is None else num_pages,
                                          float(softmax_scale), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return out


def spec_accept_chunk_workspace_size(batch, total_q, vocab) -> int:
    return int(load_library().spec_accept_chunk_workspace_size(batch, total_q, vocab))


def spec_accept_chunk(logits, draft_tokens, cu_q, chunk_begin, cu_chunk, tree_parent=None, *,
                      chunk_size, target_argmax, accept_len, accepted_path, out_tokens, next_begin,
                      next_cu, workspace, stream=None):
    """Acceptance after one chunk: logits [T,V] fp32, one row per verify token (the chunk's rows are
    read).  Fills the chunk's entries of target_argmax [T]; requests that end here get accept_len /
    accepted_path / out_tokens; next_begin [B] and next_cu [B+1] describe the next chunk (next_cu[B] =
    its rows, 0 once every request has ended)."""
    lib = load_library()
    _dev(logits, torch.float32, "logits")
    for t, nm in ((draft_tokens, "draft_tokens"), (cu_q, "cu_q"), (chunk_begin, "chunk_begin"),
                  (cu_chunk, "cu_chunk"), (tree_parent, "tree_parent"), (target_argmax, "target_argmax"),
                  (accept_len, "accept_len"), (accepted_path, "accepted_path"), (out_tokens, "out_tokens"),
                  (next_begin, "next_begin"), (next_cu, "next_cu")):
        _dev(t, torch.int32, nm)
    TL, V = logits.shape
    B = cu_q.shape[0] - 1
    T = draft_tokens.shape[0]
    if TL != T or any(t.numel() != T for t in (target_argmax, accepted_path, out_tokens)) or \
            (tree_parent is not None and tree_parent.numel() != T) or accept_len.numel() != B or \
            next_cu.numel() != B + 1 or cu_chunk.numel() != B + 1 or chunk_begin.numel() < B or \
            next_begin.numel() < B:
        raise ValueError("chunk acceptance arrays do not match the batch or the step's verify tokens")
    _check(lib.spec_accept_chunk(_ptr(logits), V, _ptr(draft_tokens), _ptr(cu_q), _ptr(tree_parent),
                                 _ptr(chunk_begin), _ptr(cu_chunk), B, T, int(chunk_size),
                                 _ptr(target_argmax), _ptr(accept_len), _ptr(accepted_path),
                                 _ptr(out_tokens), _ptr(next_begin), _ptr(next_cu), _ptr(workspace),
                                 workspace.numel(), _stream(stream)))
    return next_begin, next_cu


# ----------------------------------------------------------------------------
# Verify-budget scheduling (host function; numpy in, numpy out)
def spec_verify_budget(cond_survival, cu_draft, sps_rows, sps_value):
    """Returns (verify_len [B] int32, batch_rows, theta) -- see spec_verify_budget in the header."""
    import numpy as np
    lib = load_library()
    c = np.ascontiguousarray(cond_survival, dtype=np.float32)
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    r = np.ascontiguousarray(sps_rows, dtype=np.float32)
    v = np.ascontiguousarray(sps_value, dtype=np.float32)
    B = len(cu) - 1
    out = np.zeros(max(B, 1), dtype=np.int32)
    rows = ctypes.c_int32(0)
    th = ctypes.c_double(0.0)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(lib.spec_verify_budget(p(c) if c.size else None, p(cu), B, p(r), p(v), len(r), p(out),
                                  ctypes.byref(rows), ctypes.byref(th)))
    return out[:B], int(rows.value), float(th.value)


# ----------------------------------------------------------------------------
# Fused acceptance + compaction
def spec_accept_compact_workspace_size(batch, total_q, vocab) -> int:
    return int(load_library().spec_accept_compact_workspace_size(batch, total_q, vocab))


def spec_accept_compact(logits, draft_tokens, cu_q, tree_parent, k_cache, v_cache, block_tables,
                        context_lens, *, workspace, num_layers=1, layer_stride_elems=None,
                        target_argmax=None, accept_len=None, accepted_path=None, out_tokens=None,
                        new_context_lens=None, stream=None):
    """spec_accept + kv_compact in one launch.  `workspace` (uint8, at least
    spec_accept_compact_workspace_size bytes) must be zero-filled before its first use.
    Returns (target_argmax, accept_len, accepted_path, out_tokens, new_context_lens)."""
    return _accept_compact_call("spec_accept_compact", logits, draft_tokens, cu_q, tree_parent, k_cache, v_cache,
                                block_tables, context_lens, workspace, num_layers, layer_stride_elems,
                                target_argmax, accept_len, accepted_path, out_tokens, new_context_lens, stream)


def spec_accept_compact_vt(logits, draft_tokens, cu_q, tree_parent, k_cache, v_cache, block_tables,
                           context_lens, *, workspace, num_layers=1, layer_stride_elems=None,
                           target_argmax=None, accept_len=None, accepted_path=None, out_tokens=None,
                           new_context_lens=None, stream=None):
    """spec_accept_compact with v_cache [(layers,) pages, Hkv, D, 16] (each page's V block transposed)."""
    return _accept_compact_call("spec_accept_compact_vt", logits, draft_tokens, cu_q, tree_parent, k_cache,
                                v_cache, block_tables, context_lens, workspace, num_layers, layer_stride_elems,
                                target_argmax, accept_len, accepted_path, out_tokens, new_context_lens, stream)


def _accept_compact_call(fn, logits, draft_tokens, cu_q, tree_parent, k_cache, v_cache, block_tables,
                         context_lens, workspace, num_layers, layer_stride_elems, target_argmax, accept_len,
                         accepted_path, out_tokens, new_context_lens, stream):
    lib = load_library()
    _dev(logits, torch.float32, "logits")
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    for t, nm in ((draft_tokens, "draft_tokens"), (cu_q, "cu_q"), (tree_parent, "tree_parent"),
                  (block_tables, "block_tables"), (context_lens, "context_lens")):
        _dev(t, torch.int32, nm)
    T, V = logits.shape
    B = cu_q.shape[0] - 1
    dev = logits.device
    if draft_tokens.numel() != T or (tree_parent is not None and tree_parent.numel() != T):
        raise ValueError("draft_tokens (and tree_parent) must hold one entry per logits row")
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    target_argmax = mk(T) if target_argmax is None else target_argmax
    accept_len = mk(B) if accept_len is None else accept_len
    accepted_path = mk(T) if accepted_path is None else accepted_path
    out_tokens = mk(T) if out_tokens is None else out_tokens
    new_context_lens = mk(B) if new_context_lens is None else new_context_lens
    _check_cache_pair(k_cache, v_cache, fn.endswith("_vt"))
    shp = k_cache.shape
    num_kv_heads, head_dim, num_pages = shp[-3], shp[-1], shp[-4]
    if layer_stride_elems is None:
        layer_stride_elems = num_pages * num_kv_heads * 16 * head_dim
    # the launch moves K/V of every layer in place: all of them must lie inside both tensors
    need = (int(num_layers) - 1) * int(layer_stride_elems) + num_pages * num_kv_heads * 16 * head_dim
    if num_layers > 0 and (need > k_cache.numel() or v_cache.numel() != k_cache.numel()):
        raise ValueError(f"{num_layers} layers {layer_stride_elems} elements apart do not fit the caches")
    if context_lens.numel() != B or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("context_lens and block_tables must match the batch of cu_q")
    _check(getattr(lib, fn)(_ptr(logits), V, _ptr(draft_tokens), _ptr(cu_q), _ptr(tree_parent), B, T,
                                   _ptr(target_argmax), _ptr(accept_len), _ptr(accepted_path), _ptr(out_tokens),
                                   _ptr(k_cache), _ptr(v_cache), int(layer_stride_elems), int(num_layers),
                                   _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                   _ptr(new_context_lens), num_kv_heads, head_dim, 16, num_pages,
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return target_argmax, accept_len, accepted_path, out_tokens, new_context_lens


# ----------------------------------------------------------------------------
# Lossless stochastic acceptance (chains and trees)
def spec_accept_stochastic_workspace_size(batch, total_q, vocab) -> int:
    return int(load_library().spec_accept_stochastic_workspace_size(batch, total_q, vocab))


def spec_accept_stochastic(logits, draft_probs, draft_tokens, uniform_accept, uniform_sample, cu_q, *,
                           temperature=1.0, workspace=None, accept_len=None, accepted_path=None,
                           out_tokens=None, stream=None):
    """Speculative sampling over chains; returns (accept_len [B], accepted_path [T], out_tokens [T])."""
    lib = load_library()
    _dev(logits, torch.float32, "logits")
    _dev(draft_probs, torch.float32, "draft_probs")
    _dev(uniform_accept, torch.float32, "uniform_accept")
    _dev(uniform_sample, torch.float32, "uniform_sample")
    _dev(draft_tokens, torch.int32, "draft_tokens")
    _dev(cu_q, torch.int32, "cu_q")
    T, V = logits.shape
    B = cu_q.shape[0] - 1
    dev = logits.device
    if draft_tokens.numel() != T or uniform_accept.numel() != T or uniform_sample.numel() != B \
            or tuple(draft_probs.shape) != (T, V):
        raise ValueError("draft_tokens, uniform_accept and draft_probs must match the logits rows, "
                         "uniform_sample the batch")
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    accept_len = mk(B) if accept_len is None else accept_len
    accepted_path = mk(T) if accepted_path is None else accepted_path
    out_tokens = mk(T) if out_tokens is None else out_tokens
    if workspace is None:
        workspace = torch.empty(spec_accept_stochastic_workspace_size(B, T, V), dtype=torch.uint8, device=dev)
    _check(lib.spec_accept_stochastic(_ptr(logits), _ptr(draft_probs), V, float(temperature), _ptr(draft_tokens),
                                      _ptr(uniform_accept), _ptr(uniform_sample), _ptr(cu_q), B, T,
                                      _ptr(accept_len), _ptr(accepted_path), _ptr(out_tokens), _ptr(workspace),
                                      workspace.numel(), _stream(stream)))
    return accept_len, accepted_path, out_tokens


def spec_accept_stochastic_tree(logits, draft_probs, draft_tokens, tree_parent, uniform_accept, uniform_sample,
                                cu_q, *, temperature=1.0, workspace=None, accept_len=None, accepted_path=None,
                                out_tokens=None, stream=None):
    """Multi-draft speculative sampling over draft trees (tree_parent int32 [T],
    per request: root -1, else the parent's index within the request); returns
    (accept_len [B], accepted_path [T] node indices, out_tokens [T])."""
    lib = load_library()
    _dev(logits, torch.float32, "logits")
    _dev(draft_probs, torch.float32, "draft_probs")
    _dev(uniform_accept, torch.float32, "uniform_accept")
    _dev(uniform_sample, torch.float32, "uniform_sample")
    _dev(draft_tokens, torch.int32, "draft_tokens")
    _dev(tree_parent, torch.int32, "tree_parent")
    _dev(cu_q, torch.int32, "cu_q")
    T, V = logits.shape
    B = cu_q.shape[0] - 1
    dev = logits.device
    if draft_tokens.numel() != T or tree_parent.numel() != T or uniform_accept.numel() != T \
            or uniform_sample.numel() != B or tuple(draft_probs.shape) != (T, V):
        raise ValueError("draft_tokens, tree_parent, uniform_accept and draft_probs must match the logits rows, "
                         "uniform_sample the batch")
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    accept_len = mk(B) if accept_len is None else accept_len
    accepted_path = mk(T) if accepted_path is None else accepted_path
    out_tokens = mk(T) if out_tokens is None else out_tokens
    if workspace is None:
        workspace = torch.empty(spec_accept_stochastic_workspace_size(B, T, V), dtype=torch.uint8, device=dev)
    _check(lib.spec_accept_stochastic_tree(_ptr(logits), _ptr(draft_probs), V, float(temperature),
                                           _ptr(draft_tokens), _ptr(tree_parent), _ptr(uniform_accept),
                                           _ptr(uniform_sample), _ptr(cu_q), B, T, _ptr(accept_len),
                                           _ptr(accepted_path), _ptr(out_tokens), _ptr(workspace),
                                           workspace.numel(), _stream(stream)))
    return accept_len, accepted_path, out_tokens


def spec_accept_stochastic_device_status(workspace, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(load_library().spec_accept_stochastic_device_status(_ptr(workspace), ctypes.byref(flags),
                                                               _stream(stream)))
    return int(flags.value)


# ----------------------------------------------------------------------------
# HBM read-ceiling probe (a measurement aid beside the verify step)
# ----------------------------------------------------------------------------
PROBE_SINK_WORDS = 131072


def spec_hbm_read_probe(k_cache, v_cache, chunks, *, sink=None, stream=None):
    """Stream the (page, KV head) blocks listed in `chunks` (int32, page * Hkv +
    head) of both caches with the attention kernel's load pattern; returns the
    sink tensor (zeroed here unless given) the lanes write their XOR to."""
    lib = load_library()
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    _dev(chunks, torch.int32, "chunks")
    if k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape[:2]) + (k_cache.shape[3], k_cache.shape[2]):
        raise ValueError("caches must be K [num_pages, Hkv, 16, D] and V [num_pages, Hkv, D, 16]")
    chunk_bytes = k_cache.shape[2] * k_cache.shape[3] * 2
    buffer_chunks = k_cache.shape[0] * k_cache.shape[1]
    if sink is None:
        sink = torch.zeros(PROBE_SINK_WORDS, dtype=torch.int32, device=k_cache.device)
    _check(lib.spec_hbm_read_probe(_ptr(k_cache), _ptr(v_cache), _ptr(chunks), chunks.numel(), chunk_bytes,
                                   buffer_chunks, _ptr(sink), sink.numel(), _stream(stream)))
    return sink
