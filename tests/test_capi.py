"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments with the documented status codes before
any HIP call (so these run without a GPU; no kernel is launched)."""
import ctypes
import functools
import os
import re

import pytest

from speculative_decoding_verification_attn_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def lib():
    return ops.load_library()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("spec_verify_attn", "spec_accept", "kv_compact", "spec_verify_attn_workspace_size",
              "spec_accept_workspace_size", "sv_status_string", "sv_last_error"):
        assert n in names, names


def test_library_exports_every_declared_function(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert sorted(ops.EXPORTED) == declared_functions()


def test_status_strings(lib):
    for code in range(0, 7):
        assert lib.sv_status_string(code)
    assert lib.sv_status_string(99) == b"unknown status"


NULL = None
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation rejects the call first


def attn(lib, fn="spec_verify_attn", **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, mb=4, ctx=FAKE, cu=FAKE, par=NULL, out=ctypes.c_void_p(0x90000000),
                B=2, T=8, Hq=8, Hkv=2, D=64, P=16, pages=10, scale=0.0, ws=ctypes.c_void_p(0x20000000),
                wsb=1 << 40, stream=NULL)
    args.update(kw)
    return getattr(lib, fn)(args["q"], args["k"], args["v"], args["bt"], args["mb"], args["ctx"], args["cu"],
                                args["par"], args["out"], args["B"], args["T"], args["Hq"], args["Hkv"], args["D"],
                                args["P"], args["pages"], args["scale"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("fn", ["spec_verify_attn", "spec_verify_attn_vt", "spec_verify_attn_run",
                                "spec_verify_attn_run_vt"])
def test_verify_attn_validation(lib, fn):
    attn = functools.partial(globals()["attn"], fn=fn)
    assert attn(lib, D=96) == ops.SV_ERR_UNSUPPORTED
    assert attn(lib, P=32) == ops.SV_ERR_UNSUPPORTED
    assert attn(lib, Hq=6, Hkv=4) == ops.SV_ERR_SHAPE
    assert attn(lib, Hq=130, Hkv=2) == ops.SV_ERR_UNSUPPORTED
    assert attn(lib, B=-1) == ops.SV_ERR_SHAPE
    assert attn(lib, T=129) == ops.SV_ERR_SHAPE          # > 64 tokens per request
    assert attn(lib, q=NULL) == ops.SV_ERR_NULL
    assert attn(lib, ws=NULL) == ops.SV_ERR_NULL
    assert attn(lib, mb=0) == ops.SV_ERR_SHAPE
    assert attn(lib, wsb=16) == ops.SV_ERR_WORKSPACE
    assert attn(lib, scale=float("inf")) == ops.SV_ERR_SHAPE
    assert attn(lib, scale=-0.125) == ops.SV_ERR_SHAPE    # the scale is folded into exp2 args
    assert attn(lib, out=FAKE) == ops.SV_ERR_ALIAS       # out overlaps q
    attn(lib, D=96)
    assert b"head_dim" in lib.sv_last_error()
    # empty work: accepted without touching any pointer
    assert attn(lib, B=0, T=0, q=NULL, out=NULL, ws=NULL) == ops.SV_OK
    assert attn(lib, T=0, q=NULL, out=NULL, ws=NULL) == ops.SV_OK


def test_verify_attn_workspace_size(lib):
    s1 = lib.spec_verify_attn_workspace_size(1, 5, 8, 2, 64)
    s2 = lib.spec_verify_attn_workspace_size(256, 1024, 64, 8, 128)
    assert 0 < s1 < s2
    assert lib.spec_verify_attn_workspace_size(1, 5, 7, 2, 64) == 0


def test_accept_validation(lib):
    def call(**kw):
        a = dict(logits=FAKE, V=100, dr=FAKE, cu=FAKE, par=NULL, B=2, T=8, t=ctypes.c_void_p(0x100000),
                 acc=ctypes.c_void_p(0x200000), path=ctypes.c_void_p(0x300000), toks=ctypes.c_void_p(0x400000),
                 ws=FAKE, wsb=1 << 30, stream=NULL)
        a.update(kw)
        return lib.spec_accept(a["logits"], a["V"], a["dr"], a["cu"], a["par"], a["B"], a["T"], a["t"], a["acc"],
                               a["path"], a["toks"], a["ws"], a["wsb"], a["stream"])
    assert call(V=0) == ops.SV_ERR_SHAPE
    assert call(T=200) == ops.SV_ERR_SHAPE
    assert call(logits=NULL) == ops.SV_ERR_NULL
    assert call(wsb=8) == ops.SV_ERR_WORKSPACE
    assert call(path=ctypes.c_void_p(0x100000)) == ops.SV_ERR_ALIAS
    assert call(B=0, T=0) == ops.SV_OK
    assert lib.spec_accept_workspace_size(4, 20, 128256) > 0


@pytest.mark.parametrize("fn", ["kv_compact", "kv_compact_vt"])
def test_compact_validation(lib, fn):
    def call(**kw):
        a = dict(k=FAKE, v=FAKE, stride=10 * 2 * 16 * 64, L=1, bt=FAKE, mb=4, ctx=ctypes.c_void_p(0x100000),
                 cu=FAKE, path=FAKE, acc=FAKE, new=ctypes.c_void_p(0x200000), B=2, T=8, Hkv=2, D=64, P=16,
                 pages=10, stream=NULL)
        a.update(kw)
        return getattr(lib, fn)(a["k"], a["v"], a["stride"], a["L"], a["bt"], a["mb"], a["ctx"], a["cu"], a["path"],
                                a["acc"], a["new"], a["B"], a["T"], a["Hkv"], a["D"], a["P"], a["pages"], a["stream"])
    assert call(D=80) == ops.SV_ERR_UNSUPPORTED
    assert call(P=8) == ops.SV_ERR_UNSUPPORTED
    assert call(new=ctypes.c_void_p(0x100000)) == ops.SV_ERR_ALIAS
    assert call(k=NULL) == ops.SV_ERR_NULL
    assert call(L=2, stride=5) == ops.SV_ERR_SHAPE
    assert call(B=0) == ops.SV_OK


def test_chunk_validation(lib):
    def start(**kw):
        a = dict(cu=FAKE, B=2, T=8, c=3, begin=ctypes.c_void_p(0x100000), cuc=ctypes.c_void_p(0x200000),
                 stream=NULL)
        a.update(kw)
        return lib.spec_chunk_start(a["cu"], a["B"], a["T"], a["c"], a["begin"], a["cuc"], a["stream"])
    assert start(c=0) == ops.SV_ERR_SHAPE
    assert start(T=200) == ops.SV_ERR_SHAPE
    assert start(cuc=NULL) == ops.SV_ERR_NULL
    assert start(cuc=ctypes.c_void_p(0x100004)) == ops.SV_ERR_ALIAS

    def acc(**kw):
        a = dict(logits=FAKE, V=100, dr=FAKE, cu=FAKE, par=NULL, cb=ctypes.c_void_p(0x500000),
                 cuc=ctypes.c_void_p(0x600000), B=2, T=8, c=2, t=ctypes.c_void_p(0x100000),
                 acc=ctypes.c_void_p(0x200000), path=ctypes.c_void_p(0x300000), toks=ctypes.c_void_p(0x400000),
                 nb=ctypes.c_void_p(0x700000), ncu=ctypes.c_void_p(0x800000), ws=FAKE, wsb=1 << 30, stream=NULL)
        a.update(kw)
        return lib.spec_accept_chunk(a["logits"], a["V"], a["dr"], a["cu"], a["par"], a["cb"], a["cuc"], a["B"],
                                     a["T"], a["c"], a["t"], a["acc"], a["path"], a["toks"], a["nb"],
                                     a["ncu"], a["ws"], a["wsb"], a["stream"])
    assert acc(T=-1) == ops.SV_ERR_SHAPE
    assert acc(T=200) == ops.SV_ERR_SHAPE
    assert acc(c=0) == ops.SV_ERR_SHAPE
    assert acc(V=0) == ops.SV_ERR_SHAPE
    assert acc(nb=NULL) == ops.SV_ERR_NULL
    assert acc(logits=NULL) == ops.SV_ERR_NULL
    assert acc(wsb=8) == ops.SV_ERR_WORKSPACE
    assert acc(nb=ctypes.c_void_p(0x500000)) == ops.SV_ERR_ALIAS   # next_begin over chunk_begin
    assert acc(ncu=ctypes.c_void_p(0x600004)) == ops.SV_ERR_ALIAS  # next_cu over cu_chunk
    assert acc(B=0, T=0) == ops.SV_OK
    assert lib.spec_accept_chunk_workspace_size(4, 20, 128256) >= lib.spec_accept_workspace_size(4, 20, 128256)

    def plan(**kw):
        a = dict(ctx=FAKE, cu=FAKE, T=8, cb=FAKE, cuc=FAKE, mb=4, B=2, Hq=8, Hkv=2, D=64, pages=10,
                 ws=FAKE, wsb=1 << 30, stream=NULL)
        a.update(kw)
        return lib.spec_verify_attn_chunk_plan(a["ctx"], a["cu"], a["T"], a["cb"], a["cuc"], a["mb"],
                                               a["B"], a["Hq"], a["Hkv"], a["D"], a["pages"], a["ws"], a["wsb"],
                                               a["stream"])
    assert plan(cb=NULL) == ops.SV_ERR_NULL
    assert plan(T=200) == ops.SV_ERR_SHAPE
    assert plan(D=96) == ops.SV_ERR_UNSUPPORTED
    assert plan(wsb=8) == ops.SV_ERR_WORKSPACE
    assert plan(T=0) == ops.SV_OK


def test_fused_validation(lib):
    def call(**kw):
        a = dict(logits=FAKE, V=100, dr=FAKE, cu=FAKE, par=NULL, B=2, T=8, t=ctypes.c_void_p(0x100000),
                 acc=ctypes.c_void_p(0x200000), path=ctypes.c_void_p(0x300000), toks=ctypes.c_void_p(0x400000),
                 k=FAKE, v=FAKE, stride=10 * 2 * 16 * 64, L=1, bt=FAKE, mb=4, ctx=ctypes.c_void_p(0x500000),
                 new=ctypes.c_void_p(0x600000), Hkv=2, D=64, P=16, pages=10, ws=FAKE, wsb=1 << 30, stream=NULL)
        a.update(kw)
        return lib.spec_accept_compact(a["logits"], a["V"], a["dr"], a["cu"], a["par"], a["B"], a["T"], a["t"],
                                       a["acc"], a["path"], a["toks"], a["k"], a["v"], a["stride"], a["L"],
                                       a["bt"], a["mb"], a["ctx"], a["new"], a["Hkv"], a["D"], a["P"], a["pages"],
                                       a["ws"], a["wsb"], a["stream"])
    assert call(V=0) == ops.SV_ERR_SHAPE
    assert call(D=96) == ops.SV_ERR_UNSUPPORTED
    assert call(logits=NULL) == ops.SV_ERR_NULL
    assert call(bt=NULL) == ops.SV_ERR_NULL
    assert call(wsb=8) == ops.SV_ERR_WORKSPACE
    assert call(new=ctypes.c_void_p(0x500000)) == ops.SV_ERR_ALIAS
    assert call(new=ctypes.c_void_p(0x200004)) == ops.SV_ERR_ALIAS
    assert call(B=0, T=0) == ops.SV_OK
    assert lib.spec_accept_compact_workspace_size(4, 20, 128256) > lib.spec_accept_workspace_size(4, 20, 128256)


@pytest.mark.parametrize("fn", ["spec_accept_stochastic", "spec_accept_stochastic_tree"])
def test_stochastic_validation(lib, fn):
    def call(**kw):
        a = dict(logits=FAKE, dp=FAKE, V=100, temp=1.0, dr=FAKE, par=FAKE, u=FAKE, w=FAKE, cu=FAKE, B=2, T=8,
                 acc=ctypes.c_void_p(0x200000), path=ctypes.c_void_p(0x300000), toks=ctypes.c_void_p(0x400000),
                 ws=FAKE, wsb=1 << 30, stream=NULL)
        a.update(kw)
        head = (a["logits"], a["dp"], a["V"], ctypes.c_float(a["temp"]), a["dr"])
        tail = (a["u"], a["w"], a["cu"], a["B"], a["T"], a["acc"], a["path"], a["toks"], a["ws"], a["wsb"],
                a["stream"])
        if fn == "spec_accept_stochastic_tree":
            return lib.spec_accept_stochastic_tree(*head, a["par"], *tail)
        return lib.spec_accept_stochastic(*head, *tail)
    assert call(V=0) == ops.SV_ERR_SHAPE
    assert call(temp=0.0) == ops.SV_ERR_SHAPE
    assert call(temp=float("inf")) == ops.SV_ERR_SHAPE
    assert call(T=2 * 64 + 1) == ops.SV_ERR_SHAPE
    assert call(dp=NULL) == ops.SV_ERR_NULL
    assert call(w=NULL) == ops.SV_ERR_NULL
    assert call(wsb=8) == ops.SV_ERR_WORKSPACE
    assert call(toks=ctypes.c_void_p(0x300010)) == ops.SV_ERR_ALIAS
    assert call(B=0, T=0) == ops.SV_OK
    if fn == "spec_accept_stochastic_tree":
        assert call(par=NULL) == ops.SV_ERR_NULL
    assert lib.spec_accept_stochastic_workspace_size(4, 20, 1000) >= 4 * 64 * 8


def test_read_probe_validation(lib):
    def call(**kw):
        a = dict(k=FAKE, v=FAKE, ch=FAKE, n=10, cb=4096, nb=100, sink=FAKE, sw=ops.PROBE_SINK_WORDS, stream=NULL)
        a.update(kw)
        return lib.spec_hbm_read_probe(a["k"], a["v"], a["ch"], a["n"], a["cb"], a["nb"], a["sink"], a["sw"],
                                       a["stream"])
    assert call(cb=1024) == ops.SV_ERR_UNSUPPORTED
    assert call(n=-1) == ops.SV_ERR_SHAPE
    assert call(nb=0) == ops.SV_ERR_SHAPE
    assert call(sw=ops.PROBE_SINK_WORDS - 1) == ops.SV_ERR_SHAPE
    assert call(ch=NULL) == ops.SV_ERR_NULL
    assert call(n=0, k=NULL, v=NULL, ch=NULL, sink=NULL) == ops.SV_OK  # nothing to read


def test_cache_pair_layout_check():
    """The binding tells the two V page layouts apart: the plain calls take V
    pages like K, [.., pages, Hkv, 16, D]; the *_vt calls take every page
    block transposed, [.., pages, Hkv, D, 16].  A V of the other layout (same
    size) is refused."""
    import torch
    k = torch.empty((3, 5, 2, 16, 64), dtype=torch.bfloat16)
    vt = torch.empty((3, 5, 2, 64, 16), dtype=torch.bfloat16)
    ops._check_cache_pair(k, vt, True)
    ops._check_cache_pair(k, k.clone(), False)
    ops._check_cache_pair(k[0], torch.empty((5, 2, 64, 16), dtype=torch.bfloat16), True)
    ops._check_cache_pair(k[0], torch.empty((5, 2, 16, 64), dtype=torch.bfloat16), False)
    for bad in ((3, 5, 2, 16, 64), (5, 2, 64, 16), (3, 5, 2, 64, 8)):
        with pytest.raises(ValueError):
            ops._check_cache_pair(k, torch.empty(bad, dtype=torch.bfloat16), True)
    for bad in ((3, 5, 2, 64, 16), (5, 2, 16, 64), (3, 5, 2, 16, 32)):
        with pytest.raises(ValueError):
            ops._check_cache_pair(k, torch.empty(bad, dtype=torch.bfloat16), False)
    with pytest.raises(ValueError):
        ops._check_cache_pair(torch.empty((2, 16, 64), dtype=torch.bfloat16),
                              torch.empty((2, 64, 16), dtype=torch.bfloat16), True)


def test_noalloc_host_checks(lib):
    """spec_verify_attn_noalloc checks its arguments like spec_verify_attn and
    refuses sizes whose workspace exceeds its static scratch, all on the host
    before any HIP call (so this runs without a GPU)."""
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, mb=4, ctx=FAKE, cu=FAKE, par=NULL, out=ctypes.c_void_p(0x90000000),
                 B=2, T=8, Hq=8, Hkv=2, D=64, P=16, pages=10, scale=0.0, status=NULL, stream=NULL)
        a.update(kw)
        return lib.spec_verify_attn_noalloc(a["q"], a["k"], a["v"], a["bt"], a["mb"], a["ctx"], a["cu"], a["par"],
                                            a["out"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["P"], a["pages"],
                                            a["scale"], a["status"], a["stream"])
    assert call(D=96) == ops.SV_ERR_UNSUPPORTED
    assert call(P=32) == ops.SV_ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=4) == ops.SV_ERR_SHAPE
    assert call(q=NULL) == ops.SV_ERR_NULL
    assert call(mb=0) == ops.SV_ERR_SHAPE
    assert call(scale=-1.0) == ops.SV_ERR_SHAPE
    assert call(B=0, T=0, q=NULL, out=NULL) == ops.SV_OK
    big = dict(B=40000, T=40000 * 64, Hq=64, Hkv=8, D=128)
    assert lib.spec_verify_attn_workspace_size(40000, 40000 * 64, 64, 8, 128) > ops.NOALLOC_SCRATCH_BYTES
    assert call(**big) == ops.SV_ERR_WORKSPACE
    assert b"static scratch" in lib.sv_last_error()
    # the 70B batch-256 shape fits
    assert lib.spec_verify_attn_workspace_size(256, 1024, 64, 8, 128) <= ops.NOALLOC_SCRATCH_BYTES
    # the binding's constant is the header's
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                            "spec_verify.h")).read()
    assert "#define SV_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)" in hdr and ops.NOALLOC_SCRATCH_BYTES == 40 << 20


def test_phase_trace_only_in_the_trace_build(lib):
    """The production library answers the phase-trace call with
    SV_ERR_UNSUPPORTED (no HIP call is made); the trace build, when present,
    exports every declared function too."""
    total = ctypes.c_size_t(123)
    assert lib.spec_verify_attn_phase_trace(None, 0, 0, ctypes.byref(total)) == 3  # SV_ERR_UNSUPPORTED
    assert total.value == 0
    from speculative_decoding_verification_attn_amd import build
    if os.path.exists(build.TRACE_LIB):
        tlib = ctypes.CDLL(build.TRACE_LIB)
        for n in declared_functions():
            assert hasattr(tlib, n), n
