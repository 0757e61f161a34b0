"""Host-side checks of the C ABI that need no GPU: the library loads, exports every function
include/attnres.h declares, and rejects out-of-contract arguments before touching the device."""
import ctypes
import os
import re

import pytest
import torch

import attention_residuals_amd as A
from attention_residuals_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "attnres.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP = range(6)

# The argument-check tests below pass made-up device addresses. They must never reach a kernel
# launch, so they only run where no GPU is present (the host logic is the same everywhere).
host_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                               reason="uses fake device pointers; host-only check")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attnres_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = A.load()
    decl = declared_functions()
    assert decl == sorted(B.EXPORTS), decl
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = A.load()
    for s in range(6):
        assert lib.attnres_status_str(s)
    assert lib.attnres_status_str(99) == b"unknown status"


def _desc(**kw):
    base = dict(S=4, N=16, D=256, R=256, dtype=torch.bfloat16)
    base.update(kw)
    extra = {k: base.pop(k) for k in list(base) if k not in ("S", "N", "D", "R", "dtype")}
    return B.make_desc(base["S"], base["N"], base["D"], base["R"], base["dtype"], **extra)


def _o32(desc):
    n = ctypes.c_size_t(123)
    st = A.load().attnres_o32_elems(ctypes.byref(desc), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,expect", [
    (dict(S=0), INVALID), (dict(S=65), INVALID), (dict(R=0), INVALID), (dict(R=257), INVALID),
    (dict(N=-1), INVALID), (dict(D=252, R=252), UNSUPPORTED), (dict(D=16392, R=16), UNSUPPORTED),
    (dict(D=12, R=12, dtype=torch.float32), OK), (dict(D=10, R=10, dtype=torch.float32), UNSUPPORTED),
    (dict(D=16384, R=16384, dtype=torch.float32), UNSUPPORTED),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(has_out_weight=True), INVALID), (dict(deterministic=2), INVALID),
    (dict(accumulate_dvalues=2), INVALID), (dict(accumulate_dvalues=1), OK),
])
def test_descriptor_validation(kw, expect):
    st, _ = _o32(_desc(**kw))
    assert st == expect, (kw, st, A.load().attnres_last_error())
    if st != OK:
        assert A.load().attnres_last_error()


def test_forward_workspace_size():
    n = ctypes.c_size_t(0)
    assert A.load().attnres_fwd_workspace_bytes(ctypes.byref(_desc()), ctypes.byref(n)) == OK
    assert n.value == 256
    assert A.load().attnres_fwd_workspace_bytes(ctypes.byref(_desc(S=0)), ctypes.byref(n)) == INVALID


def test_o32_needed_only_when_backward_streams():
    assert _o32(_desc(S=10, N=32768, D=4096, R=4096)) == (OK, 0)
    assert _o32(_desc(S=24, N=16384, D=2048, R=512)) == (OK, 0)
    assert _o32(_desc(S=64, N=8192, D=8192, R=8192, out_norm=True)) == (OK, 8192 * 8192)
    assert _o32(_desc(S=3, N=5, D=64, R=64, out_norm=True)) == (OK, 5 * 64)
    assert _o32(_desc(S=64, N=7, D=8192, R=8192)) == (OK, 7 * 8192)


def _fake(addr):
    return ctypes.c_void_p(addr)


def _call_fwd(desc, src, query=0x10000, norm_w=None, out_w=None, out=0x20000, lse=0x30000,
              rstd=None, o32=None, ws=None, ws_bytes=0):
    lib = A.load()
    return lib.attnres_fwd(ctypes.byref(desc), ctypes.byref(src) if src is not None else None,
                           query, norm_w, out_w, out, lse, rstd, o32, ws, ws_bytes, None)


def _packed(base=0x100000, src_stride=16 * 256, row_stride=256):
    return B.Sources(packed=base, src_stride=src_stride, list=None, row_stride=row_stride)


@host_only
@pytest.mark.parametrize("case,expect", [
    ("null_sources", INVALID), ("both_packed_and_list", INVALID), ("short_row_stride", INVALID),
    ("misaligned_base", ALIGN), ("odd_row_stride", ALIGN), ("null_query", INVALID),
    ("unwanted_norm_w", INVALID), ("missing_rstd", INVALID), ("null_out", INVALID),
    ("misaligned_out", ALIGN), ("out_overlaps_values", INVALID), ("unwanted_o32", INVALID),
    ("workspace_too_small", WORKSPACE), ("workspace_misaligned", WORKSPACE),
    ("workspace_bytes_without_pointer", WORKSPACE),
])
def test_forward_argument_checks(case, expect):
    desc = _desc()
    src = _packed()
    kw = {}
    if case == "null_sources":
        src = None
    elif case == "both_packed_and_list":
        arr = (ctypes.c_void_p * 4)(0x1000, 0x2000, 0x3000, 0x4000)
        src = B.Sources(packed=0x100000, src_stride=4096, list=ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), row_stride=256)
        kw["_keep"] = arr
    elif case == "short_row_stride":
        src = _packed(row_stride=128)
    elif case == "misaligned_base":
        src = _packed(base=0x100002)
    elif case == "odd_row_stride":
        src = _packed(row_stride=260)
    elif case == "null_query":
        kw["query"] = None
    elif case == "unwanted_norm_w":
        kw["norm_w"] = 0x50000
    elif case == "missing_rstd":
        desc = _desc(out_norm=True)
        kw["o32"] = 0x900000
    elif case == "null_out":
        kw["out"] = None
    elif case == "misaligned_out":
        kw["out"] = 0x20008
    elif case == "out_overlaps_values":
        kw["out"] = 0x100000 + 64 * 2
    elif case == "unwanted_o32":
        kw["o32"] = 0x900000
    elif case == "workspace_too_small":
        kw.update(ws=0xA00000, ws_bytes=128)
    elif case == "workspace_misaligned":
        kw.update(ws=0xA00010, ws_bytes=256)
    elif case == "workspace_bytes_without_pointer":
        kw.update(ws=None, ws_bytes=256)
    kw.pop("_keep", None)
    st = _call_fwd(desc, src, **kw)
    assert st == expect, (case, st, A.load().attnres_last_error())


@host_only
def test_backward_argument_checks_before_device():
    lib = A.load()
    desc = _desc(has_norm_weight=True)
    src = _packed()
    dsrc = _packed(base=0x4000000)
    common = dict(query=0x10000, norm_w=0x11000, out_w=None, lse=0x30000, rstd=None, o32=None,
                  dout=0x8000000, dstride=256, dq=0x12000, dw=0x13000, dow=None, ws=0x20000000)

    def call(desc=desc, src=src, dsrc=dsrc, ws_bytes=0, **over):
        a = dict(common)
        a.update(over)
        return lib.attnres_bwd(ctypes.byref(desc), ctypes.byref(src), a["query"], a["norm_w"],
                               a["out_w"], a["lse"], a["rstd"], a["o32"], a["dout"], a["dstride"],
                               ctypes.byref(dsrc), a["dq"], a["dw"], a["dow"], a["ws"], ws_bytes,
                               None)
    assert call(dw=None) == INVALID                       # dw required with the norm weight
    assert call(dsrc=_packed(base=0x100000)) == INVALID   # dvalues alias values
    assert call(dsrc=_packed(base=0x4000000, src_stride=0)) == INVALID  # dvalues overlap
    assert call(dstride=100) == ALIGN
    assert call(dout=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(ws=0x20000010) == ALIGN
    assert call(dq=0x100000 + 512) == INVALID             # dq inside values
    # repeated input sources are allowed (a source read twice): the call gets past every argument
    # check and stops at the device step (no device here; with one, the zero-byte workspace)
    arr = (ctypes.c_void_p * 4)(0x100000, 0x100000, 0x200000, 0x300000)
    lst = B.Sources(packed=None, src_stride=0,
                    list=ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), row_stride=256)
    st = call(src=lst)
    assert st in (HIP, WORKSPACE), (st, lib.attnres_last_error())


def test_python_binding_rejects_bad_dtype():
    with pytest.raises(TypeError):
        B.make_desc(2, 4, 64, 64, torch.float16)


def _multi_status(**kw):
    base = dict(S=4, N=16, D=256, R=256, M=2, dtype=torch.bfloat16)
    base.update(kw)
    extra = {k: base.pop(k) for k in list(base) if k not in ("S", "N", "D", "R", "M", "dtype")}
    layout = extra.pop("layout_code", None)
    d = B.make_multi_desc(base["S"], base["N"], base["D"], base["R"], base["M"], base["dtype"],
                          **extra)
    if layout is not None:
        d.layout = layout
    n = ctypes.c_size_t(0)
    return A.load().attnres_multi_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n))


@pytest.mark.parametrize("kw,expect", [
    (dict(), OK), (dict(M=16), OK), (dict(M=0), INVALID), (dict(M=17), INVALID),
    (dict(layout_code=2), INVALID), (dict(S=0), INVALID), (dict(R=300), INVALID),
    (dict(S=64, D=8192, R=8192), UNSUPPORTED), (dict(S=24, D=4096, R=4096), OK),
    (dict(S=25, D=4096, R=4096), UNSUPPORTED), (dict(accumulate_dvalues=True), OK),
])
def test_multi_descriptor_validation(kw, expect):
    st = _multi_status(**kw)
    assert st == expect, (kw, st, A.load().attnres_last_error())


def _selected_status(**kw):
    base = dict(S=4, N=16, D=256, R=256, E=8, K=2, dtype=torch.bfloat16)
    base.update(kw)
    d = B.make_selected_desc(base["S"], base["N"], base["D"], base["R"], base["E"], base["K"],
                             base["dtype"])
    n = ctypes.c_size_t(0)
    return A.load().attnres_selected_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(n))


@pytest.mark.parametrize("kw,expect", [
    (dict(), OK), (dict(K=16), OK), (dict(K=0), INVALID), (dict(K=17), INVALID),
    (dict(E=0), INVALID), (dict(R=300), INVALID), (dict(R=5), OK),
    (dict(S=24, D=4096, R=4096), OK), (dict(S=12, D=8192, R=8192), OK),
    (dict(S=4, D=8192, R=8192), OK),
    (dict(S=13, D=8192, R=8192), UNSUPPORTED), (dict(D=16384, R=16384), UNSUPPORTED),
    (dict(E=1 << 18, D=4096, R=4096), UNSUPPORTED), (dict(E=1 << 17, D=4096, R=4096), UNSUPPORTED),
    (dict(E=(1 << 17) - 1, D=4096, R=4096), OK),
])
def test_selected_descriptor_validation(kw, expect):
    st = _selected_status(**kw)
    assert st == expect, (kw, st, A.load().attnres_last_error())


@host_only
def test_device_errors_are_reported_as_hip_status():
    # a call that passes every argument check and then fails in the HIP runtime (no device here)
    # returns ATTNRES_ERR_HIP with the runtime's error in the thread's last-error text; the
    # argument checks before it return their own codes
    lib = A.load()
    flag = ctypes.c_int32(7)
    assert lib.attnres_selected_ids_flag(None, 256, 0, ctypes.byref(flag), None) == WORKSPACE
    assert lib.attnres_selected_ids_flag(0x20000000, 128, 0, ctypes.byref(flag), None) == WORKSPACE
    assert lib.attnres_selected_ids_flag(0x20000010, 256, 0, ctypes.byref(flag), None) == WORKSPACE
    assert lib.attnres_selected_ids_flag(0x20000000, 256, 0, None, None) == INVALID
    st = lib.attnres_selected_ids_flag(0x20000000, 256, 1, ctypes.byref(flag), None)
    assert st == HIP, (st, lib.attnres_last_error())
    msg = lib.attnres_last_error().decode()
    assert "id flag" in msg and msg.strip(), msg
    assert flag.value == 7                                # untouched on failure


@host_only
def test_stream_probe_argument_checks():
    lib = A.load()

    def arr(*p):
        return (ctypes.c_void_p * len(p))(*p)
    ins, outs = arr(0x100000, 0x200000), arr(0x300000)

    def call(i=ins, ni=2, o=outs, no=1, rows=16, rb=256, cpt=1, bpc=8):
        return lib.attnres_stream_probe(i, ni, o, no, rows, rb, cpt, bpc, None)
    assert call(i=None) == INVALID
    assert call(ni=0) == INVALID
    assert call(no=129) == INVALID
    assert call(rb=100) == INVALID                                   # not 16-byte rows
    assert call(cpt=3) == INVALID
    assert call(bpc=0) == INVALID
    assert call(i=arr(0x100008, 0x200000)) == ALIGN
    assert call(o=arr(0x100000 + 256)) == INVALID                    # output overlaps an input
    assert call(rows=0) == OK                                        # no rows: nothing to do
