"""Host-only checks of the C-ABI library (no GPU needed): it loads, exports
every function include/fp8lin.h declares, and rejects bad arguments before
touching a device."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8lin.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(fp8_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def f():
    import fp8_tensor_scaled_amd as f
    return f


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fp8_quantize", "fp8_scale_ring_finalize", "fp8_mm", "fp8_mm_ex", "fp8_mm_pair",
              "fp8_linear_fwd",
              "fp8_linear_bwd", "fp8_colsum", "fp8_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(f):
    out = subprocess.run(["nm", "-D", "--defined-only", f.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    assert set(f.EXPORTED_SYMBOLS) == set(declared_functions())


def test_pure_helpers(f):
    lib = f._lib
    # len + 4 rounded up to 32 words, plus 16 x 32 words of fold scratch
    assert lib.fp8_ring_state_floats(16) == 32 + 512
    assert lib.fp8_ring_state_floats(28) == 32 + 512
    assert lib.fp8_ring_state_floats(29) == 64 + 512
    assert lib.fp8_ring_state_floats(0) == 0
    assert lib.fp8_format_max(0) == 448.0 and lib.fp8_format_max(1) == 57344.0
    assert lib.fp8_format_max(7) == 0.0
    assert f.fp8_linear_fwd_workspace(0, 1, 1) == 0
    M, N, K = 2048, 4096, 1024
    assert f.fp8_linear_fwd_workspace(M, N, K) >= 256 + M * K + N * K
    assert f.fp8_linear_fwd_x8_offset(M, N, K) % 256 == 0
    assert f.fp8_linear_fwd_w8_offset(M, N, K) >= f.fp8_linear_fwd_x8_offset(M, N, K) + M * K
    assert f.fp8_linear_bwd_workspace(M, N, K) >= 256 + M * N + M * K + N * K
    # with the caller's codes of x and w the two code regions are not needed
    codes = f.fp8_linear_bwd_workspace_codes(M, N, K)
    assert codes >= 256 + M * N + f.fp8_colsum_workspace(M, N)
    assert codes + M * K + N * K <= f.fp8_linear_bwd_workspace(M, N, K)
    assert f.fp8_linear_bwd_workspace_codes(0, 1, 1) == 0
    assert b"gfx950" in lib.fp8_version()


P = ctypes.c_void_p
FAKE = P(0x1000)  # never dereferenced: validation fails first


def _err(lib):
    return lib.fp8_last_error().decode()


@pytest.mark.parametrize("args,needle", [
    ((None, 10, 0, FAKE, FAKE, None, None, 0, None, None), "x is NULL"),
    ((FAKE, 10, 2, FAKE, FAKE, None, None, 0, None, None), "format"),
    ((FAKE, -1, 0, FAKE, FAKE, None, None, 0, None, None), "numel"),
    ((FAKE, 10, 0, None, None, None, None, 0, None, None), "neither out nor amax_out nor ring"),
    ((FAKE, 10, 0, None, FAKE, None, None, 0, None, None), "scale is NULL"),
    ((FAKE, 10, 0, FAKE, FAKE, None, None, 65, None, None), "margin"),
    ((FAKE, 10, 0, None, None, FAKE, None, 0, FAKE, None), "scale_used needs"),
])
def test_quantize_validation(f, args, needle):
    st = f._lib.fp8_quantize(*args)
    assert st == 1 and needle in _err(f._lib)


def test_quantize_amax_only_and_empty_calls(f):
    """amax_out alone is a valid (measure-only) call; an empty call without
    ring and amax_out does nothing; with amax_out it still launches (the
    output is armed to +0), which without a GPU fails in the device check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert f._lib.fp8_quantize(None, 0, 0, None, None, None, None, 0, None, None) == 0
    assert f._lib.fp8_quantize(None, 0, 0, None, None, FAKE, None, 0, None, None) in (2, 3)
    assert f._lib.fp8_quantize(FAKE, 10, 0, None, None, FAKE, None, 0, None, None) in (2, 3)


@pytest.mark.parametrize("args,needle", [
    ((FAKE, 10, 0, FAKE, FAKE, 4, FAKE, None, 0, None, None), "second fp8 format"),
    ((FAKE, 10, 9, FAKE, FAKE, 1, FAKE, None, 0, None, None), "format"),
    ((FAKE, 10, 0, FAKE, FAKE, 1, None, None, 0, None, None), "out2"),
    ((FAKE, 10, 0, FAKE, None, 1, FAKE, None, 0, None, None), "out2"),
    ((FAKE, 10, 0, None, FAKE, 1, FAKE, None, 0, None, None), "scale"),
    ((None, 10, 0, FAKE, FAKE, 1, FAKE, None, 0, None, None), "NULL"),
    ((FAKE, -1, 0, FAKE, FAKE, 1, FAKE, None, 0, None, None), "numel"),
    ((FAKE, 10, 0, FAKE, FAKE, 1, FAKE, None, 65, None, None), "margin"),
])
def test_quantize2_validation(f, args, needle):
    st = f._lib.fp8_quantize2(*args)
    assert st == 1 and needle in _err(f._lib), _err(f._lib)


@pytest.mark.parametrize("in_type,kw,needle", [
    (3, {}, "input type"),
    (-1, {}, "input type"),
    (1, dict(fmt=7), "format"),
    (2, dict(x=None), "x is NULL"),
    (1, dict(out=None), "neither out nor amax_out nor ring"),
    (2, dict(scale=None), "scale is NULL"),
])
def test_quantize_ex_validation(f, in_type, kw, needle):
    a = dict(x=FAKE, in_type=in_type, numel=10, fmt=0, scale=FAKE, out=FAKE, amax_out=None,
             ring=None, margin=0, used=None, stream=None)
    a.update(kw)
    st = f._lib.fp8_quantize_ex(*a.values())
    assert st == 1 and needle in _err(f._lib), _err(f._lib)


@pytest.mark.parametrize("kw,needle", [
    (dict(fmt=3), "format"),
    (dict(rows=-1), ">= 0"),
    (dict(out_t=None), "NULL"),
    (dict(x=None), "NULL"),
    (dict(scale=None), "scale is NULL"),
    (dict(out=FAKE), "overlap"),
    (dict(margin=99), "margin"),
])
def test_quantize_t_validation(f, kw, needle):
    a = dict(x=FAKE, rows=64, cols=64, fmt=0, scale=FAKE, out=None, out_t=FAKE, ring=None,
             margin=0, used=None, stream=None)
    a.update(kw)
    st = f._lib.fp8_quantize_t(*a.values())
    assert st == 1 and needle in _err(f._lib), _err(f._lib)


def test_quantize2_empty_without_ring_is_a_noop(f):
    assert f._lib.fp8_quantize2(None, 0, 0, None, None, 1, None, None, 0, None, None) == 0


def qc(lib, **kw):
    a = dict(g=FAKE, m=64, n=64, fmt=0, scale=FAKE, out=FAKE, ring=None, margin=0, used=None,
             db=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.fp8_quantize_colsum(*a.values())


@pytest.mark.parametrize("kw,needle", [
    (dict(fmt=3), "format"),
    (dict(m=0), ">= 1"),
    (dict(g=None), "NULL"),
    (dict(db=None), "NULL"),
    (dict(scale=None), "NULL"),
    (dict(ws=None), "NULL"),
    (dict(ws_bytes=4), "workspace"),
    (dict(margin=-1), "margin"),
])
def test_quantize_colsum_validation(f, kw, needle):
    st = qc(f._lib, **kw)
    assert st == 1 and needle in _err(f._lib), _err(f._lib)


def test_ring_validation(f):
    lib = f._lib
    r = f._RingC(0x1000, 16, 16, 0, 0)
    st = lib.fp8_quantize(FAKE, 10, 0, None, None, None, ctypes.byref(r), 0, None, None)
    assert st == 1 and "idx" in _err(lib)
    r = f._RingC(0x1000, 0, 0, 0, 0)
    st = lib.fp8_scale_ring_finalize(ctypes.byref(r), 0, FAKE, 0, None)
    assert st == 1 and "len" in _err(lib)
    r = f._RingC(None, 4, 0, 0, 0)
    st = lib.fp8_scale_ring_finalize(ctypes.byref(r), 0, FAKE, 0, None)
    assert st == 1 and "state" in _err(lib)


def mm(lib, **kw):
    a = dict(a=FAKE, b=FAKE, fmt=0, ta=0, tb=1, m=64, n=64, k=64, lda=64, ldb=64, batch=1,
             sta=0, stb=0, sa=FAKE, sb=FAKE, bias=None, out=FAKE, stream=None)
    a.update(kw)
    return lib.fp8_mm(*a.values())


@pytest.mark.parametrize("kw,needle", [
    (dict(fmt=5), "format"),
    (dict(a=None), "NULL"),
    (dict(sa=None), "NULL"),
    (dict(ta=2), "trans"),
    (dict(k=0), ">= 1"),
    (dict(batch=0), "batch"),
    (dict(batch=70000), "batch"),
    (dict(lda=32), "lda"),
    (dict(tb=0, ldb=63), "ldb"),
    (dict(batch=2, sta=-1), "stride"),
])
def test_mm_validation(f, kw, needle):
    st = mm(f._lib, **kw)
    assert st == 1 and needle in _err(f._lib), _err(f._lib)


def mm_ex(lib, **kw):
    a = dict(a=FAKE, b=FAKE, fmt=0, ta=0, tb=1, m=64, n=64, k=64, lda=64, ldb=64, batch=1,
             sta=0, stb=0, sa=FAKE, sb=FAKE, bias=None, bias_scale=None, out_type=1,
             out_scale=FAKE, out=FAKE, stream=None)
    a.update(kw)
    return lib.fp8_mm_ex(*a.values())


@pytest.mark.parametrize("kw,needle", [
    (dict(out_type=3), "output type"),
    (dict(out_type=-1), "output type"),
    (dict(out_type=0), "out_scale given for a bf16 output"),
    (dict(out_type=2, out_scale=None), "needs out_scale"),
    (dict(bias_scale=FAKE), "bias_scale without a bias"),
    (dict(fmt=5), "fp8_mm_ex: unsupported fp8 format"),
    (dict(out=None), "NULL"),
    (dict(lda=32), "lda"),
])
def test_mm_ex_validation(f, kw, needle):
    st = mm_ex(f._lib, **kw)
    assert st == 1 and needle in _err(f._lib), _err(f._lib)


def test_mm_ex_valid_call_without_gpu_reports_hip_error(f):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert mm_ex(f._lib, bias=FAKE, bias_scale=FAKE) in (2, 3)
    assert mm_ex(f._lib, out_type=0, out_scale=None) in (2, 3)


def mm_args(f, **kw):
    a = dict(a=FAKE, b=FAKE, fmt=0, trans_a=0, trans_b=0, reserved=0, m=4096, n=4096, k=4096,
             lda=4096, ldb=4096, batch=1, stride_a=0, stride_b=0, scale_a=FAKE, scale_b=FAKE,
             bias=None, out=FAKE)
    a.update(kw)
    return f._MmArgs(**a)


def test_mm_args_layout(f):
    """The binding's struct matches fp8_mm_args_t: pointers, three int32
    flags and a reserved word, eight int64, four pointers (128 bytes)."""
    A = f._MmArgs
    assert ctypes.sizeof(A) == 128
    assert (A.fmt.offset, A.trans_a.offset, A.m.offset, A.stride_b.offset,
            A.scale_a.offset, A.out.offset) == (16, 20, 32, 88, 96, 120)
    text = open(HEADER).read()
    body = text[text.index("typedef struct fp8_mm_args {"):text.index("} fp8_mm_args_t;")]
    fields = re.findall(r"\b(\w+)(?:,|;)", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == [n for n, _ in A._fields_]


@pytest.mark.parametrize("which,kw,needle", [
    (0, dict(fmt=5), "(problem 0): unsupported fp8 format"),
    (1, dict(trans_a=2), "(problem 1): trans"),
    (0, dict(lda=100), "(problem 0): lda"),
    (1, dict(m=0), "(problem 1): m, n, k"),
    (1, dict(out=None), "(problem 1): NULL"),
])
def test_mm_pair_validation(f, which, kw, needle):
    p = [mm_args(f, out=FAKE), mm_args(f, trans_a=1, out=P(FAKE.value + (1 << 30)))]
    p[which] = mm_args(f, **{**dict(out=p[which].out, trans_a=p[which].trans_a), **kw})
    st = f._lib.fp8_mm_pair(ctypes.byref(p[0]), ctypes.byref(p[1]), None)
    assert st == 1 and needle in _err(f._lib), _err(f._lib)


def test_mm_pair_rejects_overlapping_outputs_and_null(f):
    p0 = mm_args(f)
    p1 = mm_args(f, trans_a=1, out=P(FAKE.value + 4096 * 4096))  # inside p0's output
    st = f._lib.fp8_mm_pair(ctypes.byref(p0), ctypes.byref(p1), None)
    assert st == 1 and "overlap" in _err(f._lib)
    st = f._lib.fp8_mm_pair(None, ctypes.byref(p1), None)
    assert st == 1 and "NULL" in _err(f._lib)


def test_valid_call_without_gpu_reports_hip_error(f):
    """With valid arguments and no device, the call fails in the device
    check (status FP8_EHIP or FP8_EUNSUPPORTED) and enqueues nothing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = mm(f._lib)
    assert st in (2, 3)


def test_linear_validation(f):
    lib = f._lib
    st = lib.fp8_linear_fwd(FAKE, FAKE, None, 32, 32, 32, 0, 0, 0, None, None, FAKE, 1 << 20,
                            FAKE, FAKE, 1, None, None, None)
    assert st == 1 and "ring" in _err(lib)
    st = lib.fp8_linear_fwd(FAKE, FAKE, None, 32, 32, 32, 0, 1, 0, None, None, FAKE, 16, FAKE,
                            FAKE, 1, None, None, None)
    assert st == 1 and "workspace" in _err(lib)
    st = lib.fp8_linear_fwd(FAKE, FAKE, None, 32, 32, 32, 0, 1, 0, None, None, FAKE, 1 << 20,
                            FAKE, FAKE, 1, FAKE, None, None)
    assert st == 1 and "delayed scaling" in _err(lib)
    r = f._RingC(0x1000, 16, 0, 0, 0)
    r2 = f._RingC(0x2000, 16, 0, 0, 0)
    st = lib.fp8_linear_fwd(FAKE, FAKE, None, 32, 32, 32, 0, 0, 0, ctypes.byref(r),
                            ctypes.byref(r2), FAKE, 1 << 20, FAKE, FAKE, 7, None, FAKE, None)
    assert st == 1 and "backward format" in _err(lib)
    st = lib.fp8_linear_bwd(FAKE, FAKE, FAKE, 32, 32, 32, 1, 0, 0, None, None, FAKE, 1 << 20,
                            None, FAKE, FAKE, FAKE, None, None, None)
    assert st == 1 and "scales_fwd" in _err(lib)
    st = lib.fp8_linear_bwd(FAKE, None, FAKE, 32, 32, 32, 1, 1, 0, None, None, FAKE, 1 << 20,
                            None, FAKE, FAKE, FAKE, None, None, None)
    assert st == 1 and "dw needs x or x8_bwd" in _err(lib)
    st = lib.fp8_linear_bwd(FAKE, None, FAKE, 32, 32, 32, 1, 1, 0, None, None, FAKE, 1 << 20,
                            None, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == 1 and "delayed scaling" in _err(lib)
    st = lib.fp8_colsum(FAKE, 10, 10, FAKE, FAKE, 4, None)
    assert st == 1 and "workspace" in _err(lib)
