"""The C ABI of include/mxq.h on the host: the library loads, exports every
declared symbol, and rejects bad arguments before anything is enqueued (so these
run without a GPU).  Error classes follow the pages' interface lessons: split
sections must be multiples of 128 (TransformerEngine PR #2555, cast.cpp comment),
an unsupported request is an error rather than a fallback (onnxruntime PR #33644,
Description), and the workspace is the caller's, sized by a query (TransformerEngine
PR #2564, review thread)."""
import ctypes
import os
import re

import pytest

import nvfp4_quantization_amd as mxq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, MISALIGNED, WS_SMALL, UNSUPPORTED, HIP = range(6)
A = 1 << 20          # a fake, 16-byte aligned device address: never dereferenced on these paths


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mxq.LIB_PATH):
        pytest.skip("libmxq.so not built")
    return mxq.lib()


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0          # counts devices without initializing them


# The rejection tests pass fake device addresses: a host check that wrongly accepted
# one would launch a kernel on them.  Where no GPU is visible that launch fails
# (MXQ_ERR_HIP, a failed assertion); where one is, it could fault the device, so
# they run only without one (the CPU tier).
no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: run where no GPU is visible")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mxq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|mxq_status|size_t)\s+(mxq_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(mxq.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in mxq.STATUS.items():
        assert mxq.mxq_status_string(code) == name
    assert "gfx950" in mxq.mxq_version()


def fp8(L, x=A, m=4, k=256, ldx=256, q=A, ldq=256, s=A, sr=2, sg=1):
    return L.mxq_quant_fp8_1x128(x, m, k, ldx, q, ldq, s, sr, sg, None)


@no_gpu
def test_fp8_argument_errors(L):
    assert fp8(L, k=200, ldx=200, ldq=208) == MISALIGNED
    assert fp8(L, m=-1) == INVALID
    assert fp8(L, ldx=128) == INVALID
    assert fp8(L, x=None) == INVALID
    assert fp8(L, q=None) == INVALID
    assert fp8(L, s=None) == INVALID
    assert fp8(L, x=A + 8) == MISALIGNED
    assert fp8(L, s=A + 2) == MISALIGNED
    assert fp8(L, ldq=264) == MISALIGNED
    assert fp8(L, m=0, x=None, q=None, s=None) == OK      # empty call: nothing to do
    assert fp8(L, m=1 << 31) == UNSUPPORTED


def dsa(L, pe=A, ld_pe=64, d_pe=64, nope=A, ld_nope=64, m=8, q=A, s=A):
    return L.mxq_hadamard_quant_fp8(pe, ld_pe, d_pe, nope, ld_nope, m, q, s, None)


@no_gpu
def test_dsa_argument_errors(L):
    assert dsa(L, d_pe=60, ld_pe=60, ld_nope=68) == MISALIGNED
    assert dsa(L, d_pe=129) == INVALID
    assert dsa(L, ld_pe=32) == INVALID
    assert dsa(L, pe=None) == INVALID
    assert dsa(L, nope=None) == INVALID
    assert dsa(L, q=A + 4) == MISALIGNED
    assert dsa(L, m=0) == OK
    assert dsa(L, m=-3) == INVALID


def grouped(L, x=A, k=256, sections=(128, 256), mask=0, flags=3, sr=None, row=True, col=True, f8=True,
            ws=A, ws_bytes=None, row_ptrs=(A, A, A), col_ptrs=(A, A, A), fp8_ptrs=(A, A)):
    S = len(sections)
    arr = (ctypes.c_int64 * max(S, 1))(*sections)
    r = mxq._NVFP4Out(*row_ptrs)
    c = mxq._NVFP4Out(*col_ptrs)
    f = mxq._FP8Out(*fp8_ptrs)
    if ws_bytes is None:
        ws_bytes = 1 << 30
    return L.mxq_group_rht_quant_nvfp4(
        x, k, ctypes.addressof(arr), S, mask, flags, sr,
        ctypes.addressof(r) if row else None, ctypes.addressof(c) if col else None,
        ctypes.addressof(f) if f8 else None, ws, ws_bytes, None)


@no_gpu
def test_grouped_argument_errors(L):
    assert grouped(L, sections=(128, 192)) == MISALIGNED          # split_section % 128 != 0
    assert grouped(L, sections=(64,)) == MISALIGNED
    assert grouped(L, k=192) == MISALIGNED
    assert grouped(L, sections=(128, -128)) == INVALID
    assert grouped(L, sections=()) == INVALID
    assert grouped(L, sections=(128,) * 257) == UNSUPPORTED
    assert grouped(L, flags=0) == INVALID
    assert grouped(L, flags=8) == INVALID
    assert grouped(L, row=False) == INVALID                       # requested output missing
    assert grouped(L, row_ptrs=(A, None, A)) == INVALID
    assert grouped(L, col_ptrs=(None, A, A)) == INVALID
    assert grouped(L, flags=7, f8=False) == INVALID
    assert grouped(L, x=None) == INVALID
    assert grouped(L, x=A + 2) == MISALIGNED
    assert grouped(L, col_ptrs=(A + 8, A, A)) == MISALIGNED
    assert grouped(L, ws=None) == INVALID
    need = mxq.mxq_group_rht_quant_nvfp4_workspace_size(384, 256, 2, 3)
    assert need > 0 and need % 256 == 0
    assert grouped(L, ws_bytes=need - 1) == WS_SMALL
    assert grouped(L, ws=A + 64) == MISALIGNED
    assert grouped(L, sections=(1 << 31,)) == UNSUPPORTED
    assert grouped(L, k=(1 << 26) + 128) == UNSUPPORTED           # tile rows use 32-bit offsets


def test_workspace_size_query(L):
    q = mxq.mxq_group_rht_quant_nvfp4_workspace_size
    assert q(16384, 4096, 8, 4) == 0                              # FP8 only: no amax pass
    # two status lines, scale tables (32 sections x 2 directions x 128 x 16 B) and
    # the single-read form's 1024 partial words of one launch group, then the amax
    # pass's 8-byte partials, one per 16 rows x 1024 columns (or part)
    fixed = 512 + 32 * 2 * 128 * 16 + 4 * 1024
    assert fixed == mxq.WORKSPACE_FIXED == 135680
    for total, k, S in [(0, 4096, 8), (16384, 4096, 8), (65536, 7168, 32), (128, 128, 1), (16384, 4096, 256)]:
        for flags in (1, 2, 3, 7):
            need = q(total, k, S, flags)
            partials = (total // 16) * -(-k // 1024)
            assert need % 256 == 0
            assert fixed + 8 * partials <= need < fixed + 8 * partials + 256


def test_no_forbidden_calls_in_host_sources():
    """The quantize path allocates nothing, never synchronizes and reads no
    environment variable (TransformerEngine PR #2564 / #2555 lessons)."""
    src = open(os.path.join(ROOT, "nvfp4_quantization_amd", "csrc", "mxq_api.cpp")).read()
    code = re.sub(r"//.*", "", src)
    for bad in ("hipMalloc", "hipFree", "hipMemset", "hipDeviceSynchronize", "hipStreamSynchronize",
                "getenv", "malloc(", "new "):
        assert bad not in code, bad


def grouped_amax(L, amax, flags=3):
    S = 2
    arr = (ctypes.c_int64 * S)(128, 256)
    r = mxq._NVFP4Out(A, A, A)
    c = mxq._NVFP4Out(A, A, A)
    f = mxq._FP8Out(A, A)
    a = mxq._Amax(*amax)
    return L.mxq_group_rht_quant_nvfp4_with_amax(
        A, 256, ctypes.addressof(arr), S, 0, flags, None, ctypes.addressof(r), ctypes.addressof(c),
        ctypes.addressof(f), ctypes.addressof(a), A, 1 << 30, None)


@no_gpu
def test_grouped_amax_argument_errors(L):
    """Supplied maxima come for every requested NVFP4 direction or for none, 4-byte
    aligned; every rejected call returns before anything is enqueued."""
    assert grouped_amax(L, (A, None, None, None)) == INVALID       # column maxima missing
    assert grouped_amax(L, (None, A, None, None)) == INVALID       # row maxima missing
    assert grouped_amax(L, (A + 2, A, None, None)) == MISALIGNED
    assert grouped_amax(L, (None, None, A + 1, None)) == MISALIGNED
    assert grouped_amax(L, (A, A, None, None), flags=0) == INVALID


def dsa4(L, pe=A, ld_pe=64, d_pe=64, nope=A, ld_nope=64, m=8, amax_in=None, amax_out=None, codes=A, scales=A,
         g=A, ws=A, ws_bytes=1 << 20):
    return L.mxq_hadamard_quant_nvfp4(pe, ld_pe, d_pe, nope, ld_nope, m, amax_in, amax_out, codes, scales, g,
                                      ws, ws_bytes, None)


@no_gpu
def test_dsa_nvfp4_argument_errors(L):
    """The DSA rotate + NVFP4 call checks everything on the host; a call without
    rows needs no workspace but still writes the tensor scale."""
    assert dsa4(L, d_pe=60, ld_pe=60, ld_nope=68) == MISALIGNED
    assert dsa4(L, d_pe=136) == INVALID
    assert dsa4(L, ld_nope=32) == INVALID
    assert dsa4(L, pe=None) == INVALID
    assert dsa4(L, codes=None) == INVALID
    assert dsa4(L, g=None) == INVALID
    assert dsa4(L, g=A + 2) == MISALIGNED
    assert dsa4(L, amax_in=A + 1) == MISALIGNED
    assert dsa4(L, amax_out=A + 2) == MISALIGNED
    assert dsa4(L, scales=A + 8) == MISALIGNED
    assert dsa4(L, ws=None) == INVALID
    assert dsa4(L, ws=A + 128) == MISALIGNED
    assert dsa4(L, m=-1) == INVALID
    assert dsa4(L, m=1 << 31) == UNSUPPORTED
    need = L.mxq_hadamard_quant_nvfp4_workspace_size(8)
    assert dsa4(L, ws_bytes=need - 1) == 3                        # MXQ_ERR_WORKSPACE_TOO_SMALL


def test_dsa_nvfp4_workspace_size(L):
    """128 table entries, then 4 bytes per 64 rows, rounded to 256."""
    q = L.mxq_hadamard_quant_nvfp4_workspace_size
    fixed = 2048
    assert q(0) == 0 and q(-5) == 0
    assert q(1) == fixed + 256
    assert q(64 * 64) == fixed + 256
    assert q(64 * 64 + 1) == fixed + 512
    assert q(262144) == fixed + 4 * 4096


def swiglu(L, g=A, ldg=256, u=A, ldu=256, m=8, n=256, q=A, ldq=256, s=A, sr=2, sg=1):
    return L.mxq_swiglu_quant_fp8(g, ldg, u, ldu, m, n, q, ldq, s, sr, sg, None)


@no_gpu
def test_swiglu_argument_errors(L):
    assert swiglu(L, n=192, ldg=192, ldu=192, ldq=192) == MISALIGNED
    assert swiglu(L, ldg=128) == INVALID
    assert swiglu(L, ldu=264, u=A + 8) == MISALIGNED
    assert swiglu(L, ldq=264) == MISALIGNED
    assert swiglu(L, g=None) == INVALID
    assert swiglu(L, s=A + 2) == MISALIGNED
    assert swiglu(L, sr=-1) == INVALID
    assert swiglu(L, m=0, g=None, u=None, q=None, s=None) == OK
    assert swiglu(L, m=1 << 31) == UNSUPPORTED


def blockwise(L, x=A, m=256, k=256, ldx=256, options=0, row=(A, 256, A, 2, 1), col=(A, 256, A, 2, 1)):
    r = mxq._FP8BlockOut(*row) if row is not None else None
    c = mxq._FP8BlockOut(*col) if col is not None else None
    return L.mxq_quant_fp8_blockwise(x, m, k, ldx, options, ctypes.byref(r) if r is not None else None,
                                     ctypes.byref(c) if c is not None else None, None)


@no_gpu
def test_fp8_blockwise_argument_errors(L):
    assert blockwise(L, row=None, col=None) == INVALID
    assert blockwise(L, options=2) == INVALID
    assert blockwise(L, k=192, ldx=192) == MISALIGNED
    assert blockwise(L, row=(A, 264, A, 2, 1)) == MISALIGNED
    assert blockwise(L, col=(A, 128, A, 2, 1)) == INVALID           # ld < m
    assert blockwise(L, col=(A + 8, 256, A, 2, 1)) == MISALIGNED
    assert blockwise(L, col=(A, 256, A + 1, 2, 1)) == MISALIGNED
    assert blockwise(L, row=(None, 256, A, 2, 1)) == INVALID
    assert blockwise(L, m=0, x=None) == OK
    assert blockwise(L, m=1 << 31, col=None) == UNSUPPORTED


@no_gpu
def test_dsa_fp8_ex_argument_errors(L):
    def ex(**kw):
        a = dict(pe=A, ld_pe=64, d_pe=64, nope=A, ld_nope=64, m=8, options=0, heads=2, q=A, s=A, st=2, sh=1)
        a.update(kw)
        return L.mxq_hadamard_quant_fp8_ex(a["pe"], a["ld_pe"], a["d_pe"], a["nope"], a["ld_nope"], a["m"],
                                           a["options"], a["heads"], a["q"], a["s"], a["st"], a["sh"], None)
    assert ex(options=4) == INVALID
    assert ex(heads=0) == INVALID
    assert ex(st=-1) == INVALID
    assert ex(d_pe=60, ld_pe=60, ld_nope=68) == MISALIGNED
    assert ex(s=A + 2) == MISALIGNED
    assert ex(m=0) == OK
    assert ex(st=1 << 40) == UNSUPPORTED                            # scale index 3 * 2^40
    assert ex(heads=1 << 62, sh=1 << 40) == UNSUPPORTED             # no overflow forming the token count


@no_gpu
def test_extent_limits(L):
    """No array a call addresses may span 2^40 or more elements (MXQ_MAX_EXTENT):
    such calls are rejected without forming an overflowing product, and the grouped
    size query answers 0 beyond the supported profile.  Only rejected calls are made
    here: an accepted one would launch on the fake addresses."""
    big = 1 << 40
    assert fp8(L, k=1 << 62, ldx=1 << 62, ldq=1 << 62) == UNSUPPORTED    # m * k would overflow int64
    assert fp8(L, ldx=big) == UNSUPPORTED
    edge = (big - 256) // 3                                              # 3 rows of stride edge + 256 = 2^40
    assert edge % 8 == 0 and 3 * edge + 256 == big
    assert fp8(L, ldx=edge) == UNSUPPORTED
    assert fp8(L, ldq=big) == UNSUPPORTED
    assert fp8(L, sr=big) == UNSUPPORTED
    assert fp8(L, sg=big) == UNSUPPORTED
    assert swiglu(L, ldu=big) == UNSUPPORTED
    assert swiglu(L, sg=big) == UNSUPPORTED
    assert dsa(L, ld_nope=big) == UNSUPPORTED
    assert dsa(L, ld_pe=big) == UNSUPPORTED
    assert dsa4(L, ld_pe=big) == UNSUPPORTED
    assert blockwise(L, col=(A, big, A, 2, 1)) == UNSUPPORTED
    assert blockwise(L, row=(A, 256, A, big, 1)) == UNSUPPORTED
    assert blockwise(L, col=(A, 256, A, 2, big)) == UNSUPPORTED
    q = mxq.mxq_group_rht_quant_nvfp4_workspace_size
    assert q(1 << 40, 4096, 8, 3) == 0 and q(16384, 1 << 40, 8, 3) == 0


@no_gpu
def test_noalloc_rejects_beyond_scratch(L):
    """The grouped call without a workspace refuses, before anything is enqueued, a
    call whose workspace would exceed its scratch array (MXQ_NOALLOC_SCRATCH_BYTES)."""
    text = open(os.path.join(ROOT, "include", "mxq.h")).read()
    limit = int(eval(re.search(r"#define MXQ_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text).expand(r"\1 << \2")))
    q = mxq.mxq_group_rht_quant_nvfp4_workspace_size
    rows = 1 << 20                                      # 2^20 x 8192: 524,288 amax partials
    assert q(rows, 8192, 1, 3) > limit
    sections = (ctypes.c_int64 * 1)(rows)
    out = mxq._NVFP4Out(A, A, A)
    st = L.mxq_group_rht_quant_nvfp4_noalloc(ctypes.c_void_p(A), 8192, ctypes.addressof(sections), 1, 0, 3,
                                             None, ctypes.addressof(out), ctypes.addressof(out), None, None)
    assert st == UNSUPPORTED
    # invalid arguments: the grouped call's own checks answer first
    sections = (ctypes.c_int64 * 1)(100)                 # not a multiple of 128
    assert L.mxq_group_rht_quant_nvfp4_noalloc(ctypes.c_void_p(A), 256, ctypes.addressof(sections), 1, 0, 3,
                                               None, ctypes.addressof(out), ctypes.addressof(out), None,
                                               None) == MISALIGNED
    sections = (ctypes.c_int64 * 1)(128)
    assert L.mxq_group_rht_quant_nvfp4_noalloc(ctypes.c_void_p(A), 8192, ctypes.addressof(sections), 1, 0, 3,
                                               None, None, None, None, None) == INVALID        # no outputs
