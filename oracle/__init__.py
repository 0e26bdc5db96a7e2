"""ctypes wrapper of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  It never touches the HIP library and the HIP library never
touches it.  All arrays are numpy arrays on the host.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

_LIB = None

ROWWISE, COLUMNWISE, FP8_ROWWISE = 1, 2, 4

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64


def lib():
    """Load (building it first if absent) the oracle shared library."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_e4m3_value.restype = ctypes.c_float
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_value.restype = ctypes.c_float
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_sr.restype = ctypes.c_uint8
        L.oracle_e2m1_encode_sr.argtypes = [ctypes.c_float, ctypes.c_uint8]
        L.oracle_amax.restype = ctypes.c_float
        L.oracle_amax.argtypes = [_p, _i64]
        L.oracle_philox4x32_10.restype = None
        L.oracle_philox4x32_10.argtypes = [_p, _p, _p]
        L.oracle_wht.restype = None
        L.oracle_wht.argtypes = [_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_float, _p]
        L.oracle_fp8_group.restype = ctypes.c_float
        L.oracle_fp8_group.argtypes = [_p, _p]
        L.oracle_quant_fp8_1x128.restype = None
        L.oracle_quant_fp8_1x128.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64]
        L.oracle_hadamard_quant_fp8.restype = None
        L.oracle_hadamard_quant_fp8.argtypes = [_p, _i64, ctypes.c_int32, _p, _i64, _i64, _p, _p]
        L.oracle_pow2_ceil.restype = ctypes.c_float
        L.oracle_pow2_ceil.argtypes = [ctypes.c_float]
        L.oracle_fp8_block.restype = ctypes.c_float
        L.oracle_fp8_block.argtypes = [_p, ctypes.c_int, ctypes.c_uint32, _p]
        L.oracle_quant_fp8_blockwise.restype = None
        L.oracle_quant_fp8_blockwise.argtypes = [_p, _i64, _i64, _i64, ctypes.c_uint32,
                                                 _p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64]
        L.oracle_hadamard_quant_fp8_ex.restype = None
        L.oracle_hadamard_quant_fp8_ex.argtypes = [_p, _i64, ctypes.c_int32, _p, _i64, _i64, ctypes.c_uint32,
                                                   _i64, _p, _p, _i64, _i64]
        L.oracle_exp.restype = ctypes.c_float
        L.oracle_exp.argtypes = [ctypes.c_float]
        L.oracle_silu.restype = ctypes.c_float
        L.oracle_silu.argtypes = [ctypes.c_float]
        L.oracle_exp_n.argtypes = [_p, _i64, _p]
        L.oracle_silu_n.argtypes = [_p, _i64, _p]
        L.oracle_swiglu_quant_fp8.restype = None
        L.oracle_swiglu_quant_fp8.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64]
        L.oracle_hadamard_quant_nvfp4.restype = None
        L.oracle_hadamard_quant_nvfp4.argtypes = [_p, _i64, ctypes.c_int32, _p, _i64, _i64, _p, _p, _p, _p, _p]
        L.oracle_nvfp4_global_scale.restype = ctypes.c_float
        L.oracle_nvfp4_global_scale.argtypes = [ctypes.c_float]
        L.oracle_nvfp4_block.restype = None
        L.oracle_nvfp4_block.argtypes = [_p, ctypes.c_float, _p, _p, _p]
        L.oracle_nvfp4_section_amax.restype = None
        L.oracle_nvfp4_section_amax.argtypes = [_p, _i64, _i64, ctypes.c_uint16, _p, _p]
        L.oracle_nvfp4_section.restype = None
        L.oracle_nvfp4_section.argtypes = [_p, _i64, _i64, ctypes.c_uint16, ctypes.c_uint32,
                                           ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                           _u64, _u64, _u64, _i64, _i64, _i64, _i64,
                                           _p, _p, _p, _p, _p, _p]
        L.oracle_group_rht_quant_nvfp4.restype = ctypes.c_int
        L.oracle_group_rht_quant_nvfp4.argtypes = [_p, _i64, _p, _i64, ctypes.c_uint16, ctypes.c_uint32,
                                                   _u64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]
        L.oracle_group_rht_quant_nvfp4_amax.restype = ctypes.c_int
        L.oracle_group_rht_quant_nvfp4_amax.argtypes = [_p, _i64, _p, _i64, ctypes.c_uint16, ctypes.c_uint32,
                                                        _u64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                        _p, _p, _p, _p]
        for name in ("oracle_e4m3_encode_n", "oracle_e2m1_encode_n", "oracle_f32_to_bf16_n"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [_p, _i64, _p]
        L.oracle_e2m1_encode_sr_n.restype = None
        L.oracle_e2m1_encode_sr_n.argtypes = [_p, _p, _i64, _p]
        L.oracle_wht_n.restype = None
        L.oracle_wht_n.argtypes = [_p, _i64, ctypes.c_int, ctypes.c_uint32, ctypes.c_float, _p]
        _LIB = L
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- formats ----------------------------------------------------------------
def e4m3_encode(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_value(code):
    return lib().oracle_e4m3_value(int(code))


def e2m1_encode(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e2m1_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_encode_sr(v, r):
    v = _c(v, np.float32)
    r = _c(np.broadcast_to(r, v.shape), np.uint8)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e2m1_encode_sr_n(_ptr(v), _ptr(r), v.size, _ptr(out))
    return out


def e2m1_value(code):
    return lib().oracle_e2m1_value(int(code))


def f32_to_bf16(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(_ptr(v), v.size, _ptr(out))
    return out


def philox4x32_10(ctr, key):
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.empty(4, np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def wht(v, sign_mask=0, c=None):
    """Batch WHT over the last axis (length 16 or 128)."""
    v = _c(v, np.float32)
    n = v.shape[-1]
    if c is None:
        c = 0.25 if n == 16 else float(np.float32(np.sqrt(np.float32(2.0))) / np.float32(16.0))
    out = np.empty_like(v)
    lib().oracle_wht_n(_ptr(v), v.size // n, n, sign_mask, c, _ptr(out))
    return out


# ---- FP8 ------------------------------------------------------------------------
def quant_fp8_1x128(x_bf16, scale_transposed=False):
    """x_bf16: [m][k] uint16.  Returns (codes [m][k] uint8, scales float32)."""
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    q = np.empty((m, k), np.uint8)
    if scale_transposed:
        s = np.empty((k // 128, m), np.float32)
        sr, sg = 1, m
    else:
        s = np.empty((m, k // 128), np.float32)
        sr, sg = k // 128, 1
    lib().oracle_quant_fp8_1x128(_ptr(x), m, k, k, _ptr(q), k, _ptr(s), sr, sg)
    return q, s


def hadamard_quant_fp8(pe, nope):
    """pe: [m][d_pe], nope: [m][128-d_pe] uint16.  Returns (codes [m][128], scales [m])."""
    pe = _c(pe, np.uint16)
    nope = _c(nope, np.uint16)
    m, d_pe = pe.shape
    assert nope.shape == (m, 128 - d_pe)
    q = np.empty((m, 128), np.uint8)
    s = np.empty((m,), np.float32)
    lib().oracle_hadamard_quant_fp8(_ptr(pe), max(d_pe, 1), d_pe, _ptr(nope), max(128 - d_pe, 1),
                                    m, _ptr(q), _ptr(s))
    return q, s


def fp8_group(x):
    """FP8 1x128 of one group of 128 float32 values: (scale, codes [128])."""
    x = _c(x, np.float32)
    assert x.size == 128
    codes = np.empty(128, np.uint8)
    s = lib().oracle_fp8_group(_ptr(x), _ptr(codes))
    return np.float32(s), codes


FP8_UE8M0 = 1


def quant_fp8_blockwise(x_bf16, options=0, rowwise=True, columnwise=True):
    """x: [m][k] uint16, k % 128 == 0.  Returns (row_codes [m][k], row_scales [m][k/128],
    col_codes [k][m] (row c = column c of x), col_scales [k][ceil(m/128)]), with None
    for an output not asked for."""
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    nb = (m + 127) // 128
    rq = np.empty((m, k), np.uint8) if rowwise else None
    rs = np.empty((m, k // 128), np.float32) if rowwise else None
    cq = np.empty((k, m), np.uint8) if columnwise else None
    cs = np.empty((k, nb), np.float32) if columnwise else None
    lib().oracle_quant_fp8_blockwise(_ptr(x), m, k, k, options, _ptr(rq), k, _ptr(rs), k // 128, 1,
                                     _ptr(cq), m, _ptr(cs), nb, 1)
    return rq, rs, cq, cs


def hadamard_quant_fp8_ex(pe, nope, options=0, heads=1, token_stride=None, head_stride=None, scale_size=None):
    """The DSA rotate + FP8 with options and scale index token*token_stride +
    head*head_stride (defaults: [tokens][heads]).  Returns (codes [m][128], scales
    (flat array of scale_size floats, NaN where nothing is written))."""
    pe = _c(pe, np.uint16)
    nope = _c(nope, np.uint16)
    m, d_pe = pe.shape
    tokens = m // heads
    ts = heads if token_stride is None else token_stride
    hs = 1 if head_stride is None else head_stride
    size = m if scale_size is None else scale_size
    q = np.empty((m, 128), np.uint8)
    s = np.full(size, np.nan, np.float32)
    lib().oracle_hadamard_quant_fp8_ex(_ptr(pe), max(d_pe, 1), d_pe, _ptr(nope), max(128 - d_pe, 1), m, options,
                                       heads, _ptr(q), _ptr(s), ts, hs)
    return q, s


def exp(x):
    """EXP over an array of float32 values."""
    x = _c(x, np.float32)
    out = np.empty_like(x)
    lib().oracle_exp_n(_ptr(x), x.size, _ptr(out))
    return out


def silu(x):
    """SILU over an array of float32 values."""
    x = _c(x, np.float32)
    out = np.empty_like(x)
    lib().oracle_silu_n(_ptr(x), x.size, _ptr(out))
    return out


def swiglu_quant_fp8(gate, up, scale_transposed=False):
    """gate, up: [m][n] uint16 (BF16 bits), n % 128 == 0.  Returns (codes [m][n],
    scales [m][n/128] or [n/128][m] when scale_transposed)."""
    gate = _c(gate, np.uint16)
    up = _c(up, np.uint16)
    m, n = gate.shape
    assert up.shape == (m, n) and n % 128 == 0
    q = np.empty((m, n), np.uint8)
    if scale_transposed:
        s = np.empty((n // 128, m), np.float32)
        sr, sg = 1, m
    else:
        s = np.empty((m, n // 128), np.float32)
        sr, sg = n // 128, 1
    lib().oracle_swiglu_quant_fp8(_ptr(gate), n, _ptr(up), n, m, n, _ptr(q), n, _ptr(s), sr, sg)
    return q, s


class DsaNVFP4Outputs:
    """codes [m][64] uint8, scales [m][8] uint8 (E4M3), global_scale float32, amax float32
    (the measured A)."""

    def __init__(self, codes, scales, global_scale, amax):
        self.codes, self.scales, self.global_scale, self.amax = codes, scales, global_scale, amax


def hadamard_quant_nvfp4(pe, nope, amax_in=None):
    """pe: [m][d_pe], nope: [m][128-d_pe] uint16.  amax_in: None (measure) or the A to use."""
    pe = _c(pe, np.uint16)
    nope = _c(nope, np.uint16)
    m, d_pe = pe.shape
    assert nope.shape == (m, 128 - d_pe)
    codes = np.empty((m, 64), np.uint8)
    scales = np.empty((m, 8), np.uint8)
    g = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    ain = None if amax_in is None else np.array([amax_in], np.float32)
    lib().oracle_hadamard_quant_nvfp4(_ptr(pe), max(d_pe, 1), d_pe, _ptr(nope), max(128 - d_pe, 1), m,
                                      _ptr(ain), _ptr(codes), _ptr(scales), _ptr(g), _ptr(a))
    return DsaNVFP4Outputs(codes, scales, np.float32(g[0]), np.float32(a[0]))


# ---- NVFP4 ----------------------------------------------------------------------
def nvfp4_global_scale(amax):
    return np.float32(lib().oracle_nvfp4_global_scale(float(np.float32(amax))))


def nvfp4_block(v, g, rbits=None):
    v = _c(v, np.float32)
    assert v.size == 16
    sc = np.zeros(1, np.uint8)
    codes = np.zeros(16, np.uint8)
    r = None if rbits is None else _c(rbits, np.uint8)
    lib().oracle_nvfp4_block(_ptr(v), float(np.float32(g)), _ptr(r), _ptr(sc), _ptr(codes))
    return int(sc[0]), codes


def nvfp4_section_amax(x_bf16, sign_mask):
    x = _c(x_bf16, np.uint16)
    rows, k = x.shape
    ar = np.zeros(1, np.float32)
    ac = np.zeros(1, np.float32)
    lib().oracle_nvfp4_section_amax(_ptr(x), rows, k, sign_mask, _ptr(ar), _ptr(ac))
    return ar[0], ac[0]


class NVFP4Outputs:
    """Host buffers with the library's layouts for one grouped call."""

    def __init__(self, total_rows, k, num_sections, flags):
        self.flags = flags
        row = bool(flags & ROWWISE)
        col = bool(flags & COLUMNWISE)
        f8 = bool(flags & FP8_ROWWISE)
        self.row_codes = np.zeros(total_rows * k // 2 if row else 0, np.uint8)
        self.row_scales = np.zeros(total_rows * k // 16 if row else 0, np.uint8)
        self.row_global = np.zeros(num_sections if row else 0, np.float32)
        self.col_codes = np.zeros(total_rows * k // 2 if col else 0, np.uint8)
        self.col_scales = np.zeros(total_rows * k // 16 if col else 0, np.uint8)
        self.col_global = np.zeros(num_sections if col else 0, np.float32)
        self.fp8_codes = np.zeros(total_rows * k if f8 else 0, np.uint8)
        self.fp8_scales = np.zeros(total_rows * k // 128 if f8 else 0, np.float32)
        # measured section maxima (row values, column values), always filled
        self.row_amax = np.zeros(num_sections, np.float32)
        self.col_amax = np.zeros(num_sections, np.float32)


def group_rht_quant_nvfp4(x_bf16, split_sections, sign_mask, flags, seed=0,
                          row_offsets=None, col_offsets=None, threads=1, amax_in=None):
    """The whole grouped call.  threads > 1 runs independent sections and column
    ranges of the same oracle functions on worker threads (ctypes releases the GIL).
    amax_in: None, or (row maxima, column maxima) per section supplied by the caller
    (either may be None) that replace the measured maxima in the tensor scales.  The
    measured maxima are returned in out.row_amax / out.col_amax."""
    x = _c(x_bf16, np.uint16)
    total, k = x.shape
    sections = _c(split_sections, np.int64)
    S = sections.size
    assert int(sections.sum()) == total
    out = NVFP4Outputs(total, k, S, flags)
    ro = None if row_offsets is None else _c(row_offsets, np.uint64)
    co = None if col_offsets is None else _c(col_offsets, np.uint64)
    ain_r = ain_c = None
    if amax_in is not None:
        ain_r = None if amax_in[0] is None else _c(amax_in[0], np.float32)
        ain_c = None if amax_in[1] is None else _c(amax_in[1], np.float32)
    if threads <= 1:
        rc = lib().oracle_group_rht_quant_nvfp4_amax(
            _ptr(x), k, _ptr(sections), S, sign_mask, flags, seed, _ptr(ro), _ptr(co),
            _ptr(out.row_codes), _ptr(out.row_scales), _ptr(out.row_global),
            _ptr(out.col_codes), _ptr(out.col_scales), _ptr(out.col_global),
            _ptr(out.fp8_codes), _ptr(out.fp8_scales),
            _ptr(ain_r), _ptr(ain_c), _ptr(out.row_amax), _ptr(out.col_amax))
        if rc != 0:
            raise ValueError(f"oracle rejected the call ({rc})")
        return out
    _threaded_group(x, sections, sign_mask, flags, seed, ro, co, out, threads, ain_r, ain_c)
    return out


def _threaded_group(x, sections, sign_mask, flags, seed, ro, co, out, threads, ain_r=None, ain_c=None):
    total, k = x.shape
    L = lib()
    starts = np.concatenate([[0], np.cumsum(sections)[:-1]]).astype(np.int64)
    chunk_rows = 128
    chunk_cols = 128

    def amax_job(s, r0, r1):
        ar = np.zeros(1, np.float32)
        ac = np.zeros(1, np.float32)
        sub = x[r0:r1]
        L.oracle_nvfp4_section_amax(_ptr(sub), r1 - r0, k, sign_mask, _ptr(ar), _ptr(ac))
        return s, ar[0], ac[0]

    jobs = []
    for s, (R, m) in enumerate(zip(starts, sections)):
        for r0 in range(0, int(m), chunk_rows):
            jobs.append((s, int(R + r0), int(R + min(m, r0 + chunk_rows))))
    amax_r = np.zeros(len(sections), np.float32)
    amax_c = np.zeros(len(sections), np.float32)
    with ThreadPoolExecutor(threads) as ex:
        for s, ar, ac in ex.map(lambda j: amax_job(*j), jobs):
            amax_r[s] = max(amax_r[s], ar)
            amax_c[s] = max(amax_c[s], ac)
    out.row_amax[:] = amax_r
    out.col_amax[:] = amax_c
    g_r = np.array([nvfp4_global_scale(a) for a in (amax_r if ain_r is None else ain_r)], np.float32)
    g_c = np.array([nvfp4_global_scale(a) for a in (amax_c if ain_c is None else ain_c)], np.float32)
    if flags & ROWWISE:
        out.row_global[:] = g_r
    if flags & COLUMNWISE:
        out.col_global[:] = g_c

    def sec_job(s, rb, re, cb, ce, fl):
        R = int(starts[s])
        m = int(sections[s])
        xs = x[R:R + m]

        def sub(a, off):
            return None if a.size == 0 else a[off:]
        L.oracle_nvfp4_section(
            _ptr(xs), m, k, sign_mask, fl, float(g_r[s]), float(g_c[s]),
            int(ro is not None), int(co is not None), seed,
            int(ro[s]) if ro is not None else 0, int(co[s]) if co is not None else 0,
            rb, re, cb, ce,
            _ptr(sub(out.row_codes, R * k // 2)), _ptr(sub(out.row_scales, R * k // 16)),
            _ptr(sub(out.col_codes, k * R // 2)), _ptr(sub(out.col_scales, k * R // 16)),
            _ptr(sub(out.fp8_codes, R * k)), _ptr(sub(out.fp8_scales, R * k // 128)))

    jobs = []
    row_flags = flags & (ROWWISE | FP8_ROWWISE)
    for s, m in enumerate(sections):
        m = int(m)
        if m == 0:
            continue
        if row_flags:
            for r0 in range(0, m, chunk_rows):
                jobs.append((s, r0, min(m, r0 + chunk_rows), 0, 0, row_flags))
        if flags & COLUMNWISE:
            for c0 in range(0, k, chunk_cols):
                jobs.append((s, 0, 0, c0, min(k, c0 + chunk_cols), COLUMNWISE))
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda j: sec_job(*j), jobs))
