"""mxq: MI355X-native (gfx950) block quantization of BF16 activations.

A thin ctypes binding of the C ABI in include/mxq.h.  The functions here only
marshal arguments: every step of the quantization runs in the HIP kernels of
libmxq.so.  PyTorch supplies device memory and the current stream.  If the
library is missing or cannot be loaded, every entry point raises; there is no
CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmxq.so")

MXQ_ROWWISE, MXQ_COLUMNWISE, MXQ_FP8_ROWWISE = 1, 2, 4
MXQ_MAX_SECTIONS = 256
STATUS = {0: "MXQ_OK", 1: "MXQ_ERR_INVALID_ARGUMENT", 2: "MXQ_ERR_MISALIGNED",
          3: "MXQ_ERR_WORKSPACE_TOO_SMALL", 4: "MXQ_ERR_UNSUPPORTED", 5: "MXQ_ERR_HIP"}

EXPORTED = ("mxq_status_string", "mxq_version", "mxq_quant_fp8_1x128", "mxq_hadamard_quant_fp8",
            "mxq_group_rht_quant_nvfp4_workspace_size", "mxq_group_rht_quant_nvfp4",
            "mxq_group_rht_quant_nvfp4_with_amax",
            "mxq_hadamard_quant_nvfp4_workspace_size", "mxq_hadamard_quant_nvfp4", "mxq_swiglu_quant_fp8",
            "mxq_quant_fp8_blockwise", "mxq_hadamard_quant_fp8_ex", "mxq_group_rht_quant_nvfp4_noalloc")
MXQ_FP8_UE8M0 = 1


class MxqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class _NVFP4Out(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("block_scales", ctypes.c_void_p), ("global_scales", ctypes.c_void_p)]


class _FP8Out(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _FP8BlockOut(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("ld", ctypes.c_int64), ("scales", ctypes.c_void_p),
                ("scale_stride_a", ctypes.c_int64), ("scale_stride_b", ctypes.c_int64)]


class _SR(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("row_offsets", ctypes.c_void_p), ("col_offsets", ctypes.c_void_p)]


class _Amax(ctypes.Structure):
    _fields_ = [("row_in", ctypes.c_void_p), ("col_in", ctypes.c_void_p),
                ("row_out", ctypes.c_void_p), ("col_out", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmxq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m nvfp4_quantization_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64
        L.mxq_status_string.restype = ctypes.c_char_p
        L.mxq_status_string.argtypes = [ctypes.c_int]
        L.mxq_version.restype = ctypes.c_char_p
        L.mxq_version.argtypes = []
        L.mxq_quant_fp8_1x128.restype = ctypes.c_int
        L.mxq_quant_fp8_1x128.argtypes = [p, i64, i64, i64, p, i64, p, i64, i64, p]
        L.mxq_hadamard_quant_fp8.restype = ctypes.c_int
        L.mxq_hadamard_quant_fp8.argtypes = [p, i64, ctypes.c_int32, p, i64, i64, p, p, p]
        L.mxq_group_rht_quant_nvfp4_workspace_size.restype = ctypes.c_size_t
        L.mxq_group_rht_quant_nvfp4_workspace_size.argtypes = [i64, i64, i64, ctypes.c_uint32]
        L.mxq_group_rht_quant_nvfp4.restype = ctypes.c_int
        L.mxq_group_rht_quant_nvfp4.argtypes = [p, i64, p, i64, ctypes.c_uint16, ctypes.c_uint32, p,
                                                p, p, p, p, ctypes.c_size_t, p]
        L.mxq_group_rht_quant_nvfp4_with_amax.restype = ctypes.c_int
        L.mxq_group_rht_quant_nvfp4_with_amax.argtypes = [p, i64, p, i64, ctypes.c_uint16, ctypes.c_uint32, p,
                                                          p, p, p, p, p, ctypes.c_size_t, p]
        L.mxq_quant_fp8_blockwise.restype = ctypes.c_int
        L.mxq_quant_fp8_blockwise.argtypes = [p, i64, i64, i64, ctypes.c_uint32, p, p, p]
        L.mxq_hadamard_quant_fp8_ex.restype = ctypes.c_int
        L.mxq_hadamard_quant_fp8_ex.argtypes = [p, i64, ctypes.c_int32, p, i64, i64, ctypes.c_uint32, i64, p, p,
                                                i64, i64, p]
        L.mxq_swiglu_quant_fp8.restype = ctypes.c_int
        L.mxq_swiglu_quant_fp8.argtypes = [p, i64, p, i64, i64, i64, p, i64, p, i64, i64, p]
        L.mxq_hadamard_quant_nvfp4_workspace_size.restype = ctypes.c_size_t
        L.mxq_hadamard_quant_nvfp4_workspace_size.argtypes = [i64]
        L.mxq_hadamard_quant_nvfp4.restype = ctypes.c_int
        L.mxq_hadamard_quant_nvfp4.argtypes = [p, i64, ctypes.c_int32, p, i64, i64, p, p, p, p, p, p,
                                               ctypes.c_size_t, p]
        L.mxq_group_rht_quant_nvfp4_noalloc.restype = ctypes.c_int
        L.mxq_group_rht_quant_nvfp4_noalloc.argtypes = [p, i64, p, i64, ctypes.c_uint16, ctypes.c_uint32, p,
                                                        p, p, p, p]
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, *tensors) -> ctypes.c_void_p:
    """Handle of the stream a call is enqueued on: torch's current stream by default,
    else a torch stream or a raw HIP stream handle.  The binding allocates outputs and
    workspaces (and fills workspaces) on the current stream, so a call on another stream
    first makes that stream wait for the current one, and records on it every tensor
    the call reads or writes: torch's caching allocator then keeps their memory from
    other work until the call has ended."""
    cur = torch.cuda.current_stream()
    if stream is None:
        return ctypes.c_void_p(cur.cuda_stream)
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    if stream.cuda_stream != cur.cuda_stream:
        stream.wait_stream(cur)
        for t in tensors:
            if isinstance(t, torch.Tensor) and t.is_cuda:
                t.record_stream(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise MxqError(status, what)


def _row_stride(t: Optional[torch.Tensor]) -> int:
    """Row stride in elements of a 2-D tensor (its width when it holds nothing)."""
    if t is None:
        return 0
    return t.stride(0) if t.numel() > 0 else t.shape[1]


def _bf16_bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected bfloat16 (or its 16-bit pattern), got {t.dtype}")


def mxq_status_string(status: int) -> str:
    return lib().mxq_status_string(status).decode()


def mxq_version() -> str:
    return lib().mxq_version().decode()


# ---------------------------------------------------------------------------- FP8 1x128
def mxq_quant_fp8_1x128(x: torch.Tensor, q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                        scale_transposed: bool = False, stream=None):
    """FP8 E4M3 codes [m][k] (uint8) and FP32 scales ([m][k/128], or [k/128][m]
    when scale_transposed) of a BF16 [m][k] tensor (row stride may exceed k)."""
    x = _bf16_bits(x)
    m, k = x.shape
    ldx = x.stride(0) if m > 0 else k
    if x.stride(1) != 1:
        raise ValueError("x must be contiguous along k")
    if q is None:
        q = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        shape = (k // 128, m) if scale_transposed else (m, k // 128)
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    srow, sgroup = (1, m) if scale_transposed else (k // 128, 1)
    ldq = q.stride(0) if m > 0 else k
    _check(lib().mxq_quant_fp8_1x128(_ptr(x), m, k, ldx, _ptr(q), ldq, _ptr(scales), srow, sgroup,
                                     _stream(stream, x, q, scales)), "mxq_quant_fp8_1x128")
    return q, scales


# ---------------------------------------------------------------------------- DSA rotate + FP8
def mxq_hadamard_quant_fp8(pe: Optional[torch.Tensor], nope: Optional[torch.Tensor],
                           q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None, stream=None):
    """cat[pe, nope] along the last dim -> normalized 128-point WHT -> FP8 1x128.
    pe: [m][d_pe], nope: [m][128-d_pe] BF16 (either may be None when empty)."""
    ref = pe if pe is not None else nope
    m = ref.shape[0]
    d_pe = pe.shape[1] if pe is not None else 0
    if pe is not None:
        pe = _bf16_bits(pe)
    if nope is not None:
        nope = _bf16_bits(nope)
    if q is None:
        q = torch.empty((m, 128), dtype=torch.uint8, device=ref.device)
    if scales is None:
        scales = torch.empty((m,), dtype=torch.float32, device=ref.device)
    ld_pe = _row_stride(pe)
    ld_nope = _row_stride(nope)
    _check(lib().mxq_hadamard_quant_fp8(_ptr(pe), ld_pe, d_pe, _ptr(nope), ld_nope, m, _ptr(q), _ptr(scales),
                                        _stream(stream, pe, nope, q, scales)), "mxq_hadamard_quant_fp8")
    return q, scales


# ---------------------------------------------------------------------------- FP8 block variants
def mxq_quant_fp8_blockwise(x: torch.Tensor, options: int = 0, rowwise: bool = True, columnwise: bool = False,
                            stream=None):
    """Row-wise 1x128 and/or column-wise 128x1 FP8 (codes of x^T) from one read of x
    [m][k] BF16.  options: 0 or MXQ_FP8_UE8M0.  Returns (row_codes [m][k], row_scales
    [m][k/128], col_codes [k][ld >= m], col_scales [k][ceil(m/128)]), None where not asked."""
    m, k = x.shape
    x = _bf16_bits(x)
    dev = x.device
    nb = (m + 127) // 128
    ro = co = None
    rq = rs = cq = cs = None
    if rowwise:
        rq = torch.empty((m, k), dtype=torch.uint8, device=dev)
        rs = torch.empty((m, k // 128), dtype=torch.float32, device=dev)
        ro = _FP8BlockOut(_ptr(rq), k, _ptr(rs), k // 128, 1)
    if columnwise:
        ld = (m + 15) // 16 * 16
        cq = torch.empty((k, ld), dtype=torch.uint8, device=dev)
        cs = torch.empty((k, nb), dtype=torch.float32, device=dev)
        co = _FP8BlockOut(_ptr(cq), ld, _ptr(cs), nb, 1)
    _check(lib().mxq_quant_fp8_blockwise(_ptr(x), m, k, _row_stride(x), options,
                                         ctypes.byref(ro) if ro is not None else None,
                                         ctypes.byref(co) if co is not None else None,
                                         _stream(stream, x, rq, rs, cq, cs)),
           "mxq_quant_fp8_blockwise")
    return rq, rs, (cq[:, :m] if cq is not None else None), cs


def mxq_hadamard_quant_fp8_ex(pe: Optional[torch.Tensor], nope: Optional[torch.Tensor], options: int = 0,
                              heads: int = 1, scales: Optional[torch.Tensor] = None, scale_stride_token: int = None,
                              scale_stride_head: int = None, q: Optional[torch.Tensor] = None, stream=None):
    """mxq_hadamard_quant_fp8 with options (MXQ_FP8_UE8M0) and a (token, head) scale
    layout: the scale of row r goes to scales[(r // heads) * scale_stride_token +
    (r % heads) * scale_stride_head] (defaults: [tokens][heads]).  Returns (q, scales)."""
    ref = pe if pe is not None else nope
    m = ref.shape[0]
    d_pe = pe.shape[1] if pe is not None else 0
    pe = _bf16_bits(pe) if pe is not None else None
    nope = _bf16_bits(nope) if nope is not None else None
    if q is None:
        q = torch.empty((m, 128), dtype=torch.uint8, device=ref.device)
    st = heads if scale_stride_token is None else scale_stride_token
    sh = 1 if scale_stride_head is None else scale_stride_head
    if scales is None:
        scales = torch.empty((m,), dtype=torch.float32, device=ref.device)
    _check(lib().mxq_hadamard_quant_fp8_ex(_ptr(pe), _row_stride(pe), d_pe, _ptr(nope), _row_stride(nope), m,
                                           options, heads, _ptr(q), _ptr(scales), st, sh,
                                           _stream(stream, pe, nope, q, scales)),
           "mxq_hadamard_quant_fp8_ex")
    return q, scales


# ---------------------------------------------------------------------------- SwiGLU -> FP8
def mxq_swiglu_quant_fp8(gate: torch.Tensor, up: torch.Tensor, q: Optional[torch.Tensor] = None,
                         scales: Optional[torch.Tensor] = None, scale_transposed: bool = False, stream=None):
    """FP32 SiLU(gate) * up -> FP8 1x128 along the last dim.  gate, up: [m][n] BF16 with
    unit column stride (row strides may differ: two halves of one [m][2n] buffer
    work).  Returns (codes [m][n], scales [m][n/128], or [n/128][m] when transposed)."""
    m, n = gate.shape
    if up.shape != (m, n):
        raise ValueError("gate and up must have the same shape")
    for t in (gate, up):
        if t.numel() > 0 and t.stride(1) != 1:
            raise ValueError("gate / up need unit column stride")
    gate, up = _bf16_bits(gate), _bf16_bits(up)
    if q is None:
        q = torch.empty((m, n), dtype=torch.uint8, device=gate.device)
    if scales is None:
        shape = (n // 128, m) if scale_transposed else (m, n // 128)
        scales = torch.empty(shape, dtype=torch.float32, device=gate.device)
    sr, sg = (1, m) if scale_transposed else (n // 128, 1)
    _check(lib().mxq_swiglu_quant_fp8(_ptr(gate), _row_stride(gate), _ptr(up), _row_stride(up), m, n,
                                      _ptr(q), _row_stride(q), _ptr(scales), sr, sg,
                                      _stream(stream, gate, up, q, scales)),
           "mxq_swiglu_quant_fp8")
    return q, scales


# ---------------------------------------------------------------------------- DSA rotate + NVFP4
@dataclass
class DsaNVFP4Result:
    codes: torch.Tensor                           # [m][64] uint8, even element in the low nibble
    scales: torch.Tensor                          # [m][8] uint8 (E4M3)
    global_scale: torch.Tensor                    # [1] float32
    amax: Optional[torch.Tensor] = None           # [1] float32, the measured max |y| (when asked for)


def mxq_hadamard_quant_nvfp4_workspace_size(m: int) -> int:
    return int(lib().mxq_hadamard_quant_nvfp4_workspace_size(m))


class HadamardNVFP4:
    """A prepared DSA rotate + NVFP4 call: outputs and a workspace (any contents) are
    allocated once; each call runs the quantizer on `pe`, `nope` as they are then.
    pe: [m][d_pe], nope: [m][128-d_pe] BF16 with unit column stride (either may be
    None when empty).  amax_in: None (measure), a float, or a device float32 tensor
    of one element.  amax_out: also return the measured max |y|."""

    def __init__(self, pe: Optional[torch.Tensor], nope: Optional[torch.Tensor], amax_in=None,
                 amax_out: bool = False, workspace: Optional[torch.Tensor] = None):
        ref = pe if pe is not None else nope
        self.m = ref.shape[0]
        self.d_pe = pe.shape[1] if pe is not None else 0
        for t in (pe, nope):
            if t is not None and t.numel() > 0 and t.stride(1) != 1:
                raise ValueError("pe / nope need unit column stride")
        self.pe = _bf16_bits(pe) if pe is not None else None
        self.nope = _bf16_bits(nope) if nope is not None else None
        dev = ref.device
        self.out = DsaNVFP4Result(torch.empty((self.m, 64), dtype=torch.uint8, device=dev),
                                  torch.empty((self.m, 8), dtype=torch.uint8, device=dev),
                                  torch.empty((1,), dtype=torch.float32, device=dev),
                                  torch.empty((1,), dtype=torch.float32, device=dev) if amax_out else None)
        if amax_in is not None and not isinstance(amax_in, torch.Tensor):
            amax_in = torch.tensor([float(amax_in)], dtype=torch.float32, device=dev)
        self.amax_in = amax_in
        need = mxq_hadamard_quant_nvfp4_workspace_size(self.m)
        if workspace is None:
            workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
        self.workspace = workspace

    def __call__(self, stream=None) -> DsaNVFP4Result:
        o = self.out
        _check(lib().mxq_hadamard_quant_nvfp4(
            _ptr(self.pe), _row_stride(self.pe), self.d_pe, _ptr(self.nope), _row_stride(self.nope), self.m,
            _ptr(self.amax_in), _ptr(o.amax), _ptr(o.codes), _ptr(o.scales), _ptr(o.global_scale),
            _ptr(self.workspace), self.workspace.numel(),
            _stream(stream, self.pe, self.nope, self.amax_in, o.amax, o.codes, o.scales, o.global_scale,
                    self.workspace)), "mxq_hadamard_quant_nvfp4")
        return o


def mxq_hadamard_quant_nvfp4(pe: Optional[torch.Tensor], nope: Optional[torch.Tensor], amax_in=None,
                             amax_out: bool = False, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> DsaNVFP4Result:
    """cat[pe, nope] -> normalized 128-point WHT -> BF16 -> NVFP4 row-wise (1x16 blocks,
    one tensor scale over the call)."""
    return HadamardNVFP4(pe, nope, amax_in, amax_out, workspace)(stream)


# ---------------------------------------------------------------------------- grouped NVFP4
@dataclass
class NVFP4Result:
    row_codes: Optional[torch.Tensor] = None      # [total][k/2] uint8
    row_scales: Optional[torch.Tensor] = None     # [total][k/16] uint8 (E4M3)
    row_global: Optional[torch.Tensor] = None     # [S] float32
    col_codes: Optional[torch.Tensor] = None      # flat; section s at k*R_s/2 as [k][m_s/2]
    col_scales: Optional[torch.Tensor] = None     # flat; section s at k*R_s/16 as [k][m_s/16]
    col_global: Optional[torch.Tensor] = None     # [S] float32
    fp8_codes: Optional[torch.Tensor] = None      # [total][k] uint8
    fp8_scales: Optional[torch.Tensor] = None     # [total][k/128] float32
    row_amax: Optional[torch.Tensor] = None       # [S] float32, measured (when asked for)
    col_amax: Optional[torch.Tensor] = None       # [S] float32, measured (when asked for)


def mxq_group_rht_quant_nvfp4_workspace_size(total_rows: int, k: int, num_sections: int, flags: int) -> int:
    return int(lib().mxq_group_rht_quant_nvfp4_workspace_size(total_rows, k, num_sections, flags))


def alloc_nvfp4_outputs(total_rows: int, k: int, num_sections: int, flags: int, device) -> NVFP4Result:
    r = NVFP4Result()
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    if flags & MXQ_ROWWISE:
        r.row_codes = torch.empty((total_rows, k // 2), **u8)
        r.row_scales = torch.empty((total_rows, k // 16), **u8)
        r.row_global = torch.empty((num_sections,), **f32)
    if flags & MXQ_COLUMNWISE:
        r.col_codes = torch.empty((total_rows * k // 2,), **u8)
        r.col_scales = torch.empty((total_rows * k // 16,), **u8)
        r.col_global = torch.empty((num_sections,), **f32)
    if flags & MXQ_FP8_ROWWISE:
        r.fp8_codes = torch.empty((total_rows, k), **u8)
        r.fp8_scales = torch.empty((total_rows, k // 128), **f32)
    return r


def alloc_workspace(total_rows: int, k: int, num_sections: int, flags: int, device) -> torch.Tensor:
    """Zero-filled workspace of the size the library asks for (the single-read form
    needs its partial words and error word at zero before the first use and leaves
    them at zero)."""
    n = mxq_group_rht_quant_nvfp4_workspace_size(total_rows, k, num_sections, flags)
    return torch.zeros((max(n, 256),), dtype=torch.uint8, device=device)


WORKSPACE_STATUS = 0                                  # byte offset of the single-read form's error word
WORKSPACE_TABLES = WORKSPACE_STATUS + 512            # float4 (d, 1/d, multiplier, mask) at (s * 2 + dir) * 128 + code
WORKSPACE_SLOTS = WORKSPACE_TABLES + 32 * 2 * 128 * 16         # the single-read form's partial words
WORKSPACE_SLOTS_BYTES = 4 * 1024
WORKSPACE_FIXED = WORKSPACE_SLOTS + WORKSPACE_SLOTS_BYTES      # then the amax pass's partials


def workspace_protocol_clear(workspace: torch.Tensor) -> bool:
    """After a finished call: True when the single-read form's error word and partial
    words are back at zero (the only workspace words a call needs at zero)."""
    if int(workspace[WORKSPACE_STATUS:WORKSPACE_STATUS + 4].view(torch.int32).item()) != 0:
        return False
    slots = workspace[WORKSPACE_SLOTS:WORKSPACE_SLOTS + WORKSPACE_SLOTS_BYTES]
    return bool((slots == 0).all().item())


class GroupedNVFP4:
    """A prepared grouped call: the ctypes argument structures are built once, so
    repeated calls (benchmarks, stream capture) only pay for the launch itself."""

    def __init__(self, x: torch.Tensor, split_sections: Sequence[int], rht_sign_mask: int, flags: int,
                 seed: Optional[int] = None, row_offsets: Optional[Sequence[int]] = None,
                 col_offsets: Optional[Sequence[int]] = None, out: Optional[NVFP4Result] = None,
                 workspace: Optional[torch.Tensor] = None, amax_in: Optional[tuple] = None,
                 amax_out: bool = False):
        """amax_in: None, or (row maxima, column maxima) device float32 [S] tensors (None
        for a direction not requested) that replace the measured section maxima;
        amax_out: also return the measured maxima (out.row_amax / out.col_amax)."""
        x = _bf16_bits(x)
        if not x.is_contiguous():
            raise ValueError("x must be contiguous [total_rows][k]")
        self.x = x
        total, k = x.shape
        S = len(split_sections)
        self.k, self.total, self.S, self.flags, self.mask = k, total, S, flags, rht_sign_mask & 0xFFFF
        self.sections = (ctypes.c_int64 * max(S, 1))(*[int(v) for v in split_sections])
        self.out = out if out is not None else alloc_nvfp4_outputs(total, k, S, flags, x.device)
        self.workspace = workspace if workspace is not None else alloc_workspace(total, k, S, flags, x.device)
        o = self.out
        self._row = _NVFP4Out(o.row_codes.data_ptr() if o.row_codes is not None else None,
                              o.row_scales.data_ptr() if o.row_scales is not None else None,
                              o.row_global.data_ptr() if o.row_global is not None else None)
        self._col = _NVFP4Out(o.col_codes.data_ptr() if o.col_codes is not None else None,
                              o.col_scales.data_ptr() if o.col_scales is not None else None,
                              o.col_global.data_ptr() if o.col_global is not None else None)
        self._fp8 = _FP8Out(o.fp8_codes.data_ptr() if o.fp8_codes is not None else None,
                            o.fp8_scales.data_ptr() if o.fp8_scales is not None else None)
        self._amax = None
        if amax_in is not None or amax_out:
            f32 = dict(dtype=torch.float32, device=x.device)
            if amax_out:
                o.row_amax = torch.zeros((S,), **f32) if flags & MXQ_ROWWISE else None
                o.col_amax = torch.zeros((S,), **f32) if flags & MXQ_COLUMNWISE else None
            self._amax_in = [None if a is None else a.contiguous().float() for a in (amax_in or (None, None))]
            self._amax = _Amax(*[None if a is None else a.data_ptr() for a in self._amax_in],
                               o.row_amax.data_ptr() if o.row_amax is not None else None,
                               o.col_amax.data_ptr() if o.col_amax is not None else None)
        self._sr = None
        if seed is not None and (row_offsets is not None or col_offsets is not None):
            self._ro = (ctypes.c_uint64 * S)(*row_offsets) if row_offsets is not None else None
            self._co = (ctypes.c_uint64 * S)(*col_offsets) if col_offsets is not None else None
            self._sr = _SR(seed & ((1 << 64) - 1),
                           ctypes.addressof(self._ro) if self._ro is not None else None,
                           ctypes.addressof(self._co) if self._co is not None else None)

    def _tensors(self) -> list:
        return [self.x, self.workspace, *_out_tensors(self.out),
                *(self._amax_in if self._amax is not None else ())]

    def __call__(self, stream=None) -> NVFP4Result:
        if self._amax is None:
            st = lib().mxq_group_rht_quant_nvfp4(
                _ptr(self.x), self.k, ctypes.addressof(self.sections), self.S, self.mask, self.flags,
                ctypes.addressof(self._sr) if self._sr is not None else None,
                ctypes.addressof(self._row), ctypes.addressof(self._col), ctypes.addressof(self._fp8),
                _ptr(self.workspace), self.workspace.numel(), _stream(stream, *self._tensors()))
            _check(st, "mxq_group_rht_quant_nvfp4")
        else:
            st = lib().mxq_group_rht_quant_nvfp4_with_amax(
                _ptr(self.x), self.k, ctypes.addressof(self.sections), self.S, self.mask, self.flags,
                ctypes.addressof(self._sr) if self._sr is not None else None,
                ctypes.addressof(self._row), ctypes.addressof(self._col), ctypes.addressof(self._fp8),
                ctypes.addressof(self._amax), _ptr(self.workspace), self.workspace.numel(),
                _stream(stream, *self._tensors()))
            _check(st, "mxq_group_rht_quant_nvfp4_with_amax")
        return self.out


def mxq_group_rht_quant_nvfp4_noalloc(x: torch.Tensor, split_sections: Sequence[int], rht_sign_mask: int,
                                      flags: int, seed: Optional[int] = None,
                                      row_offsets: Optional[Sequence[int]] = None,
                                      col_offsets: Optional[Sequence[int]] = None,
                                      out: NVFP4Result = None, stream=None) -> NVFP4Result:
    """The grouped call without a workspace: the library's per-device scratch array
    (MXQ_NOALLOC_SCRATCH_BYTES) stands in for it.  `out` must be allocated beforehand
    (alloc_nvfp4_outputs) by a caller that cannot allocate during the call."""
    x = _bf16_bits(x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous [total_rows][k]")
    total, k = x.shape
    S = len(split_sections)
    if out is None:
        out = alloc_nvfp4_outputs(total, k, S, flags, x.device)
    sections = (ctypes.c_int64 * max(S, 1))(*[int(v) for v in split_sections])
    row = _NVFP4Out(_addr(out.row_codes), _addr(out.row_scales), _addr(out.row_global))
    col = _NVFP4Out(_addr(out.col_codes), _addr(out.col_scales), _addr(out.col_global))
    fp8 = _FP8Out(_addr(out.fp8_codes), _addr(out.fp8_scales))
    sr = ro = co = None
    if seed is not None and (row_offsets is not None or col_offsets is not None):
        ro = (ctypes.c_uint64 * S)(*row_offsets) if row_offsets is not None else None
        co = (ctypes.c_uint64 * S)(*col_offsets) if col_offsets is not None else None
        sr = _SR(seed & ((1 << 64) - 1), ctypes.addressof(ro) if ro is not None else None,
                 ctypes.addressof(co) if co is not None else None)
    st = lib().mxq_group_rht_quant_nvfp4_noalloc(
        _ptr(x), k, ctypes.addressof(sections), S, rht_sign_mask & 0xFFFF, flags,
        ctypes.addressof(sr) if sr is not None else None, ctypes.addressof(row), ctypes.addressof(col),
        ctypes.addressof(fp8), _stream(stream, x, *_out_tensors(out)))
    _check(st, "mxq_group_rht_quant_nvfp4_noalloc")
    return out


def _out_tensors(o: NVFP4Result) -> list:
    return [o.row_codes, o.row_scales, o.row_global, o.col_codes, o.col_scales, o.col_global, o.fp8_codes,
            o.fp8_scales, o.row_amax, o.col_amax]


def _addr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def mxq_group_rht_quant_nvfp4(x: torch.Tensor, split_sections: Sequence[int], rht_sign_mask: int, flags: int,
                              seed: Optional[int] = None, row_offsets: Optional[Sequence[int]] = None,
                              col_offsets: Optional[Sequence[int]] = None, out: Optional[NVFP4Result] = None,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> NVFP4Result:
    """Grouped NVFP4 (row-wise; column-wise after the 16-point RHT) and optional
    FP8 1x128 row-wise outputs of a BF16 [total_rows][k] tensor."""
    return GroupedNVFP4(x, split_sections, rht_sign_mask, flags, seed, row_offsets, col_offsets, out,
                        workspace)(stream)
