"""Thin Python binding of libpdq (include/pdq.h), same names without the prefix.

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI.  PyTorch provides device memory (outputs are allocated with
torch.empty on the input's device) and the stream (the current stream).
There is no fallback: if libpdq.so is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

LIB_PATH = os.environ.get("PDQ_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                      "libpdq.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pdq.h")

F32, BF16, F16 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}

_vp, _i64, _f32, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32, ctypes.c_size_t

SIGNATURES = {
    "pdq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pdq_quantize_weight": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "pdq_calibrate_static": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "pdq_linear_prefill": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _i64,
                                          _vp, _vp, _vp, _i64, _vp, _vp]),
    "pdq_linear_decode": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _i32, _vp, _vp,
                                         _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp]),
    "pdq_quantize_per_token": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp]),
    "pdq_gemm_per_token": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                          _vp]),
    "pdq_quantize_static": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _i32, _vp, _vp,
                                           _vp]),
    "pdq_gemm_static": (ctypes.c_int, [_vp, _i64, _i64, _f32, _i32, _vp, _vp, _vp, _vp, _i64, _vp,
                                       _i64, _vp, _vp]),
    "pdq_quantize_per_token_asym": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp,
                                                   _vp]),
    "pdq_gemm_per_token_asym": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp,
                                               _i64, _vp, _vp]),
    "pdq_linear_prefill_asym": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                                               _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp]),
    "pdq_calibrate_static_sym": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp]),
    "pdq_quantize_static_sym": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _vp, _vp, _vp]),
    "pdq_linear_static_sym": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _i64,
                                             _vp, _vp, _i64, _vp, _vp, _vp]),
    "pdq_calibrate_zeropoint": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "pdq_quantize_zeropoint": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _i32, _vp, _vp, _vp]),
    "pdq_linear_zeropoint": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _i32, _vp, _vp, _vp, _vp,
                                            _i64, _vp, _vp, _i64, _vp, _vp, _vp]),
    "pdq_silu_mul_quantize_per_token": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _vp,
                                                       _vp, _i64, _vp]),
    "pdq_linear_prefill_silu_mul": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                                   _i64, _vp, _vp, _vp, _i64, _vp, _vp]),
    "pdq_linear_int8_outlier_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "pdq_weight_bytes": (_sz, [_i64, _i64]),
    "pdq_act_bytes": (_sz, [_i64, _i64]),
    "pdq_gemm_kernel": (ctypes.c_int, [_i64, _i64]),
    "pdq_skinny_channels": (ctypes.c_int, [_i64, _i64]),
    "pdq_pack_int8": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "pdq_unpack_int8": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp]),
    "pdq_linear_int8_outlier": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _vp, _vp,
                                               _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                               _i64, _vp, _sz, _vp, _vp]),
    "pdq_noalloc_scratch_bytes": (_sz, []),
    "pdq_linear_int8_outlier_noalloc": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _vp, _vp,
                                                       _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                                       _i64, _vp, _vp]),
}

_lib = None


class PdqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions include/pdq.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(pdq_\w+)\s*\(", text, flags=re.M)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(python -m w8a8_int8_quantized_absmax_amd.build_lib)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pdq_status_string(status).decode()


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise PdqError(name, st)


def _p(t):
    if t is None:
        return None
    return ctypes.c_void_p((t.data if isinstance(t, Codes) else t).data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_mat(t: torch.Tensor, name: str, dtypes=_DT):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or (t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit stride in the last dimension")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")


def _ld(t: torch.Tensor) -> int:
    """Row pitch in elements (a single or empty row has no meaningful stride)."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


# ---------------------------------------------------------------------------

def weight_bytes(n: int, k: int) -> int:
    """Bytes of the packed INT8 weight of N output channels x K (include/pdq.h)."""
    return int(lib().pdq_weight_bytes(n, k))


def act_bytes(m: int, k: int) -> int:
    """Bytes of the packed INT8 activation codes of M rows x K (include/pdq.h)."""
    return int(lib().pdq_act_bytes(m, k))


def unpack(buf: torch.Tensor, rows: int, k: int, padded: bool = False):
    """The codes [rows, k] of a packed INT8 matrix (weight or activations) as a host int8 array.

    Layout (include/pdq.h): 1024-byte blocks of 16 rows x 64 K values, block
    (g, s) at (g * ceil(K / 64) + s) * 1024, row r at r * 64 in it, its
    16-byte chunk c at position c ^ ((r >> 2) & 3).  padded: the whole
    [16 ceil(rows / 16), 64 ceil(k / 64)] matrix, padding included.
    """
    import numpy as np

    ng, kt = (rows + 15) // 16, (k + 63) // 64
    b = buf.detach().cpu().numpy()[:ng * kt * 1024].reshape(ng, kt, 16, 4, 16)
    r = np.arange(16)[:, None]
    pos = np.arange(4)[None, :] ^ ((r >> 2) & 3)  # [r, c] -> position of chunk c
    out = b[:, :, r, pos, :]                      # [ng, kt, 16, 4, 16], chunks in K order
    out = out.transpose(0, 2, 1, 3, 4).reshape(ng * 16, kt * 64)
    return out if padded else out[:rows, :k]


unpack_weight = unpack


def gemm_kernel(m: int, n: int) -> str:
    """The GEMM kernel the library runs for M activation rows x N channels: "skinny" or "tiled"."""
    return {0: "skinny", 1: "tiled"}.get(int(lib().pdq_gemm_kernel(m, n)), "none")


def pack_int8(x: torch.Tensor) -> torch.Tensor:
    """A plain int8 [rows, K] device matrix -> its packed image (pdq_weight_bytes(rows, K) bytes), the
    layout every GEMM takes its weight and activation codes in."""
    _check_mat(x, "x", (torch.int8,))
    rows, k = x.shape
    out = torch.empty(weight_bytes(rows, k), dtype=torch.int8, device=x.device)
    _call("pdq_pack_int8", _p(x), rows, k, _ld(x), _p(out), _stream(x.device))
    return out


def unpack_int8(packed: torch.Tensor, rows: int, k: int, out=None) -> torch.Tensor:
    """The packed image of an int8 [rows, K] matrix -> the plain [rows, K] int8 matrix on the device."""
    dst = out if out is not None else torch.empty((rows, k), dtype=torch.int8, device=packed.device)
    _call("pdq_unpack_int8", _p(packed), rows, k, _p(dst), _ld(dst), _stream(packed.device))
    return dst


def skinny_channels(m: int, n: int) -> int:
    """Weight channels per workgroup of the skinny kernel for M rows x N channels (16 .. 64)."""
    return int(lib().pdq_skinny_channels(m, n))


class Codes:
    """INT8 activation codes of a [rows, k] matrix in the packed layout (include/pdq.h).

    data: contiguous int8 device tensor of at least act_bytes(rows, k) bytes.
    """

    __slots__ = ("data", "rows", "k")

    def __init__(self, data: torch.Tensor, rows: int, k: int):
        if not data.is_cuda or data.dtype != torch.int8 or not data.is_contiguous():
            raise ValueError("packed codes must be a contiguous int8 device tensor")
        if data.numel() < act_bytes(rows, k):
            raise ValueError(f"{data.numel()} bytes cannot hold packed {rows} x {k} codes "
                             f"({act_bytes(rows, k)} needed)")
        self.data, self.rows, self.k = data, int(rows), int(k)

    @classmethod
    def empty(cls, rows: int, k: int, device) -> "Codes":
        return cls(torch.empty(max(act_bytes(rows, k), 1), dtype=torch.int8, device=device), rows, k)

    @property
    def shape(self):
        return (self.rows, self.k)

    def unpack(self, padded: bool = False):
        """Host int8 array [rows, k] (padded: with the zero padding rows and K values)."""
        return unpack(self.data, self.rows, self.k, padded)


def _codes_out(xq, m: int, k: int, device) -> Codes:
    if xq is None:
        return Codes.empty(m, k, device)
    if isinstance(xq, Codes):
        if xq.shape != (m, k):
            raise ValueError(f"codes of shape {xq.shape} given for a {m} x {k} activation")
        return xq
    return Codes(xq, m, k)


def _codes_in(xq) -> Codes:
    if not isinstance(xq, Codes):
        raise ValueError("xq must be packed activation codes (a Codes object)")
    return xq


def _check_weight(wq: torch.Tensor, n: int, k: int):
    if not wq.is_cuda or wq.dtype != torch.int8 or not wq.is_contiguous():
        raise ValueError("wq must be a contiguous int8 device tensor (a packed weight)")
    if wq.numel() < weight_bytes(n, k):
        raise ValueError(f"wq holds {wq.numel()} bytes, a packed {n} x {k} weight needs {weight_bytes(n, k)}")


def quantize_weight(w: torch.Tensor):
    """Per-output-channel symmetric INT8 weight -> (packed wq int8, w_scale f32 [N], colsum i32 [N])."""
    _check_mat(w, "w")
    n, k = w.shape
    wq = torch.empty(weight_bytes(n, k), dtype=torch.int8, device=w.device)
    ws = torch.empty(n, dtype=torch.float32, device=w.device)
    cs = torch.empty(n, dtype=torch.int32, device=w.device)
    _call("pdq_quantize_weight", _p(w), _DT[w.dtype], n, k, _ld(w), _p(wq), _p(ws), _p(cs),
          _stream(w.device))
    return wq, ws, cs


def minmax_state(device) -> torch.Tensor:
    """A fresh MinMax observer state {+INF, -INF}."""
    return torch.tensor([float("inf"), float("-inf")], dtype=torch.float32, device=device)


def calibrate_static(x: torch.Tensor, minmax: torch.Tensor, finalize: bool = False):
    """Update the MinMax state with batch x; if finalize, return (a_scale, a_zp) device tensors."""
    _check_mat(x, "x")
    m, k = x.shape
    s = z = None
    if finalize:
        s = torch.empty(1, dtype=torch.float32, device=x.device)
        z = torch.empty(1, dtype=torch.int32, device=x.device)
    _call("pdq_calibrate_static", _p(x), _DT[x.dtype], m, k, _ld(x), _p(minmax), _p(s), _p(z),
          _stream(x.device))
    return (s, z) if finalize else None


def linear_prefill(x, wq, w_scale, bias=None, want_acc: bool = False, out=None):
    """Per-token dynamic symmetric W8A8 linear -> dict(y bf16, xq, x_scale[, acc])."""
    _check_mat(x, "x")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    xq = Codes.empty(m, k, x.device)
    xs = torch.empty(m, dtype=torch.float32, device=x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if want_acc else None
    _call("pdq_linear_prefill", _p(x), _DT[x.dtype], m, k, _ld(x), _p(wq), _p(w_scale), _p(bias),
          n, _p(xq), _p(xs), _p(y), _ld(y), _p(acc), _stream(x.device))
    return dict(y=y, xq=xq, x_scale=xs, acc=acc)


def linear_prefill_asym(x, wq, w_scale, colsum, bias=None, want_acc: bool = False, out=None):
    """Per-token dynamic asymmetric W8A8 linear -> dict(y bf16, xq, x_scale, x_zp[, acc])."""
    _check_mat(x, "x")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    xq = Codes.empty(m, k, x.device)
    xs = torch.empty(m, dtype=torch.float32, device=x.device)
    xz = torch.empty(m, dtype=torch.int32, device=x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if want_acc else None
    _call("pdq_linear_prefill_asym", _p(x), _DT[x.dtype], m, k, _ld(x), _p(wq), _p(w_scale), _p(colsum),
          _p(bias), n, _p(xq), _p(xs), _p(xz), _p(y), _ld(y), _p(acc), _stream(x.device))
    return dict(y=y, xq=xq, x_scale=xs, x_zp=xz, acc=acc)


def quantize_per_token_asym(x, xq=None, x_scale=None, x_zp=None):
    """Per-token dynamic asymmetric INT8 -> (xq packed Codes [M,K], x_scale f32 [M], x_zp i32 [M])."""
    _check_mat(x, "x")
    m, k = x.shape
    xq = _codes_out(xq, m, k, x.device)
    xs = x_scale if x_scale is not None else torch.empty(m, dtype=torch.float32, device=x.device)
    xz = x_zp if x_zp is not None else torch.empty(m, dtype=torch.int32, device=x.device)
    _call("pdq_quantize_per_token_asym", _p(x), _DT[x.dtype], m, k, _ld(x), _p(xq), _p(xs), _p(xz),
          _stream(x.device))
    return xq, xs, xz


def gemm_per_token_asym(xq, x_scale, x_zp, wq, w_scale, colsum, bias=None, want_acc: bool = False, out=None):
    """INT8 GEMM + per-token zero-point correction + dequant epilogue -> dict(y bf16[, acc])."""
    xq = _codes_in(xq)
    m, k = xq.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    dev = xq.data.device
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    _call("pdq_gemm_per_token_asym", _p(xq), _p(x_scale), _p(x_zp), m, k, _p(wq), _p(w_scale), _p(colsum),
          _p(bias), n, _p(y), _ld(y), _p(acc), _stream(dev))
    return dict(y=y, acc=acc)


def linear_decode(x, a_scale: float, a_zp: int, wq, w_scale, colsum, bias=None,
                  sat_count=None, want_acc: bool = False, out=None, xq=None):
    """Per-tensor static asymmetric W8A8 linear -> dict(y bf16, xq[, acc])."""
    _check_mat(x, "x")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    xq = _codes_out(xq, m, k, x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if want_acc else None
    _call("pdq_linear_decode", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), int(a_zp),
          _p(wq), _p(w_scale), _p(colsum), _p(bias), n, _p(xq), _p(y), _ld(y), _p(acc),
          _p(sat_count), _stream(x.device))
    return dict(y=y, xq=xq, acc=acc)


def calibrate_static_sym(x: torch.Tensor, minmax: torch.Tensor, finalize: bool = False):
    """Update the MinMax state with batch x; if finalize, return the tensor-wise absmax scale (device [1])."""
    _check_mat(x, "x")
    m, k = x.shape
    s = torch.empty(1, dtype=torch.float32, device=x.device) if finalize else None
    _call("pdq_calibrate_static_sym", _p(x), _DT[x.dtype], m, k, _ld(x), _p(minmax), _p(s), _stream(x.device))
    return s


def quantize_static_sym(x, a_scale: float, xq=None, sat_count=None):
    """Static tensor-wise symmetric INT8 -> xq packed Codes [M,K]."""
    _check_mat(x, "x")
    m, k = x.shape
    xq = _codes_out(xq, m, k, x.device)
    _call("pdq_quantize_static_sym", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), _p(xq),
          _p(sat_count), _stream(x.device))
    return xq


def linear_static_sym(x, a_scale: float, wq, w_scale, bias=None, sat_count=None, want_acc: bool = False,
                      out=None, xq=None):
    """Static tensor-wise symmetric W8A8 linear -> dict(y bf16, xq[, acc])."""
    _check_mat(x, "x")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    xq = _codes_out(xq, m, k, x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if want_acc else None
    _call("pdq_linear_static_sym", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), _p(wq), _p(w_scale),
          _p(bias), n, _p(xq), _p(y), _ld(y), _p(acc), _p(sat_count), _stream(x.device))
    return dict(y=y, xq=xq, acc=acc)


def calibrate_zeropoint(x: torch.Tensor, minmax: torch.Tensor, finalize: bool = False):
    """Update the MinMax state with batch x; if finalize, return the 254-level zero-point grid's (S, Z) device tensors."""
    _check_mat(x, "x")
    m, k = x.shape
    s = z = None
    if finalize:
        s = torch.empty(1, dtype=torch.float32, device=x.device)
        z = torch.empty(1, dtype=torch.int32, device=x.device)
    _call("pdq_calibrate_zeropoint", _p(x), _DT[x.dtype], m, k, _ld(x), _p(minmax), _p(s), _p(z),
          _stream(x.device))
    return (s, z) if finalize else None


def quantize_zeropoint(x, a_scale: float, a_zp: int, xq=None, sat_count=None):
    """Static tensor-wise zero-point INT8 (254 levels) -> xq packed Codes [M,K]."""
    _check_mat(x, "x")
    m, k = x.shape
    xq = _codes_out(xq, m, k, x.device)
    _call("pdq_quantize_zeropoint", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), int(a_zp), _p(xq),
          _p(sat_count), _stream(x.device))
    return xq


def linear_zeropoint(x, a_scale: float, a_zp: int, wq, w_scale, colsum, bias=None, sat_count=None,
                     want_acc: bool = False, out=None, xq=None):
    """Static tensor-wise zero-point W8A8 linear (254 levels) -> dict(y bf16, xq[, acc])."""
    _check_mat(x, "x")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    xq = _codes_out(xq, m, k, x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if want_acc else None
    _call("pdq_linear_zeropoint", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), int(a_zp), _p(wq),
          _p(w_scale), _p(colsum), _p(bias), n, _p(xq), _p(y), _ld(y), _p(acc), _p(sat_count), _stream(x.device))
    return dict(y=y, xq=xq, acc=acc)


def int8_outlier_workspace_bytes(m: int, n: int, k: int, max_outliers: int) -> int:
    return int(lib().pdq_linear_int8_outlier_workspace(m, n, k, max_outliers))


def linear_int8_outlier(x, threshold: float, wq, w_scale, w16, bias=None, max_outliers: int = 64,
                        want_acc: bool = False, workspace=None, out=None):
    """LLM.int8() vector-wise INT8 + 16-bit outlier decomposition -> dict(y, xq, x_scale, idx, count[, acc])."""
    _check_mat(x, "x")
    _check_mat(w16, "w16")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    dev = x.device
    max_outliers = min(max_outliers, k)
    xq = Codes.empty(m, k, dev)
    xs = torch.empty(m, dtype=torch.float32, device=dev)
    idx = torch.empty(max(max_outliers, 1), dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    y = out if out is not None else torch.empty((m, n), dtype=x.dtype, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    need = int8_outlier_workspace_bytes(m, n, k, max_outliers)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _call("pdq_linear_int8_outlier", _p(x), _DT[x.dtype], m, k, _ld(x), float(threshold), _p(wq),
          _p(w_scale), _p(w16), _ld(w16), _p(bias), n, _p(y), _ld(y), _p(xq), _p(xs), _p(idx),
          _p(cnt), max_outliers, _p(workspace), workspace.numel(), _p(acc), _stream(dev))
    return dict(y=y, xq=xq, x_scale=xs, idx=idx, count=cnt, acc=acc)


def linear_int8_outlier_noalloc(x, threshold: float, wq, w_scale, w16, bias=None, max_outliers: int = 64,
                                want_acc: bool = False, out=None, xq=None, x_scale=None, idx=None, count=None):
    """linear_int8_outlier on the library's own scratch instead of a workspace (the
    call itself allocates nothing; outputs not given are allocated here)."""
    _check_mat(x, "x")
    _check_mat(w16, "w16")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    dev = x.device
    max_outliers = min(max_outliers, k)
    xq = _codes_out(xq, m, k, dev)
    xs = x_scale if x_scale is not None else torch.empty(m, dtype=torch.float32, device=dev)
    idx = idx if idx is not None else torch.empty(max(max_outliers, 1), dtype=torch.int32, device=dev)
    cnt = count if count is not None else torch.empty(1, dtype=torch.int32, device=dev)
    y = out if out is not None else torch.empty((m, n), dtype=x.dtype, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    _call("pdq_linear_int8_outlier_noalloc", _p(x), _DT[x.dtype], m, k, _ld(x), float(threshold), _p(wq),
          _p(w_scale), _p(w16), _ld(w16), _p(bias), n, _p(y), _ld(y), _p(xq), _p(xs), _p(idx),
          _p(cnt), max_outliers, _p(acc), _stream(dev))
    return dict(y=y, xq=xq, x_scale=xs, idx=idx, count=cnt, acc=acc)


def noalloc_scratch_bytes() -> int:
    return int(lib().pdq_noalloc_scratch_bytes())


def quantize_per_token(x, xq=None, x_scale=None):
    """Per-token dynamic symmetric INT8 -> (xq packed Codes [M,K], x_scale f32 [M])."""
    _check_mat(x, "x")
    m, k = x.shape
    xq = _codes_out(xq, m, k, x.device)
    xs = x_scale if x_scale is not None else torch.empty(m, dtype=torch.float32, device=x.device)
    _call("pdq_quantize_per_token", _p(x), _DT[x.dtype], m, k, _ld(x), _p(xq), _p(xs), _stream(x.device))
    return xq, xs


_HALF = (torch.bfloat16, torch.float16)


def _check_gate_up(gate, up):
    _check_mat(gate, "gate", _HALF)
    _check_mat(up, "up", _HALF)
    if up.shape != gate.shape or up.dtype != gate.dtype:
        raise ValueError("gate and up must have the same shape and dtype")
    return gate.shape


def silu_mul_quantize_per_token(gate, up, xq=None, x_scale=None, h=None):
    """h = SiLU(gate) * up (rounded to gate's 16-bit dtype) quantized per token
    -> (xq packed Codes [M,K], x_scale f32 [M]).  h: optional [M,K] tensor of
    that dtype that also receives the product."""
    m, k = _check_gate_up(gate, up)
    xq = _codes_out(xq, m, k, gate.device)
    xs = x_scale if x_scale is not None else torch.empty(m, dtype=torch.float32, device=gate.device)
    if h is not None:
        _check_mat(h, "h", (gate.dtype,))
        if h.shape != gate.shape:
            raise ValueError("h must have gate's shape")
    _call("pdq_silu_mul_quantize_per_token", _p(gate), _p(up), _DT[gate.dtype], m, k, _ld(gate), _ld(up),
          _p(xq), _p(xs), _p(h), _ld(h) if h is not None else 0, _stream(gate.device))
    return xq, xs


def linear_prefill_silu_mul(gate, up, wq, w_scale, bias=None, want_acc: bool = False, out=None):
    """Down projection of h = SiLU(gate) * up, per-token dynamic symmetric W8A8
    -> dict(y bf16, xq, x_scale[, acc]); K is the intermediate size."""
    m, k = _check_gate_up(gate, up)
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    xq = Codes.empty(m, k, gate.device)
    xs = torch.empty(m, dtype=torch.float32, device=gate.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=gate.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=gate.device) if want_acc else None
    _call("pdq_linear_prefill_silu_mul", _p(gate), _p(up), _DT[gate.dtype], m, k, _ld(gate), _ld(up), _p(wq),
          _p(w_scale), _p(bias), n, _p(xq), _p(xs), _p(y), _ld(y), _p(acc), _stream(gate.device))
    return dict(y=y, xq=xq, x_scale=xs, acc=acc)


def gemm_per_token(xq, x_scale, wq, w_scale, bias=None, want_acc: bool = False, out=None):
    """INT8 GEMM + per-token/per-channel dequant epilogue -> dict(y bf16[, acc])."""
    xq = _codes_in(xq)
    m, k = xq.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    dev = xq.data.device
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    _call("pdq_gemm_per_token", _p(xq), _p(x_scale), m, k, _p(wq), _p(w_scale), _p(bias), n, _p(y),
          _ld(y), _p(acc), _stream(dev))
    return dict(y=y, acc=acc)


def quantize_static(x, a_scale: float, a_zp: int, xq=None, sat_count=None):
    """Per-tensor static asymmetric INT8 -> xq packed Codes [M,K]."""
    _check_mat(x, "x")
    m, k = x.shape
    xq = _codes_out(xq, m, k, x.device)
    _call("pdq_quantize_static", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), int(a_zp), _p(xq),
          _p(sat_count), _stream(x.device))
    return xq


def gemm_static(xq, a_scale: float, a_zp: int, wq, w_scale, colsum, bias=None, want_acc: bool = False,
                out=None):
    """INT8 GEMM + zero-point correction + dequant epilogue -> dict(y bf16[, acc])."""
    xq = _codes_in(xq)
    m, k = xq.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    dev = xq.data.device
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    _call("pdq_gemm_static", _p(xq), m, k, float(a_scale), int(a_zp), _p(wq), _p(w_scale), _p(colsum),
          _p(bias), n, _p(y), _ld(y), _p(acc), _stream(dev))
    return dict(y=y, acc=acc)
