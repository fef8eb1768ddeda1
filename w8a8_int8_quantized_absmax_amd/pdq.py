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
    "pdq_linear_int8_outlier_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "pdq_weight_bytes": (_sz, [_i64, _i64]),
    "pdq_linear_int8_outlier": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _vp, _vp,
                                               _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                               _i64, _vp, _sz, _vp, _vp]),
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
    return None if t is None else ctypes.c_void_p(t.data_ptr())


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


def unpack_weight(wq: torch.Tensor, n: int, k: int):
    """The codes wq[n, k] of a packed weight as a host int8 array [N, K].

    Layout (include/pdq.h): 1024-byte blocks of 16 channels x 64 K values,
    block (g, s) at (g * ceil(K / 64) + s) * 1024, channel r at r * 64 in it,
    its 16-byte chunk c at position c ^ ((r >> 2) & 3).
    """
    import numpy as np

    ng, kt = (n + 15) // 16, (k + 63) // 64
    b = wq.detach().cpu().numpy()[:ng * kt * 1024].reshape(ng, kt, 16, 4, 16)
    r = np.arange(16)[:, None]
    pos = np.arange(4)[None, :] ^ ((r >> 2) & 3)  # [r, c] -> position of chunk c
    out = b[:, :, r, pos, :]                      # [ng, kt, 16, 4, 16], chunks in K order
    return out.transpose(0, 2, 1, 3, 4).reshape(ng * 16, kt * 64)[:n, :k]


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
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    xs = torch.empty(m, dtype=torch.float32, device=x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if want_acc else None
    _call("pdq_linear_prefill", _p(x), _DT[x.dtype], m, k, _ld(x), _p(wq), _p(w_scale), _p(bias),
          n, _p(xq), _p(xs), _p(y), _ld(y), _p(acc), _stream(x.device))
    return dict(y=y, xq=xq, x_scale=xs, acc=acc)


def linear_decode(x, a_scale: float, a_zp: int, wq, w_scale, colsum, bias=None,
                  sat_count=None, want_acc: bool = False, out=None, xq=None):
    """Per-tensor static asymmetric W8A8 linear -> dict(y bf16, xq[, acc])."""
    _check_mat(x, "x")
    m, k = x.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    xq = xq if xq is not None else torch.empty((m, k), dtype=torch.int8, device=x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=x.device) if want_acc else None
    _call("pdq_linear_decode", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), int(a_zp),
          _p(wq), _p(w_scale), _p(colsum), _p(bias), n, _p(xq), _p(y), _ld(y), _p(acc),
          _p(sat_count), _stream(x.device))
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
    xq = torch.empty((m, k), dtype=torch.int8, device=dev)
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


def quantize_per_token(x, xq=None, x_scale=None):
    """Per-token dynamic symmetric INT8 -> (xq int8 [M,K], x_scale f32 [M])."""
    _check_mat(x, "x")
    m, k = x.shape
    xq = xq if xq is not None else torch.empty((m, k), dtype=torch.int8, device=x.device)
    xs = x_scale if x_scale is not None else torch.empty(m, dtype=torch.float32, device=x.device)
    _call("pdq_quantize_per_token", _p(x), _DT[x.dtype], m, k, _ld(x), _p(xq), _p(xs), _stream(x.device))
    return xq, xs


def gemm_per_token(xq, x_scale, wq, w_scale, bias=None, want_acc: bool = False, out=None):
    """INT8 GEMM + per-token/per-channel dequant epilogue -> dict(y bf16[, acc])."""
    _check_mat(xq, "xq", (torch.int8,))
    m, k = xq.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=xq.device) if want_acc else None
    _call("pdq_gemm_per_token", _p(xq), _p(x_scale), m, k, _p(wq), _p(w_scale), _p(bias), n, _p(y),
          _ld(y), _p(acc), _stream(xq.device))
    return dict(y=y, acc=acc)


def quantize_static(x, a_scale: float, a_zp: int, xq=None, sat_count=None):
    """Per-tensor static asymmetric INT8 -> xq int8 [M,K]."""
    _check_mat(x, "x")
    m, k = x.shape
    xq = xq if xq is not None else torch.empty((m, k), dtype=torch.int8, device=x.device)
    _call("pdq_quantize_static", _p(x), _DT[x.dtype], m, k, _ld(x), float(a_scale), int(a_zp), _p(xq),
          _p(sat_count), _stream(x.device))
    return xq


def gemm_static(xq, a_scale: float, a_zp: int, wq, w_scale, colsum, bias=None, want_acc: bool = False,
                out=None):
    """Skinny INT8 GEMM + zero-point correction + dequant epilogue -> dict(y bf16[, acc])."""
    _check_mat(xq, "xq", (torch.int8,))
    m, k = xq.shape
    n = w_scale.shape[0]
    _check_weight(wq, n, k)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=xq.device) if want_acc else None
    _call("pdq_gemm_static", _p(xq), m, k, float(a_scale), int(a_zp), _p(wq), _p(w_scale), _p(colsum),
          _p(bias), n, _p(y), _ld(y), _p(acc), _stream(xq.device))
    return dict(y=y, acc=acc)
