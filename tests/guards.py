"""Sentinel margins around the outputs of the library's calls (GPU tests).

Inside `guarded()` every buffer the Python binding allocates for a call's
outputs (y, the INT32 accumulators, the packed codes, scales, zero points,
outlier indices and count, the LLM.int8 workspace) is carved out of a larger
allocation whose margins before and after hold a sentinel byte pattern; on
leaving the block the margins are read back and must be untouched.  A store
past the end of an output -- an epilogue writing columns past N or rows past
M, a quantizer writing past the packed code image -- then fails the test
instead of landing silently in memory nobody reads.

`gapped(m, n, dtype)` gives a [m, n] output whose rows sit `gap` elements
apart inside a [m, n + gap] sentinel-filled buffer, so that stores past
column N of any row are caught as well (with a row pitch of exactly N such a
store lands in the next row, where the correct value may overwrite it).
"""
from __future__ import annotations

import contextlib

import torch

from w8a8_int8_quantized_absmax_amd import pdq

SENTINEL = 0xA5
MARGIN_BYTES = 4096


class _TorchProxy:
    """torch, except that empty() returns a view into a sentinel-margined buffer."""

    def __init__(self, real, record):
        self._real = real
        self._record = record

    def __getattr__(self, name):
        return getattr(self._real, name)

    def empty(self, *size, dtype=None, device=None, **kw):
        real = self._real
        if len(size) == 1 and isinstance(size[0], (tuple, list, torch.Size)):
            size = tuple(size[0])
        dtype = dtype or real.get_default_dtype()
        if device is None or real.device(device).type != "cuda":
            return real.empty(*size, dtype=dtype, device=device, **kw)
        numel = 1
        for s in size:
            numel *= int(s)
        es = real.empty((), dtype=dtype).element_size()
        marg = MARGIN_BYTES // es
        buf = real.empty(numel + 2 * marg, dtype=dtype, device=device)
        buf.view(real.uint8).fill_(SENTINEL)
        self._record.append((buf, marg * es, numel * es))
        return buf[marg:marg + numel].view(size)


def _check(record):
    torch.cuda.synchronize()
    for buf, front, body in record:
        b = buf.view(torch.uint8)
        head = b[:front]
        tail = b[front + body:]
        assert bool((head == SENTINEL).all()), f"store before an output of {body} bytes"
        assert bool((tail == SENTINEL).all()), f"store past the end of an output of {body} bytes"


@contextlib.contextmanager
def guarded():
    record = []
    real = pdq.torch
    pdq.torch = _TorchProxy(real, record)
    try:
        yield record
    finally:
        pdq.torch = real
    _check(record)


def gapped(m: int, n: int, dtype=torch.bfloat16, gap: int = 24):
    """(y, check): y a [m, n] view with row pitch n + gap into a sentinel-filled
    buffer; check() asserts that the gap columns and the margins are untouched."""
    es = torch.empty((), dtype=dtype).element_size()
    marg = MARGIN_BYTES // es
    pitch = n + gap
    buf = torch.empty(m * pitch + 2 * marg, dtype=dtype, device="cuda")
    buf.view(torch.uint8).fill_(SENTINEL)
    full = buf[marg:marg + m * pitch].view(m, pitch)
    y = full[:, :n]

    def check():
        torch.cuda.synchronize()
        b = buf.view(torch.uint8)
        assert bool((b[:marg * es] == SENTINEL).all()), "store before y"
        assert bool((b[(marg + m * pitch) * es:] == SENTINEL).all()), "store past the end of y"
        g = full[:, n:].contiguous().view(torch.uint8)
        assert bool((g == SENTINEL).all()), "store into the gap past column N"

    return y, check
