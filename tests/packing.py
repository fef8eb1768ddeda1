"""The packed INT8 layout of include/pdq.h, written out in numpy for the tests.

Test infrastructure only: the byte image that pdq_quantize_weight (weights)
and every quantizer of activations (xq) must produce for given codes, from
the header's definition (1024-byte blocks of 16 rows x 64 K values; block
(g, s) at (g * ceil(K / 64) + s) * 1024; row r at r * 64 in it; its 16-byte
chunk c at position c ^ ((r >> 2) & 3); padding 0).
"""
from __future__ import annotations

import numpy as np


def pack_weight(codes: np.ndarray) -> np.ndarray:
    n, k = codes.shape
    ng, kt = -(-n // 16), -(-k // 64)
    full = np.zeros((ng * 16, kt * 64), np.int8)
    full[:n, :k] = codes
    blocks = full.reshape(ng, 16, kt, 4, 16).transpose(0, 2, 1, 3, 4)  # [g, s, r, c, byte]
    r = np.arange(16)[:, None]
    pos = np.arange(4)[None, :] ^ ((r >> 2) & 3)
    out = np.empty_like(blocks)
    out[:, :, r, pos, :] = blocks  # chunk c of channel r lands at position pos[r, c]
    return out.reshape(-1)


pack = pack_weight  # activation codes use the same layout
