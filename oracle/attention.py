"""Native scaled-dot-product attention over the retained KV, in float64.

Test infrastructure only (see the package header).

Pages: DensityKV card page, Figure 2 (current queries read the retained
history -- sink, per-head bank, local window -- through the backbone's native
attention); Forcing-KV paper-notes page, section 3.3 (the chunk's queries
attend over [sink, transition frame, current chunk] with no mask inside the
chunk).  Reading: scale 1/sqrt(d), softmax over every retained key, no mask;
the order of the KV rows does not matter.

Parity pins (tests/test_oracle_attention.py): a textbook per-row loop on tiny
shapes, and torch's scaled_dot_product_attention in float64 on the CPU.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .density import _map_blocks


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: Optional[float] = None,
              block: int = 1024) -> np.ndarray:
    """O = softmax(Q K^T * scale) V with the row maximum subtracted first."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(Q.shape[-1])
    out = np.empty((Q.shape[0], V.shape[1]), dtype=np.float64)
    if K.shape[0] == 0:
        out[:] = 0.0
        return out

    def rows(i):
        s = (Q[i:i + block] @ K.T) * scale
        s -= s.max(axis=1, keepdims=True)
        np.exp(s, out=s)
        out[i:i + block] = (s @ V) / s.sum(axis=1, keepdims=True)
    # query blocks are independent (threads with the density module's worker count)
    _map_blocks(rows, range(0, Q.shape[0], block))
    return out
