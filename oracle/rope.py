"""Memory-key re-rotation in float64 (oracle; test infrastructure only).

Page: "DensityKV: Density-Guided KV Cache Compression for Long Video
Generation" (paper summary), supplementary "Post-RoPE Attention Geometry":
the backbones zero the temporal rotary coordinate of non-local memory keys
and keep their spatial coordinates; DensityKV stores those post-RoPE keys.
Method, "Online Density-Constrained Bank Update": candidates are the tokens
of frames that leave the local window.

A key that sat in the window with temporal coordinate t therefore enters the
bank as the same key with its temporal rotary pairs turned back by t: each
temporal pair (x_2i, x_2i+1) is multiplied by the 2x2 rotation through
-t * w_i, w_i = base^(-i / n_t); spatial pairs are unchanged.

Readings (not fixed by the pages; also used by the input generator):
interleaved pairs, n_t = d/2 - 2 floor(d/6) temporal pairs first, then
floor(d/6) row and floor(d/6) column pairs, base 10000.

Parity pins (tests/test_oracle_rope.py): turning generator keys written at
coordinate t back by t gives the generator's own keys at coordinate 0 (an
independent rotation); t = 0 is the identity; norms, spatial pairs and
inner products of same-coordinate keys are preserved; turning by t then by
-t is the identity.
"""
from __future__ import annotations

import math

import numpy as np


def temporal_pairs(d: int) -> int:
    """Number of temporal rotary pairs at head dimension d."""
    return d // 2 - 2 * (d // 6)


def rerotate_temporal(K: np.ndarray, t: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """K [n, d] post-RoPE keys whose temporal coordinate is t[n]; returns the
    same keys at temporal coordinate 0 (float64)."""
    K = np.asarray(K, np.float64)
    n, d = K.shape
    nt = temporal_pairs(d)
    out = K.copy()
    t = np.asarray(t, np.float64).reshape(n)
    for i in range(nt):
        w = base ** (-i / nt)
        a = -t * w                     # turn back by t * w_i
        c, s = np.cos(a), np.sin(a)
        x, y = K[:, 2 * i], K[:, 2 * i + 1]
        out[:, 2 * i] = c * x - s * y
        out[:, 2 * i + 1] = s * x + c * y
    return out


def window_advance(ring_k: np.ndarray, ring_v: np.ndarray, start: int, n_rows: int, frame_tokens: int,
                   t_first: int, new_k=None, new_v=None, base: float = 10000.0):
    """The n_rows ring rows from position start (mod cap) leave the window.

    ring_k, ring_v: [H][cap][d].  Row r of the departing block belongs to
    frame r // frame_tokens, whose temporal coordinate is t_first + that
    index.  Returns (cand_k [H][n_rows][d] at coordinate 0, cand_v, new
    ring_k, new ring_v) where the departed slots hold new_k / new_v rows
    when given.
    """
    ring_k = np.asarray(ring_k, np.float64)
    ring_v = np.asarray(ring_v, np.float64)
    H, cap, d = ring_k.shape
    slots = (start + np.arange(n_rows)) % cap
    t = t_first + np.arange(n_rows) // frame_tokens
    cand_k = np.stack([rerotate_temporal(ring_k[h, slots], t, base) for h in range(H)])
    cand_v = ring_v[:, slots].copy()
    rk, rv = ring_k.copy(), ring_v.copy()
    if new_k is not None:
        rk[:, slots] = np.asarray(new_k, np.float64)
        rv[:, slots] = np.asarray(new_v, np.float64)
    return cand_k, cand_v, rk, rv
