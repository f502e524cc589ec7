"""Seeded synthetic inputs for the head-wise compressed KV cache path.

This module is shared by the fp64 oracle and by the HIP path.  It holds no
part of the method's arithmetic (no density, admission, eviction, similarity
or attention); it only draws keys, values and queries with the shapes and the
temporal structure of the pages' workloads:

* Wan2.1-T2V-1.3B-like layer shapes: 12 heads, head_dim 128, 1,560 tokens per
  latent frame at 480P, three latent frames per generated chunk (DensityKV
  page, appendix D).
* Post-RoPE keys, with the temporal rotary coordinate zeroed for non-local
  memory keys (sink and bank) and kept for local keys (DensityKV page,
  supplementary material, "Post-RoPE Attention Geometry").

Key model (per layer, head, spatial position p and latent frame t):

    k_pre[t, p] = base[p] + drift[t, p] + noise[t, p]
    base  ~ N(0, I_d)
    drift : AR(1), drift[0] = 0, drift[t] = 0.95 drift[t-1] + sqrt(1-0.95^2) z
    noise ~ N(0, 0.1^2 I_d)
    q, v  ~ N(0, I_d)

then 3D rotary embedding over (t, row, col) and one rounding to the storage
dtype (bf16 round-to-nearest-even, or fp32).  Every draw comes from a NumPy
Philox stream keyed by (seed, layer, head, stream, frame) through
``SeedSequence``, so any frame of any head can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "LayerGen", "LayerStream", "round_bf16", "bf16_bits",
    "rope_split", "head_labels", "frame_tokens",
]

AR_RHO = 0.95
NOISE_STD = 0.1
ROPE_BASE = 10000.0

# stream ids for the Philox key
_S_BASE, _S_INNOV, _S_NOISE, _S_VAL, _S_QRY, _S_LABEL = range(6)

HEAD_DENSITY, HEAD_STATIC, HEAD_DYNAMIC = 0, 1, 2


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even); returns float32 values."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    b &= np.uint32(0xFFFF0000)
    return b.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bf16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable")
    return (b >> np.uint32(16)).astype(np.uint16)


def rope_split(d: int) -> Tuple[int, int, int]:
    """Rotary pair counts for (t, row, col): d/2 - 2*floor(d/6), floor(d/6), floor(d/6)."""
    n = d // 6
    return d // 2 - 2 * n, n, n


def _rope_angles(d: int, t: np.ndarray, row: np.ndarray, col: np.ndarray) -> np.ndarray:
    """Angles [len, d/2] for positions given per token."""
    nt, nh, nw = rope_split(d)
    parts = []
    for pos, n in ((t, nt), (row, nh), (col, nw)):
        freq = ROPE_BASE ** (-np.arange(n, dtype=np.float64) / n)
        parts.append(np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :])
    return np.concatenate(parts, axis=1)


def _apply_rope(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs (x[2i], x[2i+1]) by ang[:, i]."""
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes and frame roles of one synthetic workload (one attention layer)."""
    name: str
    H: int
    d: int
    width: int                  # patches per row
    height: int                 # patch rows
    dtype: str                  # "bf16" or "f32"
    M: int                      # bank capacity per head
    tau: float = 2.0
    sigma: float = 8.0
    eps: float = 1.0
    p: float = 2.0
    chunk_frames: int = 3
    window_frames: int = 6
    # frame roles (latent frame indices); frame 0 is the sink
    bank_updates: Tuple[Tuple[int, int], ...] = ()   # [t0, t1) frame ranges offered as candidates, in order
    window: Tuple[int, int] = (0, 0)                 # [t0, t1) local-window history frames
    chunk: Tuple[int, int] = (0, 0)                  # [t0, t1) current chunk
    # Forcing-KV
    n_static: int = 0                                # heads labelled static (rest dynamic) when > 0
    history: Tuple[int, int] = (0, 0)                # [t0, t1) Forcing-KV history frames
    seg_len: int = 0                                 # tokens per segment
    retention: float = 0.0                           # kept fraction r
    layers: int = 1
    chunks: int = 0                                  # streaming rollout length

    @property
    def F(self) -> int:
        return self.width * self.height

    @property
    def Lq(self) -> int:
        return self.chunk_frames * self.F


def frame_tokens(wl: Workload, t0: int, t1: int) -> np.ndarray:
    """Token ids frame*F + p for frames [t0, t1) (int32)."""
    F = wl.F
    return (np.arange(t0, t1, dtype=np.int64)[:, None] * F + np.arange(F)[None, :]).reshape(-1).astype(np.int32)


def head_labels(wl: Workload, seed: int, layer: int = 0) -> np.ndarray:
    """uint8 label per head: 0 density bank, 1 static, 2 dynamic (Forcing-KV)."""
    lab = np.zeros(wl.H, dtype=np.uint8)
    if wl.n_static > 0:
        rng = np.random.Generator(np.random.Philox(np.random.SeedSequence(seed, spawn_key=(layer, _S_LABEL))))
        perm = rng.permutation(wl.H)
        lab[:] = HEAD_DYNAMIC
        lab[perm[: wl.n_static]] = HEAD_STATIC
    return lab


WORKLOADS: Dict[str, Workload] = {
    # 1 layer, 2 heads, head_dim 64, fp32, 4x4 frames; frames 1-9 enter the bank in
    # three updates of 48 candidates; chunk = frames 10-12; no local window.
    "tiny": Workload(name="tiny", H=2, d=64, width=4, height=4, dtype="f32", M=64, tau=2.0,
                     window_frames=0, bank_updates=((1, 4), (4, 7), (7, 10)), window=(10, 10),
                     chunk=(10, 13)),
    # 480P Wan-1.3B-like layer: bank cold-built from frames 1-6 (n = M = 9,360), one
    # update offering frames 7-21 (N = 23,400), window 22-27, chunk 28-30.
    "480p": Workload(name="480p", H=12, d=128, width=52, height=30, dtype="bf16", M=9360, tau=2.0,
                     bank_updates=((1, 7), (7, 22)), window=(22, 28), chunk=(28, 31)),
    # 480P, one finalized block: the same layer with the pages' per-block pool,
    # frames 7-9 (N = 4,680) offered to the full bank of frames 1-6; window
    # 10-15, chunk 16-18.  Part of the bank survives (partial eviction).
    "480p_block": Workload(name="480p_block", H=12, d=128, width=52, height=30, dtype="bf16", M=9360, tau=2.0,
                           bank_updates=((1, 7), (7, 10)), window=(10, 16), chunk=(16, 19)),
    # Forcing-KV hybrid heads at 480P: 6 static / 6 dynamic (seeded), history frames
    # 1-12, chunk 13-15, 1,560-token segments, 70% of segments kept.
    "fkv480p": Workload(name="fkv480p", H=12, d=128, width=52, height=30, dtype="bf16", M=0,
                        window_frames=0, chunk=(13, 16), n_static=6, history=(1, 13),
                        seg_len=1560, retention=0.7),
    # 1080P layer: bank cold-built from frames 1-6 (n = M = 48,960), one update
    # offering frames 7-27 (N = 171,360), window 28-33, chunk 34-36.
    "1080p": Workload(name="1080p", H=12, d=128, width=120, height=68, dtype="bf16", M=48960, tau=2.0,
                      bank_updates=((1, 7), (7, 28)), window=(28, 34), chunk=(34, 37)),
    # streaming rollout: 30 layers, 80 chunks of 3 frames at 480P, M = 9,360, W = 6.
    "rollout": Workload(name="rollout", H=12, d=128, width=52, height=30, dtype="bf16", M=9360, tau=2.0,
                        layers=30, chunks=80),
}


def _rng(seed: int, layer: int, head: int, stream: int, frame: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(layer, head, stream, frame))
    return np.random.Generator(np.random.Philox(ss))


class LayerGen:
    """Random-access generator of one layer's keys, values and queries.

    ``keys(h, frames, rope_t)`` returns post-RoPE keys of the given frames for
    head ``h`` with the temporal rotary coordinate of each frame taken from
    ``rope_t`` (0 for memory keys).  Results are float32 holding values already
    rounded to the workload dtype.
    """

    def __init__(self, wl: Workload, seed: int = 0, layer: int = 0):
        self.wl, self.seed, self.layer = wl, seed, layer
        self._base: Dict[int, np.ndarray] = {}
        self._drift: Dict[int, np.ndarray] = {}   # head -> [T, F, d] float64 (grown lazily)
        F = wl.F
        p = np.arange(F)
        self._row, self._col = p // wl.width, p % wl.width

    # -- raw draws --------------------------------------------------------
    def _base_of(self, h: int) -> np.ndarray:
        if h not in self._base:
            self._base[h] = _rng(self.seed, self.layer, h, _S_BASE).standard_normal((self.wl.F, self.wl.d))
        return self._base[h]

    def _drift_upto(self, h: int, t_end: int) -> np.ndarray:
        wl = self.wl
        cur = self._drift.get(h)
        have = 0 if cur is None else cur.shape[0]
        if have >= t_end:
            return cur
        new = np.empty((t_end, wl.F, wl.d), dtype=np.float64)
        if have:
            new[:have] = cur
        innov = math.sqrt(1.0 - AR_RHO * AR_RHO)
        for t in range(have, t_end):
            if t == 0:
                new[0] = 0.0
            else:
                z = _rng(self.seed, self.layer, h, _S_INNOV, t).standard_normal((wl.F, wl.d))
                new[t] = AR_RHO * new[t - 1] + innov * z
        self._drift[h] = new
        return new

    def _round(self, x: np.ndarray) -> np.ndarray:
        x32 = x.astype(np.float32)
        return round_bf16(x32) if self.wl.dtype == "bf16" else x32

    def _rotate(self, x: np.ndarray, rope_t: Sequence[int]) -> np.ndarray:
        # x: [nf, F, d] float64
        nf, F = x.shape[0], x.shape[1]
        t = np.repeat(np.asarray(rope_t, dtype=np.float64), F)
        ang = _rope_angles(self.wl.d, t, np.tile(self._row, nf), np.tile(self._col, nf))
        return _apply_rope(x.reshape(nf * F, -1), ang).reshape(x.shape)

    # -- public ------------------------------------------------------------
    def prerope_keys(self, h: int, frames: Sequence[int]) -> np.ndarray:
        frames = list(frames)
        drift = self._drift_upto(h, max(frames) + 1 if frames else 0)
        base = self._base_of(h)
        out = np.empty((len(frames), self.wl.F, self.wl.d), dtype=np.float64)
        for i, t in enumerate(frames):
            noise = _rng(self.seed, self.layer, h, _S_NOISE, t).standard_normal((self.wl.F, self.wl.d))
            out[i] = base + drift[t] + NOISE_STD * noise
        return out

    def keys(self, h: int, frames: Sequence[int], rope_t: Optional[Sequence[int]] = None) -> np.ndarray:
        frames = list(frames)
        if not frames:
            return np.zeros((0, self.wl.d), dtype=np.float32)
        if rope_t is None:
            rope_t = [0] * len(frames)
        k = self._rotate(self.prerope_keys(h, frames), rope_t)
        return self._round(k).reshape(len(frames) * self.wl.F, self.wl.d)

    def values(self, h: int, frames: Sequence[int]) -> np.ndarray:
        out = [
            _rng(self.seed, self.layer, h, _S_VAL, t).standard_normal((self.wl.F, self.wl.d)) for t in frames
        ]
        return self._round(np.concatenate(out, axis=0) if out else np.zeros((0, self.wl.d)))

    def queries(self, h: int, frames: Sequence[int], rope_t: Sequence[int]) -> np.ndarray:
        frames = list(frames)
        if not frames:
            return np.zeros((0, self.wl.d), dtype=np.float32)
        q = np.stack([_rng(self.seed, self.layer, h, _S_QRY, t).standard_normal((self.wl.F, self.wl.d))
                      for t in frames]) if frames else np.zeros((0, self.wl.F, self.wl.d))
        q = self._rotate(q, rope_t)
        return self._round(q).reshape(len(frames) * self.wl.F, self.wl.d)

    # -- stacked helpers ([H][tokens][d]) ----------------------------------
    def keys_all(self, frames: Sequence[int], rope_t: Optional[Sequence[int]] = None,
                 heads: Optional[Sequence[int]] = None) -> np.ndarray:
        heads = range(self.wl.H) if heads is None else heads
        return np.stack([self.keys(h, frames, rope_t) for h in heads])

    def values_all(self, frames: Sequence[int], heads: Optional[Sequence[int]] = None) -> np.ndarray:
        heads = range(self.wl.H) if heads is None else heads
        return np.stack([self.values(h, frames) for h in heads])

    def queries_all(self, frames: Sequence[int], rope_t: Sequence[int],
                    heads: Optional[Sequence[int]] = None) -> np.ndarray:
        heads = range(self.wl.H) if heads is None else heads
        return np.stack([self.queries(h, frames, rope_t) for h in heads])


class LayerStream:
    """One layer's frames in time order with bounded memory.

    Holds only the current AR(1) drift state per head, so a rollout of any
    length costs the same memory.  ``frame(t)`` must be called with
    t = 0, 1, 2, ... in order and returns post-RoPE keys at temporal
    coordinate ``rope_t`` (default t), values and queries at the same
    coordinate, each [H][F][d] float32 rounded to the workload dtype.  The
    draws and the arithmetic are those of ``LayerGen``, so frame t equals
    ``LayerGen(wl, seed, layer).keys_all([t], [rope_t])`` bit for bit.
    """

    def __init__(self, wl: Workload, seed: int = 0, layer: int = 0):
        self.wl, self.seed, self.layer = wl, seed, layer
        self._g = LayerGen(wl, seed, layer)
        self._drift = None   # [H][F][d] float64, drift of frame self.t - 1
        self.t = 0

    def frame(self, t: int, rope_t: Optional[int] = None):
        if t != self.t:
            raise ValueError(f"frames come in order: expected {self.t}, got {t}")
        wl, g = self.wl, self._g
        rt = t if rope_t is None else rope_t
        innov = math.sqrt(1.0 - AR_RHO * AR_RHO)
        if t == 0:
            drift = np.zeros((wl.H, wl.F, wl.d))
        else:
            z = np.stack([_rng(self.seed, self.layer, h, _S_INNOV, t).standard_normal((wl.F, wl.d))
                          for h in range(wl.H)])
            drift = AR_RHO * self._drift + innov * z
        self._drift = drift
        self.t += 1
        keys = np.empty((wl.H, wl.F, wl.d), np.float32)
        for h in range(wl.H):
            noise = _rng(self.seed, self.layer, h, _S_NOISE, t).standard_normal((wl.F, wl.d))
            pre = g._base_of(h) + drift[h] + NOISE_STD * noise
            keys[h] = g._round(g._rotate(pre[None], [rt]))[0]
        values = g.values_all([t])
        queries = g.queries_all([t], [rt])
        return keys, values, queries
