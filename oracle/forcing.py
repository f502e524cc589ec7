"""Forcing-KV static / dynamic head retention in float64.

Test infrastructure only (see the package header).

Page: "Forcing-KV: Hybrid KV Cache Compression for Efficient Autoregressive
Video Diffusion Models" (paper notes).

* Section 3.3 (static structural pruning): a static head's chunk queries
  attend over the sink frame, the transition frame -- the frame just before
  the chunk, token range [(iC-1)F, iCF) -- and the current chunk
  [iCF, (i+1)CF).
* Section 3.4 (dynamic similarity pruning): every latent frame is cut into
  contiguous segments; segment j of frame t scores the cosine similarity of
  the keys of frame t and frame t+1 on that segment; BottomK keeps the
  floor(r * n) lowest scores (least redundant).
* Section 3.5 sketch: the adjacent-frame chain ends with the first frame of
  the new chunk; a segment's score is the mean of token-wise cosines; token
  features concatenate all dynamic heads, so the kept indices are shared by
  the dynamic heads; the selection is one global BottomK over all (frame,
  segment) items; kept items are gathered in token order.

Variant (section 3.4 as printed): BottomK within each frame, keeping
floor(r * n) of its n segments (ties: lower index); with the appendix
defaults n = 6, r = 0.3 that is one segment per frame.

Section 3.2 (offline head profiling): with A the attention mass of the
profiling chunk's queries on the whole key set (total), the generated chunk,
the transition frame and the sink frame, a head is static when
(A_generate + A_transition) / (A_total - A_sink) > alpha (0.8 in the
appendix), else dynamic.  Reading: A_region = sum over the chunk's queries of
the softmax weights on that region's keys (so A_total = number of queries);
the comparison is the formula's strict '>' (the printed sketch uses '>=').

Readings: cos(a, b) = a.b / max(|a| |b|, 1e-8); r is the kept fraction and
the kept count is floor(r * items) computed in double precision; ties in the
BottomK go to the lower item index.

Parity pins (tests/test_oracle_forcing.py): r = 1 keeps everything (full
attention), r = 0 keeps nothing, identical adjacent frames score exactly 1,
the cosine agrees with torch's cosine_similarity in float64, and the static
token ranges reproduce the section 3.3 formula.
"""
from __future__ import annotations

import math

import numpy as np

COS_EPS = 1e-8


def segment_scores(hist: np.ndarray, nxt: np.ndarray, F: int, seg_len: int) -> np.ndarray:
    """Scores s[t * nseg + j] for history frames t and segments j.

    hist: [H_dyn][T*F][d] history keys of the dynamic heads (time order);
    nxt:  [H_dyn][F][d] keys of the first frame of the new chunk.
    Token features concatenate the dynamic heads.
    """
    hist = np.asarray(hist, np.float64)
    nxt = np.asarray(nxt, np.float64)
    Hd, TF, d = hist.shape
    T = TF // F
    nseg = F // seg_len
    chain = np.concatenate([hist, nxt], axis=1)               # [Hd][(T+1)F][d]
    feats = chain.transpose(1, 0, 2).reshape((T + 1), F, Hd * d)
    a, b = feats[:-1], feats[1:]                               # [T][F][Hd*d]
    dot = np.einsum("tfx,tfx->tf", a, b)
    na = np.sqrt(np.einsum("tfx,tfx->tf", a, a))
    nb = np.sqrt(np.einsum("tfx,tfx->tf", b, b))
    cos = dot / np.maximum(na * nb, COS_EPS)
    return cos.reshape(T, nseg, seg_len).mean(axis=2).reshape(-1)


def keep_count(r: float, items: int) -> int:
    return int(math.floor(float(r) * items))


def bottomk(scores: np.ndarray, r: float) -> np.ndarray:
    """Indices of the floor(r * n) lowest scores (ties: lower index), ascending."""
    k = keep_count(r, scores.shape[0])
    order = np.lexsort((np.arange(scores.shape[0]), np.asarray(scores, np.float64)))
    return np.sort(order[:k])


def bottomk_per_frame(scores: np.ndarray, r: float, nseg: int) -> np.ndarray:
    """Per frame, the floor(r * nseg) lowest scores of its nseg segments
    (ties: lower index); kept item indices ascending."""
    scores = np.asarray(scores, np.float64)
    k = keep_count(r, nseg)
    kept = []
    for t in range(scores.shape[0] // nseg):
        s = scores[t * nseg:(t + 1) * nseg]
        kept.extend(t * nseg + i for i in sorted(range(nseg), key=lambda i: (s[i], i))[:k])
    return np.array(sorted(kept), dtype=np.int64)


def kept_token_rows(kept: np.ndarray, F: int, seg_len: int) -> np.ndarray:
    """History row indices covered by the kept (frame, segment) items, in token order."""
    nseg = F // seg_len
    rows = [np.arange(seg_len) + (i // nseg) * F + (i % nseg) * seg_len for i in np.asarray(kept)]
    return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


REGION_OTHER, REGION_SINK, REGION_TRANSITION, REGION_GENERATE = 0, 1, 2, 3


def attention_mass(Q: np.ndarray, K: np.ndarray, region: np.ndarray, scale: float = None) -> np.ndarray:
    """[4] masses (other, sink, transition, generate): sums over queries of the
    softmax(Q K^T scale) weights on each region's keys."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    region = np.asarray(region)
    if scale is None:
        scale = 1.0 / math.sqrt(Q.shape[1])
    s = (Q @ K.T) * scale
    s -= s.max(axis=1, keepdims=True)
    P = np.exp(s)
    P /= P.sum(axis=1, keepdims=True)
    return np.array([P[:, region == r].sum() for r in range(4)])


def head_score(mass: np.ndarray) -> float:
    """(A_generate + A_transition) / (A_total - A_sink)."""
    total = float(np.sum(mass))
    return (mass[REGION_GENERATE] + mass[REGION_TRANSITION]) / (total - mass[REGION_SINK])


def head_is_static(mass: np.ndarray, alpha: float = 0.8) -> bool:
    return head_score(mass) > alpha


def static_rows(T: int, F: int) -> np.ndarray:
    """History rows a static head keeps: the transition frame [(T-1)F, TF)."""
    return np.arange((T - 1) * F, T * F) if T > 0 else np.zeros(0, dtype=np.int64)
