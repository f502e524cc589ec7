"""Streaming chunk-by-chunk rollout over several layers (orchestration only).

Timeline (DensityKV card page, Figure 2; paper summary, appendix D: a sink
frame, a local window and a bounded bank per head, one finalized block of
three latent frames per step).  Chunk c generates frames [3c, 3c + 3).  Frame
0 becomes the sink.  The local window holds the last W history frames
[max(1, 3c - W), 3c) in a device ring of W frames per layer: frame f >= 1
lives in ring slot (f - 1) mod W.  Before chunk c attends, the previous
chunk's frames join the ring; the frames pushed out of it leave through
``kvbank_window_advance``, which turns their keys back to temporal coordinate
0 (the memory-key convention: paper summary, supplementary "Post-RoPE
Attention Geometry") and writes the arriving frames into the freed slots in
the same pass.  The departed frames are the bank candidates of this chunk:
``kvbank_score`` and ``kvbank_update``, then ``chunk_attention`` of the
chunk's queries over sink + bank + window + chunk.

Coordinates: a frame's keys and queries are produced at temporal rotary
coordinate equal to the frame index and are never rotated again while they
are local (attention depends only on differences of local coordinates); the
sink (frame 0) sits at 0 already.

Frames come from a seeded stream per layer: ``kvsynth.LayerStream`` on the
host (the tests, whose oracle needs the same frames) or
``kvsynth.device.DeviceStream`` on the GPU (the benchmark).  Every step of
the method runs in libkvbank through ``LayerCache``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Union

import numpy as np
import torch

from kvsynth import ROPE_BASE, LayerStream, Workload

from . import KVB_BF16, KVB_F32, KVLayout, LayerDesc, kvbank_window_advance
from .pipeline import LayerCache


@dataclasses.dataclass
class ChunkPlan:
    chunk: int
    frames: range          # current chunk
    window: range          # local window frames attended by this chunk
    arriving: range        # frames joining the ring now (the previous chunk, minus the sink)
    departed: range        # frames leaving the ring now (bank candidates)


def plan(c: int, chunk_frames: int = 3, window_frames: int = 6) -> ChunkPlan:
    f0 = chunk_frames * c
    w0 = max(1, f0 - window_frames)
    prev_w0 = max(1, f0 - chunk_frames - window_frames) if c > 0 else 1
    arr = range(max(1, f0 - chunk_frames), f0) if c > 0 else range(0)
    dep = range(prev_w0, w0) if w0 > prev_w0 else range(0)
    return ChunkPlan(c, range(f0, f0 + chunk_frames), range(w0, f0) if f0 > w0 else range(0), arr, dep)


class _Layer:
    """Device state of one layer: bank (in the LayerCache), window ring, sink,
    the previous chunk's K/V, and the frame stream."""

    def __init__(self, wl: Workload, layer: int, seed: int, cache: LayerCache, source: str, kdt):
        H, F, d, W = wl.H, wl.F, wl.d, wl.window_frames
        self.layer, self.cache = layer, cache
        self.ring_k = torch.zeros(H, W * F, d, dtype=kdt, device="cuda")
        self.ring_v = torch.zeros_like(self.ring_k)
        self.sink_k = self.sink_v = None
        self.prev_k = self.prev_v = None       # [H][3F][d] chunk K/V of the previous step
        self.cand_k = torch.empty(H * wl.chunk_frames * F * d, dtype=kdt, device="cuda")
        self.cand_v = torch.empty_like(self.cand_k)
        if source == "host":
            self.stream = LayerStream(wl, seed, layer)
        else:
            from kvsynth.device import DeviceStream
            self.stream = DeviceStream(wl, seed, layer, dtype=kdt)
        self.recent: Dict[int, tuple] = {}      # host streams: frame -> (k, v, q) numpy, last W + C frames


class Rollout:
    """Per-layer caches, window rings and input streams of a streaming rollout.

    layers: a count (layers 0 .. n-1) or the list of layer indices to run
    (each layer's stream is keyed by its index, so running a subset gives
    the same per-layer results as running them all).  source: "host"
    (seeded NumPy frames; the oracle can regenerate them) or "device"
    (seeded frames drawn on the GPU).  policy: KVB_POL_* bits of every
    layer's bank (0: the method as the pages state it)."""

    def __init__(self, wl: Workload, layers: Union[int, Sequence[int]], seed: int = 0, diagnostics: bool = False,
                 source: str = "host", policy: int = 0):
        self.wl, self.seed, self.source = wl, seed, source
        self.layer_ids = list(range(layers)) if isinstance(layers, int) else list(layers)
        self.kdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        dt = KVB_BF16 if wl.dtype == "bf16" else KVB_F32
        self.desc = LayerDesc(H=wl.H, d=wl.d, M=wl.M, dtype=dt, frame_tokens=wl.F, labels=[0] * wl.H,
                              tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p, policy=policy)
        self.L: List[_Layer] = []
        for l in self.layer_ids:
            lc = LayerCache(self.desc, seg_cap=8, max_N=wl.chunk_frames * wl.F, diagnostics=diagnostics)
            self.L.append(_Layer(wl, l, seed, lc, source, self.kdt))
        self.c = 0
        self._prepared = None
        # host streams: the next chunk's frames are drawn in worker threads
        # (one per layer) while the current chunk runs
        self._pool = None
        self._next = None
        if source == "host":
            import concurrent.futures as cf
            self._pool = cf.ThreadPoolExecutor(max_workers=max(1, len(self.L)))

    def _draw(self, x: "_Layer", frames: range):
        return [x.stream.frame(f) for f in frames]

    def _draw_all(self, c: int):
        p = plan(c, self.wl.chunk_frames, self.wl.window_frames)
        if self._next is not None and self._next[0] == c:
            futs = self._next[1]
        else:
            futs = [self._pool.submit(self._draw, x, p.frames) for x in self.L]
        self._next = None
        out = [f.result() for f in futs]
        pn = plan(c + 1, self.wl.chunk_frames, self.wl.window_frames)
        self._next = (c + 1, [self._pool.submit(self._draw, x, pn.frames) for x in self.L])
        return out

    @property
    def caches(self) -> List[LayerCache]:
        return [x.cache for x in self.L]

    def _slot(self, f: int) -> int:
        return ((f - 1) % self.wl.window_frames) * self.wl.F

    def _dev(self, x):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(self.kdt).contiguous()

    # -- inputs of one chunk (not part of the timed work) --------------------
    def prepare(self):
        """Draw the current chunk's frames for every layer: keys, values and
        queries at temporal coordinate = frame index, [H][3F][d] on the device."""
        p = plan(self.c, self.wl.chunk_frames, self.wl.window_frames)
        keep = self.wl.window_frames + self.wl.chunk_frames
        drawn = self._draw_all(self.c) if self.source == "host" else None
        out = []
        for li, x in enumerate(self.L):
            ks, vs, qs = [], [], []
            for fi, f in enumerate(p.frames):
                k, v, q = drawn[li][fi] if drawn is not None else x.stream.frame(f)
                if self.source == "host":
                    x.recent[f] = (k, v, q)
                    for old in [g for g in x.recent if 0 < g < f - keep + 1]:   # frame 0 is the sink
                        del x.recent[old]
                    k, v, q = self._dev(k), self._dev(v), self._dev(q)
                ks.append(k)
                vs.append(v)
                qs.append(q)
            out.append((torch.cat(ks, dim=1).contiguous(), torch.cat(vs, dim=1).contiguous(),
                        torch.cat(qs, dim=1).contiguous()))
        self._prepared = (p, out)
        return p

    # -- the library calls of one chunk ---------------------------------------
    def run(self, hook=None):
        """Window advance, bank update and chunk attention of every layer for
        the prepared chunk; returns the attention outputs (fp32)."""
        if self._prepared is None:
            self.prepare()
        p, inputs = self._prepared
        wl, F, W = self.wl, self.wl.F, self.wl.window_frames
        cap = W * F
        outs = []
        for x, (chk, chv, q) in zip(self.L, inputs):
            lc = x.cache
            if p.chunk == 1:
                # frame 0 becomes the sink (its keys are at coordinate 0 already)
                x.sink_k = x.prev_k[:, :F].contiguous()
                x.sink_v = x.prev_v[:, :F].contiguous()
            arr, dep = list(p.arriving), list(p.departed)
            j0 = (arr[0] - (p.chunk - 1) * wl.chunk_frames) if arr else 0   # first arriving frame in prev_*
            n_free = len(arr) - len(dep)
            # arrivals that find free ring slots (the ring is not yet full)
            for i in range(n_free):
                f = arr[i]
                s = self._slot(f)
                x.ring_k[:, s:s + F].copy_(x.prev_k[:, (j0 + i) * F:(j0 + i + 1) * F])
                x.ring_v[:, s:s + F].copy_(x.prev_v[:, (j0 + i) * F:(j0 + i + 1) * F])
            N = len(dep) * F
            ck = cv = ct = None
            if N:
                ck = x.cand_k[: wl.H * N * wl.d].view(wl.H, N, wl.d)
                cv = x.cand_v[: wl.H * N * wl.d].view(wl.H, N, wl.d)
                a0 = (j0 + n_free) * F
                new_k = x.prev_k[:, a0:a0 + N].contiguous()
                new_v = x.prev_v[:, a0:a0 + N].contiguous()
                ring_before = None
                if hook is not None:
                    ring_before = (x.ring_k.clone(), x.ring_v.clone())
                kvbank_window_advance(self.desc, x.ring_k, x.ring_v, self._slot(dep[0]), N, dep[0], ck, cv,
                                      new_k, new_v, rope_base=ROPE_BASE)
                # token ids frame * F + p of the departed frames: one contiguous
                # range, made on the device (a host-to-device copy here would
                # wait for the stream and stall the launches of every layer)
                ct = torch.arange(dep[0] * F, (dep[-1] + 1) * F, dtype=torch.int32, device="cuda")
            lay = KVLayout()
            if x.sink_k is not None:
                lay.sink_k, lay.sink_v = x.sink_k, x.sink_v
            if len(p.window):
                lay.win_k, lay.win_v = x.ring_k, x.ring_v
                lay.win_start, lay.win_len = self._slot(p.window[0]), len(p.window) * F
            lay.chunk_k, lay.chunk_v = chk, chv
            if N:
                if hook is not None:
                    hook("before", x, p, lc, dict(candK=ck, candV=cv, candT=ct, ring_before=ring_before, N=N))
                lc.step(ck, cv, ct, lay)
                if hook is not None:
                    hook("after", x, p, lc, dict(candK=ck, candV=cv, candT=ct, N=N))
            else:
                lc.update(None, None, None, None, None, lay)
            outs.append(lc.attention(q, out_f32=True))
            x.prev_k, x.prev_v = chk, chv
        self.c += 1
        self._prepared = None
        return outs, p

    def step(self, hook=None):
        """prepare() and run() of the next chunk."""
        self.prepare()
        return self.run(hook)

    # -- checkpoint / resume of the persistent temporal state ----------------
    def state(self) -> Dict:
        """Bank, window ring, sink and previous chunk of every layer, the
        chunk counter, and each frame stream's position (device streams:
        their generator state and drift)."""
        st = {"chunk": self.c, "layers": []}
        for x in self.L:
            e = {"bank": x.cache.bank.clone(), "ring": (x.ring_k.clone(), x.ring_v.clone()),
                 "sink": None if x.sink_k is None else (x.sink_k.clone(), x.sink_v.clone()),
                 "prev": None if x.prev_k is None else (x.prev_k.clone(), x.prev_v.clone())}
            if self.source == "device":
                e["stream"] = (x.stream.gen.get_state(), x.stream.drift.clone(), x.stream.t)
            st["layers"].append(e)
        return st

    def load_state(self, st: Dict):
        if self.source != "device":
            raise ValueError("resume needs device streams (host streams cannot seek)")
        self.c = int(st["chunk"])
        for x, e in zip(self.L, st["layers"]):
            x.cache.bank.copy_(e["bank"])
            x.ring_k.copy_(e["ring"][0])
            x.ring_v.copy_(e["ring"][1])
            x.sink_k, x.sink_v = (None, None) if e["sink"] is None else (e["sink"][0].clone(), e["sink"][1].clone())
            x.prev_k, x.prev_v = (None, None) if e["prev"] is None else (e["prev"][0].clone(), e["prev"][1].clone())
            gs, drift, t = e["stream"]
            x.stream.gen.set_state(gs)
            x.stream.drift.copy_(drift)
            x.stream.t = t
