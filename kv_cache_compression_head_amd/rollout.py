"""Streaming chunk-by-chunk rollout over several layers (orchestration only).

Timeline for chunk c (three latent frames [3c, 3c+3)): the sink is frame 0,
the local window holds the last W history frames [max(1, 3c-W), 3c), and the
frames that left the window since the previous chunk are offered to each
layer's per-head banks before the chunk's queries attend over
sink + bank + window + chunk (DensityKV card page, Figure 2; paper-summary
page, appendix D: sink frame + local window + bounded bank, N = 3 frames per
finalized block).  Keys use the memory-key rotary convention: sink and bank
keys carry temporal position 0, local keys and queries their position
relative to the window start.

Inputs come from the seeded ``kvsynth`` generator; every step of the method
runs in libkvbank through ``LayerCache``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

from kvsynth import LayerGen, Workload, frame_tokens

from . import KVB_BF16, KVB_F32, KVLayout, LayerDesc
from .pipeline import LayerCache


@dataclasses.dataclass
class ChunkPlan:
    chunk: int
    frames: range          # current chunk
    window: range          # local history window
    departed: range        # frames leaving the window now (bank candidates)
    rope_base: int


def plan(c: int, chunk_frames: int = 3, window_frames: int = 6) -> ChunkPlan:
    f0 = chunk_frames * c
    w0 = max(1, f0 - window_frames)
    prev = max(1, chunk_frames * (c - 1) - window_frames) if c > 0 else 1
    dep = range(prev, w0) if w0 > prev else range(0)
    win = range(w0, f0) if f0 > w0 else range(0)
    base = win.start if len(win) else f0
    return ChunkPlan(c, range(f0, f0 + chunk_frames), win, dep, base)


class Rollout:
    """Per-layer LayerCache state plus the synthetic input streams."""

    def __init__(self, wl: Workload, layers: int, seed: int = 0, diagnostics: bool = False):
        self.wl, self.layers, self.seed = wl, layers, seed
        self.kdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        dt = KVB_BF16 if wl.dtype == "bf16" else KVB_F32
        self.caches: List[LayerCache] = []
        self.gens: List[LayerGen] = []
        for l in range(layers):
            desc = LayerDesc(H=wl.H, d=wl.d, M=wl.M, dtype=dt, frame_tokens=wl.F, labels=[0] * wl.H,
                             tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
            self.caches.append(LayerCache(desc, seg_cap=8, max_N=3 * wl.F, diagnostics=diagnostics))
            self.gens.append(LayerGen(wl, seed, l))
        self.c = 0

    def _dev(self, x):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(self.kdt).contiguous()

    def inputs(self, l: int, p: ChunkPlan) -> Dict[str, np.ndarray]:
        g = self.gens[l]
        rt = lambda fr: [f - p.rope_base for f in fr]
        out = {
            "candK": g.keys_all(p.departed), "candV": g.values_all(p.departed),
            "candT": frame_tokens(self.wl, p.departed.start, p.departed.stop) if len(p.departed) else
            np.zeros(0, np.int32),
            "winK": g.keys_all(p.window, rt(p.window)), "winV": g.values_all(p.window),
            "chK": g.keys_all(p.frames, rt(p.frames)), "chV": g.values_all(p.frames),
            "Q": g.queries_all(p.frames, rt(p.frames)),
        }
        if p.chunk > 0:
            out["sinkK"], out["sinkV"] = g.keys_all([0]), g.values_all([0])
        return out

    def step(self, hook=None):
        """Advance one chunk over every layer; returns the attention outputs."""
        p = plan(self.c, self.wl.chunk_frames, self.wl.window_frames)
        outs = []
        for l, lc in enumerate(self.caches):
            x = self.inputs(l, p)
            lay = KVLayout()
            keep = {}
            if "sinkK" in x:
                keep["sk"], keep["sv"] = self._dev(x["sinkK"]), self._dev(x["sinkV"])
                lay.sink_k, lay.sink_v = keep["sk"], keep["sv"]
            if len(p.window):
                keep["wk"], keep["wv"] = self._dev(x["winK"]), self._dev(x["winV"])
                lay.win_k, lay.win_v, lay.win_start, lay.win_len = keep["wk"], keep["wv"], 0, len(p.window) * self.wl.F
            keep["ck"], keep["cv"] = self._dev(x["chK"]), self._dev(x["chV"])
            lay.chunk_k, lay.chunk_v = keep["ck"], keep["cv"]
            N = int(x["candT"].shape[0])
            if N:
                cK, cV = self._dev(x["candK"]), self._dev(x["candV"])
                cT = torch.from_numpy(x["candT"].astype(np.int32)).to("cuda")
                if hook is not None:
                    hook("before", l, p, lc, x)
                lc.step(cK, cV, cT, lay)
                if hook is not None:
                    hook("after", l, p, lc, x)
            else:
                lc.update(None, None, None, None, None, lay)
            outs.append(lc.attention(self._dev(x["Q"]), out_f32=True))
        self.c += 1
        return outs, p

    # -- checkpoint / resume of the persistent temporal state ----------------
    def state(self) -> Dict:
        return {"chunk": self.c, "banks": [lc.bank.clone() for lc in self.caches]}

    def load_state(self, st: Dict):
        self.c = int(st["chunk"])
        for lc, b in zip(self.caches, st["banks"]):
            lc.bank.copy_(b)
