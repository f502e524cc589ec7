"""Seeded synthetic frames generated on the GPU with PyTorch (input synthesis
only; none of the method's arithmetic).

The streaming rollout of 30 layers x 240 latent frames needs about 40 GB of
fresh keys, values and queries; drawing them with NumPy would take most of
an hour, so the benchmark draws them on the device.  The key model is the one
of ``kvsynth.LayerGen`` -- per-position Gaussian base, AR(1) temporal drift
(coefficient 0.95, stationary unit variance, drift of frame 0 zero), N(0, 0.1^2)
noise, N(0, 1) values and queries, 3D rotary embedding with interleaved pairs
(temporal pairs first) and base 10000, one rounding to bf16 -- with draws
from a per-layer ``torch.Generator`` instead of NumPy's Philox streams, so
the frames are statistically alike but not equal to LayerGen's.
"""
from __future__ import annotations

import math

import torch

from . import AR_RHO, NOISE_STD, ROPE_BASE, Workload, rope_split


class DeviceStream:
    """Frames of one layer in time order, on the current CUDA device."""

    def __init__(self, wl: Workload, seed: int = 0, layer: int = 0, dtype=torch.bfloat16):
        self.wl, self.dtype = wl, dtype
        dev = torch.device("cuda")
        self.gen = torch.Generator(device=dev)
        self.gen.manual_seed((seed * 1_000_003 + layer * 7919 + 17) & 0x7FFFFFFF)
        H, F, d = wl.H, wl.F, wl.d
        self.base = torch.randn(H, F, d, generator=self.gen, device=dev)
        self.drift = torch.zeros(H, F, d, device=dev)
        nt, nh, nw = rope_split(d)
        self.nt = nt
        p = torch.arange(F, device=dev)
        row, col = (p // wl.width).double(), (p % wl.width).double()
        fh = ROPE_BASE ** (-torch.arange(nh, device=dev, dtype=torch.float64) / nh)
        fw = ROPE_BASE ** (-torch.arange(nw, device=dev, dtype=torch.float64) / nw)
        ang = torch.cat([row[:, None] * fh[None, :], col[:, None] * fw[None, :]], dim=1)   # [F, nh + nw]
        self.cs_sp = torch.cos(ang).float(), torch.sin(ang).float()
        self.ft = ROPE_BASE ** (-torch.arange(nt, device=dev, dtype=torch.float64) / nt)
        self.t = 0

    def _rotate(self, x: torch.Tensor, t: int) -> torch.Tensor:
        a = (t * self.ft).float()
        ct, st = torch.cos(a), torch.sin(a)
        c = torch.cat([ct[None, :].expand(x.shape[1], -1), self.cs_sp[0]], dim=1)   # [F, d/2]
        s = torch.cat([st[None, :].expand(x.shape[1], -1), self.cs_sp[1]], dim=1)
        xe, xo = x[..., 0::2], x[..., 1::2]
        out = torch.empty_like(x)
        out[..., 0::2] = xe * c - xo * s
        out[..., 1::2] = xe * s + xo * c
        return out

    def frame(self, t: int, rope_t=None):
        """(keys, values, queries) [H][F][d] of frame t (t = 0, 1, ... in order)."""
        if t != self.t:
            raise ValueError(f"frames come in order: expected {self.t}, got {t}")
        wl = self.wl
        shape = (wl.H, wl.F, wl.d)
        if t > 0:
            z = torch.randn(shape, generator=self.gen, device="cuda")
            self.drift.mul_(AR_RHO).add_(z, alpha=math.sqrt(1.0 - AR_RHO * AR_RHO))
        noise = torch.randn(shape, generator=self.gen, device="cuda")
        pre = self.base + self.drift + NOISE_STD * noise
        rt = t if rope_t is None else rope_t
        keys = self._rotate(pre, rt).to(self.dtype)
        values = torch.randn(shape, generator=self.gen, device="cuda").to(self.dtype)
        queries = self._rotate(torch.randn(shape, generator=self.gen, device="cuda"), rt).to(self.dtype)
        self.t += 1
        return keys, values, queries
