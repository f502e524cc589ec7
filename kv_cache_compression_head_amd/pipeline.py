"""One attention layer's compressed KV cache driven through libkvbank.

Plumbing only: allocates device tensors with PyTorch and calls the C ABI in
stream order (score -> update -> attention).  No arithmetic of the method
happens here.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import (KVB_BF16, KVB_F32, Bank, KVLayout, LayerDesc, UpdateOut, chunk_attention,
               chunk_attention_workspace_size, kvb_segment,
               kvbank_score, kvbank_update, kvbank_workspace_size)


def torch_dtype(dtype: int):
    return torch.bfloat16 if dtype == KVB_BF16 else torch.float32


class LayerCache:
    """Bank, workspace and outputs of one layer on the current device."""

    def __init__(self, desc: LayerDesc, seg_cap: int = 8, max_N: int = 0, diagnostics: bool = False):
        self.desc = desc
        self.H, self.d, self.M = desc.H, desc.d, desc.M
        self.kdt = torch_dtype(desc.dtype)
        self.bank = Bank.empty(self.H, max(self.M, 1), self.d, self.kdt, desc.desc_dim) if self.M > 0 else None
        self.out = UpdateOut.alloc(self.H, seg_cap, self.M, diagnostics)
        self.ws = None
        self._aws = None
        self._ws_N = -1
        self._bufs = {}
        if max_N:
            self.reserve(max_N)

    def reserve(self, N: int):
        if N > self._ws_N:
            nbytes = kvbank_workspace_size(self.desc, N)
            self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
            self._ws_N = N
            self._bufs["D"] = torch.empty(self.H, N, dtype=torch.float32, device="cuda")
            self._bufs["score"] = torch.empty(self.H, N, dtype=torch.float32, device="cuda")
            self._bufs["order"] = torch.empty(self.H, N, dtype=torch.int32, device="cuda")

    def outputs(self, N: int):
        """(D, score, order) views of the reserved buffers for N candidates."""
        self.reserve(N)
        if N == self._ws_N:
            return self._bufs["D"], self._bufs["score"], self._bufs["order"]
        return (self._bufs["D"].view(-1)[: self.H * N].view(self.H, N),
                self._bufs["score"].view(-1)[: self.H * N].view(self.H, N),
                self._bufs["order"].view(-1)[: self.H * N].view(self.H, N))

    def score(self, cand_k, cand_tok, lay: Optional[KVLayout] = None):
        N = 0 if cand_k is None else int(cand_k.shape[1])
        D, s, o = self.outputs(N)
        kvbank_score(self.desc, self.bank, cand_k, cand_tok, N, lay, D, s, o, self.ws)
        return D, s, o

    def update(self, cand_k, cand_v, cand_tok, D, order, lay: KVLayout):
        N = 0 if cand_k is None else int(cand_k.shape[1])
        self.reserve(N)
        kvbank_update(self.desc, self.bank, cand_k, cand_v, cand_tok, N, D, order, lay, self.out, self.ws)

    def step(self, cand_k, cand_v, cand_tok, lay: KVLayout):
        D, s, o = self.score(cand_k, cand_tok, lay)
        self.update(cand_k, cand_v, cand_tok, D, o, lay)
        return D, s, o

    def attention(self, Q, O=None, out_f32: bool = False):
        H, Lq, d = Q.shape
        if O is None:
            O = torch.empty(H, Lq, d, dtype=torch.float32 if out_f32 else Q.dtype, device=Q.device)
        # the balanced grid's partials: kept between calls, grown on demand
        n = chunk_attention_workspace_size(H, d, Lq, self.desc.dtype)
        if n > 0 and (self._aws is None or self._aws.numel() < n):
            self._aws = torch.empty(n, dtype=torch.uint8, device=Q.device)
        chunk_attention(H, d, Lq, self.desc.dtype, Q, self.out.segs, self.out.nseg, self.out.seg_cap, O,
                        out_f32=out_f32, ws=self._aws if n > 0 else None)
        return O

    # -- host views of the results (synchronising) --------------------------
    def segments(self):
        """Per head list of (k_ptr, v_ptr, len) from the device segment table."""
        raw = self.out.segs.cpu().numpy().tobytes()
        ns = self.out.nseg.cpu().tolist()
        arr = (kvb_segment * (self.H * self.out.seg_cap)).from_buffer_copy(raw)
        res = []
        for h in range(self.H):
            res.append([(arr[h * self.out.seg_cap + i].k, arr[h * self.out.seg_cap + i].v,
                         arr[h * self.out.seg_cap + i].len) for i in range(ns[h])])
        return res


def to_dev(x, dtype) -> torch.Tensor:
    """numpy float32 (already rounded to dtype) -> contiguous device tensor."""
    return torch.from_numpy(x).to(device="cuda").to(dtype).contiguous()
