"""Python binding of libkvbank (head-wise compressed KV cache, MI355X).

Argument marshalling only: every step runs in the HIP kernels of
``libkvbank.so``.  PyTorch provides device memory and the current HIP stream.
The names mirror the C ABI in ``include/kvbank.h``.  There is no fallback:
if the library is missing or the device is not a gfx950 GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

__all__ = [
    "KVB_BF16", "KVB_F32", "KVB_HEAD_DENSITY", "KVB_HEAD_STATIC", "KVB_HEAD_DYNAMIC", "KVB_POL_SOURCE_ORDER",
    "KVB_POL_REFRESH_BASELINE", "KVB_POL_EVICT_DENSEST", "KVB_POL_EVICT_OLDEST", "KVB_POL_HEAD_PREFIX",
    "KVB_POL_FILL_BELOW_CAP", "KVB_POL_FRAME_BOTTOMK", "KVB_POL_SEQUENTIAL",
    "KvbError", "load_library", "kvbank_workspace_size", "kvbank_score", "kvbank_update",
    "kvbank_score_layers", "kvbank_score_layers_workspace_size",
    "chunk_attention", "chunk_attention_noalloc", "chunk_attention_workspace_size", "kvbank_window_advance",
    "forcing_head_profile",
    "forcing_head_profile_workspace_size", "kvb_last_error", "LayerDesc", "Bank", "KVLayout", "UpdateOut",
    "HEADER_FUNCTIONS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvbank.so")

KVB_BF16, KVB_F32 = 0, 1
KVB_HEAD_DENSITY, KVB_HEAD_STATIC, KVB_HEAD_DYNAMIC = 0, 1, 2
# DensityKV policy variants (kvb_params.policy); 0 is the method
KVB_POL_SOURCE_ORDER, KVB_POL_REFRESH_BASELINE, KVB_POL_EVICT_DENSEST = 1, 2, 4
KVB_POL_EVICT_OLDEST, KVB_POL_HEAD_PREFIX, KVB_POL_FILL_BELOW_CAP = 8, 16, 32
KVB_POL_FRAME_BOTTOMK = 64
KVB_POL_SEQUENTIAL = 128
KVB_MAX_SEGMENTS = 256
HEADER_FUNCTIONS = ("kvbank_workspace_size", "kvbank_score", "kvbank_update", "chunk_attention",
                    "chunk_attention_workspace_size", "kvbank_window_advance", "forcing_head_profile_workspace_size",
                    "forcing_head_profile", "kvb_last_error", "kvb_source_hash", "chunk_attention_noalloc",
                    "kvbank_score_layers_workspace_size", "kvbank_score_layers")

_c_i32, _c_f32, _c_f64, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_void_p


class kvb_params(ctypes.Structure):
    _fields_ = [("tau", _c_f32), ("sigma", _c_f32), ("eps", _c_f32), ("p", _c_f32),
                ("seg_len", _c_i32), ("policy", ctypes.c_uint32), ("retention", _c_f64)]


class kvb_layer_desc(ctypes.Structure):
    _fields_ = [("H", _c_i32), ("d", _c_i32), ("M", _c_i32), ("dtype", _c_i32), ("frame_tokens", _c_i32),
                ("desc_dim", _c_i32), ("label", ctypes.POINTER(ctypes.c_uint8)), ("params", kvb_params)]


class kvb_bank(ctypes.Structure):
    _fields_ = [("K", _vp), ("V", _vp), ("tok", _vp), ("rho0", _vp), ("rho", _vp), ("count", _vp), ("X", _vp)]


class kvb_kv_layout(ctypes.Structure):
    _fields_ = [("sink_k", _vp), ("sink_v", _vp), ("sink_len", _c_i32), ("win_cap", _c_i32),
                ("win_k", _vp), ("win_v", _vp), ("win_start", _c_i32), ("win_len", _c_i32),
                ("chunk_k", _vp), ("chunk_v", _vp), ("chunk_len", _c_i32), ("reserved", _c_i32),
                ("cand_x", _vp)]


class kvb_segment(ctypes.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("len", _c_i32), ("reserved", _c_i32)]


class kvb_update_out(ctypes.Structure):
    _fields_ = [("k_star", _vp), ("n_mandatory", _vp), ("n_evicted", _vp), ("status", _vp),
                ("segs", _vp), ("nseg", _vp), ("seg_cap", _c_i32), ("reserved", _c_i32),
                ("t_cross", _vp), ("rho_proj", _vp)]


class kvb_attn_desc(ctypes.Structure):
    _fields_ = [("H", _c_i32), ("d", _c_i32), ("Lq", _c_i32), ("dtype", _c_i32), ("scale", _c_f32),
                ("seg_cap", _c_i32), ("out_f32", _c_i32), ("reserved", _c_i32)]


class KvbError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"kvbank status {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libkvbank.so (built by ``kv_cache_compression_head_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m kv_cache_compression_head_amd.build`")
    lib = ctypes.CDLL(p)
    lib.kvbank_workspace_size.argtypes = [ctypes.POINTER(kvb_layer_desc), _c_i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.kvbank_score.argtypes = [ctypes.POINTER(kvb_layer_desc), ctypes.POINTER(kvb_bank), _vp, _vp, _c_i32,
                                 ctypes.POINTER(kvb_kv_layout), _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.kvbank_update.argtypes = [ctypes.POINTER(kvb_layer_desc), ctypes.POINTER(kvb_bank), _vp, _vp, _vp, _c_i32,
                                  _vp, _vp, ctypes.POINTER(kvb_kv_layout), ctypes.POINTER(kvb_update_out), _vp,
                                  ctypes.c_size_t, _vp]
    lib.kvbank_score_layers_workspace_size.argtypes = [ctypes.POINTER(kvb_layer_desc), _c_i32, _c_i32,
                                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.kvbank_score_layers.argtypes = [ctypes.POINTER(kvb_layer_desc), _c_i32, _vp, ctypes.c_int64, _vp,
                                        ctypes.c_int64, _c_i32, _c_i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.chunk_attention.argtypes = [ctypes.POINTER(kvb_attn_desc), _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.chunk_attention_noalloc.argtypes = [ctypes.POINTER(kvb_attn_desc), _vp, _vp, _vp, _vp, _vp]
    lib.chunk_attention_workspace_size.argtypes = [ctypes.POINTER(kvb_attn_desc), ctypes.POINTER(ctypes.c_size_t)]
    lib.kvbank_window_advance.argtypes = [ctypes.POINTER(kvb_layer_desc), _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                          _c_f32, _vp, _vp, _vp, _vp, _vp]
    lib.forcing_head_profile_workspace_size.argtypes = [ctypes.POINTER(kvb_attn_desc), _c_i32,
                                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.forcing_head_profile.argtypes = [ctypes.POINTER(kvb_attn_desc), _vp, _vp, _vp, _vp, _c_i32, _c_f32, _vp, _vp,
                                         _vp, _vp, ctypes.c_size_t, _vp]
    for f in ("kvbank_workspace_size", "kvbank_score", "kvbank_update", "chunk_attention", "chunk_attention_noalloc",
              "kvbank_score_layers_workspace_size", "kvbank_score_layers",
              "chunk_attention_workspace_size", "kvbank_window_advance", "forcing_head_profile_workspace_size",
              "forcing_head_profile"):
        getattr(lib, f).restype = ctypes.c_int
    lib.kvb_last_error.restype = ctypes.c_char_p
    lib.kvb_last_error.argtypes = []
    lib.kvb_source_hash.restype = ctypes.c_char_p
    lib.kvb_source_hash.argtypes = []
    if os.path.abspath(p) == LIB_PATH:
        # the in-tree library must have been built from the sources beside it
        from .build import source_hash
        built, here = lib.kvb_source_hash().decode(), source_hash()
        if built != here:
            raise ImportError(f"{p} is stale (built from sources {built[:12]}, the tree holds {here[:12]}): "
                              "rebuild it with `python -m kv_cache_compression_head_amd.build`")
    if path is None:
        _lib = lib
    return lib


def kvb_last_error() -> str:
    return load_library().kvb_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise KvbError(rc, kvb_last_error())


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LayerDesc:
    H: int
    d: int
    M: int
    dtype: int
    frame_tokens: int
    labels: Sequence[int]
    tau: float = 2.0
    sigma: float = 8.0
    eps: float = 1.0
    p: float = 2.0
    seg_len: int = 0
    retention: float = 0.0
    policy: int = 0          # OR of KVB_POL_*
    desc_dim: int = 0        # 0: keys are the density descriptors; 64 / 128 / 256 (bf16): Bank.X and KVLayout.cand_x

    def c(self):
        lab = (ctypes.c_uint8 * max(1, len(self.labels)))(*[int(x) for x in self.labels])
        prm = kvb_params(float(self.tau), float(self.sigma), float(self.eps), float(self.p), int(self.seg_len),
                         int(self.policy), float(self.retention))
        desc = kvb_layer_desc(int(self.H), int(self.d), int(self.M), int(self.dtype), int(self.frame_tokens),
                              int(self.desc_dim), ctypes.cast(lab, ctypes.POINTER(ctypes.c_uint8)), prm)
        desc._keep = lab   # keep the label array alive with the descriptor
        return desc


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _req(t, name, dtype=None, shape=None):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _kv_dtype(desc_dtype: int):
    import torch
    return torch.bfloat16 if desc_dtype == KVB_BF16 else torch.float32


@dataclasses.dataclass
class Bank:
    """Device SoA of one layer's banks (all [H][M][...] tensors)."""
    K: "object"
    V: "object"
    tok: "object"
    rho0: "object"
    rho: "object"
    count: "object"
    X: "object" = None       # [H][M][desc_dim] density descriptors (desc_dim > 0)

    @staticmethod
    def empty(H: int, M: int, d: int, dtype, desc_dim: int = 0):
        import torch
        dev = torch.device("cuda")
        return Bank(torch.zeros(H, M, d, dtype=dtype, device=dev), torch.zeros(H, M, d, dtype=dtype, device=dev),
                    torch.full((H, M), -1, dtype=torch.int32, device=dev),
                    torch.zeros(H, M, dtype=torch.float32, device=dev),
                    torch.zeros(H, M, dtype=torch.float32, device=dev),
                    torch.zeros(H, dtype=torch.int32, device=dev),
                    torch.zeros(H, M, desc_dim, dtype=dtype, device=dev) if desc_dim else None)

    def _parts(self):
        return tuple(x for x in (self.K, self.V, self.tok, self.rho0, self.rho, self.count, self.X) if x is not None)

    def clone(self) -> "Bank":
        return Bank(*(x.clone() for x in (self.K, self.V, self.tok, self.rho0, self.rho, self.count)),
                    None if self.X is None else self.X.clone())

    def copy_(self, other: "Bank"):
        for a, b in zip(self._parts(), other._parts()):
            a.copy_(b, non_blocking=True)

    def c(self):
        return kvb_bank(_ptr(self.K), _ptr(self.V), _ptr(self.tok), _ptr(self.rho0), _ptr(self.rho), _ptr(self.count),
                        _ptr(self.X))


@dataclasses.dataclass
class KVLayout:
    """Non-bank KV of the layer: sink, local-window ring and current chunk ([H][rows][d])."""
    sink_k: "object" = None
    sink_v: "object" = None
    win_k: "object" = None
    win_v: "object" = None
    win_start: int = 0
    win_len: int = 0
    chunk_k: "object" = None
    chunk_v: "object" = None
    cand_x: "object" = None   # [H][N][desc_dim] candidate density descriptors (desc_dim > 0)

    def c(self):
        sl = 0 if self.sink_k is None else int(self.sink_k.shape[1])
        wc = 0 if self.win_k is None else int(self.win_k.shape[1])
        cl = 0 if self.chunk_k is None else int(self.chunk_k.shape[1])
        return kvb_kv_layout(_ptr(self.sink_k), _ptr(self.sink_v), sl, wc, _ptr(self.win_k), _ptr(self.win_v),
                             int(self.win_start), int(self.win_len), _ptr(self.chunk_k), _ptr(self.chunk_v), cl, 0,
                             _ptr(self.cand_x))


@dataclasses.dataclass
class UpdateOut:
    k_star: "object"
    n_mandatory: "object"
    n_evicted: "object"
    status: "object"
    segs: "object"      # uint8 [H * seg_cap * 24] device buffer of kvb_segment
    nseg: "object"
    seg_cap: int
    t_cross: "object" = None     # optional [H][M] int32
    rho_proj: "object" = None    # optional [H][M] float32

    @staticmethod
    def alloc(H: int, seg_cap: int = 8, M: int = 0, diagnostics: bool = False):
        import torch
        dev = torch.device("cuda")
        # k_star: [H] so that a per-head prefix (KVB_POL_HEAD_PREFIX) fits; a shared one is entry 0
        o = UpdateOut(torch.zeros(H, dtype=torch.int32, device=dev), torch.zeros(H, dtype=torch.int32, device=dev),
                      torch.zeros(H, dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev),
                      torch.zeros(H * seg_cap * ctypes.sizeof(kvb_segment), dtype=torch.uint8, device=dev),
                      torch.zeros(H, dtype=torch.int32, device=dev), int(seg_cap))
        if diagnostics and M > 0:
            o.t_cross = torch.zeros(H, M, dtype=torch.int32, device=dev)
            o.rho_proj = torch.zeros(H, M, dtype=torch.float32, device=dev)
        return o

    def c(self):
        return kvb_update_out(_ptr(self.k_star), _ptr(self.n_mandatory), _ptr(self.n_evicted), _ptr(self.status),
                              _ptr(self.segs), _ptr(self.nseg), int(self.seg_cap), 0, _ptr(self.t_cross),
                              _ptr(self.rho_proj))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def kvbank_workspace_size(layer: LayerDesc, N: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    desc = layer.c()
    _check(lib.kvbank_workspace_size(ctypes.byref(desc), int(N), ctypes.byref(out)))
    return int(out.value)


def _req_desc(layer: LayerDesc, bank: Optional[Bank], lay: Optional[KVLayout], N: int):
    """Shapes of the density descriptors when the layer uses its own (desc_dim > 0)."""
    if not layer.desc_dim:
        return
    kd = _kv_dtype(layer.dtype)
    if bank is not None:
        _req(bank.X, "bank.X", kd, (layer.H, layer.M, layer.desc_dim))
    if lay is None or lay.cand_x is None:
        raise ValueError("desc_dim > 0 needs KVLayout.cand_x")
    _req(lay.cand_x, "cand_x", kd, (layer.H, N, layer.desc_dim))


def kvbank_score(layer: LayerDesc, bank: Optional[Bank], cand_k, cand_tok, N: int, lay: Optional[KVLayout],
                 out_D, out_score, out_order, ws, stream=None):
    import torch
    lib = load_library()
    desc = layer.c()
    kd = _kv_dtype(layer.dtype)
    if N > 0:
        _req(cand_k, "cand_k", kd, (layer.H, N, layer.d))
        _req(out_score, "out_score", torch.float32, (layer.H, N))
        _req(out_order, "out_order", torch.int32, (layer.H, N))
        _req_desc(layer, bank, lay, N)
    cb = bank.c() if bank is not None else None
    cl = lay.c() if lay is not None else None
    _check(lib.kvbank_score(ctypes.byref(desc), ctypes.byref(cb) if cb is not None else None, _ptr(cand_k),
                            _ptr(cand_tok), int(N), ctypes.byref(cl) if cl is not None else None, _ptr(out_D),
                            _ptr(out_score), _ptr(out_order), _ptr(ws), 0 if ws is None else ws.numel(),
                            _stream(stream)))


def kvbank_score_layers_workspace_size(layer: LayerDesc, nlayers: int, N: int) -> int:
    lib = load_library()
    desc = layer.c()
    n = ctypes.c_size_t(0)
    _check(lib.kvbank_score_layers_workspace_size(ctypes.byref(desc), int(nlayers), int(N), ctypes.byref(n)))
    return int(n.value)


def kvbank_score_layers(layer: LayerDesc, cand_k, chunk_k, out_score, out_order, ws=None, stream=None):
    """Forcing-KV segment scoring of several layers that share `layer`:
    cand_k [L][H][N][d] history keys, chunk_k [L][H][chunk_len][d] the
    chunk's keys, out_score float32 / out_order int32 [L][H][N].  Allocates
    the workspace when none is given."""
    import torch
    lib = load_library()
    desc = layer.c()
    kd = _kv_dtype(layer.dtype)
    if cand_k.dim() != 4 or chunk_k.dim() != 4:
        raise ValueError("cand_k and chunk_k must be [L][H][rows][d]")
    nl, N, cl = int(cand_k.shape[0]), int(cand_k.shape[2]), int(chunk_k.shape[2])
    _req(cand_k, "cand_k", kd, (nl, layer.H, N, layer.d))
    _req(chunk_k, "chunk_k", kd, (nl, layer.H, cl, layer.d))
    _req(out_score, "out_score", torch.float32, (nl, layer.H, N))
    _req(out_order, "out_order", torch.int32, (nl, layer.H, N))
    if ws is None:
        ws = torch.empty(max(1, kvbank_score_layers_workspace_size(layer, nl, N)), dtype=torch.uint8,
                         device=cand_k.device)
    _check(lib.kvbank_score_layers(ctypes.byref(desc), nl, _ptr(cand_k), layer.H * N * layer.d, _ptr(chunk_k),
                                   layer.H * cl * layer.d, cl, N, _ptr(out_score), _ptr(out_order), _ptr(ws),
                                   ws.numel(), _stream(stream)))


def kvbank_update(layer: LayerDesc, bank: Optional[Bank], cand_k, cand_v, cand_tok, N: int, D, order,
                  lay: KVLayout, out: UpdateOut, ws, stream=None):
    lib = load_library()
    desc = layer.c()
    kd = _kv_dtype(layer.dtype)
    if N > 0:
        _req(cand_k, "cand_k", kd, (layer.H, N, layer.d))
        _req(cand_v, "cand_v", kd, (layer.H, N, layer.d))
        _req_desc(layer, bank, lay, N)
    cb = bank.c() if bank is not None else None
    cl = lay.c()
    co = out.c()
    _check(lib.kvbank_update(ctypes.byref(desc), ctypes.byref(cb) if cb is not None else None, _ptr(cand_k),
                             _ptr(cand_v), _ptr(cand_tok), int(N), _ptr(D), _ptr(order), ctypes.byref(cl),
                             ctypes.byref(co), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def chunk_attention_workspace_size(H: int, d: int, Lq: int, dtype: int) -> int:
    lib = load_library()
    desc = kvb_attn_desc(int(H), int(d), int(Lq), int(dtype), 0.0, 1, 0, 0)
    n = ctypes.c_size_t(0)
    _check(lib.chunk_attention_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def chunk_attention(H: int, d: int, Lq: int, dtype: int, Q, segs, nseg, seg_cap: int, O, scale: float = 0.0,
                    out_f32: bool = False, stream=None, ws="auto"):
    """ws: a device uint8 tensor of at least chunk_attention_workspace_size
    bytes (balanced grid), None (one work-group per item), or "auto" (a
    workspace tensor is allocated here)."""
    lib = load_library()
    kd = _kv_dtype(dtype)
    _req(Q, "Q", kd, (H, Lq, d))
    desc = kvb_attn_desc(int(H), int(d), int(Lq), int(dtype), float(scale), int(seg_cap), int(bool(out_f32)), 0)
    if isinstance(ws, str):
        import torch
        n = chunk_attention_workspace_size(H, d, Lq, dtype)
        ws = torch.empty(n, dtype=torch.uint8, device=Q.device) if n > 0 else None
    _check(lib.chunk_attention(ctypes.byref(desc), _ptr(Q), _ptr(segs), _ptr(nseg), _ptr(O), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream)))


def chunk_attention_noalloc(H: int, d: int, Lq: int, dtype: int, Q, segs, nseg, seg_cap: int, O,
                            scale: float = 0.0, out_f32: bool = False, stream=None):
    """chunk_attention without a workspace: the balanced grid's partials live
    in the library's static per-GPU scratch array (nothing is allocated).
    Calls that overlap on one GPU race on that array."""
    lib = load_library()
    kd = _kv_dtype(dtype)
    _req(Q, "Q", kd, (H, Lq, d))
    desc = kvb_attn_desc(int(H), int(d), int(Lq), int(dtype), float(scale), int(seg_cap), int(bool(out_f32)), 0)
    _check(lib.chunk_attention_noalloc(ctypes.byref(desc), _ptr(Q), _ptr(segs), _ptr(nseg), _ptr(O), _stream(stream)))


def kvbank_window_advance(layer: LayerDesc, ring_k, ring_v, start: int, n_rows: int, t_first: int, cand_k, cand_v,
                          new_k=None, new_v=None, rope_base: float = 10000.0, stream=None):
    """Departing window rows -> bank candidates at temporal coordinate 0;
    arriving rows (optional) into the freed ring slots.  ring_* [H][cap][d],
    cand_* / new_* [H][n_rows][d], all of the layer's dtype."""
    lib = load_library()
    kd = _kv_dtype(layer.dtype)
    cap = int(ring_k.shape[1])
    _req(ring_k, "ring_k", kd, (layer.H, cap, layer.d))
    _req(ring_v, "ring_v", kd, (layer.H, cap, layer.d))
    _req(cand_k, "cand_k", kd, (layer.H, n_rows, layer.d))
    _req(cand_v, "cand_v", kd, (layer.H, n_rows, layer.d))
    if new_k is not None:
        _req(new_k, "new_k", kd, (layer.H, n_rows, layer.d))
        _req(new_v, "new_v", kd, (layer.H, n_rows, layer.d))
    desc = layer.c()
    _check(lib.kvbank_window_advance(ctypes.byref(desc), _ptr(ring_k), _ptr(ring_v), cap, int(start), int(n_rows),
                                     int(t_first), float(rope_base), _ptr(new_k), _ptr(new_v), _ptr(cand_k),
                                     _ptr(cand_v), _stream(stream)))


def forcing_head_profile_workspace_size(H: int, d: int, Lq: int, dtype: int, seg_cap: int, max_len: int) -> int:
    lib = load_library()
    desc = kvb_attn_desc(int(H), int(d), int(Lq), int(dtype), 0.0, int(seg_cap), 1, 0)
    n = ctypes.c_size_t(0)
    _check(lib.forcing_head_profile_workspace_size(ctypes.byref(desc), int(max_len), ctypes.byref(n)))
    return int(n.value)


def forcing_head_profile(H: int, d: int, Lq: int, dtype: int, Q, segs, nseg, seg_cap: int, region, max_len: int,
                         score, label, mass=None, alpha: float = 0.8, scale: float = 0.0, ws=None, stream=None):
    """Per-head attention masses, score and static/dynamic label (see
    forcing_head_profile in the C header).  ws: a device uint8 tensor of
    forcing_head_profile_workspace_size bytes, or None to allocate one."""
    lib = load_library()
    _req(Q, "Q", _kv_dtype(dtype), (H, Lq, d))
    desc = kvb_attn_desc(int(H), int(d), int(Lq), int(dtype), float(scale), int(seg_cap), 1, 0)
    if ws is None:
        import torch
        ws = torch.empty(forcing_head_profile_workspace_size(H, d, Lq, dtype, seg_cap, max_len), dtype=torch.uint8,
                         device=Q.device)
    _check(lib.forcing_head_profile(ctypes.byref(desc), _ptr(Q), _ptr(segs), _ptr(nseg), _ptr(region), int(max_len),
                                    float(alpha), _ptr(mass), _ptr(score), _ptr(label), _ptr(ws), ws.numel(),
                                    _stream(stream)))
