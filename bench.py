"""Benchmark: the head-wise compressed KV cache hot path on one GPU.

The headline step is one layer-chunk at 480P (Wan2.1-1.3B-like layer: 12
heads, head_dim 128, bf16, 1,560 tokens per latent frame):

  kvbank_score   Soft-Riesz disturbance of 23,400 candidate keys against the
                 9,360-state bank of every head, mean-normalised, ordered
  kvbank_update  crossing scan, shared prefix, eviction, density fix-ups,
                 gather into the bank, segment tables
  chunk_attention  4,680 chunk queries over sink + bank + 6-frame window +
                 chunk (up to 24,960 keys per head)

The bank is restored from a device snapshot at the start of every step (the
same update is replayed), and that copy is inside the timed region.  Inputs
are synthetic (seeded kvsynth generator), resident in HBM before timing
starts.  The same JSON line also carries the 1080P layer-chunk, the
Forcing-KV hybrid layer at 480P and the 30-layer streaming rollout, each
timed with HIP events on the stream the library launches on.  Prints one
JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/chunk/layer + attention TFLOP/s (% of bf16 peak) at 480P and 1080P, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def attn_traffic_file(config: str) -> str:
    """The committed attention HBM-traffic record of a workload."""
    return os.path.join(ROOT, "profiles", f"attn_bf16_kernel_{config}_hbm_traffic.md")


ATTN_SOURCES = ("kv_cache_compression_head_amd/csrc/kvb_attention.hip",
                "kv_cache_compression_head_amd/csrc/kvb_common.hpp")
HBM_SOURCES = ("kv_cache_compression_head_amd/csrc/kvb_select.hip",
               "kv_cache_compression_head_amd/csrc/kvb_forcing.hip",
               "kv_cache_compression_head_amd/csrc/kvb_common.hpp")
DENSITY_SOURCES = ("kv_cache_compression_head_amd/csrc/kvb_gram.hip",
                   "kv_cache_compression_head_amd/csrc/kvb_common.hpp")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def setup(name: str, seed: int = 0, policy: int = 0, tau=None):
    import numpy as np
    import torch
    import kv_cache_compression_head_amd as kb
    from kv_cache_compression_head_amd.pipeline import LayerCache
    from kvsynth import WORKLOADS, LayerGen, frame_tokens

    wl = WORKLOADS[name]
    if tau is not None:
        import dataclasses
        wl = dataclasses.replace(wl, tau=float(tau))
    gen = LayerGen(wl, seed, 0)
    kdt = torch.bfloat16
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(kdt).contiguous()
    devi = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")
    (b0, b1), (c0, c1) = wl.bank_updates
    w0, w1 = wl.window
    q0, q1 = wl.chunk
    t = time.time()
    inp = {}
    inp["bankK"], inp["bankV"], inp["bankT"] = dev(gen.keys_all(range(b0, b1))), dev(gen.values_all(range(b0, b1))), devi(frame_tokens(wl, b0, b1))
    inp["candK"], inp["candV"], inp["candT"] = dev(gen.keys_all(range(c0, c1))), dev(gen.values_all(range(c0, c1))), devi(frame_tokens(wl, c0, c1))
    rw = [f - w0 for f in range(w0, w1)]
    rc = [f - w0 for f in range(q0, q1)]
    lay = kb.KVLayout(sink_k=dev(gen.keys_all([0])), sink_v=dev(gen.values_all([0])),
                      win_k=dev(gen.keys_all(range(w0, w1), rw)), win_v=dev(gen.values_all(range(w0, w1))),
                      win_start=0, win_len=(w1 - w0) * wl.F,
                      chunk_k=dev(gen.keys_all(range(q0, q1), rc)), chunk_v=dev(gen.values_all(range(q0, q1))))
    Q = dev(gen.queries_all(range(q0, q1), rc))
    log(f"inputs generated in {time.time() - t:.1f}s")
    desc = kb.LayerDesc(H=wl.H, d=wl.d, M=wl.M, dtype=kb.KVB_BF16, frame_tokens=wl.F, labels=[0] * wl.H,
                        tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p, policy=policy)
    lc = LayerCache(desc, seg_cap=8, max_N=max(inp["candK"].shape[1], inp["bankK"].shape[1]))
    # cold bank: frames b0..b1 admitted together into the empty bank
    lc.step(inp["bankK"], inp["bankV"], inp["bankT"], lay)
    torch.cuda.synchronize()
    assert int(lc.bank.count.min().cpu()) == wl.M, "cold bank not full"
    snap = lc.bank.clone()
    O = torch.empty(wl.H, wl.Lq, wl.d, dtype=kdt, device="cuda")
    return wl, lc, snap, inp, lay, Q, O


def one_step(lc, snap, inp, lay, Q, O, ev=None):
    if ev is not None:
        ev[0].record()
    lc.bank.copy_(snap)
    if ev is not None:
        ev[1].record()
    D, s, o = lc.score(inp["candK"], inp["candT"], lay)
    if ev is not None:
        ev[2].record()
    lc.update(inp["candK"], inp["candV"], inp["candT"], D, o, lay)
    if ev is not None:
        ev[3].record()
    lc.attention(Q, O)
    if ev is not None:
        ev[4].record()


def attention_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_attention_traffic(config: str):
    """HBM bytes per attention launch from the committed FETCH_SIZE /
    WRITE_SIZE profile, or None when that profile was taken on other kernel
    sources (or another workload)."""
    try:
        with open(attn_traffic_file(config)) as fh:
            kv = dict(l.split(":", 1) for l in fh.read().splitlines() if l.startswith("record."))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("record.workload") != config or kv.get("record.kernel_sources_sha256") != attention_source_digest():
        return None
    return int(kv["record.traffic_bytes_per_launch"])


def memory_keys_bench(wl, iters: int = 20):
    """Timing of the memory-key write path on the workload's window: the
    oldest 3 of its frames leave the ring (re-rotated to temporal coordinate
    0, values copied) and 3 arriving frames take their slots.  HBM-bound:
    bytes per launch = read departing K,V + write candidates + read arriving
    + write ring = 4 x 2 x H x rows x d x 2."""
    import torch
    import kv_cache_compression_head_amd as kb
    W = wl.window[1] - wl.window[0]
    n = 3 * wl.F
    cap = W * wl.F
    g = torch.Generator(device="cuda").manual_seed(0)
    mk = lambda r: torch.randn(wl.H, r, wl.d, device="cuda", generator=g).to(torch.bfloat16)
    rk, rv, nk, nv = mk(cap), mk(cap), mk(n), mk(n)
    ck, cv = torch.empty_like(nk), torch.empty_like(nv)
    desc = kb.LayerDesc(H=wl.H, d=wl.d, M=wl.M, dtype=kb.KVB_BF16, frame_tokens=wl.F, labels=[0] * wl.H)
    call = lambda i: kb.kvbank_window_advance(desc, rk, rv, (i * n) % cap, n, 1, ck, cv, nk, nv)
    for i in range(3):
        call(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = 4 * 2 * wl.H * n * wl.d * 2
    return {"kernel": "window_advance_kernel (kvbank_window_advance)", "rows": n, "ms": round(ms, 4),
            "bytes_per_launch": nbytes, "GB/s": round(nbytes / ms / 1e6, 1),
            "frac_hbm_peak": round(nbytes / ms / 1e6 / 8000.0, 4)}


def head_profile_bench(wl, iters: int = 3):
    """Timing of the Forcing-KV offline head profiling on the workload's
    attention shape: the chunk's queries over sink + history + transition +
    chunk keys (one call: one-hot fill, table rewrite, the attention kernels
    with one-hot values, the per-head reduction)."""
    import numpy as np
    import torch
    import kv_cache_compression_head_amd as kb
    H, d, F, Lq = wl.H, wl.d, wl.F, wl.Lq
    W = wl.window[1] - wl.window[0]
    sizes = [(1, F), (0, wl.M + (W - 1) * F), (2, F), (3, Lq)]   # sink, bank + older window, transition, chunk
    g = torch.Generator(device="cuda").manual_seed(1)
    Q = torch.randn(H, Lq, d, device="cuda", generator=g).to(torch.bfloat16)
    Ks = [torch.randn(H, n, d, device="cuda", generator=g).to(torch.bfloat16) for _, n in sizes]
    seg_cap = 4
    arr = (kb.kvb_segment * (H * seg_cap))()
    reg = np.zeros((H, seg_cap), np.int32)
    for h in range(H):
        for i, ((r, n), K) in enumerate(zip(sizes, Ks)):
            arr[h * seg_cap + i] = kb.kvb_segment(K[h].data_ptr(), 0, n, 0)
            reg[h, i] = r
    segs = torch.from_numpy(np.frombuffer(bytes(arr), dtype=np.uint8).copy()).to("cuda")
    nseg = torch.full((H,), seg_cap, dtype=torch.int32, device="cuda")
    region = torch.from_numpy(reg).to("cuda")
    max_len = max(n for _, n in sizes)
    ws = torch.empty(kb.forcing_head_profile_workspace_size(H, d, Lq, kb.KVB_BF16, seg_cap, max_len),
                     dtype=torch.uint8, device="cuda")
    score = torch.empty(H, dtype=torch.float32, device="cuda")
    label = torch.empty(H, dtype=torch.uint8, device="cuda")
    call = lambda: kb.forcing_head_profile(H, d, Lq, kb.KVB_BF16, Q, segs, nseg, seg_cap, region, max_len, score,
                                           label, ws=ws)
    call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    lkv = sum(n for _, n in sizes)
    flop = 4.0 * H * Lq * lkv * d
    return {"call": "forcing_head_profile", "ms": round(ms, 4), "Lkv": lkv,
            "TFLOP/s": round(flop / ms / 1e9, 1), "frac_bf16_peak": round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


def copy_calibration(mib: int, copies: int):
    """A plain device-to-device copy of known size, the yardstick for the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(copies):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": copies}), flush=True)


def cpu_baseline(name: str, seed: int = 0, heads=(0,)):
    """The fp64 oracle on a bounded sample: the same layer-chunk for a subset
    of heads (prefix computed over that subset), extrapolated to all heads."""
    import numpy as np
    from kvsynth import WORKLOADS, LayerGen, frame_tokens
    from oracle import density as od
    from oracle.attention import attention

    wl = WORKLOADS[name]
    gen = LayerGen(wl, seed, 0)
    prm = od.Params(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    (b0, b1), (c0, c1) = wl.bank_updates
    w0, w1 = wl.window
    q0, q1 = wl.chunk
    rw = [f - w0 for f in range(w0, w1)]
    rc = [f - w0 for f in range(q0, q1)]
    data = {}
    for h in heads:
        data[h] = dict(bK=gen.keys(h, range(b0, b1)).astype(np.float64), bV=gen.values(h, range(b0, b1)).astype(np.float64),
                       cK=gen.keys(h, range(c0, c1)).astype(np.float64), cV=gen.values(h, range(c0, c1)).astype(np.float64),
                       sK=gen.keys(h, [0]).astype(np.float64), sV=gen.values(h, [0]).astype(np.float64),
                       wK=gen.keys(h, range(w0, w1), rw).astype(np.float64), wV=gen.values(h, range(w0, w1)).astype(np.float64),
                       qK=gen.keys(h, range(q0, q1), rc).astype(np.float64), qV=gen.values(h, range(q0, q1)).astype(np.float64),
                       Q=gen.queries(h, range(q0, q1), rc).astype(np.float64))
    btok, ctok = frame_tokens(wl, b0, b1), frame_tokens(wl, c0, c1)
    # cold bank (not timed): co-admitted, baselines = in-bank density
    banks = [None] * wl.H
    for h in heads:
        banks[h] = od.HeadBank(btok.astype(np.int64), data[h]["bK"], data[h]["bV"], od.density(data[h]["bK"], prm))
    cK = np.zeros((wl.H, 0, wl.d))
    t = time.perf_counter()
    cK = {h: data[h]["cK"] for h in heads}
    cV = {h: data[h]["cV"] for h in heads}
    new, info = od.update_layer(banks, cK, cV, ctok, prm, heads=list(heads))
    for h in heads:
        K = np.concatenate([data[h]["sK"], new[h].K, data[h]["wK"], data[h]["qK"]])
        V = np.concatenate([data[h]["sV"], new[h].V, data[h]["wV"], data[h]["qV"]])
        attention(data[h]["Q"], K, V)
    dt = time.perf_counter() - t
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    return dt, threads, info.kstar


def blas_info():
    """BLAS library and thread count NumPy runs on (for the CPU baseline)."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "arch": i.get("architecture")}
    except Exception:
        pass
    return {"vendor": None, "version": None, "threads": None, "arch": None}


def cpu_baseline_sampled(name: str, seed: int = 0, head: int = 0, rows: int = 4096):
    """The fp64 oracle on a bounded, row-sampled piece of one head of the
    layer-chunk, extrapolated to the layer.  Every stage of the oracle is a
    sum over independent rows (candidates for the disturbance, bank states
    for the crossing scan and the new bank's densities, queries for
    attention), so each stage is timed on its first `rows` rows and scaled by
    its full row count and by the head count."""
    import numpy as np
    from kvsynth import WORKLOADS, LayerGen, frame_tokens
    from oracle import density as od
    from oracle.attention import attention

    wl = WORKLOADS[name]
    gen = LayerGen(wl, seed, 0)
    prm = od.Params(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    (b0, b1), (c0, c1) = wl.bank_updates
    w0, w1 = wl.window
    q0, q1 = wl.chunk
    rw = [f - w0 for f in range(w0, w1)]
    rc = [f - w0 for f in range(q0, q1)]
    bK = gen.keys(head, range(b0, b1)).astype(np.float64)
    cK = gen.keys(head, range(c0, c1)).astype(np.float64)
    Q = gen.queries(head, range(q0, q1), rc).astype(np.float64)
    Kall = np.concatenate([gen.keys(head, [0]), bK, gen.keys(head, range(w0, w1), rw), gen.keys(head, range(q0, q1), rc)]
                          ).astype(np.float64)
    Vall = np.concatenate([gen.values(head, [0]), gen.values(head, range(b0, b1)), gen.values(head, range(w0, w1)),
                           gen.values(head, range(q0, q1))]).astype(np.float64)
    n, N = bK.shape[0], cK.shape[0]
    kmax = min(N, wl.M)
    parts = {}
    t = time.perf_counter()
    od.phi_rowsum(cK[:rows], bK, prm)                       # disturbance of `rows` candidates
    parts["disturbance"] = (time.perf_counter() - t) * N / rows
    r0 = od.phi_rowsum(bK[:rows], bK, prm) - 1.0
    t = time.perf_counter()
    od.crossing_times(bK[:rows], r0, r0, cK[:kmax], prm)    # crossing scan of `rows` bank states
    parts["crossing_scan"] = (time.perf_counter() - t) * n / rows
    t = time.perf_counter()
    od.phi_rowsum(bK[:rows], bK, prm)                       # `rows` states' densities in an n-state bank
    # the update computes them for the bank before and after the update
    parts["bank_densities"] = 2.0 * (time.perf_counter() - t) * n / rows
    t = time.perf_counter()
    attention(Q[:rows], Kall, Vall)
    parts["attention"] = (time.perf_counter() - t) * wl.Lq / rows
    total_ms = sum(parts.values()) * wl.H * 1000.0
    return total_ms, {k: round(v * wl.H * 1000.0, 1) for k, v in parts.items()}


def layer_chunk(name: str, steps: int, warmup: int, policy: int = 0, tau=None):
    """Time `steps` layer-chunk steps after `warmup` untimed ones; returns the
    step's figures (stage times from events on the library's stream)."""
    import torch
    import kv_cache_compression_head_amd as kb
    wl, lc, snap, inp, lay, Q, O = setup(name, policy=policy, tau=tau)
    log(f"{name}: setup done")
    for _ in range(warmup):
        one_step(lc, snap, inp, lay, Q, O)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(lc, snap, inp, lay, Q, O, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = {"restore": [], "score": [], "update": [], "attention": []}
    for e in evs:
        stage["restore"].append(e[0].elapsed_time(e[1]))
        stage["score"].append(e[1].elapsed_time(e[2]))
        stage["update"].append(e[2].elapsed_time(e[3]))
        stage["attention"].append(e[3].elapsed_time(e[4]))
    avg = {k: sum(v) / len(v) for k, v in stage.items()}
    kstar = int(lc.out.k_star.cpu()[0])
    counts = lc.bank.count.cpu().tolist()
    lkv = [wl.F + c + (wl.window[1] - wl.window[0]) * wl.F + wl.Lq for c in counts]
    attn_flop = sum(4.0 * wl.Lq * l * wl.d for l in lkv)
    attn_tflops = attn_flop / (avg["attention"] * 1e-3) / 1e12
    # algorithmic bytes of the attention launch: Q + O + each head's K and V once
    attn_bytes = sum(2 * wl.Lq * wl.d * 2 + 2 * l * wl.d * 2 for l in lkv)
    # the chunk_attention call: attn_bf16_kernel, plus attn_merge_kernel when
    # the balanced grid splits items (timed together, as one call)
    bal = kb.chunk_attention_workspace_size(wl.H, wl.d, wl.Lq, kb.KVB_BF16) > 0
    kname = "attn_bf16_kernel + attn_merge_kernel" if bal else "attn_bf16_kernel"
    roof = {"kernel": f"{kname} (chunk_attention)", "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_attention_traffic(name), "algorithmic_flop_per_launch": attn_flop,
            "algorithmic_bytes_per_launch": attn_bytes}
    # Soft-Riesz pair counts of the density stages (the algorithmic work; the
    # crossing scan's figure is its upper bound n * min(N, M))
    n0 = int(snap.count.min().cpu())
    N = inp["candK"].shape[1]
    ev = lc.out.n_evicted.cpu().tolist()
    # the crossing scan runs unless the whole bank is replaced (min(N, M) = M:
    # k* = M without it, reported as n_mandatory = -1)
    scanned = min(lc.out.n_mandatory.cpu().tolist()) >= 0
    score_pairs = wl.H * n0 * N
    upd_pairs = sum((n0 * min(N, wl.M) if scanned else 0) + (n0 - e) * e + kstar * min(e, n0 - e)
                    + kstar * (kstar - 1) // 2 for e in ev)
    valu = recorded_valu_per_pair(name)

    def pair_roof(pairs, ms, stage_name):
        rate = pairs / (ms * 1e-3)
        r = {"pairs": pairs, "pairs_per_s": rate, "mfma_equiv_tflops": round(rate * 2 * wl.d / 1e12, 2),
             "frac_bf16_peak": round(rate * 2 * wl.d / 1e12 / PEAK_BF16_TFLOPS, 4)}
        v = valu.get(stage_name) if valu else None
        if v is not None:
            # counted VALU issue cycles per pair (SIMD cycles, from the
            # instruction counters) against 1,024 SIMDs at 2.4 GHz
            r["valu_cycles_per_pair"] = v
            r["frac_valu_bound"] = round(rate * v / (256 * 4 * 2.4e9), 4)
        else:
            r["valu_cycles_per_pair"] = None
            r["frac_valu_bound"] = None
        return r
    density_roof = {"score": pair_roof(score_pairs, avg["score"], "score"),
                    "update": pair_roof(upd_pairs, avg["update"], "update")}
    res = {"ms_per_step": wall * 1000.0 / steps, "stages_ms": {k: round(v, 4) for k, v in avg.items()},
           "attention_tflops": round(attn_tflops, 2),
           "attention_frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
           "k_star": kstar, "evicted_per_head": ev[:1] + ([] if len(set(ev)) == 1 else ev[1:]),
           "crossing_scan": scanned,
           "roofline": roof, "density_stages": density_roof, "hbm_kernels": recorded_hbm_kernels(name),
           "workload": f"{name}: one layer-chunk, H={wl.H}, d={wl.d}, F={wl.F}, M={wl.M}, N={N}, Lq={wl.Lq}, "
                       f"window={wl.window[1] - wl.window[0]} frames, tau={wl.tau}, sigma={wl.sigma}, p={wl.p}"
                       + (f", policy={policy}" if policy else "")}
    del lc, snap, inp, lay, Q, O
    torch.cuda.empty_cache()
    return wl, res


def recorded_valu_per_pair(config: str):
    """VALU issue cycles per Soft-Riesz pair of the scoring and update stages,
    from the committed instruction-counter profile (null when that profile
    was taken on other kernel sources)."""
    path = os.path.join(ROOT, "profiles", f"density_stages_{config}_valu.md")
    try:
        with open(path) as fh:
            kv = dict(l.split(":", 1) for l in fh.read().splitlines() if l.startswith("record."))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("record.kernel_sources_sha256") != density_source_digest():
        return None
    return {"score": float(kv["record.score_valu_cycles_per_pair"]),
            "update": float(kv["record.update_valu_cycles_per_pair"])}


def recorded_hbm_kernels(config: str):
    """HBM-bound kernels of the workload (the gather of admitted rows, the
    segment cosine) from the committed FETCH_SIZE / WRITE_SIZE profile:
    counted and algorithmic bytes over the dispatch's duration in that run,
    against 8 TB/s.  Null when the profile was taken on other kernel
    sources.  These kernels run inside kvbank_update / kvbank_score, so the
    bench's events cannot time them alone."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"kernels_{config}_hbm_traffic.md")
    try:
        with open(path) as fh:
            kv = dict(l.split(":", 1) for l in fh.read().splitlines() if l.startswith("record."))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    h = hashlib.sha256()
    for f in HBM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if kv.get("record.kernel_sources_sha256") != h.hexdigest():
        return None
    out = {}
    for name in ("gather", "segment_cosine", "segment_cosine_30_layers"):
        if f"record.{name}_us" not in kv:
            continue
        us = float(kv[f"record.{name}_us"])
        cb, ab = int(kv[f"record.{name}_counted_bytes"]), int(kv[f"record.{name}_algorithmic_bytes"])
        out[name] = {"kernel": kv[f"record.{name}_kernel"], "us": us, "algorithmic_bytes": ab, "counted_bytes": cb,
                     "GB/s_algorithmic": round(ab / us / 1e3, 1), "GB/s_counted": round(cb / us / 1e3, 1),
                     "frac_hbm_peak": round(ab / us / 1e3 / PEAK_HBM_GBS, 4),
                     "source": f"profiles/kernels_{config}_hbm_traffic.md"}
    return out or None


def density_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in DENSITY_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def forcing_bench(steps: int = 10, seed: int = 0):
    """Forcing-KV hybrid layer at 480P (6 static / 6 dynamic heads, 12
    history frames of 1,560-token segments, 70 % kept): segment cosine and
    BottomK (kvbank_score), segment tables (kvbank_update) and the ragged
    chunk attention (static heads 7,800 keys, dynamic heads 18,720)."""
    import numpy as np
    import torch
    import kv_cache_compression_head_amd as kb
    from kv_cache_compression_head_amd.pipeline import LayerCache
    from kvsynth import WORKLOADS, LayerGen, frame_tokens, head_labels
    wl = WORKLOADS["fkv480p"]
    gen = LayerGen(wl, seed, 0)
    labels = head_labels(wl, seed)
    F, H, d = wl.F, wl.H, wl.d
    h0, h1 = wl.history
    c0, c1 = wl.chunk
    hist_f, ch_f = list(range(h0, h1)), list(range(c0, c1))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch.bfloat16).contiguous()
    hk, hv = dev(gen.keys_all(hist_f, hist_f)), dev(gen.values_all(hist_f))
    tok = torch.from_numpy(frame_tokens(wl, h0, h1)).to("cuda")
    lay = kb.KVLayout(sink_k=dev(gen.keys_all([0], [0])), sink_v=dev(gen.values_all([0])),
                      chunk_k=dev(gen.keys_all(ch_f, ch_f)), chunk_v=dev(gen.values_all(ch_f)))
    Q = dev(gen.queries_all(ch_f, ch_f))
    T = len(hist_f)
    items = T * (F // wl.seg_len)
    keep = int(math.floor(wl.retention * items))
    desc = kb.LayerDesc(H=H, d=d, M=0, dtype=kb.KVB_BF16, frame_tokens=F, labels=labels.tolist(),
                        seg_len=wl.seg_len, retention=wl.retention)
    lc = LayerCache(desc, seg_cap=min(256, 3 + keep))
    O = torch.empty(H, wl.Lq, d, dtype=torch.bfloat16, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        D, s, o = lc.score(hk, tok, lay)
        if ev is not None:
            ev[1].record()
        lc.update(hk, hv, tok, D, o, lay)
        if ev is not None:
            ev[2].record()
        lc.attention(Q, O)
        if ev is not None:
            ev[3].record()
    for _ in range(3):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    sc = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    up = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    at = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    ndyn = int((labels == 2).sum())
    cos_bytes = (T + 1) * F * ndyn * d * 2
    lkv = [F + (F if labels[h] == 1 else keep * wl.seg_len) + wl.Lq for h in range(H)]
    flop = sum(4.0 * wl.Lq * l * d for l in lkv)
    return {"workload": f"fkv480p: H={H} (6 static / 6 dynamic), d={d}, F={F}, {T} history frames, "
                        f"seg_len={wl.seg_len}, r={wl.retention}, Lq={wl.Lq}",
            "score_ms": round(sc, 4), "update_ms": round(up, 4), "attention_ms": round(at, 4),
            "step_ms": round(sc + up + at, 4),
            "segment_cosine": {"call": "kvbank_score (cos_rows_kernel + segmean_kernel + rank_sort_kernel)",
                               "bytes_read": cos_bytes, "GB/s": round(cos_bytes / sc / 1e6, 1),
                               "frac_hbm_peak": round(cos_bytes / sc / 1e6 / PEAK_HBM_GBS, 4)},
            "hbm_kernels": recorded_hbm_kernels("fkv480p"),
            "segment_scoring_layers": score_layers_bench(wl, labels, T),
            "attention": {"Lkv_static": F + F + wl.Lq, "Lkv_dynamic": F + keep * wl.seg_len + wl.Lq,
                          "TFLOP/s": round(flop / at / 1e9, 1),
                          "frac_bf16_peak": round(flop / at / 1e9 / PEAK_BF16_TFLOPS, 4)}}


def score_layers_bench(wl, labels, T, layers: int = 30, iters: int = 10):
    """kvbank_score_layers on the hybrid layer's shape for the 30 layers of
    the model at once (every layer's own history and chunk keys, drawn on the
    device): one launch each for the cosines, the segment means and the
    BottomK orders.  Bytes = the dynamic heads' history and first chunk frame
    of every layer, read once."""
    import torch
    import kv_cache_compression_head_amd as kb
    H, d, F = wl.H, wl.d, wl.F
    N = T * F
    desc = kb.LayerDesc(H=H, d=d, M=0, dtype=kb.KVB_BF16, frame_tokens=F, labels=[int(x) for x in labels],
                        seg_len=wl.seg_len, retention=wl.retention)
    g = torch.Generator(device="cuda").manual_seed(3)
    K = torch.randn(layers, H, N, d, device="cuda", generator=g).to(torch.bfloat16)
    C = torch.randn(layers, H, wl.Lq, d, device="cuda", generator=g).to(torch.bfloat16)
    sc = torch.empty(layers, H, N, dtype=torch.float32, device="cuda")
    od = torch.empty(layers, H, N, dtype=torch.int32, device="cuda")
    ws = torch.empty(kb.kvbank_score_layers_workspace_size(desc, layers, N), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        kb.kvbank_score_layers(desc, K, C, sc, od, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        kb.kvbank_score_layers(desc, K, C, sc, od, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    ndyn = int(sum(1 for x in labels if int(x) == 2))
    nbytes = layers * (T + 1) * F * ndyn * d * 2
    del K, C, sc, od, ws
    torch.cuda.empty_cache()
    return {"call": "kvbank_score_layers (cos_rows_kernel + segmean_kernel + rank_sort_kernel, all layers)",
            "layers": layers, "ms": round(ms, 4), "bytes_read": nbytes, "GB/s": round(nbytes / ms / 1e6, 1),
            "frac_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}


def rollout_bench(chunks: int, layers: int = 0, seed: int = 0, policy: int = 0):
    """Streaming rollout: every chunk runs, for each of the 30 layers, the
    window advance (departing frames re-rotated into bank candidates),
    kvbank_score, kvbank_update and chunk_attention.  Each layer draws its
    own seeded frames on the GPU before the chunk's timed region (prepare);
    the library calls of all layers are timed with events around run()."""
    import numpy as np
    import torch
    from kv_cache_compression_head_amd.rollout import Rollout
    from kvsynth import WORKLOADS
    wl = WORKLOADS["rollout"]
    L = layers or wl.layers
    r = Rollout(wl, L, seed=seed, source="device", policy=policy)
    ms, ks, counts, evs = [], [], [], []
    for c in range(chunks):
        r.prepare()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _, p = r.run()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        lc0 = r.L[0].cache
        ks.append(int(lc0.out.k_star.cpu()[0]) if len(p.departed) else None)
        evs.append(int(lc0.out.n_evicted.cpu().sum()) if len(p.departed) else None)
        counts.append(int(lc0.bank.count.max().cpu()))
    steady = [m for c, m in enumerate(ms) if c >= 4]   # every chunk from the fourth on offers 3 frames
    a = np.asarray(steady)
    adm = [k for k in ks if k is not None]
    return {"workload": f"rollout: {L} layers x {wl.H} heads, 480P (F={wl.F}), M={wl.M}, W={wl.window_frames} frames, "
                        f"{chunks} chunks of {wl.chunk_frames} frames; per chunk and layer: window advance, score, "
                        f"update, attention" + (f"; policy={policy}" if policy else ""),
            "chunks": chunks, "layers": L, "total_ms": round(float(sum(ms)), 2),
            "ms_per_chunk_steady": {"mean": round(float(a.mean()), 3), "p50": round(float(np.percentile(a, 50)), 3),
                                    "p99": round(float(np.percentile(a, 99)), 3)},
            "ms_per_layer_chunk_steady": round(float(a.mean()) / L, 4),
            "layer0_k_star_per_update": adm, "layer0_admitted_total": int(sum(adm)),
            "layer0_evicted_per_update_all_heads": [e for e in evs if e is not None],
            "layer0_bank_count_per_chunk": counts,
            "bank_bytes_per_layer": int(r.L[0].cache.bank.K.numel() * 2 * 2)}


# ---------------------------------------------------------------------------
# rocprofv3 summaries (the tables under profiles/ are printed by these)
# ---------------------------------------------------------------------------

def kernel_role(name: str, seq: dict) -> str:
    """Short role label of a dispatch from its (demangled, untruncated)
    kernel name.  gram_kernel<E, D, MODE, SELF, CLIST, DIRECT>: scoring
    (no lists), the two fix-ups on index lists (survivors x evicted, then
    admitted x fix-list, in launch order), the symmetric admitted x admitted
    pass; scan_kernel<E, D, MODE, SUM, DIRECT>: crossing scan or rho' at k*."""
    import re
    base = re.sub(r"^void\s+", "", name).split("(")[0]
    short = base.split("<")[0].split("::")[-1]
    args = re.findall(r"<(.*)>", base)
    targs = [a.strip() for a in args[0].split(",")] if args else []
    if short == "gram_kernel" and len(targs) >= 6:
        self_, clist = targs[3] == "true", targs[4] == "true"
        if not clist:
            return "gram_kernel [scoring: candidates x bank]"
        if self_:
            return "gram_kernel [fix-up: admitted x admitted, symmetric]"
        k = seq.get("fix", 0)
        seq["fix"] = k + 1
        return "gram_kernel [fix-up: survivors x evicted]" if k % 2 == 0 else \
            "gram_kernel [fix-up: admitted x survivors-or-evicted]"
    if short == "scan_kernel" and len(targs) >= 5:
        return "scan_kernel [rho' at k*]" if targs[3] == "true" else "scan_kernel [crossing scan]"
    return short


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_trace(d: str):
    """Markdown table of kernel durations per role and grid size from a
    `rocprofv3 --kernel-trace` csv output directory."""
    rows = sorted(_csv_rows(d, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    seq, agg = {}, {}
    for r in rows:
        role = kernel_role(r["Kernel_Name"], seq)
        grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0) * int(r.get("Grid_Size_Y", 1) or 1) * \
            int(r.get("Grid_Size_Z", 1) or 1)
        wg = int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 1)) or 1)
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        agg.setdefault((role, grid // max(wg, 1)), []).append(us)
    tot = sum(sum(v) for v in agg.values())
    print("| kernel (role) | work-groups | calls | total ms | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|---|---|")
    for (role, wgs), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {role} | {wgs} | {len(v)} | {sum(v) / 1000:.3f} | {sum(v) / len(v):.1f} | {min(v):.1f} | "
              f"{max(v):.1f} | {100 * sum(v) / tot:.2f}% |")


def summarize_counters(d: str, min_us: float = 0.0):
    """Markdown table of per-dispatch counter averages per role from a
    `rocprofv3 --pmc` csv output directory (one row per dispatch and
    counter), with the dispatch duration."""
    rows = _csv_rows(d, "counter_collection.csv")
    disp = {}
    for r in rows:
        key = (int(r["Dispatch_Id"]), r.get("Agent_Id", ""))
        wg = int(r.get("Workgroup_Size", 0) or 0) or 1
        e = disp.setdefault(key, {"name": r["Kernel_Name"], "start": int(r.get("Start_Timestamp", 0) or 0),
                                  "end": int(r.get("End_Timestamp", 0) or 0), "c": {},
                                  "wgs": int(r.get("Grid_Size", 0) or 0) // wg})
        e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    seq, agg = {}, {}
    for key in sorted(disp, key=lambda k: disp[k]["start"] or k[0]):
        e = disp[key]
        role = kernel_role(e["name"], seq)
        us = (e["end"] - e["start"]) / 1000.0
        if us < min_us:
            continue
        a = agg.setdefault((role, e["wgs"]), {"n": 0, "us": 0.0, "c": {}})
        a["n"] += 1
        a["us"] += us
        for k, v in e["c"].items():
            a["c"][k] = a["c"].get(k, 0.0) + v
    names = sorted({k for a in agg.values() for k in a["c"]})
    print("| kernel (role) | work-groups | dispatches | avg us | " + " | ".join(f"{n} / dispatch" for n in names)
          + " |")
    print("|---|---|---|---|" + "---|" * len(names))
    for (role, wgs), a in sorted(agg.items(), key=lambda kv: -kv[1]["us"]):
        vals = " | ".join(f"{a['c'].get(n, 0.0) / a['n']:.6g}" for n in names)
        print(f"| {role} | {wgs} | {a['n']} | {a['us'] / a['n']:.1f} | {vals} |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="480p", choices=["480p", "480p_block", "1080p", "fkv480p", "rollout"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="480p/1080p: time that layer-chunk only (no other workloads, side benches)")
    ap.add_argument("--chunks", type=int, default=80, help="rollout chunks (rollout config and the default line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter yardstick) and exit")
    ap.add_argument("--policy", type=int, default=0,
                    help="DensityKV policy variant bits (KVB_POL_*; 0 = the method)")
    ap.add_argument("--tau", type=float, default=None, help="override the workload's density growth bound")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the per-role kernel-time table of a rocprofv3 --kernel-trace csv directory and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the per-role counter table of a rocprofv3 --pmc csv directory and exit")
    ap.add_argument("--min-us", type=float, default=0.0, help="with --summarize-counters: skip shorter dispatches")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.min_us)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              "multi-GPU component to run)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 4)
        return
    import kv_cache_compression_head_amd as kb
    kb.load_library()
    base = {"n_gpus": 1, "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic"}
    if args.config == "rollout":
        ro = rollout_bench(args.chunks, policy=args.policy)
        ms = ro["ms_per_chunk_steady"]["mean"]
        print(json.dumps({"metric": METRIC, "value": ms, "unit": "ms/chunk (30 layers)", "steps": args.chunks,
                          "warmup": 0, "ms_per_step": ms, **base, "config": {"workload": ro["workload"]},
                          "rollout": ro}), flush=True)
        return
    if args.config == "fkv480p":
        fk = forcing_bench(args.steps)
        print(json.dumps({"metric": METRIC, "value": fk["step_ms"], "unit": "ms/chunk/layer", "steps": args.steps,
                          "warmup": 3, "ms_per_step": fk["step_ms"], **base, "config": {"workload": fk["workload"]},
                          "fkv480p": fk}), flush=True)
        return
    if (args.policy or args.tau is not None) and not args.no_cpu_baseline:
        print("bench.py: --policy / --tau measure variants; run them with --no-cpu-baseline", file=sys.stderr)
        sys.exit(2)
    wl, main_res = layer_chunk(args.config, args.steps, args.warmup, args.policy, args.tau)
    ms_step = main_res.pop("ms_per_step")
    res = {"metric": METRIC, "value": round(ms_step, 4), "unit": "ms/chunk/layer", "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), **base,
           "config": {"workload": main_res.pop("workload")}, **main_res}
    if not args.no_extras:
        res["memory_keys"] = memory_keys_bench(wl)
        res["head_profile"] = head_profile_bench(wl)
    cpu = None
    if not args.no_cpu_baseline:
        blas = blas_info()
        if args.config == "480p":
            # a bounded sample of about 10-30 s of CPU work: one head first, then
            # as many heads as fill about 12 s when one head is quicker than 10 s
            log("cpu baseline (oracle, 1 head)")
            nh = 1
            dt, threads, ks_cpu = cpu_baseline(args.config)
            if dt < 10.0 and wl.H > 1:
                nh = min(wl.H, int(math.ceil(12.0 / max(dt, 1e-3))))
                log(f"cpu baseline (oracle, {nh} heads)")
                dt, threads, ks_cpu = cpu_baseline(args.config, heads=tuple(range(nh)))
            cpu = {"value": round(dt / nh * wl.H * 1000.0, 1), "unit": "ms/chunk/layer", "cores": threads,
                   "kind": "oracle",
                   "sample": f"fp64 oracle, {nh} of {wl.H} heads of the same layer-chunk (score + update + "
                             f"attention, prefix over those heads alone, k*={ks_cpu}), measured {dt:.2f} s, "
                             f"scaled x{wl.H / nh:.2f}",
                   "blas": blas, "host_cpus": len(os.sched_getaffinity(0))}
        else:
            log(f"cpu baseline ({args.config}, row-sampled oracle)")
            v, parts = cpu_baseline_sampled(args.config)
            cpu = {"value": round(v, 1), "unit": "ms/chunk/layer", "cores": blas["threads"], "kind": "oracle",
                   "sample": "fp64 oracle on head 0, each stage timed on its first 4,096 rows and scaled by its "
                             "row count and by 12 heads (extrapolation)", "stages_ms": parts, "blas": blas,
                   "host_cpus": len(os.sched_getaffinity(0))}
    res["cpu_baseline"] = cpu
    if args.config == "480p" and not args.no_extras and args.policy == 0 and args.tau is None:
        log("1080p layer-chunk")
        wl1, r1 = layer_chunk("1080p", max(3, min(args.steps, 5)), 2)
        r1["value_ms_per_chunk_layer"] = round(r1.pop("ms_per_step"), 3)
        if not args.no_cpu_baseline:
            log("cpu baseline (1080p, row-sampled oracle)")
            v, parts = cpu_baseline_sampled("1080p")
            r1["cpu_baseline"] = {"value": round(v, 1), "unit": "ms/chunk/layer", "cores": blas["threads"],
                                  "kind": "oracle",
                                  "sample": "fp64 oracle on head 0, each stage timed on its first 4,096 rows and "
                                            "scaled by its row count and by 12 heads (extrapolation)",
                                  "stages_ms": parts, "blas": blas}
        res["1080p"] = r1
        log("480p_block layer-chunk (one finalized block into a full bank)")
        wlb, rb = layer_chunk("480p_block", max(5, min(args.steps, 20)), 3)
        rb["value_ms_per_chunk_layer"] = round(rb.pop("ms_per_step"), 4)
        res["480p_block"] = rb
        log("fkv480p hybrid layer")
        res["fkv480p"] = forcing_bench()
        log(f"rollout ({args.chunks} chunks x 30 layers)")
        res["rollout"] = rollout_bench(args.chunks)
        # under the method's own rule the banks stop admitting once every
        # prefix would push a state past tau while the bank is below capacity
        # (layer0_k_star_per_update above); with the fill-below-capacity
        # variant the banks reach M and then admit and evict at every update
        nf = min(args.chunks, 40)
        log(f"rollout, fill below capacity ({nf} chunks x 30 layers)")
        res["rollout_fill"] = rollout_bench(nf, policy=kb.KVB_POL_FILL_BELOW_CAP)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
