"""Benchmark: one layer-chunk of the head-wise compressed KV cache on one GPU.

A step is the whole hot path for one layer and one chunk at 480P
(Wan2.1-1.3B-like layer: 12 heads, head_dim 128, bf16, 1,560 tokens per
latent frame):

  kvbank_score   Soft-Riesz disturbance of 23,400 candidate keys against the
                 9,360-state bank of every head, mean-normalised, ordered
  kvbank_update  crossing scan, shared prefix, eviction, density fix-ups,
                 gather into the bank, segment tables
  chunk_attention  4,680 chunk queries over sink + bank + 6-frame window +
                 chunk (up to 24,960 keys per head)

The bank is restored from a device snapshot at the start of every step (the
same update is replayed), and that copy is inside the timed region.
Inputs are synthetic (seeded kvsynth generator), resident in HBM before
timing starts.  Prints one JSON line.
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
# fp32 VALU lane-operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
PEAK_VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
# VALU issue slots per Soft-Riesz pair at p = 2 (fma, max, reciprocal at half
# rate = 2 slots, accumulate)
VALU_SLOTS_PER_PAIR = 5.0
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_kernel_480p_hbm_traffic.md")
ATTN_SOURCES = ("kv_cache_compression_head_amd/csrc/kvb_attention.hip",
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
        with open(ATTN_TRAFFIC_FILE) as fh:
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


def rollout_bench(steps: int, warmup_chunks: int):
    """Streaming rollout timing: every chunk runs score + update + attention
    for each of the 30 layers (480P, M = 9,360, 3 departing frames per
    chunk).  One seeded layer stream supplies the inputs of all layers (each
    layer keeps its own bank), so the inputs of a chunk are generated once;
    the banks are first streamed through warmup_chunks chunks to reach the
    steady state.  Returns (ms per chunk over all layers, details)."""
    import numpy as np
    import torch
    import kv_cache_compression_head_amd as kb
    from kv_cache_compression_head_amd.pipeline import LayerCache
    from kv_cache_compression_head_amd.rollout import plan
    from kvsynth import WORKLOADS, LayerGen, frame_tokens

    wl = WORKLOADS["rollout"]
    gen = LayerGen(wl, 0, 0)
    kdt = torch.bfloat16
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(kdt).contiguous()

    def chunk_inputs(c):
        p = plan(c, wl.chunk_frames, wl.window_frames)
        rt = lambda fr: [f - p.rope_base for f in fr]
        x = {"N": len(p.departed) * wl.F}
        if len(p.departed):
            x["cK"], x["cV"] = dev(gen.keys_all(p.departed)), dev(gen.values_all(p.departed))
            x["cT"] = torch.from_numpy(frame_tokens(wl, p.departed.start, p.departed.stop).astype(np.int32)).cuda()
        lay = kb.KVLayout()
        keep = []
        if c > 0:
            sk, sv = dev(gen.keys_all([0])), dev(gen.values_all([0]))
            keep += [sk, sv]
            lay.sink_k, lay.sink_v = sk, sv
        if len(p.window):
            wk, wv = dev(gen.keys_all(p.window, rt(p.window))), dev(gen.values_all(p.window))
            keep += [wk, wv]
            lay.win_k, lay.win_v, lay.win_start, lay.win_len = wk, wv, 0, len(p.window) * wl.F
        ck, cv = dev(gen.keys_all(p.frames, rt(p.frames))), dev(gen.values_all(p.frames))
        keep += [ck, cv]
        lay.chunk_k, lay.chunk_v = ck, cv
        x["lay"], x["keep"] = lay, keep
        x["Q"] = dev(gen.queries_all(p.frames, rt(p.frames)))
        return x

    t = time.time()
    chunks = [chunk_inputs(c) for c in range(warmup_chunks + steps)]
    log(f"rollout inputs for {len(chunks)} chunks generated in {time.time() - t:.1f}s")
    desc = kb.LayerDesc(H=wl.H, d=wl.d, M=wl.M, dtype=kb.KVB_BF16, frame_tokens=wl.F, labels=[0] * wl.H,
                        tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    caches = [LayerCache(desc, seg_cap=8, max_N=3 * wl.F) for _ in range(wl.layers)]
    O = torch.empty(wl.H, wl.Lq, wl.d, dtype=kdt, device="cuda")

    def run_chunk(x):
        for lc in caches:
            if x["N"]:
                lc.step(x["cK"], x["cV"], x["cT"], x["lay"])
            else:
                lc.update(None, None, None, None, None, x["lay"])
            lc.attention(x["Q"], O)

    for c in range(warmup_chunks):
        run_chunk(chunks[c])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in range(warmup_chunks, warmup_chunks + steps):
        run_chunk(chunks[c])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    counts = caches[0].bank.count.cpu().tolist()
    return ms, {"layers": wl.layers, "chunks_timed": steps, "first_timed_chunk": warmup_chunks,
                "bank_count_layer0": counts, "k_star_last": int(caches[0].out.k_star.cpu()[0]),
                "bank_bytes_per_layer": int(caches[0].bank.K.numel() * 2 * 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="480p", choices=["480p", "1080p", "rollout"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter yardstick) and exit")
    ap.add_argument("--policy", type=int, default=0,
                    help="DensityKV policy variant bits (KVB_POL_*; 0 = the method)")
    ap.add_argument("--tau", type=float, default=None, help="override the workload's density growth bound")
    args = ap.parse_args()
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
    if args.config == "rollout":
        ms, info = rollout_bench(args.steps, max(args.warmup, 6))
        print(json.dumps({
            "metric": METRIC, "value": round(ms, 3), "unit": "ms/chunk (30 layers)", "n_gpus": 1,
            "steps": args.steps, "warmup": max(args.warmup, 6), "ms_per_step": round(ms, 3),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "rollout: 30 layers x 12 heads, 480P (1,560 tokens/frame), M=9360, 3 departing "
                                   "frames per chunk, 6-frame window, 3-frame chunk; steady-state chunks"},
            "ms_per_layer_chunk": round(ms / info["layers"], 4), "rollout": info}), flush=True)
        return
    if (args.policy or args.tau is not None) and not args.no_cpu_baseline:
        print("bench.py: --policy / --tau measure variants; run them with --no-cpu-baseline", file=sys.stderr)
        sys.exit(2)
    wl, lc, snap, inp, lay, Q, O = setup(args.config, policy=args.policy, tau=args.tau)
    log("setup done")
    for _ in range(args.warmup):
        one_step(lc, snap, inp, lay, Q, O)
    torch.cuda.synchronize()
    # timed region: exactly K steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(lc, snap, inp, lay, Q, O, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1000.0 / args.steps
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
    import kv_cache_compression_head_amd as kb
    bal = kb.chunk_attention_workspace_size(wl.H, wl.d, wl.Lq, kb.KVB_BF16) > 0
    kname = "attn_bf16_kernel + attn_merge_kernel" if bal else "attn_bf16_kernel"
    roof = {"kernel": f"{kname} (chunk_attention)", "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_attention_traffic(args.config), "algorithmic_flop_per_launch": attn_flop,
            "algorithmic_bytes_per_launch": attn_bytes}
    # Soft-Riesz pair counts of the density stages (the algorithmic work; the
    # crossing scan's figure is its upper bound n * min(N, M))
    n0 = int(snap.count.min().cpu())
    N = inp["candK"].shape[1]
    ev = lc.out.n_evicted.cpu().tolist()
    score_pairs = wl.H * n0 * N
    upd_pairs = sum(n0 * min(N, wl.M) + (n0 - e) * e + kstar * min(e, n0 - e) + kstar * (kstar - 1) // 2 for e in ev)

    def pair_roof(pairs, ms):
        rate = pairs / (ms * 1e-3)
        return {"pairs": pairs, "pairs_per_s": rate, "mfma_equiv_tflops": round(rate * 2 * wl.d / 1e12, 2),
                "frac_bf16_peak": round(rate * 2 * wl.d / 1e12 / PEAK_BF16_TFLOPS, 4),
                "frac_valu_bound": round(rate * VALU_SLOTS_PER_PAIR / PEAK_VALU_LANE_OPS, 4)}
    density_roof = {"score": pair_roof(score_pairs, avg["score"]), "update": pair_roof(upd_pairs, avg["update"])}
    mem_keys = memory_keys_bench(wl)
    profile = head_profile_bench(wl)
    cpu = None
    if not args.no_cpu_baseline:
        # a bounded sample of about 10-30 s of CPU work: one head first, then
        # as many heads as fill about 12 s when one head is quicker than 10 s
        log("cpu baseline (oracle, 1 head)")
        nh = 1
        dt, threads, ks_cpu = cpu_baseline(args.config)
        if dt < 10.0 and wl.H > 1:
            nh = min(wl.H, int(math.ceil(12.0 / max(dt, 1e-3))))
            log(f"cpu baseline (oracle, {nh} heads)")
            dt, threads, ks_cpu = cpu_baseline(args.config, heads=tuple(range(nh)))
        cpu = {"value": round(dt / nh * wl.H * 1000.0, 1), "unit": "ms/chunk/layer", "cores": threads, "kind": "oracle",
               "sample": f"fp64 oracle, {nh} of {wl.H} heads of the same layer-chunk (score + update + attention, "
                         f"prefix over those heads alone, k*={ks_cpu}), measured {dt:.2f} s, scaled x{wl.H / nh:.2f}",
               "host_cpus": len(os.sched_getaffinity(0))}
    res = {
        "metric": METRIC, "value": round(ms_step, 4), "unit": "ms/chunk/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: one layer-chunk, H={wl.H}, d={wl.d}, F={wl.F}, M={wl.M}, "
                               f"N={inp['candK'].shape[1]}, Lq={wl.Lq}, window={wl.window[1] - wl.window[0]} frames, "
                               f"tau={wl.tau}, sigma={wl.sigma}, p={wl.p}"
                               + (f", policy={args.policy}" if args.policy else "")},
        "stages_ms": {k: round(v, 4) for k, v in avg.items()},
        "attention_tflops": round(attn_tflops, 2), "attention_frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "k_star": kstar, "roofline": roof, "density_stages": density_roof, "memory_keys": mem_keys,
        "head_profile": profile,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
