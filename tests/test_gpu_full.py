"""Full-size GPU parity.

480P layer-chunk, all 12 heads, unsampled: every disturbance, the whole
order, every crossing time, the shared prefix, the eviction set, every
density of the new bank and every attention row, against the fp64 oracle
with stage replay.  A second 480P case offers the pages' own per-block
candidate count (N = 4,680; DensityKV paper summary, appendix D) to a full
bank, so that part of the bank is evicted (densest completion and survivor
fix-ups at d = 128, M = 9,360).  1080P: every head's integer decisions, and
two heads replayed in fp64 without sampling, plus 1,024 query rows of every
head's attention.  The oracle's row blocks run in threads on the host.
"""
import math

import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, frame_tokens
from oracle import density as od

import gpu_common as gc
from _parity import GpuBank, default_workers, replay_update, sampled_update

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    od.set_workers(default_workers())
    yield
    od.set_workers(1)


def _layer_chunk(name, cand_frames=None, fp64_heads=None, qrows=None):
    """Cold bank (the first frame range co-admitted into the empty bank),
    then one update offering cand_frames (default: the workload's second
    range), then chunk attention.  fp64_heads: heads replayed in fp64
    (default all); qrows: attention rows checked per head (default all)."""
    import torch
    wl = WORKLOADS[name]
    prm = od.Params(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    gc.banner(f"full-size {name}: generating inputs")
    gen = LayerGen(wl, 0, 0)
    lc = gc.layer_for(wl, prm)
    heads = list(range(wl.H))
    rep_heads = heads if fp64_heads is None else list(fp64_heads)
    (b0, b1), (c0, c1) = wl.bank_updates
    if cand_frames is not None:
        c0, c1 = cand_frames
    gc.run_update(lc, gen, wl, prm, (b0, b1), heads, replay=False)
    cold = GpuBank.read(lc.bank)
    assert np.all(cold.count == wl.M)
    for h in heads:
        assert sorted(cold.tok[h].tolist()) == frame_tokens(wl, b0, b1).tolist()
        # co-admitted states share their baselines with their densities
        assert np.array_equal(cold.rho0[h], cold.rho[h])
    N = (c1 - c0) * wl.F
    gc.banner(f"full-size {name}: update with N={N}")
    candK, candV = gen.keys_all(range(c0, c1)), gen.values_all(range(c0, c1))
    ctok = frame_tokens(wl, c0, c1)
    kdt = gc.kv_dtype(wl)
    ai = gc.attn_inputs(gen, wl)
    lay = gc.layout_for(ai, kdt, win_start=777)
    cK, cV, ct = gc.dev(candK, kdt), gc.dev(candV, kdt), gc.dev_i32(ctok)
    D, s, o = lc.score(cK, ct, lay)
    lc.update(cK, cV, ct, D, o, lay)
    O = lc.attention(gc.dev(ai.Q, kdt), out_f32=True)
    torch.cuda.synchronize()
    assert int(lc.out.status.cpu()[0]) == 0
    after = GpuBank.read(lc.bank)
    gc.banner(f"full-size {name}: stage replay of heads {rep_heads[0]}..{rep_heads[-1]} ({len(rep_heads)} heads)")
    rep = replay_update(cold, after, candK.astype(np.float64), candV.astype(np.float64), np.asarray(ctok),
                        D.cpu().numpy(), s.cpu().numpy(), o.cpu().numpy(), lc.out.t_cross.cpu().numpy(),
                        lc.out.rho_proj.cpu().numpy(), lc.out.k_star.cpu().numpy(), lc.out.n_mandatory.cpu().numpy(),
                        lc.out.n_evicted.cpu().numpy(), prm, rep_heads, workers=1, kstar_heads=heads)
    rows = None if qrows is None else np.random.default_rng(2).choice(wl.Lq, qrows, replace=False)
    gc.banner(f"full-size {name}: attention of {'all' if rows is None else qrows} query rows per head")
    mx, mn = gc.check_attention(O.cpu().numpy(), ai, after, heads, 2e-2, 2e-3, rows=rows)
    gc.banner(f"full-size {name}: k*={rep.kstar} evicted/head={rep.evicted[:3]} order near-ties="
              f"{rep.order_near_ties} crossing near-ties={rep.crossing_near_ties} attention max-abs {mx:.2e} "
              f"mean-abs {mn:.2e}")
    return rep, cold, after


def test_480p_layer_chunk():
    rep, _, _ = _layer_chunk("480p")
    assert rep.kstar > 0


def test_480p_whole_bank_replaced_without_scan():
    """The 480P layer-chunk (N = 23,400 > M) without per-state diagnostics
    takes the path without the crossing scan (every state leaves at k* = M
    whatever crossed): the same bank, bit for bit, as with the scan."""
    import torch
    import kv_cache_compression_head_amd as kb
    wl = WORKLOADS["480p"]
    prm = od.Params(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    gen = LayerGen(wl, 0, 0)
    kdt = gc.kv_dtype(wl)
    a = gc.layer_for(wl, prm, diagnostics=True)
    b = gc.layer_for(wl, prm, diagnostics=False)
    for (t0, t1) in wl.bank_updates:
        gc.banner(f"480p whole-bank replacement: frames {t0}..{t1}")
        cK, cV = gc.dev(gen.keys_all(range(t0, t1)), kdt), gc.dev(gen.values_all(range(t0, t1)), kdt)
        ct = gc.dev_i32(frame_tokens(wl, t0, t1))
        for lc in (a, b):
            D, s, o = lc.score(cK, ct, kb.KVLayout())
            lc.update(cK, cV, ct, D, o, kb.KVLayout())
        torch.cuda.synchronize()
    assert b.out.n_mandatory.cpu().tolist() == [-1] * wl.H
    assert int(a.out.k_star.cpu()[0]) == wl.M
    for x, y in ((a.bank.K, b.bank.K), (a.bank.V, b.bank.V), (a.bank.tok, b.bank.tok), (a.bank.rho0, b.bank.rho0),
                 (a.bank.rho, b.bank.rho), (a.bank.count, b.bank.count)):
        assert torch.equal(x, y)


@pytest.mark.timeout(600)
def test_480p_partial_eviction():
    """One finalized block, N = 4,680 candidates (three frames), offered to
    a full bank of 9,360 (the 480p_block workload that bench.py times): the
    new bank keeps part of the old one."""
    wl = WORKLOADS["480p_block"]
    rep, cold, after = _layer_chunk("480p_block")
    assert 0 < rep.kstar <= 3 * wl.F
    for h in range(wl.H):
        e = rep.evicted[h]
        assert 0 < e < wl.M, f"head {h}: evicted {e}"
        kept = np.isin(cold.tok[h], after.tok[h, :after.count[h]])
        assert int(kept.sum()) == wl.M - e


@pytest.mark.timeout(900)
def test_1080p_layer_chunk():
    rep, _, _ = _layer_chunk("1080p", fp64_heads=(0, 11), qrows=1024)
    assert rep.kstar > 0


def _check_window_advance(ring_before, cand_k, cand_v, start, n_rows, F, t_first):
    """The GPU's departing rows against the oracle's memory-key re-rotation:
    values and spatial pairs bit for bit, temporal pairs within one bf16
    rounding of the exact rotation."""
    from oracle import rope as orope
    rk = ring_before[0].float().cpu().numpy()
    rv = ring_before[1].float().cpu().numpy()
    ref_k, ref_v, _, _ = orope.window_advance(rk, rv, start, n_rows, F, t_first)
    got_k = cand_k.float().cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(cand_v.float().cpu().numpy(), ref_v)
    nt = orope.temporal_pairs(got_k.shape[-1])
    np.testing.assert_array_equal(got_k[..., 2 * nt:], ref_k[..., 2 * nt:])
    err = np.abs(got_k[..., :2 * nt] - ref_k[..., :2 * nt])
    assert np.all(err <= 2.0 ** -8 * np.abs(ref_k[..., :2 * nt]) + 1e-30), err.max()
    return got_k


ROLLOUT_PARTS = 4


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", range(ROLLOUT_PARTS))
def test_rollout_layers_0_29_every_chunk(part):
    """Streaming rollout of layers 0 and 29 (each with its own seeded frame
    stream) over all 80 chunks, checked in four parts of 20 chunks (each
    part runs the rollout from chunk 0 and checks its own chunks, so no test
    runs for minutes).  At every bank update of both layers: the departing
    window rows against the oracle's re-rotation, then a full stage replay
    of all 12 heads (disturbance, order, crossings, prefix, evictions,
    new-bank densities and pairing).  Attention rows against the oracle at
    every chunk that admitted candidates and every tenth chunk.  Storage
    stays bounded by M."""
    import torch
    from kv_cache_compression_head_amd.rollout import Rollout
    from oracle.attention import attention as oracle_attention
    wl = WORKLOADS["rollout"]
    prm = od.Params(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    F, H = wl.F, wl.H
    layers = [0, wl.layers - 1]
    held, rho_prev, kstars = {}, {l: None for l in layers}, {l: [] for l in layers}

    per = wl.chunks // ROLLOUT_PARTS
    c_lo, c_hi = part * per, (part + 1) * per if part < ROLLOUT_PARTS - 1 else wl.chunks

    def hook(stage, x, p, lc, a):
        torch.cuda.synchronize()
        if not c_lo <= p.chunk < c_hi:
            assert np.all(lc.bank.count.cpu().numpy() <= wl.M)
            return
        if stage == "before":
            held[x.layer] = (GpuBank.read(lc.bank), a["ring_before"])
            return
        before, ring_before = held.pop(x.layer)
        N = a["N"]
        d0 = p.departed[0]
        candK = _check_window_advance(ring_before, a["candK"], a["candV"], ((d0 - 1) % wl.window_frames) * F,
                                      N, F, d0)
        candV = a["candV"].float().cpu().numpy().astype(np.float64)
        ctok = a["candT"].cpu().numpy()
        after = GpuBank.read(lc.bank)
        assert np.all(after.count <= wl.M) and lc.bank.K.shape[1] == wl.M
        assert int(lc.out.status.cpu()[0]) == 0
        D, s, o = lc.outputs(N)
        rep = replay_update(before, after, candK, candV, ctok, D.cpu().numpy(), s.cpu().numpy(), o.cpu().numpy(),
                            lc.out.t_cross.cpu().numpy(), lc.out.rho_proj.cpu().numpy(), lc.out.k_star.cpu().numpy(),
                            lc.out.n_mandatory.cpu().numpy(), lc.out.n_evicted.cpu().numpy(), prm, list(range(H)),
                            rho_before=rho_prev[x.layer])
        rho_prev[x.layer] = rep.rho_after
        kstars[x.layer].append(rep.kstar)
        gc.banner(f"  rollout layer {x.layer} chunk {p.chunk}: N={N} k*={rep.kstar} evicted/head={rep.evicted[:3]} "
                  f"count={int(after.count.min())}..{int(after.count.max())}")

    gc.banner(f"rollout: layers 0 and 29, chunks {c_lo}..{c_hi - 1} of {wl.chunks}, stage replay at every update")
    r = Rollout(wl, layers, seed=0, diagnostics=True, source="host")
    worst = (0.0, 0.0)
    for c in range(c_hi):
        outs, p = r.step(hook)
        if c < c_lo:
            continue
        admitted = any(len(kstars[l]) and kstars[l][-1] > 0 and len(p.departed) for l in layers)
        if not (admitted or c % 10 == 0):
            continue
        torch.cuda.synchronize()
        rows = np.random.default_rng(c).choice(wl.Lq, 256, replace=False)
        for x, O in zip(r.L, outs):
            bank = GpuBank.read(x.cache.bank)
            On = O.cpu().numpy()
            errs = []
            for h in range(H):
                parts = []
                if c > 0:
                    parts.append(x.recent[0])
                pk = [a[0][h] for a in parts] + [bank.K[h, :bank.count[h]]] + \
                     [x.recent[f][0][h] for f in list(p.window) + list(p.frames)]
                pv = [a[1][h] for a in parts] + [bank.V[h, :bank.count[h]]] + \
                     [x.recent[f][1][h] for f in list(p.window) + list(p.frames)]
                Q = np.concatenate([x.recent[f][2][h] for f in p.frames])[rows]
                ref = oracle_attention(np.asarray(Q, np.float64), np.concatenate(pk).astype(np.float64),
                                       np.concatenate(pv).astype(np.float64), block=64)
                errs.append(np.abs(On[h][rows] - ref))
            e = np.concatenate([v.reshape(-1) for v in errs])
            assert e.max() <= 2e-2 and e.mean() <= 2e-3, (c, x.layer, e.max(), e.mean())
            worst = (max(worst[0], float(e.max())), max(worst[1], float(e.mean())))
        gc.banner(f"  rollout chunk {c}: attention checked (worst so far max-abs {worst[0]:.2e} "
                  f"mean-abs {worst[1]:.2e})")
    for l in layers:
        if part == 0:
            assert kstars[l][0] == 2 * F, "the first bank update admits every departed row into the empty bank"
        gc.banner(f"rollout layer {l}: k* per update of chunks {c_lo}..{c_hi - 1}: {kstars[l]}")


@pytest.mark.timeout(600)
def test_rollout_deterministic_and_resumable():
    """Device-drawn frames, layers 0 and 29, 16 chunks: a second run is
    bitwise identical, and a run resumed from a checkpoint at chunk 10
    (banks, window rings, sink, previous chunk, stream positions) ends in the
    same state with the same outputs."""
    import torch
    from kv_cache_compression_head_amd.rollout import Rollout
    wl = WORKLOADS["rollout"]
    layers, chunks, resume_at = [0, wl.layers - 1], 16, 10

    def run(r, n):
        outs = None
        for _ in range(n):
            outs, _ = r.step()
        torch.cuda.synchronize()
        return outs

    gc.banner("rollout determinism: straight run")
    r1 = Rollout(wl, layers, seed=0, source="device")
    run(r1, resume_at)
    snap = r1.state()
    outs1 = run(r1, chunks - resume_at)
    gc.banner("rollout determinism: second run")
    r2 = Rollout(wl, layers, seed=0, source="device")
    outs2 = run(r2, chunks)
    gc.banner("rollout determinism: resumed run")
    r3 = Rollout(wl, layers, seed=0, source="device")
    r3.load_state(snap)
    outs3 = run(r3, chunks - resume_at)
    for other, oo in ((r2, outs2), (r3, outs3)):
        for a, b in zip(r1.L, other.L):
            for x, y in zip((a.cache.bank.K, a.cache.bank.V, a.cache.bank.tok, a.cache.bank.rho0, a.cache.bank.rho,
                             a.cache.bank.count, a.ring_k, a.ring_v),
                            (b.cache.bank.K, b.cache.bank.V, b.cache.bank.tok, b.cache.bank.rho0, b.cache.bank.rho,
                             b.cache.bank.count, b.ring_k, b.ring_v)):
                assert torch.equal(x, y), "state differs from the straight run"
        for x, y in zip(outs1, oo):
            assert torch.equal(x, y), "attention output differs from the straight run"
    for x in r1.L:
        assert x.cache.bank.K.shape[1] == wl.M and int(x.cache.bank.count.max()) <= wl.M


@pytest.mark.timeout(600)
def test_rollout_fill_below_capacity_layer0():
    """Streaming rollout of layer 0 under the fill-below-capacity variant
    (KVB_POL_FILL_BELOW_CAP) for 14 chunks: the bank fills to M and then
    admits and evicts at every update, so the crossing scan, the eviction and
    the density fix-ups run on streaming inputs.  Every update is replayed
    stage by stage against the oracle under the same policy; attention rows
    are checked at the last chunk."""
    import dataclasses
    import torch
    import kv_cache_compression_head_amd as kb
    from kv_cache_compression_head_amd.rollout import Rollout
    from oracle.attention import attention as oracle_attention
    wl = WORKLOADS["rollout"]
    prm = dataclasses.replace(od.Params(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p),
                              fill_below_capacity=True)
    F, H = wl.F, wl.H
    held, rho_prev, log = {}, [None], []

    def hook(stage, x, p, lc, a):
        torch.cuda.synchronize()
        if stage == "before":
            held[x.layer] = (GpuBank.read(lc.bank), a["ring_before"])
            return
        before, ring_before = held.pop(x.layer)
        N = a["N"]
        d0 = p.departed[0]
        candK = _check_window_advance(ring_before, a["candK"], a["candV"], ((d0 - 1) % wl.window_frames) * F,
                                      N, F, d0)
        candV = a["candV"].float().cpu().numpy().astype(np.float64)
        after = GpuBank.read(lc.bank)
        assert np.all(after.count <= wl.M)
        assert int(lc.out.status.cpu()[0]) == 0
        D, s, o = lc.outputs(N)
        rep = replay_update(before, after, candK, candV, a["candT"].cpu().numpy(), D.cpu().numpy(), s.cpu().numpy(),
                            o.cpu().numpy(), lc.out.t_cross.cpu().numpy(), lc.out.rho_proj.cpu().numpy(),
                            lc.out.k_star.cpu().numpy(), lc.out.n_mandatory.cpu().numpy(),
                            lc.out.n_evicted.cpu().numpy(), prm, list(range(H)), workers=1,
                            rho_before=rho_prev[0])
        rho_prev[0] = rep.rho_after
        log.append((p.chunk, rep.kstar, int(np.sum(rep.evicted)), int(after.count.min())))
        gc.banner(f"  fill rollout chunk {p.chunk}: N={N} k*={rep.kstar} evicted={int(np.sum(rep.evicted))} "
                  f"count={int(after.count.min())}..{int(after.count.max())}")

    r = Rollout(wl, [0], seed=0, diagnostics=True, source="host", policy=kb.KVB_POL_FILL_BELOW_CAP)
    outs = p = None
    for c in range(14):
        outs, p = r.step(hook)
    torch.cuda.synchronize()
    # the bank reached capacity, then kept admitting with evictions
    assert any(cnt == wl.M for _, _, _, cnt in log)
    steady = [(k, e) for (c, k, e, cnt) in log if cnt == wl.M]
    assert len(steady) >= 3 and any(k > 0 and e > 0 for k, e in steady)
    x = r.L[0]
    bank = GpuBank.read(x.cache.bank)
    rows = np.random.default_rng(5).choice(wl.Lq, 256, replace=False)
    On = outs[0].cpu().numpy()
    errs = []
    for h in range(H):
        pk = [x.recent[0][0][h], bank.K[h, :bank.count[h]]] + [x.recent[f][0][h] for f in list(p.window) + list(p.frames)]
        pv = [x.recent[0][1][h], bank.V[h, :bank.count[h]]] + [x.recent[f][1][h] for f in list(p.window) + list(p.frames)]
        Q = np.concatenate([x.recent[f][2][h] for f in p.frames])[rows]
        ref = oracle_attention(np.asarray(Q, np.float64), np.concatenate(pk).astype(np.float64),
                               np.concatenate(pv).astype(np.float64), block=64)
        errs.append(np.abs(On[h][rows] - ref).reshape(-1))
    e = np.concatenate(errs)
    assert e.max() <= 2e-2 and e.mean() <= 2e-3, (e.max(), e.mean())
