"""GPU parity of the Forcing-KV path (segment similarity, BottomK, static /
dynamic segment tables, ragged chunk attention) against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, frame_tokens, head_labels
from oracle import forcing as of
from oracle.attention import attention as oracle_attention

import gpu_common as gc
from _parity import check_order

pytestmark = pytest.mark.gpu


def _run(wl, seed=0, rows=None, per_frame=False):
    import torch
    import kv_cache_compression_head_amd as kb
    gc.banner(f"forcing {wl.name} seg_len={wl.seg_len} r={wl.retention} seed={seed} per_frame={per_frame}")
    gen = LayerGen(wl, seed, 0)
    labels = head_labels(wl, seed)
    F, H, d = wl.F, wl.H, wl.d
    h0, h1 = wl.history
    c0, c1 = wl.chunk
    hist_f = list(range(h0, h1))
    ch_f = list(range(c0, c1))
    histK = gen.keys_all(hist_f, hist_f)
    histV = gen.values_all(hist_f)
    sinkK, sinkV = gen.keys_all([0], [0]), gen.values_all([0])
    chK, chV = gen.keys_all(ch_f, ch_f), gen.values_all(ch_f)
    Q = gen.queries_all(ch_f, ch_f)
    T = len(hist_f)
    items = T * (F // wl.seg_len)
    nseg = F // wl.seg_len
    keep = T * of.keep_count(wl.retention, nseg) if per_frame else of.keep_count(wl.retention, items)
    seg_cap = min(256, 2 + keep + 1)
    from kvsynth import Workload
    prm_M = 0
    import kv_cache_compression_head_amd.pipeline as pl
    desc = kb.LayerDesc(H=H, d=d, M=prm_M, dtype=kb.KVB_BF16, frame_tokens=F, labels=labels.tolist(),
                        seg_len=wl.seg_len, retention=wl.retention,
                        policy=kb.KVB_POL_FRAME_BOTTOMK if per_frame else 0)
    lc = pl.LayerCache(desc, seg_cap=seg_cap)
    kdt = torch.bfloat16
    N = T * F
    hk, hv = gc.dev(histK, kdt), gc.dev(histV, kdt)
    tok = gc.dev_i32(frame_tokens(wl, h0, h1))
    lay = kb.KVLayout(sink_k=gc.dev(sinkK, kdt), sink_v=gc.dev(sinkV, kdt),
                      chunk_k=gc.dev(chK, kdt), chunk_v=gc.dev(chV, kdt))
    D, s, o = lc.score(hk, tok, lay)
    lc.update(hk, hv, tok, D, o, lay)
    O = lc.attention(gc.dev(Q, kdt), out_f32=True)
    torch.cuda.synchronize()
    assert int(lc.out.status.cpu()[0]) == 0
    dyn = [h for h in range(H) if labels[h] == 2]
    stat = [h for h in range(H) if labels[h] == 1]
    # segment scores (shared by the dynamic heads)
    ref = of.segment_scores(histK[dyn], chK[dyn][:, :F], F, wl.seg_len)
    s_np, o_np = s.cpu().numpy(), o.cpu().numpy()
    for h in dyn:
        np.testing.assert_allclose(s_np[h, :items], ref, rtol=2e-5, atol=2e-6)
        if not per_frame:
            check_order(o_np[h, :items], ref, np.arange(items))
    kept = np.sort(o_np[dyn[0], :keep])
    if per_frame:
        # the per-frame selection, decided on the GPU's own scores (fp32),
        # is exactly the oracle's rule applied to them
        for h in dyn:
            assert np.sort(o_np[h, :keep]).tolist() == of.bottomk_per_frame(s_np[h, :items], wl.retention,
                                                                             nseg).tolist()
    # segment tables
    segs = lc.segments()
    esz = 2
    base_k = hk.data_ptr()
    for h in range(H):
        sg = segs[h]
        assert sg[0][2] == F and sg[-1][2] == wl.Lq
        mid = sg[1:-1]
        if labels[h] == 1:
            assert len(mid) == 1 and mid[0][2] == F
            assert mid[0][0] == base_k + (h * N + (T - 1) * F) * d * esz
        else:
            got_rows = []
            for (kp, vp, ln) in mid:
                r0 = (kp - base_k) // (d * esz) - h * N
                got_rows.extend(range(r0, r0 + ln))
            assert got_rows == of.kept_token_rows(kept, F, wl.seg_len).tolist()
    # attention rows (sampled at large sizes)
    O_np = O.cpu().numpy()
    rr = np.arange(wl.Lq) if rows is None else rows
    errs = []
    for h in range(H):
        if labels[h] == 1:
            sel = of.static_rows(T, F)
        else:
            sel = of.kept_token_rows(kept, F, wl.seg_len)
        K = np.concatenate([sinkK[h], histK[h][sel], chK[h]]).astype(np.float64)
        V = np.concatenate([sinkV[h], histV[h][sel], chV[h]]).astype(np.float64)
        refo = oracle_attention(Q[h][rr].astype(np.float64), K, V)
        errs.append(np.abs(O_np[h][rr] - refo))
    e = np.concatenate([x.reshape(-1) for x in errs])
    assert e.max() <= 2e-2 and e.mean() <= 2e-3, (e.max(), e.mean())
    gc.banner(f"forcing {wl.name}: kept items {kept.tolist()[:12]} attention max-abs {e.max():.2e} mean-abs {e.mean():.2e}")
    return kept


def test_forcing_480p_full():
    wl = WORKLOADS["fkv480p"]
    kept = _run(wl, rows=np.random.default_rng(0).choice(wl.Lq, 512, replace=False))
    assert kept.shape[0] == 8


def test_forcing_six_segments_per_frame():
    wl = dataclasses.replace(WORKLOADS["fkv480p"], seg_len=260, retention=0.33, name="fkv-n6")
    _run(wl, rows=np.arange(0, 4680, 37))


def test_forcing_small_shapes():
    wl = dataclasses.replace(WORKLOADS["fkv480p"], width=8, height=4, H=4, n_static=2, seg_len=8, retention=0.5,
                             history=(1, 6), chunk=(6, 9), name="fkv-small")
    _run(wl)


def test_forcing_many_dynamic_heads():
    """Ten dynamic heads: more than the row-group cosine kernel holds, so
    the segment similarity takes the per-token kernel."""
    wl = dataclasses.replace(WORKLOADS["fkv480p"], width=8, height=4, H=12, n_static=2, seg_len=8, retention=0.5,
                             history=(1, 6), chunk=(6, 9), name="fkv-10dyn")
    _run(wl)


@pytest.mark.parametrize("r", [0.3, 0.33, 0.5])
def test_forcing_per_frame_bottomk(r):
    """Section 3.4 as printed: six segments per frame, floor(r 6) kept in
    every frame (one at the appendix's r = 0.3 and the YAML's 0.33)."""
    wl = dataclasses.replace(WORKLOADS["fkv480p"], seg_len=260, retention=r, name=f"fkv-frame-{r}")
    kept = _run(wl, rows=np.arange(0, wl.Lq, 37), per_frame=True)
    T = wl.history[1] - wl.history[0]
    assert len(kept) == T * int(np.floor(r * 6))


def test_forcing_order_shared_across_layers():
    """Section 3.4's proxy: segment scores computed once (here on layer 0)
    and the BottomK indices reused by another layer. kvbank_update takes the
    order as an input, so layer 1's segment table must cover exactly the rows
    that layer 0's scores select, inside layer 1's own history buffer."""
    import torch
    import kv_cache_compression_head_amd as kb
    import kv_cache_compression_head_amd.pipeline as pl
    wl = dataclasses.replace(WORKLOADS["fkv480p"], width=8, height=4, H=4, n_static=2, seg_len=8, retention=0.5,
                             history=(1, 6), chunk=(6, 9), name="fkv-small")
    seed = 3
    gc.banner(f"forcing order shared across layers {wl.name} seed={seed}")
    labels = head_labels(wl, seed)
    F, H, d = wl.F, wl.H, wl.d
    h0, h1 = wl.history
    c0, c1 = wl.chunk
    hist_f, ch_f = list(range(h0, h1)), list(range(c0, c1))
    T = len(hist_f)
    items = T * (F // wl.seg_len)
    keep = of.keep_count(wl.retention, items)
    kdt = torch.bfloat16
    tok = gc.dev_i32(frame_tokens(wl, h0, h1))
    dyn = [h for h in range(H) if labels[h] == 2]
    caches, bufs, scores = [], [], []
    for layer in (0, 1):
        gen = LayerGen(wl, seed, layer)
        histK, histV = gen.keys_all(hist_f, hist_f), gen.values_all(hist_f)
        chK, chV = gen.keys_all(ch_f, ch_f), gen.values_all(ch_f)
        lay = kb.KVLayout(sink_k=gc.dev(gen.keys_all([0], [0]), kdt), sink_v=gc.dev(gen.values_all([0]), kdt),
                          chunk_k=gc.dev(chK, kdt), chunk_v=gc.dev(chV, kdt))
        desc = kb.LayerDesc(H=H, d=d, M=0, dtype=kb.KVB_BF16, frame_tokens=F, labels=labels.tolist(),
                            seg_len=wl.seg_len, retention=wl.retention)
        caches.append(pl.LayerCache(desc, seg_cap=min(256, keep + 3)))
        bufs.append((gc.dev(histK, kdt), gc.dev(histV, kdt), lay))
        scores.append(of.segment_scores(histK[dyn], chK[dyn][:, :F], F, wl.seg_len))
    hk0, hv0, lay0 = bufs[0]
    D0, s0, o0 = caches[0].score(hk0, tok, lay0)
    hk1, hv1, lay1 = bufs[1]
    caches[1].update(hk1, hv1, tok, D0, o0, lay1)
    torch.cuda.synchronize()
    assert int(caches[1].out.status.cpu()[0]) == 0
    kept0 = of.bottomk(scores[0], wl.retention)
    rows = of.kept_token_rows(kept0, F, wl.seg_len).tolist()
    base_k = hk1.data_ptr()
    segs = caches[1].segments()
    for h in dyn:
        got = []
        for (kp, vp, ln) in segs[h][1:-1]:
            r0 = (kp - base_k) // (d * 2) - h * T * F
            got.extend(range(r0, r0 + ln))
        assert got == rows
    # layer 1 scored on its own would keep another set: the shared indices
    # really come from layer 0
    kept1 = of.bottomk(scores[1], wl.retention)
    assert kept1.tolist() != kept0.tolist()
    gc.banner(f"shared order: layer-0 kept {kept0.tolist()} layer-1 own {kept1.tolist()}")


@pytest.mark.parametrize("case", ["fkv480p", "fkv-10dyn"])
def test_score_layers_matches_per_layer(case):
    """kvbank_score_layers on three layers (each with its own seeded keys)
    gives, bit for bit, kvbank_score's segment scores and BottomK orders of
    each layer, leaves static heads' rows untouched, and matches the oracle's
    segment scores.  fkv-10dyn takes the per-token cosine kernel."""
    import torch
    import kv_cache_compression_head_amd as kb
    if case == "fkv480p":
        wl = WORKLOADS["fkv480p"]
    else:
        wl = dataclasses.replace(WORKLOADS["fkv480p"], width=8, height=4, H=12, n_static=2, seg_len=8,
                                 retention=0.5, history=(1, 6), chunk=(6, 9), name="fkv-10dyn")
    labels = head_labels(wl, 0)
    desc = kb.LayerDesc(H=wl.H, d=wl.d, M=0, dtype=kb.KVB_BF16, frame_tokens=wl.F, labels=labels.tolist(),
                        seg_len=wl.seg_len, retention=wl.retention)
    h0, h1 = wl.history
    c0, c1 = wl.chunk
    hist_f, ch_f = list(range(h0, h1)), list(range(c0, c1))
    nl = 3
    K, C = [], []
    for layer in range(nl):
        gen = LayerGen(wl, 0, layer)
        K.append(gen.keys_all(hist_f, hist_f))
        C.append(gen.keys_all(ch_f, ch_f))
    kdt = torch.bfloat16
    Kd, Cd = gc.dev(np.stack(K), kdt), gc.dev(np.stack(C), kdt)
    N = Kd.shape[2]
    items = N // wl.seg_len
    gc.banner(f"score_layers {case}: {nl} layers, N={N}, items={items}")
    sc = torch.full((nl, wl.H, N), -7.0, dtype=torch.float32, device="cuda")
    od = torch.full((nl, wl.H, N), -1, dtype=torch.int32, device="cuda")
    kb.kvbank_score_layers(desc, Kd, Cd, sc, od)
    torch.cuda.synchronize()
    ws = torch.empty(kb.kvbank_workspace_size(desc, N), dtype=torch.uint8, device="cuda")
    dyn = [h for h in range(wl.H) if labels[h] == 2]
    stat = [h for h in range(wl.H) if labels[h] == 1]
    for layer in range(nl):
        s1 = torch.full((wl.H, N), -7.0, dtype=torch.float32, device="cuda")
        o1 = torch.full((wl.H, N), -1, dtype=torch.int32, device="cuda")
        kb.kvbank_score(desc, None, Kd[layer], None, N, kb.KVLayout(chunk_k=Cd[layer]), None, s1, o1, ws)
        torch.cuda.synchronize()
        for h in dyn:
            assert torch.equal(sc[layer, h, :items], s1[h, :items]), (layer, h)
            assert torch.equal(od[layer, h, :items], o1[h, :items]), (layer, h)
        for h in stat:
            assert bool((sc[layer, h] == -7.0).all()) and bool((od[layer, h] == -1).all()), (layer, h)
        ref = of.segment_scores(K[layer][dyn], C[layer][dyn][:, :wl.F], wl.F, wl.seg_len)
        np.testing.assert_allclose(sc[layer, dyn[0], :items].cpu().numpy(), ref, rtol=2e-5, atol=2e-6)
