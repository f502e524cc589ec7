"""GPU parity of the DensityKV path (scoring, admission/eviction, attention)
through the C ABI against the fp64 oracle, with stage replay."""
import dataclasses
import math

import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, Workload, frame_tokens, round_bf16
from oracle import density as od

import gpu_common as gc
from _parity import GpuBank

pytestmark = pytest.mark.gpu


def _prm(wl, **kw):
    base = dict(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    base.update(kw)
    return od.Params(**base)


def _stream(wl, prm, seed=0, attn=True, max_abs=1e-4, mean_abs=1e-5, win_start=0):
    import torch
    gc.banner(f"density stream {wl.name} dtype={wl.dtype} M={prm.M} tau={prm.tau} p={prm.p} seed={seed}")
    gen = LayerGen(wl, seed, 0)
    lc = gc.layer_for(wl, prm)
    heads = list(range(wl.H))
    reps = []
    for fr in wl.bank_updates:
        r = gc.run_update(lc, gen, wl, prm, fr, heads)
        gc.banner(f"  update {fr}: k*={r.kstar} evicted/head={r.evicted[:4]} order near-ties={r.order_near_ties} "
                  f"crossing near-ties={r.crossing_near_ties}")
        reps.append(r)
    if attn:
        ai = gc.attn_inputs(gen, wl)
        kdt = gc.kv_dtype(wl)
        lay = gc.layout_for(ai, kdt, win_start=win_start)
        lc.update(None, None, None, None, None, lay)      # N = 0: segment table only
        Q = gc.dev(ai.Q, kdt)
        O = lc.attention(Q, out_f32=True)
        torch.cuda.synchronize()
        bank = GpuBank.read(lc.bank)
        mx, mn = gc.check_attention(O.cpu().numpy(), ai, bank, heads, max_abs, mean_abs)
        gc.banner(f"  attention max-abs {mx:.2e} mean-abs {mn:.2e}")
    return reps, lc


def test_tiny_f32_default():
    wl = WORKLOADS["tiny"]
    reps, _ = _stream(wl, _prm(wl))
    assert [r.kstar for r in reps][0] == 48


def test_tiny_bf16():
    wl = dataclasses.replace(WORKLOADS["tiny"], dtype="bf16", name="tiny-bf16")
    _stream(wl, _prm(wl), max_abs=2e-2, mean_abs=2e-3)


def test_tiny_fifo_p0_tau_inf():
    wl = WORKLOADS["tiny"]
    prm = _prm(wl, tau=math.inf, p=0.0)
    _, lc = _stream(wl, prm, attn=False)
    bank = GpuBank.read(lc.bank)
    last = wl.bank_updates[-1][1] * wl.F
    for h in range(wl.H):
        assert sorted(bank.tok[h, :bank.count[h]].tolist()) == list(range(last - 64, last))


def test_tiny_full_admission():
    wl = WORKLOADS["tiny"]
    prm = _prm(wl, M=144, tau=math.inf)
    reps, lc = _stream(wl, prm)
    assert all(r.kstar == 48 for r in reps)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p,tau", [(1.0, 1.3), (4.0, 1.3), (3.0, 1.2), (2.0, 1.05)])
def test_tiny_phi_modes(p, tau, dtype):
    wl = dataclasses.replace(WORKLOADS["tiny"], dtype=dtype, name=f"tiny-{dtype}")
    _stream(wl, _prm(wl, p=p, tau=tau), attn=False)


def test_duplicate_rejected_on_gpu():
    """Far-apart bank keys plus a candidate duplicating one: the duplicate is
    ordered last and is the only candidate rejected."""
    import torch
    import kv_cache_compression_head_amd as kb
    d, n = 64, 60
    wl = dataclasses.replace(WORKLOADS["tiny"], H=1, M=100)
    prm = od.Params(M=100, tau=2.0)
    lc = gc.layer_for(wl, prm)
    K = (np.eye(d)[:n] * 200.0).astype(np.float32)[None]
    V = np.random.default_rng(0).normal(size=(1, n, d)).astype(np.float32)
    gc.run_update(lc, None, wl, prm, (0, 0), [0], candK=K, candV=V, ctok=np.arange(n, dtype=np.int32))
    cK = np.concatenate([np.eye(d)[n:n + 3] * 200.0, K[0, 5:6]]).astype(np.float32)[None]
    cV = np.ones((1, 4, d), np.float32)
    rep = gc.run_update(lc, None, wl, prm, (0, 0), [0], candK=cK, candV=cV,
                        ctok=np.array([100, 101, 102, 103], np.int32))
    assert rep.kstar == 3
    bank = GpuBank.read(lc.bank)
    toks = set(bank.tok[0, :bank.count[0]].tolist())
    assert 103 not in toks and {100, 101, 102, 5} <= toks


def test_duplicate_rejected_on_gpu_bf16():
    """The same invariant through the bf16 direct form (sigma^2 a power of
    two): the duplicate's softened distance is exactly eps."""
    wl = dataclasses.replace(WORKLOADS["tiny"], H=1, M=100, dtype="bf16", name="tiny-bf16")
    prm = od.Params(M=100, tau=2.0)
    lc = gc.layer_for(wl, prm)
    d, n = 64, 60
    K = (np.eye(d)[:n] * 200.0).astype(np.float32)[None]
    # values as stored in bf16, so that the pairing check compares like with like
    V = round_bf16(np.random.default_rng(0).normal(size=(1, n, d)).astype(np.float32))
    gc.run_update(lc, None, wl, prm, (0, 0), [0], candK=K, candV=V, ctok=np.arange(n, dtype=np.int32))
    cK = np.concatenate([np.eye(d)[n:n + 3] * 200.0, K[0, 5:6]]).astype(np.float32)[None]
    cV = np.ones((1, 4, d), np.float32)
    rep = gc.run_update(lc, None, wl, prm, (0, 0), [0], candK=cK, candV=cV,
                        ctok=np.array([100, 101, 102, 103], np.int32))
    assert rep.kstar == 3
    bank = GpuBank.read(lc.bank)
    toks = set(bank.tok[0, :bank.count[0]].tolist())
    assert 103 not in toks and {100, 101, 102, 5} <= toks


MID = Workload(name="mid", H=4, d=128, width=52, height=30, dtype="bf16", M=3120, tau=2.0,
               bank_updates=((1, 3), (3, 7)), window=(7, 9), chunk=(9, 12))


def test_mid_bf16_default():
    _stream(MID, _prm(MID), max_abs=2e-2, mean_abs=2e-3, win_start=1000)


def test_mid_bf16_tight_tau():
    _stream(MID, _prm(MID, tau=1.02), attn=False, seed=1)


@pytest.mark.parametrize("sigma,eps", [(7.0, 1.0), (8.0, 1e-3)])
def test_mid_bf16_general_form(sigma, eps):
    """bf16 keys where the Soft-Riesz argument is formed with a multiply-add
    (sigma^2 not a power of two, or a small eps that needs the clamp)."""
    _stream(MID, _prm(MID, sigma=sigma, eps=eps), max_abs=2e-2, mean_abs=2e-3, seed=2)


def test_mid_f32_head_prefix():
    """fp32 keys over many 256-row blocks with a different admitted count per
    head (per-head prefix, early crossings): the symmetric admitted Gram's
    column sums and their ordered combine on the fp32 path."""
    wl = dataclasses.replace(MID, dtype="f32", name="mid-f32")
    _stream(wl, _prm(wl, tau=1.05, prefix="head"), attn=False, seed=5)


def test_mid_bf16_d64():
    """Head dimension 64 in bf16 over many 256-row blocks: the d = 64 Gram,
    scan and symmetric admitted Gram, and the d = 64 attention kernel on the
    layer's segment table."""
    wl = dataclasses.replace(MID, d=64, name="mid-d64")
    _stream(wl, _prm(wl, tau=1.1), max_abs=2e-2, mean_abs=2e-3, seed=6)


def test_empty_update_and_zero_candidates():
    import torch
    import kv_cache_compression_head_amd as kb
    wl = WORKLOADS["tiny"]
    prm = _prm(wl)
    lc = gc.layer_for(wl, prm)
    lc.update(None, None, None, None, None, kb.KVLayout())
    torch.cuda.synchronize()
    assert int(lc.bank.count.sum().cpu()) == 0
    assert lc.out.nseg.cpu().tolist() == [0, 0]


# DensityKV policy variants (the page's appendix E ablations), each checked
# stage by stage against the oracle's rules for that variant
POLICY_CASES = {
    "source": dict(order="source"),
    "refresh": dict(baseline="refresh"),
    "densest": dict(eviction="densest"),
    "oldest": dict(eviction="oldest"),
    "head": dict(prefix="head"),
    "fill": dict(fill_below_capacity=True),
    "all": dict(order="source", baseline="refresh", eviction="oldest", prefix="head", fill_below_capacity=True),
    "densest-fill-head": dict(eviction="densest", fill_below_capacity=True, prefix="head"),
}


@pytest.mark.parametrize("name", list(POLICY_CASES))
def test_tiny_policy_variants(name):
    wl = WORKLOADS["tiny"]
    for tau in (1.3, 2.0):
        _stream(wl, _prm(wl, tau=tau, **POLICY_CASES[name]), attn=False, seed=4)


@pytest.mark.parametrize("name", ["source", "refresh", "densest", "oldest", "head", "fill", "all"])
def test_mid_bf16_policy_variants(name):
    _stream(MID, _prm(MID, tau=1.05, **POLICY_CASES[name]), attn=False, seed=3)


def test_tiny_source_order_oldest_is_a_window():
    """tau = inf, source order, oldest-first completion, p = 2: the bank is
    the M most recent tokens after every update (a sliding window for any
    interaction)."""
    wl = WORKLOADS["tiny"]
    prm = _prm(wl, tau=math.inf, order="source", eviction="oldest")
    _, lc = _stream(wl, prm, attn=False)
    bank = GpuBank.read(lc.bank)
    last = wl.bank_updates[-1][1] * wl.F
    for h in range(wl.H):
        assert sorted(bank.tok[h, :bank.count[h]].tolist()) == list(range(last - 64, last))


def _replace_all_pair(wl, prm, seed=0):
    """The same stream through two layers: one asks for the per-state
    diagnostics (crossing scan), the other does not, so that its updates with
    min(N, M) = M take the path without the scan.  Returns both layers."""
    import torch
    import kv_cache_compression_head_amd as kb
    gen = LayerGen(wl, seed, 0)
    a = gc.layer_for(wl, prm, diagnostics=True)
    b = gc.layer_for(wl, prm, diagnostics=False)
    kdt = gc.kv_dtype(wl)
    for (t0, t1) in wl.bank_updates:
        cK, cV = gc.dev(gen.keys_all(range(t0, t1)), kdt), gc.dev(gen.values_all(range(t0, t1)), kdt)
        ct = gc.dev_i32(frame_tokens(wl, t0, t1))
        for lc in (a, b):
            lc.out.status.zero_()
            D, s, o = lc.score(cK, ct, kb.KVLayout())
            lc.update(cK, cV, ct, D, o, kb.KVLayout())
        torch.cuda.synchronize()
        assert int(a.out.status.cpu()[0]) == 0 and int(b.out.status.cpu()[0]) == 0
        N = cK.shape[1]
        if N >= prm.M:
            assert b.out.n_mandatory.cpu().tolist() == [-1] * wl.H
        for x, y in ((a.bank.K, b.bank.K), (a.bank.V, b.bank.V), (a.bank.tok, b.bank.tok),
                     (a.bank.rho0, b.bank.rho0), (a.bank.rho, b.bank.rho), (a.bank.count, b.bank.count),
                     (a.out.k_star, b.out.k_star), (a.out.n_evicted, b.out.n_evicted)):
            assert torch.equal(x, y), "the path without the crossing scan differs"
    return a, b


@pytest.mark.parametrize("tau", [2.0, 1.05])
def test_tiny_whole_bank_replaced_without_scan(tau):
    """Blocks of 48 candidates into a bank of 40: k* = M and every state
    leaves, whatever crossed; the path without the crossing scan gives the
    same bank bit for bit, and the diagnostics path replays against the
    oracle."""
    wl = WORKLOADS["tiny"]
    prm = _prm(wl, M=40, tau=tau)
    _stream(wl, prm, attn=False)
    _replace_all_pair(wl, prm)
