"""GPU parity of sequential within-block admission (KVB_POL_SEQUENTIAL;
DensityKV paper summary, appendix E, within-block competition) against the
fp64 oracle (oracle/sequential.py), replayed on the GPU's validated order and
its bank before each block: the final per-head token sets exactly, every
K/V row paired with its token, baselines and densities in fp64, and the
admission and eviction counts."""
import dataclasses

import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, Workload, frame_tokens
from oracle import density as od
from oracle import sequential as oseq

import gpu_common as gc
from _parity import GpuBank, check_order

pytestmark = pytest.mark.gpu


def _prm(wl, **kw):
    base = dict(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)
    base.update(kw)
    return od.Params(**base)


def _seq_stream(wl, prm, seed=0, attn=False):
    import torch
    import kv_cache_compression_head_amd as kb
    gc.banner(f"sequential {wl.name} dtype={wl.dtype} M={prm.M} tau={prm.tau} policy={prm} seed={seed}")
    gen = LayerGen(wl, seed, 0)
    lc = gc.layer_for(wl, prm, extra_policy=kb.KVB_POL_SEQUENTIAL)
    kdt = gc.kv_dtype(wl)
    H = wl.H
    stats = []
    for (t0, t1) in wl.bank_updates:
        candK, candV = gen.keys_all(range(t0, t1)), gen.values_all(range(t0, t1))
        ctok = frame_tokens(wl, t0, t1)
        before = GpuBank.read(lc.bank)
        cK, cV, ct = gc.dev(candK, kdt), gc.dev(candV, kdt), gc.dev_i32(ctok)
        lc.out.status.zero_()
        D, s, o = lc.score(cK, ct, kb.KVLayout())
        lc.update(cK, cV, ct, D, o, kb.KVLayout())
        torch.cuda.synchronize()
        assert int(lc.out.status.cpu()[0]) == 0, f"status {int(lc.out.status.cpu()[0]):#x}"
        after = GpuBank.read(lc.bank)
        o_np = o.cpu().numpy().astype(np.int64)
        banks = [before.head(h) for h in range(H)]
        K64, V64 = candK.astype(np.float64), candV.astype(np.float64)
        for h in range(H):
            _, delta = od.disturbance(banks[h].K, K64[h], prm)
            if prm.order == "source":
                assert o_np[h].tolist() == np.argsort(ctok, kind="stable").tolist()
            else:
                check_order(o_np[h], delta, ctok.astype(np.int64))
        new, info = oseq.update_layer_sequential(banks, K64, V64, ctok, prm, order=[o_np[h] for h in range(H)])
        ks = lc.out.k_star.cpu().numpy()
        nev = lc.out.n_evicted.cpu().numpy()
        for h in range(H):
            kgpu = int(ks[h] if prm.prefix == "head" else ks[0])
            assert kgpu == len(info.admitted_h[h]), f"head {h}: admitted {kgpu} != oracle {len(info.admitted_h[h])}"
            assert int(nev[h]) == len(info.evicted_h[h]), f"head {h}: evictions"
            n = int(after.count[h])
            nb = new[h]
            assert n == nb.n, f"head {h}: count {n} != oracle {nb.n}"
            gtok = after.tok[h, :n]
            assert sorted(gtok.tolist()) == sorted(nb.tok.tolist()), f"head {h}: bank sets differ"
            pos = {int(t): i for i, t in enumerate(nb.tok.tolist())}
            idx = np.array([pos[int(t)] for t in gtok])
            np.testing.assert_array_equal(after.K[h, :n], nb.K[idx])
            np.testing.assert_array_equal(after.V[h, :n], nb.V[idx])
            np.testing.assert_allclose(after.rho0[h, :n], nb.rho0[idx], rtol=1e-4, atol=1e-6)
            np.testing.assert_allclose(after.rho[h, :n], od.density(nb.K, prm)[idx], rtol=1e-4, atol=1e-6)
        stats.append((int(ks[0]), int(nev[0]), int(after.count[0])))
    gc.banner(f"  (admitted, evicted, count) per block on head 0: {stats}")
    if attn:
        ai = gc.attn_inputs(gen, wl)
        lay = gc.layout_for(ai, kdt)
        lc.update(None, None, None, None, None, lay)
        O = lc.attention(gc.dev(ai.Q, kdt), out_f32=True)
        torch.cuda.synchronize()
        tol = (1e-4, 1e-5) if wl.dtype == "f32" else (2e-2, 2e-3)
        gc.check_attention(O.cpu().numpy(), ai, GpuBank.read(lc.bank), list(range(H)), *tol)
    return stats


@pytest.mark.parametrize("tau", [2.0, 1.3, 1.05])
def test_tiny_f32(tau):
    stats = _seq_stream(WORKLOADS["tiny"], _prm(WORKLOADS["tiny"], tau=tau), attn=tau == 2.0)
    assert stats[0][0] == 48


def test_tiny_bf16():
    wl = dataclasses.replace(WORKLOADS["tiny"], dtype="bf16", name="tiny-bf16")
    _seq_stream(wl, _prm(wl, tau=1.3), attn=True)


POLICY_CASES = {
    "source": dict(order="source"),
    "refresh": dict(baseline="refresh"),
    "densest": dict(eviction="densest"),
    "oldest": dict(eviction="oldest"),
    "head": dict(prefix="head"),
    "fill": dict(fill_below_capacity=True),
    "all": dict(order="source", baseline="refresh", eviction="oldest", prefix="head", fill_below_capacity=True),
}


@pytest.mark.parametrize("name", list(POLICY_CASES))
def test_tiny_policy_variants(name):
    wl = WORKLOADS["tiny"]
    _seq_stream(wl, _prm(wl, tau=1.2, M=40, **POLICY_CASES[name]), seed=4)


MID = Workload(name="mid", H=4, d=128, width=16, height=12, dtype="bf16", M=576, tau=2.0,
               bank_updates=((1, 4), (4, 7), (7, 10), (10, 13)), window=(13, 15), chunk=(15, 18))


@pytest.mark.parametrize("tau", [1.05, 2.0])
def test_mid_bf16(tau):
    """d = 128 bf16, 192-token frames, a bank of 576 filled then churned by
    blocks of 576 candidates: admissions, rejections and evictions at every
    block after the first."""
    stats = _seq_stream(MID, _prm(MID, tau=tau), seed=2, attn=tau == 2.0)
    assert stats[0][0] > 0


def test_mid_bf16_d64_head():
    wl = dataclasses.replace(MID, d=64, name="mid-d64")
    _seq_stream(wl, _prm(wl, tau=1.1, prefix="head"), seed=3)
