"""GPU parity of density descriptors other than the post-RoPE key
(DensityKV paper summary, appendix E, descriptor ablation: pre-RoPE keys and
[K; V]) for the prefix method and for sequential admission, against the fp64
oracle on the GPU's validated order and its bank before each block: the
final token sets exactly, every K, V and descriptor row paired with its
token, baselines and densities (from scratch on the descriptors) in fp64."""
import dataclasses

import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, Workload, frame_tokens
from oracle import density as od
from oracle import sequential as oseq

import gpu_common as gc
from _parity import GpuBank, check_order

pytestmark = pytest.mark.gpu


def _descriptors(gen, wl, frames, kind):
    K = gen.keys_all(frames)
    if kind == "prerope":
        return np.stack([gen._round(gen.prerope_keys(h, frames)).reshape(-1, wl.d) for h in range(wl.H)])
    if kind == "kv":
        return np.concatenate([K, gen.values_all(frames)], axis=2)
    if kind == "k":
        return K
    raise ValueError(kind)


def _stream(wl, prm, kind, sequential=False, seed=0):
    import torch
    import kv_cache_compression_head_amd as kb
    from kv_cache_compression_head_amd.pipeline import LayerCache
    gc.banner(f"descriptors {kind} {wl.name} {wl.dtype} d={wl.d} tau={prm.tau} sequential={sequential}")
    gen = LayerGen(wl, seed, 0)
    dx = wl.d * (2 if kind == "kv" else 1)
    desc = kb.LayerDesc(H=wl.H, d=wl.d, M=prm.M, dtype=kb.KVB_BF16 if wl.dtype == "bf16" else kb.KVB_F32,
                        frame_tokens=wl.F, labels=[0] * wl.H, tau=prm.tau, sigma=prm.sigma, eps=prm.eps, p=prm.p,
                        policy=gc.policy_bits(prm) | (kb.KVB_POL_SEQUENTIAL if sequential else 0), desc_dim=dx)
    lc = LayerCache(desc, diagnostics=True)
    kdt = gc.kv_dtype(wl)
    H = wl.H
    Xbank = np.zeros((H, prm.M, dx))
    for (t0, t1) in wl.bank_updates:
        fr = range(t0, t1)
        candK, candV, candX = gen.keys_all(fr), gen.values_all(fr), _descriptors(gen, wl, fr, kind)
        ctok = frame_tokens(wl, t0, t1)
        before = GpuBank.read(lc.bank)
        Xb = lc.bank.X.float().cpu().numpy().astype(np.float64)
        lay = kb.KVLayout(cand_x=gc.dev(candX, kdt))
        cK, cV, ct = gc.dev(candK, kdt), gc.dev(candV, kdt), gc.dev_i32(ctok)
        lc.out.status.zero_()
        D, s, o = lc.score(cK, ct, lay)
        lc.update(cK, cV, ct, D, o, lay)
        torch.cuda.synchronize()
        assert int(lc.out.status.cpu()[0]) == 0
        after = GpuBank.read(lc.bank)
        Xa = lc.bank.X.float().cpu().numpy().astype(np.float64)
        o_np = o.cpu().numpy().astype(np.int64)
        banks = []
        for h in range(H):
            b = before.head(h)
            banks.append(od.HeadBank(b.tok, b.K, b.V, b.rho0, Xb[h, :b.n]))
        X64 = candX.astype(np.float64)
        for h in range(H):
            _, delta = od.disturbance(banks[h].X, X64[h], prm)
            check_order(o_np[h], delta, ctok.astype(np.int64))
        orders = [o_np[h] for h in range(H)]
        if sequential:
            new, _ = oseq.update_layer_sequential(banks, candK.astype(np.float64), candV.astype(np.float64), ctok, prm,
                                                  candX=X64, order=orders)
        else:
            new, info = od.update_layer(banks, candK.astype(np.float64), candV.astype(np.float64), ctok, prm,
                                        order=orders, candX=X64)
            assert int(lc.out.k_star.cpu()[0]) == info.kstar
        for h in range(H):
            n = int(after.count[h])
            nb = new[h]
            assert n == nb.n and sorted(after.tok[h, :n].tolist()) == sorted(nb.tok.tolist()), f"head {h}"
            pos = {int(t): i for i, t in enumerate(nb.tok.tolist())}
            idx = np.array([pos[int(t)] for t in after.tok[h, :n]])
            np.testing.assert_array_equal(after.K[h, :n], nb.K[idx])
            np.testing.assert_array_equal(after.V[h, :n], nb.V[idx])
            np.testing.assert_array_equal(Xa[h, :n], nb.X[idx])
            np.testing.assert_allclose(after.rho0[h, :n], nb.rho0[idx], rtol=1e-4, atol=1e-6)
            np.testing.assert_allclose(after.rho[h, :n], od.density(nb.X, prm)[idx], rtol=1e-4, atol=1e-6)
    return lc


@pytest.mark.parametrize("sequential", [False, True])
def test_tiny_prerope(sequential):
    wl = WORKLOADS["tiny"]
    prm = od.Params(M=wl.M, tau=1.3)
    _stream(wl, prm, "prerope", sequential)


@pytest.mark.parametrize("sequential", [False, True])
def test_tiny_kv_d64(sequential):
    """[K; V] at head dimension 64: 128-wide descriptors."""
    wl = WORKLOADS["tiny"]
    prm = od.Params(M=wl.M, tau=1.3)
    _stream(wl, prm, "kv", sequential)


MID = Workload(name="mid", H=4, d=64, width=16, height=12, dtype="bf16", M=576, tau=2.0,
               bank_updates=((1, 4), (4, 7), (7, 10)), window=(10, 12), chunk=(12, 15))


def test_mid_bf16_kv_d64():
    _stream(MID, od.Params(M=MID.M, tau=1.1), "kv")


@pytest.mark.parametrize("sequential", [False, True])
def test_mid_bf16_kv_d128(sequential):
    """[K; V] at head dimension 128: 256-wide descriptors (the appendix E
    ablation at the head width of the pages' backbone)."""
    wl = dataclasses.replace(MID, d=128, name="mid-d128")
    _stream(wl, od.Params(M=wl.M, tau=1.1), "kv", sequential)


def test_mid_bf16_prerope_d128():
    wl = dataclasses.replace(MID, d=128, name="mid-d128")
    _stream(wl, od.Params(M=wl.M, tau=1.1), "prerope")


def test_key_descriptor_equals_the_method():
    """desc_dim = d with the keys themselves as descriptors gives the bank of
    desc_dim = 0 bit for bit."""
    import torch
    wl = dataclasses.replace(MID, d=128, name="mid-d128")
    prm = od.Params(M=wl.M, tau=1.1)
    a = _stream(wl, prm, "k")
    lc = gc.layer_for(wl, prm)
    gen = LayerGen(wl, 0, 0)
    import kv_cache_compression_head_amd as kb
    for fr in wl.bank_updates:
        gc.run_update(lc, gen, wl, prm, fr, list(range(wl.H)), replay=False)
    for x, y in ((a.bank.K, lc.bank.K), (a.bank.V, lc.bank.V), (a.bank.tok, lc.bank.tok), (a.bank.rho0, lc.bank.rho0),
                 (a.bank.rho, lc.bank.rho), (a.bank.count, lc.bank.count)):
        assert torch.equal(x, y)
