"""Pins of the oracle's sequential within-block admission and of density
descriptors other than the post-RoPE key (DensityKV paper summary, appendix
E): a hand-derived example, the brute-force tier for every policy
combination, the one-candidate reduction to the prefix method, the FIFO
window, the density-growth invariant, and descriptor reductions."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import density as od
from oracle import sequential as oseq
from kvsynth import WORKLOADS, LayerGen, frame_tokens

GOLD = os.path.join(os.path.dirname(__file__), "golden")
POLICIES = list(itertools.product(("delta", "source"), ("frozen", "refresh"), ("threshold", "densest", "oldest"),
                                  ("shared", "head"), (False, True)))


def _axis_keys(xs, d=4):
    K = np.zeros((len(xs), d))
    K[:, 0] = xs
    return K


def test_golden_sequential_example():
    g = json.load(open(os.path.join(GOLD, "sequential_admission.json")))
    P = g["params"]
    prm = od.Params(M=P["M"], tau=P["tau"], sigma=P["sigma"], eps=P["eps"], p=P["p"])
    bK = _axis_keys(g["bank"]["x"], g["d"])
    bank = od.HeadBank(np.array(g["bank"]["tok"], np.int64), bK, bK.copy(),
                       np.array([float(Fraction(x)) for x in g["bank"]["rho0"]]))
    cK = _axis_keys(g["candidates"]["x"], g["d"])[None]
    ctok = np.array(g["candidates"]["tok"], np.int32)
    D, _ = od.disturbance(bank.K, cK[0], prm)
    np.testing.assert_allclose(D, [float(Fraction(x)) for x in g["disturbance"]], rtol=1e-14)
    new, info = oseq.update_layer_sequential([bank], cK, cK, ctok, prm)
    assert ctok[info.order[0]].tolist() == g["order_tok"]
    s = g["sequential"]
    nb = new[0].sorted_by_tok()
    assert nb.tok.tolist() == s["final_tok"]
    np.testing.assert_allclose(nb.rho0, [float(Fraction(s["final_rho0"][str(t)])) for t in nb.tok], rtol=1e-13)
    np.testing.assert_allclose(od.density(nb.K, prm), [float(Fraction(s["final_density"][str(t)])) for t in nb.tok],
                               rtol=1e-13)
    # the prefix method on the same block stops before the rejected candidate
    newp, infop = od.update_layer([bank], cK, cK, ctok, prm)
    assert infop.kstar == g["prefix_method"]["kstar"]
    nbp = newp[0].sorted_by_tok()
    assert nbp.tok.tolist() == g["prefix_method"]["final_tok"]
    assert nbp.rho0[-1] == pytest.approx(float(Fraction(g["prefix_method"]["rho0_10"])), rel=1e-13)
    # the brute tier agrees
    newb, adm, _ = oseq.update_layer_sequential_brute([bank], cK, cK, ctok, prm)
    nbb = newb[0].sorted_by_tok()
    assert nbb.tok.tolist() == s["final_tok"]
    np.testing.assert_allclose(nbb.rho0, [float(Fraction(s["final_rho0"][str(t)])) for t in nbb.tok], rtol=1e-13)


def _random_layer(rng, M, heads=2, d=6):
    banks = []
    for h in range(heads):
        n = int(rng.integers(0, M + 1))
        K = rng.normal(size=(n, d)) * 6
        prm = od.Params(M=M)
        banks.append(od.HeadBank(np.arange(n, dtype=np.int64) + 1000 * h, K, K + 0.5,
                                 od.density(K, prm) * rng.uniform(1.0, 1.4, size=n)))
    return banks


@pytest.mark.parametrize("case", range(len(POLICIES)))
def test_brute_tier_agrees_for_every_policy(case):
    order, baseline, eviction, prefix, fill = POLICIES[case]
    rng = np.random.default_rng([7031, case])
    for trial in range(3):
        M = int(rng.integers(6, 14))
        tau = float(rng.choice([1.2, 1.5, 2.0]))
        prm = od.Params(M=M, tau=tau, order=order, baseline=baseline, eviction=eviction, prefix=prefix,
                        fill_below_capacity=fill)
        banks = _random_layer(rng, M)
        N = int(rng.integers(1, 10))
        cK = rng.normal(size=(2, N, 6)) * 6
        ctok = (5000 + rng.permutation(N)).astype(np.int32)
        new_p, info = oseq.update_layer_sequential(banks, cK, cK + 0.5, ctok, prm)
        new_b, adm_b, orders_b = oseq.update_layer_sequential_brute(banks, cK, cK + 0.5, ctok, prm)
        for h in range(2):
            assert info.order[h].tolist() == orders_b[h].tolist()
            assert info.admitted_h[h] == adm_b[h]
            a, b = new_p[h].sorted_by_tok(), new_b[h].sorted_by_tok()
            assert a.tok.tolist() == b.tok.tolist()
            np.testing.assert_allclose(a.rho0, b.rho0, rtol=1e-11, atol=1e-14)
            np.testing.assert_array_equal(a.V, b.V)
            assert a.n <= M


def test_one_candidate_is_the_prefix_method():
    rng = np.random.default_rng(5)
    for trial in range(20):
        M = int(rng.integers(4, 10))
        prm = od.Params(M=M, tau=float(rng.choice([1.1, 1.5, 2.0])))
        banks = _random_layer(rng, M, heads=3)
        cK = rng.normal(size=(3, 1, 6)) * 6
        ctok = np.array([777], np.int32)
        a, _ = oseq.update_layer_sequential(banks, cK, cK, ctok, prm)
        b, info = od.update_layer(banks, cK, cK, ctok, prm)
        for h in range(3):
            x, y = a[h].sorted_by_tok(), b[h].sorted_by_tok()
            assert x.tok.tolist() == y.tok.tolist()
            np.testing.assert_allclose(x.rho0, y.rho0, rtol=1e-12)


def test_fifo_window_at_p0_tau_inf():
    """p = 0, tau = inf, token order, oldest-first eviction: every candidate
    is admitted and the oldest state leaves, so the bank is the M most recent
    tokens."""
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, 4, 0)
    prm = od.Params(M=40, tau=math.inf, p=0.0, order="source", eviction="oldest")
    banks = [od.HeadBank.empty(wl.d) for _ in range(wl.H)]
    seen = []
    for (t0, t1) in wl.bank_updates:
        ctok = frame_tokens(wl, t0, t1)
        cK = gen.keys_all(range(t0, t1)).astype(np.float64)
        banks, info = oseq.update_layer_sequential(banks, cK, cK, ctok, prm)
        seen += sorted(ctok.tolist())
        for h in range(wl.H):
            assert sorted(banks[h].tok.tolist()) == sorted(seen[-prm.M:])


def test_empty_bank_admits_the_whole_first_block():
    """From an empty bank nothing can cross (the block's candidates take their
    baselines at the end), so the first block is admitted whole, as with the
    prefix method."""
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, 2, 0)
    prm = od.Params(M=64, tau=2.0)
    t0, t1 = wl.bank_updates[0]
    ctok = frame_tokens(wl, t0, t1)
    cK = gen.keys_all(range(t0, t1)).astype(np.float64)
    empty = [od.HeadBank.empty(wl.d) for _ in range(wl.H)]
    a, info = oseq.update_layer_sequential(empty, cK, cK, ctok, prm)
    b, _ = od.update_layer(empty, cK, cK, ctok, prm)
    for h in range(wl.H):
        assert len(info.admitted_h[h]) == len(ctok)
        x, y = a[h].sorted_by_tok(), b[h].sorted_by_tok()
        assert x.tok.tolist() == y.tok.tolist()
        np.testing.assert_allclose(x.rho0, y.rho0, rtol=1e-12)


def test_growth_invariant_and_capacity_after_every_block():
    """Threshold eviction with frozen baselines: every state left in the bank
    satisfies rho <= tau rho0 (its density from scratch), and the bank never
    exceeds M."""
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, 1, 0)
    for M, tau in ((64, 2.0), (40, 1.3), (100, 1.1)):
        prm = od.Params(M=M, tau=tau)
        banks = [od.HeadBank.empty(wl.d) for _ in range(wl.H)]
        for (t0, t1) in wl.bank_updates:
            ctok = frame_tokens(wl, t0, t1)
            cK = gen.keys_all(range(t0, t1)).astype(np.float64)
            banks, info = oseq.update_layer_sequential(banks, cK, cK, ctok, prm)
            for h in range(wl.H):
                b = banks[h]
                assert b.n <= M
                assert np.all(od.density(b.K, prm) <= tau * b.rho0 * (1 + 1e-12))


def test_kv_descriptor_with_zero_values_is_the_key_descriptor():
    """[K; V] descriptors with all values zero have the keys' distances."""
    rng = np.random.default_rng(9)
    M = 12
    prm = od.Params(M=M, tau=1.4)
    banks = _random_layer(rng, M)
    N = 9
    cK = rng.normal(size=(2, N, 6)) * 6
    ctok = (300 + rng.permutation(N)).astype(np.int32)
    banksX = [od.HeadBank(b.tok, b.K, np.zeros_like(b.V), b.rho0, np.concatenate([b.K, 0 * b.V], axis=1))
              for b in banks]
    cX = np.concatenate([cK, np.zeros_like(cK)], axis=2)
    for fn in (od.update_layer, oseq.update_layer_sequential):
        a, _ = fn(banks, cK, np.zeros_like(cK), ctok, prm)
        b, _ = fn(banksX, cK, np.zeros_like(cK), ctok, prm, candX=cX)
        for h in range(2):
            assert a[h].sorted_by_tok().tok.tolist() == b[h].sorted_by_tok().tok.tolist()
            np.testing.assert_allclose(a[h].sorted_by_tok().rho0, b[h].sorted_by_tok().rho0, rtol=1e-12)


def test_rotated_descriptor_gives_the_same_bank():
    """Density is invariant under one orthogonal map applied to every
    descriptor (a pre-RoPE descriptor differs from the key by per-position
    rotations; a common rotation changes nothing)."""
    rng = np.random.default_rng(10)
    M = 10
    prm = od.Params(M=M, tau=1.3)
    banks = _random_layer(rng, M)
    N = 8
    cK = rng.normal(size=(2, N, 6)) * 6
    ctok = (90 + rng.permutation(N)).astype(np.int32)
    R, _ = np.linalg.qr(rng.normal(size=(6, 6)))
    banksX = [od.HeadBank(b.tok, b.K, b.V, b.rho0, b.K @ R) for b in banks]
    for fn in (od.update_layer, oseq.update_layer_sequential):
        a, _ = fn(banks, cK, cK, ctok, prm)
        b, _ = fn(banksX, cK, cK, ctok, prm, candX=cK @ R)
        for h in range(2):
            x, y = a[h].sorted_by_tok(), b[h].sorted_by_tok()
            assert x.tok.tolist() == y.tok.tolist()
            np.testing.assert_allclose(x.rho0, y.rho0, rtol=1e-9)
            np.testing.assert_array_equal(x.K, y.K)
