"""Pins of the oracle's DensityKV policy variants (the DensityKV page's
appendix E ablations: candidate order, baselines, eviction completion,
cross-head prefix; plus the fill-below-capacity reading of where the growth
bound binds).  Each variant is pinned by a textbook reduction or an
invariant, and the blocked prefix-sum tier must agree with the brute-force
tier for every combination."""
import itertools
import math

import numpy as np
import pytest

from oracle import density as od
from kvsynth import WORKLOADS, LayerGen, frame_tokens

POLICIES = list(itertools.product(("delta", "source"), ("frozen", "refresh"), ("threshold", "densest", "oldest"),
                                  ("shared", "head"), (False, True)))


def _prm(M, tau=2.0, p=2.0, **kw):
    return od.Params(M=M, tau=tau, sigma=8.0, eps=1.0, p=p, **kw)


def _random_layer(rng, M, heads=2, d=8):
    banks = []
    for h in range(heads):
        n = int(rng.integers(0, M + 1))
        K = rng.normal(size=(n, d)) * 6
        prm = _prm(M)
        banks.append(od.HeadBank(np.arange(n, dtype=np.int64) + 1000 * h, K, K + 0.5,
                                 od.density(K, prm) * rng.uniform(1.0, 1.3, size=n)))
    return banks


@pytest.mark.parametrize("case", range(len(POLICIES)))
def test_brute_tier_agrees_for_every_policy(case):
    # a fixed seed per combination, so that a failure replays exactly
    order, baseline, eviction, prefix, fill = POLICIES[case]
    rng = np.random.default_rng([20240611, case])
    for trial in range(3):
        M = int(rng.integers(8, 18))
        tau = float(rng.choice([1.2, 1.5, 2.0]))
        prm = _prm(M, tau=tau, order=order, baseline=baseline, eviction=eviction, prefix=prefix,
                   fill_below_capacity=fill)
        banks = _random_layer(rng, M)
        N = int(rng.integers(1, 12))
        cK = rng.normal(size=(2, N, 8)) * 6
        # token ids not in input order, so that source order is a real sort
        ctok = (5000 + rng.permutation(N)).astype(np.int32)
        new_p, info = od.update_layer(banks, cK, cK + 0.5, ctok, prm)
        new_b, kst_b, orders_b = od.update_layer_brute(banks, cK, cK + 0.5, ctok, prm)
        for h in range(2):
            assert info.kstar_h[h] == kst_b[h]
            assert info.order[h].tolist() == orders_b[h].tolist()
            a, b = new_p[h].sorted_by_tok(), new_b[h].sorted_by_tok()
            assert a.tok.tolist() == b.tok.tolist()
            np.testing.assert_allclose(a.rho0, b.rho0, rtol=1e-12)
            np.testing.assert_array_equal(a.V, b.V)


def test_source_order_oldest_tau_inf_is_a_fifo_window():
    """tau = inf, candidates in source order, eviction completed oldest
    first, N <= M: every update admits all candidates and evicts the oldest,
    so the bank is exactly the M most recent tokens (a sliding window),
    whatever the interaction."""
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, 2, 0)
    for p in (2.0, 1.0):
        prm = _prm(64, tau=math.inf, p=p, order="source", eviction="oldest")
        banks = [od.HeadBank.empty(wl.d) for _ in range(wl.H)]
        seen = []
        for (t0, t1) in wl.bank_updates:
            ctok = frame_tokens(wl, t0, t1)
            cK = gen.keys_all(range(t0, t1)).astype(np.float64)
            banks, info = od.update_layer(banks, cK, cK, ctok, prm)
            seen += sorted(ctok.tolist())
            for h in range(wl.H):
                assert sorted(banks[h].tok.tolist()) == sorted(seen[-prm.M:])
                assert info.order[h].tolist() == np.argsort(ctok, kind="stable").tolist()


def test_fill_below_capacity_admits_everything_that_fits():
    """n + N <= M: every prefix length fits without eviction, so the fill
    variant admits all N candidates at any tau, while the default (gating at
    every occupancy) stops at the first crossing."""
    rng = np.random.default_rng(5)
    d, M = 8, 40
    K = rng.normal(size=(10, d)) * 3
    bank = od.HeadBank(np.arange(10, dtype=np.int64), K, K, od.density(K, _prm(M)))
    cK = (rng.normal(size=(1, 12, d)) * 3)
    ctok = np.arange(100, 112, dtype=np.int32)
    for tau in (1.0001, 1.5, math.inf):
        new, info = od.update_layer([bank], cK, cK, ctok, _prm(M, tau=tau, fill_below_capacity=True))
        assert info.kstar == 12 and new[0].n == 22 and set(range(10)) <= set(new[0].tok.tolist())
    new, info = od.update_layer([bank], cK, cK, ctok, _prm(M, tau=1.0001))
    assert info.kstar < 12


def test_refreshed_baselines_equal_the_new_densities():
    """baseline "refresh": after each update every state's baseline is its
    density in the new bank (from scratch); frozen baselines keep the
    survivors' insertion values."""
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, 3, 0)
    for baseline in ("refresh", "frozen"):
        prm = _prm(40, tau=1.4, baseline=baseline)
        banks = [od.HeadBank.empty(wl.d) for _ in range(wl.H)]
        for (t0, t1) in wl.bank_updates:
            cK = gen.keys_all(range(t0, t1)).astype(np.float64)
            old = banks
            banks, info = od.update_layer(banks, cK, cK, frame_tokens(wl, t0, t1), prm)
            for h in range(wl.H):
                rho = od.density(banks[h].K, prm)
                if baseline == "refresh":
                    np.testing.assert_allclose(banks[h].rho0, rho, rtol=1e-13)
                else:
                    prev = dict(zip(old[h].tok.tolist(), old[h].rho0.tolist()))
                    for t, r0 in zip(banks[h].tok.tolist(), banks[h].rho0.tolist()):
                        if t in prev:
                            assert r0 == prev[t]


def test_per_head_prefix_is_each_head_alone():
    """prefix "head": each head's result is that head's single-head update
    (where shared and per-head prefixes coincide), and no head takes less
    than the shared prefix."""
    rng = np.random.default_rng(11)
    for trial in range(8):
        M = 14
        banks = _random_layer(rng, M, heads=3)
        N = 10
        cK = rng.normal(size=(3, N, 8)) * 6
        ctok = np.arange(7000, 7000 + N, dtype=np.int32)
        prm_h = _prm(M, tau=1.3, prefix="head")
        new_h, info_h = od.update_layer(banks, cK, cK, ctok, prm_h)
        _, info_s = od.update_layer(banks, cK, cK, ctok, _prm(M, tau=1.3))
        for h in range(3):
            alone, info_a = od.update_layer([banks[h]], cK[h:h + 1], cK[h:h + 1], ctok, _prm(M, tau=1.3))
            assert info_h.kstar_h[h] == info_a.kstar >= info_s.kstar
            assert sorted(new_h[h].tok.tolist()) == sorted(alone[0].tok.tolist())


def test_densest_only_matches_threshold_first_without_crossings():
    """With tau = inf nothing crosses, so densest-only eviction and the
    threshold-first default pick the same states; with a finite tau the
    densest-only set is exactly the top-e projected densities."""
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, 4, 0)
    for tau in (math.inf, 1.3):
        banks = {e: [od.HeadBank.empty(wl.d) for _ in range(wl.H)] for e in ("threshold", "densest")}
        for (t0, t1) in wl.bank_updates:
            cK = gen.keys_all(range(t0, t1)).astype(np.float64)
            ctok = frame_tokens(wl, t0, t1)
            outs = {}
            for ev in ("threshold", "densest"):
                prm = _prm(40, tau=tau, eviction=ev)
                banks[ev], outs[ev] = od.update_layer(banks[ev], cK, cK, ctok, prm)
            if tau == math.inf:
                for h in range(wl.H):
                    assert sorted(banks["threshold"][h].tok.tolist()) == sorted(banks["densest"][h].tok.tolist())
            info = outs["densest"]
            for h in range(wl.H):
                e = info.e[h]
                ev = info.evicted[h]
                if e and (~ev).any():
                    assert info.proj[h][ev].min() >= info.proj[h][~ev].max()
