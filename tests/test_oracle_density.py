"""Pins of the fp64 DensityKV oracle against closed forms, invariants,
textbook special cases, a hand-computed example and a brute-force tier."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import density as od
from kvsynth import WORKLOADS, LayerGen, frame_tokens

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _prm(M, tau=2.0, p=2.0, sigma=8.0, eps=1.0):
    return od.Params(M=M, tau=tau, sigma=sigma, eps=eps, p=p)


def _axis_keys(xs, d=4, axis=0):
    K = np.zeros((len(xs), d))
    K[:, axis] = xs
    return K


# -- interaction / density ----------------------------------------------------

def test_phi_closed_forms():
    prm = _prm(8)
    # phi(64) = 1/(1 + 1) and phi(256) = 1/(1 + 4) at sigma = 8, p = 2, eps = 1
    assert od.phi(np.array([0.0, 64.0, 256.0]), prm).tolist() == [1.0, 0.5, 0.2]
    # p = 4 squares the p = 2 value; p = 0 is constant 1
    assert od.phi(np.array([64.0]), _prm(8, p=4))[0] == pytest.approx(0.25, abs=0, rel=1e-15)
    assert od.phi(np.array([123.0]), _prm(8, p=0))[0] == 1.0
    # p = 1 is the inverse softened distance
    assert od.phi(np.array([192.0]), _prm(8, p=1))[0] == pytest.approx(0.5, rel=1e-15)


def test_density_collinear_keys():
    K = _axis_keys([0.0, 8.0, 16.0])
    rho = od.density(K, _prm(8))
    np.testing.assert_allclose(rho, [0.7, 1.0, 0.7], rtol=1e-15)


def test_density_two_keys():
    for dist in (0.0, 3.0, 8.0, 40.0):
        K = _axis_keys([1.0, 1.0 + dist])
        rho = od.density(K, _prm(8))
        expect = 1.0 / (1.0 + dist * dist / 64.0)
        np.testing.assert_allclose(rho, [expect, expect], rtol=1e-15)


def test_sqdist_forms_agree():
    rng = np.random.default_rng(3)
    A, B = rng.normal(size=(70, 128)) * 2, rng.normal(size=(90, 128)) * 2
    d1 = od.sqdist_direct(A, B)
    d2 = od.sqdist_gram(A, B)
    np.testing.assert_allclose(d1, d2, rtol=1e-11, atol=1e-9)
    # direct form against a per-pair python loop
    for i, j in ((0, 0), (5, 17), (69, 89)):
        assert d1[i, j] == pytest.approx(sum((A[i, t] - B[j, t]) ** 2 for t in range(128)), rel=1e-13)


def test_density_permutation_and_rotation_invariance():
    rng = np.random.default_rng(11)
    K = rng.normal(size=(50, 16)) * 3
    prm = _prm(8)
    rho = od.density(K, prm)
    perm = rng.permutation(50)
    np.testing.assert_allclose(od.density(K[perm], prm), rho[perm], rtol=1e-13)
    Qm, _ = np.linalg.qr(rng.normal(size=(16, 16)))
    np.testing.assert_allclose(od.density(K @ Qm.T, prm), rho, rtol=1e-11)


def test_logit_gap_bound_a1():
    """|q.k1 - q.k2| <= |q| |k1 - k2|, equality for q parallel to k1 - k2."""
    rng = np.random.default_rng(5)
    k1, k2 = rng.normal(size=64), rng.normal(size=64)
    dist = math.sqrt(od.sqdist_direct(k1[None], k2[None])[0, 0])
    for _ in range(200):
        q = rng.normal(size=64)
        q /= np.linalg.norm(q)
        assert abs(q @ k1 - q @ k2) <= dist * (1 + 1e-12)
    qs = (k1 - k2) / np.linalg.norm(k1 - k2)
    assert abs(qs @ k1 - qs @ k2) == pytest.approx(dist, rel=1e-12)


# -- hand-computed admission example ------------------------------------------

def _fr(s):
    return float(Fraction(s))


@pytest.mark.parametrize("case_idx", [0, 1])
def test_golden_collinear_admission(case_idx):
    g = json.load(open(os.path.join(GOLD, "collinear_admission.json")))
    case = g["cases"][case_idx]
    d = g["d"]
    prm = od.Params(M=case["M"], **g["params"])
    bank = od.HeadBank(np.array(g["bank"]["tok"], np.int64), _axis_keys(g["bank"]["x"], d),
                       _axis_keys(g["bank"]["x"], d) + 1.0, np.array([_fr(s) for s in g["bank"]["rho0"]]))
    np.testing.assert_allclose(od.density(bank.K, prm), [_fr(s) for s in g["bank_density"]], rtol=1e-14)
    cK = _axis_keys(g["candidates"]["x"], d)[None]
    cV = cK + 2.0
    ctok = np.array(g["candidates"]["tok"], np.int32)
    new, info = od.update_layer([bank], cK, cV, ctok, prm)
    np.testing.assert_allclose(info.D[0], [_fr(s) for s in g["disturbance"]], rtol=1e-14)
    assert ctok[info.order[0]].tolist() == g["order_tok"]
    assert info.kstar == case["kstar"]
    assert sorted(bank.tok[info.evicted[0]].tolist()) == case["evicted_tok"]
    if "projected_at_kstar" in case:
        np.testing.assert_allclose(info.proj[0], [_fr(s) for s in case["projected_at_kstar"]], rtol=1e-14)
    nb = new[0].sorted_by_tok()
    assert nb.tok.tolist() == case["final_tok"]
    for t, r0 in case["final_rho0"].items():
        i = nb.tok.tolist().index(int(t))
        assert nb.rho0[i] == pytest.approx(_fr(r0), rel=1e-14)
    for t, r in case.get("final_density", {}).items():
        i = nb.tok.tolist().index(int(t))
        assert od.density(nb.K, prm)[i] == pytest.approx(_fr(r), rel=1e-14)
    # values stay paired with their keys
    np.testing.assert_array_equal(nb.V, nb.K + np.where(np.isin(nb.tok, ctok), 2.0, 1.0)[:, None])


def test_storage_pin():
    g = json.load(open(os.path.join(GOLD, "storage.json")))
    b = od.bank_payload_bytes(g["L"], g["H"], g["M"], g["dk"], g["dv"], 2)
    assert round(b / 2 ** 30, 2) == g["payload_gib_printed"]


# -- special cases reducing to textbook routines ------------------------------

def _tiny_stream(prm, seed=0, updates=None, heads=(0, 1)):
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, seed, 0)
    banks = [od.HeadBank.empty(wl.d) for _ in range(wl.H)]
    infos = []
    for (t0, t1) in (updates or wl.bank_updates):
        fr = range(t0, t1)
        cK = gen.keys_all(fr).astype(np.float64)
        cV = gen.values_all(fr).astype(np.float64)
        banks, info = od.update_layer(banks, cK, cV, frame_tokens(wl, t0, t1), prm, heads=heads)
        infos.append(info)
    return banks, infos, gen


def test_fifo_at_p0_tau_inf():
    """p = 0 (phi = 1), tau = inf, N <= M: the bank is the M most recent tokens."""
    prm = _prm(64, tau=math.inf, p=0.0)
    banks, infos, _ = _tiny_stream(prm)
    wl = WORKLOADS["tiny"]
    last = wl.bank_updates[-1][1] * wl.F
    for h in range(wl.H):
        assert sorted(banks[h].tok.tolist()) == list(range(last - 64, last))


def test_full_admission_reproduces_full_attention():
    """M >= history and tau = inf: everything is admitted; attention over
    sink + bank + chunk equals attention over the whole history."""
    from oracle.attention import attention
    wl = WORKLOADS["tiny"]
    prm = _prm(144, tau=math.inf)
    banks, infos, gen = _tiny_stream(prm)
    assert all(i.kstar == 48 for i in infos)
    for h in range(wl.H):
        assert sorted(banks[h].tok.tolist()) == list(range(16, 160))
        Q = gen.queries(h, range(10, 13), [10, 11, 12]).astype(np.float64)
        chunkK = gen.keys(h, range(10, 13), [10, 11, 12]).astype(np.float64)
        chunkV = gen.values(h, range(10, 13)).astype(np.float64)
        sinkK, sinkV = gen.keys(h, [0]).astype(np.float64), gen.values(h, [0]).astype(np.float64)
        Kc = np.concatenate([sinkK, banks[h].K, chunkK])
        Vc = np.concatenate([sinkV, banks[h].V, chunkV])
        allK = np.concatenate([gen.keys(h, range(0, 10)).astype(np.float64), chunkK])
        allV = np.concatenate([gen.values(h, range(0, 10)).astype(np.float64), chunkV])
        np.testing.assert_allclose(attention(Q, Kc, Vc), attention(Q, allK, allV), rtol=1e-12, atol=1e-13)


def test_tau_inf_full_bank_evicts_top_density():
    """tau = inf, full bank: the eviction set is plain top-e by projected density."""
    rng = np.random.default_rng(2)
    M, d = 40, 16
    prm = _prm(M, tau=math.inf)
    K = rng.normal(size=(M, d)) * 4
    bank = od.HeadBank(np.arange(M, dtype=np.int64), K, K * 0, od.density(K, prm))
    cK = rng.normal(size=(1, 12, d)) * 4
    ctok = np.arange(100, 112, dtype=np.int32)
    new, info = od.update_layer([bank], cK, cK, ctok, prm)
    assert info.kstar == 12 and info.e[0] == 12
    adm = cK[0][info.order[0][:12]]
    proj = np.array([sum(1.0 / (1.0 + np.sum((K[b] - y) ** 2) / 64.0) for y in np.concatenate([np.delete(K, b, 0), adm]))
                     for b in range(M)])
    top = set(np.argsort(-proj, kind="stable")[:12].tolist())
    assert set(np.nonzero(info.evicted[0])[0].tolist()) == top


def test_duplicate_key_rejected_first():
    """Far-apart bank keys plus one candidate duplicating a bank key: the
    duplicate has the highest disturbance, is ordered last, and is the one
    candidate rejected because its twin would cross tau * rho0."""
    d, n = 64, 60
    K = np.eye(d)[:n] * 200.0
    prm = _prm(100, tau=2.0)
    rho = od.density(K, prm)
    bank = od.HeadBank(np.arange(n, dtype=np.int64), K, K + 1, rho.copy())
    cK = np.concatenate([np.eye(d)[n:n + 3] * 200.0, K[5:6]])[None]
    ctok = np.array([100, 101, 102, 103], np.int32)
    new, info = od.update_layer([bank], cK, cK, ctok, prm)
    assert int(np.argmax(info.delta[0])) == 3
    assert info.order[0][-1] == 3
    assert info.kstar == 3
    assert 103 not in new[0].tok.tolist() and 5 in new[0].tok.tolist()
    assert info.t[0][5] == 4 and np.all(np.delete(info.t[0], 5) == 5)


def test_brute_tier_agrees_with_plain_tier():
    rng = np.random.default_rng(0)
    for trial in range(6):
        M = int(rng.integers(8, 20))
        d = 8
        tau = float(rng.choice([1.2, 1.5, 2.0]))
        prm = _prm(M, tau=tau)
        banks = []
        for h in range(2):
            n = int(rng.integers(0, M + 1))
            K = rng.normal(size=(n, d)) * 6
            banks.append(od.HeadBank(np.arange(n, dtype=np.int64) + 1000 * h, K, K + 0.5,
                                     od.density(K, prm) * rng.uniform(1.0, 1.3, size=n)))
        N = int(rng.integers(1, 14))
        cK = rng.normal(size=(2, N, d)) * 6
        ctok = np.arange(5000, 5000 + N, dtype=np.int32)
        new_p, info = od.update_layer(banks, cK, cK + 0.5, ctok, prm)
        new_b, kstar_b, orders_b = od.update_layer_brute(banks, cK, cK + 0.5, ctok, prm)
        assert all(v == info.kstar for v in kstar_b.values())
        for h in range(2):
            assert info.order[h].tolist() == orders_b[h].tolist()
            a, b = new_p[h].sorted_by_tok(), new_b[h].sorted_by_tok()
            assert a.tok.tolist() == b.tok.tolist()
            np.testing.assert_allclose(a.rho0, b.rho0, rtol=1e-12)
            np.testing.assert_array_equal(a.V, b.V)


def test_permutation_of_inputs_gives_same_sets():
    prm = _prm(64, tau=1.3)
    banks, infos, gen = _tiny_stream(prm, updates=((1, 4), (4, 7)))
    wl = WORKLOADS["tiny"]
    cK = gen.keys_all(range(7, 10)).astype(np.float64)
    cV = gen.values_all(range(7, 10)).astype(np.float64)
    ctok = frame_tokens(wl, 7, 10)
    ref, rinfo = od.update_layer(banks, cK, cV, ctok, prm)
    rng = np.random.default_rng(9)
    pc = rng.permutation(ctok.shape[0])
    pb = [rng.permutation(b.n) for b in banks]
    banks2 = [od.HeadBank(b.tok[p], b.K[p], b.V[p], b.rho0[p]) for b, p in zip(banks, pb)]
    out, oinfo = od.update_layer(banks2, cK[:, pc], cV[:, pc], ctok[pc], prm)
    assert oinfo.kstar == rinfo.kstar
    for h in range(wl.H):
        assert sorted(out[h].tok.tolist()) == sorted(ref[h].tok.tolist())


def test_rotation_invariance_of_decisions():
    prm = _prm(64, tau=1.3)
    banks, infos, gen = _tiny_stream(prm, updates=((1, 4), (4, 7)))
    wl = WORKLOADS["tiny"]
    cK = gen.keys_all(range(7, 10)).astype(np.float64)
    ctok = frame_tokens(wl, 7, 10)
    ref, rinfo = od.update_layer(banks, cK, cK, ctok, prm)
    Qm, _ = np.linalg.qr(np.random.default_rng(4).normal(size=(wl.d, wl.d)))
    banks2 = [od.HeadBank(b.tok, b.K @ Qm.T, b.V, b.rho0) for b in banks]
    out, oinfo = od.update_layer(banks2, cK @ Qm.T, cK, ctok, prm)
    assert oinfo.kstar == rinfo.kstar
    for h in range(wl.H):
        assert sorted(out[h].tok.tolist()) == sorted(ref[h].tok.tolist())


def test_bank_bookkeeping_invariants():
    prm = _prm(64, tau=1.5)
    wl = WORKLOADS["tiny"]
    gen = LayerGen(wl, 1, 0)
    banks = [od.HeadBank.empty(wl.d) for _ in range(wl.H)]
    for (t0, t1) in wl.bank_updates:
        fr = range(t0, t1)
        cK = gen.keys_all(fr).astype(np.float64)
        cV = gen.values_all(fr).astype(np.float64)
        banks, info = od.update_layer(banks, cK, cV, frame_tokens(wl, t0, t1), prm)
        for h in range(wl.H):
            b = banks[h]
            assert b.n <= prm.M
            assert len(set(b.tok.tolist())) == b.n
            rho = od.density(b.K, prm)
            assert np.all(rho <= prm.tau * b.rho0 * (1 + 1e-12))
            # exact K/V pairing: rows equal the generator's rows for their token
            for i in range(b.n):
                f, p = divmod(int(b.tok[i]), wl.F)
                assert np.array_equal(b.V[i], gen.values(h, [f])[p].astype(np.float64))
                assert np.array_equal(b.K[i], gen.keys(h, [f])[p].astype(np.float64))


def test_threaded_row_blocks_match_serial():
    """The row blocks of the pairwise sums run in threads when workers > 1;
    each row is the same fp64 sum, so results agree with the serial run to
    BLAS rounding order."""
    rng = np.random.default_rng(11)
    prm = od.Params(M=64)
    K = rng.normal(size=(700, 16)) * 4
    C = rng.normal(size=(500, 16)) * 4
    r1 = od.density(K, prm)
    D1, _ = od.disturbance(K, C, prm)
    t1, (v1,) = od.crossing_times(K, r1, r1 * 1.02, C, prm, at=[np.full(700, 37)])
    try:
        od.set_workers(4)
        r2 = od.density(K, prm)
        D2, _ = od.disturbance(K, C, prm)
        t2, (v2,) = od.crossing_times(K, r2, r2 * 1.02, C, prm, at=[np.full(700, 37)])
    finally:
        od.set_workers(1)
    np.testing.assert_allclose(r2, r1, rtol=1e-13)
    np.testing.assert_allclose(D2, D1, rtol=1e-13)
    np.testing.assert_allclose(v2, v1, rtol=1e-13)
    assert np.array_equal(t1, t2)
