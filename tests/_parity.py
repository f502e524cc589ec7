"""Stage-replay parity checks of the HIP bank update against the fp64 oracle.

Each stage of the GPU update is compared with the oracle's stage computed on
the GPU's validated decision of the previous stage, so one floating-point
near-tie cannot cascade into later stages.  A discrete mismatch is accepted
only where the oracle's deciding gap is below ``GAP`` (relative):

* order inversions: |delta_i - delta_j| / delta_j
* crossing flips:  |rho'(k) - tau rho0| / (tau rho0)
* eviction swaps:  |rho'_a - rho'_b| / rho'_b
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from oracle import density as od

GAP = 1e-4


@dataclass
class GpuBank:
    tok: np.ndarray      # [H][M] int
    K: np.ndarray        # [H][M][d] float64
    V: np.ndarray
    rho0: np.ndarray     # [H][M]
    rho: np.ndarray
    count: np.ndarray    # [H]

    @staticmethod
    def read(bank) -> "GpuBank":
        return GpuBank(bank.tok.cpu().numpy().astype(np.int64), bank.K.float().cpu().numpy().astype(np.float64),
                       bank.V.float().cpu().numpy().astype(np.float64), bank.rho0.cpu().numpy().astype(np.float64),
                       bank.rho.cpu().numpy().astype(np.float64), bank.count.cpu().numpy().astype(np.int64))

    def head(self, h) -> od.HeadBank:
        n = int(self.count[h])
        return od.HeadBank(self.tok[h, :n].copy(), self.K[h, :n].copy(), self.V[h, :n].copy(), self.rho0[h, :n].copy())


def check_order(order: np.ndarray, delta: np.ndarray, tok: np.ndarray, gap: float = GAP) -> int:
    """GPU permutation vs oracle delta: every inversion must be a near-tie;
    exactly equal deltas must be ordered by token id.  Returns the number of
    adjacent near-tie inversions."""
    n = delta.shape[0]
    assert np.array_equal(np.sort(order), np.arange(n)), "order is not a permutation"
    d = delta[order]
    t = tok[order]
    runmax = np.maximum.accumulate(d)
    scale = np.maximum(np.abs(runmax), 1e-30)
    bad = (runmax - d) > gap * scale
    assert not bad.any(), f"order inversion beyond the gap at positions {np.nonzero(bad)[0][:10]}"
    eq = d[1:] == d[:-1]
    assert np.all(t[1:][eq] > t[:-1][eq]), "equal scores not ordered by token id"
    return int(np.sum(d[1:] < d[:-1]))


def check_crossings(t_gpu, bankK, rho, rho0, candK_sorted, prm, gap=GAP) -> int:
    """GPU crossing prefix lengths vs the oracle's on the same order.  Rows that
    differ must be near-ties at the disputed prefix lengths."""
    t_or, _ = od.crossing_times(bankK, rho, rho0, candK_sorted, prm)
    diff = np.nonzero(t_gpu != t_or)[0]
    if diff.size == 0:
        return 0
    kmax = candK_sorted.shape[0]
    # oracle crosses earlier -> check at the last k the GPU did not cross;
    # GPU crosses earlier -> check at the first k the GPU did cross
    k_check = np.clip(np.where(t_or[diff] < t_gpu[diff], t_gpu[diff] - 1, t_gpu[diff]), 0, kmax)
    _, (vals,) = od.crossing_times(bankK[diff], rho[diff], rho0[diff], candK_sorted, prm, at=[k_check])
    thr = prm.tau * rho0[diff]
    rel = np.abs(vals - thr) / np.maximum(thr, 1e-30)
    assert np.all(rel < gap), f"crossing mismatch beyond the gap: rows {diff[rel >= gap][:10]} rel {rel[rel >= gap][:5]}"
    return int(diff.size)


def check_evictions(ev_gpu: np.ndarray, mand: np.ndarray, proj: np.ndarray, gap=GAP):
    """GPU eviction completion must be a densest top-r of the oracle's
    projected densities, up to near-ties."""
    assert np.all(ev_gpu[mand]), "a crossed state was not evicted"
    rest = ~mand
    evd = ev_gpu & rest
    kept = (~ev_gpu) & rest
    if evd.any() and kept.any():
        lo = proj[evd].min()
        hi = proj[kept].max()
        assert lo >= hi - gap * max(abs(hi), 1e-30), f"eviction completion not densest: min evicted {lo} < max kept {hi}"


@dataclass
class Report:
    kstar: int
    order_near_ties: int = 0
    crossing_near_ties: int = 0
    admitted: List[int] = field(default_factory=list)
    evicted: List[int] = field(default_factory=list)
    rho_after: Dict[int, np.ndarray] = field(default_factory=dict)   # from-scratch densities of the new bank


def check_evictions_oldest(ev_gpu: np.ndarray, mand: np.ndarray, tok: np.ndarray):
    """Source-order completion: the crossed states, then the oldest (lowest
    token id) of the rest; token ids are unique, so the set is exact."""
    assert np.all(ev_gpu[mand]), "a crossed state was not evicted"
    evd = ev_gpu & ~mand
    kept = (~ev_gpu) & ~mand
    if evd.any() and kept.any():
        assert tok[evd].max() < tok[kept].min(), "completion is not the oldest states"


def _pool_map(fn, items, workers):
    """map over items in threads: the oracle's numpy work releases the GIL,
    so heads are checked side by side on the host's cores."""
    items = list(items)
    if workers <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def replay_update(before: GpuBank, after: GpuBank, candK, candV, cand_tok, D_gpu, delta_gpu, order_gpu,
                  t_gpu, rhoP_gpu, kstar_gpu, n_mand_gpu, n_ev_gpu, prm: od.Params, heads: List[int],
                  rtol_D=2e-5, rtol_rho=1e-4, workers: int = 0, kstar_heads: Optional[List[int]] = None,
                  rho_before: Optional[Dict[int, np.ndarray]] = None) -> Report:
    """Stage-replay check of one layer update over the listed density heads,
    under the policy fields of prm.  kstar_gpu: the device's k_star array
    (entry 0 the shared prefix, or one entry per head).

    Every value of the listed heads is checked (no sampling).  kstar_heads:
    the layer's density heads whose GPU crossing times enter the shared
    prefix check (default: heads); only the listed heads are replayed in
    fp64.  rho_before: from-scratch densities of the bank before the update
    per head (a previous replay's rho_after), reused instead of recomputed.
    The report's rho_after holds the new bank's from-scratch densities."""
    N = cand_tok.shape[0]
    kmax = min(N, prm.M)
    tok = cand_tok.astype(np.int64)
    ks_arr = np.atleast_1d(np.asarray(kstar_gpu)).astype(np.int64)
    per_head = prm.prefix == "head"
    kof = (lambda h: int(ks_arr[h])) if per_head else (lambda h: int(ks_arr[0]))
    k = int(ks_arr[heads].max()) if per_head else int(ks_arr[0])
    fill = prm.fill_below_capacity
    # crossed rows survive (and carry rho') under densest-only eviction and below capacity with fill
    keep_crossed = prm.eviction == "densest" or fill
    rep = Report(kstar=k)
    workers = workers or default_workers()

    def stage12(h):
        b = before.head(h)
        rho_def = rho_before[h] if rho_before is not None and h in rho_before else od.density(b.K, prm)
        # stored density (maintained incrementally on the GPU) vs its definition
        np.testing.assert_allclose(before.rho[h, :b.n], rho_def, rtol=rtol_rho, atol=1e-6)
        # stage 1: disturbance and order
        D, delta = od.disturbance(b.K, candK[h], prm)
        np.testing.assert_allclose(D_gpu[h], D, rtol=rtol_D, atol=1e-6)
        np.testing.assert_allclose(delta_gpu[h], delta, rtol=rtol_D, atol=1e-6)
        nt = 0
        if prm.order == "source":
            assert order_gpu[h].tolist() == np.argsort(tok, kind="stable").tolist(), "source order"
        else:
            nt = check_order(order_gpu[h], delta, tok)
        # stage 2: crossing prefix lengths on the GPU's order
        pi = order_gpu[h].astype(np.int64)
        cs = np.asarray(candK[h], np.float64)[pi[:kmax]]
        tg = t_gpu[h, :b.n].astype(np.int64)
        nc = check_crossings(tg, b.K, rho_def, b.rho0, cs, prm)
        return (b, rho_def, cs, pi, tg, nt, nc)

    res = dict(zip(heads, _pool_map(stage12, heads, workers)))
    for h in heads:
        rep.order_near_ties += res[h][5]
        rep.crossing_near_ties += res[h][6]
    # stage 3: prefix lengths from the GPU's crossing times (integer logic, exact)
    kh_list = list(heads) if kstar_heads is None else list(kstar_heads)
    tl = [t_gpu[h, :int(before.count[h])].astype(np.int64) for h in kh_list]
    ns = [int(before.count[h]) for h in kh_list]
    if per_head:
        for h, tg_h, n_h in zip(kh_list, tl, ns):
            kh = int(np.nonzero(od.feasible_head(tg_h, n_h, prm.M, kmax, fill))[0].max())
            assert kh == kof(h), f"head {h}: k* {kof(h)} != oracle prefix {kh} on the GPU crossing times"
    else:
        ks_ref, _ = od.feasible_prefix(tl, ns, prm.M, kmax, fill)
        assert ks_ref == k, f"k* {k} != oracle prefix {ks_ref} on the GPU crossing times"

    def stage45(h):
        b, rho_def, cs, pi, tg = res[h][:5]
        k = kof(h)
        e = max(0, b.n + k - prm.M) if k > 0 else 0
        assert int(n_ev_gpu[h]) == e, f"head {h}: evicted {int(n_ev_gpu[h])} != e {e}"
        gated = k > 0 and not (fill and b.n + k <= prm.M)
        crossed = (tg <= k) if gated else np.zeros(b.n, bool)
        assert int(n_mand_gpu[h]) == int(crossed.sum()), f"head {h}: n_mandatory"
        mand = crossed if prm.eviction != "densest" else np.zeros(b.n, bool)
        # stage 4: projected densities and eviction set
        proj = od.projected_density(b.K, rho_def, cs, k, prm) if k > 0 else rho_def
        live = np.ones(b.n, bool) if keep_crossed else ~crossed
        np.testing.assert_allclose(rhoP_gpu[h, :b.n][live], proj[live], rtol=rtol_rho, atol=1e-6)
        new_n = int(after.count[h])
        assert new_n == b.n - e + k, f"head {h}: count {new_n} != {b.n - e + k}"
        new_toks = set(after.tok[h, :new_n].tolist())
        assert len(new_toks) == new_n, f"head {h}: duplicate token in the bank"
        adm_toks = tok[pi[:k]]
        assert set(adm_toks.tolist()) <= new_toks, f"head {h}: admitted tokens missing"
        ev_gpu = np.array([t not in new_toks for t in b.tok.tolist()], dtype=bool)
        assert int(ev_gpu.sum()) == e
        if prm.eviction == "oldest":
            check_evictions_oldest(ev_gpu, mand, b.tok)
        else:
            check_evictions(ev_gpu, mand, proj)
        # stage 5: new bank -- exact pairing, frozen baselines, densities
        hb = after.head(h)
        if k == 0:
            # nothing admitted or evicted: the bank and its densities are unchanged
            assert np.array_equal(after.tok[h, :new_n], before.tok[h, :b.n])
            assert np.array_equal(after.K[h, :new_n], before.K[h, :b.n])
            assert np.array_equal(after.V[h, :new_n], before.V[h, :b.n])
            assert np.array_equal(after.rho0[h, :new_n], before.rho0[h, :b.n])
            assert np.array_equal(after.rho[h, :new_n], before.rho[h, :b.n])
            return (k, e, rho_def)
        oldpos = {int(t): i for i, t in enumerate(b.tok.tolist())}
        cpos = {int(t): i for i, t in enumerate(tok.tolist())}
        is_new = np.zeros(hb.n, bool)
        for i, t in enumerate(hb.tok.tolist()):
            if t in oldpos:
                j = oldpos[t]
                assert np.array_equal(hb.K[i], b.K[j]) and np.array_equal(hb.V[i], b.V[j]), "survivor row moved"
                if prm.baseline == "frozen":
                    assert hb.rho0[i] == b.rho0[j], "survivor baseline changed"
            else:
                is_new[i] = True
                j = cpos[t]
                assert np.array_equal(hb.K[i], np.asarray(candK[h][j], np.float64)), "admitted K not exact"
                assert np.array_equal(hb.V[i], np.asarray(candV[h][j], np.float64)), "admitted V not paired"
        rho_new = od.density(hb.K, prm)
        np.testing.assert_allclose(after.rho[h, :hb.n], rho_new, rtol=rtol_rho, atol=1e-6)
        np.testing.assert_allclose(hb.rho0[is_new], rho_new[is_new], rtol=rtol_rho, atol=1e-6)
        if prm.baseline == "refresh":
            np.testing.assert_allclose(hb.rho0, rho_new, rtol=rtol_rho, atol=1e-6)
        return (k, e, rho_new)

    out = _pool_map(stage45, heads, workers)
    for h, (kk, e, rn) in zip(heads, out):
        rep.admitted.append(kk)
        rep.evicted.append(e)
        rep.rho_after[h] = rn
    return rep


def sampled_update(before: GpuBank, after: GpuBank, candK, candV, cand_tok, D_gpu, delta_gpu, order_gpu,
                   t_gpu, rhoP_gpu, kstar_gpu, n_mand_gpu, n_ev_gpu, prm: od.Params, heads: List[int],
                   nsample: int = 48, full_order_heads=(), seed: int = 0, rtol=2e-5) -> Report:
    """Full-size check: every integer decision is verified exactly from the
    GPU's own outputs (order sortedness, k* from the crossing times, eviction
    structure, bank contents and K/V pairing); floating-point stages are
    compared with the oracle on sampled rows (and the full order on
    ``full_order_heads``)."""
    rng = np.random.default_rng(seed)
    N = cand_tok.shape[0]
    kmax = min(N, prm.M)
    tok = cand_tok.astype(np.int64)
    k = int(kstar_gpu)
    rep = Report(kstar=k)
    tl, ns = [], []
    for h in heads:
        n = int(before.count[h])
        bK = before.K[h, :n]
        pi = order_gpu[h].astype(np.int64)
        # order: a permutation, non-decreasing in the GPU's delta, ties by token
        assert np.array_equal(np.sort(pi), np.arange(N))
        dg = delta_gpu[h][pi]
        assert np.all(np.diff(dg) >= 0), "GPU order not sorted by its own delta"
        eq = dg[1:] == dg[:-1]
        assert np.all(tok[pi][1:][eq] > tok[pi][:-1][eq])
        # disturbance on sampled candidates; delta = D / mean(D)
        cs = rng.choice(N, size=min(nsample, N), replace=False)
        Dref = od.phi_rowsum(np.asarray(candK[h][cs], np.float64), bK, prm)
        np.testing.assert_allclose(D_gpu[h][cs], Dref, rtol=rtol, atol=1e-6)
        mean = np.mean(D_gpu[h].astype(np.float64))
        if n > 0 and mean > 0:
            np.testing.assert_allclose(delta_gpu[h], D_gpu[h] / mean, rtol=1e-5)
        if h in full_order_heads:
            Dfull, deltafull = od.disturbance(bK, candK[h], prm)
            np.testing.assert_allclose(D_gpu[h], Dfull, rtol=rtol, atol=1e-6)
            rep.order_near_ties += check_order(pi, deltafull, tok)
        # crossing times on sampled bank rows, on the GPU's order
        rows = rng.choice(n, size=min(nsample, n), replace=False) if n else np.zeros(0, np.int64)
        tg = t_gpu[h, :n].astype(np.int64)
        if rows.size:
            rho_rows = od.phi_rowsum(bK[rows], bK, prm) - od.phi(np.zeros(1), prm)[0]
            np.testing.assert_allclose(before.rho[h, rows], rho_rows, rtol=1e-4, atol=1e-6)
            csorted = np.asarray(candK[h], np.float64)[pi[:kmax]]
            rep.crossing_near_ties += check_crossings(tg[rows], bK[rows], rho_rows, before.rho0[h, rows], csorted, prm)
            # projected density at k* on sampled rows that did not cross
            live = rows[tg[rows] > k] if k > 0 else rows
            if live.size:
                pr = od.projected_density(bK[live], od.phi_rowsum(bK[live], bK, prm) - od.phi(np.zeros(1), prm)[0],
                                          csorted, k, prm)
                np.testing.assert_allclose(rhoP_gpu[h, live], pr, rtol=1e-4, atol=1e-6)
        tl.append(tg)
        ns.append(n)
    ks_ref, _ = od.feasible_prefix(tl, ns, prm.M, kmax)
    assert ks_ref == k, f"k* {k} != prefix {ks_ref} on the GPU crossing times"
    for h, tg in zip(heads, tl):
        n = int(before.count[h])
        e = max(0, n + k - prm.M) if k > 0 else 0
        assert int(n_ev_gpu[h]) == e
        mand = (tg <= k) if k > 0 else np.zeros(n, bool)
        assert int(n_mand_gpu[h]) == int(mand.sum())
        new_n = int(after.count[h])
        assert new_n == n - e + k
        pi = order_gpu[h].astype(np.int64)
        new_toks = after.tok[h, :new_n]
        assert len(set(new_toks.tolist())) == new_n, "duplicate token in bank"
        old = before.tok[h, :n]
        keep = np.isin(old, new_toks)
        ev = ~keep
        assert int(ev.sum()) == e and np.all(ev[mand])
        # completion = densest non-crossed states on the GPU's projected density (ties: lower token)
        rp = rhoP_gpu[h, :n].astype(np.float64)
        rest_ev = ev & ~mand
        rest_kp = keep & ~mand
        if rest_ev.any() and rest_kp.any():
            lo_i = np.lexsort((old[rest_ev], -rp[rest_ev]))[-1]
            worst_ev = (rp[rest_ev][lo_i], old[rest_ev][lo_i])
            hi_i = np.lexsort((old[rest_kp], -rp[rest_kp]))[0]
            best_kp = (rp[rest_kp][hi_i], old[rest_kp][hi_i])
            assert (worst_ev[0] > best_kp[0]) or (worst_ev[0] == best_kp[0] and worst_ev[1] < best_kp[1]), \
                "eviction completion is not the densest set"
        adm = tok[pi[:k]]
        assert set(adm.tolist()) | set(old[keep].tolist()) == set(new_toks.tolist())
        # exact K/V pairing of every live row
        cpos = {int(t): i for i, t in enumerate(tok.tolist())}
        opos = {int(t): i for i, t in enumerate(old.tolist())}
        for i, t in enumerate(new_toks.tolist()):
            if t in opos:
                j = opos[t]
                assert np.array_equal(after.K[h, i], before.K[h, j]) and np.array_equal(after.V[h, i], before.V[h, j])
                assert after.rho0[h, i] == before.rho0[h, j]
            else:
                j = cpos[t]
                assert np.array_equal(after.K[h, i], np.asarray(candK[h][j], np.float64))
                assert np.array_equal(after.V[h, i], np.asarray(candV[h][j], np.float64))
        # densities of sampled rows of the new bank
        nK = after.K[h, :new_n]
        rows = rng.choice(new_n, size=min(nsample, new_n), replace=False)
        rd = od.phi_rowsum(nK[rows], nK, prm) - od.phi(np.zeros(1), prm)[0]
        np.testing.assert_allclose(after.rho[h, rows], rd, rtol=1e-4, atol=1e-6)
        isnew = ~np.isin(new_toks[rows], old)
        np.testing.assert_allclose(after.rho0[h, rows][isnew], rd[isnew], rtol=1e-4, atol=1e-6)
        rep.admitted.append(k)
        rep.evicted.append(e)
    return rep
