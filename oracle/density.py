"""DensityKV per-head token banks in float64 (oracle; test infrastructure only).

Page: "DensityKV: Density-Guided KV Cache Compression for Long Video
Generation" (paper summary).  Sections used:

* Method, "Soft-Riesz Density" and appendix B.1: a regularised inverse-power
  interaction of the squared post-RoPE key distance, with bandwidth sigma,
  decay p and softening eps; the density of a state is the sum of its
  interactions with the other states of the same (layer, head) bank.
* Method, "Online Density-Constrained Bank Update" and appendix B.1 "Online
  Bank Update": candidates ordered by mean-normalised insertion disturbance
  (lower first); the largest prefix length k that every head of the layer can
  admit; each bank state's density may grow to at most tau times its frozen
  insertion baseline; evictions take the states that cross that bound, then
  the densest, until capacity is released; co-admitted states set their
  baselines together; values stay paired with their keys.
* Appendix D: defaults M = 9,360, tau = 2.0, sigma = 8; appendix E: eps = 1,
  p = 2, the candidate order, baseline, eviction and prefix ablations.

Readings where the page is silent (each is listed in the design notes):

* phi(d2) = (eps + d2 / sigma^2) ** (-p / 2)   (Riesz 1/r^p on the softened distance)
* the self term is excluded from a state's density; the density counts bank
  states only (not sink, window or rejected candidates)
* disturbance D(c) = sum over bank states of phi(c, b); delta = D / mean D over
  the head's candidates (0 when the bank is empty or the mean is 0); order is
  ascending (delta, token id), per head
* for prefix length k: projected density rho'(k) = rho + sum over the first k
  candidates of phi; a state crosses when rho'(k) > tau * rho0 (strict; never
  when tau is infinite); eviction count e(k) = max(0, n + k - M); k is
  feasible when every density head has |crossed| <= e(k) and k <= min(N, M);
  k = 0 (admit nothing, evict nothing) is always feasible
* eviction set = crossed states plus the highest projected densities among the
  rest (ties: lower token id first) until e(k*) states are chosen
* admitted states get rho0 = their density in the new bank; survivors keep rho0

Policy variants (the page's appendix E ablations; Params fields, defaults
are the method above):

* order "source": candidates in spatiotemporal source order, read as
  ascending token id (frame, then row-major position), instead of by delta
* baseline "refresh": after every update each state's baseline is its
  density in the new bank (instead of frozen insertion-time baselines)
* eviction "densest": the e(k*) states with the highest projected density
  (ties: lower token id), crossed or not; "oldest": the crossed states, then
  ascending token id (source-order completion)
* prefix "head": every density head takes its own largest feasible k
  instead of the layer's shared one
* fill_below_capacity: a prefix length k with n + k <= M needs no density
  check and evicts nothing (a reading of where the growth bound binds; the
  page's default gates at every occupancy)

Parity pins (tests/test_oracle_density.py): closed-form densities on collinear
keys, permutation and rotation invariance, the A.1 logit-gap bound, FIFO
reduction at p = 0 and tau = inf, full admission when capacity exceeds the
history, top-e-by-density eviction at tau = inf, the duplicate-key invariant,
a hand-computed admission example under tests/golden/, and agreement of the
blocked prefix-sum tier with a from-scratch brute-force tier.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

# Row blocks of the pairwise sums are independent: with more than one worker
# they are computed side by side in threads (BLAS then single-threaded per
# block, and blocks small enough to give every worker a few).  Each row is
# still the same fp64 sum over the same columns in the same order; only the
# BLAS rounding order of the dot products may differ (by ~1e-16 relative).
_WORKERS = 1


def set_workers(n: int) -> None:
    """Threads used for the row blocks of phi_rowsum, density and
    crossing_times (1: serial)."""
    global _WORKERS
    _WORKERS = max(1, int(n))


def _map_blocks(fn, starts) -> None:
    starts = list(starts)
    if _WORKERS <= 1 or len(starts) <= 1:
        for i in starts:
            fn(i)
        return
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), cf.ThreadPoolExecutor(max_workers=_WORKERS) as ex:
        for _ in ex.map(fn, starts):
            pass


@dataclasses.dataclass(frozen=True)
class Params:
    M: int
    tau: float = 2.0
    sigma: float = 8.0
    eps: float = 1.0
    p: float = 2.0
    # policy variants (see the module header); defaults are the method
    order: str = "delta"             # "delta" | "source"
    baseline: str = "frozen"         # "frozen" | "refresh"
    eviction: str = "threshold"      # "threshold" | "densest" | "oldest"
    prefix: str = "shared"           # "shared" | "head"
    fill_below_capacity: bool = False


# ---------------------------------------------------------------------------
# interaction and density
# ---------------------------------------------------------------------------

def phi(d2: np.ndarray, prm: Params) -> np.ndarray:
    """Soft-Riesz interaction of squared distances: (eps + d2/sigma^2)^(-p/2)."""
    base = prm.eps + np.asarray(d2, dtype=np.float64) / (prm.sigma * prm.sigma)
    if prm.p == 0.0:
        return np.ones_like(base)
    return base ** (-prm.p / 2.0)


def sqdist_direct(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """sum_i (a_i - b_i)^2 for every row pair, from the differences themselves."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    out = np.empty((A.shape[0], B.shape[0]), dtype=np.float64)
    step = max(1, int(4_000_000 // max(1, B.shape[0] * max(1, A.shape[1]))))
    for i in range(0, A.shape[0], step):
        diff = A[i:i + step, None, :] - B[None, :, :]
        out[i:i + step] = np.einsum("mnd,mnd->mn", diff, diff)
    return out


def sqdist_gram(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Same quantity through ||a||^2 + ||b||^2 - 2 a.b in float64 (large shapes)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    na = np.einsum("md,md->m", A, A)
    nb = np.einsum("nd,nd->n", B, B)
    return np.maximum(na[:, None] + nb[None, :] - 2.0 * (A @ B.T), 0.0)


def sqdist(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    if A.shape[0] * B.shape[0] * max(1, A.shape[1]) <= 2_000_000:
        return sqdist_direct(A, B)
    return sqdist_gram(A, B)


def phi_matrix(A: np.ndarray, B: np.ndarray, prm: Params) -> np.ndarray:
    return phi(sqdist(A, B), prm)


def _row_block(ncols: int, nrows: int = 0) -> int:
    step = max(1, int(16_000_000 // max(1, ncols)))
    if _WORKERS > 1 and nrows > 0:
        step = min(step, max(64, -(-nrows // (3 * _WORKERS))))
    return step


def phi_rowsum(A: np.ndarray, B: np.ndarray, prm: Params) -> np.ndarray:
    """For each row a of A: sum over rows b of B of phi(a, b)."""
    out = np.zeros(A.shape[0], dtype=np.float64)
    if B.shape[0] == 0:
        return out
    step = _row_block(B.shape[0], A.shape[0])

    def block(i):
        out[i:i + step] = phi_matrix(A[i:i + step], B, prm).sum(axis=1)
    _map_blocks(block, range(0, A.shape[0], step))
    return out


def density(K: np.ndarray, prm: Params) -> np.ndarray:
    """rho_x = sum over y != x in the same set of phi(||x - y||^2)."""
    n = K.shape[0]
    out = np.zeros(n, dtype=np.float64)
    if n == 0:
        return out
    step = _row_block(n, n)

    def block(i):
        blk = phi_matrix(K[i:i + step], K, prm)
        rows = np.arange(blk.shape[0])
        blk[rows, i + rows] = 0.0
        out[i:i + step] = blk.sum(axis=1)
    _map_blocks(block, range(0, n, step))
    return out


# ---------------------------------------------------------------------------
# bank state
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class HeadBank:
    """One (layer, head) bank: exact K/V rows, token ids and frozen baselines.

    Xd: density descriptor rows when they are not the keys themselves (the
    appendix E descriptor ablation: pre-RoPE keys, or [K; V]); X is the
    descriptor the density uses (Xd, else K)."""
    tok: np.ndarray      # int64 [n]
    K: np.ndarray        # float64 [n, d]
    V: np.ndarray        # float64 [n, d]
    rho0: np.ndarray     # float64 [n]
    Xd: Optional[np.ndarray] = None   # float64 [n, dx]

    @staticmethod
    def empty(d: int, dx: Optional[int] = None) -> "HeadBank":
        return HeadBank(np.zeros(0, np.int64), np.zeros((0, d)), np.zeros((0, d)), np.zeros(0),
                        None if dx is None else np.zeros((0, dx)))

    @property
    def n(self) -> int:
        return int(self.tok.shape[0])

    @property
    def X(self) -> np.ndarray:
        return self.K if self.Xd is None else self.Xd

    def sorted_by_tok(self) -> "HeadBank":
        o = np.argsort(self.tok, kind="stable")
        return HeadBank(self.tok[o], self.K[o], self.V[o], self.rho0[o], None if self.Xd is None else self.Xd[o])


# ---------------------------------------------------------------------------
# stages (one head)
# ---------------------------------------------------------------------------

def disturbance(bankK: np.ndarray, candK: np.ndarray, prm: Params):
    """Insertion disturbance D(c) and its mean-normalised form delta(c)."""
    D = phi_rowsum(np.asarray(candK, np.float64), np.asarray(bankK, np.float64), prm)
    mean = D.mean() if D.size else 0.0
    delta = D / mean if (bankK.shape[0] > 0 and mean > 0.0) else np.zeros_like(D)
    return D, delta


def candidate_order(delta: np.ndarray, tok: np.ndarray, order: str = "delta") -> np.ndarray:
    """Permutation sorting candidates by ascending (delta, token id), or by
    token id alone for the source-order variant."""
    if order == "source":
        return np.argsort(np.asarray(tok, np.int64), kind="stable").astype(np.int64)
    return np.lexsort((np.asarray(tok, np.int64), np.asarray(delta, np.float64))).astype(np.int64)


def crossing_times(bankK, rho, rho0, candK_sorted, prm: Params, at: Sequence[np.ndarray] = ()):
    """First prefix length k at which each bank state crosses tau * rho0.

    Returns (t, vals) where t[b] in [0, kmax] is the smallest k with
    rho'_b(k) = rho_b + sum_{j<k} phi(b, c_j) > tau * rho0_b, or kmax + 1 when
    the state never crosses within kmax = len(candK_sorted).  The running sum
    follows the candidate order.  For each per-row array of prefix lengths in
    ``at`` the projected densities rho'_b(at[b]) are returned in ``vals``.
    """
    n, kmax = bankK.shape[0], candK_sorted.shape[0]
    t = np.full(n, kmax + 1, dtype=np.int64)
    vals = [np.empty(n, dtype=np.float64) for _ in at]
    step = _row_block(kmax + 1, n)
    finite = math.isfinite(prm.tau)

    def block(i):
        m = min(step, n - i)
        blk = np.empty((m, kmax + 1), dtype=np.float64)
        blk[:, 0] = 0.0
        if kmax:
            np.cumsum(phi_matrix(bankK[i:i + m], candK_sorted, prm), axis=1, out=blk[:, 1:])
        blk += rho[i:i + m, None]
        if finite:
            crossed = blk > (prm.tau * rho0[i:i + m])[:, None]
            anyc = crossed.any(axis=1)
            tt = t[i:i + m]
            tt[anyc] = np.argmax(crossed[anyc], axis=1)
        for a, o in zip(at, vals):
            o[i:i + m] = blk[np.arange(m), np.asarray(a)[i:i + m]]
    _map_blocks(block, range(0, n, step))
    return t, vals


def projected_density(bankK, rho, candK_sorted, k: int, prm: Params) -> np.ndarray:
    """rho'_b(k) = rho_b + sum over the first k ordered candidates of phi(b, c)."""
    return rho + phi_rowsum(bankK, np.asarray(candK_sorted, np.float64)[:k], prm)


def feasible_head(t: np.ndarray, n: int, M: int, kmax: int, fill_below_capacity: bool = False) -> np.ndarray:
    """feasible[k], k in [0, kmax], for one head: |V(k)| = #{b : t_b <= k} <=
    e(k) = max(0, n + k - M); with fill_below_capacity every k with
    n + k <= M is feasible as well.  k = 0 is always feasible."""
    ks = np.arange(kmax + 1)
    hist = np.bincount(np.minimum(t, kmax + 1), minlength=kmax + 2)[: kmax + 1]
    Vk = np.cumsum(hist)
    feas = Vk <= np.maximum(0, n + ks - M)
    if fill_below_capacity:
        feas |= n + ks <= M
    feas[0] = True
    return feas


def feasible_prefix(ts: Sequence[np.ndarray], ns: Sequence[int], M: int, kmax: int,
                    fill_below_capacity: bool = False):
    """Largest k in [0, kmax] feasible for every density head (see
    feasible_head).  Returns (kstar, feasible[k] boolean array)."""
    feas = np.ones(kmax + 1, dtype=bool)
    for t, n in zip(ts, ns):
        feas &= feasible_head(t, n, M, kmax, fill_below_capacity)
    return int(np.nonzero(feas)[0].max()), feas


def eviction_set(proj_k: np.ndarray, crossed: np.ndarray, tok: np.ndarray, e: int,
                 eviction: str = "threshold") -> np.ndarray:
    """Boolean mask of e evicted states.

    "threshold": the crossed states, then the highest projected densities
    (ties: lower token id first); "oldest": the crossed states, then
    ascending token id; "densest": the e highest projected densities
    (ties: lower token id), crossed or not.  The crossed set never exceeds e
    at a feasible k.
    """
    n = proj_k.shape[0]
    ev = np.zeros(n, bool) if eviction == "densest" else np.array(crossed, dtype=bool, copy=True)
    r = e - int(ev.sum())
    if r < 0:
        raise ValueError("crossed set exceeds the eviction count")
    if r > 0:
        rest = np.nonzero(~ev)[0]
        o = np.argsort(tok[rest], kind="stable") if eviction == "oldest" else np.lexsort((tok[rest], -proj_k[rest]))
        ev[rest[o[:r]]] = True
    assert int(ev.sum()) == e and n >= e
    return ev


# ---------------------------------------------------------------------------
# one layer update (all heads)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class UpdateInfo:
    kstar: int                               # shared prefix (the largest per-head one with prefix "head")
    kmax: int
    D: List[Optional[np.ndarray]]
    delta: List[Optional[np.ndarray]]
    order: List[Optional[np.ndarray]]
    t: List[Optional[np.ndarray]]
    rho: List[Optional[np.ndarray]]          # density before the update
    proj: List[Optional[np.ndarray]]         # projected density at k*
    crossed: List[Optional[np.ndarray]]      # mask over old bank rows at k*
    evicted: List[Optional[np.ndarray]]      # mask over old bank rows
    e: List[int]
    feasible: Optional[np.ndarray]
    kstar_h: List[int] = dataclasses.field(default_factory=list)   # prefix applied per head


def update_layer(banks: List[Optional[HeadBank]], candK: np.ndarray, candV: np.ndarray,
                 cand_tok: np.ndarray, prm: Params, heads: Optional[Sequence[int]] = None,
                 order: Optional[Sequence[np.ndarray]] = None, kstar: Optional[int] = None, candX=None):
    """Apply one admission/eviction update to the density heads of a layer.

    ``banks[h]`` is None for heads that do not keep a density bank; ``heads``
    restricts the update to those heads (default: every head with a bank).
    ``order`` may supply a per-head candidate permutation (stage replay) and
    ``kstar`` a prefix length to apply instead of the computed one.
    ``candX``: the candidates' density descriptors [H][N][dx] when they are
    not the keys (the banks then carry theirs in HeadBank.Xd).
    Returns (new_banks, UpdateInfo).  Candidate rows are [H][N][d].
    """
    Xc_all = candK if candX is None else candX
    H = len(banks)
    heads = [h for h in range(H) if banks[h] is not None] if heads is None else list(heads)
    N = int(cand_tok.shape[0])
    kmax = min(N, prm.M)
    tok = np.asarray(cand_tok, np.int64)
    info = UpdateInfo(0, kmax, [None] * H, [None] * H, [None] * H, [None] * H, [None] * H,
                      [None] * H, [None] * H, [None] * H, [0] * H, None)
    for h in heads:
        b = banks[h]
        D, delta = disturbance(b.X, Xc_all[h], prm)
        pi = candidate_order(delta, tok, prm.order) if order is None else np.asarray(order[h], np.int64)
        rho = density(b.X, prm)
        t, _ = crossing_times(b.X, rho, b.rho0, np.asarray(Xc_all[h], np.float64)[pi[:kmax]], prm)
        info.D[h], info.delta[h], info.order[h], info.t[h], info.rho[h] = D, delta, pi, t, rho
    fill = prm.fill_below_capacity
    if prm.prefix == "head":
        kh = {h: int(np.nonzero(feasible_head(info.t[h], banks[h].n, prm.M, kmax, fill))[0].max()) for h in heads}
        if kstar is not None:
            kh = {h: int(kstar[h]) if np.ndim(kstar) else int(kstar) for h in heads}
        info.kstar = max(kh.values()) if kh else 0
    else:
        ks, feas = feasible_prefix([info.t[h] for h in heads], [banks[h].n for h in heads], prm.M, kmax, fill)
        info.feasible = feas
        info.kstar = ks if kstar is None else int(kstar)
        kh = {h: info.kstar for h in heads}
    info.kstar_h = [kh.get(h, 0) for h in range(H)]
    new = list(banks)
    for h in heads:
        b = banks[h]
        k = kh[h]
        e = max(0, b.n + k - prm.M)
        proj_k = projected_density(b.X, info.rho[h], np.asarray(Xc_all[h], np.float64)[info.order[h]], k, prm)
        # no density check below capacity in the fill variant: nothing crossed counts
        gated = k > 0 and not (fill and b.n + k <= prm.M)
        crossed = (info.t[h] <= k) if gated else np.zeros(b.n, bool)
        ev = eviction_set(proj_k, crossed, b.tok, e, prm.eviction) if k > 0 else np.zeros(b.n, bool)
        info.proj[h], info.crossed[h], info.evicted[h], info.e[h] = proj_k, crossed, ev, e
        adm = info.order[h][:k]
        keep = ~ev
        K2 = np.concatenate([b.K[keep], np.asarray(candK[h], np.float64)[adm]])
        V2 = np.concatenate([b.V[keep], np.asarray(candV[h], np.float64)[adm]])
        tok2 = np.concatenate([b.tok[keep], tok[adm]])
        X2 = None if candX is None else np.concatenate([b.X[keep], np.asarray(candX[h], np.float64)[adm]])
        rho_new = density(K2 if X2 is None else X2, prm)
        if prm.baseline == "refresh":
            rho0 = rho_new
        else:
            rho0 = np.concatenate([b.rho0[keep], rho_new[keep.sum():]])
        new[h] = HeadBank(tok2, K2, V2, rho0, X2)
    return new, info


def update_layer_brute(banks: List[Optional[HeadBank]], candK, candV, cand_tok, prm: Params,
                       heads: Optional[Sequence[int]] = None, candX=None):
    """Same update recomputing every prefix length from scratch (tiny inputs).

    For each k the projected density of every bank state is summed directly
    over the first k ordered candidates, with distances from explicit
    differences; no running sums, no Gram form.  Policy variants follow the
    same Params fields, each written out with plain sorts and loops.
    Returns (new_banks, kstar per head, orders).  candX: candidate
    descriptors when they are not the keys (banks carry theirs in Xd).
    """
    Xc_all = candK if candX is None else candX
    H = len(banks)
    heads = [h for h in range(H) if banks[h] is not None] if heads is None else list(heads)
    N = int(cand_tok.shape[0])
    kmax = min(N, prm.M)
    tok = np.asarray(cand_tok, np.int64)
    orders, rhos = {}, {}
    for h in heads:
        b = banks[h]
        Dmat = phi(sqdist_direct(np.asarray(Xc_all[h], np.float64), b.X), prm)
        D = Dmat.sum(axis=1)
        mean = D.mean() if D.size else 0.0
        delta = D / mean if (b.n > 0 and mean > 0) else np.zeros(N)
        if prm.order == "source":
            orders[h] = np.array(sorted(range(N), key=lambda c: tok[c]), dtype=np.int64)
        else:
            orders[h] = np.array(sorted(range(N), key=lambda c: (delta[c], tok[c])), dtype=np.int64)
        Bm = phi(sqdist_direct(b.X, b.X), prm)
        np.fill_diagonal(Bm, 0.0)
        rhos[h] = Bm.sum(axis=1)

    def projected(h, k):
        b = banks[h]
        if k == 0:
            return rhos[h].copy()
        adm = np.asarray(Xc_all[h], np.float64)[orders[h][:k]]
        return rhos[h] + phi(sqdist_direct(b.X, adm), prm).sum(axis=1)

    def crossed_at(h, k):
        b = banks[h]
        below = prm.fill_below_capacity and b.n + k <= prm.M
        if k == 0 or below or not math.isfinite(prm.tau):
            return np.zeros(b.n, bool)
        return projected(h, k) > prm.tau * b.rho0

    def ok(h, k):
        if k == 0 or (prm.fill_below_capacity and banks[h].n + k <= prm.M):
            return True
        return int(crossed_at(h, k).sum()) <= max(0, banks[h].n + k - prm.M)

    if prm.prefix == "head":
        kst = {h: max(k for k in range(kmax + 1) if ok(h, k)) for h in heads}
    else:
        shared = max(k for k in range(kmax + 1) if all(ok(h, k) for h in heads))
        kst = {h: shared for h in heads}
    new = list(banks)
    for h in heads:
        b = banks[h]
        k = kst[h]
        c, pr = crossed_at(h, k), projected(h, k)
        e = max(0, b.n + k - prm.M)
        if prm.eviction == "densest":
            ev = np.zeros(b.n, bool)
        else:
            ev = c.copy()
        rest = [i for i in range(b.n) if not ev[i]]
        if prm.eviction == "oldest":
            rest = sorted(rest, key=lambda i: b.tok[i])
        else:
            rest = sorted(rest, key=lambda i: (-pr[i], b.tok[i]))
        for i in rest[: e - int(ev.sum())]:
            ev[i] = True
        adm = orders[h][:k]
        keep = ~ev
        K2 = np.concatenate([b.K[keep], np.asarray(candK[h], np.float64)[adm]])
        V2 = np.concatenate([b.V[keep], np.asarray(candV[h], np.float64)[adm]])
        tok2 = np.concatenate([b.tok[keep], tok[adm]])
        X2 = None if candX is None else np.concatenate([b.X[keep], np.asarray(candX[h], np.float64)[adm]])
        Bm = phi(sqdist_direct(K2 if X2 is None else X2, K2 if X2 is None else X2), prm)
        np.fill_diagonal(Bm, 0.0)
        rnew = Bm.sum(axis=1)
        rho0 = rnew if prm.baseline == "refresh" else np.concatenate([b.rho0[keep], rnew[keep.sum():]])
        new[h] = HeadBank(tok2, K2, V2, rho0, X2)
    return new, kst, orders


def bank_payload_bytes(L: int, H: int, M: int, dk: int, dv: int, elem_bytes: int = 2) -> int:
    """Bytes of the exact K/V payload of L layers x H heads x M states."""
    return L * H * M * (dk + dv) * elem_bytes
