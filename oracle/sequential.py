"""Sequential within-block admission in float64 (oracle; test infrastructure only).

Page: "DensityKV: Density-Guided KV Cache Compression for Long Video
Generation" (paper summary), appendix E, within-block competition: instead
of admitting the largest feasible prefix of a block at once, candidates are
gated one at a time, so that every admitted candidate takes part in the
density of the candidates after it.  The page calls this a mechanism
comparison, not a one-factor ablation, and gives no further rule; the
readings below keep every other part of the method (Method, "Online
Density-Constrained Bank Update"; appendix B.1, "Online Bank Update"):

* the order is the method's: per head, ascending (delta, token id), scored
  once against the bank before the block (or token order for the source-order
  variant)
* step j offers every density head its j-th candidate c.  Each live state x
  of the head (a bank state or a candidate admitted at an earlier step) has
  the projected density rho'_x = rho_x + phi(x, c); it crosses when
  rho'_x > tau * rho0_x.  The eviction count is e = max(0, n + 1 - M) for the
  head's occupancy n
* the step is feasible when every density head has |crossed| <= e (the heads
  share the decision, as they share the prefix length in the method; with
  the per-head prefix variant each head decides alone); with the
  fill-below-capacity variant a step with n + 1 <= M is feasible unchecked
* a feasible step admits c in every head: the eviction set is the crossed
  states, then the highest rho' (ties: lower token id) up to e (or the
  densest-only / oldest-first variants), over every live state; survivors
  take rho_x = rho'_x - sum over the evicted y of phi(x, y); c enters with
  its density among the states live after the eviction
* baselines: the page's update rule lets only growth from later blocks count
  against a baseline, and co-admitted candidates set theirs together.  So a
  candidate admitted during the block has no baseline until the block ends
  (it cannot cross, though it adds density and takes capacity, and can be
  evicted as the densest); at the end every candidate of the block still in
  the bank takes rho0 = its density in the bank
* an infeasible step rejects c in every head and changes nothing
* after the last step, the refresh-baseline variant sets every live state's
  baseline to its density

A candidate admitted at one step can be evicted at a later one.  From an
empty bank every candidate of the first block is admitted, as with the
prefix method.  With one candidate per block the walk is the method's rule
for k <= 1.

Descriptors: the density is computed on descriptor rows X (post-RoPE keys by
default; pre-RoPE keys or [K; V] in the appendix E descriptor ablation),
given per bank state (HeadBank.X) and per candidate (candX); the attention
K/V rows are carried unchanged.

Parity pins (tests/test_oracle_sequential.py): the plain tier (incremental
densities from a pair matrix) against the brute tier (every density from
scratch at every step, from explicit differences) for every policy
combination; one candidate per block equals the prefix method; the FIFO
window at p = 0, tau = inf, token order and oldest-first eviction; the
density-growth invariant after every step; a hand-derived example under
tests/golden/.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

from .density import HeadBank, Params, candidate_order, disturbance, phi, phi_matrix, sqdist_direct


@dataclasses.dataclass
class SeqInfo:
    order: List[Optional[np.ndarray]]      # per head: candidate permutation
    admitted_steps: List[int]              # steps j admitted (shared decision: the same for every head)
    admitted_h: List[List[int]]            # per head: steps admitted (differs only with per-head decisions)
    evicted_h: List[List[int]]             # per head: token ids evicted, in step order
    n_final: List[int]


def _evict_pick(proj, crossed, tok, live, e, eviction):
    """Indices (into the state arrays) evicted at one admitted step."""
    if eviction == "densest":
        ev = []
    else:
        ev = [int(i) for i in np.nonzero(live & crossed)[0]]
    r = e - len(ev)
    if r < 0:
        raise ValueError("crossed set exceeds the eviction count")
    if r > 0:
        rest = [int(i) for i in np.nonzero(live)[0] if int(i) not in set(ev)]
        if eviction == "oldest":
            rest.sort(key=lambda i: tok[i])
        else:
            rest.sort(key=lambda i: (-proj[i], tok[i]))
        ev += rest[:r]
    return ev


def update_layer_sequential(banks: List[Optional[HeadBank]], candK, candV, cand_tok, prm: Params,
                            heads: Optional[Sequence[int]] = None, candX=None,
                            order: Optional[Sequence[np.ndarray]] = None):
    """Sequential density-gated admission of one block into the layer's
    density heads (plain tier: the pair interactions of each head's states
    precomputed once, densities maintained incrementally).  Returns
    (new_banks, SeqInfo).  candX: descriptor rows of the candidates
    [H][N][dx] (default: candK)."""
    H = len(banks)
    heads = [h for h in range(H) if banks[h] is not None] if heads is None else list(heads)
    N = int(np.asarray(cand_tok).shape[0])
    tok_c = np.asarray(cand_tok, np.int64)
    candX = candK if candX is None else candX
    per_head = prm.prefix == "head"
    finite = math.isfinite(prm.tau)
    info = SeqInfo([None] * H, [], [[] for _ in range(H)], [[] for _ in range(H)], [0] * H)
    st = {}
    for h in heads:
        b = banks[h]
        Xc = np.asarray(candX[h], np.float64)
        _, delta = disturbance(b.X, Xc, prm)
        pi = candidate_order(delta, tok_c, prm.order) if order is None else np.asarray(order[h], np.int64)
        info.order[h] = pi
        # states: the bank's n rows, then the N candidates
        X = np.concatenate([b.X, Xc])
        P = phi_matrix(X, X, prm)
        n0 = b.n
        live = np.zeros(n0 + N, bool)
        live[:n0] = True
        rho = np.zeros(n0 + N)
        Pb = P[:n0, :n0].copy()
        np.fill_diagonal(Pb, 0.0)
        rho[:n0] = Pb.sum(axis=1)
        rho0 = np.concatenate([b.rho0, np.zeros(N)])
        tok = np.concatenate([b.tok, tok_c])
        st[h] = dict(P=P, live=live, rho=rho, rho0=rho0, tok=tok, n=n0, n0=n0)

    def check(h, j):
        """(feasible, proj, crossed, e) of offering step j to head h."""
        s = st[h]
        c = s["n0"] + int(info.order[h][j])
        proj = s["rho"] + s["P"][c]
        e = max(0, s["n"] + 1 - prm.M)
        if prm.fill_below_capacity and s["n"] + 1 <= prm.M:
            return True, proj, np.zeros_like(s["live"]), 0
        crossed = (proj > prm.tau * s["rho0"]) & s["live"] if finite else np.zeros_like(s["live"])
        return int(crossed.sum()) <= e, proj, crossed, e

    def admit(h, j, proj, crossed, e):
        s = st[h]
        c = s["n0"] + int(info.order[h][j])
        ev = _evict_pick(proj, crossed, s["tok"], s["live"], e, prm.eviction)
        live = s["live"]
        upd = live.copy()
        rho = s["rho"]
        rho[upd] = proj[upd]
        for y in ev:
            live[y] = False
        for y in ev:
            rho[live] -= s["P"][y][live]
        # the candidate's density among the states now live; its baseline is
        # set when the block ends
        rc = float(s["P"][c][live].sum())
        live[c] = True
        rho[c] = rc
        s["rho0"][c] = math.inf
        s["n"] += 1 - len(ev)
        info.admitted_h[h].append(j)
        info.evicted_h[h].extend(int(s["tok"][y]) for y in ev)

    for j in range(N):
        res = {h: check(h, j) for h in heads}
        if per_head:
            for h in heads:
                if res[h][0]:
                    admit(h, j, *res[h][1:])
        else:
            if all(r[0] for r in res.values()):
                info.admitted_steps.append(j)
                for h in heads:
                    admit(h, j, *res[h][1:])
    new = list(banks)
    for h in heads:
        s, b = st[h], banks[h]
        n0 = s["n0"]
        keep = s["live"][:n0]
        adm = [n0 + int(info.order[h][j]) for j in info.admitted_h[h] if s["live"][n0 + int(info.order[h][j])]]
        idx_c = [a - n0 for a in adm]
        K2 = np.concatenate([b.K[keep], np.asarray(candK[h], np.float64)[idx_c]])
        V2 = np.concatenate([b.V[keep], np.asarray(candV[h], np.float64)[idx_c]])
        X2 = np.concatenate([b.X[keep], np.asarray(candX[h], np.float64)[idx_c]])
        tok2 = np.concatenate([b.tok[keep], tok_c[idx_c]])
        # the block's candidates take their baselines together, at the end
        rho0 = np.concatenate([s["rho0"][:n0][keep], s["rho"][adm]])
        if prm.baseline == "refresh":
            rho0 = np.concatenate([s["rho"][:n0][keep], s["rho"][adm]])
        new[h] = HeadBank(tok2, K2, V2, rho0, None if b.Xd is None and candX is candK else X2)
        info.n_final[h] = new[h].n
    return new, info


def _density_direct(X: np.ndarray, prm: Params) -> np.ndarray:
    if X.shape[0] == 0:
        return np.zeros(0)
    Pm = phi(sqdist_direct(X, X), prm)
    np.fill_diagonal(Pm, 0.0)
    return Pm.sum(axis=1)


def update_layer_sequential_brute(banks: List[Optional[HeadBank]], candK, candV, cand_tok, prm: Params,
                                  heads: Optional[Sequence[int]] = None, candX=None):
    """Same walk with no stored densities: at every step each head's
    projected densities are the densities of the tentative set (live states
    plus the offered candidate) computed from scratch from explicit
    differences, and the admitted candidate's baseline is its from-scratch
    density in the set left after the eviction (tiny inputs).  Returns
    (new_banks, admitted steps per head, orders)."""
    H = len(banks)
    heads = [h for h in range(H) if banks[h] is not None] if heads is None else list(heads)
    N = int(np.asarray(cand_tok).shape[0])
    tok_c = np.asarray(cand_tok, np.int64)
    candX = candK if candX is None else candX
    finite = math.isfinite(prm.tau)
    orders, cur = {}, {}
    for h in heads:
        b = banks[h]
        Xc = np.asarray(candX[h], np.float64)
        D = phi(sqdist_direct(Xc, b.X), prm).sum(axis=1)
        mean = D.mean() if D.size else 0.0
        delta = D / mean if (b.n > 0 and mean > 0) else np.zeros(N)
        if prm.order == "source":
            orders[h] = np.array(sorted(range(N), key=lambda c: tok_c[c]), dtype=np.int64)
        else:
            orders[h] = np.array(sorted(range(N), key=lambda c: (delta[c], tok_c[c])), dtype=np.int64)
        # live states as lists of (token, K, V, X, rho0)
        cur[h] = [(int(b.tok[i]), b.K[i], b.V[i], b.X[i], float(b.rho0[i])) for i in range(b.n)]
    adm = {h: [] for h in heads}

    def offer(h, j):
        c = int(orders[h][j])
        live = cur[h]
        n = len(live)
        e = max(0, n + 1 - prm.M)
        Xt = np.array([s[3] for s in live] + [np.asarray(candX[h][c], np.float64)])
        proj = _density_direct(Xt, prm)[:n]
        if prm.fill_below_capacity and n + 1 <= prm.M:
            crossed = [False] * n
            e = 0
        else:
            crossed = [finite and proj[i] > prm.tau * live[i][4] for i in range(n)]
        return sum(crossed) <= e, c, proj, crossed, e

    def apply(h, c, proj, crossed, e):
        live = cur[h]
        n = len(live)
        ev = [] if prm.eviction == "densest" else [i for i in range(n) if crossed[i]]
        rest = [i for i in range(n) if i not in ev]
        if prm.eviction == "oldest":
            rest.sort(key=lambda i: live[i][0])
        else:
            rest.sort(key=lambda i: (-proj[i], live[i][0]))
        ev += rest[: e - len(ev)]
        kept = [live[i] for i in range(n) if i not in ev]
        # no baseline until the block ends (inf: never crosses)
        kept.append((int(tok_c[c]), np.asarray(candK[h][c], np.float64), np.asarray(candV[h][c], np.float64),
                     np.asarray(candX[h][c], np.float64), math.inf))
        cur[h] = kept

    for j in range(N):
        res = {h: offer(h, j) for h in heads}
        if prm.prefix == "head":
            for h in heads:
                if res[h][0]:
                    apply(h, *res[h][1:])
                    adm[h].append(j)
        elif all(r[0] for r in res.values()):
            for h in heads:
                apply(h, *res[h][1:])
                adm[h].append(j)
    new = list(banks)
    for h in heads:
        live = cur[h]
        d = banks[h].K.shape[1]
        dx = banks[h].X.shape[1]
        tok2 = np.array([s[0] for s in live], np.int64)
        K2 = np.array([s[1] for s in live]).reshape(-1, d)
        V2 = np.array([s[2] for s in live]).reshape(-1, d)
        X2 = np.array([s[3] for s in live]).reshape(-1, dx)
        rho0 = np.array([s[4] for s in live])
        dens = _density_direct(X2, prm)
        # this block's candidates take their densities in the final bank
        rho0 = np.where(np.isinf(rho0), dens, rho0)
        if prm.baseline == "refresh":
            rho0 = dens
        new[h] = HeadBank(tok2, K2, V2, rho0, X2)
    return new, adm, orders
