"""CPU checks of the stage-replay checker itself (tests/_parity.py): a
bank update laid out the way the device lays it out, built from the
oracle's own decisions, passes; the same update with one planted mistake
(a wrong admitted row, a density off by more than the tolerance, a wrong
eviction, a wrong prefix length) fails."""
import copy

import numpy as np
import pytest

from oracle import density as od
from _parity import GpuBank, replay_update


def _layout(H, M, d):
    g = GpuBank(np.full((H, M), -1, np.int64), np.zeros((H, M, d)), np.zeros((H, M, d)), np.zeros((H, M)),
                np.zeros((H, M)), np.zeros(H, np.int64))
    return g


def _device_like_update(seed=3, H=3, M=24, N=14, d=8, tau=1.4):
    """A small layer update and its outputs in the device's layout: survivors
    keep their slots, admitted rows fill freed slots in ascending order, then
    append after the old occupancy."""
    rng = np.random.default_rng(seed)
    prm = od.Params(M=M, tau=tau)
    banks = []
    before = _layout(H, M, d)
    for h in range(H):
        n = M if h == 0 else int(rng.integers(M // 2, M))
        K = rng.normal(size=(n, d)) * 5
        V = rng.normal(size=(n, d))
        tok = rng.permutation(1000)[:n].astype(np.int64)
        rho = od.density(K, prm)
        rho0 = rho * rng.uniform(1.0, 1.2, size=n)
        banks.append(od.HeadBank(tok, K, V, rho0))
        before.tok[h, :n], before.K[h, :n], before.V[h, :n] = tok, K, V
        before.rho0[h, :n], before.rho[h, :n], before.count[h] = rho0, rho, n
    cK = rng.normal(size=(H, N, d)) * 5
    cV = rng.normal(size=(H, N, d))
    ctok = (5000 + rng.permutation(N)).astype(np.int32)
    new, info = od.update_layer(banks, cK, cV, ctok, prm)
    after = copy.deepcopy(before)
    t_dev = np.zeros((H, M), np.int64)
    rhoP = np.zeros((H, M))
    for h in range(H):
        b, nb = banks[h], new[h]
        n = b.n
        t_dev[h, :n] = info.t[h]
        rhoP[h, :n] = np.where(info.crossed[h], before.rho[h, :n], info.proj[h])
        freed = list(np.nonzero(info.evicted[h])[0])
        slots = freed + list(range(n, n + info.kstar - len(freed)))
        surv = np.nonzero(~info.evicted[h])[0]
        rows = {int(t): i for i, t in enumerate(nb.tok.tolist())}
        rho_new = od.density(nb.K, prm)
        for s_ in surv:
            i = rows[int(b.tok[s_])]
            after.rho[h, s_] = rho_new[i]
        for j, c in enumerate(info.order[h][:info.kstar]):
            s_ = slots[j]
            i = rows[int(ctok[c])]
            after.tok[h, s_], after.K[h, s_], after.V[h, s_] = ctok[c], cK[h, c], cV[h, c]
            after.rho[h, s_], after.rho0[h, s_] = rho_new[i], rho_new[i]
        after.count[h] = n - info.e[h] + info.kstar
    n_mand = np.array([int(info.crossed[h].sum()) for h in range(H)])
    n_ev = np.array(info.e)
    order = np.stack(info.order).astype(np.int64)
    args = dict(before=before, after=after, candK=cK, candV=cV, cand_tok=ctok, D_gpu=np.stack(info.D),
                delta_gpu=np.stack(info.delta), order_gpu=order, t_gpu=t_dev, rhoP_gpu=rhoP,
                kstar_gpu=np.array([info.kstar]), n_mand_gpu=n_mand, n_ev_gpu=n_ev, prm=prm, heads=list(range(H)))
    return args, info


def test_device_like_update_passes():
    args, info = _device_like_update()
    assert info.kstar > 0 and max(info.e) > 0, "the case must admit and evict"
    rep = replay_update(**args, workers=2)
    assert rep.kstar == info.kstar
    # the new bank's from-scratch densities are returned for reuse
    rep2 = replay_update(**args, workers=1, rho_before={h: np.asarray(args["before"].rho[h, :args["before"].count[h]])
                                                          for h in args["heads"]})
    assert rep2.kstar == rep.kstar


@pytest.mark.parametrize("mistake", ["admitted_v", "density", "eviction", "kstar", "order"])
def test_planted_mistake_fails(mistake):
    args, info = _device_like_update()
    a = args["after"]
    if mistake == "admitted_v":
        h = 0
        s_ = int(np.nonzero(~np.isin(a.tok[h, :a.count[h]], args["before"].tok[h]))[0][0])
        a.V[h, s_, 0] += 1.0
    elif mistake == "density":
        a.rho[1, 0] *= 1.01
    elif mistake == "eviction":
        # keep an evicted state instead of an admitted one in head 0
        h = 0
        ev = info.evicted[h]
        assert ev.any()
        j = int(np.nonzero(ev)[0][0])
        s_ = int(np.nonzero(~np.isin(a.tok[h, :a.count[h]], args["before"].tok[h]))[0][0])
        a.tok[h, s_] = args["before"].tok[h, j]
    elif mistake == "kstar":
        args["kstar_gpu"] = np.array([info.kstar - 1])
    elif mistake == "order":
        o = args["order_gpu"]
        o[2, [0, -1]] = o[2, [-1, 0]]
    with pytest.raises(AssertionError):
        replay_update(**args, workers=2)


def test_kstar_heads_use_every_head():
    """The shared prefix is checked from every density head's crossing times
    even when only a subset is replayed in fp64."""
    args, info = _device_like_update()
    rep = replay_update(**{**args, "heads": [1]}, kstar_heads=[0, 1, 2], workers=1)
    assert rep.kstar == info.kstar
