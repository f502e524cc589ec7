"""Device-side conditions of kvbank_update (status bits, never a trap).

A head's bank holds no more than M pairs (DensityKV paper summary, appendix
B.1, online bank update): a count outside [0, M] is read clamped and reported
with KVB_DEV_COUNT.  A key with a non-finite squared norm has no Soft-Riesz
density (Method, Soft-Riesz density): KVB_DEV_NONFINITE, with every access
still inside the head's slices."""
import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, frame_tokens
from oracle import density as od

import gpu_common as gc
from _parity import GpuBank

pytestmark = pytest.mark.gpu

KVB_DEV_NONFINITE, KVB_DEV_COUNT = 1, 2


def _cold(wl, prm):
    """Layer with its bank after the first update of the tiny stream."""
    gen = LayerGen(wl, 0, 0)
    lc = gc.layer_for(wl, prm)
    gc.run_update(lc, gen, wl, prm, wl.bank_updates[0], list(range(wl.H)), replay=False)
    return gen, lc


def _update(lc, gen, wl, frames, candK=None):
    import torch
    import kv_cache_compression_head_amd as kb
    t0, t1 = frames
    cK = gen.keys_all(range(t0, t1)) if candK is None else candK
    cV = gen.values_all(range(t0, t1))
    ctok = frame_tokens(wl, t0, t1)
    kdt = gc.kv_dtype(wl)
    lc.out.status.zero_()
    D, s, o = lc.score(gc.dev(cK, kdt), gc.dev_i32(ctok), kb.KVLayout())
    lc.update(gc.dev(cK, kdt), gc.dev(cV, kdt), gc.dev_i32(ctok), D, o, kb.KVLayout())
    torch.cuda.synchronize()
    return int(lc.out.status.cpu()[0])


def _prm(wl):
    return od.Params(M=wl.M, tau=wl.tau, sigma=wl.sigma, eps=wl.eps, p=wl.p)


def test_count_above_capacity_is_clamped_and_reported():
    import torch
    wl = WORKLOADS["tiny"]
    prm = _prm(wl)
    gc.banner("status: bank count M + 1 on head 0, -3 on head 1")
    gen, lc = _cold(wl, prm)
    snap = [t.clone() for t in (lc.bank.K, lc.bank.V, lc.bank.tok, lc.bank.rho0, lc.bank.rho)]
    # reference: the same update from the clamped counts, given in range
    ref_gen, ref = _cold(wl, prm)
    # the clamped head 0 reads M rows (the slots past the cold count hold the
    # allocation's contents): both layers hold identical data in every slot
    for t, s in zip((ref.bank.K, ref.bank.V, ref.bank.tok, ref.bank.rho0, ref.bank.rho), snap):
        t.copy_(s)
    ref.bank.count.copy_(torch.tensor([wl.M, 0], dtype=torch.int32))
    lc.bank.count.copy_(torch.tensor([wl.M + 1, -3], dtype=torch.int32))
    st_ref = _update(ref, ref_gen, wl, wl.bank_updates[1])
    st = _update(lc, gen, wl, wl.bank_updates[1])
    assert st_ref & KVB_DEV_COUNT == 0
    assert st & KVB_DEV_COUNT, f"status {st:#x}"
    a, b = GpuBank.read(lc.bank), GpuBank.read(ref.bank)
    assert np.all(a.count <= wl.M) and np.all(a.count >= 0)
    assert np.array_equal(a.count, b.count)
    for h in range(wl.H):
        n = int(a.count[h])
        assert np.array_equal(a.tok[h, :n], b.tok[h, :n])
        assert np.array_equal(a.K[h, :n], b.K[h, :n]) and np.array_equal(a.V[h, :n], b.V[h, :n])
        assert np.array_equal(a.rho[h, :n], b.rho[h, :n]) and np.array_equal(a.rho0[h, :n], b.rho0[h, :n])
    assert int(lc.out.k_star.cpu()[0]) == int(ref.out.k_star.cpu()[0])


def test_count_out_of_range_without_candidates():
    """N = 0 writes the segment table only: the bank segment is clamped to M
    rows and the count is reported."""
    import torch
    import kv_cache_compression_head_amd as kb
    wl = WORKLOADS["tiny"]
    prm = _prm(wl)
    gen, lc = _cold(wl, prm)
    lc.bank.count.copy_(torch.tensor([wl.M + 5, 7], dtype=torch.int32))
    lc.out.status.zero_()
    lc.update(None, None, None, None, None, kb.KVLayout())
    torch.cuda.synchronize()
    assert int(lc.out.status.cpu()[0]) & KVB_DEV_COUNT
    segs = lc.segments()
    assert segs[0][0][2] == wl.M and segs[1][0][2] == 7


def test_nonfinite_candidate_key_is_reported():
    wl = WORKLOADS["tiny"]
    prm = _prm(wl)
    gc.banner("status: a NaN element in one candidate key of head 1")
    gen, lc = _cold(wl, prm)
    t0, t1 = wl.bank_updates[1]
    cK = gen.keys_all(range(t0, t1)).copy()
    cK[1, 5, 3] = np.nan
    st = _update(lc, gen, wl, (t0, t1), candK=cK)
    assert st & KVB_DEV_NONFINITE, f"status {st:#x}"
    a = GpuBank.read(lc.bank)
    assert np.all(a.count <= wl.M) and np.all(a.count >= 0)


def test_nonfinite_only_in_dead_bank_rows_is_not_reported():
    """Rows at or past a head's count hold no state: whatever they hold is
    not a key of the bank."""
    import torch
    wl = WORKLOADS["tiny"]
    prm = _prm(wl)
    gen, lc = _cold(wl, prm)
    n = int(lc.bank.count.cpu()[0])
    assert n < wl.M
    lc.bank.K[0, n:].fill_(float("inf"))
    st = _update(lc, gen, wl, wl.bank_updates[1])
    assert st & KVB_DEV_NONFINITE == 0, f"status {st:#x}"
    # a live row with an infinite element is reported
    gen, lc = _cold(wl, prm)
    lc.bank.K[1, 0, 0] = float("inf")
    st = _update(lc, gen, wl, wl.bank_updates[1])
    assert st & KVB_DEV_NONFINITE, f"status {st:#x}"
