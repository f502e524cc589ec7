"""Pins of the oracle's memory-key re-rotation (DensityKV supplementary,
"Post-RoPE Attention Geometry")."""
import numpy as np

from kvsynth import WORKLOADS, LayerGen
from oracle import rope


def test_generator_keys_turned_back_to_coordinate_zero():
    """Keys the generator writes at temporal coordinate t, turned back by t,
    are the generator's keys at coordinate 0 (exact in float64: the
    generator's pre-RoPE keys rotated without rounding)."""
    for name in ("tiny", "480p"):
        wl = WORKLOADS[name]
        gen = LayerGen(wl, 0, 0)
        pre = gen.prerope_keys(0, [3, 4])                     # [2, F, d] float64
        for t in (1, 5, 17):
            at_t = gen._rotate(pre, [t, t]).reshape(-1, wl.d)
            at_0 = gen._rotate(pre, [0, 0]).reshape(-1, wl.d)
            back = rope.rerotate_temporal(at_t, np.full(at_t.shape[0], t))
            np.testing.assert_allclose(back, at_0, rtol=0, atol=1e-11 * np.abs(at_0).max())


def test_identity_inverse_and_invariants():
    rng = np.random.default_rng(0)
    for d in (64, 128):
        K = rng.normal(size=(50, d))
        t = rng.integers(0, 30, size=50)
        nt = rope.temporal_pairs(d)
        assert nt == d // 2 - 2 * (d // 6)
        np.testing.assert_array_equal(rope.rerotate_temporal(K, np.zeros(50)), K)
        R = rope.rerotate_temporal(K, t)
        # spatial pairs untouched, norms and per-pair norms kept
        np.testing.assert_array_equal(R[:, 2 * nt:], K[:, 2 * nt:])
        np.testing.assert_allclose(np.linalg.norm(R, axis=1), np.linalg.norm(K, axis=1), rtol=1e-14)
        pr = R[:, :2 * nt].reshape(50, nt, 2)
        pk = K[:, :2 * nt].reshape(50, nt, 2)
        np.testing.assert_allclose(np.linalg.norm(pr, axis=2), np.linalg.norm(pk, axis=2), rtol=1e-13)
        # turning by t then by -t is the identity
        np.testing.assert_allclose(rope.rerotate_temporal(R, -t), K, atol=1e-12)
        # keys of one coordinate keep their inner products
        same = rope.rerotate_temporal(K[:10], np.full(10, 7))
        np.testing.assert_allclose(same @ same.T, K[:10] @ K[:10].T, atol=1e-10)


def test_first_pair_turns_by_t_radians():
    """The first temporal pair has frequency base^0 = 1: (1, 0) at
    coordinate t comes back to (cos -t, sin -t) turned by t, i.e. (1, 0)
    maps to (cos t, -sin t)."""
    K = np.zeros((1, 64))
    K[0, 0] = 1.0
    R = rope.rerotate_temporal(K, np.array([2.0]))
    np.testing.assert_allclose(R[0, :2], [np.cos(2.0), -np.sin(2.0)], rtol=1e-15)


def test_window_advance_wraps_and_writes_new_rows():
    rng = np.random.default_rng(1)
    H, cap, d, F = 2, 10, 64, 4
    rk, rv = rng.normal(size=(H, cap, d)), rng.normal(size=(H, cap, d))
    nk, nv = rng.normal(size=(H, 8, d)), rng.normal(size=(H, 8, d))
    ck, cv, rk2, rv2 = rope.window_advance(rk, rv, 6, 8, F, 3, nk, nv)
    slots = [6, 7, 8, 9, 0, 1, 2, 3]
    for j, s in enumerate(slots):
        t = 3 + j // F
        np.testing.assert_allclose(ck[:, j], np.stack([rope.rerotate_temporal(rk[h, s:s + 1], [t])[0]
                                                       for h in range(H)]))
        np.testing.assert_array_equal(cv[:, j], rv[:, s])
        np.testing.assert_array_equal(rk2[:, s], nk[:, j])
        np.testing.assert_array_equal(rv2[:, s], nv[:, j])
    np.testing.assert_array_equal(rk2[:, 4:6], rk[:, 4:6])
