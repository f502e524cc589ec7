"""Checks of the seeded input generator (shared by oracle and HIP path)."""
import numpy as np
import pytest

from kvsynth import WORKLOADS, LayerGen, round_bf16, bf16_bits, rope_split, frame_tokens, head_labels


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).normal(size=10000).astype(np.float32) * 7
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]   # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)
    bits = bf16_bits(round_bf16(x))
    assert bits.dtype == np.uint16


def test_determinism_and_random_access():
    wl = WORKLOADS["tiny"]
    a = LayerGen(wl, 0, 0).keys(1, [3, 4], [0, 0])
    g = LayerGen(wl, 0, 0)
    g.keys(1, [9])
    b = g.keys(1, [3, 4], [0, 0])
    np.testing.assert_array_equal(a, b)
    c = LayerGen(wl, 1, 0).keys(1, [3, 4], [0, 0])
    assert not np.array_equal(a, c)


def test_rope_preserves_norm_and_memory_convention():
    wl = WORKLOADS["tiny"]
    g = LayerGen(wl, 0, 0)
    pre = g.prerope_keys(0, [2])[0]
    k_mem = g._rotate(pre[None], [0])[0]
    k_loc = g._rotate(pre[None], [5])[0]
    np.testing.assert_allclose(np.linalg.norm(k_mem, axis=1), np.linalg.norm(pre, axis=1), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(k_loc, axis=1), np.linalg.norm(pre, axis=1), rtol=1e-12)
    # t only moves the temporal pairs
    nt, nh, nw = rope_split(wl.d)
    np.testing.assert_array_equal(k_mem[:, 2 * nt:], k_loc[:, 2 * nt:])
    assert rope_split(128) == (22, 21, 21)


def test_ar1_drift_correlation():
    wl = WORKLOADS["480p"]
    g = LayerGen(wl, 0, 0)
    dr = g._drift_upto(0, 30)
    a, b = dr[10:29].reshape(-1), dr[11:30].reshape(-1)
    assert np.corrcoef(a, b)[0, 1] == pytest.approx(0.95, abs=0.01)


def test_tokens_and_labels():
    wl = WORKLOADS["480p"]
    t = frame_tokens(wl, 7, 22)
    assert t.shape[0] == 23400 and t[0] == 7 * 1560 and t[-1] == 22 * 1560 - 1
    lab = head_labels(WORKLOADS["fkv480p"], 0)
    assert (lab == 1).sum() == 6 and (lab == 2).sum() == 6
    assert np.array_equal(lab, head_labels(WORKLOADS["fkv480p"], 0))
