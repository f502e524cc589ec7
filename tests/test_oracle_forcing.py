"""Pins of the fp64 Forcing-KV oracle."""
import numpy as np
import pytest

from oracle import forcing as of
from oracle.attention import attention


def test_cosine_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    Hd, T, F, d = 3, 4, 10, 16
    hist = rng.normal(size=(Hd, T * F, d))
    nxt = rng.normal(size=(Hd, F, d))
    s = of.segment_scores(hist, nxt, F, seg_len=5)
    chain = np.concatenate([hist, nxt], axis=1).transpose(1, 0, 2).reshape(T + 1, F, Hd * d)
    cos = torch.nn.functional.cosine_similarity(torch.from_numpy(chain[:-1]), torch.from_numpy(chain[1:]), dim=-1)
    ref = cos.reshape(T, 2, 5).mean(dim=2).reshape(-1).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-13)


def test_identical_frames_score_one_and_are_dropped_first():
    rng = np.random.default_rng(1)
    Hd, T, F, d = 2, 5, 8, 8
    hist = rng.normal(size=(Hd, T * F, d))
    hist[:, 2 * F:3 * F] = hist[:, 3 * F:4 * F]        # frame 2 == frame 3
    s = of.segment_scores(hist, rng.normal(size=(Hd, F, d)), F, seg_len=F)
    assert s[2] == pytest.approx(1.0, abs=1e-14)
    kept = of.bottomk(s, 0.8)                          # keep 4 of 5
    assert 2 not in kept.tolist() and kept.tolist() == sorted(kept.tolist())


def test_retention_extremes():
    rng = np.random.default_rng(2)
    s = rng.normal(size=12)
    assert of.bottomk(s, 1.0).tolist() == list(range(12))
    assert of.bottomk(s, 0.0).tolist() == []
    assert of.keep_count(0.7, 12) == 8 and of.keep_count(0.33, 6) == 1 and of.keep_count(0.3, 6) == 1


def test_bottomk_ties_lower_index_first():
    s = np.array([0.5, 0.1, 0.5, 0.1, 0.9])
    assert of.bottomk(s, 0.6).tolist() == [0, 1, 3]


def test_r1_dynamic_head_is_full_attention():
    rng = np.random.default_rng(3)
    T, F, d = 6, 8, 16
    hist = rng.normal(size=(1, T * F, d))
    histV = rng.normal(size=(T * F, d))
    s = of.segment_scores(hist, rng.normal(size=(1, F, d)), F, seg_len=4)
    rows = of.kept_token_rows(of.bottomk(s, 1.0), F, 4)
    assert rows.tolist() == list(range(T * F))
    Q = rng.normal(size=(5, d))
    np.testing.assert_allclose(attention(Q, hist[0][rows], histV[rows]), attention(Q, hist[0], histV), rtol=1e-13)


def test_static_rows_match_transition_formula():
    """Section 3.3: for chunk i with C frames of F tokens the transition frame
    is token range [(iC-1)F, iCF).  With history frames 1..12 (sink 0 kept
    separately) and chunk i = 13/C... we index from the history start."""
    C, F = 3, 7
    for i in range(1, 6):
        hist_start_frame = 1
        T = i * C - hist_start_frame            # history frames 1 .. iC-1
        rows = of.static_rows(T, F)
        absolute = rows + hist_start_frame * F
        assert absolute.tolist() == list(range((i * C - 1) * F, i * C * F))


def test_per_frame_bottomk():
    """Section 3.4 as printed: each frame keeps floor(r n) of its n
    segments, the lowest scores (ties to the lower index).  One frame is the
    global BottomK; r = 1 keeps all, r = 0 none; n = 1 with r < 1 keeps
    none (the degenerate case of one segment per frame)."""
    rng = np.random.default_rng(3)
    n = 6
    s = rng.uniform(size=5 * n)
    for r in (0.3, 0.33, 0.5, 0.99):
        kept = of.bottomk_per_frame(s, r, n)
        k = int(np.floor(r * n))
        assert len(kept) == 5 * k
        for t in range(5):
            mine = [i for i in kept if t * n <= i < (t + 1) * n]
            assert len(mine) == k
            rest = [i for i in range(t * n, (t + 1) * n) if i not in mine]
            if mine and rest:
                assert max(s[mine]) <= min(s[rest])
    np.testing.assert_array_equal(of.bottomk_per_frame(s[:n], 0.5, n), of.bottomk(s[:n], 0.5))
    assert of.bottomk_per_frame(s, 1.0, n).tolist() == list(range(5 * n))
    assert of.bottomk_per_frame(s, 0.0, n).size == 0
    assert of.bottomk_per_frame(s, 0.9, 1).size == 0
    # ties: equal scores keep the lower index
    tie = np.array([0.5, 0.5, 0.1, 0.5, 0.2, 0.5])
    assert of.bottomk_per_frame(tie, 0.5, 6).tolist() == [0, 2, 4]


def test_attention_mass_closed_form_and_brute_force():
    """Section 3.2 masses.  Equal logits (Q = 0) spread every query's weight
    evenly: A_region = Lq * |region| / Lkv.  A_total is the query count.
    A per-query Python loop agrees; so does attention with one-hot values."""
    rng = np.random.default_rng(0)
    Lq, d = 7, 16
    region = np.array([1] * 4 + [0] * 10 + [2] * 4 + [3] * 6)
    K = rng.normal(size=(region.size, d))
    m = of.attention_mass(np.zeros((Lq, d)), K, region)
    np.testing.assert_allclose(m, [Lq * np.sum(region == r) / region.size for r in range(4)], rtol=1e-14)
    Q = rng.normal(size=(Lq, d)) * 2
    m = of.attention_mass(Q, K, region)
    assert abs(m.sum() - Lq) < 1e-12
    brute = np.zeros(4)
    for q in range(Lq):
        e = [np.exp(sum(Q[q, i] * K[k, i] for i in range(d)) / 4.0) for k in range(region.size)]
        z = sum(e)
        for k in range(region.size):
            brute[region[k]] += e[k] / z
    np.testing.assert_allclose(m, brute, rtol=1e-12)
    onehot = np.eye(4)[region]
    np.testing.assert_allclose(attention(Q, K, onehot).sum(axis=0), m, rtol=1e-12)


def test_head_score_and_label():
    """score = (A_gen + A_trans) / (A_total - A_sink), static when > alpha
    (strict, as in the formula)."""
    assert of.head_score(np.array([1.0, 5.0, 1.0, 3.0])) == 4.0 / 5.0
    assert not of.head_is_static(np.array([1.0, 5.0, 1.0, 3.0]), 0.8)
    assert of.head_is_static(np.array([0.5, 5.0, 1.0, 3.5]), 0.8)
    # sink mass cancels out: the same ratio whatever the sink holds
    assert of.head_score(np.array([1.0, 0.0, 1.0, 3.0])) == of.head_score(np.array([1.0, 9.0, 1.0, 3.0]))
