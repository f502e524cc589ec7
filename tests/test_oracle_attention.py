"""Pins of the fp64 attention oracle: textbook per-row loop and torch's
scaled_dot_product_attention in float64 on the CPU."""
import math

import numpy as np
import pytest

from oracle.attention import attention


def _textbook(Q, K, V):
    out = np.zeros((Q.shape[0], V.shape[1]))
    d = Q.shape[1]
    for i in range(Q.shape[0]):
        s = [float(np.dot(Q[i], K[j])) / math.sqrt(d) for j in range(K.shape[0])]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for j in range(K.shape[0]):
            out[i] += (w[j] / z) * V[j]
    return out


def test_attention_textbook_tiny():
    rng = np.random.default_rng(0)
    Q, K, V = rng.normal(size=(48, 64)), rng.normal(size=(128, 64)), rng.normal(size=(128, 64))
    np.testing.assert_allclose(attention(Q, K, V), _textbook(Q, K, V), rtol=1e-12, atol=1e-13)


def test_attention_against_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    Q, K, V = rng.normal(size=(200, 128)) * 2, rng.normal(size=(333, 128)) * 2, rng.normal(size=(333, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None]).numpy()[0]
    np.testing.assert_allclose(attention(Q, K, V, block=64), ref, rtol=1e-11, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    V = rng.normal(size=(10, 8))
    Q = rng.normal(size=(3, 8))
    # identical keys: uniform weights -> mean of the values
    K = np.tile(rng.normal(size=(1, 8)), (10, 1))
    np.testing.assert_allclose(attention(Q, K, V), np.tile(V.mean(0), (3, 1)), rtol=1e-13)
    # one key: output is that value
    np.testing.assert_allclose(attention(Q, K[:1], V[:1]), np.tile(V[0], (3, 1)), rtol=0, atol=0)
    # permutation of KV rows leaves the output unchanged
    K2 = rng.normal(size=(10, 8))
    p = rng.permutation(10)
    np.testing.assert_allclose(attention(Q, K2[p], V[p]), attention(Q, K2, V), rtol=1e-13)
