"""Pins for oracle/attention.py: brute force on tiny inputs, special cases that
reduce to closed forms or a library routine, the key- and value-error algebra
of the nalar page, the sigma/sqrt(N) averaging claim of the troisinh page,
GQA = repeated-head MHA, and split-half RoPE."""

import math

import numpy as np
import pytest
import torch

from conftest import golden_kv
from oracle import attention as at

EX = golden_kv("page_size_examples.txt")


def brute(q, K, V, scale):
    """Pure-Python loops with math.exp and math.fsum (T <= 8)."""
    T, D = K.shape
    s = [math.fsum(q[d] * K[i, d] for d in range(D)) * scale for i in range(T)]
    m = max(s)
    e = [math.exp(v - m) for v in s]
    tot = math.fsum(e)
    return np.array([math.fsum(e[i] / tot * V[i, d] for i in range(T)) for d in range(D)])


@pytest.mark.parametrize("T", [1, 2, 3, 8])
def test_brute_force_tiny(T):
    rng = np.random.default_rng(T)
    q = rng.standard_normal((1, 1, 128))
    K = rng.standard_normal((1, T, 1, 128)) * 2
    V = rng.standard_normal((1, T, 1, 128))
    out = at.decode_f64(q, K, V)
    ref = brute(q[0, 0], K[0, :, 0], V[0, :, 0], 1 / math.sqrt(128))
    assert np.allclose(out[0, 0], ref, rtol=1e-13, atol=1e-14)


def test_special_cases():
    rng = np.random.default_rng(1)
    V = rng.standard_normal((1, 50, 1, 128))
    K = rng.standard_normal((1, 50, 1, 128))
    # one token: the output is that token's value
    out = at.decode_f64(rng.standard_normal((1, 1, 128)), K[:, :1], V[:, :1])
    assert np.allclose(out[0, 0], V[0, 0, 0], rtol=0, atol=1e-15)
    # zero query: uniform weights, the mean of the values
    out = at.decode_f64(np.zeros((1, 1, 128)), K, V)
    assert np.allclose(out[0, 0], V[0, :, 0].mean(axis=0), atol=1e-14)
    # a huge query: one-hot on the argmax score
    q = rng.standard_normal((1, 1, 128))
    out = at.decode_f64(q * 1e4, K, V)
    assert np.allclose(out[0, 0], V[0, np.argmax(K[0, :, 0] @ q[0, 0]), 0], atol=1e-12)


def test_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(2)
    B, Hq, Hkv, T = 2, 8, 2, 77
    q = rng.standard_normal((B, Hq, 128))
    K = rng.standard_normal((B, T, Hkv, 128))
    V = rng.standard_normal((B, T, Hkv, 128))
    out = at.decode_f64(q, K, V)
    qt = torch.from_numpy(q)[:, :, None, :]
    kt = torch.from_numpy(np.repeat(np.transpose(K, (0, 2, 1, 3)), Hq // Hkv, axis=1))
    vt = torch.from_numpy(np.repeat(np.transpose(V, (0, 2, 1, 3)), Hq // Hkv, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, T = 1, 8, 2, 33
    q = rng.standard_normal((B, Hq, 128))
    K = rng.standard_normal((B, T, Hkv, 128))
    V = rng.standard_normal((B, T, Hkv, 128))
    rep = lambda x: np.repeat(x, Hq // Hkv, axis=2)
    assert np.allclose(at.decode_f64(q, K, V), at.decode_f64(q, rep(K), rep(V)), atol=1e-15)


def test_key_error_shifts_score_by_projection():
    # k_i + e_i changes the score by exactly (q . e_i) / sqrt(D)
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128)
    k = rng.standard_normal((10, 128))
    e = rng.standard_normal((10, 128)) * 0.01
    s = k @ q / math.sqrt(128)
    s2 = (k + e) @ q / math.sqrt(128)
    assert np.allclose(s2 - s, e @ q / math.sqrt(128), rtol=1e-10, atol=1e-14)
    # an error orthogonal to q leaves the score unchanged
    e_perp = e[0] - (e[0] @ q) / (q @ q) * q
    assert abs((k[0] + e_perp) @ q - k[0] @ q) < 1e-12


def test_value_error_adds_weighted_sum():
    # with the probabilities fixed, v_i + r_i shifts the output by sum_i p_i r_i
    rng = np.random.default_rng(5)
    B, T = 1, 40
    q = rng.standard_normal((B, 1, 128))
    K = rng.standard_normal((B, T, 1, 128))
    V = rng.standard_normal((B, T, 1, 128))
    r = rng.standard_normal((B, T, 1, 128)) * 0.05
    p = at.softmax_f64(K[0, :, 0] @ q[0, 0] / math.sqrt(128))
    delta = at.decode_f64(q, K, V + r) - at.decode_f64(q, K, V)
    assert np.allclose(delta[0, 0], p @ r[0, :, 0], atol=1e-14)


def test_sigma_over_sqrt_n_averaging():
    # zero query (uniform p), iid value errors of std sigma: the output error is
    # about sigma / sqrt(N); the page quotes ~300x at N = 100k
    N = EX["averaging_n"]
    sigma = 0.1
    rng = np.random.default_rng(6)
    r = rng.standard_normal((1, N, 1, 128)) * sigma
    V = np.zeros_like(r)
    K = rng.standard_normal((1, N, 1, 128))
    delta = at.decode_f64(np.zeros((1, 1, 128)), K, V + r)[0, 0]
    rms = np.sqrt(np.mean(delta ** 2))
    expected = sigma / math.sqrt(N)
    # 128 samples of a chi-square: 3-sigma band on the RMS
    assert abs(rms / expected - 1) < 3 * math.sqrt(1 / (2 * 128))
    assert abs(math.sqrt(N) / EX["averaging_factor_approx"] - 1) < 0.06


def test_rope_properties():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 128))
    base = 500000.0
    assert np.array_equal(at.rope_f64(x, np.zeros(5), base), x)          # R(0) = I
    y = at.rope_f64(x, np.arange(5) * 1000 + 3, base)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # split-half pairs (j, j+64) rotate like complex numbers x_j + i x_{j+64}
    pos = np.array([12345.0] * 5)
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * pos[:, None] * at.rope_freqs(base)[None, :])
    y2 = at.rope_f64(x, pos, base)
    assert np.allclose(y2[:, :64], z.real, atol=1e-12) and np.allclose(y2[:, 64:], z.imag, atol=1e-12)
    # scores depend only on the position difference
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    s1 = at.rope_f64(q[None], [1000], base) @ at.rope_f64(k[None], [400], base).T
    s2 = at.rope_f64(q[None], [131072 + 1000], base) @ at.rope_f64(k[None], [131072 + 400], base).T
    assert abs(s1.item() - s2.item()) < 1e-9
    # theta_j = base^(-2j/128)
    assert at.rope_freqs(base)[0] == 1.0
    assert math.isclose(at.rope_freqs(base)[32], base ** -0.5, rel_tol=1e-15)
