"""Pins for oracle/hadamard.py: the Sylvester matrix, orthogonality, the fixed
fp32 schedule on exactly representable inputs, norm preservation and the
dot-product identity q.k = (Hq).(Hk)."""

import numpy as np
import scipy.linalg

from oracle import hadamard as hd


def test_butterflies_build_sylvester_matrix():
    # apply the unnormalized butterflies to e_0..e_127 (exact integers)
    H = hd.fwht128_unnormalized_exact(np.eye(128, dtype=np.int64)).T
    assert np.array_equal(H, hd.sylvester(128))
    assert np.array_equal(H, scipy.linalg.hadamard(128))
    # H H^T = D I with D = 128 (exact), and H is symmetric
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, H.T)
    # entry rule (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(H, (-1) ** pc)


def test_normalization_constant():
    assert hd.C32.view(np.uint32) == 0x3DB504F3
    assert hd.C32 == np.float32(1.0 / np.sqrt(128.0))
    assert hd.C32 == np.float32(np.sqrt(np.float32(2))) / np.float32(16)


def test_fp32_schedule_exact_on_integers():
    # small integers: every butterfly sum is exact in fp32, so the result must
    # be the exact product rounded once by the final scaling
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1000, size=(64, 128))
    y = hd.fwht128_f32(x.astype(np.float16))
    exact = (x @ scipy.linalg.hadamard(128)).astype(np.float32)
    assert np.array_equal(y, exact * hd.C32)


def test_norm_involution_and_dot_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((256, 128)).astype(np.float16)
    y = hd.fwht128_f32(x)
    xf = x.astype(np.float64)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(xf, axis=1), rtol=1e-5)
    back = hd.fwht128_f32(y.astype(np.float32))
    assert np.allclose(back, xf, atol=1e-4, rtol=1e-5)
    # fp64 rotation agrees with the fp32 schedule to fp32 rounding
    assert np.allclose(hd.rotate_f64(xf), y, atol=1e-5, rtol=1e-5)
    q = rng.standard_normal((8, 128))
    k = rng.standard_normal((8, 128))
    lhs = np.sum(hd.rotate_f64(q) * hd.rotate_f64(k), axis=1)
    assert np.allclose(lhs, np.sum(q * k, axis=1), rtol=1e-12, atol=1e-12)
    # an outlier spreads over every coordinate
    e = np.zeros(128)
    e[17] = 100.0
    r = hd.rotate_f64(e)
    assert np.allclose(np.abs(r), 100.0 / np.sqrt(128))
