"""Pins for oracle/codebook.py (TBQ4: Lloyd-Max levels of N(0, 1/sqrt(128))
and the norm + index block quantizer, [trefon] "Jak 4-bitowemu cache to
uchodzi: najpierw obrót").

The levels are pinned by the Lloyd-Max optimality conditions evaluated by
numerical integration (independent of the closed-form cell means the oracle
iterates), by symmetry, by the classical 16-level table for the unit normal
(Max, 1960) and by its mean squared error; the quantizer by brute-force
nearest level, its boundary rule and its edge cases."""

import math

import numpy as np
import pytest
import scipy.integrate
import scipy.stats

from oracle import codebook as cb
from oracle import sizes

SIG = 1.0 / math.sqrt(128.0)


def test_levels_are_symmetric_sorted_and_scaled():
    c = cb.centroids()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    # the unit-normal levels scaled by sigma = 1/sqrt(128)
    assert np.allclose(cb.lloyd_max_normal(16) * SIG, c.astype(np.float64), rtol=1e-6, atol=0)


def test_lloyd_max_conditions_by_integration():
    lv = cb.lloyd_max_normal(16)                     # unit normal, fp64
    b = np.concatenate([[-np.inf], (lv[:-1] + lv[1:]) / 2, [np.inf]])
    pdf = scipy.stats.norm.pdf
    for k in range(16):
        mass = scipy.integrate.quad(pdf, b[k], b[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        mom = scipy.integrate.quad(lambda x: x * pdf(x), b[k], b[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(mom / mass - lv[k]) < 1e-9, k


def test_classical_table_and_distortion():
    # Max (1960), 16-level quantizer for the unit normal: output levels
    published = [0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6181, 2.0690, 2.7326]
    lv = cb.lloyd_max_normal(16)
    assert np.allclose(lv[8:], published, atol=6e-5)
    b = np.concatenate([[-np.inf], (lv[:-1] + lv[1:]) / 2, [np.inf]])
    pdf = scipy.stats.norm.pdf
    mse = sum(scipy.integrate.quad(lambda x, c=lv[k]: (x - c) ** 2 * pdf(x), b[k], b[k + 1])[0]
              for k in range(16))
    # the table lists 0.009497; it was computed to about four digits (its
    # levels above agree to ~5e-5), the optimum evaluated here is 0.009501
    assert abs(mse - 0.009497) < 1e-5


def test_boundaries_are_fp32_midpoints():
    c = cb.centroids().astype(np.float64)
    b = cb.boundaries()
    assert b.dtype == np.float32 and b.shape == (15,)
    for k in range(15):
        m = (c[k] + c[k + 1]) / 2              # exact in fp64
        assert b[k] == np.float32(m)
        assert c[k] < b[k] < c[k + 1] or c[k] <= b[k] <= c[k + 1]
    assert b[7] == 0.0


def test_indices_are_the_nearest_level():
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((400, 128)) * rng.uniform(0.01, 30, (400, 1))).astype(np.float32)
    idx, n_h = cb.quant_tbq4(y)
    u = (y / n_h.astype(np.float32)[:, None]).astype(np.float64)
    c = cb.centroids().astype(np.float64)
    near = np.argmin(np.abs(u[..., None] - c), axis=-1)
    b = cb.boundaries().astype(np.float64)
    clear = np.min(np.abs(u[..., None] - b), axis=-1) > 1e-6      # away from a boundary
    assert clear.mean() > 0.99
    assert np.array_equal(idx[clear], near[clear])


def test_norm_definition_and_edges():
    e = np.zeros((1, 128), np.float32)
    e[0, 5] = 3.0
    assert cb.block_norm(e)[0] == np.float16(3.0)
    big = np.full((1, 128), 60000.0, np.float32)
    assert cb.block_norm(big)[0] == np.float16(65504)          # clamped, finite
    y = np.random.default_rng(4).standard_normal((64, 128)).astype(np.float32)
    ref = np.float16(np.float32(np.sqrt(np.sum(y.astype(np.float64) ** 2, axis=1))))
    assert np.array_equal(cb.block_norm(y), ref)
    # zero block: u = 0, index 7 (b_7 = 0 is not below 0), dequant zero
    idx, n_h = cb.quant_tbq4(np.zeros((2, 128), np.float32))
    assert np.all(idx == 7) and np.all(n_h == 0)
    assert np.all(cb.dequant_tbq4(idx, n_h) == 0)


def test_boundary_values_take_the_lower_level():
    b = cb.boundaries()
    n = np.float16(1.0)
    y = np.zeros((1, 128), np.float32)
    y[0, :15] = b                     # u = b_k exactly (n_h = 1 -> norm must be 1)
    y[0, 15] = np.sqrt(np.float32(1.0) - np.sum(b.astype(np.float64) ** 2)).astype(np.float32)
    idx, n_h = cb.quant_tbq4(y)
    assert n_h[0] == n                # the construction keeps the norm at 1
    assert list(idx[0, :15]) == list(range(15))


def test_dequant_and_round_trip():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((256, 128)).astype(np.float32)
    idx, n_h = cb.quant_tbq4(y)
    yh = cb.dequant_tbq4(idx, n_h)
    c = cb.centroids()
    assert np.array_equal(yh, (c[idx] * n_h.astype(np.float32)[:, None]).astype(np.float32))
    # between the outer levels, |u - c[idx]| <= half the gap of its two levels
    gap = np.max(np.diff(c.astype(np.float64)))
    u = y.astype(np.float64) / n_h.astype(np.float64)[:, None]
    inner = np.abs(u) < c[-1]
    err = np.abs(u - c[idx].astype(np.float64))
    assert np.all(err[inner] <= gap / 2 + 1e-6)
    # and the relative error of a block is what a 16-level Gaussian quantizer gives
    rel = np.linalg.norm(yh - y, axis=1) / np.linalg.norm(y, axis=1)
    assert 0.05 < np.mean(rel) < 0.15


def test_container_bits_per_value():
    assert sizes.block128_bytes_per_token_head() == 2 * 66
    assert 66 * 8 / 128 == 4.125
