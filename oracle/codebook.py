"""Lloyd-Max codebook of TBQ4 and its block quantizer (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the page fixes ([trefon] "Jak 4-bitowemu cache to uchodzi: najpierw
obrót"; the 66-byte container in "Przykład: model 27B przy 262K"):
  * every 128-value block is rotated (randomized Walsh-Hadamard) first, after
    which its coordinates look nearly normal;
  * the 16 centroids are Lloyd-Max levels fitted to N(0, 1/sqrt(128)), so a
    block is a 4-bit index per value plus one fp16 norm;
  * decode reads a value as centroid x norm.

Readings (the page prints no centroids, no norm definition and no rounding):
  * N(0, 1/sqrt(128)) names the standard deviation sigma = 1/sqrt(128), the
    spread of one coordinate of a random unit vector in 128 dimensions.
  * Lloyd-Max levels of a density are the fixed point of Lloyd's iteration:
    every boundary is the midpoint of its two neighbouring levels and every
    level is the mean of the density over its cell.  For the normal density
    the cell mean has a closed form, sigma (phi(a) - phi(b)) / (Phi(b) - Phi(a))
    for the cell (a sigma, b sigma].  Iterated in fp64 from evenly spaced
    levels until no level moves by 1e-14 (the fixed point is unique for a
    log-concave density; the levels then sit within ~3e-13 of it, far inside
    the fp32 rounding margins of every level).  Used as fp32:
    c_k = fl32(level_k).
  * Decision boundaries in fp32: b_k = fl32((fl64(c_k) + fl64(c_k+1)) / 2)
    (the exact midpoint of two fp32 levels, rounded once), k = 0 .. 14.
  * The norm is the Euclidean norm of the rotated block:
    n = fl32(sqrt(sum y_i^2)) with the sum and the square root in fp64, then
    n_h = fp16(min(n, 65504)).  (fp64 sums of 128 fp32 squares differ between
    summation orders only in their last bits, which the two roundings that
    follow absorb.)
  * u_i = fl32(y_i / n_h) (u_i = 0 where n_h == 0); index = the number of
    boundaries strictly below u_i, so a value on a boundary takes the lower
    level, and values beyond the outer levels take the outer index.
  * Dequantized value: fl32(n_h * c_index).
"""

import functools
import math

import numpy as np

F16 = np.float16
F32 = np.float32
D = 128
SIGMA = 1.0 / math.sqrt(128.0)


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cell_mass(a, b):
    """Phi(b) - Phi(a) for the standard normal, accurate in both tails."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / math.sqrt(2.0)) - math.erfc(b / math.sqrt(2.0)))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / math.sqrt(2.0)) - math.erfc(-a / math.sqrt(2.0)))
    return 1.0 - 0.5 * math.erfc(-a / math.sqrt(2.0)) - 0.5 * math.erfc(b / math.sqrt(2.0))


def lloyd_max_normal(levels=16, sigma=1.0, tol=1e-14, iters=10000):
    """Lloyd-Max levels (ascending, fp64) of N(0, sigma^2).

    Lloyd's iteration on the unit normal from evenly spaced levels on
    [-3, 3], until no level moves by tol or more (the error is then about 25
    tol: the iteration contracts by ~0.965 a step), then scaled by sigma."""
    c = [(-3.0 + 6.0 * (k + 0.5) / levels) for k in range(levels)]
    for _ in range(iters):
        b = [-math.inf] + [0.5 * (c[k] + c[k + 1]) for k in range(levels - 1)] + [math.inf]
        new = []
        for k in range(levels):
            lo, hi = b[k], b[k + 1]
            plo = 0.0 if lo == -math.inf else _phi(lo)
            phi_ = 0.0 if hi == math.inf else _phi(hi)
            new.append((plo - phi_) / _cell_mass(lo, hi))
        moved = max(abs(x - y) for x, y in zip(new, c))
        c = new
        if moved < tol:
            break
    return np.array(c, dtype=np.float64) * sigma


@functools.lru_cache(maxsize=None)
def _centroids_cached():
    return tuple(float(x) for x in lloyd_max_normal(16, SIGMA).astype(F32))


def centroids():
    """The 16 TBQ4 levels as float32 (ascending)."""
    return np.array(_centroids_cached(), dtype=F32)


def boundaries(c32=None):
    """The 15 fp32 decision boundaries between consecutive fp32 levels."""
    c = centroids() if c32 is None else np.asarray(c32, dtype=F32)
    c64 = c.astype(np.float64)
    return ((c64[:-1] + c64[1:]) / 2.0).astype(F32)


def block_norm(y):
    """n_h over the last axis (128): fp16(min(fl32(sqrt(sum y^2) in fp64), 65504))."""
    y64 = np.asarray(y, dtype=F32).astype(np.float64)
    n = np.sqrt(np.sum(y64 * y64, axis=-1)).astype(F32)
    return np.minimum(n, F32(65504.0)).astype(F16)


def quant_tbq4(y):
    """(indices uint8 0..15, n_h fp16) of float32 rotated blocks (last axis 128)."""
    y = np.asarray(y, dtype=F32)
    if not np.all(np.isfinite(y)):
        raise ValueError("oracle inputs must be finite")
    if y.shape[-1] != D:
        raise ValueError("block length must be 128")
    n_h = block_norm(y)
    nx = n_h.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (y / nx).astype(F32)
    u = np.where(nx == 0, F32(0), u)
    b = boundaries()
    idx = np.zeros(y.shape, np.uint8)
    for k in range(15):
        idx += (u > b[k]).astype(np.uint8)
    return idx, n_h


def dequant_tbq4(idx, n_h):
    """fl32(n_h * c[idx])."""
    c = centroids()
    return (c[np.asarray(idx, dtype=np.int64)] * np.asarray(n_h, dtype=F16).astype(F32)[..., None]).astype(F32)
