"""Pins for oracle/quant.py: round-trip error bounds, brute-force nearest level,
invariants of the asymmetric and symmetric quantizers, dequant exactness."""

import itertools

import numpy as np
import pytest

from oracle import quant

F16, F32 = np.float16, np.float32
SLACK = 1 + 2.0 ** -20   # quotient rounding


def fp16_groups(rng, n, size, kind):
    if kind == "normal":
        x = rng.standard_normal((n, size))
    elif kind == "outlier":
        x = rng.standard_normal((n, size))
        x[:, 3] *= 20
    elif kind == "student":
        x = rng.standard_t(3, size=(n, size))
    elif kind == "tiny":      # fp16 subnormal range
        x = rng.standard_normal((n, size)) * 1e-6
    elif kind == "offset":    # narrow range far from zero
        x = 50 + rng.standard_normal((n, size)) * 1e-2
    elif kind == "signed_zero":
        x = np.where(rng.random((n, size)) < 0.5, -0.0, 0.0)
        x[:, 0] = 1.0
    return x.astype(F16)


KINDS = ["normal", "outlier", "student", "tiny", "offset", "signed_zero"]


@pytest.mark.parametrize("bits,kind", list(itertools.product([4, 3, 2], KINDS)))
def test_asym_roundtrip_bound_fp16_inputs(bits, kind):
    rng = np.random.default_rng([bits, KINDS.index(kind)])
    x = fp16_groups(rng, 2000, 32, kind).astype(F32)
    c, s, z = quant.quant_asym(x, bits, axis=-1)
    xh = quant.dequant_asym(c, s, z, axis=-1)
    err = np.abs(x.astype(np.float64) - xh)
    Q = 2 ** bits - 1
    sh = s.astype(np.float64)[:, None]
    bound = sh / 2 * SLACK
    # a normal fp16 scale is within 2^-11 of the exact step, so the range
    # [z, z + Q s_h] covers the group and the error is at most half a step
    normal = (s.astype(np.float64) >= 2.0 ** -14)[:, None] | (s == 0)[:, None]
    assert np.all((err <= bound + 1e-30) | ~normal)
    # a subnormal scale can be far from the exact step; then values past the
    # top level are clamped: the error is half a step plus the overshoot
    top = z.astype(np.float64)[:, None] + Q * sh
    over = np.maximum(0.0, x.astype(np.float64) - top)
    assert np.all(err <= bound + over + 1e-30)
    pos = s >= 2.0 ** -14
    # the min maps to 0 and the max to Q in every group with a nonzero scale
    assert np.all(c[pos].min(axis=1) == 0)
    assert np.all(c[pos].max(axis=1) == Q)
    # codes are monotone in x within a group
    order = np.argsort(x, axis=1, kind="stable")
    cs = np.take_along_axis(c, order, axis=1)
    assert np.all(np.diff(cs.astype(int), axis=1) >= 0)


def test_asym_fp32_inputs_bound():
    # Hadamard-rotated values are fp32: the zero point is fp16(min), so the bound
    # widens by |z_h - min|
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((5000, 32)) * 3).astype(F32)
    for bits in (4, 3, 2):
        c, s, z = quant.quant_asym(x, bits, axis=-1)
        xh = quant.dequant_asym(c, s, z, axis=-1)
        mn = x.min(axis=1).astype(np.float64)
        extra = np.abs(z.astype(np.float64) - mn)
        bound = (s.astype(np.float64) / 2 * SLACK + extra)[:, None]
        assert np.all(np.abs(x - xh) <= bound * (1 + 1e-6))


def test_asym_constant_and_zero_groups():
    x = np.full((4, 32), 3.25, F32)
    x[1] = 0.0
    x[2] = -0.0
    x[3] = -7.5
    c, s, z = quant.quant_asym(x, 4, axis=-1)
    assert np.all(c == 0) and np.all(s == 0)
    assert np.array_equal(quant.dequant_asym(c, s, z, axis=-1), x)
    # -0 is canonicalized to +0
    assert z.view(np.uint16)[2] == 0x0000
    # a group of mixed signed zeros: both parameters are +0 whatever min/max pick
    xz = np.zeros((2, 32), F32)
    xz[0, ::2] = -0.0
    xz[1, 1::3] = -0.0
    cz, sz, zz = quant.quant_asym(xz, 2, axis=-1)
    assert np.all(sz.view(np.uint16) == 0) and np.all(zz.view(np.uint16) == 0)
    assert np.all(cz == 0)


def test_asym_brute_force_nearest_level():
    # tiny groups: every code is the nearest of the 2^b levels z + k s (fp64),
    # unless two levels are (nearly) tied
    rng = np.random.default_rng(7)
    for bits in (4, 3, 2):
        Q = 2 ** bits - 1
        x = (rng.standard_normal((3000, 4)) * rng.uniform(0.1, 10, (3000, 1))).astype(F16).astype(F32)
        c, s, z = quant.quant_asym(x, bits, axis=-1)
        for g in range(x.shape[0]):
            sh, zh = float(s[g]), float(z[g])
            if sh == 0:
                assert np.all(c[g] == 0)
                continue
            levels = zh + sh * np.arange(Q + 1)
            for i in range(4):
                d = np.abs(levels - float(x[g, i]))
                best = np.argsort(d)
                if d[best[1]] - d[best[0]] < 1e-6 * sh:
                    continue
                assert c[g, i] == best[0], (g, i)


def test_kivi_group_axes():
    # keys: one range per channel over the 32 tokens; values: one range per
    # token over each 32-dim slice
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 128)).astype(F16).astype(F32)
    x[:, 5] *= 20
    ck, sk, zk = quant.quant_k_group(x, 4)
    assert sk.shape == (128,) and zk.shape == (128,)
    assert zk[5] == F16(x[:, 5].min())
    assert sk[5] == F16(F32(x[:, 5].max() - x[:, 5].min()) / F32(15))
    cv, sv, zv = quant.quant_v_group(x, 4)
    assert sv.shape == (32, 4)
    assert zv[7, 2] == F16(x[7, 64:96].min())
    assert np.array_equal(quant.dequant_v_group(cv, sv, zv)[:, :32],
                          quant.dequant_asym(cv[:, :32], sv[:, 0], zv[:, 0], axis=-1))


def test_symmetric_block():
    rng = np.random.default_rng(11)
    y = (rng.standard_normal((4000, 128)) * rng.uniform(0.01, 100, (4000, 1))).astype(F32)
    n, s = quant.quant_sym128(y)
    yh = quant.dequant_sym128(n, s)
    assert n.min() >= 1 and n.max() <= 15
    assert np.all(np.abs(y - yh) <= s.astype(np.float64)[:, None] / 2 * SLACK)
    # the absmax element maps to +-7
    am = np.argmax(np.abs(y), axis=1)
    c_am = n[np.arange(len(y)), am].astype(int) - 8
    assert np.all(np.abs(c_am) == 7)
    assert np.all(np.sign(c_am) == np.sign(y[np.arange(len(y)), am]))
    zn, zs = quant.quant_sym128(np.zeros((1, 128), F32))
    assert np.all(zn == 8) and zs[0] == 0


def test_dequant_exactness():
    # c * s_h is exact in fp32 (4-bit x 11-bit significands), so mul-then-add
    # equals the fp64 value rounded once
    rng = np.random.default_rng(13)
    c = rng.integers(0, 16, size=100000).astype(np.uint8)
    s = rng.standard_normal(100000).astype(F16)
    z = rng.standard_normal(100000).astype(F16)
    got = quant.dequant_asym(c[:, None], s, z, axis=-1)[:, 0]
    prod = c.astype(np.float64) * s.astype(np.float64)
    assert np.array_equal(prod.astype(F32).astype(np.float64), prod)
    assert np.array_equal(got, (prod + z.astype(np.float64)).astype(F32))


def test_symmetric_32_value_blocks():
    """Q4_0-style slices: the 128-block quantizer applied to each 32-value
    slice on its own (embedded in zeros, so its absmax is the slice's) must
    give the same codes and scale; bound, absmax level, byte image."""
    from oracle import layout
    rng = np.random.default_rng(12)
    y = (rng.standard_normal((500, 128)) * rng.uniform(0.01, 100, (500, 4)).repeat(32, axis=1)).astype(F32)
    n, s = quant.quant_sym32(y)
    assert n.shape == y.shape and s.shape == (500, 4)
    for g in range(4):
        emb = np.zeros_like(y)
        emb[:, 32 * g:32 * g + 32] = y[:, 32 * g:32 * g + 32]
        n1, s1 = quant.quant_sym128(emb)
        assert np.array_equal(s1.view(np.uint16), s[:, g].view(np.uint16))
        assert np.array_equal(n1[:, 32 * g:32 * g + 32], n[:, 32 * g:32 * g + 32])
    yh = quant.dequant_sym32(n, s)
    bound = np.repeat(s.astype(np.float64), 32, axis=1) / 2 * SLACK
    assert np.all(np.abs(y - yh) <= bound)
    img = layout.block18(n[:3], s[:3])
    assert img.shape == (3, 4, 18)
    assert np.array_equal(img[..., :2].copy().view("<f2")[..., 0], s[:3])
    # element 2k in the low nibble of byte k of its slice
    assert np.array_equal(img[..., 2:] & 0xF, n[:3].reshape(3, 4, 32)[..., 0::2])
    assert np.array_equal(img[..., 2:] >> 4, n[:3].reshape(3, 4, 32)[..., 1::2])
    # 18 B per 32 values = 4.5 bits per value (the page's Q4_0 row)
    assert img.shape[-1] * 8 / 32 == 4.5


def test_symmetric_block_3bit():
    rng = np.random.default_rng(14)
    y = (rng.standard_normal((3000, 128)) * rng.uniform(0.01, 100, (3000, 1))).astype(F32)
    n, s = quant.quant_sym128(y, 3)
    yh = quant.dequant_sym128(n, s, 3)
    assert n.min() >= 1 and n.max() <= 7
    assert np.all(np.abs(y - yh) <= s.astype(np.float64)[:, None] / 2 * SLACK)
    am = np.argmax(np.abs(y), axis=1)
    c_am = n[np.arange(len(y)), am].astype(int) - 4
    assert np.all(np.abs(c_am) == 3)
    assert np.all(np.sign(c_am) == np.sign(y[np.arange(len(y)), am]))
    # brute force: every code is the nearest of the 7 levels (away from ties)
    c = n.astype(np.float64) - 4
    q = y.astype(np.float64) / s.astype(np.float64)[:, None]
    near = np.clip(np.round(q), -3, 3)
    clear = np.abs(np.abs(q - np.floor(q)) - 0.5) > 1e-4
    assert np.array_equal(c[clear], near[clear])
    zn, zs = quant.quant_sym128(np.zeros((1, 128), F32), 3)
    assert np.all(zn == 4) and zs[0] == 0


def test_symmetric_32_value_blocks_8bit():
    """Q8_0-style slices: every code is the nearest of the 255 levels k s_h,
    k in [-127, 127] (fp64 brute force over all levels, away from ties); the
    absmax element takes the end level of its sign; half-step bound; zero
    slices; the 34-byte image and 8.5 bits per value (the page's Q8_0 row)."""
    from oracle import layout
    rng = np.random.default_rng(15)
    y = (rng.standard_normal((400, 128)) * rng.uniform(0.01, 100, (400, 4)).repeat(32, axis=1)).astype(F32)
    y[0, 32:64] = 0.0                                  # an all-zero slice
    n, s = quant.quant_sym32(y, 8)
    assert n.shape == y.shape and s.shape == (400, 4)
    assert n.min() >= 1 and n.max() <= 255
    assert s[0, 1] == 0 and np.all(n[0, 32:64] == 128)
    sx = np.repeat(s.astype(np.float64), 32, axis=1)
    c = n.astype(np.float64) - 128
    levels = np.arange(-127, 128, dtype=np.float64)
    for r in range(0, 400, 7):
        for j in range(128):
            if sx[r, j] == 0:
                continue
            d = np.abs(levels * sx[r, j] - float(y[r, j]))
            best = np.argsort(d)
            if d[best[1]] - d[best[0]] < 1e-6 * sx[r, j]:
                continue
            assert c[r, j] == levels[best[0]], (r, j)
    ys = y.reshape(400, 4, 32)
    am = np.argmax(np.abs(ys), axis=-1)
    c_am = np.take_along_axis(c.reshape(400, 4, 32), am[..., None], axis=-1)[..., 0]
    y_am = np.take_along_axis(ys, am[..., None], axis=-1)[..., 0]
    nz = s != 0
    assert np.all(np.abs(c_am[nz]) == 127)
    assert np.all(np.sign(c_am[nz]) == np.sign(y_am[nz]))
    yh = quant.dequant_sym32(n, s, 8)
    assert np.all(np.abs(y - yh) <= sx / 2 * SLACK)
    img = layout.block34(n[:3], s[:3])
    assert img.shape == (3, 4, 34)
    assert np.array_equal(img[..., :2].copy().view("<f2")[..., 0], s[:3])
    assert np.array_equal(img[..., 2:], n[:3].reshape(3, 4, 32))   # element k in byte k
    assert img.shape[-1] * 8 / 32 == 8.5


def _even_neighbour(k):
    """The code of a quotient k + 1/2 (k >= 0 an integer) under round half to
    even: k when k is even, k + 1 when it is odd."""
    return k if k % 2 == 0 else k + 1


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_asym_exact_ties_round_to_even(bits):
    # A group with min 0 and max Q has s = Q / Q = 1 and z = 0 exactly, so the
    # element k + 1/2 (fp16-exact) has the quotient k + 1/2 exactly: every
    # element but the two ends is a tie, which the fixed fp32 rule rounds half
    # to even (the pages give no tie rule; this is the reading the oracle takes).
    Q = 2 ** bits - 1
    rows, want = [], []
    for r in range(8):
        ks = [(r + i) % Q for i in range(30)]
        rows.append([0.0, float(Q)] + [k + 0.5 for k in ks])
        want.append([0, Q] + [_even_neighbour(k) for k in ks])
    x = np.array(rows, dtype=F16).astype(F32)
    c, s, z = quant.quant_asym(x, bits, axis=-1)
    assert np.all(s == F16(1.0)) and np.all(z == F16(0.0))
    assert np.array_equal(c.astype(np.int64), np.array(want))
    # the same groups as KIVI keys (tokens on axis -2) and values (32 dims)
    xk = np.repeat(x.T[:, :1], 128, axis=1)          # [32 tokens, 128 channels]
    ck, _, _ = quant.quant_k_group(xk, bits)
    assert np.array_equal(ck[:, 0].astype(np.int64), np.array(want[0]))
    xv = np.tile(x[0], 4)[None, :].repeat(32, axis=0)  # every token: four copies of group 0
    cv, sv, zv = quant.quant_v_group(xv, bits)
    assert np.all(sv == F16(1.0)) and np.all(zv == F16(0.0))
    assert np.array_equal(cv[3].astype(np.int64), np.tile(want[0], 4))


@pytest.mark.parametrize("bits", [4, 3])
def test_sym128_exact_ties_round_to_even(bits):
    # absmax = top gives s = 1 exactly; +-(k + 1/2) are ties, rounded to the
    # even neighbour with the sign kept (rint(-2.5) = -2); stored c + top + 1.
    top = (1 << (bits - 1)) - 1
    vals, want = [float(top), -float(top)], [top, -top]
    k = 0
    while len(vals) < 128:
        kk = k % top
        sgn = 1 if (k // top) % 2 == 0 else -1
        vals.append(sgn * (kk + 0.5))
        want.append(sgn * _even_neighbour(kk))
        k += 1
    y = np.array([vals], dtype=F16).astype(F32)
    c, s = quant.quant_sym128(y, bits)
    assert s[0] == F16(1.0)
    assert np.array_equal(c[0].astype(np.int64), np.array(want) + top + 1)


@pytest.mark.parametrize("bits", [4, 8])
def test_sym32_exact_ties_round_to_even(bits):
    # each 32-value slice: absmax = top (s = 1), the rest +-(k + 1/2)
    top = (1 << (bits - 1)) - 1
    vals, want = [], []
    for sl in range(4):
        vals += [float(top)]
        want += [top]
        for i in range(31):
            kk = (7 * sl + 5 * i) % top
            sgn = 1 if (i + sl) % 2 == 0 else -1
            vals.append(sgn * (kk + 0.5))
            want.append(sgn * _even_neighbour(kk))
    y = np.array([vals], dtype=F16).astype(F32)
    assert np.array_equal(np.abs(y[0]) % 1, np.array([0.0] + [0.5] * 31 + ([0.0] + [0.5] * 31) * 3))
    c, s = quant.quant_sym32(y, bits)
    assert np.all(s == F16(1.0))
    assert np.array_equal(c[0].astype(np.int64), np.array(want) + top + 1)
