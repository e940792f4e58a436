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


# ---------------------------------------------------------------------------
# Randomized form D_out H D_in / sqrt(128): signs, transform, signs ([trefon]
# "Jak 4-bitowemu cache to uchodzi: najpierw obrót").  The sign vectors here
# are built from the mask words by byte unpacking, independently of the
# oracle's bit loop.

def _signs(words):
    bits = np.unpackbits(np.array(words, dtype="<u4").view(np.uint8), bitorder="little")
    return 1 - 2 * bits.astype(np.int64)


MASK_IN = [0x9E3779B9, 0x7F4A7C15, 0x00000001, 0x80000000]
MASK_OUT = [0x12345678, 0xDEADBEEF, 0xFFFFFFFF, 0x0F0F0F0F]


def test_signed_fp32_schedule_exact_on_integers():
    rng = np.random.default_rng(3)
    x = rng.integers(-1000, 1000, size=(64, 128))
    y = hd.fwht128_f32(x.astype(np.float16), MASK_IN, MASK_OUT)
    sin, sout = _signs(MASK_IN), _signs(MASK_OUT)
    H = scipy.linalg.hadamard(128)
    exact = ((x * sin) @ H) * sout          # D_out H D_in x, rows as vectors (H symmetric)
    assert np.array_equal(y, (exact.astype(np.float32) * hd.C32))
    # the sides matter: D_in H D_out is another matrix
    swapped = ((x * sout) @ H) * sin
    assert not np.array_equal(y, swapped.astype(np.float32) * hd.C32)


def test_signed_zero_masks_are_the_plain_transform():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 128)).astype(np.float16)
    plain = hd.fwht128_f32(x)
    assert np.array_equal(hd.fwht128_f32(x, [0, 0, 0, 0], [0, 0, 0, 0]).view(np.uint32), plain.view(np.uint32))
    assert np.array_equal(hd.fwht128_f32(x, None, None).view(np.uint32), plain.view(np.uint32))


def test_signed_mask_bit_order():
    # bit 37 = word 1, bit 5: negates input coordinate 37 only
    m = [0, 1 << 5, 0, 0]
    e37 = np.zeros((1, 128), np.float16)
    e37[0, 37] = 1
    e36 = np.zeros((1, 128), np.float16)
    e36[0, 36] = 1
    assert np.array_equal(hd.fwht128_f32(e37, m, None), -hd.fwht128_f32(e37))
    assert np.array_equal(hd.fwht128_f32(e36, m, None), hd.fwht128_f32(e36))
    # on the output side it negates output coordinate 37 only
    x = np.random.default_rng(5).standard_normal((1, 128)).astype(np.float16)
    y, z = hd.fwht128_f32(x), hd.fwht128_f32(x, None, m)
    flip = np.ones(128, np.float32)
    flip[37] = -1
    assert np.array_equal(z, y * flip)
    assert hd.mask_signs(m)[37] == -1 and np.sum(hd.mask_signs(m) < 0) == 1


def test_signed_orthogonal_inverse_and_dot_identity():
    rng = np.random.default_rng(6)
    sin, sout = _signs(MASK_IN).astype(np.float64), _signs(MASK_OUT).astype(np.float64)
    R = np.diag(sout) @ scipy.linalg.hadamard(128).astype(np.float64) @ np.diag(sin) / np.sqrt(128)
    assert np.allclose(R @ R.T, np.eye(128), atol=1e-13)
    x = rng.standard_normal((128, 128)).astype(np.float16)
    y = hd.fwht128_f32(x, MASK_IN, MASK_OUT)
    # forward = R x for column vectors
    assert np.allclose(y, x.astype(np.float64) @ R.T, atol=1e-5, rtol=1e-5)
    # rotate_f64 with the same masks undoes it (rows: x R)
    assert np.allclose(hd.rotate_f64(y, MASK_IN, MASK_OUT), x.astype(np.float64), atol=1e-4)
    q, k = rng.standard_normal((8, 128)), rng.standard_normal((8, 128))
    lhs = np.sum((q @ R.T) * (k @ R.T), axis=1)
    assert np.allclose(lhs, np.sum(q * k, axis=1), rtol=1e-12, atol=1e-12)
    # an outlier still spreads over every coordinate
    e = np.zeros((1, 128), np.float16)
    e[0, 100] = 64
    assert np.allclose(np.abs(hd.fwht128_f32(e, MASK_IN, MASK_OUT)), 64 / np.sqrt(128), rtol=1e-6)


def test_fp32_stage_order_is_pinned():
    # The butterfly order changes fp32 results, and the stored codes of a
    # rotated cache ([trefon] "Jak 4-bitowemu cache to uchodzi: najpierw
    # obrot") are defined by the order h = 1, 2, ..., 64 (the pages give no
    # schedule; this is the reading the oracle takes).  For each adjacent pair
    # of stages (h, 2h) the input
    # x[0] = 1, x[h] = x[3h] = 2^-24 (all fp16-exact) gives, in that order:
    #   stage h:  x[0] = fl32(1 + 2^-24) = 1 (a tie, to even), x[h] = 1 - 2^-24,
    #             x[2h] = 2^-24, x[3h] = -2^-24 (all exact);
    #   stage 2h: x[0] = fl32(1 + 2^-24) = 1, x[h] = 1 - 2^-23, x[2h] = 1 - 2^-24,
    #             x[3h] = 1 (exact);
    # every other stage only copies these values (it adds zeros).  With 2h
    # first, x[0] would end at 1 + 2^-23 instead: stage 2h makes x[h] = 2^-23
    # exactly, and stage h then adds it to 1 without a tie.  Every order other
    # than 1, 2, ..., 64 puts some 2h before h, so these six vectors pin it.
    tiny = 2.0 ** -24
    for h in (1, 2, 4, 8, 16, 32):
        x = np.zeros(128, dtype=np.float16)
        x[0] = 1.0
        x[h] = tiny
        x[3 * h] = tiny
        assert float(x[h]) == tiny   # the smallest fp16 subnormal
        y = hd.fwht128_f32(x)
        want = {0: np.float32(1.0), h: np.float32(1.0 - 2.0 ** -23),
                2 * h: np.float32(1.0 - 2.0 ** -24), 3 * h: np.float32(1.0)}
        for i, v in want.items():
            assert y[i] == np.float32(v * hd.C32), (h, i)
        # the other order would be seen: (1 + 2^-23) C32 rounds to another float
        assert np.float32(np.float32(1.0 + 2.0 ** -23) * hd.C32) != y[0]
        # the randomized form flips signs exactly around the same schedule
        ys = hd.fwht128_f32(x, sign_in=[1, 0, 0, 0], sign_out=[0, 0, 0, 1 << 31])
        xs = x.copy()
        xs[0] = -xs[0]
        yn = hd.fwht128_f32(xs)
        yn[127] = -yn[127]
        assert np.array_equal(ys.view(np.uint32), yn.view(np.uint32))
