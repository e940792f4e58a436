"""Hadamard-128 rotation (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages rotate each 128-value vector by a Hadamard transform before
quantizing so that an outlier's energy is spread over all coordinates; the
transform is orthonormal, so nothing is lost, and dot products survive it,
q.k = (Hq).(Hk)  ([troisinh] "Tại sao nó hoạt động", item 2; [trefon] "Jak
4-bitowemu cache to uchodzi: najpierw obrót").  They fix neither the ordering
nor the floating-point schedule.  Readings used here:

  * H is the 128x128 Sylvester matrix in natural order,
    H[i, j] = (-1) ** popcount(i & j), applied as H / sqrt(128); H is symmetric
    and (H / sqrt(128)) is its own inverse.
  * The randomized form flips signs, transforms, and flips signs again
    ([trefon] "Jak 4-bitowemu cache to uchodzi: najpierw obrót"):
    y = D_out H D_in x / sqrt(128) with D = diag(+-1).  The two sign vectors
    are inputs (128-bit masks, four little-endian uint32 words; bit i of word
    i // 32 set negates coordinate i).  With both masks zero this is the plain
    transform above.  Sign flips are exact, so the fp32 schedule is the
    plain one with x negated where D_in says before it and y negated where
    D_out says after it.  The inverse is D_in H D_out / sqrt(128).
  * Because codes must be bit-exact, the float32 schedule is fixed:
    x <- float32(input); for h = 1, 2, 4, ..., 64 in that order, every pair
    (x[i], x[i + h]) with bit log2(h) of i clear becomes (a + b, a - b), each a
    single float32 operation; finally every element is multiplied by
    C32 = float32(1 / sqrt(128)) (bits 0x3DB504F3).
"""

import numpy as np

D = 128
C32 = np.float32(np.frombuffer(bytes.fromhex("f304b53d"), dtype="<f4")[0])


def mask_signs(words):
    """float32 +-1 vector of a 128-bit sign mask (four uint32 words, word
    i // 32, bit i % 32 negates coordinate i); None or zeros give all +1."""
    s = np.ones(D, dtype=np.float32)
    if words is None:
        return s
    words = [int(w) & 0xFFFFFFFF for w in words]
    if len(words) != 4:
        raise ValueError("a sign mask is four uint32 words")
    for i in range(D):
        if (words[i // 32] >> (i % 32)) & 1:
            s[i] = -1.0
    return s


def fwht128_f32(x, sign_in=None, sign_out=None):
    """Normalized FWHT over the last axis (length 128), fixed fp32 schedule;
    with sign masks, the randomized form D_out H D_in / sqrt(128)."""
    y = np.array(x, dtype=np.float32, copy=True) * mask_signs(sign_in)
    if y.shape[-1] != D:
        raise ValueError("last axis must be 128")
    shape = y.shape
    y = y.reshape(-1, D)
    h = 1
    while h < D:
        v = y.reshape(-1, D // (2 * h), 2, h)  # view: i = blk*2h + half*h + r
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        h *= 2
    y = y * C32
    return y.reshape(shape) * mask_signs(sign_out)


def fwht128_unnormalized_exact(x):
    """The same butterflies without the final scaling, in int64 (exact).

    Used to build H itself from unit vectors; integer inputs only."""
    y = np.array(x, dtype=np.int64, copy=True)
    shape = y.shape
    y = y.reshape(-1, D)
    h = 1
    while h < D:
        v = y.reshape(-1, D // (2 * h), 2, h)
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        h *= 2
    return y.reshape(shape)


def sylvester(n=D):
    """Dense +-1 Sylvester matrix by repeated Kronecker products of [[1,1],[1,-1]]."""
    h = np.array([[1]], dtype=np.int64)
    base = np.array([[1, 1], [1, -1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.kron(h, base)
    if h.shape[0] != n:
        raise ValueError("n must be a power of two")
    return h


def rotate_f64(x, sign_in=None, sign_out=None):
    """x -> x (H / sqrt(128)) in float64 over the last axis (its own inverse);
    with sign masks, x -> x (D_out H D_in / sqrt(128)): the inverse of the
    randomized rotation for row vectors (R = D_out H D_in / sqrt(128) maps a
    column k to R k, and x R = (R^T x^T)^T undoes it)."""
    H = sylvester(D).astype(np.float64) / np.sqrt(D)
    R = np.diag(mask_signs(sign_out).astype(np.float64)) @ H @ np.diag(mask_signs(sign_in).astype(np.float64))
    return np.asarray(x, dtype=np.float64) @ R
