"""Pins for oracle/layout.py: exhaustive code packing (every code value at every
position, the bug class of a 3-bit codec the trefon page reports), tile
permutations, the 66-byte block image."""

import numpy as np
import pytest

from oracle import layout


@pytest.mark.parametrize("bits", [4, 2])
def test_every_code_at_every_position(bits):
    per = 8 // bits
    for p in range(128):
        for v in range(2 ** bits):
            codes = np.zeros(128, np.uint8)
            codes[p] = v
            packed = layout.pack_rows(codes, bits)
            expect = np.zeros(128 // per, np.uint8)
            expect[p // per] = v << (bits * (p % per))
            assert np.array_equal(packed, expect), (bits, p, v)
            assert np.array_equal(layout.unpack_rows(packed, bits, 128), codes)


def test_hand_packed_examples():
    assert list(layout.pack_rows(np.array([1, 2, 3, 4], np.uint8), 4)) == [0x21, 0x43]
    assert list(layout.pack_rows(np.array([1, 2, 3, 0], np.uint8), 2)) == [0b00111001]
    assert list(layout.pack_rows(np.array([15, 0, 0, 15], np.uint8), 4)) == [0x0F, 0xF0]
    with pytest.raises(ValueError):
        layout.pack_rows(np.array([16, 0], np.uint8), 4)


@pytest.mark.parametrize("bits", [4, 2])
def test_key_tile_offsets(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 2 ** bits, size=(32, 128)).astype(np.uint8)
    tile = layout.k_tile(codes, bits)
    assert tile.shape == (512 * bits,)
    rows = layout.pack_rows(codes, bits)
    # token 5, canonical byte 17 -> chunk 1 (bytes 16..31), offset 512 + 5*16 + 1
    assert tile[512 + 80 + 1] == rows[5, 17]
    assert tile[31 * 16 + 15] == rows[31, 15]
    assert np.array_equal(layout.k_tile_decode(tile, bits), codes)
    # a permutation: every canonical byte appears exactly once
    marker = np.arange(32 * 128 * bits // 8).reshape(32, -1)
    seen = np.zeros(512 * bits, int)
    for t in range(32):
        for c in range(marker.shape[1]):
            seen[(c // 16) * 512 + t * 16 + c % 16] += 1
    assert np.all(seen == 1)


@pytest.mark.parametrize("bits", [4, 2])
def test_value_tile_channel_major(bits):
    rng = np.random.default_rng(10 + bits)
    codes = rng.integers(0, 2 ** bits, size=(32, 128)).astype(np.uint8)
    tile = layout.v_tile(codes, bits)
    per = 8 // bits
    rb = 32 // per
    for d in (0, 1, 77, 127):
        for t in (0, 1, 5, 31):
            byte = tile[d * rb + t // per]
            assert (byte >> (bits * (t % per))) & (2 ** bits - 1) == codes[t, d]
    assert np.array_equal(layout.v_tile_decode(tile, bits), codes)


def test_block66_image():
    rng = np.random.default_rng(3)
    nib = rng.integers(1, 16, size=(5, 128)).astype(np.uint8)
    s = rng.standard_normal(5).astype(np.float16)
    img = layout.block66(nib, s)
    assert img.shape == (5, 66)
    assert np.array_equal(img[:, :2].copy().view("<f2")[:, 0], s)
    assert np.array_equal(img[:, 2:], layout.pack_rows(nib, 4))
    assert img.shape[1] * 8 / 128 == 4.125


def test_meta_images():
    rng = np.random.default_rng(4)
    s = rng.standard_normal(128).astype(np.float16)
    z = rng.standard_normal(128).astype(np.float16)
    m = layout.k_meta(s, z)
    assert m.shape == (512,)
    mh = m.view("<f2")
    assert np.array_equal(mh[0::2], s) and np.array_equal(mh[1::2], z)
    assert m[4 * 9:4 * 9 + 2].view("<f2")[0] == s[9]
    sv = rng.standard_normal((32, 4)).astype(np.float16)
    zv = rng.standard_normal((32, 4)).astype(np.float16)
    mv = layout.v_meta(sv, zv)
    assert mv.shape == (512,)
    # token 7, dim group 2 at bytes 16*7 + 4*2: (s, z)
    assert mv[16 * 7 + 8:16 * 7 + 10].view("<f2")[0] == sv[7, 2]
    assert mv[16 * 31 + 14:16 * 31 + 16].view("<f2")[0] == zv[31, 3]


def test_every_3bit_code_at_every_position():
    # element i at bits 3i .. 3i + 2 of the little-endian bit string: built
    # here bit by bit, independently of the packer's 24-bit words
    for p in range(128):
        for v in range(8):
            codes = np.zeros(128, np.uint8)
            codes[p] = v
            packed = layout.pack_rows(codes, 3)
            assert packed.shape == (48,)
            expect = np.zeros(48, np.uint8)
            for k in range(3):
                if (v >> k) & 1:
                    bit = 3 * p + k
                    expect[bit // 8] |= 1 << (bit % 8)
            assert np.array_equal(packed, expect), (p, v)
            assert np.array_equal(layout.unpack_rows(packed, 3, 128), codes)
    # all codes at once, random rows, round trip
    rng = np.random.default_rng(33)
    rows = rng.integers(0, 8, size=(50, 128)).astype(np.uint8)
    assert np.array_equal(layout.unpack_rows(layout.pack_rows(rows, 3), 3, 128), rows)
    with pytest.raises(ValueError):
        layout.pack_rows(np.array([8] + [0] * 7, np.uint8), 3)


def test_3bit_tiles_and_block50():
    rng = np.random.default_rng(34)
    codes = rng.integers(0, 8, size=(32, 128)).astype(np.uint8)
    kt, vt = layout.k_tile(codes, 3), layout.v_tile(codes, 3)
    assert kt.shape == (1536,) and vt.shape == (1536,)
    assert np.array_equal(layout.k_tile_decode(kt, 3), codes)
    assert np.array_equal(layout.v_tile_decode(vt, 3), codes)
    rows = layout.pack_rows(codes, 3)              # [32, 48]
    assert kt[2 * 512 + 7 * 16 + 3] == rows[7, 35]
    # value row d: 12 bytes, token t at bits 3t
    for d in (0, 64, 127):
        r = vt[12 * d:12 * d + 12]
        stream = int.from_bytes(r.tobytes(), "little")
        assert [(stream >> (3 * t)) & 7 for t in range(32)] == list(codes[:, d])
    s = np.array([1.5, -0.25], np.float16)
    img = layout.block50(codes[:2] % 8, s)
    assert img.shape == (2, 50)
    assert np.array_equal(img[:, :2].copy().view("<f2")[:, 0], s)
    assert np.array_equal(img[:, 2:], layout.pack_rows(codes[:2], 3))
    assert 50 * 8 / 128 == 3.125
