"""Quantizers and dequantizers (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:
  * keys are quantized per channel and values per token, both asymmetric
    ([troisinh] "Tại sao nó hoạt động", item 1; [trefon] "Dlaczego cache
    trudniej skwantyzować niż wagi");
  * a group of elements shares a scale and optionally a zero point; finer
    groups follow local ranges at a metadata cost; clipping trades resolution
    against saturation ([nalar] "Granularitas kuantisasi mengendalikan rentang
    yang harus dicakup setiap scale");
  * scales come from the values observed at run time, no calibration
    ([nalar] "Pertumbuhan cache dinamis mengubah persoalan kalibrasi");
  * the 128-value block holds a 2-byte fp16 scale and 64 bytes of 4-bit codes
    ([trefon] "Przykład: model 27B przy 262K").

Readings where the pages are silent (all float32 one op at a time, RNE):
  asymmetric, b bits (4, 3 or 2; the page's title names INT4 and INT3 caches,
  [troisinh] "KV Cache Quantization - Nén cache INT4/INT3"), Q = 2**b - 1,
  over a group x:
    mn, mx = min(x), max(x)
    s  = fl32(fl32(mx - mn) / Q);  s_h = fp16(s) + (+0.0)
    z_h = fp16(mn) + (+0.0)         (the additions turn -0 into +0: over a
                                     group of signed zeros min and max may be
                                     either zero, so the sign bits would
                                     depend on reduction order)
    c  = clamp(rint(fl32(fl32(x - z_h) / s_h)), 0, Q);   c = 0 wherever s_h == 0
    x^ = fl32(c * s_h + z_h)        (c * s_h is exact in fp32)
  symmetric 128-block, 4 bits:
    a = max|y|;  s_h = fp16(fl32(a / 7))
    c = clamp(rint(fl32(y / s_h)), -7, 7);  c = 0 wherever s_h == 0
    stored nibble n = c + 8 (1..15);  y^ = fl32((n - 8) * s_h)  (exact)
  the same at 3 bits (the 50-byte block, "3 bity (50 B / 128)" in the format
  table of [trefon] "Przykład: model 27B przy 262K"): s_h = fp16(fl32(a / 3)),
  c in [-3, 3], stored n = c + 4 (1..7), y^ = fl32((n - 4) * s_h).
  symmetric 32-value blocks, 4 bits ("Q4_0", 18 B per 32 values in the
  format table of [trefon] "Przykład: model 27B przy 262K"): the same
  quantizer over each 32-value slice of a vector, one fp16 scale per slice;
  at 8 bits ("Q8_0", 34 B per 32 values, the table's row above it):
  s_h = fp16(fl32(a / 127)), c in [-127, 127], stored byte c + 128 (1..255),
  y^ = fl32((n - 128) * s_h).
  No clipping: the full [min, max] range is used.
"""

import numpy as np

F16 = np.float16
F32 = np.float32


def _check_finite(x):
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle inputs must be finite")


def quant_asym(x, bits, axis):
    """Asymmetric quantization of float32 ``x`` with groups along ``axis``.

    Returns (codes uint8 shaped like x, s_h fp16, z_h fp16), where s_h and z_h
    have ``axis`` removed."""
    x = np.asarray(x, dtype=F32)
    _check_finite(x)
    Q = F32(2 ** bits - 1)
    mn = x.min(axis=axis)
    mx = x.max(axis=axis)
    s = (mx - mn).astype(F32) / Q
    s_h = (s.astype(F16) + F16(0.0)).astype(F16)
    z_h = (mn.astype(F16) + F16(0.0)).astype(F16)
    sx = np.expand_dims(s_h.astype(F32), axis)
    zx = np.expand_dims(z_h.astype(F32), axis)
    diff = (x - zx).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = (diff / sx).astype(F32)
    quo = np.where(sx == 0, F32(0), quo)
    c = np.clip(np.rint(quo), F32(0), Q)
    return c.astype(np.uint8), s_h, z_h


def dequant_asym(codes, s_h, z_h, axis):
    """x^ = fl32(c * s_h + z_h) with the group parameters broadcast on ``axis``."""
    c = np.asarray(codes).astype(F32)
    s = np.expand_dims(np.asarray(s_h, dtype=F16).astype(F32), axis)
    z = np.expand_dims(np.asarray(z_h, dtype=F16).astype(F32), axis)
    return ((c * s).astype(F32) + z).astype(F32)


def quant_sym128(y, bits=4):
    """Symmetric quantization of float32 vectors along the last axis (128) at
    4 or 3 bits.  Returns (codes uint8 in 1 .. 2^bits - 1 (the middle code for
    an all-zero vector), s_h fp16)."""
    y = np.asarray(y, dtype=F32)
    _check_finite(y)
    if y.shape[-1] != 128:
        raise ValueError("block length must be 128")
    if bits not in (4, 3):
        raise ValueError("4 or 3 bits")
    top = (1 << (bits - 1)) - 1                    # 7 or 3
    a = np.abs(y).max(axis=-1)
    s_h = (a / F32(top)).astype(F32).astype(F16)
    sx = s_h.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = (y / sx).astype(F32)
    quo = np.where(sx == 0, F32(0), quo)
    c = np.clip(np.rint(quo), F32(-top), F32(top)).astype(np.int16)
    return (c + top + 1).astype(np.uint8), s_h


def dequant_sym128(nibbles, s_h, bits=4):
    """y^ = fl32((n - 2^(bits-1)) * s_h), exact."""
    c = np.asarray(nibbles).astype(np.int16) - (1 << (bits - 1))
    return (c.astype(F32) * np.asarray(s_h, dtype=F16).astype(F32)[..., None]).astype(F32)


def quant_sym32(y, bits=4):
    """Symmetric quantization of float32 vectors (last axis 128) in four
    32-value slices at 4 bits (Q4_0: codes -7..7 stored + 8, 1..15) or 8 bits
    (Q8_0: codes -127..127 stored + 128, 1..255): (codes uint8, s_h fp16
    [..., 4])."""
    if bits not in (4, 8):
        raise ValueError("4 or 8 bits")
    top = (1 << (bits - 1)) - 1                    # 7 or 127
    y = np.asarray(y, dtype=F32)
    _check_finite(y)
    if y.shape[-1] != 128:
        raise ValueError("vector length must be 128")
    ys = y.reshape(y.shape[:-1] + (4, 32))
    a = np.abs(ys).max(axis=-1)
    s_h = (a / F32(top)).astype(F32).astype(F16)
    sx = s_h.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = (ys / sx).astype(F32)
    quo = np.where(sx == 0, F32(0), quo)
    c = np.clip(np.rint(quo), F32(-top), F32(top)).astype(np.int16)
    return (c + top + 1).astype(np.uint8).reshape(y.shape), s_h


def dequant_sym32(codes, s_h, bits=4):
    """y^ = fl32((n - 2^(bits-1)) * s_h of the value's slice), exact."""
    n = np.asarray(codes)
    c = (n.astype(np.int16) - (1 << (bits - 1))).reshape(n.shape[:-1] + (4, 32)).astype(F32)
    y = c * np.asarray(s_h, dtype=F16).astype(F32)[..., None]
    return y.astype(F32).reshape(n.shape)


# --- KIVI groups -------------------------------------------------------------

def quant_k_group(x, bits):
    """Keys, one group: x [..., 32 tokens, 128 channels] float32.

    Per-channel ranges over the 32 tokens.  Returns codes [..., 32, 128],
    s_h [..., 128], z_h [..., 128]."""
    return quant_asym(x, bits, axis=-2)


def dequant_k_group(codes, s_h, z_h):
    return dequant_asym(codes, s_h, z_h, axis=-2)


def quant_v_group(x, bits, dims=32):
    """Values, one group of 32 tokens: x [..., 32, 128] float32.

    Per-token ranges over 32 consecutive dims.  Returns codes [..., 32, 128],
    s_h [..., 32, 4], z_h [..., 32, 4]."""
    x = np.asarray(x, dtype=F32)
    shp = x.shape
    xg = x.reshape(shp[:-1] + (shp[-1] // dims, dims))
    c, s_h, z_h = quant_asym(xg, bits, axis=-1)
    return c.reshape(shp), s_h, z_h


def dequant_v_group(codes, s_h, z_h, dims=32):
    c = np.asarray(codes)
    shp = c.shape
    cg = c.reshape(shp[:-1] + (shp[-1] // dims, dims))
    return dequant_asym(cg, s_h, z_h, axis=-1).reshape(shp)
