"""Byte image of the cache planes (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages fix only the container of the 128-value block: a 2-byte fp16 scale
followed by 64 bytes of 4-bit indices, 66 bytes, 4.125 bits per value
([trefon] "Przykład: model 27B przy 262K").  Everything else below is this
package's own layout, written out so that a test can compare a device plane
byte for byte.  It is restated here from the layout's definition, not shared
with the library.

Packing of codes into bytes (canonical):
  4 bits: element 2k -> low nibble of byte k, element 2k+1 -> high nibble.
  2 bits: element 4k+j -> bits [2j, 2j+1] of byte k.
  3 bits: element i -> bits [3i, 3i+2] of the row read as one little-endian
          bit string, so eight codes fill three bytes and codes 2, 5 (mod 8)
          straddle a byte boundary.
  8 bits: element k -> byte k.

Tiles.  Quantized tokens live in tiles of 32 consecutive tokens (one key group):
  key tile   -- token-major: row t = packed codes of token t over the 128
                channels (128 B at 8 bits, 64 B at 4, 32 B at 2).  Byte c of row t is
                stored at offset (c // 16) * 512 + t * 16 + (c % 16), so the
                16-byte chunk j of all 32 rows is one contiguous 512-byte run.
  value tile -- channel-major: row d = packed codes of channel d over the 32
                tokens (32 B at 8 bits, 16 B at 4, 8 B at 2), row d at offset
                d * rowbytes.
  A tile holds 512 * bits bytes.

Planes (all [batch][kv_head][...], row-major, little-endian fp16/fp32):
  0 K_HI   KIVI: key tiles of the high-bit tier.  With a high-bit window of N
           tokens the plane is a ring of N/32 slots and group g uses slot
           g mod (N/32); otherwise it has one slot per group.
           Block schemes: key tiles of every group (4-bit, 3-bit for the
           50-byte block, 8-bit for Q8_0).
  1 V_HI   same for values.
  2 K_LO   KIVI with a high-bit window only: low-bit key tiles, slot g = group g.
  3 V_LO   same for values.
  4 K_META KIVI: 512 B per group: (s, z) fp16 pairs per channel, channel d at
           bytes 4d..4d+3.  BLOCK128: one fp16 scale per token; Q4_0 and
           Q8_0: four per token (32-value slices in order).
  5 V_META KIVI: 512 B per group: token-major, token t and 32-dim group g at
           bytes 16t + 4g: (s, z).  Block schemes: as K_META.
  6 K_WIN  KIVI: fp16 key window ring, 160 rows x 128 channels; token t in
           row t mod 160.
  7 V_WIN  KIVI: fp16 value window ring, channel-major: 128 rows (channels) x
           160 slots; token t in slot t mod 160 of every row.
  8 ROPE   pre-RoPE keys only: float32 [32 * ceil(max_tokens/32)][64][2],
           row t = (cos(t * theta_j), sin(t * theta_j)) for j = 0..63.
Group count Gmax = ceil(max_tokens / 32).  Unused planes have size 0.
"""

import numpy as np

TILE_TOKENS = 32
RING = 160
N_PLANES = 9
K_HI, V_HI, K_LO, V_LO, K_META, V_META, K_WIN, V_WIN, ROPE = range(N_PLANES)
PLANE_NAMES = ["K_HI", "V_HI", "K_LO", "V_LO", "K_META", "V_META", "K_WIN",
               "V_WIN", "ROPE"]


def pack_rows(codes, bits):
    """Pack the last axis of ``codes`` (uint8 values < 2**bits) canonically."""
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 3:
        if c.shape[-1] % 8:
            raise ValueError("3-bit rows pack 8 codes into 3 bytes")
        if np.any(c >= 8):
            raise ValueError("code out of range")
        g = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8)).astype(np.uint32)
        word = np.zeros(g.shape[:-1], dtype=np.uint32)       # 24 bits per 8 codes
        for j in range(8):
            word |= g[..., j] << (3 * j)
        out = np.stack([(word >> (8 * b)) & 0xFF for b in range(3)], axis=-1).astype(np.uint8)
        return out.reshape(c.shape[:-1] + (c.shape[-1] * 3 // 8,))
    per = 8 // bits
    if c.shape[-1] % per:
        raise ValueError("row length not a multiple of codes per byte")
    if np.any(c >= (1 << bits)):
        raise ValueError("code out of range")
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per)).astype(np.uint16)
    out = np.zeros(g.shape[:-1], dtype=np.uint16)
    for j in range(per):
        out |= g[..., j] << (bits * j)
    return out.astype(np.uint8)


def unpack_rows(packed, bits, n):
    """Inverse of pack_rows: bytes -> n codes per row."""
    p = np.asarray(packed, dtype=np.uint8)
    if bits == 3:
        b = p.reshape(p.shape[:-1] + (p.shape[-1] // 3, 3)).astype(np.uint32)
        word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
        out = np.stack([(word >> (3 * j)) & 7 for j in range(8)], axis=-1)
        return out.reshape(p.shape[:-1] + (-1,))[..., :n].astype(np.uint8)
    per = 8 // bits
    mask = (1 << bits) - 1
    parts = [(p >> (bits * j)) & mask for j in range(per)]
    out = np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * per,))
    return out[..., :n].astype(np.uint8)


def _k_tile_perm(bits):
    """perm[t * rowbytes + c] = offset of canonical byte c of token t."""
    rb = 128 * bits // 8
    t = np.arange(TILE_TOKENS)[:, None]
    c = np.arange(rb)[None, :]
    return ((c // 16) * 512 + t * 16 + (c % 16)).reshape(-1)


def k_tile(codes, bits):
    """Key tile image: codes [..., 32, 128] -> uint8 [..., 512 * bits]."""
    rows = pack_rows(codes, bits)                    # [..., 32, rowbytes]
    lead = rows.shape[:-2]
    out = np.zeros(lead + (512 * bits,), dtype=np.uint8)
    out[..., _k_tile_perm(bits)] = rows.reshape(lead + (-1,))
    return out


def k_tile_decode(tile, bits):
    """Key tile image -> codes [..., 32, 128]."""
    tile = np.asarray(tile, dtype=np.uint8)
    rb = 128 * bits // 8
    rows = tile[..., _k_tile_perm(bits)].reshape(tile.shape[:-1] + (TILE_TOKENS, rb))
    return unpack_rows(rows, bits, 128)


def v_tile(codes, bits):
    """Value tile image: codes [..., 32 tokens, 128 channels] -> [..., 512 * bits]."""
    ct = np.swapaxes(np.asarray(codes, dtype=np.uint8), -1, -2)   # [..., 128, 32]
    rows = pack_rows(ct, bits)                                     # [..., 128, rb]
    return rows.reshape(rows.shape[:-2] + (-1,))


def v_tile_decode(tile, bits):
    tile = np.asarray(tile, dtype=np.uint8)
    rb = 32 * bits // 8
    rows = tile.reshape(tile.shape[:-1] + (128, rb))
    ct = unpack_rows(rows, bits, 32)                               # [..., 128, 32]
    return np.swapaxes(ct, -1, -2)


def k_meta(s_h, z_h):
    """512-byte key metadata of one group: (s, z) per channel (fp16 LE)."""
    s = np.asarray(s_h, dtype="<f2")
    z = np.asarray(z_h, dtype="<f2")
    both = np.ascontiguousarray(np.stack([s, z], axis=-1))          # [..., 128, 2]
    return both.view(np.uint8).reshape(s.shape[:-1] + (512,))


def v_meta(s_h, z_h):
    """512-byte value metadata of one group from s_h, z_h [..., 32 tokens, 4]:
    token-major, (s, z) per 32-dim group."""
    s = np.asarray(s_h, dtype="<f2")
    z = np.asarray(z_h, dtype="<f2")
    both = np.ascontiguousarray(np.stack([s, z], axis=-1))          # [..., 32, 4, 2]
    return both.view(np.uint8).reshape(s.shape[:-2] + (512,))


def block66(nibbles, s_h):
    """The 66-byte block of one 128-value vector: fp16 scale (LE) + 64 code bytes."""
    s = np.asarray(s_h, dtype="<f2").reshape(-1, 1).view(np.uint8)
    codes = pack_rows(nibbles, 4).reshape(-1, 64)
    out = np.concatenate([s.reshape(-1, 2), codes], axis=-1)
    return out.reshape(np.shape(nibbles)[:-1] + (66,))


def block18(nibbles, s_h):
    """The 18-byte blocks of one 128-value vector's four 32-value slices: per
    slice an fp16 scale (LE) + 16 code bytes (element 2k low nibble of byte k)."""
    n = np.asarray(nibbles)
    codes = pack_rows(n.reshape(n.shape[:-1] + (4, 32)), 4)          # [..., 4, 16]
    s = np.asarray(s_h, dtype="<f2").reshape(n.shape[:-1] + (4, 1)).view(np.uint8)
    return np.concatenate([s, codes], axis=-1)                       # [..., 4, 18]


def block34(codes, s_h):
    """The 34-byte blocks of one 128-value vector's four 32-value slices at 8
    bits: per slice an fp16 scale (LE) + 32 code bytes, element k in byte k
    (the format table's "Q8_0 (34 B / 32)" row)."""
    n = np.asarray(codes)
    body = pack_rows(n.reshape(n.shape[:-1] + (4, 32)), 8)           # [..., 4, 32]
    s = np.asarray(s_h, dtype="<f2").reshape(n.shape[:-1] + (4, 1)).view(np.uint8)
    return np.concatenate([s, body], axis=-1)                        # [..., 4, 34]


def block50(codes, s_h):
    """The 50-byte block of one 128-value vector at 3 bits: fp16 scale (LE) +
    48 code bytes (the format table's "3 bity (50 B / 128)" row)."""
    s = np.asarray(s_h, dtype="<f2").reshape(-1, 1).view(np.uint8)
    body = pack_rows(codes, 3).reshape(-1, 48)
    out = np.concatenate([s.reshape(-1, 2), body], axis=-1)
    return out.reshape(np.shape(codes)[:-1] + (50,))


def gmax(max_tokens):
    return (max_tokens + TILE_TOKENS - 1) // TILE_TOKENS


def hi_slots(cfg, max_tokens):
    if cfg["scheme"] == "kivi" and cfg["hi_window"] >= 0:
        return cfg["hi_window"] // TILE_TOKENS
    return gmax(max_tokens)


def plane_sizes(cfg, batch, max_tokens):
    """Byte size of every plane, indexed like the plane list above."""
    pairs = batch * cfg["num_kv_heads"]
    G = gmax(max_tokens)
    sz = [0] * N_PLANES
    if cfg["scheme"] == "kivi":
        hs = hi_slots(cfg, max_tokens)
        sz[K_HI] = pairs * hs * 512 * cfg["k_bits"]
        sz[V_HI] = pairs * hs * 512 * cfg["v_bits"]
        if cfg["hi_window"] >= 0:
            sz[K_LO] = pairs * G * 512 * cfg["low_bits"]
            sz[V_LO] = pairs * G * 512 * cfg["low_bits"]
        sz[K_META] = pairs * G * 512
        sz[V_META] = pairs * G * 512
        sz[K_WIN] = pairs * RING * 128 * 2
        sz[V_WIN] = pairs * RING * 128 * 2
    else:
        per_token = 4 if cfg["scheme"] in ("q4_0", "q8_0") else 1     # fp16 per token
        sz[K_HI] = pairs * G * 512 * cfg["k_bits"]
        sz[V_HI] = pairs * G * 512 * cfg["v_bits"]
        sz[K_META] = pairs * G * TILE_TOKENS * 2 * per_token
        sz[V_META] = pairs * G * TILE_TOKENS * 2 * per_token
    if cfg["pre_rope"]:
        sz[ROPE] = G * TILE_TOKENS * 64 * 2 * 4
    return sz
