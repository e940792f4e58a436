"""A whole low-bit KV cache: append, dequantize, decode (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The cache is per sequence and grows by one entry per token per layer
([trefon] "Czym jest cache KV"); it is written at run time, token by token, so
quantization parameters come from the observed values ([trefon] "Dlaczego cache
trudniej skwantyzować niż wagi"; [nalar] "Pertumbuhan cache dinamis mengubah
persoalan kalibrasi").  Four schemes:

``kivi``: keys per channel over 32-token groups, values per token over 32-dim
  groups, asymmetric at 4, 3 or 2 bits, fp16 scale and zero (3-bit codes
  pack as one bit string per tile row, layout.py); a fp16 window of recent tokens
  (tiers.py); optionally a high-bit window with older groups at ``low_bits``
  ([troisinh] "Ý tưởng cốt lõi", "Mixed Precision"); optionally the Hadamard
  rotation before quantizing ([troisinh] "Tại sao nó hoạt động", item 2),
  plain or randomized by the sign masks ``sign_in`` / ``sign_out``
  (hadamard.py), and keys kept before RoPE (item 3).
``block128``: every token's 128-vector, optionally Hadamard-rotated, becomes one
  symmetric 4-bit block with an fp16 scale ([trefon] "Przykład: model 27B przy
  262K" and "Jak 4-bitowemu cache to uchodzi: najpierw obrót"); no window.
``tbq4``: every token's 128-vector, always rotated, becomes 16 Lloyd-Max
  indices and an fp16 norm in the same 66-byte container (codebook.py); no
  window.
``q4_0``: every token's 128-vector, optionally rotated, becomes four
  symmetric 4-bit 32-value blocks with an fp16 scale each (18 B per 32 values,
  [trefon] "Przykład: model 27B przy 262K"); no window.
``q8_0``: the same at 8 bits (34 B per 32 values, the table's Q8_0 row).

Append order (reading; the pages give none): groups that leave the high-bit
tier are requantized to ``low_bits`` from their dequantized high-bit values
(the fp16 source is gone by then); groups quantized for the first time go
straight from their fp16 source (rotated if configured) to the tier their age
dictates after the append.  Hence appending in pieces gives the same bytes as
one append unless a demotion happens in between.

Decode (reading): the attended keys and values are the dequantized cache in
its stored domain, the fp16 window taken exactly; Hadamard-rotated tokens are
rotated back with H / sqrt(128) in fp64 (D_in H D_out / sqrt(128) for the
randomized form; equivalently the query is rotated and
the output rotated back, q.k = (Hq).(Hk), [trefon] "Jak 4-bitowemu cache to
uchodzi"); pre-RoPE keys are rotated to their positions and the query to
``q_pos`` (default: the cache length).  Window tokens are stored unrotated.
"""

import numpy as np

from . import tiers, quant, layout, codebook
from .hadamard import fwht128_f32, rotate_f64
from .attention import rope_f64, decode_f64

F16 = np.float16
F32 = np.float32

DEFAULTS = dict(head_dim=128, group=32, vdims=32, window=128, hi_window=-1, k_bits=4, v_bits=4,
                low_bits=2, hadamard=False, pre_rope=False, rope_theta=10000.0,
                sign_in=None, sign_out=None)


def make_config(**kw):
    cfg = dict(DEFAULTS)
    cfg.update(kw)
    if cfg["scheme"] in BLOCK_SCHEMES:
        cfg["window"] = 0
        cfg.setdefault("k_bits", 4)
        cfg.setdefault("v_bits", 4)
    if cfg["scheme"] == "tbq4" and not cfg["hadamard"]:
        raise ValueError("tbq4 quantizes rotated blocks: hadamard must be on")
    return cfg


# per-token 128-value block schemes: nibbles + one fp16 per token and tensor
BLOCK_SCHEMES = ("block128", "tbq4", "q4_0", "q8_0")


def _tile_token_of_byte(key_tile, bits=4):
    """Token index whose codes a 4- or 3-bit tile byte holds (for a value
    tile, whose bytes hold codes of several tokens of one channel, the first
    token with bits in the byte)."""
    rb_k = 128 * bits // 8
    tok = np.zeros(512 * bits, np.int64)
    if key_tile:
        for cb in range(rb_k):
            for t in range(32):
                tok[(cb // 16) * 512 + t * 16 + (cb % 16)] = t
    else:
        rb_v = 32 * bits // 8
        tok[:] = np.tile((8 * np.arange(rb_v)) // bits, 128)
    return tok


class OracleCache:
    """Canonical (unpacked) cache state for [batch, num_kv_heads] sequences."""

    def __init__(self, cfg, batch, max_tokens):
        self.cfg = make_config(**cfg)
        c = self.cfg
        if c["head_dim"] != 128:
            raise ValueError("head_dim must be 128")
        if c["k_bits"] != c["v_bits"]:
            raise ValueError("key and value tiers must share bit widths")
        self.B, self.H = batch, c["num_kv_heads"]
        self.max_tokens = max_tokens
        self.length = 0
        G = layout.gmax(max_tokens)
        self.G = G
        B, H = self.B, self.H
        if c["scheme"] == "kivi":
            self.k_codes = np.zeros((B, H, G, 32, 128), np.uint8)
            self.v_codes = np.zeros((B, H, G, 32, 128), np.uint8)
            self.bits = np.zeros(G, np.int64)            # 0: not quantized
            self.k_s = np.zeros((B, H, G, 128), F16)
            self.k_z = np.zeros((B, H, G, 128), F16)
            self.v_s = np.zeros((B, H, G, 32, 4), F16)
            self.v_z = np.zeros((B, H, G, 32, 4), F16)
            self.win_k = np.zeros((B, H, 0, 128), F16)
            self.win_v = np.zeros((B, H, 0, 128), F16)
        else:
            Tp = G * 32
            self.k_nib = np.zeros((B, H, Tp, 128), np.uint8)
            self.v_nib = np.zeros((B, H, Tp, 128), np.uint8)
            sc_shape = (B, H, Tp, 4) if c["scheme"] in ("q4_0", "q8_0") else (B, H, Tp)
            self.k_sc = np.zeros(sc_shape, F16)
            self.v_sc = np.zeros(sc_shape, F16)

    # -- tiers ---------------------------------------------------------------
    @property
    def Tq(self):
        return tiers.quantized_prefix(self.length, self.cfg["window"])

    def _source_rows(self, x):
        """fp16 rows -> the float32 values the quantizer sees."""
        if self.cfg["hadamard"]:
            return fwht128_f32(x, self.cfg["sign_in"], self.cfg["sign_out"])
        return np.asarray(x, dtype=F16).astype(F32)

    # -- append --------------------------------------------------------------
    def append(self, k_new, v_new):
        """k_new, v_new: fp16 [B, n, H, 128] (token-major, like a projection)."""
        k_new = np.asarray(k_new, dtype=F16)
        v_new = np.asarray(v_new, dtype=F16)
        B, n, H, Dd = k_new.shape
        if (B, H, Dd) != (self.B, self.H, 128) or v_new.shape != k_new.shape:
            raise ValueError("shape mismatch")
        T0, T1 = self.length, self.length + n
        if T1 > self.max_tokens:
            raise ValueError("capacity exceeded")
        kn = np.transpose(k_new, (0, 2, 1, 3))       # [B, H, n, 128]
        vn = np.transpose(v_new, (0, 2, 1, 3))
        c = self.cfg
        if c["scheme"] in BLOCK_SCHEMES:
            quantize = {"block128": lambda y: quant.quant_sym128(y, c["k_bits"]),
                        "tbq4": codebook.quant_tbq4, "q4_0": quant.quant_sym32,
                        "q8_0": lambda y: quant.quant_sym32(y, 8)}[c["scheme"]]
            for name, src, nib, sc in (("k", kn, self.k_nib, self.k_sc),
                                       ("v", vn, self.v_nib, self.v_sc)):
                y = self._source_rows(src)
                q, s = quantize(y)
                nib[:, :, T0:T1] = q
                sc[:, :, T0:T1] = s
            self.length = T1
            return
        plan = tiers.append_plan(T0, T1, c["hi_window"], c["window"])
        Tq0, Tq1 = plan["Tq0"], plan["Tq1"]
        lo = c["low_bits"]
        for g in plan["demoted"]:
            xk = quant.dequant_k_group(self.k_codes[:, :, g], self.k_s[:, :, g], self.k_z[:, :, g])
            xv = quant.dequant_v_group(self.v_codes[:, :, g], self.v_s[:, :, g], self.v_z[:, :, g])
            self.k_codes[:, :, g], self.k_s[:, :, g], self.k_z[:, :, g] = quant.quant_k_group(xk, lo)
            self.v_codes[:, :, g], self.v_s[:, :, g], self.v_z[:, :, g] = quant.quant_v_group(xv, lo)
            self.bits[g] = lo
        src_k = np.concatenate([self.win_k, kn], axis=2)   # tokens [Tq0, T1)
        src_v = np.concatenate([self.win_v, vn], axis=2)
        # every new group at once: [B, H, groups, 32, 128], split by tier
        ng = len(plan["new_groups"])
        if ng:
            g0 = plan["new_groups"][0]
            rows_k = src_k[:, :, g0 * 32 - Tq0:(g0 + ng) * 32 - Tq0].reshape(B, H, ng, 32, 128)
            rows_v = src_v[:, :, g0 * 32 - Tq0:(g0 + ng) * 32 - Tq0].reshape(B, H, ng, 32, 128)
            gbits = np.array([tiers.group_bits(g, Tq1, c["hi_window"], c["k_bits"], lo)
                              for g in plan["new_groups"]])
            for bits in np.unique(gbits):
                sel = np.nonzero(gbits == bits)[0]
                gs = g0 + sel
                xk = self._source_rows(rows_k[:, :, sel])
                xv = self._source_rows(rows_v[:, :, sel])
                self.k_codes[:, :, gs], self.k_s[:, :, gs], self.k_z[:, :, gs] = quant.quant_k_group(xk, int(bits))
                self.v_codes[:, :, gs], self.v_s[:, :, gs], self.v_z[:, :, gs] = quant.quant_v_group(xv, int(bits))
                self.bits[gs] = bits
        self.win_k = src_k[:, :, Tq1 - Tq0:].copy()
        self.win_v = src_v[:, :, Tq1 - Tq0:].copy()
        self.length = T1

    # -- dequant -------------------------------------------------------------
    def dequant(self, t0=0, t1=None):
        """Stored-domain values: fp32 [B, t1 - t0, H, 128] for keys and values.

        Quantized tokens: the dequantized value (rotated if the config rotates,
        keys before RoPE).  Window tokens: their fp16 value exactly."""
        t1 = self.length if t1 is None else t1
        if not (0 <= t0 <= t1 <= self.length):
            raise ValueError("bad token range")
        c = self.cfg
        B, H = self.B, self.H
        K = np.zeros((B, H, t1 - t0, 128), F32)
        V = np.zeros((B, H, t1 - t0, 128), F32)
        if c["scheme"] in BLOCK_SCHEMES:
            deq = {"block128": lambda n, s: quant.dequant_sym128(n, s, c["k_bits"]),
                   "tbq4": codebook.dequant_tbq4, "q4_0": quant.dequant_sym32,
                   "q8_0": lambda n, s: quant.dequant_sym32(n, s, 8)}[c["scheme"]]
            K[:] = deq(self.k_nib[:, :, t0:t1], self.k_sc[:, :, t0:t1])
            V[:] = deq(self.v_nib[:, :, t0:t1], self.v_sc[:, :, t0:t1])
        else:
            Tq = self.Tq
            qa, qb = t0, min(t1, Tq)
            if qb > qa:
                g0, g1 = qa // 32, (qb + 31) // 32
                kd = quant.dequant_k_group(self.k_codes[:, :, g0:g1], self.k_s[:, :, g0:g1],
                                           self.k_z[:, :, g0:g1])
                vd = quant.dequant_v_group(self.v_codes[:, :, g0:g1], self.v_s[:, :, g0:g1],
                                           self.v_z[:, :, g0:g1])
                kd = kd.reshape(B, H, -1, 128)[:, :, qa - g0 * 32: qb - g0 * 32]
                vd = vd.reshape(B, H, -1, 128)[:, :, qa - g0 * 32: qb - g0 * 32]
                K[:, :, :qb - qa] = kd
                V[:, :, :qb - qa] = vd
            wa, wb = max(t0, Tq), t1
            if wb > wa:
                K[:, :, wa - t0:] = self.win_k[:, :, wa - Tq:wb - Tq].astype(F32)
                V[:, :, wa - t0:] = self.win_v[:, :, wa - Tq:wb - Tq].astype(F32)
        return np.transpose(K, (0, 2, 1, 3)), np.transpose(V, (0, 2, 1, 3))

    # -- decode --------------------------------------------------------------
    def attended_kv(self, q_pos=None):
        """The fp64 keys and values attention uses, [B, T, H, 128]."""
        c = self.cfg
        K, V = self.dequant()
        K = K.astype(np.float64)
        V = V.astype(np.float64)
        if c["hadamard"]:
            nq = self.length if c["scheme"] in BLOCK_SCHEMES else self.Tq
            K[:, :nq] = rotate_f64(K[:, :nq], c["sign_in"], c["sign_out"])
            V[:, :nq] = rotate_f64(V[:, :nq], c["sign_in"], c["sign_out"])
        if c["pre_rope"]:
            Kt = np.transpose(K, (0, 2, 1, 3))
            Kt = rope_f64(Kt, np.arange(self.length), c["rope_theta"])
            K = np.transpose(Kt, (0, 2, 1, 3))
        return K, V

    def decode(self, q, q_pos=None, sm_scale=None):
        """q: fp16 [B, Hq, 128] (before RoPE when keys are pre-RoPE)."""
        c = self.cfg
        q = np.asarray(q).astype(np.float64)
        if c["pre_rope"]:
            pos = self.length if q_pos is None else q_pos
            q = rope_f64(q[:, :, None, :], np.array([pos]), c["rope_theta"])[:, :, 0, :]
        K, V = self.attended_kv()
        return decode_f64(q, K, V, sm_scale)

    # -- byte image ----------------------------------------------------------
    def plane_images(self):
        """(images, live): uint8 images of planes 0..7 and masks of defined bytes."""
        c = self.cfg
        B, H = self.B, self.H
        sizes = layout.plane_sizes(c, B, self.max_tokens)
        img = [np.zeros(s, np.uint8) for s in sizes]
        live = [np.zeros(s, bool) for s in sizes]
        pair = lambda a: a.reshape(B, H, -1)
        T = self.length
        if c["scheme"] in BLOCK_SCHEMES:
            G = self.G
            for plane, nib, sc in ((layout.K_HI, self.k_nib, self.k_sc),
                                   (layout.V_HI, self.v_nib, self.v_sc)):
                tiles = nib.reshape(B, H, G, 32, 128)
                tb = 512 * c["k_bits"]
                im = pair(img[plane]).reshape(B, H, G, tb)
                lv = pair(live[plane]).reshape(B, H, G, tb)
                tok = np.arange(G)[:, None] * 32 + _tile_token_of_byte(plane == layout.K_HI, c["k_bits"])[None, :]
                im[:] = (layout.k_tile if plane == layout.K_HI else layout.v_tile)(tiles, c["k_bits"])
                lv[:] = (tok < T)[None, None]
                meta = layout.K_META if plane == layout.K_HI else layout.V_META
                pair(img[meta])[:] = sc.reshape(B, H, -1).astype("<f2").view(np.uint8)
                ml = np.repeat(np.arange(G * 32) < T, 2 * (4 if c["scheme"] in ("q4_0", "q8_0") else 1))
                pair(live[meta])[:] = ml[None, None]
            return img, live
        hs = layout.hi_slots(c, self.max_tokens)
        Tq = self.Tq
        gq = np.arange(Tq // 32)
        hi_mask = gq * 32 >= tiers.hi_start(Tq, c["hi_window"])
        for is_hi in (True, False):
            gs = gq[hi_mask == is_hi]
            if gs.size == 0:
                continue
            b = int(self.bits[gs[0]])
            assert np.all(self.bits[gs] == b)
            kp, vp = (layout.K_HI, layout.V_HI) if is_hi else (layout.K_LO, layout.V_LO)
            slots = gs % hs if is_hi else gs
            tb = 512 * b
            for p, im_fn, codes in ((kp, layout.k_tile, self.k_codes), (vp, layout.v_tile, self.v_codes)):
                im = pair(img[p]).reshape(B, H, -1, tb)
                lv = pair(live[p]).reshape(B, H, -1, tb)
                im[:, :, slots] = im_fn(codes[:, :, gs], b)
                lv[:, :, slots] = True
        if gq.size:
            km = pair(img[layout.K_META]).reshape(B, H, -1, 512)
            vm = pair(img[layout.V_META]).reshape(B, H, -1, 512)
            km[:, :, gq] = layout.k_meta(self.k_s[:, :, gq], self.k_z[:, :, gq])
            vm[:, :, gq] = layout.v_meta(self.v_s[:, :, gq], self.v_z[:, :, gq])
            pair(live[layout.K_META]).reshape(B, H, -1, 512)[:, :, gq] = True
            pair(live[layout.V_META]).reshape(B, H, -1, 512)[:, :, gq] = True
        ring = np.arange(Tq, T) % layout.RING
        im = pair(img[layout.K_WIN]).reshape(B, H, layout.RING, 256)
        lv = pair(live[layout.K_WIN]).reshape(B, H, layout.RING, 256)
        im[:, :, ring] = np.ascontiguousarray(self.win_k.astype("<f2")).view(np.uint8).reshape(B, H, -1, 256)
        lv[:, :, ring] = True
        im = pair(img[layout.V_WIN]).reshape(B, H, 128, layout.RING, 2)
        lv = pair(live[layout.V_WIN]).reshape(B, H, 128, layout.RING, 2)
        wv = np.ascontiguousarray(np.swapaxes(self.win_v.astype("<f2"), 2, 3)).view(np.uint8)
        im[:, :, :, ring] = wv.reshape(B, H, 128, -1, 2)
        lv[:, :, :, ring] = True
        return img, live
