"""Tier map: which cached tokens are fp16, high-bit or low-bit (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages say that a recent window kept at higher precision is part of the
cache representation ([nalar] "Evaluasi harus memisahkan peningkatan kapasitas
dari dampak model") and that recent tokens keep 4 bits while old ones drop to
2 bits ([troisinh] "Ý tưởng cốt lõi", paragraph "Mixed Precision — Nóng và
Lạnh").  They fix no rule for where the window ends.  The reading used here:

  * keys are quantized per channel over groups of G = 32 tokens aligned to
    absolute token 0, so only whole groups ever leave the fp16 window;
  * with W = 128, the quantized prefix of a cache of length T is
        Tq(T) = max(0, floor((T - W) / G) * G)
    and tokens [Tq, T) stay fp16: between W and W + G - 1 of them once
    T >= W (all T tokens while T < W);
  * with a high-bit window of N tokens (N a multiple of G, or -1 for "all"),
    quantized tokens [max(0, Tq - N), Tq) are high-bit and [0, Tq - N) low-bit;
  * the symmetric 128-value block format has no fp16 window: Tq(T) = T.
"""

GROUP = 32
WINDOW = 128


def quantized_prefix(T, window=WINDOW, group=GROUP):
    """Tq(T): number of leading tokens held quantized (always a multiple of group
    when window > 0).  ``window == 0`` means every token is quantized."""
    if T < 0:
        raise ValueError("negative length")
    if window == 0:
        return T
    return max(0, ((T - window) // group) * group)


def hi_start(Tq, hi_window):
    """First token of the high-bit tier; tokens [0, hi_start) are low-bit."""
    if hi_window < 0:
        return 0
    return max(0, Tq - hi_window)


def group_bits(g, Tq, hi_window, hi_bits, lo_bits, group=GROUP):
    """Bit width of quantized group g (tokens [g*group, (g+1)*group))."""
    return hi_bits if g * group >= hi_start(Tq, hi_window) else lo_bits


def append_plan(T0, T1, hi_window, window=WINDOW, group=GROUP):
    """What an append from length T0 to T1 does, as plain sets of group indices.

    Returns a dict with
      new_groups : groups quantized for the first time, [Tq0/G, Tq1/G)
      demoted    : groups that were high-bit at T0 and are low-bit at T1
      tail       : (Tq1, T1), the fp16 tokens after the append
    A new group goes straight to the tier its age dictates at T1.
    """
    if T1 < T0:
        raise ValueError("append cannot shrink the cache")
    Tq0 = quantized_prefix(T0, window, group)
    Tq1 = quantized_prefix(T1, window, group)
    new_groups = list(range(Tq0 // group, Tq1 // group)) if window else []
    demoted = []
    if hi_window >= 0 and window:
        h0 = hi_start(Tq0, hi_window)
        h1 = hi_start(Tq1, hi_window)
        # high-bit at T0: [h0, Tq0); low-bit at T1: [0, h1)
        demoted = list(range(h0 // group, min(Tq0, h1) // group))
    return {"new_groups": new_groups, "demoted": demoted, "tail": (Tq1, T1),
            "Tq0": Tq0, "Tq1": Tq1}
