"""Cache size accounting (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Closed forms from the pages:
  * a decoder with L attention layers, H_kv key/value heads of dimension D and
    T cached tokens stores 2 * L * T * H_kv * D scalars (keys and values);
    times the bytes per stored element gives the payload of one sequence
    ([nalar] "Ukuran cache mengikuti jumlah elemen tersimpan dan bit width");
  * the same count per token times bytes per value is the cache cost of one
    token ([trefon] "Bajty na token");
  * block formats store b bytes per n values: 66/128 (4-bit rotated, fp16
    scale + 64 code bytes), 50/128 (3-bit), 34/32 (Q8_0), 18/32 (Q4_0)
    ([trefon] "Przykład: model 27B przy 262K", format table).
"""

from fractions import Fraction

KIB = 1024
MIB = 1024 ** 2
GIB = 1024 ** 3

# bytes per block and values per block of the formats in the table
FORMATS = {
    "FP16": (2, 1),
    "Q8_0": (34, 32),
    "Q4_0": (18, 32),
    "TBQ4": (66, 128),
    "3-bit": (50, 128),
}


def cache_scalars(L, T, H_kv, D):
    return 2 * L * T * H_kv * D


def cache_bytes(L, T, H_kv, D, bytes_per_value):
    return cache_scalars(L, T, H_kv, D) * bytes_per_value


def bits_per_value(fmt):
    b, n = FORMATS[fmt]
    return Fraction(8 * b, n)


def bytes_per_token(fmt, values_per_token):
    """Exact bytes per token (a Fraction) for a block format."""
    b, n = FORMATS[fmt]
    return Fraction(values_per_token * b, n)


def values_per_token_from_total(total_bytes, tokens, fmt):
    """Invert a quoted cache size: values per token = bytes/token / bytes-per-value."""
    b, n = FORMATS[fmt]
    per_token = Fraction(total_bytes, tokens)
    return per_token * n / b


def tokens_in_budget(budget_bytes, fmt, values_per_token):
    return Fraction(budget_bytes) / bytes_per_token(fmt, values_per_token)


# --- this package's own formats (per cached token per key/value head) -------

def kivi_bytes_per_token_head(bits, group=32, vdims=32, d=128):
    """Codes + fp16 scale and zero, keys (per channel over `group` tokens) and
    values (per token over `vdims` dims), per token and head."""
    k = Fraction(d * bits, 8) + Fraction(d * 2 * 2, group)
    v = Fraction(d * bits, 8) + Fraction(d // vdims * 2 * 2, 1)
    return k + v


def block128_bytes_per_token_head(d=128):
    return 2 * Fraction(66 * d, 128)


def fp16_bytes_per_token_head(d=128):
    return 2 * d * 2
