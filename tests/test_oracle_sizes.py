"""Pins for oracle/sizes.py and the plane sizes of oracle/layout.py.

Everything here is checked against numbers the pages print (tests/golden/)."""

from fractions import Fraction

import pytest

from conftest import golden_kv, golden_table
from oracle import sizes, layout
from oracle.cache import make_config

EX = golden_kv("page_size_examples.txt")
TOKENS = {"8K": 8192, "32K": 32768, "128K": 131072, "262K": 262144}
UNIT = {"KiB": sizes.KIB, "MiB": sizes.MIB, "GiB": sizes.GIB}


def test_tbq4_worked_example():
    # 4224 MiB at 262144 tokens -> bytes/token -> values/token
    total = EX["tbq4_total_mib"] * sizes.MIB
    per_token = Fraction(total, EX["tbq4_tokens"])
    assert per_token == EX["tbq4_bytes_per_token"]
    vals = sizes.values_per_token_from_total(total, EX["tbq4_tokens"], "TBQ4")
    assert vals == EX["tbq4_values_per_token"]
    assert EX["tbq4_scale_bytes"] + EX["tbq4_code_bytes"] == EX["tbq4_block_bytes"]
    assert EX["tbq4_code_bytes"] * 8 == 4 * EX["tbq4_block_values"]
    assert sizes.bits_per_value("TBQ4") == Fraction(EX["tbq4_bits_per_value"]).limit_denominator()


def _fmt(x, printed):
    """Round an exact value the way the page prints it (its number of decimals)."""
    dec = len(printed.split(".")[1]) if "." in printed else 0
    return round(float(x), dec), float(printed)


@pytest.mark.parametrize("row", golden_table("trefon_format_table.txt"), ids=lambda r: r[0])
def test_format_table_row(row):
    fmt, bits, per_token = row[0], row[1], row[2]
    vpt = EX["tbq4_values_per_token"]
    assert float(sizes.bits_per_value(fmt)) == float(bits)
    num, unit = per_token.split()
    got = sizes.bytes_per_token(fmt, vpt) / UNIT[unit]
    assert got == Fraction(num)
    for col, cell in zip(TOKENS, row[3:]):
        num, unit = cell.split()
        exact = sizes.bytes_per_token(fmt, vpt) * TOKENS[col] / UNIT[unit]
        mine, page = _fmt(exact, num)
        assert mine == page, (fmt, col, float(exact), cell)


def test_budget_paragraph():
    budget = EX["budget_gib"] * sizes.GIB
    vpt = EX["tbq4_values_per_token"]
    fp16 = sizes.tokens_in_budget(budget, "FP16", vpt)
    q8 = sizes.tokens_in_budget(budget, "Q8_0", vpt)
    tbq4 = sizes.tokens_in_budget(budget, "TBQ4", vpt)
    assert fp16 == 114688
    # "roughly 110K" / "roughly 210K": within 5 %
    assert abs(float(fp16) / EX["budget_fp16_tokens_approx"] - 1) < 0.05
    assert abs(float(q8) / EX["budget_q8_0_tokens_approx"] - 1) < 0.05
    assert tbq4 >= EX["budget_4bit_tokens_min"]
    # concurrency multiplies the cache
    per = sizes.bytes_per_token("TBQ4", vpt)
    assert EX["concurrency_agents"] * EX["concurrency_tokens_each"] * per == \
        EX["concurrency_tokens_single"] * per


def test_llama2_7b_fp16_cache():
    # Llama-2-7B: 32 layers, 32 KV heads (MHA), head dim 128, fp16.
    per_token = sizes.cache_bytes(32, 1, 32, 128, 2)
    assert per_token == 524288
    gb = lambda t: sizes.cache_bytes(32, t, 32, 128, 2) / 1e9
    assert abs(gb(10_000) / EX["llama2_7b_fp16_10k_gb_approx"] - 1) < 0.1
    assert gb(100_000) > EX["llama2_7b_fp16_100k_gb_min"]
    assert gb(1_000_000) > EX["llama2_7b_fp16_1m_gb_min"]
    # GQA with 8 of 32 KV heads: 4x smaller
    assert sizes.cache_bytes(32, 1, 32, 128, 2) == EX["gqa_reduction"] * sizes.cache_bytes(32, 1, 8, 128, 2)
    # the closed form is the per-token bytes times T
    assert sizes.cache_scalars(32, 10, 32, 128) * 2 == 10 * per_token


def test_own_format_bytes():
    # per cached token per KV head: INT4 KIVI = 2 x (64 code bytes + 16 metadata bytes)
    assert sizes.kivi_bytes_per_token_head(4) == 160
    assert sizes.kivi_bytes_per_token_head(2) == 96
    # INT3: 48 code bytes + 16 metadata bytes per tensor, 4 bits per value
    assert sizes.kivi_bytes_per_token_head(3) == 128
    assert sizes.kivi_bytes_per_token_head(3) * 8 / (2 * 128) == 4
    # the symmetric block is the page's 66-byte block, once for K and once for V
    assert sizes.block128_bytes_per_token_head() == 2 * EX["tbq4_block_bytes"]
    assert sizes.fp16_bytes_per_token_head() == 512
    # 4 bits + 2 x fp16 per 32 elements = 5 bits per value
    assert sizes.kivi_bytes_per_token_head(4) * 8 / (2 * 128) == 5


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_plane_sizes_match_per_token_bytes(bits):
    cfg = make_config(scheme="kivi", k_bits=bits, v_bits=bits, num_q_heads=4, num_kv_heads=2)
    B, T = 3, 32 * 1000
    sz = layout.plane_sizes(cfg, B, T)
    codes_meta = sum(sz[p] for p in (layout.K_HI, layout.V_HI, layout.K_META, layout.V_META))
    assert codes_meta == B * 2 * T * sizes.kivi_bytes_per_token_head(bits)
    assert sz[layout.K_WIN] == B * 2 * 160 * 256
    cfgb = make_config(scheme="block128", num_q_heads=4, num_kv_heads=2)
    szb = layout.plane_sizes(cfgb, B, T)
    assert sum(szb) == B * 2 * T * sizes.block128_bytes_per_token_head()
    # four 18-byte blocks per token and tensor
    cfgq = make_config(scheme="q4_0", num_q_heads=4, num_kv_heads=2)
    assert sum(layout.plane_sizes(cfgq, B, T)) == B * 2 * T * 2 * 4 * 18   # K and V
    # four 34-byte blocks per token and tensor (the page's Q8_0 row)
    cfg8 = make_config(scheme="q8_0", k_bits=8, v_bits=8, num_q_heads=4, num_kv_heads=2)
    assert sum(layout.plane_sizes(cfg8, B, T)) == B * 2 * T * 2 * 4 * 34
