"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Small shapes that span several tiles and chunks plus ragged tails; every
scheme and option; streaming appends with demotion; edge cases (empty cache,
all-window caches, one token)."""

import numpy as np
import pytest
import torch

from gpu_helpers import (build_pair, compare_planes, compare_dequant, compare_rope_table,
                         check_decode, say)
from quantized_decode_attention_02_amd import workloads as wl

pytestmark = pytest.mark.gpu

SIGNS = wl.random_signs(11)

VARIANTS = {
    "int4": dict(),
    "int2": dict(k_bits=2, v_bits=2),
    "int3": dict(k_bits=3, v_bits=3),
    "int3-hadamard-signed": dict(k_bits=3, v_bits=3, hadamard=True, **SIGNS),
    "int4-hadamard": dict(hadamard=True),
    "int4-prerope": dict(pre_rope=True, rope_theta=500000.0),
    "int2-prerope": dict(k_bits=2, v_bits=2, pre_rope=True, rope_theta=500000.0),
    "mixed-prerope": dict(hi_window=64, low_bits=2, pre_rope=True, rope_theta=500000.0),
    "mixed-hadamard": dict(hadamard=True, hi_window=96),
    "mixed": dict(hi_window=64),
    "mixed-int3": dict(hi_window=64, low_bits=3),
    "mixed-int3-hadamard-signed": dict(hadamard=True, hi_window=96, low_bits=3, **SIGNS),
    "mixed-hadamard-signed": dict(hadamard=True, hi_window=96, **SIGNS),
    "block128": None,
    "block128-plain": dict(hadamard=False),
    "block128-signed": dict(SIGNS),
    "block128-3bit": dict(k_bits=3, v_bits=3),
    "block128-3bit-plain": dict(k_bits=3, v_bits=3, hadamard=False),
    "tbq4": dict(),
    "tbq4-signed": dict(SIGNS),
    "q4_0": dict(),
    "q4_0-hadamard": dict(hadamard=True),
    "q8_0": dict(),
    "q8_0-hadamard-signed": dict(hadamard=True, **SIGNS),
}


def make_w(wid, variant, T, batch=2, hq=8, hkv=2, dist="normal", outliers=None):
    kw = VARIANTS[variant]
    if variant.startswith("block128"):
        cfg = wl._block128(**(kw or {}))
    elif variant.startswith("tbq4"):
        cfg = wl._tbq4(**kw)
    elif variant.startswith("q4_0"):
        cfg = wl._q4_0(**kw)
    elif variant.startswith("q8_0"):
        cfg = wl._q8_0(**kw)
    else:
        cfg = wl._kivi(**kw)
    return wl.custom(wid, batch, hq, hkv, T, cfg, dist=dist, outliers=outliers)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("T", [1, 31, 33, 128, 129, 159, 160, 161, 300, 4096 + 17])
def test_one_shot(variant, T):
    w = make_w(1000 + T, variant, T, outliers=("channels", 3, 20.0))
    say(f"one-shot {variant} T={T}")
    g, o, s, h = build_pair(w, [T], max_tokens=T + 40)
    compare_planes(g, o, s, h)
    compare_rope_table(g, o)
    compare_dequant(g, o, s, h)
    check_decode(g, o, w, s, h)


STREAMS = {
    "decode-steps": [200] + [1] * 70,
    "ragged": [5, 27, 1, 64, 100, 3, 31, 32, 33, 250, 7],
    "big-then-steps": [1500] + [1] * 40 + [77],
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("stream", list(STREAMS))
def test_streaming(variant, stream):
    chunks = STREAMS[stream]
    w = make_w(2000 + len(chunks), variant, sum(chunks), hq=4, dist="student3")
    say(f"streaming {variant} {stream}")
    g, o, s, h = build_pair(w, chunks, max_tokens=sum(chunks) + 5)
    compare_planes(g, o, s, h)
    compare_dequant(g, o, s, h)
    check_decode(g, o, w, s, h)


@pytest.mark.parametrize("variant", ["int4", "int3", "int4-prerope", "int2-prerope", "block128-3bit",
                                     "tbq4-signed", "q4_0", "q8_0"])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 1), (8, 8)])
def test_gqa_shapes(hq, hkv, variant):
    # every query-group size (1, 2, 4) of every decode kernel family
    w = make_w(3000 + hq * 10 + hkv, variant, 777, batch=3, hq=hq, hkv=hkv)
    say(f"gqa {variant} hq={hq} hkv={hkv}")
    g, o, s, h = build_pair(w, [777])
    compare_planes(g, o, s, h)
    compare_dequant(g, o, s, h)
    check_decode(g, o, w, s, h)


def test_empty_cache_and_query_position():
    w = make_w(3100, "int4-prerope", 500)
    from quantized_decode_attention_02_amd import kvq
    g0 = kvq.KVCache(wl.library_config(w), w["batch"], 64)
    out = g0.decode(torch.from_numpy(wl.queries(w)).cuda())
    assert torch.count_nonzero(out).item() == 0
    g, o, s, h = build_pair(w, [500])
    check_decode(g, o, w, s, h, q_pos=480)
    check_decode(g, o, w, s, h, sm_scale=0.03)


def test_partial_dequant_ranges():
    w = make_w(3200, "mixed-hadamard", 1000)
    g, o, s, h = build_pair(w, [600, 400])
    for t0, t1 in [(0, 1), (31, 33), (500, 1000), (871, 872), (999, 1000)]:
        compare_dequant(g, o, s, h, t0, t1)


def test_length_rollback_reappend_is_idempotent():
    # decode-step pattern: cache at T-1, append one token, decode; roll back to
    # T-1 and append the same token again
    w = make_w(3300, "int4", 4096)
    g, o, s, h = build_pair(w, [4095, 1])
    K1, V1 = wl.kv_tokens(w, 4095, 4096)
    before = [p.clone() if p is not None else None for p in g.planes]
    for _ in range(3):
        g.length = 4095
        g.append(torch.from_numpy(K1).cuda(), torch.from_numpy(V1).cuda())
    torch.cuda.synchronize()
    for a, b in zip(before, g.planes):
        if a is not None:
            assert torch.equal(a, b)
    check_decode(g, o, w, s, h)


def test_capacity_error_leaves_cache_untouched():
    from quantized_decode_attention_02_amd import kvq
    w = make_w(3400, "int4", 100)
    g, o, s, h = build_pair(w, [100], max_tokens=120)
    K, V = wl.kv_tokens(w, 100, 121)
    with pytest.raises(kvq.KvqError) as ei:
        g.append(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda())
    assert ei.value.status == -3 and g.length == 100
    compare_planes(g, o, s, h)


def tie_tokens(rng, T, hkv, q_levels, s, base):
    """fp16 keys and values [1, T, hkv, 128] whose quantization hits exact
    rounding ties: in every 32-token key group (per channel) and every 32-dim
    value slice (per token) one element is the minimum `base`, one is
    base + q_levels * s, and the rest are base + (k + 1/2) s, so that
    (x - z) / s = k + 1/2 exactly and round-to-nearest-even decides."""
    k = rng.integers(0, q_levels, size=(1, T, hkv, 128))
    x = base + (k + 0.5) * s
    kx = x.copy()
    kx[:, 0::32] = base                       # per-channel group minimum
    kx[:, 1::32] = base + q_levels * s        # and maximum
    vx = x.copy()
    vx[..., 0::32] = base                     # per-token slice minimum
    vx[..., 1::32] = base + q_levels * s      # and maximum
    assert np.all(kx.astype(np.float16).astype(np.float64) == kx)
    assert np.all(vx.astype(np.float16).astype(np.float64) == vx)
    return kx.astype(np.float16), vx.astype(np.float16)


@pytest.mark.parametrize("variant", ["int4", "int3", "int2", "block128-plain", "q8_0"])
def test_rounding_ties(variant):
    """Quotients exactly halfway between two codes: the kernels' reciprocal
    fast path must fall back to the division and round to even like the
    oracle (fp32 round-to-nearest-even on fl32((x - z) / s))."""
    from oracle.cache import OracleCache
    from quantized_decode_attention_02_amd import kvq
    T, hkv = 32 * 6 + 128, 2
    s = 3.0 / 32.0   # an fp16 scale that is not a power of two
    if variant == "q8_0":
        # 8-bit slices: a = 127 s in every 32-value slice, y = (k + 1/2) s with
        # k in -127 .. 126 (all exact in fp16)
        rng = np.random.default_rng(8)
        k = rng.integers(-127, 127, size=(1, T, hkv, 128))
        y = (k + 0.5) * s
        y[..., 0::32] = 127 * s
        K = y.astype(np.float16)
        V = (-y).astype(np.float16)
        assert np.all(K.astype(np.float64) == y)
    elif variant == "block128-plain":
        # symmetric: a = max |y| = 7 s, y = (k + 1/2) s with k in -7 .. 6
        rng = np.random.default_rng(7)
        k = rng.integers(-7, 7, size=(1, T, hkv, 128))
        y = (k + 0.5) * s
        y[..., 0] = 7 * s
        K = y.astype(np.float16)
        V = (-y).astype(np.float16)
        assert np.all(K.astype(np.float64) == y)
    else:
        q = {"int4": 15, "int3": 7, "int2": 3}[variant]
        K, V = tie_tokens(np.random.default_rng(5), T, hkv, q, s, base=-0.75)
    w = make_w(3000, variant, T, batch=1, hq=2 * hkv, hkv=hkv)
    cfg = wl.library_config(w)
    g = kvq.KVCache(cfg, 1, T)
    g.append(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda())
    o = OracleCache(cfg, 1, T)
    o.append(K, V)
    torch.cuda.synchronize()
    say(f"rounding ties {variant}")
    compare_planes(g, o, [0], list(range(hkv)))
    compare_dequant(g, o, [0], list(range(hkv)))


@pytest.mark.parametrize("variant", ["int4", "int4-prerope"])
def test_pairs_outnumber_waves(variant):
    """4096 (sequence, kv head) pairs: more than the waves one launch keeps
    resident (at most 3 work-groups of 4 waves on each of 256 compute
    units), so a wave works several pairs in turn, one at a time.  Sampled
    pairs, first and last included, against the oracle."""
    B, hkv, T = 512, 8, 32 * 4 + 128 + 5
    w = make_w(4000, variant, T, batch=B, hq=8, hkv=hkv)
    seqs, heads = [0, 1, 255, B - 1], [0, hkv - 1]
    g, o, s, h = build_pair(w, [T], seqs=seqs, heads=heads)
    say(f"{B * hkv} pairs {variant}")
    compare_planes(g, o, s, h)
    check_decode(g, o, w, s, h)


def counter_bytes(cache):
    # two 256-byte lines per (sequence, kv head): the decode chunk counters
    return 2 * cache.batch * cache.hkv * 256


@pytest.mark.parametrize("variant", ["int4", "mixed-hadamard", "int4-prerope", "block128"])
def test_workspace_counters_left_zero(variant):
    """Every decode call hands the workspace back with its chunk counters at
    zero, also when the partials launch runs several times before a merge;
    a workspace reused across caches of other sizes and tiers gives the same
    output as a fresh one.  The partial records are filled with garbage
    first: every slot must be written by the call that reads it."""
    w = make_w(5000, variant, 4096 + 300, batch=3, hq=8, hkv=2)
    g, o, s, h = build_pair(w, [4096 + 300])
    q = torch.from_numpy(wl.queries(w)).cuda()
    ref = g.decode(q).clone()
    ws = g.new_workspace()
    nctr = counter_bytes(g) // 4
    for rep in range(3):
        ws[nctr:].fill_(float("nan"))
        for _ in range(rep + 1):
            g.decode_partials(q, ws, torch.empty_like(ref))
        out = torch.empty_like(ref)
        g.decode_merge(q, ws, out)
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws.view(torch.int32)).item() == 0, "workspace not left zero"
        # waves claim chunks dynamically, so partials group tokens differently
        # from call to call: equal up to the last bits of the fp32 sums
        assert torch.allclose(out, ref, rtol=1e-4, atol=1e-5), f"repeat {rep}: output differs from a fresh workspace"
    # the same workspace (large enough) serves a smaller cache of another scheme
    w2 = make_w(5001, "int2", 700, batch=2, hq=4, hkv=1)
    g2, o2, s2, h2 = build_pair(w2, [700])
    assert g2.workspace_bytes() <= ws.numel() * 4
    q2 = torch.from_numpy(wl.queries(w2)).cuda()
    out2 = g2.decode(q2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws.view(torch.int32)).item() == 0
    # and back to the first cache, whose counter area the second one's
    # partials covered
    out3 = g.decode(q, workspace=ws)
    assert torch.allclose(out3, ref, rtol=1e-4, atol=1e-5)
    assert torch.allclose(out2, g2.decode(q2), rtol=1e-4, atol=1e-5)
    say(f"workspace counters {variant}: clean")


@pytest.mark.parametrize("variant", ["int4", "int3", "int2", "mixed-hadamard", "block128-plain",
                                     "block128-3bit-plain", "tbq4", "q4_0", "q8_0"])
def test_extreme_magnitudes(variant):
    """Tokens whose magnitudes span fp16 from the subnormal range (1e-6) to
    ~1e4, all-zero tokens and constant tokens: scales that are fp16
    subnormals or large, norms that clamp at 65504 (TBQ4), degenerate groups.
    Planes and dequant bit-exact, attention within tolerance."""
    from oracle.cache import OracleCache
    from quantized_decode_attention_02_amd import kvq
    T, hkv = 32 * 8 + 128 + 7, 2
    rng = np.random.default_rng(41)
    mag = 10.0 ** rng.uniform(-6.0, 3.5, size=(1, T, hkv, 1))
    K = rng.standard_normal((1, T, hkv, 128)) * mag
    V = rng.standard_normal((1, T, hkv, 128)) * 10.0 ** rng.uniform(-6.0, 3.5, size=(1, T, hkv, 1))
    K[:, 5], V[:, 9] = 0.0, 0.0                      # all-zero tokens
    K[:, 40], V[:, 41] = 0.5, -2.0                   # constant tokens
    K[:, 64:96, :, 7] = 1e-7                         # a channel group in the subnormal range
    K, V = K.astype(np.float16), V.astype(np.float16)
    assert np.all(np.isfinite(K)) and np.all(np.isfinite(V))
    w = make_w(3700, variant, T, batch=1, hq=2 * hkv, hkv=hkv)
    cfg = wl.library_config(w)
    g = kvq.KVCache(cfg, 1, T)
    g.append(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda())
    o = OracleCache(cfg, 1, T)
    o.append(K, V)
    torch.cuda.synchronize()
    say(f"extreme magnitudes {variant}")
    compare_planes(g, o, [0], list(range(hkv)))
    compare_dequant(g, o, [0], list(range(hkv)))
    check_decode(g, o, w, [0], list(range(hkv)))


@pytest.mark.parametrize("variant", ["int4", "mixed-hadamard", "int4-prerope", "q4_0"])
def test_graph_replay_matches_eager(variant):
    """A decode step (append one token, split-K partials, merge) captured in a
    HIP graph and replayed: the library records only its own kernels (no
    allocation, memset or synchronization), so every replay must give the
    eager step's planes and output.  Replays are interleaved with eager work
    and synchronizations; outputs agree to 1e-4 relative (dynamic chunk claims
    regroup the fp32 sums), planes bit for bit."""
    from quantized_decode_attention_02_amd import kvq
    T = 4096 + 33
    w = make_w(3800, variant, T, batch=2, hq=8, hkv=2)
    g, o, s, h = build_pair(w, [T - 1, 1])
    K1, V1 = wl.kv_tokens(w, T - 1, T)
    k1, v1 = torch.from_numpy(K1).cuda(), torch.from_numpy(V1).cuda()
    q = torch.from_numpy(wl.queries(w)).cuda()
    ws = g.new_workspace()
    out = torch.empty((w["batch"], w["num_q_heads"], 128), dtype=torch.float32, device="cuda")

    def step():
        g.length = T - 1
        g.append(k1, v1)
        g.decode(q, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    planes = [p.clone() if p is not None else None for p in g.planes]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    say(f"graph replay {variant}")
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.allclose(out, ref, rtol=1e-4, atol=1e-5), f"replay {rep}: output differs from eager"
        for a, b in zip(planes, g.planes):
            if a is not None:
                assert torch.equal(a, b), f"replay {rep}: planes differ"
        eager = g.decode(q)                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.allclose(eager, ref, rtol=1e-4, atol=1e-5)
    g.length = T
    check_decode(g, o, w, s, h)
