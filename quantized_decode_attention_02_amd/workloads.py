"""Seeded synthetic workloads: cache shapes and input tensors.

This module only draws random numbers and shapes them; it holds no arithmetic
of the quantization or attention method.  The tests, the benchmark and the CPU
oracle's callers all take their inputs from here, so the GPU library and the
oracle always see the same fp16 arrays.

Recipe:
  * every 4096-token block of one (workload, sequence b, kv head h, tensor) is
    drawn from its own PCG64 stream seeded with
    SeedSequence([20261202, workload_id, b, h, tensor, block]), tensor 0 = keys,
    1 = values; any token range can be regenerated without drawing the rest;
  * draws are float64: standard normal, or Student-t with 3 degrees of freedom
    (unscaled, clipped to +-60000 so every value is a finite fp16);
  * key outliers multiply whole channels in float64 before the single cast to
    fp16 (same channels for every token and sequence);
  * queries: per sequence b, one standard-normal [Hq, 128] draw from
    SeedSequence([20261202, workload_id, b, 0, 2, 0]), cast to fp16;
  * outlier choice: a PCG64 stream seeded with
    SeedSequence([20261202, workload_id, 0, 0, 3, 0]): either the first n
    entries of a permutation of the 128 channels (shared by all heads) or n
    (head, channel) pairs drawn without replacement from Hkv * 128.

The five named workloads are the cache shapes this project is measured on:
a single INT4 head with four x20 outlier channels; a Llama-2-7B-shaped MHA
layer; a GQA layer with keys stored before RoPE; a long mixed INT4/INT2
Hadamard cache with heavy-tailed values; a chunked prefill into 66-byte/128
blocks after a Hadamard rotation.
"""

import concurrent.futures as cf
import os

import numpy as np

BASE_SEED = 20261202
BLOCK = 4096
D = 128
TENSOR_K, TENSOR_V, TENSOR_Q, TENSOR_SEL = 0, 1, 2, 3


def _kivi(**kw):
    c = dict(scheme="kivi", k_bits=4, v_bits=4, low_bits=2, hi_window=-1,
             window=128, hadamard=False, pre_rope=False, rope_theta=10000.0)
    c.update(kw)
    return c


def _block128(**kw):
    c = dict(scheme="block128", k_bits=4, v_bits=4, low_bits=2, hi_window=-1,
             window=0, hadamard=True, pre_rope=False, rope_theta=10000.0)
    c.update(kw)
    return c


def _q4_0(**kw):
    c = dict(scheme="q4_0", k_bits=4, v_bits=4, low_bits=2, hi_window=-1,
             window=0, hadamard=False, pre_rope=False, rope_theta=10000.0)
    c.update(kw)
    return c


def _q8_0(**kw):
    return _q4_0(**dict(dict(scheme="q8_0", k_bits=8, v_bits=8), **kw))


def _tbq4(**kw):
    c = dict(scheme="tbq4", k_bits=4, v_bits=4, low_bits=2, hi_window=-1,
             window=0, hadamard=True, pre_rope=False, rope_theta=10000.0)
    c.update(kw)
    return c


def random_signs(seed):
    """Sign masks of a randomized Hadamard rotation: dict(sign_in=[4 words],
    sign_out=[4 words]), 128 seeded fair coin flips each (bit i of word i // 32
    set: coordinate i negated).  Inputs only; what they do is the library's and
    the oracle's business."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 0x5167, seed])))
    words = rng.integers(0, 1 << 32, size=8, dtype=np.uint64)
    return dict(sign_in=[int(x) for x in words[:4]], sign_out=[int(x) for x in words[4:]])


WORKLOADS = [
    dict(id=0, name="int4-kivi-b1-h1-t4096-outlier4x20",
         batch=1, num_q_heads=1, num_kv_heads=1, tokens=4096, prefill=0,
         cfg=_kivi(), dist="normal", outliers=("channels", 4, 20.0)),
    dict(id=1, name="int4-kivi-llama2-7b-mha32-b8-t32768-outlier2pct-x15",
         batch=8, num_q_heads=32, num_kv_heads=32, tokens=32768, prefill=0,
         cfg=_kivi(), dist="normal", outliers=("pairs", 82, 15.0)),
    dict(id=2, name="int4-kivi-prerope-gqa32x8-b16-t131072",
         batch=16, num_q_heads=32, num_kv_heads=8, tokens=131072, prefill=0,
         cfg=_kivi(pre_rope=True, rope_theta=500000.0), dist="normal", outliers=None),
    dict(id=3, name="int4x4096-int2-hadamard-gqa32x8-b4-t262144-student3",
         batch=4, num_q_heads=32, num_kv_heads=8, tokens=262144, prefill=0,
         cfg=_kivi(hadamard=True, hi_window=4096), dist="student3", outliers=None),
    dict(id=4, name="block128-hadamard-gqa32x8-b32-t65536+8192",
         batch=32, num_q_heads=32, num_kv_heads=8, tokens=65536 + 8192, prefill=8192,
         cfg=_block128(), dist="normal", outliers=None),
]
# TBQ4 proper (Lloyd-Max levels, randomized Hadamard) at the block-128 shape
WORKLOADS.append(
    dict(id=5, name="tbq4-randomized-hadamard-gqa32x8-b32-t65536+8192",
         batch=32, num_q_heads=32, num_kv_heads=8, tokens=65536 + 8192, prefill=8192,
         cfg=_tbq4(**random_signs(5)), dist="normal", outliers=None))
# Q4_0-style 32-value blocks (the format table's baseline) at the same shape
WORKLOADS.append(
    dict(id=6, name="q4_0-gqa32x8-b32-t65536+8192",
         batch=32, num_q_heads=32, num_kv_heads=8, tokens=65536 + 8192, prefill=8192,
         cfg=_q4_0(), dist="normal", outliers=None))
# the 3-bit 50-byte block (format table row "3 bity (50 B / 128)") at the same shape
WORKLOADS.append(
    dict(id=7, name="block50-3bit-hadamard-gqa32x8-b32-t65536+8192",
         batch=32, num_q_heads=32, num_kv_heads=8, tokens=65536 + 8192, prefill=8192,
         cfg=_block128(k_bits=3, v_bits=3), dist="normal", outliers=None))
# Q8_0-style 32-value blocks (the format table's 8-bit row) at the block-128 shape
WORKLOADS.append(
    dict(id=9, name="q8_0-gqa32x8-b32-t65536+8192",
         batch=32, num_q_heads=32, num_kv_heads=8, tokens=65536 + 8192, prefill=8192,
         cfg=_q8_0(), dist="normal", outliers=None))
# the mixed-precision long-context shape with its older tier at INT3 instead of INT2
WORKLOADS.append(
    dict(id=10, name="int4x4096-int3-hadamard-gqa32x8-b4-t262144-student3",
         batch=4, num_q_heads=32, num_kv_heads=8, tokens=262144, prefill=0,
         cfg=_kivi(hadamard=True, hi_window=4096, low_bits=3), dist="student3", outliers=None))
# INT3 KIVI (the INT3 cache of [troisinh]'s title) at the Llama-2-7B layer shape
WORKLOADS.append(
    dict(id=8, name="int3-kivi-llama2-7b-mha32-b8-t32768-outlier2pct-x15",
         batch=8, num_q_heads=32, num_kv_heads=32, tokens=32768, prefill=0,
         cfg=_kivi(k_bits=3, v_bits=3), dist="normal", outliers=("pairs", 82, 15.0)))


def workload(key):
    """A workload by id or name."""
    for w in WORKLOADS:
        if w["id"] == key or w["name"] == key:
            return w
    raise KeyError(key)


def custom(wid, batch, num_q_heads, num_kv_heads, tokens, cfg, dist="normal",
           outliers=None, prefill=0, name=None):
    """An ad-hoc workload (test shapes); ``wid`` keys its random streams."""
    return dict(id=wid, name=name or f"custom-{wid}", batch=batch,
                num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, tokens=tokens,
                prefill=prefill, cfg=dict(cfg), dist=dist, outliers=outliers)


def library_config(w):
    """The config dict both the binding and the oracle build their own config from."""
    c = dict(w["cfg"])
    c.update(head_dim=D, num_q_heads=w["num_q_heads"], num_kv_heads=w["num_kv_heads"])
    return c


def _rng(wid, b, h, tensor, blk):
    ss = np.random.SeedSequence([BASE_SEED, wid, b, h, tensor, blk])
    return np.random.Generator(np.random.PCG64(ss))


def outlier_scale(w):
    """float64 [Hkv, 128] channel multipliers for keys (ones without outliers)."""
    scale = np.ones((w["num_kv_heads"], D), dtype=np.float64)
    o = w.get("outliers")
    if not o:
        return scale
    kind, n, factor = o
    rng = _rng(w["id"], 0, 0, TENSOR_SEL, 0)
    if kind == "channels":
        ch = rng.permutation(D)[:n]
        scale[:, ch] = factor
    elif kind == "pairs":
        flat = rng.choice(w["num_kv_heads"] * D, size=n, replace=False)
        scale.reshape(-1)[flat] = factor
    else:
        raise ValueError(kind)
    return scale


def kv_block(w, b, h, tensor, blk, scale=None):
    """fp16 [4096, 128]: tokens [blk*4096, (blk+1)*4096) of one head's keys or values."""
    rng = _rng(w["id"], b, h, tensor, blk)
    if w["dist"] == "normal":
        x = rng.standard_normal((BLOCK, D))
    elif w["dist"] == "student3":
        x = np.clip(rng.standard_t(3, size=(BLOCK, D)), -60000.0, 60000.0)
    else:
        raise ValueError(w["dist"])
    if tensor == TENSOR_K:
        s = outlier_scale(w) if scale is None else scale
        x = x * s[h][None, :]
    return x.astype(np.float16)


def kv_range(w, b, h, tensor, t0, t1, scale=None):
    """fp16 [t1 - t0, 128] for one (sequence, head, tensor)."""
    if t1 <= t0:
        return np.zeros((0, D), np.float16)
    parts = []
    for blk in range(t0 // BLOCK, (t1 - 1) // BLOCK + 1):
        x = kv_block(w, b, h, tensor, blk, scale)
        lo = max(t0, blk * BLOCK) - blk * BLOCK
        hi = min(t1, (blk + 1) * BLOCK) - blk * BLOCK
        parts.append(x[lo:hi])
    return np.concatenate(parts, axis=0)


def _threads():
    n = os.cpu_count() or 4
    try:
        n = min(n, len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    return max(1, min(16, n))


def kv_tokens(w, t0, t1, seqs=None, heads=None, threads=None):
    """Keys and values fp16 [len(seqs), t1 - t0, len(heads), 128] (token-major).

    ``seqs`` / ``heads`` select sequences and kv heads (default: all)."""
    seqs = list(range(w["batch"])) if seqs is None else list(seqs)
    heads = list(range(w["num_kv_heads"])) if heads is None else list(heads)
    n = t1 - t0
    K = np.empty((len(seqs), n, len(heads), D), np.float16)
    V = np.empty_like(K)
    scale = outlier_scale(w)
    jobs = [(i, b, j, h) for i, b in enumerate(seqs) for j, h in enumerate(heads)]

    def run(job):
        i, b, j, h = job
        K[i, :, j, :] = kv_range(w, b, h, TENSOR_K, t0, t1, scale)
        V[i, :, j, :] = kv_range(w, b, h, TENSOR_V, t0, t1, scale)

    nt = threads or _threads()
    if nt == 1 or len(jobs) == 1:
        for job in jobs:
            run(job)
    else:
        with cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(run, jobs))
    return K, V


def queries(w, seqs=None):
    """fp16 [len(seqs), Hq, 128] decode queries."""
    seqs = list(range(w["batch"])) if seqs is None else list(seqs)
    out = np.empty((len(seqs), w["num_q_heads"], D), np.float16)
    for i, b in enumerate(seqs):
        out[i] = _rng(w["id"], b, 0, TENSOR_Q, 0).standard_normal((w["num_q_heads"], D)).astype(np.float16)
    return out
