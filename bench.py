"""Decode-step benchmark: effective KV GB/s of decode attention over the INT4 cache.

One step is one pass of the whole hot path on every sequence of the batch:
append one fp16 token per sequence (its key/value go to the fp16 window, and
the 32-token group leaving the window is quantized: per-channel keys,
per-token values, packed INT4), then single-query decode attention over the
whole packed cache (split-K kernel + merge).  The cache starts at T - 1 tokens
and every step rolls the length back to T - 1 before appending the same token,
so every step does identical work and decode always attends T tokens.

Reported (one JSON line on stdout):
  value        algorithmic decode bytes (codes + fp16 scales/zeros + fp16
               window) / step time, GB/s; inputs resident in HBM
  value is measured over back-to-back steps, where the tail of one step's
  reads is still in the 256 MB Infinity Cache when the next step starts.
  roofline     the decode call (split-K partials kernel + merge kernel), cold:
               algorithmic bytes per call / its average duration (HIP events
               on the launch stream) over --cold-steps extra steps, each after
               a 512 MB read that sweeps the Infinity Cache and the L2s,
               against the 8 TB/s HBM peak (the back-to-back figure and the
               partials kernel alone are reported beside it); traffic =
               counter-measured HBM bytes per call (null when the kernel
               sources changed since)
  append       (chunked-prefill workloads) the workload's multi-token append
               timed apart: (fp16 read + packed write) bytes / time
  cpu_baseline the CPU oracle on the same step (append one token + dequantize
               + fp64 attention) over a bounded sample of the workload's
               (sequence, kv head) pairs, one process per core

    python bench.py [--steps K] [--warmup W] [--workload ID] [--sub-workloads 1,4]
                    [--no-cpu-baseline]

The headline workload defaults to the largest cache that one GPU holds (the
pre-RoPE GQA layer, 16 x 8 kv heads at T = 131072); the Llama-2-7B-shaped MHA
layer and the chunked-prefill block cache follow as sub-records.
"""

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from quantized_decode_attention_02_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn effective KV GB/s (% of HBM peak) + attended tokens/s, INT4, 1 GPU"

# HBM bytes of one decode call from hardware counters: rocprofv3 --pmc
# FETCH_SIZE, then WRITE_SIZE (KiB per dispatch), for the partials kernel and
# the merge kernel of the call, each scaled by what the counter reads for a
# plain 1 GiB device copy (FETCH_SIZE reads 524300 KiB for 1048576 KiB moved:
# x2.0; WRITE_SIZE reads 1048576 KiB: x1.0).  Valid only for the kernel
# sources they were taken with (sha256 over COUNTER_SOURCES); any change there
# reports traffic as null until the counters are taken again.
COUNTER_SOURCES = ["quantized_decode_attention_02_amd/csrc/decode_mfma.hip",
                   "quantized_decode_attention_02_amd/csrc/decode_rope.hip",
                   "quantized_decode_attention_02_amd/csrc/decode.hip",
                   "quantized_decode_attention_02_amd/csrc/decode_common.h",
                   "quantized_decode_attention_02_amd/csrc/kvq_device.h",
                   "quantized_decode_attention_02_amd/csrc/kvq_internal.h",
                   "quantized_decode_attention_02_amd/csrc/kvq.cpp"]
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0
# workload id -> {"sources_sha256": ..., "kernels": {kernel: [fetch_kib, write_kib]}}
COUNTERS = {
    1: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [1077.5, 2208.0], "decode_mfma_kernel<1, 4, false, false, false>": [664775.4, 4258.2]}},
    2: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [2661.6, 5456.0], "decode_rope_kernel<4, 4>": [1324162.2, 9536.3]}},
    3: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [3293.5, 6564.0], "decode_mfma_kernel<4, 2, false, false, false>": [387172.8, 5410.0], "decode_mfma_kernel<4, 4, false, false, false>": [11764.9, 2503.2]}},
    4: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [3205.5, 6752.0], "decode_mfma_kernel<4, 4, true, false, false>": [1217705.3, 11192.2]}},
    5: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [3205.5, 6752.0], "decode_mfma_kernel<4, 4, true, true, false>": [1217776.5, 11192.0]}},
    6: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [2149.5, 4672.0], "decode_mfma_kernel<4, 4, true, false, true>": [1328328.3, 9000.0]}},
    7: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [3205.5, 6752.0], "decode_mfma_kernel<4, 3, true, false, false>": [922800.3, 11192.0]}},
    8: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [1077.7, 2208.0], "decode_mfma_kernel<1, 3, false, false, false>": [532069.4, 4256.3]}},
    9: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [1125.6, 2592.0], "decode_mfma_kernel<4, 8, true, false, true>": [2507460.7, 6808.0]}},
    10: {"sources_sha256": "c1c85e570d5573762f42d986c927dd9b29fefb7c787fc01fd3d90f02dba42ba2",
        "kernels": {"decode_merge_kernel": [3293.5, 6564.0], "decode_mfma_kernel<4, 3, false, false, false>": [516146.8, 5410.0], "decode_mfma_kernel<4, 4, false, false, false>": [11765.0, 2503.8]}},
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


BLOCK_SCHEMES = ("block128", "tbq4", "q4_0", "q8_0")   # per-token blocks, no window


def block_bytes(cfg):
    """Bytes of one token's 128 values of one tensor in a block scheme."""
    if cfg["scheme"] == "q4_0":
        return 4 * 18
    if cfg["scheme"] == "q8_0":
        return 4 * 34
    return 50 if cfg["k_bits"] == 3 else 66


def tier_map(cfg, T):
    if cfg["scheme"] in BLOCK_SCHEMES:
        return T, 0
    Tq = max(0, ((T - 128) // 32) * 32)
    hi_start = 0 if cfg["hi_window"] < 0 else max(0, Tq - cfg["hi_window"])
    return Tq, hi_start


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in COUNTER_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(wid):
    """Counter-measured HBM bytes per decode call (partials + merge), or None
    when the kernel sources differ from those the counters were taken with."""
    c = COUNTERS.get(wid)
    if c is None or c["sources_sha256"] != sources_sha256():
        return None
    return int(sum(f * FETCH_FACTOR + wr * WRITE_FACTOR for f, wr in c["kernels"].values()) * 1024)


def describe_cache(cfg):
    if cfg["scheme"] == "q8_0":
        return ("Q8_0-style symmetric 8-bit blocks of 32 values + fp16 scale (34 B/32)"
                + (" after a Hadamard-128 rotation" if cfg["hadamard"] else "") + ", no fp16 window")
    if cfg["scheme"] == "q4_0":
        return ("Q4_0-style symmetric 4-bit blocks of 32 values + fp16 scale (18 B/32)"
                + (" after a Hadamard-128 rotation" if cfg["hadamard"] else "") + ", no fp16 window")
    if cfg["scheme"] == "tbq4":
        return ("TBQ4: 4-bit indices into 16 Lloyd-Max levels of N(0, 1/sqrt(128)) + fp16 norm "
                "(66 B/128) after a " + ("randomized " if cfg.get("sign_in") else "")
                + "Hadamard-128 rotation, no fp16 window")
    if cfg["scheme"] == "block128" and cfg["k_bits"] == 3:
        return ("symmetric 3-bit blocks of 128 values + fp16 scale (50 B/128)"
                + (" after a Hadamard-128 rotation" if cfg["hadamard"] else "") + ", no fp16 window")
    if cfg["scheme"] == "block128":
        return ("symmetric 4-bit blocks of 128 values + fp16 scale (66 B/128)"
                + (" after a Hadamard-128 rotation" if cfg["hadamard"] else "") + ", no fp16 window")
    tiers = (f"INT{cfg['k_bits']} newest {cfg['hi_window']} quantized tokens, INT{cfg['low_bits']} older"
             if cfg["hi_window"] >= 0 else f"INT{cfg['k_bits']}")
    extra = ""
    if cfg["hadamard"]:
        extra += ", Hadamard-128 on K and V"
    if cfg["pre_rope"]:
        extra += f", keys pre-RoPE (split-half RoPE, theta {cfg['rope_theta']:g}, at decode)"
    return (f"KIVI {tiers}: K per-channel g32, V per-token g32, fp16 scale+zero, "
            f"{cfg['window']}-token fp16 window{extra}")


def decode_bytes(w, T):
    """Algorithmic bytes one decode call must read: codes, fp16 scales and
    zeros, the fp16 window; per (sequence, kv head), times all pairs."""
    cfg = w["cfg"]
    pairs = w["batch"] * w["num_kv_heads"]
    Tq, hi_start = tier_map(cfg, T)
    if cfg["scheme"] in BLOCK_SCHEMES:
        per_pair = T * 2 * block_bytes(cfg)
    else:
        hi = Tq - hi_start
        lo = hi_start
        per_pair = hi * 2 * 128 * cfg["k_bits"] // 8 + lo * 2 * 128 * cfg["low_bits"] // 8
        per_pair += (Tq // 32) * 2 * 512          # key (s, z) per channel + value (s, z) per token
        per_pair += (T - Tq) * 2 * 128 * 2         # fp16 window, keys and values
    return pairs * per_pair


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, one process per core.

def _cpu_worker(args):
    wid, pairs, T, barrier, q_out = args
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle.cache import OracleCache
    w = wl.workload(wid)
    G = w["num_q_heads"] // w["num_kv_heads"]
    cfg = dict(wl.library_config(w), num_q_heads=G, num_kv_heads=1)
    built = []
    t_build = 0.0
    for b, h in pairs:
        K, V = wl.kv_tokens(w, 0, T, seqs=[b], heads=[h], threads=1)
        oc = OracleCache(cfg, 1, T)
        t0 = time.perf_counter()
        oc.append(K[:, :T - 1], V[:, :T - 1])
        t_build += time.perf_counter() - t0
        q = wl.queries(w, seqs=[b])[:, h * G:(h + 1) * G]
        built.append((oc, q, K[:, T - 1:], V[:, T - 1:]))
    barrier.wait()
    t0 = time.time()
    for oc, q, k1, v1 in built:
        oc.append(k1, v1)
        oc.decode(q)
    t1 = time.time()
    q_out.put((t0, t1, t_build, len(built)))


def cpu_baseline(w, T, n_pairs, workers):
    """The oracle timed on the same step as the GPU (append the last token,
    which quantizes the group leaving the window, then dequantize + fp64
    attention over the whole cache) for a sample of (sequence, kv head)
    pairs, one process per core, all started together."""
    pairs_all = [(b, h) for b in range(w["batch"]) for h in range(w["num_kv_heads"])]
    rng = np.random.default_rng(12345)
    pick = [pairs_all[i] for i in sorted(rng.choice(len(pairs_all), min(n_pairs, len(pairs_all)),
                                                    replace=False))]
    workers = max(1, min(workers, len(pick)))
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(workers + 1)
    q_out = ctx.Queue()
    chunks = [pick[i::workers] for i in range(workers)]
    procs = [ctx.Process(target=_cpu_worker, args=((w["id"], c, T, barrier, q_out),)) for c in chunks]
    for p in procs:
        p.start()
    barrier.wait()
    res = [q_out.get() for _ in procs]
    for p in procs:
        p.join()
    start = min(r[0] for r in res)
    end = max(r[1] for r in res)
    per_pair_bytes = decode_bytes(dict(w, batch=1, num_kv_heads=1), T)
    nbytes = per_pair_bytes * len(pick)
    secs = end - start
    cpu_s = sum(r[1] - r[0] for r in res)
    return {
        "value": nbytes / secs / 1e9,
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"{len(pick)} of {len(pairs_all)} (sequence, kv head) pairs at T={T}, the same "
                   f"step as the GPU (append 1 token + dequantize + fp64 attention) over "
                   f"{nbytes / 1e9:.3f} GB of the cache: {secs:.2f} s wall, {cpu_s:.1f} CPU-s on "
                   f"{workers} processes; building the {T - 1}-token caches took "
                   f"{sum(r[2] for r in res):.1f} CPU-s (untimed)"),
        "attended_tokens_per_s": len(pick) * T / secs,
    }


# ---------------------------------------------------------------------------

def measure(w, args, dev, headline):
    """Build the workload's cache on the GPU and time it.  Returns the figures
    of one workload: back-to-back steps, the cold decode call (partials +
    merge, HIP events on the launch stream, caches swept before each launch)
    and, for chunked-prefill workloads, the multi-token append."""
    import torch
    from quantized_decode_attention_02_amd import kvq

    T = w["tokens"]
    cfg = wl.library_config(w)
    decode_only = args.decode_only or (w["cfg"]["scheme"] == "kivi" and w["cfg"]["hi_window"] >= 0)
    log(f"workload {w['name']}: generating {T} tokens x {w['batch']} seqs x {w['num_kv_heads']} heads")
    K0, V0 = wl.kv_tokens(w, 0, T - 1)
    K1, V1 = wl.kv_tokens(w, T - 1, T)
    q = torch.from_numpy(wl.queries(w)).to(dev)
    log("uploading")
    k0, v0 = torch.from_numpy(K0).to(dev), torch.from_numpy(V0).to(dev)
    del K0, V0
    k1, v1 = torch.from_numpy(K1).to(dev), torch.from_numpy(V1).to(dev)
    cache = kvq.KVCache(cfg, w["batch"], T)
    cache.append(k0, v0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def ev_pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    build_rec = None
    if w["cfg"]["scheme"] == "kivi":
        # the one-shot build of the T - 1 token cache from an empty one (a
        # prefill: group quantization, fp16 window, RoPE table) timed apart
        ev_b = [ev_pair() for _ in range(3)]
        for i in range(4):
            cache.length = 0
            if i >= 1:
                ev_b[i - 1][0].record(stream)
            cache.append(k0, v0)
            if i >= 1:
                ev_b[i - 1][1].record(stream)
        torch.cuda.synchronize()
        b_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_b]))
        rd = w["batch"] * w["num_kv_heads"] * (T - 1) * 2 * 128 * 2
        wr = decode_bytes(w, T - 1)
        build_rec = {"tokens_per_seq": T - 1, "ms": round(b_ms, 5), "read_bytes": rd, "write_bytes": wr,
                     "gbs": round((rd + wr) / (b_ms / 1e3) / 1e9, 2),
                     "frac": round((rd + wr) / (b_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"one-shot build of {T - 1} tokens: {b_ms:.4f} ms")
    chunk = None
    if w.get("prefill") and w["cfg"]["scheme"] in BLOCK_SCHEMES:
        n = w["prefill"]   # the workload's chunked-prefill append: its last n tokens
        chunk = (n, torch.cat([k0[:, T - n:], k1], 1).contiguous(), torch.cat([v0[:, T - n:], v1], 1).contiguous())
    del k0, v0
    log(f"cache built: {cache.length} tokens")

    append_rec = None
    if chunk is not None:
        # the chunked-prefill append timed apart (it rewrites the same blocks)
        n, kp, vp = chunk
        ev_a = [ev_pair() for _ in range(10)]
        for i in range(12):
            cache.length = T - n
            if i >= 2:
                ev_a[i - 2][0].record(stream)
            cache.append(kp, vp)
            if i >= 2:
                ev_a[i - 2][1].record(stream)
        torch.cuda.synchronize()
        a_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_a]))
        rd = w["batch"] * n * w["num_kv_heads"] * 2 * 128 * 2
        wr = w["batch"] * n * w["num_kv_heads"] * 2 * block_bytes(w["cfg"])
        append_rec = {"tokens_per_seq": n, "ms": round(a_ms, 5), "read_bytes": rd, "write_bytes": wr,
                      "gbs": round((rd + wr) / (a_ms / 1e3) / 1e9, 2),
                      "frac": round((rd + wr) / (a_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"chunked append of {n} tokens: {a_ms:.4f} ms")
        del kp, vp, chunk
        cache.length = T - 1

    cache.append(k1, v1)
    ws = cache.new_workspace()
    out = torch.empty((w["batch"], w["num_q_heads"], 128), dtype=torch.float32, device=dev)

    def step(ev=None):
        # ev: (start, after partials, after merge) on the launch stream
        if not decode_only:
            cache.length = T - 1
            cache.append(k1, v1)
        if ev is not None:
            ev[0].record(stream)
        cache.decode_partials(q, ws, out)
        if ev is not None:
            ev[1].record(stream)
        cache.decode_merge(q, ws, out)
        if ev is not None:
            ev[2].record(stream)

    def ev3():
        return tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))

    steps = args.steps if headline else args.sub_steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [ev3() for _ in range(steps)]
    log(f"timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    call_warm = float(np.mean([a.elapsed_time(c) for a, b, c in events]))

    # The same steps with the 256 MB Infinity Cache and the L2s swept before
    # each one by reading a 512 MB buffer (clean lines, so no write-back
    # competes with the kernels), outside the events.  The roofline figure
    # uses these cold decode calls.
    scratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    cold = args.cold_steps if headline else max(5, args.cold_steps // 2)
    ev_c = [ev3() for _ in range(cold)]
    for e in ev_c:
        scratch.sum()
        step(e)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(c) for a, b, c in ev_c]
    part_ms = [a.elapsed_time(b) for a, b, c in ev_c]
    merge_ms = [b.elapsed_time(c) for a, b, c in ev_c]
    del scratch

    nbytes = decode_bytes(w, T)
    call = float(np.mean(call_ms))
    kname = "decode_rope_kernel" if w["cfg"]["pre_rope"] else "decode_mfma_kernel"
    rec = {
        "workload": w["name"],
        "decode_bytes": nbytes,
        "ms_per_step": round(ms_step, 4),
        "step": ("split-K decode + merge" if decode_only else "append 1 token/seq + split-K decode + merge"),
        "value": round(nbytes / (ms_step / 1e3) / 1e9, 2),
        "attended_tokens_per_s": round(w["batch"] * T / (ms_step / 1e3), 1),
        "bytes_per_attended_token": round(nbytes / (w["batch"] * T), 2),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (call / 1e3) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (call / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(w["id"]),
                     "traffic_unit": "HBM bytes per decode call, partials + merge "
                                     "(FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                     "algorithmic_bytes": nbytes,
                     "kernel": f"kvq_decode_attn: {kname} (split-K partials) + decode_merge_kernel",
                     "kernel_ms_avg": round(call, 5),
                     "kernel_ms_p10_p90": [round(float(np.percentile(call_ms, 10)), 5),
                                           round(float(np.percentile(call_ms, 90)), 5)],
                     "partials_ms_avg": round(float(np.mean(part_ms)), 5),
                     "merge_ms_avg": round(float(np.mean(merge_ms)), 5),
                     "caches": "Infinity Cache and L2 swept (512 MB read) before each timed call",
                     "kernel_ms_avg_back_to_back": round(call_warm, 5),
                     "achieved_back_to_back": round(nbytes / (call_warm / 1e3) / 1e9, 2)},
        "cache": describe_cache(w["cfg"]),
    }
    if append_rec is not None:
        rec["append"] = append_rec
    if build_rec is not None:
        rec["build"] = build_rec
    log(f"{w['name']}: step {ms_step:.4f} ms, decode call {call:.4f} ms cold "
        f"({rec['roofline']['frac']:.3f} of peak)")
    del cache, ws, out, q, k1, v1
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps, each after a 512 MB read that sweeps the caches; the "
                         "roofline figure is their decode call's average")
    ap.add_argument("--workload", type=int, default=2,
                    help="headline workload (default: the largest single-GPU cache, the "
                         "pre-RoPE GQA layer at T=131072)")
    ap.add_argument("--sub-workloads", default="1,4",
                    help="comma-separated workloads measured after the headline and reported "
                         "under 'sub' (empty: none)")
    ap.add_argument("--sub-steps", type=int, default=20)
    ap.add_argument("--cpu-pairs", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time decode (partials + merge) on the built T-token cache without the "
                         "per-step append (caches with a high-bit window always run this way: "
                         "replaying the same append would demote a group twice)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for "
                         "hardware byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    w = wl.workload(args.workload)
    T = w["tokens"]
    subs = [int(x) for x in args.sub_workloads.split(",") if x.strip()]

    cpu = None
    if not args.no_cpu_baseline:
        # one process per host core, at most 16 (the host share of one GPU on
        # the measurement machines, whatever the affinity mask shows)
        affinity = len(os.sched_getaffinity(0))
        workers = min(16, affinity)
        log(f"cpu baseline: {args.cpu_pairs} pairs on {workers} processes "
            f"(affinity {affinity}, cpu_count {os.cpu_count()})")
        cpu = cpu_baseline(w, T, args.cpu_pairs, workers)
        cpu["host_cpus"] = {"affinity": affinity, "cpu_count": os.cpu_count()}
        log(f"cpu baseline {cpu['value']:.3f} GB/s")

    import torch

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    head = measure(w, args, dev, headline=True)
    sub = [measure(wl.workload(s), args, dev, headline=False) for s in subs if s != args.workload]

    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w["name"], "batch": w["batch"], "q_heads": w["num_q_heads"],
                   "kv_heads": w["num_kv_heads"], "head_dim": 128, "tokens": T,
                   "cache": head["cache"], "step": head["step"], "decode_bytes": head["decode_bytes"]},
        "pct_hbm_peak": round(100 * head["value"] / HBM_PEAK_GBS, 2),
        "attended_tokens_per_s": head["attended_tokens_per_s"],
        "bytes_per_attended_token": head["bytes_per_attended_token"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
    }
    if "append" in head:
        res["append"] = head["append"]
    if "build" in head:
        res["build"] = head["build"]
    if sub:
        res["sub"] = sub
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
