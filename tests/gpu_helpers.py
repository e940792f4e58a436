"""Helpers for the GPU parity tests: drive the HIP library and the CPU oracle
on the same seeded inputs and compare.

Bar: packed codes, scales, zeros, window rows and dequantized values are
bit-exact; attention is within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the fp64
oracle applied to the same dequantized cache."""

import sys

import numpy as np
import torch

from oracle import layout as olayout
from oracle.cache import OracleCache
from quantized_decode_attention_02_amd import workloads as wl

ATOL, RTOL = 2e-3, 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def kvq():
    from quantized_decode_attention_02_amd import kvq as k
    return k


def build_pair(w, chunks, max_tokens=None, seqs=None, heads=None):
    """Append the same token chunks to a GPU cache and an oracle cache.

    The GPU cache holds every sequence and head of ``w``; the oracle holds the
    selected ones (default: all)."""
    K = kvq()
    T = sum(chunks)
    max_tokens = max_tokens or T
    cfg = wl.library_config(w)
    g = K.KVCache(cfg, w["batch"], max_tokens)
    seqs = list(range(w["batch"])) if seqs is None else seqs
    heads = list(range(w["num_kv_heads"])) if heads is None else heads
    G = w["num_q_heads"] // w["num_kv_heads"]
    ocfg = dict(cfg, num_kv_heads=len(heads), num_q_heads=G * len(heads))
    o = OracleCache(ocfg, len(seqs), max_tokens)
    t = 0
    for n in chunks:
        Kall, Vall = wl.kv_tokens(w, t, t + n)
        g.append(torch.from_numpy(Kall).cuda(), torch.from_numpy(Vall).cuda())
        o.append(Kall[seqs][:, :, heads], Vall[seqs][:, :, heads])
        t += n
    torch.cuda.synchronize()
    return g, o, seqs, heads


def compare_planes(g, o, seqs, heads):
    """Byte-exact comparison of planes 0..7 on the bytes the oracle defines."""
    img, live = o.plane_images()
    B, H = g.batch, g.hkv
    for p in range(8):
        if img[p].size == 0:
            continue
        dev = g.planes[p].cpu().numpy().reshape(B, H, -1)
        sel = dev[np.ix_(seqs, heads)]
        want = img[p].reshape(len(seqs), len(heads), -1)
        m = live[p].reshape(len(seqs), len(heads), -1)
        bad = (sel != want) & m
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"plane {olayout.PLANE_NAMES[p]}: {bad.sum()} bytes differ, "
                                 f"first at {idx.tolist()}: got {sel[bad][:5]} want {want[bad][:5]}")


def compare_rope_table(g, o):
    if g.planes[olayout.ROPE] is None:
        return
    from oracle.attention import rope_freqs
    T = o.length
    tab = g.planes[olayout.ROPE].view(torch.float32).cpu().numpy().reshape(-1, 64, 2)[:T]
    ang = np.arange(T)[:, None] * rope_freqs(o.cfg["rope_theta"])[None, :]
    assert np.max(np.abs(tab[..., 0] - np.cos(ang))) < 1e-6
    assert np.max(np.abs(tab[..., 1] - np.sin(ang))) < 1e-6


def compare_dequant(g, o, seqs, heads, t0=0, t1=None):
    kd, vd = g.dequant(t0, t1)
    kd = kd.cpu().numpy()[np.ix_(seqs, range(kd.shape[1]), heads)]
    vd = vd.cpu().numpy()[np.ix_(seqs, range(vd.shape[1]), heads)]
    ko, vo = o.dequant(t0, t1)
    assert np.array_equal(kd.view(np.uint32), ko.view(np.uint32)), "key dequant differs"
    assert np.array_equal(vd.view(np.uint32), vo.view(np.uint32)), "value dequant differs"


def check_decode(g, o, w, seqs, heads, q_pos=None, sm_scale=0.0):
    q = wl.queries(w)
    out = g.decode(torch.from_numpy(q).cuda(), q_pos=q_pos, sm_scale=sm_scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = w["num_q_heads"] // w["num_kv_heads"]
    qh = [h * G + i for h in heads for i in range(G)]
    got = out[np.ix_(seqs, qh)]
    ref = o.decode(q[np.ix_(seqs, qh)], q_pos=q_pos, sm_scale=sm_scale if sm_scale > 0 else None)
    err = np.abs(got.astype(np.float64) - ref)
    lim = ATOL + RTOL * np.abs(ref)
    worst = float(np.max(err / lim)) if err.size else 0.0
    say(f"  decode: worst {worst:.3f} of tolerance, max abs err {err.max():.2e}")
    assert np.all(err <= lim), f"decode off by {worst:.2f}x the tolerance; max abs {err.max():.3e}"
    return worst, float(err.max()) if err.size else 0.0
