"""Oracle decodes of whole workloads in a pool of CPU processes.

One task rebuilds one (sequence, kv head) pair of a workload from the seeded
inputs with the oracle, following an append schedule, and returns the fp64
decode output of its query heads.  Workers are spawned (not forked), import
numpy and the oracle only, and run single-threaded BLAS; they never touch a
GPU.  The pool size is at most 16 processes."""

import multiprocessing as mp
import os

import numpy as np

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _pair_decode(task):
    wid, schedule, b, h = task
    from oracle.cache import OracleCache
    from quantized_decode_attention_02_amd import workloads as wl
    w = wl.workload(wid)
    G = w["num_q_heads"] // w["num_kv_heads"]
    cfg = dict(wl.library_config(w), num_q_heads=G, num_kv_heads=1)
    T = sum(schedule)
    K, V = wl.kv_tokens(w, 0, T, seqs=[b], heads=[h], threads=1)
    o = OracleCache(cfg, 1, T)
    t = 0
    for n in schedule:
        o.append(K[:, t:t + n], V[:, t:t + n])
        t += n
    del K, V
    q = wl.queries(w, seqs=[b])[:, h * G:(h + 1) * G]
    return b, h, np.asarray(o.decode(q)[0], dtype=np.float64)


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


class PairDecodes:
    """Starts the oracle decodes of ``pairs`` at once; ``results()`` waits and
    returns {(b, h): fp64 [G, 128]}."""

    def __init__(self, wid, schedule, pairs):
        saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        for k in _THREAD_VARS:
            os.environ[k] = "1"
        try:
            ctx = mp.get_context("spawn")
            self.pool = ctx.Pool(min(workers(), len(pairs)))
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        tasks = [(wid, list(schedule), b, h) for b, h in pairs]
        self.pending = self.pool.map_async(_pair_decode, tasks, chunksize=1)

    def results(self, timeout=None):
        try:
            out = self.pending.get(timeout)
        finally:
            self.pool.close()
            self.pool.join()
        return {(b, h): ref for b, h, ref in out}

    def cancel(self):
        self.pool.terminate()
        self.pool.join()
