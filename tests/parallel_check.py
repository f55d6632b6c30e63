"""The oracle's code check (oracle.check_codes) over a large batch, split into
parts that worker processes check independently; the counts are summed.  Test
infrastructure: the workers are started fresh (spawn), touch no GPU and run
the oracle as it stands, one BLAS thread each."""
import multiprocessing as mp
import os

import numpy as np

import oracle


def _part(job):
    lo, x, cb, codes = job
    res = oracle.check_codes(np.asarray(x, dtype=np.float64), cb, codes)
    res["hard_examples"] = [(lo + i, s, g, zc, zo) for (i, s, g, zc, zo) in res["hard_examples"]]
    return res


def check_codes_all(x, cb, codes, workers=None, parts=None):
    """oracle.check_codes(x, cb, codes) over every row of x [N][D] (float32 or
    float64), computed in parts by ``workers`` processes (default: up to 12,
    at most the CPUs this process may use)."""
    if workers is None:
        try:
            avail = len(os.sched_getaffinity(0))
        except (AttributeError, OSError):
            avail = os.cpu_count() or 1
        workers = max(1, min(12, avail))
    n = x.shape[0]
    parts = parts or max(workers * 4, 1)
    bounds = np.linspace(0, n, parts + 1).astype(np.int64)
    jobs = [(int(lo), x[lo:hi], cb, codes[lo:hi]) for lo, hi in zip(bounds[:-1], bounds[1:])
            if hi > lo]
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    os.environ.update({k: "1" for k in saved})
    try:
        with mp.get_context("spawn").Pool(workers) as pool:
            results = pool.map(_part, jobs, chunksize=1)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    out = {"total": 0, "exact": 0, "near_tie": 0, "hard": 0, "worst_rel_excess": 0.0,
           "hard_examples": []}
    for r in results:
        for k in ("total", "exact", "near_tie", "hard"):
            out[k] += r[k]
        out["worst_rel_excess"] = max(out["worst_rel_excess"], r["worst_rel_excess"])
        out["hard_examples"] += r["hard_examples"][:16 - len(out["hard_examples"])]
    return out
