"""Times the CPU oracle on bounded samples of the benchmark workloads.

TEST INFRASTRUCTURE ONLY: the ``cpu_baseline`` leg of ``bench.py`` runs this
script as a child process (which never touches the GPU) with the thread
counts fixed in its environment, and reads the one JSON line it prints.  It
times the oracle as it stands (``oracle/rq_oracle.py``); nothing here is
tuned.

  python -m oracle.time_oracle fwht --rows 512 --procs 1 --reps 3
      the fp64 oracle rq_fwht_quant on the first ``rows`` rows of the
      4096 x 4096 fp16 workload; with --procs P the rows are split over P
      worker processes (numpy's element-wise code is single threaded).
  python -m oracle.time_oracle gemm --rows 16 --reps 2
      the oracle W4A4 GEMM (exact integer product through a float64 matrix
      product, which uses the BLAS threads of the environment) on ``rows``
      tokens of the 2048 x 8192 -> 28672 prefill shape.

Output: {"what", "rows", "procs", "seconds": [...], "median_s", "bytes" or
"int_ops"} on one line.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import rq_oracle as O  # noqa: E402
from rotation_w4a4_quantization_amd import datagen  # noqa: E402

_X = None
_S = None


def _fwht_rows(bounds):
    lo, hi = bounds
    O.fwht_quant(_X[lo:hi], _S, "f64")
    return hi - lo


def time_fwht(rows: int, procs: int, reps: int) -> dict:
    global _X, _S
    w = datagen.fwht_workload(0)
    _X, _S = w["x"][:rows], w["signs"]
    n = w["d"]
    chunks = [(i * rows // procs, (i + 1) * rows // procs) for i in range(procs)]
    secs = []
    pool = mp.get_context("fork").Pool(procs) if procs > 1 else None
    try:
        for _ in range(reps):
            t0 = time.perf_counter()
            if pool is None:
                _fwht_rows((0, rows))
            else:
                assert sum(pool.map(_fwht_rows, chunks)) == rows
            secs.append(time.perf_counter() - t0)
    finally:
        if pool is not None:
            pool.close()
            pool.join()
    nbytes = rows * n * 2 + rows * n // 2 + 2 * rows + n
    return {"what": "fwht_quant_f64", "rows": rows, "n": n, "procs": procs, "seconds": secs,
            "median_s": statistics.median(secs), "bytes": nbytes}


def time_gemm(rows: int, reps: int) -> dict:
    rng = np.random.default_rng(11)
    d, k = 8192, 28672
    ac = datagen.random_codes(rng, rows, d)
    wc = datagen.random_codes(rng, k, d)
    sa = datagen.random_scales(rng, rows)
    sw = datagen.random_scales(rng, k)
    secs = []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.w4a4_gemm(ac, sa, wc, sw)
        secs.append(time.perf_counter() - t0)
    return {"what": "w4a4_gemm", "rows": rows, "d": d, "k": k, "seconds": secs,
            "median_s": statistics.median(secs), "int_ops": 2 * rows * d * k}


def main():
    p = argparse.ArgumentParser()
    p.add_argument("what", choices=("fwht", "gemm"))
    p.add_argument("--rows", type=int, default=512)
    p.add_argument("--procs", type=int, default=1)
    p.add_argument("--reps", type=int, default=3)
    a = p.parse_args()
    if a.what == "fwht":
        r = time_fwht(a.rows, max(1, a.procs), a.reps)
    else:
        r = time_gemm(a.rows, a.reps)
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
