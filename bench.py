#!/usr/bin/env python3
"""Throughput of the rotate + INT4 + W4A4 hot path on one MI355X.

Main workload (the JSON ``value``): rq_fwht_quant on 4096 tokens x 4096 fp16
activations (0.1% of channels x100, randomized Hadamard n = 4096), in GB/s of
algorithmic HBM traffic (fp16 input + packed codes + fp16 scales + int8
signs).  One step = one call over the whole 4096 x 4096 batch; inputs and
outputs rotate over buffer sets larger than the 256 MB Infinity Cache so that
repeats cannot be served from it.

``secondary`` reports the other rows of the path on their own workloads:
the decode-shaped and prefill-shaped W4A4 GEMMs (TOPS and GB/s), the prefill
activation rotation (2048 x 8192) and the KV-cache rotation
[32, 8, 4096, 128] x {K, V}.

Kernel time is measured with HIP events recorded on the stream the kernels
are launched on (torch's current stream, which the binding passes to librq).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
FP6_PEAK_TOPS = 10100.0        # MI355X dense fp6 / fp4 MFMA, TFLOP/s
MALL_BYTES = 256 * 2 ** 20     # Infinity Cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-secondary", action="store_true", help="time only the main workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="",
                   help="comma list of secondary sections (decode, prefill, downproj, w4a8, asym, "
                        "grouped, kv, ceiling) or of single line names to run")
    p.add_argument("--lines", default="",
                   help="comma list of secondary line names: time only these within the "
                        "selected sections (for per-shape profiles)")
    p.add_argument("--replays", type=int, default=5,
                   help="timed graph replays per line (median and best are reported)")
    return p.parse_args()


def fwht_bytes(m: int, n: int) -> int:
    # fp16 input + packed int4 codes + fp16 scales + int8 signs
    return m * n * 2 + m * n // 2 + 2 * m + n


def gemm_bytes(m: int, k: int, d: int) -> int:
    # weights + weight scales + activation codes + activation scales + fp16 output
    return d * k // 2 + 2 * k + m * d // 2 + 2 * m + 2 * m * k


def fwht8_bytes(m: int, n: int) -> int:
    # fp16 input + one int8 code per element + fp16 scales + int8 signs
    return m * n * 2 + m * n + 2 * m + n


def gemm8_bytes(m: int, k: int, d: int) -> int:
    # as gemm_bytes with one byte per activation code
    return d * k // 2 + 2 * k + m * d + 2 * m + 2 * m * k


def kv_bytes(rows: int) -> int:
    return 2 * (rows * 128 * 2 + rows * 64 + rows * 2)


KERNEL_SOURCES_MAIN = ["rotation_w4a4_quantization_amd/csrc/fwht_quant.hip",
                       "rotation_w4a4_quantization_amd/csrc/rq_row_device.h"]


def sources_sha256(paths) -> str:
    """SHA-256 over the concatenated bytes of the files, in the given order."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(root, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel_sources, summary: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when any of the kernel's sources changed since it was
    measured."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, summary)) as f:
            rec = json.load(f)
        sha = sources_sha256(kernel_sources)
    except OSError:
        return None
    ok = rec.get("sources") == list(kernel_sources) and rec.get("source_sha256") == sha
    return rec["traffic_bytes_per_launch"] if ok else None


REPLAYS = 5


def time_launches(torch, fn, sets: int, steps: int, warmup: int):
    """Median per-call milliseconds of fn(i), i cycling over buffer sets.

    `warmup` eager calls, then `steps` calls are captured into one HIP graph
    (so host launch overhead does not starve the GPU), the graph is replayed
    untimed for about a quarter of a second (the shader clock settles under
    sustained load), and REPLAYS replays are timed one by one with HIP events
    recorded on the stream the kernels run on, each between two device
    synchronisations.  The median per-call time is returned; the best and
    all of them are left in time_launches.best_ms / .all_ms."""
    for i in range(warmup):
        fn(i % sets)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            fn(i % sets)
    t0 = time.perf_counter()
    for _ in range(1000):
        graph.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > 0.25:
            break
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    per_call = []
    wall = 0.0
    for _ in range(max(1, REPLAYS)):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        start.record()
        graph.replay()
        stop.record()
        torch.cuda.synchronize()
        wall += time.perf_counter() - w0
        per_call.append(start.elapsed_time(stop) / steps)
    time_launches.last_wall_s = wall
    time_launches.all_ms = per_call
    time_launches.best_ms = min(per_call)
    del graph
    return float(np.median(per_call))


def line(us_ms: float, **extra) -> dict:
    """A secondary bench line: median and best microseconds per call."""
    d = {"us": round(us_ms * 1e3, 3), "us_best": round(time_launches.best_ms * 1e3, 3)}
    d.update(extra)
    return d


def _host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, os.cpu_count() or 1, avail


def _time_oracle(args, threads: int):
    """Run oracle/time_oracle.py in a child process (it never touches the
    GPU) with `threads` BLAS / OpenMP threads; returns its JSON record."""
    import subprocess

    env = dict(os.environ)
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        env[v] = str(threads)
    root = os.path.dirname(os.path.abspath(__file__))
    out = subprocess.run([sys.executable, "-m", "oracle.time_oracle", *args], cwd=root, env=env,
                         capture_output=True, text=True, timeout=300, check=True)
    return json.loads(out.stdout.strip().splitlines()[-1])


def cpu_baseline(log) -> dict:
    """The oracle (oracle/rq_oracle.py, untuned) on the host's CPU cores:
    fp64 rq_fwht_quant on the 4096 x 4096 workload, on every core it may use
    (rows split over worker processes, capped at 16) and on one, and the
    oracle's W4A4 GEMM on a 64-token slice of the prefill shape; each the
    median of 3 runs."""
    model, nproc, avail = _host_cpu()
    procs = max(1, min(avail, 16))
    allc = _time_oracle(["fwht", "--rows", "4096", "--procs", str(procs), "--reps", "3"], 1)
    one = _time_oracle(["fwht", "--rows", "1024", "--procs", "1", "--reps", "3"], 1)
    gemm = _time_oracle(["gemm", "--rows", "64", "--reps", "3"], procs)
    gbs = allc["bytes"] / allc["median_s"] / 1e9
    gbs1 = one["bytes"] / one["median_s"] / 1e9
    tops = gemm["int_ops"] / gemm["median_s"] / 1e12
    log(f"[bench] cpu oracle: {gbs:.3f} GB/s on {procs} processes, {gbs1:.4f} GB/s on 1; "
        f"gemm {tops:.4f} TOP/s")
    return {
        "value": round(gbs, 5), "unit": "GB/s", "cores": procs, "kind": "oracle",
        "sample": f"fp64 oracle rq_fwht_quant on all 4096 x 4096 rows split over {procs} worker "
                  f"processes (1 thread each), median of 3 runs "
                  f"({allc['median_s']:.2f} s); host {model}, nproc {nproc}, {avail} usable",
        "host_cpu": model, "nproc": nproc, "usable_cores": avail,
        "single_thread": {"value": round(gbs1, 5), "unit": "GB/s", "cores": 1,
                          "sample": f"first 1024 rows, median of 3 ({one['median_s']:.2f} s)"},
        "gemm_prefill_slice": {"value": round(tops, 5), "unit": "TOP/s", "cores": procs,
                               "sample": f"oracle W4A4 GEMM on 64 of the 2048 prefill tokens x 8192 "
                                         f"-> 28672 (exact integer product through a float64 "
                                         f"matrix product, {procs} BLAS threads), median of 3 "
                                         f"({gemm['median_s']:.2f} s); the full 2048 tokens scale "
                                         f"x32"},
    }


def main():
    global REPLAYS
    args = parse()
    REPLAYS = max(1, args.replays)
    if args.gpus != 1:
        print(json.dumps({"error": "the rq kernels run on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    for v in ("RANK", "WORLD_SIZE"):
        if os.environ.get(v) not in (None, "0", "1"):
            print(json.dumps({"error": "multi-rank launch is not supported"}))
            sys.exit(2)

    import torch

    import rotation_w4a4_quantization_amd as rq
    from rotation_w4a4_quantization_amd import datagen

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    rq.load_library()
    dev = torch.device("cuda:0")
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    # ------------------------------------------------ main: fwht_quant 4096^2
    w = datagen.fwht_workload(0)
    m, n = w["m"], w["d"]
    x0 = torch.from_numpy(w["x"]).to(dev)
    signs = torch.from_numpy(w["signs"]).to(dev)
    per_set = m * n * 2 + m * n // 2 + 2 * m
    sets = max(2, -(-2 * MALL_BYTES // per_set) + 1)
    xs = [x0.clone() for _ in range(sets)]
    outs = [(torch.empty((m, n // 2), dtype=torch.uint8, device=dev),
             torch.empty((m,), dtype=torch.float16, device=dev)) for _ in range(sets)]
    lib = rq.load_library()
    from rotation_w4a4_quantization_amd.binding import RQ_F16, _ptr, _stream

    def fq(i):
        st = lib.rq_fwht_quant(_ptr(xs[i]), RQ_F16, m, n, _ptr(signs), _ptr(outs[i][0]),
                               _ptr(outs[i][1]), None, _stream())
        if st:
            raise RuntimeError(rq.status_string(st))

    log(f"[bench] fwht_quant {m}x{n} fp16: {sets} buffer sets, warmup {args.warmup}, steps {args.steps}")
    torch.cuda.synchronize()
    ms = time_launches(torch, fq, sets, args.steps, args.warmup)
    wall = time_launches.last_wall_s  # host clock around the timed replay
    nbytes = fwht_bytes(m, n)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] fwht_quant: {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% HBM)")
    del xs, outs

    result = {
        "metric": "FWHT+quant GB/s and W4A4 GEMM TOPS (% of HBM / int8-MFMA peak), 1 GPU",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_best": round(time_launches.best_ms * 1e3, 3),
        "replay_us": [round(v * 1e3, 3) for v in time_launches.all_ms],
        "timing": f"HIP events around each of {REPLAYS} graph replays of {args.steps} launches "
                  "(inputs rotating over > 2x the 256 MB Infinity Cache); value and ms_per_step "
                  "use the median replay, us_best the fastest",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; N(0,1) fp16 with 0.1% of channels x100)",
        "config": {"workload": "rq_fwht_quant 4096 tokens x 4096 fp16, n=4096 randomized Hadamard, "
                               "per-token INT4", "tokens": m, "n": n, "input_dtype": "fp16",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(KERNEL_SOURCES_MAIN,
                                                 "profiles/fwht_quant_4096x4096_traffic.json"),
                     "kernel": "fwht_row_kernel<4096, true, 4, false>",
                     "algorithmic_bytes_per_launch": nbytes},
        "wall_s_timed_region": round(wall, 3),
    }

    # ------------------------------------------------------------ secondary
    sec = {}
    only = set(filter(None, args.only.split(",")))
    lines = set(filter(None, args.lines.split(",")))
    want = (lambda k: (not only) or k in only)
    want_line = (lambda k: (not lines) or k in lines)
    if not args.no_secondary:
        steps2 = max(10, args.steps // 4)
        warm2 = max(3, args.warmup // 4)

        if want("decode"):
            dec = datagen.decode_linear(0)
            s = torch.from_numpy(dec["signs"]).to(dev)
            xa = torch.from_numpy(dec["x"]).to(dev)
            ac, sa, _ = rq.fwht_quant(xa, s)
            for k, wt in dec["wts"].items():
                wc, ws, _ = rq.fold_weights(torch.from_numpy(wt).to(dev), s)
                nsets = max(2, -(-2 * MALL_BYTES // wc.numel()) + 1)
                wcs = [wc.clone() for _ in range(nsets)]
                for mm in (1, 4, 16):
                    y = torch.empty((mm, k), dtype=torch.float16, device=dev)
                    a_m, s_m = ac[:mm].contiguous(), sa[:mm].contiguous()

                    def g(i, a_m=a_m, s_m=s_m, y=y):
                        rq.w4a4_gemm(a_m, s_m, wcs[i], ws, out=y)

                    if want_line(f"gemm_decode_m{mm}_k{k}"):
                        msg = time_launches(torch, g, nsets, steps2, warm2)
                        b = gemm_bytes(mm, k, 4096)
                        sec[f"gemm_decode_m{mm}_k{k}"] = line(
                            msg, **{"GB/s": round(b / (msg * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(b / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                    "TOPS": round(2 * mm * k * 4096 / (msg * 1e-3) / 1e12, 3)})
                        log(f"[bench] decode m={mm} k={k}: {sec[f'gemm_decode_m{mm}_k{k}']}")
                        # the same launches issued eagerly from the host (no graph): what
                        # launch gaps cost at this size
                        for i in range(warm2):
                            g(i % nsets)
                        torch.cuda.synchronize()
                        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        ev0.record()
                        for i in range(steps2):
                            g(i % nsets)
                        ev1.record()
                        torch.cuda.synchronize()
                        sec[f"gemm_decode_m{mm}_k{k}"]["us_eager"] = round(ev0.elapsed_time(ev1) / steps2 * 1e3, 3)
                    # the whole decode linear: rotate + quantize the fp16 tokens, then the GEMM
                    x_m = xa[:mm].contiguous()
                    a_q = torch.empty((mm, 2048), dtype=torch.uint8, device=dev)
                    s_q = torch.empty((mm,), dtype=torch.float16, device=dev)

                    def lin_d(i, x_m=x_m, a_q=a_q, s_q=s_q, y=y, mm=mm):
                        st = lib.rq_fwht_quant(_ptr(x_m), RQ_F16, mm, 4096, _ptr(s), _ptr(a_q),
                                               _ptr(s_q), None, _stream())
                        assert st == 0
                        rq.w4a4_gemm(a_q, s_q, wcs[i], ws, out=y)

                    if want_line(f"linear_decode_m{mm}_k{k}_rotate_plus_gemm"):
                        msl = time_launches(torch, lin_d, nsets, steps2, warm2)
                        sec[f"linear_decode_m{mm}_k{k}_rotate_plus_gemm"] = line(msl)
                    # the same linear as one launch: rotation fused into the GEMM's prologue
                    ws_ld = rq.linear_decode_workspace(mm, 4096, dev)

                    def lin_f(i, x_m=x_m, y=y, ws_ld=ws_ld):
                        rq.linear_decode(x_m, s, wcs[i], ws, workspace=ws_ld, out=y)

                    if want_line(f"linear_decode_m{mm}_k{k}_fused"):
                        msf = time_launches(torch, lin_f, nsets, steps2, warm2)
                        sec[f"linear_decode_m{mm}_k{k}_fused"] = line(msf)
                del wcs

        if want("prefill"):
            pf = datagen.prefill_linear(0)
            s = torch.from_numpy(pf["signs"]).to(dev)
            wc, ws, _ = rq.fold_weights(torch.from_numpy(pf["wt"]).to(dev), s)
            del pf["wt"]
            xa = torch.from_numpy(pf["x"]).to(dev)
            mm, d, k = pf["m"], pf["d"], pf["k"]
            ac = torch.empty((mm, d // 2), dtype=torch.uint8, device=dev)
            sa = torch.empty((mm,), dtype=torch.float16, device=dev)
            # rotate over input clones (> 2x the MALL) so repeats cannot hit in it
            fsets = -(-2 * MALL_BYTES // (xa.numel() * 2)) + 1
            xas = [xa] + [xa.clone() for _ in range(fsets - 1)]

            def f8(i):
                st = lib.rq_fwht_quant(_ptr(xas[i]), RQ_F16, mm, d, _ptr(s), _ptr(ac), _ptr(sa), None,
                                       _stream())
                assert st == 0

            if want_line("fwht_quant_2048x8192"):
                msf = time_launches(torch, f8, fsets, steps2, warm2)
                b = fwht_bytes(mm, d)
                sec["fwht_quant_2048x8192"] = line(msf, **{"GB/s": round(b / (msf * 1e-3) / 1e9, 1),
                                               "hbm_frac": round(b / (msf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                log(f"[bench] fwht_quant 2048x8192: {sec['fwht_quant_2048x8192']}")
            f8(0)
            torch.cuda.synchronize()
            del xas[1:]
            y = torch.empty((mm, k), dtype=torch.float16, device=dev)
            wcs = [wc, wc.clone()]

            def gp(i):
                rq.w4a4_gemm(ac, sa, wcs[i], ws, out=y)

            if want_line("gemm_prefill_2048x8192x28672"):
                msp = time_launches(torch, gp, 2, max(5, steps2 // 2), warm2)
                tops = 2 * mm * d * k / (msp * 1e-3) / 1e12
                sec["gemm_prefill_2048x8192x28672"] = line(msp, **{"TOPS": round(tops, 1),
                                                       "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)})
                log(f"[bench] prefill gemm: {sec['gemm_prefill_2048x8192x28672']}")

            def lin(i):
                f8(0)
                rq.w4a4_gemm(ac, sa, wcs[i], ws, out=y)

            if want_line("linear_prefill_rotate_plus_gemm"):
                msl = time_launches(torch, lin, 2, max(5, steps2 // 2), warm2)
                sec["linear_prefill_rotate_plus_gemm"] = line(msl)

            # the same GEMM on the 6-bit matrix unit: activation codes repacked
            # into the F6 layout per call, weights repacked once (offline)
            a6 = torch.empty((d // 128, mm, 96), dtype=torch.uint8, device=dev)
            w6s = [rq.pack_f6(w_) for w_ in wcs]
            del wcs, wc

            def pk(i):
                rq.pack_f6(ac, out=a6)

            if want_line("pack_f6_2048x8192"):
                msk = time_launches(torch, pk, 1, steps2, warm2)
                b = mm * d // 2 + mm * d * 3 // 4
                sec["pack_f6_2048x8192"] = line(msk, **{"GB/s": round(b / (msk * 1e-3) / 1e9, 1),
                                           "hbm_frac": round(b / (msk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            pk(0)

            def g6(i):
                rq.w4a4_gemm_f6(a6, sa, w6s[i], ws, out=y)

            if want_line("gemm_f6_prefill_2048x8192x28672"):
                ms6 = time_launches(torch, g6, 2, max(5, steps2 // 2), warm2)
                tops = 2 * mm * d * k / (ms6 * 1e-3) / 1e12
                sec["gemm_f6_prefill_2048x8192x28672"] = line(
                    ms6, **{"TOPS": round(tops, 1), "mfma_frac": round(tops / FP6_PEAK_TOPS, 4),
                            "vs_int8_peak": round(tops / INT8_PEAK_TOPS, 4)})
                log(f"[bench] prefill gemm on fp6 MFMA: {sec['gemm_f6_prefill_2048x8192x28672']}")

            def lin6(i):
                f8(0)
                rq.pack_f6(ac, out=a6)
                rq.w4a4_gemm_f6(a6, sa, w6s[i], ws, out=y)

            if want_line("linear_prefill_f6_rotate_pack_gemm"):
                msl6 = time_launches(torch, lin6, 2, max(5, steps2 // 2), warm2)
                sec["linear_prefill_f6_rotate_pack_gemm"] = line(msl6)
            del w6s, a6, y

        if want("downproj"):
            # the online rotation in front of a down projection: 2048 tokens x
            # 14336 = 28 * 512 (H_28 (x) H_512) and x 28672 = 28 * 1024
            # (H_28 (x) H_1024), same input statistics as the prefill
            # activations; then the 28672 -> 8192 down projection GEMM
            for mm, d, seed in ((2048, 14336, 4), (2048, 28672, 6)):
                key = f"fwht_quant_{mm}x{d}"
                rng = np.random.default_rng(seed)
                x28 = datagen.activations(rng, mm, d, datagen.outlier_channels(rng, d), 100.0)
                x28 = torch.from_numpy(x28).to(dev)
                s28 = torch.from_numpy(datagen.rademacher(rng, d)).to(dev)
                ac28 = torch.empty((mm, d // 2), dtype=torch.uint8, device=dev)
                sa28 = torch.empty((mm,), dtype=torch.float16, device=dev)
                fsets = -(-2 * MALL_BYTES // (x28.numel() * 2)) + 1
                x28s = [x28] + [x28.clone() for _ in range(fsets - 1)]

                def f28(i, x28s=x28s, s28=s28, ac28=ac28, sa28=sa28, mm=mm, d=d):
                    st = lib.rq_fwht_quant(_ptr(x28s[i]), RQ_F16, mm, d, _ptr(s28), _ptr(ac28),
                                           _ptr(sa28), None, _stream())
                    assert st == 0

                if want_line(key):
                    ms28 = time_launches(torch, f28, fsets, steps2, warm2)
                    b = fwht_bytes(mm, d)
                    sec[key] = line(ms28, **{"GB/s": round(b / (ms28 * 1e-3) / 1e9, 1),
                                             "hbm_frac": round(b / (ms28 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                    log(f"[bench] {key}: {sec[key]}")
                del x28s
                if d == 28672 and want_line("gemm_downproj_2048x28672x8192"):
                    f28(0)
                    k = 8192
                    wt = torch.from_numpy(datagen.gaussian(rng, (k, d), std=0.02)).to(dev)
                    wc, ws, _ = rq.fold_weights(wt, s28)
                    del wt
                    y = torch.empty((mm, k), dtype=torch.float16, device=dev)
                    wcs = [wc, wc.clone()]

                    def gd(i, wcs=wcs, ws=ws, y=y, ac28=ac28, sa28=sa28):
                        rq.w4a4_gemm(ac28, sa28, wcs[i], ws, out=y)

                    msd = time_launches(torch, gd, 2, max(5, steps2 // 2), warm2)
                    tops = 2 * mm * d * k / (msd * 1e-3) / 1e12
                    sec["gemm_downproj_2048x28672x8192"] = line(
                        msd, **{"TOPS": round(tops, 1), "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)})
                    log(f"[bench] down projection gemm: {sec['gemm_downproj_2048x28672x8192']}")
                    if want_line("gemm_f6_downproj_2048x28672x8192"):
                        a6 = rq.pack_f6(ac28)
                        w6s = [rq.pack_f6(w_) for w_ in wcs]

                        def g6d(i, w6s=w6s, a6=a6, ws=ws, y=y, sa28=sa28):
                            rq.w4a4_gemm_f6(a6, sa28, w6s[i], ws, out=y)

                        ms6 = time_launches(torch, g6d, 2, max(5, steps2 // 2), warm2)
                        tops = 2 * mm * d * k / (ms6 * 1e-3) / 1e12
                        sec["gemm_f6_downproj_2048x28672x8192"] = line(
                            ms6, **{"TOPS": round(tops, 1), "mfma_frac": round(tops / FP6_PEAK_TOPS, 4),
                                    "vs_int8_peak": round(tops / INT8_PEAK_TOPS, 4)})
                        log(f"[bench] down projection on fp6 MFMA: {sec['gemm_f6_downproj_2048x28672x8192']}")
                        del w6s, a6
                    del wcs, wc, y
                del x28

        if want("w4a8"):
            # the W4A8 variant: INT8 per-token activations against the same
            # folded INT4 weights
            w8 = datagen.fwht_workload(0)
            m8, n8 = w8["m"], w8["d"]
            x8 = torch.from_numpy(w8["x"]).to(dev)
            s8 = torch.from_numpy(w8["signs"]).to(dev)
            per8 = fwht8_bytes(m8, n8)
            sets8 = max(2, -(-2 * MALL_BYTES // per8) + 1)
            x8s = [x8] + [x8.clone() for _ in range(sets8 - 1)]
            o8 = [(torch.empty((m8, n8), dtype=torch.int8, device=dev),
                   torch.empty((m8,), dtype=torch.float16, device=dev)) for _ in range(sets8)]

            def fq8(i):
                st = lib.rq_fwht_quant8(_ptr(x8s[i]), m8, n8, _ptr(s8), _ptr(o8[i][0]),
                                        _ptr(o8[i][1]), None, _stream())
                assert st == 0

            ms8 = time_launches(torch, fq8, sets8, steps2, warm2)
            sec["fwht_quant8_4096x4096"] = line(ms8, **{"GB/s": round(per8 / (ms8 * 1e-3) / 1e9, 1),
                                            "hbm_frac": round(per8 / (ms8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            log(f"[bench] fwht_quant8 4096x4096: {sec['fwht_quant8_4096x4096']}")
            del x8s, o8, x8
            dec = datagen.decode_linear(0)
            s = torch.from_numpy(dec["signs"]).to(dev)
            xd = torch.from_numpy(dec["x"]).to(dev)
            ac8, sa8, _ = rq.fwht_quant8(xd, s)
            for k, wt in dec["wts"].items():
                wc, ws, _ = rq.fold_weights(torch.from_numpy(wt).to(dev), s)
                nsets = max(2, -(-2 * MALL_BYTES // wc.numel()) + 1)
                wcs = [wc.clone() for _ in range(nsets)]
                for mm in (1, 4, 16):
                    y = torch.empty((mm, k), dtype=torch.float16, device=dev)
                    a_m, s_m = ac8[:mm].contiguous(), sa8[:mm].contiguous()

                    def g8(i, a_m=a_m, s_m=s_m, y=y):
                        rq.w4a8_gemm(a_m, s_m, wcs[i], ws, out=y)

                    key = f"gemm_w4a8_decode_m{mm}_k{k}"
                    if want_line(key):
                        msg = time_launches(torch, g8, nsets, steps2, warm2)
                        bb = gemm8_bytes(mm, k, 4096)
                        sec[key] = line(msg, **{"GB/s": round(bb / (msg * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(bb / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                        log(f"[bench] {key}: {sec[key]}")
                    if mm > 4:
                        continue
                    # the whole W4A8 decode linear from fp16 tokens: two launches
                    # (rotate + INT8 quantise, then the GEMM), and one (the rotation
                    # as the GEMM's prologue)
                    x_m = xd[:mm].contiguous()
                    a_q = torch.empty((mm, 4096), dtype=torch.int8, device=dev)
                    s_q = torch.empty((mm,), dtype=torch.float16, device=dev)

                    def lin8_d(i, x_m=x_m, a_q=a_q, s_q=s_q, y=y, mm=mm):
                        st = lib.rq_fwht_quant8(_ptr(x_m), mm, 4096, _ptr(s), _ptr(a_q), _ptr(s_q),
                                                None, _stream())
                        assert st == 0
                        rq.w4a8_gemm(a_q, s_q, wcs[i], ws, out=y)

                    def lin8_f(i, x_m=x_m, y=y):
                        rq.linear_decode_w4a8(x_m, s, wcs[i], ws, out=y)

                    for key, fn in ((f"linear_w4a8_decode_m{mm}_k{k}_rotate_plus_gemm", lin8_d),
                                    (f"linear_w4a8_decode_m{mm}_k{k}_fused", lin8_f)):
                        if want_line(key):
                            sec[key] = line(time_launches(torch, fn, nsets, steps2, warm2))
                            log(f"[bench] {key}: {sec[key]}")
                del wcs, wc
            pf = datagen.prefill_linear(0)
            sp = torch.from_numpy(pf["signs"]).to(dev)
            wc, ws, _ = rq.fold_weights(torch.from_numpy(pf["wt"]).to(dev), sp)
            del pf["wt"]
            mm, d, k = pf["m"], pf["d"], pf["k"]
            ac8, sa8, _ = rq.fwht_quant8(torch.from_numpy(pf["x"]).to(dev), sp)
            y = torch.empty((mm, k), dtype=torch.float16, device=dev)
            wcs = [wc, wc.clone()]

            def gp8(i):
                rq.w4a8_gemm(ac8, sa8, wcs[i], ws, out=y)

            msp = time_launches(torch, gp8, 2, max(5, steps2 // 4), warm2)
            tops = 2 * mm * d * k / (msp * 1e-3) / 1e12
            sec["gemm_w4a8_prefill_2048x8192x28672"] = line(msp, **{"TOPS": round(tops, 1),
                "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)})
            log(f"[bench] w4a8 prefill gemm: {sec['gemm_w4a8_prefill_2048x8192x28672']}")
            del wcs, wc, y, ac8

        if want("asym"):
            # asymmetric activations: rotation + unsigned INT4 with zero
            # points, and the GEMM with the zero-point epilogue
            wa = datagen.fwht_workload(0)
            ma, na = wa["m"], wa["d"]
            xa0 = torch.from_numpy(wa["x"]).to(dev)
            sga = torch.from_numpy(wa["signs"]).to(dev)
            pera = ma * na * 2 + ma * na // 2 + 3 * ma + na
            setsa = max(2, -(-2 * MALL_BYTES // pera) + 1)
            xas_ = [xa0] + [xa0.clone() for _ in range(setsa - 1)]
            oa = [(torch.empty((ma, na // 2), dtype=torch.uint8, device=dev),
                   torch.empty((ma,), dtype=torch.float16, device=dev),
                   torch.empty((ma,), dtype=torch.uint8, device=dev)) for _ in range(setsa)]

            def fqa(i):
                st = lib.rq_fwht_quant_asym(_ptr(xas_[i]), ma, na, _ptr(sga), _ptr(oa[i][0]),
                                            _ptr(oa[i][1]), _ptr(oa[i][2]), None, _stream())
                assert st == 0

            msa = time_launches(torch, fqa, setsa, steps2, warm2)
            sec["fwht_quant_asym_4096x4096"] = line(msa, **{"GB/s": round(pera / (msa * 1e-3) / 1e9, 1),
                                                "hbm_frac": round(pera / (msa * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            log(f"[bench] fwht_quant_asym 4096x4096: {sec['fwht_quant_asym_4096x4096']}")
            del xas_, oa, xa0
            dec = datagen.decode_linear(0)
            s = torch.from_numpy(dec["signs"]).to(dev)
            acq, saq, zaq, _ = rq.fwht_quant_asym(torch.from_numpy(dec["x"]).to(dev), s)
            for k, wt in dec["wts"].items():
                wc, ws, _ = rq.fold_weights(torch.from_numpy(wt).to(dev), s)
                wsum = rq.weight_code_sums(wc)
                nsets = max(2, -(-2 * MALL_BYTES // wc.numel()) + 1)
                wcs = [wc.clone() for _ in range(nsets)]
                for mm in (1, 4, 16):
                    y = torch.empty((mm, k), dtype=torch.float16, device=dev)
                    a_m, s_m, z_m = acq[:mm].contiguous(), saq[:mm].contiguous(), zaq[:mm].contiguous()

                    def ga(i, a_m=a_m, s_m=s_m, z_m=z_m, y=y):
                        rq.w4a4_gemm_asym(a_m, s_m, z_m, wcs[i], ws, wsum, out=y)

                    msg = time_launches(torch, ga, nsets, steps2, warm2)
                    bb = gemm_bytes(mm, k, 4096) + mm + 4 * k
                    key = f"gemm_asym_decode_m{mm}_k{k}"
                    sec[key] = line(msg, **{"GB/s": round(bb / (msg * 1e-3) / 1e9, 1),
                                "hbm_frac": round(bb / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                    log(f"[bench] {key}: {sec[key]}")
                del wcs, wc
            # prefill: the persistent kernel with the zero-point epilogue
            pf = datagen.prefill_linear(0)
            sp = torch.from_numpy(pf["signs"]).to(dev)
            wc, ws, _ = rq.fold_weights(torch.from_numpy(pf["wt"]).to(dev), sp)
            del pf["wt"]
            wsum = rq.weight_code_sums(wc)
            mm, d, k = pf["m"], pf["d"], pf["k"]
            acp, sap, zap, _ = rq.fwht_quant_asym(torch.from_numpy(pf["x"]).to(dev), sp)
            y = torch.empty((mm, k), dtype=torch.float16, device=dev)
            wcs = [wc, wc.clone()]

            def gpa(i):
                rq.w4a4_gemm_asym(acp, sap, zap, wcs[i], ws, wsum, out=y)

            msp = time_launches(torch, gpa, 2, max(5, steps2 // 4), warm2)
            tops = 2 * mm * d * k / (msp * 1e-3) / 1e12
            sec["gemm_asym_prefill_2048x8192x28672"] = line(msp, **{"TOPS": round(tops, 1),
                "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)})
            log(f"[bench] asym prefill gemm: {sec['gemm_asym_prefill_2048x8192x28672']}")
            del wcs, wc, y, acp

        if want("grouped"):
            # per-group (128) INT4 weight scales on the decode and prefill GEMMs
            dec = datagen.decode_linear(0)
            s = torch.from_numpy(dec["signs"]).to(dev)
            acg, sag, _ = rq.fwht_quant(torch.from_numpy(dec["x"]).to(dev), s)
            for k, wt in dec["wts"].items():
                wc, wsg = rq.fold_weights_grouped(torch.from_numpy(wt).to(dev), s, 128)
                nsets = max(2, -(-2 * MALL_BYTES // wc.numel()) + 1)
                wcs = [wc.clone() for _ in range(nsets)]
                for mm in (1, 4, 16):
                    y = torch.empty((mm, k), dtype=torch.float16, device=dev)
                    a_m, s_m = acg[:mm].contiguous(), sag[:mm].contiguous()

                    def gg(i, a_m=a_m, s_m=s_m, y=y):
                        rq.w4a4_gemm_grouped(a_m, s_m, wcs[i], wsg, out=y)

                    msg = time_launches(torch, gg, nsets, steps2, warm2)
                    bb = gemm_bytes(mm, k, 4096) - 2 * k + 2 * k * (4096 // 128)
                    key = f"gemm_grouped_decode_m{mm}_k{k}"
                    sec[key] = line(msg, **{"GB/s": round(bb / (msg * 1e-3) / 1e9, 1),
                                "hbm_frac": round(bb / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                    log(f"[bench] {key}: {sec[key]}")
                del wcs, wc
            pf = datagen.prefill_linear(0)
            sp = torch.from_numpy(pf["signs"]).to(dev)
            wc, wsg = rq.fold_weights_grouped(torch.from_numpy(pf["wt"]).to(dev), sp, 128)
            del pf["wt"]
            mm, d, k = pf["m"], pf["d"], pf["k"]
            acp, sap, _ = rq.fwht_quant(torch.from_numpy(pf["x"]).to(dev), sp)
            y = torch.empty((mm, k), dtype=torch.float16, device=dev)
            wcs = [wc, wc.clone()]

            def gpg(i):
                rq.w4a4_gemm_grouped(acp, sap, wcs[i], wsg, out=y)

            msp = time_launches(torch, gpg, 2, max(5, steps2 // 4), warm2)
            tops = 2 * mm * d * k / (msp * 1e-3) / 1e12
            sec["gemm_grouped_prefill_2048x8192x28672"] = line(msp, **{"TOPS": round(tops, 1),
                "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)})
            log(f"[bench] grouped prefill gemm: {sec['gemm_grouped_prefill_2048x8192x28672']}")
            del wcs, wc, y, acp

        if want("kv"):
            kv = datagen.kv_cache(0)
            kt = torch.from_numpy(kv["k"]).to(dev)
            vt = torch.from_numpy(kv["v"]).to(dev)
            del kv
            rows = kt.numel() // 128
            kc = torch.empty((rows, 64), dtype=torch.uint8, device=dev)
            vc = torch.empty_like(kc)
            ks = torch.empty((rows,), dtype=torch.float16, device=dev)
            vs = torch.empty_like(ks)

            def fkv(i):
                st = lib.rq_kv_rotate_quant(_ptr(kt), _ptr(vt), rows, 128, None, _ptr(kc), _ptr(ks),
                                            _ptr(vc), _ptr(vs), _stream())
                assert st == 0

            mk = time_launches(torch, fkv, 1, max(5, steps2 // 2), warm2)
            b = kv_bytes(rows)
            sec["kv_rotate_quant_32x8x4096x128"] = line(mk, **{"GB/s": round(b / (mk * 1e-3) / 1e9, 1),
                                                    "hbm_frac": round(b / (mk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            log(f"[bench] kv: {sec['kv_rotate_quant_32x8x4096x128']}")
            # decode attention reading that cache: 4 query heads per KV head
            B_, H_, S_, G_ = 32, 8, 4096, 4
            del kt, vt
            # the 4-bit cache (138 MB) rotated over copies totalling more than
            # twice the Infinity Cache, so repeats read it from HBM
            cache = [(kc.view(B_, H_, S_, 64), ks.view(B_, H_, S_), vc.view(B_, H_, S_, 64),
                      vs.view(B_, H_, S_))]
            per_cache = 2 * (kc.numel() + 2 * ks.numel())
            ncache = -(-2 * MALL_BYTES // per_cache) + 1
            cache += [tuple(t.clone() for t in cache[0]) for _ in range(ncache - 1)]
            qa = torch.from_numpy(np.random.default_rng(5).standard_normal(
                (B_, H_ * G_, 128)).astype(np.float16)).to(dev)
            oa = torch.empty_like(qa)
            wsa = rq.decode_attention_workspace(B_, H_, G_, S_, dev)

            def fat(i):
                rq.decode_attention(qa, *cache[i], None, workspace=wsa, out=oa)

            mat = time_launches(torch, fat, ncache, max(5, steps2 // 2), warm2)
            ba = B_ * H_ * S_ * (64 + 64 + 2 + 2) + 2 * (B_ * H_ * G_ * 128 * 2)
            sec["decode_attention_32x8x4096_g4"] = line(mat, **{"GB/s": round(ba / (mat * 1e-3) / 1e9, 1),
                "hbm_frac": round(ba / (mat * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            sec["decode_attention_32x8x4096_g4"]["cache_sets"] = ncache
            log(f"[bench] decode attention: {sec['decode_attention_32x8x4096_g4']}")
            del cache

        if want("ceiling"):
            # what this GPU delivers for plain streams of the sizes the hot path
            # moves (buffers rotate over > 2x the Infinity Cache), and for int8
            # MFMAs on register operands
            import ctypes
            lib.rq_ceiling_read_sink_words.restype = ctypes.c_size_t
            lib.rq_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_void_p]
            lib.rq_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]
            lib.rq_ceiling_mfma_out_words.argtypes = [ctypes.c_int64]
            lib.rq_ceiling_mfma_out_words.restype = ctypes.c_size_t
            lib.rq_ceiling_mfma_i8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p]
            lib.rq_ceiling_mfma_i8.restype = ctypes.c_int64
            sink = torch.empty((int(lib.rq_ceiling_read_sink_words()),), dtype=torch.int32, device=dev)
            for name, nbytes in (("hbm_read_8MiB", 8 << 20), ("hbm_read_28MiB", 28 << 20),
                                 ("hbm_read_32MiB", 32 << 20), ("hbm_read_256MiB", 256 << 20)):
                if not want_line(name):
                    continue
                nb = -(-2 * MALL_BYTES // nbytes) + 1
                bufs = [torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(nb)]

                def rd(i, bufs=bufs, nbytes=nbytes):
                    assert lib.rq_ceiling_read(_ptr(bufs[i]), nbytes, _ptr(sink), _stream()) == 0

                mr = time_launches(torch, rd, nb, steps2, warm2)
                sec[name] = line(mr, **{"GB/s": round(nbytes / (mr * 1e-3) / 1e9, 1),
                                        "hbm_frac": round(nbytes / (mr * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                log(f"[bench] {name}: {sec[name]}")
                del bufs
            for name, nbytes in (("hbm_copy_32MiB", 32 << 20), ("hbm_copy_256MiB", 256 << 20)):
                if not want_line(name):
                    continue
                nb = -(-MALL_BYTES // nbytes) + 1
                srcs = [torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(nb)]
                dsts = [torch.empty((nbytes,), dtype=torch.uint8, device=dev) for i in range(nb)]

                def cp(i, srcs=srcs, dsts=dsts, nbytes=nbytes):
                    assert lib.rq_ceiling_copy(_ptr(srcs[i]), _ptr(dsts[i]), nbytes, _stream()) == 0

                mc = time_launches(torch, cp, nb, steps2, warm2)
                sec[name] = line(mc, **{"GB/s": round(2 * nbytes / (mc * 1e-3) / 1e9, 1),
                                        "hbm_frac": round(2 * nbytes / (mc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
                log(f"[bench] {name}: {sec[name]}")
                del srcs, dsts
            for wps in (2, 4):
                name = f"int8_mfma_loop_{wps}waves_per_simd"
                if not want_line(name):
                    continue
                outm = torch.empty((int(lib.rq_ceiling_mfma_out_words(wps)),), dtype=torch.int32, device=dev)
                ops = [0]

                def mf(i, outm=outm, wps=wps):
                    ops[0] = lib.rq_ceiling_mfma_i8(_ptr(outm), wps, 4096, _stream())
                    assert ops[0] > 0

                mm_ = time_launches(torch, mf, 1, max(5, steps2 // 4), warm2)
                tops = ops[0] / (mm_ * 1e-3) / 1e12
                sec[name] = line(mm_, **{"TOPS": round(tops, 1), "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)})
                log(f"[bench] {name}: {sec[name]}")
                del outm
            lib.rq_ceiling_mfma_f6.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p]
            lib.rq_ceiling_mfma_f6.restype = ctypes.c_int64
            for wps in (2, 4):
                name = f"fp6_mfma_loop_{wps}waves_per_simd"
                if not want_line(name):
                    continue
                outm = torch.empty((int(lib.rq_ceiling_mfma_out_words(wps)),), dtype=torch.int32, device=dev)
                ops = [0]

                def mf6(i, outm=outm, wps=wps):
                    ops[0] = lib.rq_ceiling_mfma_f6(_ptr(outm), wps, 2048, _stream())
                    assert ops[0] > 0

                mm_ = time_launches(torch, mf6, 1, max(5, steps2 // 4), warm2)
                tops = ops[0] / (mm_ * 1e-3) / 1e12
                sec[name] = line(mm_, **{"TOPS": round(tops, 1), "mfma_frac": round(tops / FP6_PEAK_TOPS, 4)})
                log(f"[bench] {name}: {sec[name]}")
                del outm
            # issue rates of the instruction classes the kernels are made of: does
            # VALU work overlap MFMA work on a SIMD (kinds 0, 1, 2 at two
            # wavefronts per SIMD, as in the prefill GEMMs), and what does a DPP
            # lane exchange cost against a plain fp32 op (kinds 3, 4 at four
            # wavefronts per SIMD, as in the rotation)
            lib.rq_ceiling_issue_out_words.argtypes = [ctypes.c_int64]
            lib.rq_ceiling_issue_out_words.restype = ctypes.c_size_t
            lib.rq_ceiling_issue.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_void_p]
            lib.rq_ceiling_issue.restype = ctypes.c_int64
            issue_ns = {}
            for name, kind, wps, per_round in (("issue_mfma8_2waves", 0, 2, 8),
                                               ("issue_cvt_fma32_2waves", 1, 2, 64),
                                               ("issue_mfma8_plus_cvt_fma32_2waves", 2, 2, 72),
                                               ("issue_fmac32_4waves", 3, 4, 32),
                                               ("issue_dpp_fmac32_4waves", 4, 4, 32)):
                if not want_line(name):
                    continue
                outi = torch.empty((int(lib.rq_ceiling_issue_out_words(wps)),), dtype=torch.float32,
                                   device=dev)
                iters = 2048

                def iss(i, outi=outi, kind=kind, wps=wps, iters=iters):
                    assert lib.rq_ceiling_issue(_ptr(outi), kind, wps, iters, _stream()) > 0

                mi = time_launches(torch, iss, 1, max(5, steps2 // 4), warm2)
                # SIMD time per wavefront round, and per wavefront instruction
                ns_round = mi * 1e6 / (iters * wps)
                issue_ns[kind] = ns_round
                extra = {"ns_per_round_per_simd": round(ns_round, 2),
                         "ns_per_instr_per_simd": round(ns_round / per_round, 3)}
                if kind == 2 and 0 in issue_ns and 1 in issue_ns:
                    # 1: the VALU block hides fully under the MFMAs; 0: the two add up
                    hid = (issue_ns[0] + issue_ns[1] - ns_round) / min(issue_ns[0], issue_ns[1])
                    extra["overlap"] = round(hid, 3)
                sec[name] = line(mi, **extra)
                log(f"[bench] {name}: {sec[name]}")
                del outi
    result["secondary"] = sec

    # ------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(log)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
