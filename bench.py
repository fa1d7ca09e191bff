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
MALL_BYTES = 256 * 2 ** 20     # Infinity Cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-secondary", action="store_true", help="time only the main workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="", help="comma list of secondary items to run")
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


def time_launches(torch, fn, sets: int, steps: int, warmup: int):
    """Average per-call milliseconds of fn(i), i cycling over buffer sets.

    `warmup` eager calls, then `steps` calls are captured into one HIP graph
    (so host launch overhead does not starve the GPU), the graph is replayed
    untimed for about a quarter of a second (the shader clock settles under
    sustained load), and one replay is timed with HIP events recorded on the
    stream the kernels run on, between two device synchronisations."""
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
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    time_launches.last_wall_s = time.perf_counter() - w0
    ms = start.elapsed_time(stop) / steps
    del graph
    return ms


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
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
    want = (lambda k: (not only) or k in only)
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

                    msg = time_launches(torch, g, nsets, steps2, warm2)
                    b = gemm_bytes(mm, k, 4096)
                    sec[f"gemm_decode_m{mm}_k{k}"] = {
                        "us": round(msg * 1e3, 3), "GB/s": round(b / (msg * 1e-3) / 1e9, 1),
                        "hbm_frac": round(b / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "TOPS": round(2 * mm * k * 4096 / (msg * 1e-3) / 1e12, 3)}
                    log(f"[bench] decode m={mm} k={k}: {sec[f'gemm_decode_m{mm}_k{k}']}")
                    # the whole decode linear: rotate + quantize the fp16 tokens, then the GEMM
                    x_m = xa[:mm].contiguous()
                    a_q = torch.empty((mm, 2048), dtype=torch.uint8, device=dev)
                    s_q = torch.empty((mm,), dtype=torch.float16, device=dev)

                    def lin_d(i, x_m=x_m, a_q=a_q, s_q=s_q, y=y, mm=mm):
                        st = lib.rq_fwht_quant(_ptr(x_m), RQ_F16, mm, 4096, _ptr(s), _ptr(a_q),
                                               _ptr(s_q), None, _stream())
                        assert st == 0
                        rq.w4a4_gemm(a_q, s_q, wcs[i], ws, out=y)

                    msl = time_launches(torch, lin_d, nsets, steps2, warm2)
                    sec[f"linear_decode_m{mm}_k{k}_rotate_plus_gemm"] = {"us": round(msl * 1e3, 3)}
                    # the same linear as one launch: rotation fused into the GEMM's prologue
                    ws_ld = rq.linear_decode_workspace(mm, 4096, dev)

                    def lin_f(i, x_m=x_m, y=y, ws_ld=ws_ld):
                        rq.linear_decode(x_m, s, wcs[i], ws, workspace=ws_ld, out=y)

                    msf = time_launches(torch, lin_f, nsets, steps2, warm2)
                    sec[f"linear_decode_m{mm}_k{k}_fused"] = {"us": round(msf * 1e3, 3)}
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

            msf = time_launches(torch, f8, fsets, steps2, warm2)
            del xas[1:]
            b = fwht_bytes(mm, d)
            sec["fwht_quant_2048x8192"] = {"us": round(msf * 1e3, 3),
                                           "GB/s": round(b / (msf * 1e-3) / 1e9, 1),
                                           "hbm_frac": round(b / (msf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] fwht_quant 2048x8192: {sec['fwht_quant_2048x8192']}")
            y = torch.empty((mm, k), dtype=torch.float16, device=dev)
            wcs = [wc, wc.clone()]

            def gp(i):
                rq.w4a4_gemm(ac, sa, wcs[i], ws, out=y)

            msp = time_launches(torch, gp, 2, max(5, steps2 // 2), warm2)
            tops = 2 * mm * d * k / (msp * 1e-3) / 1e12
            sec["gemm_prefill_2048x8192x28672"] = {"us": round(msp * 1e3, 2), "TOPS": round(tops, 1),
                                                   "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)}
            log(f"[bench] prefill gemm: {sec['gemm_prefill_2048x8192x28672']}")

            def lin(i):
                f8(0)
                rq.w4a4_gemm(ac, sa, wcs[i], ws, out=y)

            msl = time_launches(torch, lin, 2, max(5, steps2 // 2), warm2)
            sec["linear_prefill_rotate_plus_gemm"] = {"us": round(msl * 1e3, 2)}
            del wcs, wc, y

        if want("downproj"):
            # the online rotation in front of a down projection: 2048 tokens x
            # 14336 = 28 * 512 (H_28 (x) H_512), same input statistics as the
            # prefill activations
            mm, d = 2048, 14336
            rng = np.random.default_rng(4)
            x28 = datagen.activations(rng, mm, d, datagen.outlier_channels(rng, d), 100.0)
            x28 = torch.from_numpy(x28).to(dev)
            s28 = torch.from_numpy(datagen.rademacher(rng, d)).to(dev)
            ac28 = torch.empty((mm, d // 2), dtype=torch.uint8, device=dev)
            sa28 = torch.empty((mm,), dtype=torch.float16, device=dev)
            fsets = -(-2 * MALL_BYTES // (x28.numel() * 2)) + 1
            x28s = [x28] + [x28.clone() for _ in range(fsets - 1)]

            def f28(i):
                st = lib.rq_fwht_quant(_ptr(x28s[i]), RQ_F16, mm, d, _ptr(s28), _ptr(ac28),
                                       _ptr(sa28), None, _stream())
                assert st == 0

            ms28 = time_launches(torch, f28, fsets, steps2, warm2)
            b = fwht_bytes(mm, d)
            sec["fwht_quant_2048x14336"] = {"us": round(ms28 * 1e3, 3),
                                            "GB/s": round(b / (ms28 * 1e-3) / 1e9, 1),
                                            "hbm_frac": round(b / (ms28 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] fwht_quant 2048x14336: {sec['fwht_quant_2048x14336']}")
            del x28s, x28

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
            sec["fwht_quant8_4096x4096"] = {"us": round(ms8 * 1e3, 3),
                                            "GB/s": round(per8 / (ms8 * 1e-3) / 1e9, 1),
                                            "hbm_frac": round(per8 / (ms8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] fwht_quant8 4096x4096: {sec['fwht_quant8_4096x4096']}")
            del x8s, o8, x8
            dec = datagen.decode_linear(0)
            s = torch.from_numpy(dec["signs"]).to(dev)
            ac8, sa8, _ = rq.fwht_quant8(torch.from_numpy(dec["x"]).to(dev), s)
            for k, wt in dec["wts"].items():
                wc, ws, _ = rq.fold_weights(torch.from_numpy(wt).to(dev), s)
                nsets = max(2, -(-2 * MALL_BYTES // wc.numel()) + 1)
                wcs = [wc.clone() for _ in range(nsets)]
                for mm in (1, 4, 16):
                    y = torch.empty((mm, k), dtype=torch.float16, device=dev)
                    a_m, s_m = ac8[:mm].contiguous(), sa8[:mm].contiguous()

                    def g8(i, a_m=a_m, s_m=s_m, y=y):
                        rq.w4a8_gemm(a_m, s_m, wcs[i], ws, out=y)

                    msg = time_launches(torch, g8, nsets, steps2, warm2)
                    bb = gemm8_bytes(mm, k, 4096)
                    key = f"gemm_w4a8_decode_m{mm}_k{k}"
                    sec[key] = {"us": round(msg * 1e3, 3), "GB/s": round(bb / (msg * 1e-3) / 1e9, 1),
                                "hbm_frac": round(bb / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
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
            sec["gemm_w4a8_prefill_2048x8192x28672"] = {
                "us": round(msp * 1e3, 2), "TOPS": round(tops, 1),
                "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)}
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
            sec["fwht_quant_asym_4096x4096"] = {"us": round(msa * 1e3, 3),
                                                "GB/s": round(pera / (msa * 1e-3) / 1e9, 1),
                                                "hbm_frac": round(pera / (msa * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
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
                    sec[key] = {"us": round(msg * 1e3, 3), "GB/s": round(bb / (msg * 1e-3) / 1e9, 1),
                                "hbm_frac": round(bb / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
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
            sec["gemm_asym_prefill_2048x8192x28672"] = {
                "us": round(msp * 1e3, 2), "TOPS": round(tops, 1),
                "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)}
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
                    sec[key] = {"us": round(msg * 1e3, 3), "GB/s": round(bb / (msg * 1e-3) / 1e9, 1),
                                "hbm_frac": round(bb / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
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
            sec["gemm_grouped_prefill_2048x8192x28672"] = {
                "us": round(msp * 1e3, 2), "TOPS": round(tops, 1),
                "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)}
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
            sec["kv_rotate_quant_32x8x4096x128"] = {"us": round(mk * 1e3, 2),
                                                    "GB/s": round(b / (mk * 1e-3) / 1e9, 1),
                                                    "hbm_frac": round(b / (mk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] kv: {sec['kv_rotate_quant_32x8x4096x128']}")
            # decode attention reading that cache: 4 query heads per KV head
            B_, H_, S_, G_ = 32, 8, 4096, 4
            kc4, ks4 = kc.view(B_, H_, S_, 64), ks.view(B_, H_, S_)
            vc4, vs4 = vc.view(B_, H_, S_, 64), vs.view(B_, H_, S_)
            qa = torch.from_numpy(np.random.default_rng(5).standard_normal(
                (B_, H_ * G_, 128)).astype(np.float16)).to(dev)
            oa = torch.empty_like(qa)
            wsa = rq.decode_attention_workspace(B_, H_, G_, S_, dev)

            def fat(i):
                rq.decode_attention(qa, kc4, ks4, vc4, vs4, None, workspace=wsa, out=oa)

            mat = time_launches(torch, fat, 1, max(5, steps2 // 2), warm2)
            ba = B_ * H_ * S_ * (64 + 64 + 2 + 2) + 2 * (B_ * H_ * G_ * 128 * 2)
            sec["decode_attention_32x8x4096_g4"] = {
                "us": round(mat * 1e3, 2), "GB/s": round(ba / (mat * 1e-3) / 1e9, 1),
                "hbm_frac": round(ba / (mat * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] decode attention: {sec['decode_attention_32x8x4096_g4']}")
            del kt, vt
    result["secondary"] = sec

    # ------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        from oracle import rq_oracle as O
        rows = 1024
        xs_ = w["x"][:rows]
        t0 = time.perf_counter()
        reps = 0
        while True:
            O.fwht_quant(xs_, w["signs"], "f64")
            reps += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or reps >= 50:
                break
        cpu_gbs = reps * fwht_bytes(rows, n) / el / 1e9
        result["cpu_baseline"] = {
            "value": round(cpu_gbs, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"fp64 oracle fwht_quant on the first {rows} of the 4096 rows, "
                      f"{reps} repetitions, {el:.1f} s (numpy, single thread)"}
        log(f"[bench] cpu oracle: {cpu_gbs * 1e3:.3f} MB/s")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
