"""Benchmark: quantized matmul on one MI355X.

Headline (one JSON line on stdout): decode quantized_matmul GB/s on the
int4 group-64 affine weight W [14336, 4096] (bf16 scales/biases, [out, in]
layout) with x bf16 [1, 4096] -- one step is one fused quantized matmul
over one token. The second half of the metric (prefill TFLOP/s, x bf16
[2048, 4096] against W [12288, 4096]) and every other workload shape are
measured in the same run and reported alongside.

Timing: inputs resident in HBM; decode steps cycle through >= 512 MB of
distinct weight copies so that the 256 MB Infinity Cache cannot serve them;
the timed launches are captured in a HIP graph (no host overhead between
kernels) and replayed for 200 ms untimed. Each timed replay is bracketed by
torch.cuda.synchronize() and HIP events on the launch stream, with a short
spin kernel before the start event so that host launch latency stays
outside the events. The headline replays exactly `--steps` launches, as
many times as it takes to cover 2 ms (at least 5); every other workload
replays >= 2 ms of launches 5 times. The median replay is reported.
Algorithmic bytes = packed W + scales + biases + x + y, each counted once;
flops = 2*M*N*K.

cpu_baseline: the CPU oracle (test infrastructure, plain C, fp64) on a
bounded sample of the same decode workload, timed on this host; the
prefill block carries its own, on a row sample of the prefill workload.
"""
import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qmm decode GB/s (% of HBM peak) + prefill TFLOP/s; int4 g64 affine"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
ROTATE_BYTES = 512 * 2 ** 20
LOOPS = 5          # timed replays per workload (at least); the median is reported
MAX_LOOPS = 201    # cap on replays of the exact --steps headline graph
MIN_REPLAY_MS = 2.0  # timed work per workload covers at least this
WARM_MS = 200.0    # graph replays before timing, per workload


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--only", choices=["all", "decode", "prefill", "headline", "moe", "in_out", "micro",
                                      "qqmm", "quant"], default="all",
                   help="headline: the two headline workloads; moe, in_out, micro, qqmm: the "
                        "decode headline plus that family alone (for profiling runs)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain device copy of known size (counter scaling)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                          "(no multi-GPU form is implemented)"}))
        sys.exit(2)

    import torch
    import quantized_matmul_amd as qm
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # ------------------------------------------------------------ helpers
    def qw_bytes(qw):
        b = qw.value.numel() * 4 + qw.scales.numel() * qw.scales.element_size()
        if qw.biases is not None:
            b += qw.biases.numel() * qw.biases.element_size()
        return b

    def clone_qw(qw):
        return qm.QuantizedWeight(qw.value.clone(), qw.scales.clone(),
                                  None if qw.biases is None else qw.biases.clone(),
                                  qw.group_size, qw.bits, qw.transpose, qw.mode)

    def make_weight(shape, wid, mode, g, bits, transpose):
        w, _ = synth.normal(shape, 0.02, wid, synth.WEIGHT, "bf16")
        qw = qm.quantize(w.to(dev), g, bits, mode, transpose=transpose)
        del w
        return qw

    # Host launch latency must not land inside a timed region: before each
    # timed replay a spin kernel keeps the GPU busy while the host enqueues
    # the start event and the graph, so the graph's first kernel follows the
    # event at once.
    spin_cycles = calibrate_spin(torch, log)

    def timed(fn_list, steps=None, min_ms=MIN_REPLAY_MS):
        """Time launches of fn_list[s % len] captured in a HIP graph.

        steps given: every timed replay holds exactly that many launches and
        the replay is repeated until the replays cover min_ms (at least
        LOOPS times). steps None: a replay holds enough launches (a multiple
        of len(fn_list)) to last min_ms, replayed LOOPS times. Warm-up: the
        graph replayed for WARM_MS first. Returns (seconds per launch,
        launches per replay, timed replays)."""
        stream = torch.cuda.current_stream()
        for f in fn_list:
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 2 * len(fn_list)
        torch.cuda._sleep(spin_cycles)
        e0.record(stream)
        for s in range(reps):
            fn_list[s % len(fn_list)]()
        e1.record(stream)
        torch.cuda.synchronize()
        est = e0.elapsed_time(e1) / reps                 # ms per launch, eager
        if steps is None:
            n = max(len(fn_list), math.ceil(min_ms / max(est, 1e-4)))
            n = math.ceil(n / len(fn_list)) * len(fn_list)
            loops = LOOPS
        else:
            n = steps
            loops = min(MAX_LOOPS, max(LOOPS, math.ceil(min_ms / max(est * n, 1e-4))))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(n):
                fn_list[s % len(fn_list)]()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < WARM_MS / 1e3:
            g.replay()
            torch.cuda.synchronize()
        times = []
        for _ in range(loops):
            torch.cuda.synchronize()
            torch.cuda._sleep(spin_cycles)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        del g
        return ms / 1e3 / n, n, loops

    # ------------------------------------------------------------ decode
    def bias_vector(N, wid):
        b, _ = synth.normal((N,), 1.0, wid, synth.BIAS, "bf16")
        return b.to(dev)

    def decode_case(M, N, K, bits, g, mode="affine", transpose=True, wid=101, headline=False,
                    dense_bias=False):
        shape = (N, K) if transpose else (K, N)
        qw = make_weight(shape, wid, mode, g, bits, transpose)
        per = qw_bytes(qw)
        ncopy = max(1, math.ceil(ROTATE_BYTES / per))
        copies = [qw] + [clone_qw(qw) for _ in range(ncopy - 1)]
        x, _ = synth.normal((M, K), 1.0, wid, synth.ACT, "bf16")
        x = x.to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if dense_bias:   # quantized_dense: x @ W + bias (bf16, one per column)
            b = bias_vector(N, wid)
            fns = [lambda c=c: qm.quantized_dense(x, c, b, out=y) for c in copies]
        else:
            fns = [lambda c=c: qm.quantized_matmul(x, c, out=y) for c in copies]
        # the headline times exactly --steps launches per replay; the other
        # shapes time replays of >= MIN_REPLAY_MS
        sec, n, loops = timed(fns, steps=args.steps if headline else None)
        alg = per + x.numel() * 2 + y.numel() * 2 + (N * 2 if dense_bias else 0)
        gbs = alg / sec / 1e9
        del copies, fns
        torch.cuda.empty_cache()
        op = "quantized_dense (bf16 bias)" if dense_bias else "qmm"
        return {"workload": f"decode {op} {mode} {bits}-bit g{g} M{M} N{N} K{K} "
                            f"transpose={'true' if transpose else 'false'}",
                "us": sec * 1e6, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                "TFLOP/s": 2 * M * N * K / sec / 1e12, "alg_bytes": alg, "copies": ncopy,
                "steps": n, "replays": loops}

    def prefill_case(M, N, K, bits, g, mode="affine", wid=201, dense_bias=False):
        qw = make_weight((N, K), wid, mode, g, bits, True)
        x, _ = synth.normal((M, K), 1.0, wid, synth.ACT, "bf16")
        x = x.to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if dense_bias:
            b = bias_vector(N, wid)
            fns = [lambda: qm.quantized_dense(x, qw, b, out=y)]
        else:
            fns = [lambda: qm.quantized_matmul(x, qw, out=y)]
        sec, n, loops = timed(fns)
        flops = 2 * M * N * K
        tf = flops / sec / 1e12
        alg = qw_bytes(qw) + x.numel() * 2 + y.numel() * 2 + (N * 2 if dense_bias else 0)
        op = "quantized_dense (bf16 bias)" if dense_bias else "qmm"
        return {"workload": f"prefill {op} {mode} {bits}-bit g{g} M{M} N{N} K{K} transpose=true",
                "us": sec * 1e6, "TFLOP/s": tf, "frac_mfma": tf / MFMA_PEAK_TFLOPS["bf16"],
                "GB/s": alg / sec / 1e9, "flops": flops, "alg_bytes": alg, "steps": n, "replays": loops}

    def quant_case(N, K, bits, g, mode="affine", wid=401):
        """qlin_quantize of a bf16 W [N, K], then qlin_dequantize back to bf16,
        each timed on its own, cycling input copies past the Infinity Cache;
        algorithmic bytes: what each must read and write once."""
        import ctypes
        lib = qm.load_library()
        per = 32 // bits
        w, _ = synth.normal((N, K), 0.02, wid, synth.WEIGHT, "bf16")
        w = w.to(dev)
        ncopy = max(1, math.ceil(ROTATE_BYTES / (w.numel() * 2)))
        ws = [w] + [w.clone() for _ in range(ncopy - 1)]
        G = K // g
        sdt = torch.bfloat16 if mode == "affine" else torch.uint8
        outs = [(torch.empty((N, K // per), dtype=torch.int32, device=dev),
                 torch.empty((N, G), dtype=sdt, device=dev),
                 torch.empty((N, G), dtype=sdt, device=dev) if mode == "affine" else None)
                for _ in range(ncopy)]
        vp = ctypes.c_void_p
        BF16 = 2

        def stream():   # the current stream at call time (graph capture has its own)
            return vp(torch.cuda.current_stream().cuda_stream)

        def q(i):
            wq, sc, bi = outs[i]
            rc = lib.qlin_quantize(vp(ws[i].data_ptr()), BF16, N, K, g, bits, mode.encode(),
                                   vp(wq.data_ptr()), vp(sc.data_ptr()),
                                   vp(bi.data_ptr()) if bi is not None else None, stream())
            assert rc == 0, rc

        dense = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(ncopy)]

        def dq(i):
            wq, sc, bi = outs[i]
            rc = lib.qlin_dequantize(vp(wq.data_ptr()), vp(sc.data_ptr()),
                                     vp(bi.data_ptr()) if bi is not None else None,
                                     BF16 if mode == "affine" else 3, N, K, g, bits,
                                     mode.encode(), vp(dense[i].data_ptr()), BF16, stream())
            assert rc == 0, rc

        tq, n, loops = timed([lambda i=i: q(i) for i in range(ncopy)])
        td, n, loops = timed([lambda i=i: dq(i) for i in range(ncopy)])
        packed = N * K * bits // 8 + N * G * (4 if mode == "affine" else 1)
        bq = N * K * 2 + packed
        res = []
        for name, t, b in (("quantize", tq, bq), ("dequantize", td, bq)):
            res.append({"workload": f"{name} {mode} {bits}-bit g{g} W bf16 [{N},{K}]",
                        "us": t * 1e6, "GB/s": b / t / 1e9, "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS,
                        "alg_bytes": b, "copies": ncopy, "steps": n, "replays": loops})
        del ws, outs, dense
        torch.cuda.empty_cache()
        return res

    def qqmm_case(M, N, K, mode, wid=501):
        """qqmm: x quantized on the fly (one launch into the workspace) then the
        microscaled matmul; weight copies cycled like the decode cases."""
        g, bits = {"mxfp8": (32, 8), "nvfp4": (16, 4)}[mode]
        qw = make_weight((N, K), wid, mode, g, bits, True)
        per = qw_bytes(qw)
        ncopy = max(1, math.ceil(ROTATE_BYTES / per)) if M <= 16 else 1
        copies = [qw] + [clone_qw(qw) for _ in range(ncopy - 1)]
        x, _ = synth.normal((M, K), 1.0, wid, synth.ACT, "bf16")
        x = x.to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(qm.qqmm_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
        fns = [lambda c=c: qm.qqmm(x, c, workspace=ws, out=y) for c in copies]
        fns[0]()
        # mxfp8 at 32 rows or more runs on the scaled fp8 MFMA: its peak is fp8's
        mdt = "fp8" if qm.last_path() == "qqmm_scaled_mfma" else "bf16"
        sec, n, loops = timed(fns)
        # algorithmic bytes: W, its scales, x read once, y written once
        alg = per + x.numel() * 2 + y.numel() * 2
        flops = 2 * M * N * K
        del copies, fns
        torch.cuda.empty_cache()
        return {"workload": f"qqmm {mode} (x quantized on the fly) M{M} N{N} K{K} transpose=true",
                "us": sec * 1e6, "GB/s": alg / sec / 1e9, "frac_hbm": alg / sec / 1e9 / HBM_PEAK_GBS,
                "TFLOP/s": flops / sec / 1e12, "mfma_dtype": mdt,
                "frac_mfma": flops / sec / 1e12 / MFMA_PEAK_TFLOPS[mdt], "alg_bytes": alg,
                "copies": ncopy, "steps": n, "replays": loops}

    def moe_case(sorted_indices, T=512, wid=301):
        """gather_qmm over 64 stacked experts, T tokens x top-8 distinct experts;
        cycles through >= 512 MB of weight copies like the decode cases."""
        E, N, K, k = 64, 1536, 2048, 8
        qw = make_weight((E, N, K), wid, "affine", 64, 4, True)
        per = qw_bytes(qw)
        ncopy = max(1, math.ceil(ROTATE_BYTES / per))
        copies = [qw] + [clone_qw(qw) for _ in range(ncopy - 1)]
        x, _ = synth.normal((T, 1, K), 1.0, wid, synth.ACT, "bf16")
        x = x.to(dev)
        rhs = torch.from_numpy(synth.topk_distinct(T, E, k, wid).astype("int32"))
        lhs = torch.arange(T, dtype=torch.int32).repeat_interleave(k).reshape(T, k)
        if sorted_indices:
            order = torch.argsort(rhs.reshape(-1), stable=True)
            rhs_f, lhs_f = rhs.reshape(-1)[order], lhs.reshape(-1)[order]
        else:
            rhs_f, lhs_f = rhs.reshape(-1), lhs.reshape(-1)
        touched = len(set(rhs_f.tolist()))
        rhs_f, lhs_f = rhs_f.to(dev), lhs_f.to(dev)
        R = rhs_f.numel()
        ws = torch.empty(qm.gather_qmm_workspace_bytes(R, E), dtype=torch.uint8, device=dev)
        y = torch.empty((R, 1, N), dtype=torch.bfloat16, device=dev)
        fns = [lambda c=c: qm.gather_qmm(x, c, rhs_f, lhs_f, sorted_indices=sorted_indices,
                                         workspace=ws, out=y) for c in copies]
        sec, n, loops = timed(fns)
        # algorithmic bytes: the experts the indices touch, each once
        alg = per * touched // E + x.numel() * 2 + y.numel() * 2 + 2 * R * 4
        flops = 2 * R * N * K
        del copies, fns
        torch.cuda.empty_cache()
        return {"workload": f"MoE gather_qmm affine 4-bit g64 E{E} N{N} K{K} tokens{T} top{k} "
                            f"sorted={'true' if sorted_indices else 'false'}",
                "us": sec * 1e6, "GB/s": alg / sec / 1e9, "frac_hbm": alg / sec / 1e9 / HBM_PEAK_GBS,
                "TFLOP/s": flops / sec / 1e12,
                "frac_mfma": flops / sec / 1e12 / MFMA_PEAK_TFLOPS["bf16"], "alg_bytes": alg,
                "experts_touched": touched, "copies": ncopy, "steps": n, "replays": loops}

    results = []
    log("decode headline: affine int4 g64 M1 N14336 K4096")
    head = decode_case(1, 14336, 4096, 4, 64, wid=101, headline=True)
    results.append(head)
    log(json.dumps(head))
    pre = None
    if args.only in ("all", "prefill", "headline"):
        log("prefill: affine int4 g64 M2048 N12288 K4096")
        pre = prefill_case(2048, 12288, 4096, 4, 64, wid=201)
        results.append(pre)
        log(json.dumps(pre))
    if args.only in ("all", "decode"):
        for (M, bits, g, t) in [(4, 4, 64, True), (8, 4, 64, True), (1, 8, 64, True),
                                (1, 2, 32, True), (1, 4, 64, False), (4, 4, 64, False)]:
            r = decode_case(M, 14336, 4096, bits, g, transpose=t, wid=110 + bits)
            results.append(r)
            log(json.dumps(r))
        for mode, g, bits in [("mxfp4", 32, 4), ("nvfp4", 16, 4), ("mxfp8", 32, 8)]:
            for M in (1, 16):
                r = decode_case(M, 8192, 8192, bits, g, mode=mode, wid=120)
                results.append(r)
                log(json.dumps(r))
        r = decode_case(1, 14336, 4096, 4, 64, wid=101, dense_bias=True)
        results.append(r)
        log(json.dumps(r))
    if args.only in ("all", "prefill"):
        r = prefill_case(2048, 12288, 4096, 4, 128, wid=202)
        results.append(r)
        log(json.dumps(r))
        for mode, g, bits in [("mxfp4", 32, 4), ("nvfp4", 16, 4), ("mxfp8", 32, 8)]:
            r = prefill_case(512, 8192, 8192, bits, g, mode=mode, wid=203)
            results.append(r)
            log(json.dumps(r))
        r = prefill_case(2048, 12288, 4096, 4, 64, wid=201, dense_bias=True)
        results.append(r)
        log(json.dumps(r))
    if args.only in ("all", "quant"):
        for (N, K, bits, g, mode) in [(14336, 4096, 4, 64, "affine"), (8192, 8192, 4, 32, "mxfp4")]:
            for r in quant_case(N, K, bits, g, mode):
                results.append(r)
                log(json.dumps(r))
    if args.only == "quant":   # and nvfp4, whose codes divide by the E4M3 scale
        for r in quant_case(8192, 8192, 4, 16, "nvfp4"):
            results.append(r)
            log(json.dumps(r))
    if args.only == "all":
        for mode in ("mxfp8", "nvfp4"):
            for M in (1, 512):
                r = qqmm_case(M, 8192, 8192, mode)
                results.append(r)
                log(json.dumps(r))
        for s in (False, True):
            r = moe_case(s)
            results.append(r)
            log(json.dumps(r))
        for T in (1, 8):   # decode-sized expert batches
            r = moe_case(False, T=T, wid=305)
            results.append(r)
            log(json.dumps(r))
    if args.only == "in_out":   # [in,out] layout, M1 and M4
        for M in (1, 4):
            r = decode_case(M, 14336, 4096, 4, 64, transpose=False, wid=114)
            results.append(r)
            log(json.dumps(r))
    if args.only == "micro":    # microscaled weights at 16 and 512 rows
        for mode, g, bits in [("mxfp4", 32, 4), ("nvfp4", 16, 4), ("mxfp8", 32, 8)]:
            r = decode_case(16, 8192, 8192, bits, g, mode=mode, wid=120)
            results.append(r)
            log(json.dumps(r))
            r = prefill_case(512, 8192, 8192, bits, g, mode=mode, wid=203)
            results.append(r)
            log(json.dumps(r))
    if args.only == "qqmm":
        for mode in ("mxfp8", "nvfp4"):
            r = qqmm_case(512, 8192, 8192, mode)
            results.append(r)
            log(json.dumps(r))
    if args.only == "moe":
        r = moe_case(False)
        results.append(r)
        log(json.dumps(r))
    if args.copy_probe:
        n = 256 * 2 ** 20
        a = torch.empty(n // 4, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy probe: 5 device copies of {n} bytes")

    # ------------------------------------------------------------ CPU baseline
    cpu = cpu_pre = None
    if not args.no_cpu:
        cpu = cpu_baseline(args.cpu_seconds, log)
        if pre is not None:
            cpu_pre = cpu_baseline_prefill(args.cpu_seconds, log)

    # ------------------------------------------------------------ headline
    line = {
        "metric": METRIC,
        "value": round(head["GB/s"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "timed_replays": head["replays"],
        "warmup": args.warmup,
        "ms_per_step": head["us"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {"workload": "decode quantized_matmul, affine int4 group 64, bf16 scales/biases, "
                               "x bf16 [1,4096], W [14336,4096] ([out,in], transpose=true)",
                   "M": 1, "N": 14336, "K": 4096, "bits": 4, "group_size": 64, "mode": "affine",
                   "weight_copies_rotated": head["copies"]},
        "roofline": {"bound": "hbm", "achieved": round(head["GB/s"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["frac_hbm"], 4),
                     "traffic": profiled_traffic("qmm_decode_int4_g64_M1_N14336_K4096"),
                     "algorithmic_bytes": head["alg_bytes"]},
        "cpu_baseline": cpu,
    }
    if pre is not None:
        line["prefill"] = {"value": round(pre["TFLOP/s"], 2), "unit": "TFLOP/s",
                           "workload": pre["workload"],
                           "roofline": {"bound": "mfma", "achieved": round(pre["TFLOP/s"], 2),
                                        "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                                        "frac": round(pre["frac_mfma"], 4),
                                        "traffic": profiled_traffic(
                                            "qmm_prefill_int4_g64_M2048_N12288_K4096"),
                                        "algorithmic_bytes": pre["alg_bytes"]},
                           "cpu_baseline": cpu_pre}
    line["configs"] = [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                       for r in results]
    print(json.dumps(line), flush=True)


def profiled_traffic(summary):
    """HBM bytes per launch from a committed rocprofv3 counter summary.

    profiles/<summary>.md carries FETCH_SIZE/WRITE_SIZE per dispatch already
    scaled by what the same counters read for a plain device copy of known
    size. The figure is returned only while the kernel sources hash to what
    was profiled; a changed kernel reports null until it is profiled again.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", summary + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```\n(\{.*?\})\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(rec["traffic_bytes_per_launch"])


def calibrate_spin(torch, log, target_us=150.0):
    """Cycle count for torch.cuda._sleep that keeps the GPU busy about
    target_us (enough for the host to enqueue an event and a graph)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cycles = 200000
    torch.cuda._sleep(cycles)
    torch.cuda.synchronize()
    e0.record()
    torch.cuda._sleep(cycles)
    e1.record()
    torch.cuda.synchronize()
    us = max(e0.elapsed_time(e1) * 1e3, 1.0)
    out = int(min(max(cycles * target_us / us, 1000), 1e9))
    log(f"spin: {cycles} cycles took {us:.1f} us; using {out} cycles before each timed replay")
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_prefill(seconds, log):
    """The oracle on a row sample of the prefill workload (x [2048, 4096],
    W [12288, 4096] int4 g64): the first 16 rows of x against all of W,
    called repeatedly; TFLOP/s counts 2 * rows * N * K per call."""
    import oracle
    import synth

    M, N, K, rows = 2048, 12288, 4096, 16
    _, wb = synth.normal((N, K), 0.02, 201, synth.WEIGHT, "bf16")
    _, xb = synth.normal((M, K), 1.0, 201, synth.ACT, "bf16")
    wq, sc, bi = oracle.quantize(wb, "bf16", 64, 4)
    xs = xb[:rows].copy()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.quantized_matmul(xs, "bf16", wq, sc, bi, True, 64, 4)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"cpu oracle (prefill sample): {calls} calls in {el:.2f}s on {threads} threads")
    return {"value": round(2 * rows * N * K * calls / el / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{calls} oracle quantized_matmul calls on rows 0..{rows - 1} of the prefill "
                      f"x [{M},{K}] against all of W [{N},{K}] int4 g64 (each call dequantizes W "
                      f"densely, then an fp64 matmul), {el:.1f} s wall"}


def cpu_baseline(seconds, log):
    """The oracle on the decode workload, timed on this host's cores."""
    import numpy as np

    import oracle
    import synth

    M, N, K = 1, 14336, 4096
    _, wb = synth.normal((N, K), 0.02, 101, synth.WEIGHT, "bf16")
    _, xb = synth.normal((M, K), 1.0, 101, synth.ACT, "bf16")
    wq, sc, bi = oracle.quantize(wb, "bf16", 64, 4)
    alg = wq.nbytes + sc.nbytes + bi.nbytes + xb.nbytes + M * N * 2
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.quantized_matmul(xb, "bf16", wq, sc, bi, True, 64, 4)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"cpu oracle: {calls} full decode calls in {el:.2f}s on {threads} threads")
    return {"value": round(alg * calls / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{calls} complete oracle quantized_matmul calls on the decode workload "
                      f"(M1 N{N} K{K} int4 g64), {el:.1f} s wall"}


if __name__ == "__main__":
    main()
