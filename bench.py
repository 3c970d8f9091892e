#!/usr/bin/env python3
"""Benchmark of the Ozaki II FP64 GEMM emulation on one MI355X.

A step is one whole ozaki2_dgemm call (scaling, residues, s INT8 GEMMs, CRT) on the
synthetic workload, inputs already resident in HBM.  The metric is effective FP64
TFLOPS = 2 p q r / t ("Profiling Ozaki II: The Cost Behind Fast INT8 GEMMs", Part I
section 3), timed over plain calls.  The per-stage breakdown comes from a second loop of
as many calls with the HIP events the library records on the launch stream between its
stages; the GEMM stage is one kernel launch (all s moduli), so its average event interval
is that kernel's average launch duration.

Prints one JSON line.  Only one GPU is supported: --gpus above 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks used for the rooflines
PEAK_INT8_TOPS = 5000.0     # dense INT8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0       # HBM3E, GB/s
# Pages' number for this metric and workload (GH200, fast-14, n = 8192; paper Table 3)
PAGES_FAST14_N8192_GH200 = 72.1


GEMM_SOURCE = os.path.join(ROOT, "fp64_gemm_emulation_amd", "csrc", "oz2_gemm.hip")


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, or None.

    The summary records FETCH_SIZE and WRITE_SIZE of the GEMM kernel scaled by the same
    counters on a plain device copy of known size, and the SHA-256 of the GEMM source it
    was taken with; a different source means the figure is stale and None is returned.
    """
    path = os.path.join(ROOT, "profiles", f"gemm_w8_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src_hash = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if fields.get("gemm_source_sha256") != src_hash:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stage_bytes(n_p, n_q, n_r, s, accu):
    """Algorithmic HBM bytes per call of each memory-bound stage."""
    a_elems, b_elems = n_p * n_q, n_q * n_r
    scaling = 8 * (a_elems + b_elems) * (2 if accu else 1) + (2 * (a_elems + b_elems) if accu else 0)
    residues = 8 * (a_elems + b_elems) + s * (a_elems + b_elems)
    crt = s * n_p * n_r + 8 * n_p * n_r
    return scaling, residues, crt


def cpu_baseline(A, B, s, mode, rows, cols):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    p, q, r = A.shape[0], A.shape[1], B.shape[1]
    rows, cols = min(rows, p), min(cols, r)
    stage_s = {}
    t0 = time.perf_counter()
    oracle.ozaki2_sample(A, B, s, mode, np.arange(rows), np.arange(cols), timings=stage_s)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * q * cols
    # The whole product, extrapolated stage by stage from the sample by the ratio of each
    # stage's work: the fast scalings and the residues grow with the lines they cover (rows
    # of A plus columns of B), the products and the CRT with the outputs.  The accu scaling
    # of the sample already quantizes the whole operands and forms the bound product for the
    # sampled rows and columns (rows r + p cols entries); its factor is that product's ratio,
    # an upper bound since the quantization does not grow.
    line_ratio = (p + r) / (rows + cols)
    out_ratio = (p * r) / (rows * cols)
    bound_ratio = (p * r) / (rows * r + p * cols)
    factors = {"scaling": bound_ratio if mode == "accu" else line_ratio, "residues": line_ratio,
               "gemm": out_ratio, "crt": out_ratio}
    full = {k: stage_s[k] * factors[k] for k in factors}
    full_s = sum(full.values())
    return {
        "value": flops / dt / 1e12,
        "unit": "effective FP64 TFLOPS",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"C[0:{rows}, 0:{cols}] of the {p}x{q}x{r} workload "
                  f"(scalings of the sampled rows/columns, their residues, s products, CRT, inverse scaling)",
        "seconds": dt,
        "stage_seconds": stage_s,
        "full_product_extrapolated": {
            "seconds": full_s,
            "effective_tflops": 2.0 * p * q * r / full_s / 1e12,
            "stage_seconds": full,
            "stage_factors": factors,
            "sample_fraction_of_outputs": rows * cols / (p * r),
            "basis": "each stage's sample time times its work ratio: lines (p + r) / (rows + cols) "
                     "for fast scaling and residues, outputs p r / (rows cols) for products and CRT, "
                     "bound-product entries p r / (rows r + p cols) for accu scaling (an upper bound)",
        },
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def host_fp64_matmul_context(A, B, m=2048, reps=3):
    """Host FP64 BLAS (numpy) on the leading m x m blocks of the operands, for context."""
    import numpy as np
    m = min(m, A.shape[0], A.shape[1], B.shape[1])
    a = np.ascontiguousarray(A[:m, :m])
    b = np.ascontiguousarray(B[:m, :m])
    best = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        np.matmul(a, b)
        best = min(best, time.perf_counter() - t0)
    return {"host_fp64_matmul_tflops": 2.0 * m ** 3 / best / 1e12, "host_fp64_matmul_shape": m}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def native_fp64_context(Ad, Bd, n, reps=10):
    """Native FP64 GEMM of the same operands through torch (vendor library), for context."""
    import torch
    Cn = torch.matmul(Ad, Bd)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.matmul(Ad, Bd, out=Cn)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return {"native_fp64_matmul_tflops": 2.0 * n ** 3 / dt / 1e12, "native_fp64_matmul_ms": dt * 1e3}


def mfma_ceiling(blocks=1024, rounds=3584, reps=5):
    """Register-only i8 MFMA rate on random, changing operands (libozcalib.so), TOP/s.

    The default size matches the MFMA work of one n = 8192, s = 14 GEMM launch.  Under the
    board's power limit this is the practical ceiling of a GEMM on residues."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "fp64_gemm_emulation_amd", "libozcalib.so"))
    lib.oz2calib_mfma_i8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.oz2calib_mfma_i8.restype = ctypes.c_int
    gen = torch.Generator(device="cuda").manual_seed(7)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (blocks * 8 * 512 * 4,), dtype=torch.int32, device="cuda", generator=gen)
    out = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: lib.oz2calib_mfma_i8(src.data_ptr(), blocks, rounds, out.data_ptr(), stream.cuda_stream)
    assert call() == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    ops = blocks * 8 * 16 * 16384 * 2.0 * rounds  # 2^21 multiply-adds per block and round
    return ops / (ms * 1e-3) / 1e12


def gemm_vs_shape_ceiling(call, s, n, rounds=3, calls=5):
    """The GEMM stage against the register-only MFMA kernel of the GEMM's exact shape
    (libozcalib.so: the GEMM's grid of 256 x 256 tiles over all planes, 8 waves of 8 x 4
    blocks, fragments changing every 64-deep stage, one workgroup per CU), alternated in
    rounds so that both run at the same thermal state.  Both do s 2 n^3 int8 operations per
    launch; what separates them is the GEMM's memory traffic and epilogue."""
    import ctypes
    import torch
    from fp64_gemm_emulation_amd import binding
    lib = ctypes.CDLL(os.path.join(ROOT, "fp64_gemm_emulation_amd", "libozcalib.so"))
    lib.oz2calib_mfma_i8_gemm_shape.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                                ctypes.c_void_p]
    lib.oz2calib_mfma_i8_gemm_shape.restype = ctypes.c_int
    tiles, stages = (n // 256) ** 2 * s, n // 64
    gen = torch.Generator(device="cuda").manual_seed(11)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (1024 * 12 * 512 * 4,), dtype=torch.int32, device="cuda",
                        generator=gen)
    out = torch.empty(tiles * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    ops = s * 2.0 * n ** 3
    gemm_ms, ceil_ms = [], []
    for _ in range(rounds):
        assert binding.ozaki2_timing_begin(calls) == binding.OZ2_OK
        for _ in range(calls):
            call(stream)
        rc, st, k = binding.ozaki2_timing_end()
        assert rc == binding.OZ2_OK and k == calls
        gemm_ms.append(st[2] / calls)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            assert lib.oz2calib_mfma_i8_gemm_shape(src.data_ptr(), tiles, stages, out.data_ptr(), stream.cuda_stream) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        ceil_ms.append(e0.elapsed_time(e1) / calls)
    g, c = sum(gemm_ms) / rounds, sum(ceil_ms) / rounds
    return {"gemm_ms": g, "gemm_shape_ceiling_ms": c, "gemm_tops": ops / (g * 1e-3) / 1e12,
            "gemm_shape_ceiling_tops": ops / (c * 1e-3) / 1e12, "gemm_over_gemm_shape_ceiling": c / g,
            "rounds": rounds, "launches_per_round": calls}


def exact_dot_samples(A, B, rows, cols):
    """Exact (A B)_ij for the sampled entries, as Fractions (integer arithmetic on the FP64
    significands; independent of the library and of the test oracle)."""
    import numpy as np
    from fractions import Fraction

    def ints(v):
        m, e = np.frexp(v)
        return [int(x) for x in (m * 2.0 ** 53).astype(np.int64)], (e.astype(np.int64) - 53).tolist()

    out = {}
    for i in rows:
        ma, ea = ints(A[i, :])
        for j in cols:
            mb, eb = ints(B[:, j])
            ex = [x + y for x, y in zip(ea, eb)]
            e0 = min(ex)
            total = sum((x * y) << (e - e0) for x, y, e in zip(ma, mb, ex))
            out[(i, j)] = Fraction(total) * Fraction(2) ** e0 if e0 >= 0 else Fraction(total, 2 ** (-e0))
    return out


def rel_errors(C_sample, exact, absab):
    """|C_ij - (AB)_ij| / (|A||B|)_ij over the samples."""
    from fractions import Fraction
    errs = []
    for (i, j), v in exact.items():
        errs.append(float(abs(Fraction(float(C_sample[(i, j)])) - v) / Fraction(float(absab[(i, j)]))))
    return errs


def sweep(args):
    """s- and n-sweep of the emulated product (fast and accu): time per call, stage
    breakdown and error against the exact product on sampled entries; one JSON line per
    configuration.  Inputs: the phi = 0.5 generator of the headline workload."""
    import numpy as np
    import torch

    from fp64_gemm_emulation_amd import binding
    from fp64_gemm_emulation_amd.workloads import generate

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    rng = np.random.default_rng(99)
    for n in args.sweep_n:
        A = generate(n, n, args.sweep_phi, 1)
        B = generate(n, n, args.sweep_phi, 2)
        rows = sorted(rng.choice(n, size=8, replace=False).tolist())
        cols = sorted(rng.choice(n, size=8, replace=False).tolist())
        exact = exact_dot_samples(A, B, rows, cols)
        absab = {(i, j): float(np.abs(A[i, :]) @ np.abs(B[:, j])) for i in rows for j in cols}
        Ad = binding.colmajor(torch.from_numpy(np.ascontiguousarray(A)).to(dev))
        Bd = binding.colmajor(torch.from_numpy(np.ascontiguousarray(B)).to(dev))
        C = binding.empty_colmajor(n, n, device=dev)
        ri = torch.tensor(rows, device=dev)
        ci = torch.tensor(cols, device=dev)

        def samples(M):  # the sampled entries only: no full device-to-host copy
            sub = M[ri][:, ci].cpu().numpy()
            return {(i, j): sub[a, b] for a, i in enumerate(rows) for b, j in enumerate(cols)}

        nerr = rel_errors(samples(torch.matmul(Ad, Bd)), exact, absab)
        print(json.dumps({"sweep": "native_fp64", "n": n, "max_rel_err": max(nerr)}), flush=True)
        for mode in args.sweep_modes:
            for s in args.sweep_s:
                for _ in range(2):
                    binding.dgemm(Ad, Bd, s, mode, out=C, stream=stream)
                torch.cuda.synchronize()
                steps = args.sweep_steps
                assert binding.ozaki2_timing_begin(steps) == binding.OZ2_OK
                t0 = time.perf_counter()
                for _ in range(steps):
                    binding.dgemm(Ad, Bd, s, mode, out=C, stream=stream)
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) * 1e3 / steps
                rc, stage_ms, ncalls = binding.ozaki2_timing_end()
                st = [v / ncalls for v in stage_ms]
                errs = rel_errors(samples(C), exact, absab)
                print(json.dumps({"sweep": "ozaki2", "n": n, "mode": mode, "s": s, "ms_per_call": ms,
                                  "eff_tflops": 2.0 * n ** 3 / (ms * 1e-3) / 1e12,
                                  "stage_ms": {"scaling": st[0], "residues": st[1], "gemm": st[2], "crt": st[3]},
                                  "gemm_int8_tops": s * 2.0 * n ** 3 / (st[2] * 1e-3) / 1e12,
                                  "max_rel_err": max(errs), "median_rel_err": sorted(errs)[len(errs) // 2]}),
                      flush=True)
        del Ad, Bd, C
        torch.cuda.empty_cache()


def overlap_probe(args):
    """Upper bound on what overlapping one product's stages with another's can gain: the
    same K products (n x n fast, the generator of the n = 2048 workload) run back to back on
    one stream, then split over two streams of default priority with a workspace each, so
    the scheduler may run any stage of one product beside any stage of the other (the
    preprocessing of the next beside the GEMMs of the current, as in an overlap by modulus
    group, is one such schedule), and one call captured in a HIP graph and replayed (the
    GPU time of a call without the host's launch work).  One JSON line per size."""
    import numpy as np
    import torch

    from fp64_gemm_emulation_amd import binding
    from fp64_gemm_emulation_amd.workloads import generate

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for n in args.overlap_probe:
        s = args.probe_s
        A = generate(n, n, 0.5, 1)
        B = generate(n, n, 0.5, 2)
        Ad = binding.colmajor(torch.from_numpy(np.ascontiguousarray(A)).to(dev))
        Bd = binding.colmajor(torch.from_numpy(np.ascontiguousarray(B)).to(dev))
        need = binding.ozaki2_workspace_size(n, n, n, s, binding.OZ2_FAST)
        ws = [torch.empty(need + 256, dtype=torch.uint8, device=dev) for _ in range(2)]
        base = [(w.data_ptr() + 255) // 256 * 256 for w in ws]
        outs = [binding.empty_colmajor(n, n, device=dev) for _ in range(2)]
        streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
        K = args.probe_calls

        def run(two):
            for k in range(K):
                j = k % 2 if two else 0
                binding.ozaki2_set_workspace(base[j], need)
                binding.dgemm(Ad, Bd, s, "fast", out=outs[j], stream=streams[j])

        results = {}
        for label, two in (("one_stream", False), ("two_streams", True), ("one_stream_again", False)):
            run(two)                      # warm-up of this arrangement
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run(two)
            torch.cuda.synchronize()
            results[label] = (time.perf_counter() - t0) * 1e3 / K
        assert torch.equal(outs[0], outs[1])
        # one call captured in a HIP graph and replayed on one stream: the same kernels with
        # the host's per-call launch work taken out, i.e. the GPU time of a call
        binding.ozaki2_set_workspace(base[0], need)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=streams[0]):
            binding.dgemm(Ad, Bd, s, "fast", out=outs[0], stream=streams[0])
        outs[0].fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        results["one_stream_graph_replay"] = (time.perf_counter() - t0) * 1e3 / K
        assert torch.equal(outs[0], outs[1])
        del graph
        torch.cuda.synchronize()
        binding.ozaki2_set_workspace(None, 0)
        serial = 0.5 * (results["one_stream"] + results["one_stream_again"])
        print(json.dumps({"overlap_probe": "two independent products on two streams vs one stream",
                          "n": n, "s": s, "mode": "fast", "calls": K,
                          "ms_per_call": results, "two_streams_over_one_stream": results["two_streams"] / serial,
                          "eff_tflops_one_stream": 2.0 * n ** 3 / (serial * 1e-3) / 1e12,
                          "eff_tflops_two_streams": 2.0 * n ** 3 / (results["two_streams"] * 1e-3) / 1e12,
                          "eff_tflops_graph_replay": 2.0 * n ** 3 / (results["one_stream_graph_replay"] * 1e-3) / 1e12}),
              flush=True)
        del Ad, Bd, ws, outs
        torch.cuda.empty_cache()


def tile_probe(args):
    """Lower bound on a GEMM fused with the CRT: a mod GEMM in the library's form with
    256 x 256 and with 128 x 128 output tiles (libozcalib.so), alternated on the same random
    int8 planes of the n x n, s-modulus product, beside the real product's GEMM and CRT
    stages.  A fused kernel has to hold every output's s residues on chip, which rules out
    the 256 x 256 tile; if the 128 x 128 GEMM alone already takes longer than the product's
    GEMM stage plus its separate CRT, the fused kernel cannot win."""
    import ctypes
    import numpy as np
    import torch

    from fp64_gemm_emulation_amd import binding
    from fp64_gemm_emulation_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    n, s = w.n, w.s
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = ctypes.CDLL(os.path.join(ROOT, "fp64_gemm_emulation_amd", "libozcalib.so"))
    lib.oz2calib_gemm_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.oz2calib_gemm_tiles.restype = ctypes.c_int
    stream = torch.cuda.Stream(device=dev)
    gen = torch.Generator(device="cuda").manual_seed(5)
    planes = [torch.randint(-128, 128, (s * n * n,), dtype=torch.int8, device=dev, generator=gen) for _ in range(2)]
    res = torch.empty(s * n * n, dtype=torch.uint8, device=dev)
    ops = s * 2.0 * n ** 3

    def tiles_ms(tile, calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            assert lib.oz2calib_gemm_tiles(planes[0].data_ptr(), planes[1].data_ptr(), n, s, tile, res.data_ptr(),
                                           stream.cuda_stream) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls

    A, B = w.inputs()
    Ad = binding.colmajor(torch.from_numpy(np.ascontiguousarray(A)).to(dev))
    Bd = binding.colmajor(torch.from_numpy(np.ascontiguousarray(B)).to(dev))
    C = binding.empty_colmajor(n, n, device=dev)
    for _ in range(2):
        binding.dgemm(Ad, Bd, s, w.mode, out=C, stream=stream)
    tiles_ms(256, 1)
    tiles_ms(128, 1)
    t256, t128, stages = [], [], []
    for _ in range(3):
        t256.append(tiles_ms(256, 3))
        t128.append(tiles_ms(128, 3))
        assert binding.ozaki2_timing_begin(3) == binding.OZ2_OK
        for _ in range(3):
            binding.dgemm(Ad, Bd, s, w.mode, out=C, stream=stream)
        rc, st, k = binding.ozaki2_timing_end()
        assert rc == binding.OZ2_OK and k == 3
        stages.append([v / k for v in st])
    g256, g128 = sum(t256) / 3, sum(t128) / 3
    gemm_ms = sum(x[2] for x in stages) / 3
    crt_ms = sum(x[3] for x in stages) / 3
    print(json.dumps({"tile_probe": "mod GEMM with 256 x 256 vs 128 x 128 output tiles (random int8 planes), and "
                                    "the product's own GEMM and CRT stages, alternated",
                      "workload": w.name, "n": n, "s": s,
                      "gemm_tile256_ms": g256, "gemm_tile128_ms": g128,
                      "tile256_tops": ops / (g256 * 1e-3) / 1e12, "tile128_tops": ops / (g128 * 1e-3) / 1e12,
                      "product_gemm_stage_ms": gemm_ms, "product_crt_stage_ms": crt_ms,
                      "tile128_over_product_gemm_plus_crt": g128 / (gemm_ms + crt_ms)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="n8192_fast_s14")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context figures (native FP64 matmul, MFMA ceiling on random operands)")
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--cpu-cols", type=int, default=2048)
    ap.add_argument("--zero-inputs", action="store_true",
                    help="diagnostic: A = B = 0 (every residue plane is zero), to show the data-dependent "
                         "power of the INT8 MFMAs; not a benchmark of the workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="s- and n-sweep (one JSON line per configuration) instead of the benchmark line")
    ap.add_argument("--sweep-n", type=int, nargs="+", default=[1024, 2048, 4096, 8192])
    ap.add_argument("--sweep-s", type=int, nargs="+", default=list(range(2, 21)))
    ap.add_argument("--sweep-modes", nargs="+", default=["fast", "accu"])
    ap.add_argument("--sweep-phi", type=float, default=0.5)
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--overlap-probe", type=int, nargs="+", default=None, metavar="N",
                    help="two streams against one for independent n x n fast products (sizes N), instead "
                         "of the benchmark line")
    ap.add_argument("--probe-s", type=int, default=14)
    ap.add_argument("--tile-probe", action="store_true",
                    help="the mod GEMM with 256 x 256 against 128 x 128 tiles and the CRT stage (the bound on a "
                         "GEMM fused with the CRT), instead of the benchmark line")
    ap.add_argument("--probe-calls", type=int, default=60)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); the emulated GEMM is "
              f"measured on one MI355X only", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep(args)
        return
    if args.overlap_probe:
        overlap_probe(args)
        return
    if args.tile_probe:
        tile_probe(args)
        return

    import numpy as np
    import torch

    from fp64_gemm_emulation_amd import binding
    from fp64_gemm_emulation_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    n, s, accu = w.n, w.s, w.mode == "accu"
    if args.zero_inputs:
        A = np.zeros((n, n), order="F")
        B = np.zeros((n, n), order="F")
    else:
        A, B = w.inputs()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Ad = binding.colmajor(torch.from_numpy(np.ascontiguousarray(A)).to(dev))
    Bd = binding.colmajor(torch.from_numpy(np.ascontiguousarray(B)).to(dev))
    C = binding.empty_colmajor(n, n, device=dev)
    torch.cuda.synchronize()
    # a stream of our own (default priority): launches on the legacy null stream wait on
    # implicit synchronisation and leave the GPU idle between kernels
    stream = torch.cuda.Stream(device=dev)

    if args.calibrate_copy:
        src = torch.empty(1 << 27, dtype=torch.float64, device=dev).fill_(1.0)   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        binding.dgemm(Ad, Bd, s, w.mode, out=C, stream=stream)
    torch.cuda.synchronize()

    # The timed steps: plain calls, as a user makes them (no timing events between the
    # stages: each event record leaves the GPU idle for a few microseconds).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        binding.dgemm(Ad, Bd, s, w.mode, out=C, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rc, flags = binding.ozaki2_get_flags()

    # Then the same number of calls again with the library's stage events (HIP events on the
    # launch stream between the stages) for the per-stage breakdown and the GEMM kernel's
    # average duration, and one event per call for the per-call spread.
    assert binding.ozaki2_timing_begin(args.steps) == binding.OZ2_OK
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record(stream)
    for k in range(args.steps):
        binding.dgemm(Ad, Bd, s, w.mode, out=C, stream=stream)
        marks[k + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))
    rc, stage_ms, ncalls = binding.ozaki2_timing_end()
    assert rc == binding.OZ2_OK and ncalls == args.steps

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    eff_tflops = 2.0 * n ** 3 / (ms_per_step * 1e-3) / 1e12
    st = [v / ncalls for v in stage_ms]
    gemm_ops = s * 2.0 * n ** 3
    gemm_tops = gemm_ops / (st[2] * 1e-3) / 1e12
    sb, rb, cb = stage_bytes(n, n, n, s, accu)
    total_stage = sum(st)
    stages = {
        "scaling_ms": st[0], "residues_ms": st[1], "gemm_ms": st[2], "crt_ms": st[3],
        "preprocess_fraction": (st[0] + st[1]) / total_stage,
        # preprocess = scaling + residues against the HBM roof (accu's bound INT8 GEMM is
        # counted in its time but not in its bytes, so its fraction is a lower bound)
        "preprocess_ms": st[0] + st[1],
        "preprocess_frac_hbm": (sb + rb) / ((st[0] + st[1]) * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "residues_GBs": rb / (st[1] * 1e-3) / 1e9,
        "residues_frac_hbm": rb / (st[1] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "scaling_GBs": sb / (st[0] * 1e-3) / 1e9,
        "crt_GBs": cb / (st[3] * 1e-3) / 1e9,
        "crt_frac_hbm": cb / (st[3] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "gemm_frac_int8_peak": gemm_tops / PEAK_INT8_TOPS,
        "residues_per_s": 2.0 * s * n * n / (st[1] * 1e-3),
        "int8_macs_per_s": s * float(n) ** 3 / (st[2] * 1e-3),
        # per call in the stage-timed loop (includes the stage events' idle gaps)
        "step_ms_median_with_stage_events": per_step[len(per_step) // 2],
        "step_ms_min_with_stage_events": per_step[0],
        "step_ms_max_with_stage_events": per_step[-1],
    }
    result = {
        "metric": "effective FP64 TFLOPS (2n^3/t), n=8192 fast-14; per-stage ms breakdown",
        "value": eff_tflops,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (eff_tflops / PAGES_FAST14_N8192_GH200) if args.workload == "n8192_fast_s14" else None,
        "baseline_ref": "pages: GH200 fast-14 n=8192, 72.1 effective TFLOPS (paper Table 3), other hardware",
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name + ("_zero_inputs" if args.zero_inputs else ""), "n": n, "mode": w.mode, "s": s,
                   "phi": w.phi,
                   "seeds": [w.seed_a, w.seed_b], "inputs": "f64 column-major, resident in HBM"},
        "stages": stages,
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_w8_kernel (s batched INT8 GEMMs + mod epilogue)",
            "achieved": gemm_tops,
            "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tops / PEAK_INT8_TOPS,
            "traffic": measured_traffic(w.name),
        },
        "nonfinite_flag": bool(flags & 1),
    }
    if not args.no_context:
        ctx = native_fp64_context(Ad, Bd, n)
        ceil_tops = mfma_ceiling()
        ctx["mfma_i8_ceiling_random_operands_tops"] = ceil_tops
        ctx["gemm_frac_of_mfma_ceiling"] = gemm_tops / ceil_tops
        if n % 256 == 0 and n >= 2048:
            ctx["gemm_vs_gemm_shape_ceiling_interleaved"] = gemm_vs_shape_ceiling(
                lambda st: binding.dgemm(Ad, Bd, s, w.mode, out=C, stream=st), s, n)
        result["context"] = ctx
    if not args.no_cpu_baseline and not args.zero_inputs:
        result["cpu_baseline"] = cpu_baseline(A, B, s, w.mode, args.cpu_rows, args.cpu_cols)
        if "context" in result:
            result["context"].update(host_fp64_matmul_context(A, B))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
