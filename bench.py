"""Benchmark of the W8A8 linear layer on one MI355X.

A step is one pass of the run-time path over one batch: per-token int8
quantisation of X (with the smoothing divide) followed by the int8 MFMA GEMM
with the fused dequantisation epilogue to bf16. The default workload is the
Llama-3.1-8B-shaped fused QKV projection in prefill, M=2048 tokens, K=4096,
N=6144, bf16 in and out, alpha 0.5. Calibration and the weight fold are
load-time steps; they run once before the timed region and are reported
beside the step, not inside it.

Prints one JSON line. ``value`` is end-to-end TOP/s, 2*M*N*K per step over the
timed steps (run back to back, HIP events at the two ends only); ``roofline``
rates the GEMM kernel (the dominant one) against the dense int8 MFMA peak (HBM
bandwidth for decode shapes) with its mean duration from HIP events recorded
around each launch in a second pass over the same number of steps;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload.

The ``rmsnorm_*`` workloads start one step earlier, from the residual stream
before the layer's RMSNorm: the first kernel is the fused RMSNorm (gain
gamma / s) + per-token quantisation, the second the same GEMM. Their
smoothing factors come from calibration rows normalised by a plain torch
RMSNorm (load time, outside the timed region).

The ``silu_*`` workloads start from the gate/up projection's bf16 outputs:
the first kernel is the fused SiLU(gate) * up + smoothing + per-token
quantisation, the second the down projection's GEMM. Their smoothing factors
come from calibration rows of h made by plain torch ops at load time.

The ``fp8_*`` workloads run the FP8 (E4M3) variant on the same shapes: a
step is the per-token E4M3 quantisation and the E4M3 GEMM with its
dequantisation; the weights are quantised per channel at load time.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 linear TOPS (quant+int8 GEMM+dequant), 8B shapes, % int8 MFMA peak"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, GB/s
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s
PEAK_FP64_TFLOPS = 78.6   # MI355X binary64 (vector FMA and matrix), TFLOP/s


def big_kernel_suits(m: int, n: int, k: int) -> bool:
    """Whether the 256-row prefill kernel takes this GEMM (the C ABI's rule)."""
    if n < 192 or k % 128:
        return False
    if m >= 256 and m * n >= (1 << 20):
        return True
    return n >= 4096 and k // 128 >= 20 and (m >= 176 or (m >= 129 and n * k >= (1 << 25)))


def decode_steps_per_wave(m: int, n: int, k: int) -> int:
    """Steps per wave of the decode plan (the C ABI's plan, repeated here)."""
    steps = k // 128
    tiles, tb = -(-n // 64), -(-m // 64)
    wgs = tiles * tb
    want = 1 if wgs >= 192 else -(-256 // wgs)
    want = max(1, min(want, steps))
    per = min(-(-steps // want), 32)
    if -(-steps // per) > 1 and tiles * tb > 256:
        per = steps  # no room for the split's counters: K is not split
    return -(-per // 4)


def decode_ring(m: int, f8: bool = False) -> bool:
    """Whether the decode GEMM runs its LDS-ring form (17 tokens and more, int8 and E4M3)."""
    return m >= 17


def decode_kernel_runs(m: int, n: int, k: int, f8: bool = False) -> bool:
    """Whether the library routes this GEMM to its decode kernel (the
    dispatch rule of the C ABI, repeated here to label the measured kernel):
    M <= 64, or up to 256 tokens when the 256-row prefill kernel does not
    apply and the 128 x 128 tiled kernel would have at most 128 tiles; the
    unrolled form only where its 8 steps per wave cover a K slice."""
    if k % 128 or m < 1:
        return False
    if not decode_ring(m, f8) and decode_steps_per_wave(m, n, k) > 8:
        return False
    if m <= 64:
        return True
    if m > 256 or big_kernel_suits(m, n, k):
        return False
    units = (-(-m // 128)) * (-(-n // 128))
    return units <= 128


def decode_one_token_fused(m: int, n: int, k: int) -> bool:
    """Whether the one-call path fuses the quantisation into the one-token
    product (the C ABI's rule for bf16 inputs): one token, a layer at least
    2048 wide, K a multiple of 128 up to 16384."""
    return m == 1 and n >= 2048 and k % 128 == 0 and k <= 16384


def hbm_bound(m: int, n: int, k: int, out_bytes: int) -> bool:
    """Below the ridge point (dense int8 / FP8 peak over HBM bandwidth) the
    GEMM is bound by streaming its operands."""
    ops = 2.0 * m * n * k
    bytes_ = m * k + n * k + 4 * m + 4 * n + out_bytes * m * n
    return ops / bytes_ < PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
PROFILE_PMC = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="qkv_prefill",
                   help="qkv_prefill (default), gateup_prefill, down_prefill, decode_up, decode_down, tiny, "
                        "llm_int8; rmsnorm_qkv_prefill, rmsnorm_gateup_prefill, rmsnorm_decode_up (the step "
                        "starts from the residual stream: fused RMSNorm with the folded gain + quantisation, "
                        "then the GEMM); silu_down_prefill, silu_decode_down (the step starts from the gate/up "
                        "projection's bf16 outputs: fused SiLU(gate)*up + smoothing + quantisation, then the "
                        "down projection GEMM); fp8_qkv_prefill, fp8_gateup_prefill, fp8_down_prefill, fp8_decode_up (the FP8 "
                        "E4M3 variant: per-token "
                        "E4M3 quantisation, then the E4M3 GEMM; no smoothing); gptq_qkv, gptq_down (GPTQ of one "
                        "layer at load time: Hessian of 4096 calibration rows, damping, Cholesky, sweep; "
                        "reports ms per layer)")
    p.add_argument("--eps", type=float, default=1e-5, help="RMSNorm epsilon (rmsnorm_* workloads)")
    p.add_argument("--m", type=int, default=None, help="override the token count (decode workloads)")
    p.add_argument("--alpha", type=float, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle time budget")
    p.add_argument("--one-call", action="store_true",
                   help="time the step as one sq_w8a8_linear_dyn call instead of quantisation + GEMM "
                        "(the default for the one-token config records)")
    p.add_argument("--no-configs", action="store_true",
                   help="default workload only: skip the per-config records of the other configurations")
    p.add_argument("--ingest-stats", default=None,
                   help="record a rocprofv3 --stats kernel_stats.csv for --workload in profiles/pmc_traffic.json "
                        "(with --kernel-match and --kernel-file); no GPU needed")
    p.add_argument("--pmc-fetch", default=None, help="rocprofv3 --pmc FETCH_SIZE counter_collection.csv to record")
    p.add_argument("--pmc-write", default=None, help="rocprofv3 --pmc WRITE_SIZE counter_collection.csv to record")
    p.add_argument("--kernel-match", default="gemm_big_kernel", help="substring of the kernel name to record")
    p.add_argument("--kernel-file", default="gemm_big.hip", help="source file of that kernel (csrc/)")
    p.add_argument("--fetch-scale", type=float, default=1.9999,
                   help="FETCH_SIZE scale factor from the copy probe (profiles/hbm_counter_scale_copy.md)")
    p.add_argument("--write-scale", type=float, default=1.0, help="WRITE_SIZE scale factor from the copy probe")
    p.add_argument("--probe", choices=["mfma", "stream", "lds", "ldsbw", "gemmparts", "fp8sum", "quantsitu"],
                   default=None,
                   help="only run one measurement probe (libsq_probes.so) and print its JSON line: mfma = "
                        "int8 matrix-core rate and shader clock with constant and changing operands; stream = "
                        "single-kernel streaming read / read+write ceilings at the workloads' sizes; lds = "
                        "fragment-read rate of the prefill GEMM's LDS pattern beside the MFMA rate; ldsbw = LDS read "
                        "throughput by instruction width; gemmparts = the prefill GEMM's main loop taken apart "
                        "(MFMAs, fragment reads, barriers, stage transfers); fp8sum = "
                        "summation error of the E4M3 matrix instructions against exact sums; quantsitu = the "
                        "activation quantiser (libsq.so) with its input in the last-level cache, evicted by clean "
                        "reads, and evicted by writes (as after a prefill GEMM's output)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain device-to-device copy of 512 MiB (5 times), the known-size "
                        "reference that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def copy_probe():
    import torch
    n = 512 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def probe_lib():
    """The measurement probes (w8a8_int8_quantization_amd/probes/probes.hip)."""
    import ctypes

    path = os.path.join(ROOT, "w8a8_int8_quantization_amd", "libsq_probes.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built: python w8a8_int8_quantization_amd/build.py --probes")
    lib = ctypes.CDLL(path)
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    for name, argt in (("sqp_mfma_rate", [P, P, I, I, I, P]), ("sqp_stream", [P, L, P, L, P, I, I, P]),
                       ("sqp_lds_rate", [P, P, I, I, I, P]), ("sqp_fp8_mfma", [P, P, P, I, I, P]),
                       ("sqp_lds_bw", [P, P, I, I, I, I, I, I, P]), ("sqp_gemm_parts", [P, P, I, I, I, P, L, P])):
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = I
    return lib


def _probe_time(torch, launch, reps, inner=1):
    """Median HIP-event time (us) per launch over `reps` rounds of `inner`
    launches back to back on the current stream (inner > 1 hides the
    dispatch gap in front of each launch, as in a steady stream of kernels)."""
    st = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(inner):
            rc = launch()
            if rc != 0:
                raise SystemExit(f"probe launch failed: HIP error {rc}")
        e1.record(st)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / inner)
    return sorted(times)[len(times) // 2]


def _sclk_ghz(clocks):
    """Shader clock (GHz) per workgroup from its s_memtime / s_memrealtime (100 MHz) deltas."""
    c = clocks.cpu().numpy().reshape(-1, 4).astype("float64")
    ticks, real = c[:, 2] - c[:, 0], c[:, 3] - c[:, 1]
    ok = real > 0
    ghz = (ticks[ok] / real[ok]) * 0.1
    real_us = real[ok] / 100.0
    import numpy as np
    return float(np.median(ghz)), float(np.median(real_us))


def run_probe(args):
    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    stream = lambda: ctypes_stream(torch)
    out = {"probe": args.probe, "device": torch.cuda.get_device_name(0)}
    if args.probe == "quantsitu":
        # The per-token quantiser of the product library at the prefill sizes,
        # one launch per measurement (HIP events around it), after: (a) the
        # same launch (input and output in the 256 MiB last-level cache); (b)
        # a read of 1 GiB (the cache holds clean lines of other data); (c) a
        # write of 1 GiB (the cache holds dirty lines, as after a GEMM that
        # wrote a large output: every miss of the quantiser then also evicts
        # a dirty line to HBM).
        import w8a8_int8_quantization_amd as sq
        q_fn = sq.raw["sq_quant_act_per_token"]
        big = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(7)
        res = {}
        for name, m, k in (("qkv_2048x4096", 2048, 4096), ("gateup_8192x4096", 8192, 4096),
                           ("down_8192x14336", 8192, 14336)):
            x = torch.randn(m, k, device=dev).to(torch.bfloat16)
            s_ = torch.rand(k, device=dev) + 0.5
            xq = torch.empty(m, k, dtype=torch.int8, device=dev)
            dx = torch.empty(m, dtype=torch.float32, device=dev)
            args_ = (x.data_ptr(), sq.SQ_BF16, m, k, k, s_.data_ptr(), xq.data_ptr(), dx.data_ptr(), stream())
            nbytes = m * k * 2 + 4 * k + m * k + 4 * m
            for cond in ("cached", "after_clean_reads", "after_writes"):
                times = []
                for rep in range(12):
                    if cond == "after_clean_reads":
                        big.sum(dtype=torch.int64)
                    elif cond == "after_writes":
                        big.fill_(rep & 0xFF)
                    else:
                        q_fn(*args_)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    if q_fn(*args_) != 0:
                        raise SystemExit("quantiser launch failed")
                    e1.record()
                    e1.synchronize()
                    if rep >= 2:
                        times.append(e0.elapsed_time(e1) * 1e3)
                us = sorted(times)[len(times) // 2]
                res[f"{name}_{cond}"] = {"us": us, "tbs_algorithmic": nbytes / us / 1e6, "bytes": nbytes}
            del x, xq
        out["results"] = res
        out["setup"] = ("sq_quant_act_per_token on bf16 rows with smoothing factors, one launch between two HIP "
                        "events (the launch's dispatch gap included alike in every case), median of 10")
        print(json.dumps(out), flush=True)
        return
    lib = probe_lib()
    if args.probe == "mfma":
        blocks, iters = 256, 20000
        clocks = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
        sink = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
        ops_i8 = blocks * 4 * iters * 16 * 2 * 32 * 32 * 32
        for name, rnd in (("constant_operands", 0), ("changing_operands", 1), ("e4m3_constant_operands", 2),
                          ("e4m3_changing_operands", 3)):
            ops = ops_i8 * (2 if rnd >= 2 else 1)  # the E4M3 instruction is 32 x 32 x 64
            launch = lambda: lib.sqp_mfma_rate(clocks.data_ptr(), sink.data_ptr(), blocks, iters, rnd, stream())
            _probe_time(torch, launch, 2)
            us = _probe_time(torch, launch, 7)
            ghz, real_us = _sclk_ghz(clocks)
            out[name] = {"us": us, "pops": ops / us / 1e6, "frac_of_5_pops": ops / us / 1e6 / 5000.0,
                         "sclk_ghz": ghz, "in_kernel_us": real_us,
                         "pops_at_sclk_per_cu_clk": ops / (real_us * 1e-6) / (ghz * 1e9) / 256}
        out["setup"] = (f"{blocks} workgroups x 4 waves (one per SIMD), {iters} x 16 v_mfma_i32_32x32x32_i8 per wave, "
                        "8 independent accumulators; changing operands: 16 A and 16 B fragments of hashed bytes "
                        "combined in rotation, so no two consecutive MFMAs share operands; e4m3: the same with "
                        "v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales), 8 operand pairs of finite codes "
                        "(constant: 1.0), frac_of_5_pops against the 5.0 PFLOP/s dense FP8 nameplate")
    elif args.probe == "stream":
        res = {}
        sink = torch.zeros(4096 * 256, dtype=torch.int32, device=dev)
        # decode: 58.7 MB of weights per launch, rotating over copies that exceed the 256 MiB last-level cache
        wbytes = 14336 * 4096
        ncopy = 14
        bufs = [torch.empty(wbytes, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(ncopy)]
        dummy = torch.empty(16, dtype=torch.uint8, device=dev)
        best = None
        for depth in (4, 8, 16):
            for grid in (256, 512, 1024, 2048):
                it = {"i": 0}

                def launch(grid=grid, depth=depth, it=it):
                    b = bufs[it["i"] % ncopy]
                    it["i"] += 1
                    return lib.sqp_stream(b.data_ptr(), wbytes, dummy.data_ptr(), 0, sink.data_ptr(), grid, depth,
                                          stream())
                _probe_time(torch, launch, 2, ncopy)
                us = _probe_time(torch, launch, 7, ncopy)
                r = {"us": us, "tbs": wbytes / us / 1e6, "grid": grid, "depth": depth}
                res[f"read_58.7MB_grid{grid}_depth{depth}"] = r
                best = r if best is None or us < best["us"] else best
        res["read_58.7MB_best"] = best
        del bufs
        # prefill quantisation shapes: read bf16 [M x K], write int8 [M x K]
        for name, m, k in (("qkv_2048x4096", 2048, 4096), ("gateup_8192x4096", 8192, 4096),
                           ("down_8192x14336", 8192, 14336)):
            src = torch.empty(m * k * 2, dtype=torch.uint8, device=dev).fill_(3)
            dst = torch.empty(m * k, dtype=torch.uint8, device=dev)
            best = None
            for depth in (4, 8, 16):
                for grid in (512, 1024, 2048, 4096):
                    launch = lambda grid=grid, depth=depth: lib.sqp_stream(
                        src.data_ptr(), m * k * 2, dst.data_ptr(), m * k, sink.data_ptr(), grid, depth, stream())
                    _probe_time(torch, launch, 2, 10)
                    us = _probe_time(torch, launch, 7, 20)
                    r = {"us": us, "tbs": 3 * m * k / us / 1e6, "grid": grid, "depth": depth}
                    res[f"rw_{name}_grid{grid}_depth{depth}"] = r
                    best = r if best is None or us < best["us"] else best
            res[f"rw_{name}_best"] = best
            del src, dst
        out["results"] = res
        out["setup"] = ("16-byte loads, per thread a contiguous run of 16-byte vectors with `depth` loads in flight, "
                        "256-thread workgroups, launches back to back (time per launch); the read-only "
                        "case rotates over 14 copies (822 MB) so that every launch streams from HBM; the read+write "
                        "cases read M x K bf16 and write M x K bytes (the activation quantiser's traffic) with "
                        "operands that fit the last-level cache between launches")
    elif args.probe == "lds":
        blocks, iters = 256, 20000
        clocks = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
        sink = torch.zeros(blocks * 512, dtype=torch.int32, device=dev)
        for name, mode in (("reads_only", 0), ("mfma_only", 1), ("reads_and_mfma", 2), ("linear_reads_only", 3)):
            launch = lambda: lib.sqp_lds_rate(clocks.data_ptr(), sink.data_ptr(), blocks, iters, mode, stream())
            _probe_time(torch, launch, 2)
            us = _probe_time(torch, launch, 7)
            ghz, real_us = _sclk_ghz(clocks)
            cycles = real_us * 1e-6 * ghz * 1e9
            r = {"us": us, "sclk_ghz": ghz, "in_kernel_us": real_us}
            if mode != 1:
                r["lds_bytes_per_clk_per_cu"] = 8 * 64 * 5 * 16 * iters / cycles
            if mode in (1, 2):
                ops = blocks * 8 * 6 * iters * 2 * 32 * 32 * 32
                r["pops"] = ops / us / 1e6
                r["frac_of_5_pops"] = ops / us / 1e6 / 5000.0
            out[name] = r
        out["setup"] = (f"{blocks} workgroups x 8 waves (two per SIMD), 64 KiB LDS; per iteration and wave 5 "
                        "ds_read_b128 fragment reads in the prefill GEMM's swizzled 128-byte-row pattern and/or "
                        "6 v_mfma_i32_32x32x32_i8 with constant operands (the kernel's 5 reads per 6 MFMAs)")
    elif args.probe == "ldsbw":
        blocks, iters = 256, 4096
        res = {}
        for pattern, pname in ((0, "linear"), (1, "gemm_fragments")):
            for threads in (512, 1024):
                for nbytes, reads in ((16, 4), (16, 8), (8, 8), (8, 16), (4, 16)):
                    cyc = torch.zeros(blocks * 16, dtype=torch.int64, device=dev)
                    sink = torch.zeros(blocks * threads, dtype=torch.int32, device=dev)
                    launch = lambda: lib.sqp_lds_bw(cyc.data_ptr(), sink.data_ptr(), blocks, threads, iters, nbytes,
                                                    reads, pattern, stream())
                    _probe_time(torch, launch, 2)
                    cmax = float(cyc.view(blocks, 16)[:, : threads // 64].max().item())
                    per_cu = threads * iters * reads * nbytes
                    res[f"{pname}_b{nbytes * 8}_reads{reads}_waves{threads // 64}"] = {
                        "bytes_per_clk_per_cu": per_cu / cmax, "cycles": cmax}
        out["results"] = res
        out["setup"] = (f"{blocks} workgroups of 8 or 16 waves, 64 KiB LDS; each lane reads 16, 8 or 4 bytes per "
                        "instruction, 4 to 16 independent reads in flight per wave and one wait per round; bytes "
                        "per shader clock per CU from each wave's s_memtime (the slowest wave)")
    elif args.probe == "gemmparts":
        blocks, stages = 256, 2000
        kstage = 57344
        src = torch.empty(blocks * 16 * kstage, dtype=torch.int8, device=dev).fill_(1)
        names = ("mfma_only", "plus_fragment_reads", "plus_barrier", "plus_transfers_global_load_lds",
                 "plus_transfers_buffer_resource", "buffer_transfers_no_l2_reuse")
        res = {}
        for mode, name in enumerate(names):
            cyc = torch.zeros(blocks * 8, dtype=torch.int64, device=dev)
            sink = torch.zeros(blocks * 512, dtype=torch.int32, device=dev)
            launch = lambda: lib.sqp_gemm_parts(cyc.data_ptr(), sink.data_ptr(), blocks, stages, mode, src.data_ptr(),
                                                src.numel(), stream())
            _probe_time(torch, launch, 2)
            cmax = float(cyc.max().item())
            per_mfma = cmax / (2.0 * stages * 24)  # two waves per SIMD, 24 MFMAs per wave and stage
            res[name] = {"cycles_per_mfma_per_simd": per_mfma, "frac_of_matrix_core_rate": 32.0 / per_mfma}
        out["results"] = res
        out["setup"] = (f"{blocks} workgroups x 8 waves (two per SIMD), the prefill GEMM's stage structure at "
                        "256 x 192 tiles: per 128-byte stage 4 substeps of 6 v_mfma_i32_32x32x32_i8 per wave "
                        "(32 shader clocks each at the full rate), then fragment reads, one barrier per stage, and "
                        "the stage's 56 KiB of direct-to-LDS transfers added one at a time; the transfer sources "
                        "are L2-resident except in the last case")
    else:
        res = {}
        tiles = 4096
        # E4M3 (OCP) values of all 256 codes; 0x7F and 0xFF are NaN
        codes = np.arange(256)
        e, mnt, sgn = (codes >> 3) & 15, codes & 7, np.where(codes >> 7, -1.0, 1.0)
        val = np.where(e == 0, mnt / 8.0 * 2.0 ** -6, (1 + mnt / 8.0) * 2.0 ** (e - 7.0)) * sgn
        finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
        pos = np.array([c for c in range(128) if c != 0x7F])
        rng = np.random.default_rng(20240)

        def nearest_codes(x):
            # nearest finite E4M3 value (input data only: ties are immaterial here)
            a = np.abs(x)
            order = np.argsort(val[pos])
            sv = val[pos][order]
            j = np.clip(np.searchsorted(sv, a), 1, len(sv) - 1)
            pick = np.where(np.abs(sv[j] - a) < np.abs(sv[j - 1] - a), j, j - 1)
            c = pos[order][pick]
            return np.where(x < 0, c | 0x80, c).astype(np.uint8)

        for dname in ("every_finite_code", "quantised_gaussian"):
            for form, (rows, kk) in ((0, (32, 64)), (1, (16, 128))):
                if dname == "every_finite_code":
                    a8 = rng.choice(finite, size=(tiles, rows, kk)).astype(np.uint8)
                    b8 = rng.choice(finite, size=(tiles, rows, kk)).astype(np.uint8)
                else:
                    g = rng.standard_normal((2, tiles, rows, kk))
                    g = g / np.abs(g).max(axis=-1, keepdims=True) * 448.0
                    a8, b8 = nearest_codes(g[0]), nearest_codes(g[1])
                av, bv = val[a8], val[b8]
                exact = np.einsum("tnk,tmk->tnm", av, bv)
                mag = np.einsum("tnk,tmk->tnm", np.abs(av), np.abs(bv))
                ta = torch.from_numpy(a8.reshape(-1)).to(dev)
                tb = torch.from_numpy(b8.reshape(-1)).to(dev)
                td = torch.empty(tiles * rows * rows, dtype=torch.float32, device=dev)
                rc = lib.sqp_fp8_mfma(ta.data_ptr(), tb.data_ptr(), td.data_ptr(), tiles, form, stream())
                torch.cuda.synchronize()
                if rc != 0:
                    raise SystemExit(f"probe launch failed: HIP error {rc}")
                got = td.cpu().numpy().astype(np.float64).reshape(tiles, rows, rows)
                err = np.abs(got - exact)
                rel = np.where(mag > 0, err / np.where(mag > 0, mag, 1.0), 0.0)
                res[f"{dname}_{'32x32x64' if form == 0 else '16x16x128'}"] = {
                    "max_err_over_sum_abs_products": float(rel.max()),
                    "max_in_units_of_2^-12": float(rel.max() * 4096.0),
                    "p99_err_over_sum_abs_products": float(np.quantile(rel, 0.99)),
                    "exact_fraction": float((err == 0).mean()),
                    "layout_ok": bool(rel.max() < 2.0 ** -6),
                }
        out["results"] = res
        out["setup"] = (f"{tiles} tiles per case, one E4M3 MFMA each with zero accumulators and unit scales; "
                        "exact sums in binary64 (every E4M3 product and these sums are exact there)")
    print(json.dumps(out), flush=True)


def ctypes_stream(torch):
    return torch.cuda.current_stream().cuda_stream


def kernel_source_hash(name: str) -> str:
    """Hash of a kernel's source file and of the shared headers it includes."""
    csrc = os.path.join(ROOT, "w8a8_int8_quantization_amd", "csrc")
    h = hashlib.sha256()
    for path in [os.path.join(csrc, name)] + sorted(glob.glob(os.path.join(csrc, "*.hpp"))):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_entry(workload: str, kernel_file: str):
    """The committed rocprofv3 record of this workload's kernel (profiles/pmc_traffic.json), if its source is current."""
    try:
        with open(PROFILE_PMC) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("source_sha256_16") != kernel_source_hash(kernel_file):
        return None
    return e


def pmc_traffic(workload: str, kernel_file: str):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, if current."""
    e = profile_entry(workload, kernel_file)
    return e.get("hbm_bytes_per_launch") if e else None


def kernel_only(roof: dict, workload: str, kernel_file: str, per_launch: float):
    """Adds the rocprofv3 kernel-only duration of the committed profile (if
    current) and the roofline fraction computed from it, beside the
    event-timed one (HIP events also count the dispatch gap before a launch)."""
    e = profile_entry(workload, kernel_file)
    us = e.get("kernel_us") if e else None
    roof["kernel_us_rocprof"] = us
    roof["frac_kernel_only"] = (per_launch / (us * 1e-6) / (1e9 if roof["unit"] == "GB/s" else 1e12) / roof["peak"]
                                if us else None)
    roof["frac_basis"] = "frac: HIP events around each launch on its stream; frac_kernel_only: rocprofv3 kernel time"


class HipEvents:
    """hipEvent_t timing on one stream through the HIP runtime the library is linked to."""

    def __init__(self, lib, stream: int):
        import ctypes
        self.ct = ctypes
        self.stream = ctypes.c_void_p(stream)
        self._create, self._record = lib.hipEventCreate, lib.hipEventRecord
        self._elapsed, self._destroy = lib.hipEventElapsedTime, lib.hipEventDestroy
        self._create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._record.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._elapsed.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._destroy.argtypes = [ctypes.c_void_p]
        for f in (self._create, self._record, self._elapsed, self._destroy):
            f.restype = ctypes.c_int
        self.events = []

    def create(self):
        e = self.ct.c_void_p()
        if self._create(self.ct.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(e)
        return e

    def record(self, e):
        self._record(e, self.stream)

    def elapsed(self, a, b) -> float:
        ms = self.ct.c_float()
        if self._elapsed(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy_all(self):
        for e in self.events:
            self._destroy(e)
        self.events = []


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(c, s_ref, budget_s: float):
    """The CPU oracle's run-time path (quantise, int8 GEMM, dequantise) on row chunks of X."""
    import numpy as np
    import oracle

    threads = _blas_threads()
    _, wq, sw = oracle.smooth_fold_quantize(None, c.w, c.alpha, s=s_ref)
    # row chunks of X, cycling over the workload until the time budget is spent
    rows, t_total = 0, 0.0
    chunk, start = 64, 0
    while t_total < budget_s:
        r1 = min(c.m, start + chunk)
        t0 = time.perf_counter()
        oracle.smoothquant_linear(c.x[start:r1], s_ref, wq, sw, c.y_dtype)
        t_total += time.perf_counter() - t0
        rows += r1 - start
        start = 0 if r1 == c.m else r1
        chunk = min(chunk * 2, 512)
    tops = 2.0 * rows * c.n * c.k / t_total / 1e12
    return {"value": tops, "unit": "TOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} rows of X ({rows / c.m:.2f} passes over the {c.m}-row workload, all N={c.n} "
                      f"outputs, K={c.k}), {t_total:.1f} s of numpy/BLAS work"}


def cpu_baseline_norm(c, nc, eps, budget_s: float):
    """The CPU oracle's norm path (RMSNorm with the folded gain, quantisation,
    int8 GEMM, dequantisation) on row chunks of the residual stream; its
    smoothing factors from the oracle's own calibration (not timed)."""
    import oracle

    threads = _blas_threads()
    a = oracle.calibrate_absmax(oracle.rmsnorm(nc.x_calib, nc.gamma, eps))
    s_ref = oracle.smoothing_factors(a, oracle.weight_row_absmax(c.w), c.alpha)
    gain = oracle.fold_norm_gain(nc.gamma, s_ref)
    wq, sw = oracle.quantize_weights_per_channel(oracle.fold_weights(c.w, s_ref))
    rows, t_total, start, chunk = 0, 0.0, 0, 64
    while t_total < budget_s:
        r1 = min(c.m, start + chunk)
        t0 = time.perf_counter()
        xq, dx = oracle.rmsnorm_quantize(nc.x[start:r1], gain, eps)
        oracle.w8a8_linear(xq, dx, wq, sw, c.y_dtype)
        t_total += time.perf_counter() - t0
        rows += r1 - start
        start = 0 if r1 == c.m else r1
        chunk = min(chunk * 2, 512)
    return {"value": 2.0 * rows * c.n * c.k / t_total / 1e12, "unit": "TOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} rows of the residual stream ({rows / c.m:.2f} passes over the {c.m}-row workload, "
                      f"all N={c.n} outputs, K={c.k}), {t_total:.1f} s of numpy/BLAS work"}


def cpu_baseline_silu(c, gu, budget_s: float):
    """The CPU oracle's gated path (SiLU(gate) * up, smoothing, quantisation,
    int8 GEMM, dequantisation) on row chunks; smoothing factors from the
    oracle's own calibration (not timed)."""
    import oracle

    threads = _blas_threads()
    a = oracle.calibrate_absmax(oracle.gated_activation(gu.gate_calib, gu.up_calib))
    s_ref = oracle.smoothing_factors(a, oracle.weight_row_absmax(c.w), c.alpha)
    wq, sw = oracle.quantize_weights_per_channel(oracle.fold_weights(c.w, s_ref))
    rows, t_total, start, chunk = 0, 0.0, 0, 16
    while t_total < budget_s:
        r1 = min(c.m, start + chunk)
        t0 = time.perf_counter()
        xq, dx = oracle.silu_mul_quantize(gu.gate[start:r1], gu.up[start:r1], s_ref)
        oracle.w8a8_linear(xq, dx, wq, sw, c.y_dtype)
        t_total += time.perf_counter() - t0
        rows += r1 - start
        start = 0 if r1 == c.m else r1
        chunk = min(chunk * 2, 256)
    return {"value": 2.0 * rows * c.n * c.k / t_total / 1e12, "unit": "TOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} rows of the gate/up outputs ({rows / c.m:.2f} passes over the {c.m}-row workload, "
                      f"all N={c.n} outputs, K={c.k}), {t_total:.1f} s of numpy/BLAS work"}


def bench_fp8(args, dev):
    """FP8 (E4M3) W8A8: quantise X per token, E4M3 GEMM with dequantisation."""
    import numpy as np
    import torch

    import workloads
    import w8a8_int8_quantization_amd as sq

    base = {"fp8_qkv_prefill": "qkv_prefill", "fp8_decode_up": "decode_up", "fp8_gateup_prefill": "gateup_prefill",
            "fp8_down_prefill": "down_prefill"}[args.workload]
    c = workloads.linear_case(base, m=args.m)
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    x, w = to(c.x), to(c.w)
    wq, sw = sq.sq_quant_weights_fp8(w)
    xq = torch.empty((c.m, c.k), dtype=torch.uint8, device=dev)
    dx = torch.empty(c.m, dtype=torch.float32, device=dev)
    y = torch.empty((c.m, c.n), dtype=torch.bfloat16, device=dev)
    decode = decode_kernel_runs(c.m, c.n, c.k, f8=True)
    streamed = hbm_bound(c.m, c.n, c.k, 2)
    # weight-streaming shapes rotate through >= 768 MiB of weight copies so
    # that every step reads its weights from HBM, not the last-level cache
    n_w = -(-(768 << 20) // wq.numel()) if streamed else 1
    wqs = [wq] + [wq.clone() for _ in range(n_w - 1)]
    stream = torch.cuda.current_stream(dev).cuda_stream
    q_fn, g_fn = sq.raw["sq_quant_act_fp8"], sq.raw["sq_fp8_linear"]
    q_args = (x.data_ptr(), sq.SQ_BF16, c.m, c.k, c.k, xq.data_ptr(), dx.data_ptr(), stream)
    gws = sq.fp8_linear_workspace(c.m, c.n, c.k, dev)  # split-K partials and counters (decode shapes)
    gws_p, gws_n = (gws.data_ptr(), gws.numel()) if gws is not None else (None, 0)
    g_args = [(xq.data_ptr(), dx.data_ptr(), w_i.data_ptr(), sw.data_ptr(), c.m, c.n, c.k, y.data_ptr(), sq.SQ_BF16,
               c.n, gws_p, gws_n, stream) for w_i in wqs]
    hip = HipEvents(sq._lib, stream)
    print(f"[bench] workload {args.workload} M={c.m} K={c.k} N={c.n}", file=sys.stderr, flush=True)

    def run(steps, evs=None):
        bad = 0
        for i in range(steps):
            if evs:
                hip.record(evs[i][0])
            bad |= q_fn(*q_args)
            if evs:
                hip.record(evs[i][1])
            bad |= g_fn(*g_args[i % n_w])
            if evs:
                hip.record(evs[i][2])
        if bad:
            raise RuntimeError(f"a C-ABI call failed (status bits {bad})")

    run(args.warmup)
    torch.cuda.synchronize()
    t0, t1 = hip.create(), hip.create()
    hip.record(t0)
    run(args.steps)
    hip.record(t1)
    torch.cuda.synchronize()
    total_ms = hip.elapsed(t0, t1)
    evs = [[hip.create() for _ in range(3)] for _ in range(args.steps)]
    run(args.steps, evs)
    torch.cuda.synchronize()
    quant_ms = float(np.mean([hip.elapsed(e[0], e[1]) for e in evs]))
    gemm_ms = float(np.mean([hip.elapsed(e[1], e[2]) for e in evs]))
    hip.destroy_all()
    ops = 2.0 * c.m * c.n * c.k
    ms = total_ms / args.steps
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    gemm_bytes = c.m * c.k + c.n * c.k + 4 * c.m + 4 * c.n + 2 * c.m * c.n
    if streamed:
        roof = {"bound": "hbm", "achieved": gemm_bytes / (gemm_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "bytes_per_launch": gemm_bytes}
    else:
        roof = {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "ops_per_launch": ops}
    # the E4M3 forms of the decode kernel and of the prefill kernel, or the 128 x 128 kernel
    big = big_kernel_suits(c.m, c.n, c.k)
    kfile, kname = (("gemm_decode.hip", "gemm_decode_ring_kernel<kTok, kF8=true>" if decode_ring(c.m, True)
                     else "gemm_decode_kernel<kMB, kNS, kF8=true>") if decode else
                    ("gemm_big.hip", "gemm_big_kernel<BN, bf16, kVec, kF8=true>") if big else
                    ("gemm_f8.hip", "gemm_f8_kernel"))
    roof.update({"frac": roof["achieved"] / roof["peak"], "traffic": pmc_traffic(args.workload, kfile),
                 "kernel": kname, "launch_us": gemm_ms * 1e3})
    kernel_only(roof, args.workload, kfile, gemm_bytes if streamed else ops)
    result = {
        "metric": METRIC, "value": ops / (ms * 1e-3) / 1e12, "unit": "TOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": f"{args.workload}: X bf16 [{c.m} x {c.k}] -> E4M3 per token, W [{c.k} x {c.n}] E4M3 "
                               f"per channel, bf16 out", "M": c.m, "K": c.k, "N": c.n},
        "gemm_only_tops": gemm_tops, "gemm_us": gemm_ms * 1e3, "quant_us": quant_ms * 1e3,
        "weight_copies": n_w, "roofline": roof, "cpu_baseline": None if args.no_cpu_baseline else
        cpu_baseline_fp8(c, args.cpu_seconds),
    }
    return result


GPTQ_SHAPES = {"gptq_qkv": (4096, 6144), "gptq_down": (14336, 4096)}  # K, N; 8 x 512 calibration rows


def bench_gptq(args, dev):
    """GPTQ of one layer at load time: the Hessian of 4096 calibration rows,
    then damping, Cholesky and the sweep (codes and scales), all in binary64."""
    import numpy as np
    import torch

    import workloads
    import w8a8_int8_quantization_amd as sq

    k, n = GPTQ_SHAPES[args.workload]
    t = 8 * 512
    c = workloads.gptq_case(k, n, t, seed=0)
    x = torch.from_numpy(c.x_calib).to(torch.bfloat16).to(dev)
    w = torch.from_numpy(c.w).to(torch.bfloat16).to(dev)
    # SmoothQuant's calibration first (alpha 0.5): GPTQ starts from the smoothed layer
    absmax = sq.sq_calibrate_absmax(x, torch.zeros(k, dtype=torch.float32, device=dev))
    sd, _, _ = sq.sq_smooth_fold_weights(w, alpha=0.5, absmax=absmax)
    h = torch.zeros((k, k), dtype=torch.float64, device=dev)
    wq = torch.empty((n, k), dtype=torch.int8, device=dev)
    w_scale = torch.empty(n, dtype=torch.float32, device=dev)
    ws = torch.empty(sq.raw["sq_gptq_quantize_workspace_size"](k, n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    h_fn, q_fn = sq.raw["sq_gptq_hessian"], sq.raw["sq_gptq_quantize"]
    h_args = (x.data_ptr(), sq.SQ_BF16, t, k, k, sd.data_ptr(), h.data_ptr(), stream)
    q_args = (h.data_ptr(), w.data_ptr(), sq.SQ_BF16, k, n, n, sd.data_ptr(), 0.01, wq.data_ptr(),
              w_scale.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    hip = HipEvents(sq._lib, stream)
    print(f"[bench] workload {args.workload} K={k} N={n} T={t}", file=sys.stderr, flush=True)

    def run(steps, evs=None):
        bad = 0
        for i in range(steps):
            h.zero_()
            if evs:
                hip.record(evs[i][0])
            bad |= h_fn(*h_args)
            if evs:
                hip.record(evs[i][1])
            bad |= q_fn(*q_args)
            if evs:
                hip.record(evs[i][2])
        if bad:
            raise RuntimeError(f"a C-ABI call failed (status bits {bad})")

    steps = max(1, min(args.steps, 20))
    run(min(args.warmup, 2))
    torch.cuda.synchronize()
    t0, t1 = hip.create(), hip.create()
    hip.record(t0)
    run(steps)
    hip.record(t1)
    torch.cuda.synchronize()
    total_ms = hip.elapsed(t0, t1) / steps
    evs = [[hip.create() for _ in range(3)] for _ in range(steps)]
    run(steps, evs)
    torch.cuda.synchronize()
    hess_ms = float(np.median([hip.elapsed(e[0], e[1]) for e in evs]))
    quant_ms = float(np.median([hip.elapsed(e[1], e[2]) for e in evs]))
    hip.destroy_all()
    # algorithmic binary64 flops: the Hessian's distinct entries K(K+1)/2, 2T
    # flops each; Cholesky K^3/3; the sweep's compensation K^2 N (each of the
    # N channels passes every error on to every later input)
    f_hess = float(t) * k * (k + 1)
    f_chol = k ** 3 / 3.0
    f_sweep = float(k) * k * n
    roof = {"bound": "fp64", "achieved": f_hess / (hess_ms * 1e-3) / 1e12, "peak": PEAK_FP64_TFLOPS,
            "unit": "TFLOP/s", "frac": f_hess / (hess_ms * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, "traffic": None,
            "kernel": "gptq_hessian_kernel", "launch_us": hess_ms * 1e3, "flops_per_launch": f_hess}
    result = {
        "metric": "GPTQ time per layer (Hessian of the calibration rows + damping + Cholesky + sweep)",
        "value": total_ms, "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, 2),
        "ms_per_step": total_ms, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"{args.workload}: calibration X bf16 [{t} x {k}] (correlated channels, smoothed), "
                               f"W bf16 [{k} x {n}] -> GPTQ int8 [{n} x {k}] + per-channel scales",
                   "K": k, "N": n, "T": t, "damp": 0.01},
        "hessian_ms": hess_ms, "quantize_ms": quant_ms,
        "quantize_fp64_tflops": (f_chol + f_sweep) / (quant_ms * 1e-3) / 1e12,
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_gptq(c, args.cpu_seconds),
    }
    return result


def cpu_baseline_gptq(c, budget_s: float):
    """The oracle's GPTQ: its smoothing factors, Hessian and factorisation in
    full, its sweep on as many output channels as the budget allows,
    extrapolated to all N (the channels are independent given H)."""
    import oracle

    threads = _blas_threads()
    s = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w), 0.5)
    t0 = time.perf_counter()
    h = oracle.gptq_hessian(c.x_calib, s)
    t_h = time.perf_counter() - t0
    wf = oracle.fold_weights(c.w, s)
    done, t_sw, chunk = 0, 0.0, 4
    while t_h + t_sw < budget_s and done < c.n:
        cols = slice(done, min(c.n, done + chunk))
        t0 = time.perf_counter()
        oracle.gptq_quantize(wf[:, cols], h)
        t_sw += time.perf_counter() - t0
        done = cols.stop
        chunk = min(chunk * 2, 64)
    # every call repeats the damping, inverse and Cholesky; time them once more on their own
    t0 = time.perf_counter()
    oracle.gptq_quantize(wf[:, :1], h)
    t_fact = time.perf_counter() - t0
    calls = max(1, (done + 63) // 64)
    per_channel = max(0.0, t_sw - calls * t_fact) / done
    est = t_h + t_fact + per_channel * c.n
    return {"value": est * 1e3, "unit": "ms", "cores": threads, "kind": "oracle",
            "sample": f"Hessian of all {c.t} rows ({t_h:.1f} s), damping+inverse+Cholesky ({t_fact:.1f} s), sweep "
                      f"of {done} of {c.n} channels ({t_sw:.1f} s incl. per-call factorisations), per-channel "
                      f"sweep time scaled to all {c.n}"}


def cpu_baseline_fp8(c, budget_s: float):
    """The CPU oracle's FP8 path (E4M3 quantisation, exact product, dequantisation) on row chunks of X."""
    import oracle

    threads = _blas_threads()
    wq, sw = oracle.quantize_weights_fp8(c.w)
    rows, t_total, start, chunk = 0, 0.0, 0, 16
    while t_total < budget_s:
        r1 = min(c.m, start + chunk)
        t0 = time.perf_counter()
        xq, dx = oracle.quantize_activations_fp8(c.x[start:r1])
        oracle.fp8_linear(xq, dx, wq, sw, "bf16")
        t_total += time.perf_counter() - t0
        rows += r1 - start
        start = 0 if r1 == c.m else r1
        chunk = min(chunk * 2, 256)
    return {"value": 2.0 * rows * c.n * c.k / t_total / 1e12, "unit": "TOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} rows of X ({rows / c.m:.2f} passes over the {c.m}-row workload, all N={c.n} outputs, "
                      f"K={c.k}), {t_total:.1f} s of numpy/BLAS work"}


def bench_llm_int8(args, dev):
    """LLM.int8() decomposition, fp16 in and out: a step is outlier detection
    (column max + selection), the masked row-wise quantisation, and the int8
    GEMM whose epilogue adds the fp16 outlier slice, each a C-ABI call timed
    with HIP events on the launch stream."""
    import numpy as np
    import torch

    import workloads
    import w8a8_int8_quantization_amd as sq

    c = workloads.decomp_case(m=args.m)
    print(f"[bench] workload llm_int8 M={c.m} K={c.k} N={c.n} threshold={c.threshold}", file=sys.stderr, flush=True)
    h = lambda a: torch.from_numpy(a).to(torch.float16).to(dev)
    x, w16 = h(c.x), h(c.w)
    _, wq, sw = sq.sq_smooth_fold_weights(w16, flags=sq.SMOOTH_NONE)
    mask = torch.empty(c.k, dtype=torch.uint8, device=dev)
    idx = torch.empty(c.k, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    xq = torch.empty((c.m, c.k), dtype=torch.int8, device=dev)
    dx = torch.empty(c.m, dtype=torch.float32, device=dev)
    y = torch.empty((c.m, c.n), dtype=torch.float16, device=dev)
    nb = sq.raw["sq_outlier_detect_workspace_size"](c.k)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    det, qm, gm = sq.raw["sq_outlier_detect"], sq.raw["sq_quant_act_rows_masked"], sq.raw["sq_int8_decomp_gemm"]
    det_a = (x.data_ptr(), sq.SQ_F16, c.m, c.k, c.k, float(c.threshold), mask.data_ptr(), idx.data_ptr(),
             cnt.data_ptr(), ws.data_ptr(), nb, stream)
    qm_a = (x.data_ptr(), sq.SQ_F16, c.m, c.k, c.k, mask.data_ptr(), xq.data_ptr(), dx.data_ptr(), stream)
    gm_a = (xq.data_ptr(), dx.data_ptr(), x.data_ptr(), c.k, wq.data_ptr(), sw.data_ptr(), w16.data_ptr(), c.n,
            idx.data_ptr(), cnt.data_ptr(), c.m, c.n, c.k, y.data_ptr(), c.n, stream)
    hip = HipEvents(sq._lib, stream)

    def run(steps, evs=None):
        bad = 0
        for i in range(steps):
            if evs:
                hip.record(evs[i][0])
            bad |= det(*det_a)
            if evs:
                hip.record(evs[i][1])
            bad |= qm(*qm_a)
            if evs:
                hip.record(evs[i][2])
            bad |= gm(*gm_a)
            if evs:
                hip.record(evs[i][3])
        if bad:
            raise RuntimeError(f"a C-ABI call failed (status bits {bad})")

    run(args.warmup)
    torch.cuda.synchronize()
    t0, t1 = hip.create(), hip.create()
    hip.record(t0)
    run(args.steps)
    hip.record(t1)
    torch.cuda.synchronize()
    total_ms = hip.elapsed(t0, t1)
    evs = [[hip.create() for _ in range(4)] for _ in range(args.steps)]
    run(args.steps, evs)
    torch.cuda.synchronize()
    part = [float(np.mean([hip.elapsed(e[j], e[j + 1]) for e in evs])) for j in range(3)]
    hip.destroy_all()
    n_out = int(cnt.cpu()[0])
    ops = 2.0 * c.m * c.n * c.k
    ms = total_ms / args.steps
    gemm_tops = ops / (part[2] * 1e-3) / 1e12
    traffic = pmc_traffic("llm_int8" if args.m is None else f"llm_int8_m{c.m}", "gemm_big.hip")
    result = {
        "metric": METRIC, "value": ops / (ms * 1e-3) / 1e12, "unit": "TOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": f"llm_int8: X f16 [{c.m} x {c.k}] -> W [{c.k} x {c.n}], f16 out, threshold "
                               f"{c.threshold}, {n_out} outlier columns detected", "M": c.m, "K": c.k, "N": c.n},
        "detect_us": part[0] * 1e3, "quant_us": part[1] * 1e3, "gemm_us": part[2] * 1e3, "gemm_only_tops": gemm_tops,
        "outlier_columns": n_out,
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": gemm_tops / PEAK_INT8_TOPS, "traffic": traffic, "kernel": "gemm_big_kernel",
                     "ops_per_launch": ops, "launch_us": part[2] * 1e3},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_decomp(c, args.cpu_seconds),
    }
    kernel_only(result["roofline"], "llm_int8" if args.m is None else f"llm_int8_m{c.m}", "gemm_big.hip", ops)
    return result


def cpu_baseline_decomp(c, budget_s: float):
    """The CPU oracle's LLM.int8() layer on row chunks of X (the column mask from all rows, as on the GPU)."""
    import numpy as np
    import oracle

    threads = _blas_threads()
    mask = oracle.detect_outliers(c.x, c.threshold)
    wq, sw = oracle.quantize_weights_per_channel(c.w)
    rows, t_total, start, chunk = 0, 0.0, 0, 64
    while t_total < budget_s:
        r1 = min(c.m, start + chunk)
        t0 = time.perf_counter()
        oracle.int8_decomp_linear(c.x[start:r1], wq, sw, c.w, c.threshold, mask=mask)
        t_total += time.perf_counter() - t0
        rows += r1 - start
        start = 0 if r1 == c.m else r1
        chunk = min(chunk * 2, 512)
    return {"value": 2.0 * rows * c.n * c.k / t_total / 1e12, "unit": "TOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} rows of X ({rows / c.m:.2f} passes over the {c.m}-row workload, all N={c.n} "
                      f"outputs, K={c.k}), {t_total:.1f} s of numpy/BLAS work"}


def bench_linear(args, dev) -> dict:
    """The run-time path of one linear layer (quantisation + GEMM, or the
    fused RMSNorm / gated-activation variants), timed with HIP events."""
    import numpy as np
    import torch

    import workloads
    import w8a8_int8_quantization_amd as sq

    one_call = getattr(args, "one_call", False)
    norm = args.workload.startswith("rmsnorm_")
    silu = args.workload.startswith("silu_")
    base = args.workload[len("rmsnorm_"):] if norm else (
        {"silu_down_prefill": "down_prefill", "silu_decode_down": "decode_down"}[args.workload] if silu
        else args.workload)
    c = workloads.linear_case(base, m=args.m, alpha=args.alpha)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    to = lambda a, dt: torch.from_numpy(a).to(tdt[dt]).to(dev)
    w = to(c.w, c.w_dtype)
    nc = gu = None
    if silu:
        gu = workloads.gate_up_case(c.m, c.k, seed=0, calib_rows=c.x_calib.shape[0])
        gate, up = to(gu.gate, "bf16"), to(gu.up, "bf16")
        x = gate
        # calibration rows of the layer's input h = SiLU(gate) * up, by plain torch ops
        gc, uc = to(gu.gate_calib, "bf16").float(), to(gu.up_calib, "bf16").float()
        xc = (torch.nn.functional.silu(gc) * uc).to(torch.bfloat16)
        del gc, uc
    elif norm:
        nc = workloads.norm_case(c.m, c.k, seed=0, dtype=c.x_dtype, calib_rows=c.x_calib.shape[0])
        x, gamma = to(nc.x, c.x_dtype), to(nc.gamma, c.x_dtype)
        # calibration rows of the layer's input: the norm's output, by a plain torch RMSNorm
        r = to(nc.x_calib, c.x_dtype).float()
        xc = (r * torch.rsqrt(r.pow(2).mean(dim=1, keepdim=True) + args.eps) * gamma.float()).to(tdt[c.x_dtype])
        del r
    else:
        xc, x = to(c.x_calib, c.x_dtype), to(c.x, c.x_dtype)
    out_dt = tdt[c.y_dtype]
    print(f"[bench] workload {args.workload} M={c.m} K={c.k} N={c.n} alpha={c.alpha}", file=sys.stderr, flush=True)

    # ---- load-time steps (once, timed separately; torch's events on its current stream)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1, e2 = ev(), ev(), ev()
    absmax = torch.zeros(c.k, dtype=torch.float32, device=dev)
    e0.record()
    sq.sq_calibrate_absmax(xc, absmax)
    e1.record()
    s, wq, sw = sq.sq_smooth_fold_weights(w, c.alpha, absmax=absmax)
    e2.record()
    gain = sq.sq_fold_norm_gain(gamma, s) if norm else None
    torch.cuda.synchronize()
    prep = {"calibrate_ms": e0.elapsed_time(e1), "smooth_fold_ms": e1.elapsed_time(e2),
            "calib_rows": int(c.x_calib.shape[0])}

    xq = torch.empty((c.m, c.k), dtype=torch.int8, device=dev)
    dx = torch.empty(c.m, dtype=torch.float32, device=dev)
    y = torch.empty((c.m, c.n), dtype=out_dt, device=dev)
    ws = sq.linear_workspace(c.m, c.n, c.k, dev)
    decode = decode_kernel_runs(c.m, c.n, c.k)
    streamed = hbm_bound(c.m, c.n, c.k, {"f32": 4, "bf16": 2}[c.y_dtype])
    # Weight-streaming steps read the whole weight matrix once; with one copy
    # it would stay in the 256 MiB last-level cache between steps. Rotating
    # through copies totalling >= 768 MiB makes every step read it from HBM.
    n_w = -(-(768 << 20) // wq.numel()) if streamed else 1
    wqs = [wq] + [wq.clone() for _ in range(n_w - 1)]

    # The timed loop calls the C ABI directly with pre-marshalled arguments and
    # records HIP events on the launch stream, so that the host enqueues work
    # faster than the GPU drains it even for microsecond decode kernels (the
    # checked Python wrappers cost more per call than such a kernel runs).
    stream = torch.cuda.current_stream(dev).cuda_stream
    g_fn = sq.raw["sq_w8a8_linear"]
    _, _, ldx = sq._rows(x)
    if silu:
        q_fn = sq.raw["sq_silu_mul_quant"]
        q_args = (gate.data_ptr(), up.data_ptr(), sq.SQ_BF16, c.m, c.k, c.k, c.k, s.data_ptr(), xq.data_ptr(),
                  dx.data_ptr(), stream)
    elif norm:
        q_fn = sq.raw["sq_rmsnorm_quant"]
        q_args = (x.data_ptr(), sq._dt(x), c.m, c.k, ldx, gain.data_ptr(), float(args.eps), xq.data_ptr(),
                  dx.data_ptr(), stream)
    else:
        q_fn = sq.raw["sq_quant_act_per_token"]
        q_args = (x.data_ptr(), sq._dt(x), c.m, c.k, ldx, s.data_ptr(), xq.data_ptr(), dx.data_ptr(), stream)
    nb = ws.numel() if ws is not None else 0
    g_args = [(xq.data_ptr(), dx.data_ptr(), w_i.data_ptr(), sw.data_ptr(), c.m, c.n, c.k, y.data_ptr(),
               sq._dt(y), c.n, ws.data_ptr() if ws is not None else None, nb, stream) for w_i in wqs]
    hip = HipEvents(sq._lib, stream)
    dyn_fn = sq.raw["sq_w8a8_linear_dyn"]
    if one_call:
        if norm or silu:
            raise SystemExit("--one-call applies to the plain quantisation + GEMM path")
        dws = torch.zeros(sq.raw["sq_w8a8_linear_dyn_workspace_size"](c.m, c.n, c.k), dtype=torch.uint8, device=dev)
        d_args = [(x.data_ptr(), sq._dt(x), ldx, s.data_ptr(), w_i.data_ptr(), sw.data_ptr(), c.m, c.n, c.k,
                   y.data_ptr(), sq._dt(y), c.n, dws.data_ptr(), dws.numel(), stream) for w_i in wqs]

    def run(steps, evs=None):
        bad = 0
        for i in range(steps):
            if evs:
                hip.record(evs[i][0])
            if one_call:
                if evs:
                    hip.record(evs[i][1])
                bad |= dyn_fn(*d_args[i % n_w])
            else:
                bad |= q_fn(*q_args)
                if evs:
                    hip.record(evs[i][1])
                bad |= g_fn(*g_args[i % n_w])
            if evs:
                hip.record(evs[i][2])
        if bad:
            raise RuntimeError(f"a C-ABI call failed (status bits {bad})")

    run(args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps back to back, events only at its ends
    t_start, t_end = hip.create(), hip.create()
    torch.cuda.synchronize()
    hip.record(t_start)
    h0 = time.perf_counter()
    run(args.steps)
    host_us = (time.perf_counter() - h0) * 1e6 / args.steps
    hip.record(t_end)
    torch.cuda.synchronize()
    total_ms = hip.elapsed(t_start, t_end)
    # ---- the same steps again with events around each kernel (per-kernel
    # durations for the roofline; the markers add a little time of their own)
    evs = [[hip.create(), hip.create(), hip.create()] for _ in range(args.steps)]
    i_start, i_end = hip.create(), hip.create()
    hip.record(i_start)
    run(args.steps, evs)
    hip.record(i_end)
    torch.cuda.synchronize()
    instr_ms = hip.elapsed(i_start, i_end) / args.steps
    quant_ms = float(np.mean([hip.elapsed(e[0], e[1]) for e in evs]))
    gemm_ms = float(np.mean([hip.elapsed(e[1], e[2]) for e in evs]))
    # the GEMM (or the one call) alone, launches back to back
    b0, b1 = hip.create(), hip.create()
    hip.record(b0)
    for i in range(args.steps):
        if one_call:
            dyn_fn(*d_args[i % n_w])
        else:
            g_fn(*g_args[i % n_w])
    hip.record(b1)
    torch.cuda.synchronize()
    b2b_ms = hip.elapsed(b0, b1) / args.steps
    hip.destroy_all()

    ops = 2.0 * c.m * c.n * c.k
    ms_per_step = total_ms / args.steps
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    in_bytes = {"f32": 4, "bf16": 2}[c.x_dtype] * (2 if silu else 1)  # gate and up
    quant_bytes = c.m * c.k * in_bytes + 4 * c.k + c.m * c.k + 4 * c.m
    gemm_bytes = c.m * c.k + c.n * c.k + 4 * c.m + 4 * c.n + c.m * c.n * {"f32": 4, "bf16": 2}[c.y_dtype]
    big = big_kernel_suits(c.m, c.n, c.k)
    fused1 = one_call and decode_one_token_fused(c.m, c.n, c.k)
    kfile, kname = (("decode_fused.hip", "gemv_decode1_kernel") if fused1 else
                    ("gemm_decode.hip", "gemm_decode_ring_kernel" if decode_ring(c.m) else "gemm_decode_kernel")
                    if decode else
                    ("gemm_big.hip", "gemm_big_kernel") if big else ("gemm.hip", "gemm_i8_kernel"))
    tag = (args.workload if args.m is None else f"{args.workload}_m{c.m}") + (":one_call" if one_call else "")
    traffic = pmc_traffic(tag, kfile)
    if fused1:
        # one launch reads X, s, Wq and the scales and writes Y (Xq never reaches memory)
        gemm_bytes = c.m * c.k * in_bytes + 4 * c.k + c.n * c.k + 4 * c.n + c.m * c.n * {"f32": 4, "bf16": 2}[c.y_dtype]
    if streamed:
        roof = {"bound": "hbm", "achieved": gemm_bytes / (gemm_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "kernel": kname, "bytes_per_launch": gemm_bytes}
    else:
        roof = {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "kernel": kname, "ops_per_launch": ops}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["launch_us"] = gemm_ms * 1e3
    kernel_only(roof, tag, kfile, gemm_bytes if streamed else ops)
    pre = "norm_" if norm else ("silu_" if silu else "")
    norm_roof = None
    if norm or silu:
        ach = quant_bytes / (quant_ms * 1e-3) / 1e9
        norm_roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                     "traffic": pmc_traffic(tag + (":norm" if norm else ":silu"), "norm.hip" if norm else "silu.hip"),
                     "kernel": "rmsnorm_quant_kernel" if norm else "silu_quant_kernel",
                     "bytes_per_launch": quant_bytes, "launch_us": quant_ms * 1e3}

    result = {
        "metric": METRIC, "value": value, "unit": "TOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": (f"{args.workload}: residual stream {c.x_dtype} [{c.m} x {c.k}] -> RMSNorm "
                                f"(gain gamma/s, eps {args.eps:g}) -> W [{c.k} x {c.n}]" if norm else
                                f"{args.workload}: gate, up bf16 [{c.m} x {c.k}] -> SiLU(gate)*up -> "
                                f"W [{c.k} x {c.n}]" if silu else
                                f"{c.name}: X {c.x_dtype} [{c.m} x {c.k}] -> W [{c.k} x {c.n}]") +
                               f", {c.y_dtype} out, alpha {c.alpha}", "M": c.m, "K": c.k, "N": c.n,
                   "x_dtype": c.x_dtype, "y_dtype": c.y_dtype, "alpha": c.alpha},
        "pct_int8_peak": 100.0 * value / PEAK_INT8_TOPS,
        "gemm_only_tops": gemm_tops,
        "gemm_us": gemm_ms * 1e3,
        "gemm_us_back_to_back": b2b_ms * 1e3,
        "one_call": one_call,
        (pre + "quant_us"): None if one_call else quant_ms * 1e3,
        (pre + "quant_gbs"): None if one_call else quant_bytes / (quant_ms * 1e-3) / 1e9,
        (pre + "quant_frac_hbm"): None if one_call else quant_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "step_gbs_algorithmic": ((gemm_bytes if fused1 else quant_bytes + gemm_bytes) / (ms_per_step * 1e-3) / 1e9),
        "weight_copies": n_w,
        "host_enqueue_us_per_step": host_us,
        "ms_per_step_with_kernel_events": instr_ms,
        "load_time": prep,
        "roofline": roof,
    }
    if norm:
        result["norm_roofline"] = norm_roof
    if silu:
        result["silu_roofline"] = norm_roof
    if not args.no_cpu_baseline and silu:
        result["cpu_baseline"] = cpu_baseline_silu(c, gu, args.cpu_seconds)
    elif not args.no_cpu_baseline and norm:
        result["cpu_baseline"] = cpu_baseline_norm(c, nc, args.eps, args.cpu_seconds)
    elif not args.no_cpu_baseline:
        import oracle
        s_ref = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w),
                                         c.alpha)
        result["cpu_baseline"] = cpu_baseline(c, s_ref, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    return result


# Per-config records of the default run: the other configurations of the
# workload set (gate/up and down projections at 8192 tokens, alpha 0.5; the
# decode projections at 1, 8, 32 and 64 tokens; the LLM.int8() layer; the
# E4M3 variant of the QKV projection), each timed
# like the headline with fewer steps and a short oracle sample.
EXTRA_CONFIGS = [("gateup_prefill", None, 30), ("down_prefill", None, 40), ("decode_up", 1, 200),
                 ("decode_down", 1, 200), ("decode_up", 8, 200), ("decode_down", 8, 200), ("decode_up", 32, 200),
                 ("decode_down", 32, 200), ("decode_up", 64, 200), ("decode_down", 64, 200), ("llm_int8", None, 40),
                 ("fp8_qkv_prefill", None, 100)]


def config_records(args, dev) -> list:
    import copy
    recs = []
    for workload, m, steps in EXTRA_CONFIGS:
        a = copy.copy(args)
        a.workload, a.m, a.alpha, a.steps, a.warmup = workload, m, None, steps, max(3, steps // 10)
        a.cpu_seconds = min(args.cpu_seconds, 3.0)
        a.one_call = m == 1  # one token: the one-call entry point (the fused step where it applies)
        print(f"[bench] config record {workload} m={m}", file=sys.stderr, flush=True)
        r = (bench_llm_int8(a, dev) if workload == "llm_int8" else bench_fp8(a, dev) if workload.startswith("fp8_")
             else bench_linear(a, dev))
        keep = ("value", "unit", "ms_per_step", "steps", "config", "gemm_only_tops", "gemm_us", "quant_us",
                "gemm_us_back_to_back", "step_gbs_algorithmic", "detect_us", "outlier_columns", "weight_copies",
                "roofline", "cpu_baseline", "one_call")
        recs.append({k: r[k] for k in keep if k in r})
        import torch
        torch.cuda.empty_cache()
    return recs


def ingest_profile(args):
    """Record a rocprofv3 run of one workload in profiles/pmc_traffic.json:
    the named kernel's average duration from a --stats kernel_stats.csv, and,
    with --pmc-fetch / --pmc-write, its FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch) scaled by the copy-probe factors, keyed by workload and the
    kernel source file's hash (the bench ignores an entry once that file has
    changed)."""
    import csv

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    try:
        with open(PROFILE_PMC) as f:
            d = json.load(f)
    except (OSError, ValueError):
        d = {}
    e = dict(d.get(args.workload) or {})
    if e.get("source_sha256_16") != kernel_source_hash(args.kernel_file):
        e = {}
    e.update({"kernel_file": args.kernel_file, "source_sha256_16": kernel_source_hash(args.kernel_file)})
    if args.ingest_stats:
        hit = [r for r in rows(args.ingest_stats) if args.kernel_match in r["Name"]]
        if not hit:
            raise SystemExit(f"no kernel matching {args.kernel_match!r} in {args.ingest_stats}")
        r = max(hit, key=lambda r: int(r["Calls"]))
        e.update({"kernel": r["Name"], "kernel_us": float(r["AverageNs"]) / 1e3, "calls": int(r["Calls"])})
    for key, path, name in (("fetch_kib", args.pmc_fetch, "FETCH_SIZE"), ("write_kib", args.pmc_write, "WRITE_SIZE")):
        if not path:
            continue
        vals = [float(r["Counter_Value"]) for r in rows(path)
                if args.kernel_match in r["Kernel_Name"] and r["Counter_Name"] == name]
        if not vals:
            raise SystemExit(f"no {name} for {args.kernel_match!r} in {path}")
        e[key] = sorted(vals)[len(vals) // 2]
    if "fetch_kib" in e and "write_kib" in e:
        e.update({"fetch_scale": args.fetch_scale, "write_scale": args.write_scale,
                  "hbm_bytes_per_launch": 1024.0 * (e["fetch_kib"] * args.fetch_scale +
                                                    e["write_kib"] * args.write_scale)})
    d[args.workload] = e
    with open(PROFILE_PMC, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
    print(json.dumps({args.workload: e}))


def main():
    args = parse()
    if args.ingest_stats or args.pmc_fetch or args.pmc_write:
        ingest_profile(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the W8A8 linear layer is built and measured on a single "
              "MI355X (no sharding or collectives in this library); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    if args.probe:
        run_probe(args)
        return

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.workload == "llm_int8":
        result = bench_llm_int8(args, dev)
    elif args.workload.startswith("fp8_"):
        result = bench_fp8(args, dev)
    elif args.workload.startswith("gptq_"):
        result = bench_gptq(args, dev)
    else:
        args.one_call = args.one_call or False
        result = bench_linear(args, dev)
        if args.workload == "qkv_prefill" and args.m is None and not args.no_configs:
            result["configs"] = config_records(args, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
