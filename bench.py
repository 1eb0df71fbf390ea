#!/usr/bin/env python3
"""Benchmark of the fused-epilogue GEMM suite on one MI355X.

One step = one fused execution of every workload of the suite, in order:
  C0  BIAS          W[1024,2048] X[2048,512] + b[1024]
  C1  GELU_BIAS     decode x[T,4096] W[4096,4096]^T, T = 1, 4, 16
                    (weights rotated over 16 copies, 512 MiB, so every read is
                    cold in L2 and in the 256 MB Infinity Cache)
  C2  FFN           x[tok,4096] -> GELU_BIAS(W1 [11008,4096]) -> BIAS(W2 [4096,11008]),
                    tok = 512, 2048, 4x512, 16x128
  C3  RELU_AUX_BIAS A[65536,16384] B[16384,8192] + bias[65536] + mask, fp16 and bf16
  C4  DRELU_BGRAD   dY[8192,16384] W[16384,4096], mask, bgrad[4096]
value = algorithmic FLOPs of one step (2MNK per GEMM) / step time, in TFLOP/s.

Also printed in the same JSON line: per-workload fused and unfused time,
TFLOP/s or GB/s, fraction of the roofline and fusion speedup; the roofline
of the dominant kernel (the C3 fp16 GEMM: the mean of its launches in the
timed steps, each bracketed by HIP events on the stream it is launched on);
and the CPU oracle timed on a bounded sample on this host.  Inputs are seeded synthetic data already resident in HBM.

Timed beside the step but outside it ("in_step": false):
  C5  GEMM + bias + residual + LayerNorm / RMSNorm, x[2048,11008] W[4096,11008]^T
  C6  DGELU_BGRAD   C4's shape with a saved z[8192,4096] in place of the mask
  C7  GELU_AUX_BIAS C3's fp16 shape, writing gelu(z) and z
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2516.6     # MI355X dense fp16/bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_GBS = 8000.0        # MI355X HBM3E
DECODE_COPIES = 16
FFN_COPIES = 3           # 3 x (W1 + W2) = 516 MiB, beyond the 256 MB Infinity Cache


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--reps", type=int, default=0, help="reps per workload timing (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of workloads (suite c0..c4, extras c5..c7)")
    ap.add_argument("--profile-traffic", action="store_true",
                    help="only run a plain 1 GiB copy (calibration) and the C3 fp16 fused kernel "
                         "twice each, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--compare-blas", action="store_true",
                    help="instead of the step: time the fused call, the library's plain GEMM "
                         "(epilogue DEFAULT) and torch.matmul (ROCm's BLAS) on the suite's GEMM "
                         "shapes, interleaved; one JSON line per shape")
    ap.add_argument("--profile-layouts", action="store_true",
                    help="only run the C3 fp16 fused kernel twice with B stored [K,N] (as the "
                         "workload) and twice with the same B stored [N,K], for rocprofv3 --pmc runs")
    ap.add_argument("--profile-workloads", action="store_true",
                    help="only run the 1 GiB copy (calibration) and two fused executions of each "
                         "selected workload (--only, default c0,c2,c4), one after another, for "
                         "rocprofv3 --pmc runs of the tiles other than C3's")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the MFMA loop of the 256x256 tile with no memory traffic "
                         "(fp16 and bf16, normal and zero operands) and print one JSON line each")
    ap.add_argument("--profile-decode", action="store_true",
                    help="only run the 1 GiB copy (calibration) and 16 decode calls each at "
                         "T = 1 and T = 16 over 16 rotated weight copies, for rocprofv3 --pmc runs")
    return ap.parse_args()


MEASURE_LIB = os.path.join(ROOT, "activation_epilogue_gemm_amd", "libgemmepi_measure.so")
_measure = None


def measure_library():
    """libgemmepi_measure (the stream-read reference), built beside libgemmepi."""
    global _measure
    if _measure is None:
        import ctypes
        if not os.path.exists(MEASURE_LIB):
            raise RuntimeError(f"{MEASURE_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(MEASURE_LIB)
        vp = ctypes.c_void_p
        lib.gemmepi_measure_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_int, vp]
        lib.gemmepi_measure_stream_read.restype = ctypes.c_int
        lib.gemmepi_measure_mfma_loop.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, vp]
        lib.gemmepi_measure_mfma_loop.restype = ctypes.c_int
        _measure = lib
    return _measure


def stream_read(buf, nbytes, sink, threads=512, loads=16, nontemporal=0):
    """One 128-bit streaming read of the first `nbytes` bytes of `buf`
    (a device tensor) on torch's current stream."""
    import torch
    st = measure_library().gemmepi_measure_stream_read(
        buf.data_ptr(), int(nbytes), sink.data_ptr(), int(threads), int(loads), int(nontemporal),
        torch.cuda.current_stream(buf.device).cuda_stream)
    if st != 0:
        raise RuntimeError(f"gemmepi_measure_stream_read failed with status {st}")


MFMA_LOOP_WAVES, MFMA_LOOP_FRAGS = 8, 12   # per workgroup; 16-byte fragments per wave
MFMA_LOOP_FLOP = 32 * 16384                # one round of a wave: 32 MFMAs 16x16x32


def mfma_loop(src, sink, blocks, rounds, bf16):
    """One launch of the MFMA loop of the measurement library on torch's
    current stream (src: the 8 waves' operand fragments, >= 96 KiB)."""
    import torch
    st = measure_library().gemmepi_measure_mfma_loop(
        src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), int(blocks), int(rounds),
        int(bf16), torch.cuda.current_stream(src.device).cuda_stream)
    if st != 0:
        raise RuntimeError(f"gemmepi_measure_mfma_loop failed with status {st}")


def mfma_loop_rate(dt="f16", kind="normal", trials=5, launches=5, rounds=40000):
    """TFLOP/s of the MFMA loop of the 256x256 tile with no memory traffic
    (one workgroup per CU), on standard-normal or zero operands: the median
    (and minimum time) of `trials` trials of `launches` launches of ~20 ms,
    timed with HIP events on torch's current stream."""
    import statistics
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = MFMA_LOOP_WAVES * MFMA_LOOP_FRAGS * 64 * 8        # 8 halves per 16-byte fragment
    sink = torch.zeros(1024, dtype=torch.float32, device="cuda")
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    bf = 0 if dt == "f16" else 1
    g = torch.Generator(device="cuda").manual_seed(7)
    src = (torch.randn(n, device="cuda", generator=g) if kind == "normal"
           else torch.zeros(n, device="cuda")).to(tdt)
    flops = cus * MFMA_LOOP_WAVES * rounds * MFMA_LOOP_FLOP
    mfma_loop(src, sink, cus, 100, bf)                     # warm-up
    torch.cuda.synchronize()
    ms = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            mfma_loop(src, sink, cus, rounds, bf)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1) / launches)
    med = statistics.median(ms)
    return {"mfma_loop": dt, "operands": kind, "workgroups": cus, "rounds": rounds,
            "ms_median": round(med, 4), "ms_min": round(min(ms), 4),
            "tflops": round(flops / med / 1e9, 1),
            "frac_of_published": round(flops / med / 1e9 / PEAK_TFLOPS, 4)}


def mfma_ceiling():
    """The matrix cores alone at the power limit: the 256x256 tile's MFMA
    work (8 waves of 128x64 accumulators per CU) with no memory traffic, on
    standard-normal and on zero operands, fp16 and bf16, one JSON line each."""
    for dt in ("f16", "bf16"):
        for kind in ("normal", "zero"):
            rec = mfma_loop_rate(dt, kind)
            print(json.dumps(rec), flush=True)
            log(f"mfma loop {dt} {kind}: {rec['tflops']} TFLOP/s")


# launch shapes of the stream-read sweep: (threads, loads per thread, non-temporal)
STREAM_SHAPES = [(t, l, nt) for t in (256, 512, 1024) for l in (4, 8, 16, 32) for nt in (0, 1)]


def sweep_stream_read(bufs, nbytes, reps, stream, shapes=None):
    """Time every launch shape of the stream read over the rotated buffers
    (each read cold from HBM); returns {shape: ms per read}, medians of 5
    trials."""
    import statistics
    import torch
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    res = {}
    for shp in shapes or STREAM_SHAPES:
        t, l, nt = shp
        fn = lambda i: stream_read(bufs[i % len(bufs)], nbytes, sink, t, l, nt)  # noqa: E731
        for i in range(2):
            fn(i)
        res[shp] = statistics.median(time_region(fn, reps, stream) for _ in range(5))
    return res


def torch_dtype(dtype):
    import torch
    return torch.float16 if dtype == "f16" else torch.bfloat16


def upload_bits(bits, dtype, device):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch_dtype(dtype))


def upload_words(words, device):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(device)


class Workload:
    """Device buffers + fused and unfused plans of one GEMM call."""

    def __init__(self, name, case, flags=0, A_dev=None, B_dev=None, out=None):
        import torch
        import activation_epilogue_gemm_amd as ge
        self.name = name
        self.case = case
        c = case
        dev = "cuda"
        tdt = torch_dtype(c.dtype)
        self.A = A_dev if A_dev is not None else (
            c.A_dev if getattr(c, "A_dev", None) is not None else upload_bits(c.A, c.dtype, dev))
        self.B = B_dev if B_dev is not None else (
            c.B_dev if getattr(c, "B_dev", None) is not None else upload_bits(c.B, c.dtype, dev))
        self.out = out if out is not None else torch.empty(c.M, c.N, dtype=tdt, device=dev)
        self.bias = self.aux = None
        if c.epilogue in ("DRELU_BGRAD", "DGELU_BGRAD"):
            self.bias = torch.empty(c.N, dtype=torch.float32, device=dev)
            self.aux = (upload_words(c.aux, dev) if c.epilogue == "DRELU_BGRAD"
                        else upload_bits(c.aux, c.dtype, dev))
        else:
            if c.bias is not None:
                self.bias = upload_bits(c.bias, c.dtype, dev)
            if c.epilogue == "RELU_AUX_BIAS":
                self.aux = torch.empty(c.M, ge.aux_ld_words(c.N), dtype=torch.int32, device=dev)
            if c.epilogue == "GELU_AUX_BIAS":
                self.aux = torch.empty(c.M, c.N, dtype=tdt, device=dev)
        # FLAG_SPLIT_K: plan() may split K for the wave-quantised shapes (C0,
        # the 512-token down-projection); its workspace is allocated by the
        # plan at the first (warm-up) execution
        # FLAG_STAGE_B: plan() may copy a [K,N] B to [N,K] in the workspace
        # first (it does for the two large workloads, C3 and C4)
        f = flags | ge.FLAG_SPLIT_K | ge.FLAG_STAGE_B | (ge.FLAG_B_TRANS if c.b_trans else 0) | \
            (ge.FLAG_BIAS_PER_COL if c.bias_per_col else 0)
        self.fused = ge.plan(c.M, c.N, c.K, c.dtype, c.epilogue, f)
        self.unfused = ge.plan(c.M, c.N, c.K, c.dtype, c.epilogue, f | ge.FLAG_UNFUSED)
        self.flops = 2.0 * c.M * c.N * c.K
        # algorithmic bytes: each operand, bias, output, aux and bgrad moved once
        esz = 2
        self.bytes = esz * (c.M * c.K + c.N * c.K + c.M * c.N)
        if self.bias is not None:
            self.bytes += self.bias.numel() * self.bias.element_size()
        if self.aux is not None:
            self.bytes += self.aux.numel() * self.aux.element_size()
        self.rotation = None  # list of (A, B, out) for cache-cold timing of small workloads

    def run(self, unfused=False, i=0):
        p = self.unfused if unfused else self.fused
        if self.rotation:
            A, B, out = self.rotation[i % len(self.rotation)]
        else:
            A, B, out = self.A, self.B, self.out
        p.execute(A, B, self.bias, self.aux, out, check=False)


class NormWorkload:
    """Device buffers and plans of the GEMM + bias + residual + norm operator
    (structural fusion); same interface as Workload."""

    def __init__(self, name, case):
        import torch
        import activation_epilogue_gemm_amd as ge
        self.name = name
        c = self.case = case
        up = lambda x: None if x is None else upload_bits(x, c.dtype, "cuda")  # noqa: E731
        self.A, self.B = up(c.A), up(c.B)
        self.bias, self.res, self.gamma, self.beta = up(c.bias), up(c.residual), up(c.gamma), up(c.beta)
        self.out = torch.empty(c.M, c.N, dtype=torch_dtype(c.dtype), device="cuda")
        self.stats = ge.norm_stats_buffer(c.M)
        f = ge.FLAG_B_TRANS if c.b_trans else 0
        epi = "BIAS_RES_" + c.norm
        self.fused = ge.plan(c.M, c.N, c.K, c.dtype, epi, f)
        self.unfused = ge.plan(c.M, c.N, c.K, c.dtype, epi, f | ge.FLAG_UNFUSED)
        # the two-kernel form (GEMM writes y, a second kernel normalises), for
        # comparison with the single pass that `fused` runs
        self.two_pass = ge.plan(c.M, c.N, c.K, c.dtype, epi, f | ge.FLAG_NORM_TWO_PASS)
        self.flops = 2.0 * c.M * c.N * c.K
        # operands, residual, gamma/beta/bias, output and stats moved once
        self.bytes = 2 * (c.M * c.K + c.N * c.K + 2 * c.M * c.N + 3 * c.N) + 16 * c.M
        self.rotation = None

    def run(self, unfused=False, i=0, two_pass=False):
        p = self.unfused if unfused else (self.two_pass if two_pass else self.fused)
        p.execute_norm(self.A, self.B, self.bias, self.res, self.gamma, self.beta, self.case.eps,
                       self.stats, self.out, check=False)


def build_extras(only):
    """Workloads of the 'next' rows, timed and reported beside the suite but
    not part of its step: GEMM + bias + residual + LayerNorm / RMSNorm at the
    2048-token FFN down-projection shape (c5); the GELU backward at the ReLU
    backward's shape (c6); the GELU forward that saves z at the ReLU-aux
    forward's shape (c7)."""
    import workloads as wl
    sel = set(only.split(",")) if only else {"c5", "c6", "c7"}
    extras = []
    if "c5" in sel:
        for norm in ("LAYERNORM", "RMSNORM"):
            extras.append(NormWorkload(f"c5_ffn_down_res_{norm.lower()}",
                                       wl.config5_ffn_down_norm(norm)))
    if "c6" in sel:
        extras.append(Workload("c6_dgelu_bgrad", wl.config4_dgelu_bgrad()))
    if "c7" in sel:
        extras.append(Workload("c7_gelu_aux_f16", wl.config3_gelu_aux("f16")))
    return extras


def build_suite(only):
    import torch
    import workloads as wl
    sel = set(only.split(",")) if only else {"c0", "c1", "c2", "c3", "c4"}
    sel &= {"c0", "c1", "c2", "c3", "c4"}
    suite = []
    t0 = time.time()
    if "c0" in sel:
        w = Workload("c0_bias", wl.config0_bias())
        add_rotation(w, max_copies=80)  # 7 MiB per copy
        suite.append(w)
    if "c1" in sel:
        for T in (1, 4, 16):
            w = Workload(f"c1_decode_T{T}", wl.config1_decode(T))
            w.rotation = [(w.A, w.B.clone(), torch.empty_like(w.out)) for _ in range(DECODE_COPIES)]
            suite.append(w)
    if "c2" in sel:
        # FFN_COPIES copies of both weights (172 MiB each), shared by all token
        # variants; copy i of the up-projection writes the h that copy i of the
        # down-projection reads, so the chain stays a chain in every step
        W1s = W2s = None
        for v in wl.FFN_TOKENS:
            up, down = wl.config2_ffn(v)
            wu = Workload(f"c2_{v}_up", up, B_dev=W1s[0] if W1s else None)
            wd = Workload(f"c2_{v}_down", down, A_dev=wu.out, B_dev=W2s[0] if W2s else None)
            if W1s is None:
                W1s = [wu.B] + [wu.B.clone() for _ in range(FFN_COPIES - 1)]
                W2s = [wd.B] + [wd.B.clone() for _ in range(FFN_COPIES - 1)]
            xs = [wu.A] + [wu.A.clone() for _ in range(FFN_COPIES - 1)]
            hs = [wu.out] + [torch.empty_like(wu.out) for _ in range(FFN_COPIES - 1)]
            ys = [wd.out] + [torch.empty_like(wd.out) for _ in range(FFN_COPIES - 1)]
            wu.rotation = [(xs[i], W1s[i], hs[i]) for i in range(FFN_COPIES)]
            wd.rotation = [(hs[i], W2s[i], ys[i]) for i in range(FFN_COPIES)]
            suite += [wu, wd]
    if "c3" in sel:
        for dt in ("f16", "bf16"):
            suite.append(Workload(f"c3_relu_aux_{dt}", wl.config3_relu_aux(dt)))
    if "c4" in sel:
        suite.append(Workload("c4_drelu_bgrad", wl.config4_drelu_bgrad()))
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s; device memory "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB")
    return suite


def time_region(fn, reps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(reps):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps  # ms


TRIALS = 5


def bench_workload(w, reps, stream):
    """Median and minimum of TRIALS trials of `reps` back-to-back executions,
    fused and unfused."""
    import statistics
    res = {}
    for label, unf in (("fused", False), ("unfused", True)):
        for i in range(2):
            w.run(unf, i)
        trials = [time_region(lambda i: w.run(unf, i), reps, stream) for _ in range(TRIALS)]
        res[label] = statistics.median(trials)
        res[label + "_min"] = min(trials)
    return res


def reps_for(ms_per_call):
    """Executions per timing trial: at least 200 ms of work, or at least 20
    executions (and at most 400)."""
    import math
    return int(min(400, max(20, math.ceil(200.0 / max(ms_per_call, 1e-4)))))


ROTATE_BYTES = 512 << 20  # distinct operand bytes cycled through per small workload


def add_rotation(w, max_copies=16):
    """Cycle a small workload through enough copies of its operands (at least
    512 MiB together, at most `max_copies`) that each execution reads them
    from HBM, not from the 256 MB Infinity Cache or the XCDs' L2s."""
    import math
    import torch
    per = w.A.numel() * 2 + w.B.numel() * 2 + w.out.numel() * 2
    n = int(min(max_copies, max(2, math.ceil(ROTATE_BYTES / per))))
    w.rotation = [(w.A.clone(), w.B.clone(), torch.empty_like(w.out)) for _ in range(n)]
    return n


def _blas_info(cores):
    """The BLAS library numpy's fp64 matmul runs on, and its thread count."""
    try:
        import threadpoolctl
        for i in threadpoolctl.threadpool_info():
            if i.get("user_api") == "blas":
                return {"library": f"{i.get('internal_api')} {i.get('version')}",
                        "file": os.path.basename(i.get("filepath", "")),
                        "threads": int(i.get("num_threads", cores))}
    except Exception:
        pass
    return {"library": "unknown", "file": "", "threads": cores}


def _oracle_times(wl, O):
    """The oracle on each workload's own parity sample, timed once: C0, the
    T = 16 decode and the 512-token FFN up-projection in full, C3 (fp16) on
    4096 seed-chosen rows, C4 with the full G that bgrad needs."""
    out = {}

    def timed(name, flops, fn):
        t = time.perf_counter()
        fn()
        dt = time.perf_counter() - t
        out[name] = {"s": round(dt, 3), "tflops_fp64": round(flops / dt / 1e12, 3)}

    c = wl.config0_bias()
    timed("c0_bias", 2.0 * c.M * c.N * c.K, lambda: O.gemm_epilogue(
        c.A, c.B, c.bias, None, c.M, c.N, c.K, c.dtype, c.epilogue, False, False))
    c = wl.config1_decode(16)
    timed("c1_decode_T16", 2.0 * c.M * c.N * c.K, lambda: O.gemm_epilogue(
        c.A, c.B, c.bias, None, c.M, c.N, c.K, c.dtype, c.epilogue, True, True))
    up, _ = wl.config2_ffn("b1s512")
    timed("c2_b1s512_up", 2.0 * up.M * up.N * up.K, lambda: O.gemm_epilogue(
        up.A, up.B, up.bias, None, up.M, up.N, up.K, up.dtype, up.epilogue, True, True))
    c = wl.config3_relu_aux("f16")
    rows = wl.sample_rows(c.M, 4096, wl.row_sample_seed(3))
    A, B = c.host_A(rows), c.host_B()
    timed("c3_relu_aux_f16_4096_rows", 2.0 * len(rows) * c.N * c.K, lambda: O.gemm_epilogue(
        A, B, c.bias[rows], None, len(rows), c.N, c.K, "f16", "RELU_AUX_BIAS", False, False))
    del c, A, B
    c = wl.config4_drelu_bgrad()
    A, B = c.host_A(), c.host_B()
    timed("c4_drelu_bgrad_full_G", 2.0 * c.M * c.N * c.K, lambda: O.gemm_epilogue(
        A, B, None, c.aux, c.M, c.N, c.K, c.dtype, c.epilogue, False, False,
        rows=wl.sample_rows(c.M, 4096, wl.row_sample_seed(4))))
    del c, A, B
    return out


def cpu_baseline(seconds_target=12.0):
    """The oracle, as it stands, on a bounded sample of the C3 workload
    (fp16): seed-chosen output rows against the full B, sized to about
    `seconds_target` seconds of host work; with its BLAS threads pinned to
    the host cores this process may use.  Also the oracle's time on each
    workload's own parity sample."""
    import torch
    import workloads as wl
    from oracle import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        limiter = threadpoolctl.threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limiter = None
    try:
        c = wl.config3_relu_aux("f16")
        B = c.host_B()
        rows_all = wl.sample_rows(c.M, 32768, wl.row_sample_seed(3))

        # calibrate: a small warm-up call (thread pools, page faults), then a
        # 4096-row probe; size the timed sample to ~seconds_target from the probe
        def run(rs):
            A_rs = c.host_A(rs)
            t = time.perf_counter()
            O.gemm_epilogue(A_rs, B, c.bias[rs], None, len(rs), c.N, c.K, "f16",
                            "RELU_AUX_BIAS", False, False)
            return time.perf_counter() - t
        run(rows_all[:32])
        # fp64 matmul throughput still rises with the row count at this size,
        # so the probe is large (about a second) and the estimate conservative
        probe = 4096
        dt = run(rows_all[:probe])
        nrows = int(max(probe, min(len(rows_all), probe * seconds_target / max(dt, 1e-3))))
        rows = rows_all[:nrows]
        A_rows = c.host_A(rows)
        t = time.perf_counter()
        O.gemm_epilogue(A_rows, B, c.bias[rows], None, len(rows), c.N, c.K, "f16",
                        "RELU_AUX_BIAS", False, False)
        dt = time.perf_counter() - t
        del c, A_rows, B
        torch.cuda.empty_cache()
        per_config = _oracle_times(wl, O)
        blas = _blas_info(cores)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    flops = 2.0 * len(rows) * 8192 * 16384
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas["threads"]),
            "kind": "oracle", "host_cores": cores, "blas": blas, "per_config": per_config,
            "sample": f"C3 fp16 RELU_AUX_BIAS, {len(rows)} sampled rows of 65536 "
                      f"(x 8192 cols, K=16384; fp64 numpy matmul, {blas['library']}, "
                      f"{blas['threads']} threads), {dt:.1f} s, host cores {cores}"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c3_relu_aux_f16.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_c3_relu_aux_f16.json")
KERNEL_SOURCES = ["activation_epilogue_gemm_amd/csrc/gemm_mfma.hpp",
                  "activation_epilogue_gemm_amd/csrc/gemm_tiles.h",
                  "activation_epilogue_gemm_amd/csrc/gemmepi_api.cpp"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE measurement, scaled by the copy-kernel
    calibration; None when the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def measured_counters() -> dict:
    """MFMA busy share and LDS bank-conflict share of the dominant kernel from
    the committed rocprofv3 counter runs; empty when the kernel sources
    changed since."""
    try:
        with open(COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    return t if t.get("kernel_source_sha") == kernel_source_hash() else {}


def profile_traffic():
    import torch
    import activation_epilogue_gemm_amd as ge
    import workloads as wl
    n = 1 << 29  # 1 GiB of fp16
    src = torch.empty(n, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)          # calibration: reads 1 GiB, writes 1 GiB
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    w = Workload("c3_relu_aux_f16", wl.config3_relu_aux("f16"))
    torch.cuda.synchronize()
    for i in range(2):
        w.run(False, i)
    torch.cuda.synchronize()
    log(f"profile-traffic done: {w.fused.info()}")


def profile_layouts():
    """C3's fp16 operands through the fused RELU_AUX_BIAS call, B as stored
    by the workload ([K,N]) and the same B transposed to [N,K] (B_TRANS), two
    launches each: the two B layouts of the same product side by side."""
    import torch
    import activation_epilogue_gemm_amd as ge
    import workloads as wl
    c = wl.config3_relu_aux("f16")
    M, N, K = c.M, c.N, c.K
    bias = upload_bits(c.bias, c.dtype, "cuda")
    out = torch.empty(M, N, dtype=torch.float16, device="cuda")
    aux = torch.empty(M, ge.aux_ld_words(N), dtype=torch.int32, device="cuda")
    for bt in (False, True):
        B = c.B_dev.t().contiguous() if bt else c.B_dev
        with ge.plan(M, N, K, "f16", "RELU_AUX_BIAS", ge.FLAG_B_TRANS if bt else 0) as p:
            for _ in range(2):
                p.execute(c.A_dev, B, bias, aux, out)
            torch.cuda.synchronize()
            log(f"profile-layouts B {'[N,K]' if bt else '[K,N]'} done: {p.info()}")
        del B
        torch.cuda.empty_cache()


def profile_decode():
    import torch
    import workloads as wl
    n = 1 << 29
    src = torch.empty(n, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    for T in (1, 16):
        w = Workload(f"c1_decode_T{T}", wl.config1_decode(T))
        w.rotation = [(w.A, w.B.clone(), torch.empty_like(w.out)) for _ in range(DECODE_COPIES)]
        torch.cuda.synchronize()
        for i in range(DECODE_COPIES):
            w.run(False, i)
        torch.cuda.synchronize()
        log(f"profile-decode T={T} done: {w.fused.info()}")
        del w
        torch.cuda.empty_cache()


def profile_workloads(only):
    """The 1 GiB copy (the FETCH/WRITE calibration), then two fused executions
    of each selected suite workload in turn (rotated copies as in the
    timing), each workload's plan printed first."""
    import torch
    n = 1 << 29
    src = torch.empty(n, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    suite = build_suite(only or "c0,c2,c4")
    for w in suite:
        log(f"profile-workloads {w.name}: {w.fused.info()}")
        for i in range(2):
            w.run(False, i)
        torch.cuda.synchronize()


def compare_blas(only, trials=5):
    """Context for the roofline figures: the vendor BLAS on the same shapes.

    Per GEMM shape of the suite (plus C3 with B stored [N, K], the layout in
    which both operands are K-contiguous): the fused call, the library's plain
    GEMM (epilogue DEFAULT: the rounded product, no bias) and torch.matmul on
    the same device buffers (hipBLASLt on ROCm; a plain GEMM, no epilogue),
    timed interleaved so that all three see the same clock.  Each figure is
    the median of `trials` timings of back-to-back calls."""
    import statistics
    import torch
    import activation_epilogue_gemm_amd as ge
    import workloads as wl
    sel = set(only.split(",")) if only else {"c0", "c2", "c3", "c4"}
    def ffn(v, which):
        up, down = wl.config2_ffn(v)
        wu = Workload(f"c2_{v}_up", up)
        if which == "up":
            return wu
        wu.run(False)  # the down-projection reads the up-projection's output
        return Workload(f"c2_{v}_down", down, A_dev=wu.out)

    specs = []  # (name, workload builder, store B as [N, K])
    if "c0" in sel:
        specs.append(("c0_bias", lambda: Workload("c0_bias", wl.config0_bias()), False))
    if "c2" in sel:
        for v in ("b1s2048", "b1s512"):
            for which in ("up", "down"):
                specs.append((f"c2_{v}_{which}", lambda v=v, which=which: ffn(v, which), False))
    if "c3" in sel:
        for dt in ("f16", "bf16"):
            specs.append((f"c3_relu_aux_{dt}",
                          lambda dt=dt: Workload("c3", wl.config3_relu_aux(dt)), False))
        specs.append(("c3_relu_aux_f16_BNK",
                      lambda: Workload("c3", wl.config3_relu_aux("f16")), True))
    if "c4" in sel:
        specs.append(("c4_drelu_bgrad", lambda: Workload("c4", wl.config4_drelu_bgrad()), False))
    stream = torch.cuda.current_stream()
    for name, make, transpose_b in specs:
        w = make()
        c = w.case
        B, b_trans = w.B, c.b_trans
        if transpose_b:  # the same product with B stored [N, K]
            B, b_trans = w.B.t().contiguous(), True
            flags = ge.FLAG_SPLIT_K | ge.FLAG_B_TRANS | (ge.FLAG_BIAS_PER_COL if c.bias_per_col else 0)
            w.fused = ge.plan(c.M, c.N, c.K, c.dtype, c.epilogue, flags)
            w.B = B
        # the plain GEMM takes the fused plan's path (split, staged B) with
        # the DEFAULT epilogue
        f = ge.FLAG_SPLIT_K | ge.FLAG_STAGE_B | (ge.FLAG_B_TRANS if b_trans else 0)
        plain = ge.plan(c.M, c.N, c.K, c.dtype, "DEFAULT", f)
        scratch = torch.empty_like(w.out)
        Bop = B.t() if b_trans else B
        fns = {
            "fused": lambda i: w.run(False, i),
            "plain": lambda i: plain.execute(w.A, B, None, None, scratch, check=False),
            "blas": lambda i: torch.matmul(w.A, Bop, out=scratch),
        }
        reps = max(3, min(200, int(2.0e12 / w.flops * 5)))
        for fn in fns.values():
            for i in range(2):
                fn(i)
        torch.cuda.synchronize()
        res = {k: [] for k in fns}
        for _ in range(trials):
            for k, fn in fns.items():
                res[k].append(time_region(fn, reps, stream))
        med = {k: statistics.median(v) for k, v in res.items()}
        rec = {"compare": name, "M": c.M, "N": c.N, "K": c.K, "dtype": c.dtype,
               "b_layout": "[N,K]" if b_trans else "[K,N]", "epilogue": c.epilogue,
               "plan": w.fused.info(), "plain_plan": plain.info()}
        for k, ms in med.items():
            rec[f"{k}_ms"] = round(ms, 5)
            rec[f"{k}_tflops"] = round(w.flops / ms / 1e9, 1)
        rec["plain_vs_blas"] = round(med["blas"] / med["plain"], 3)
        rec["fused_vs_blas"] = round(med["blas"] / med["fused"], 3)
        print(json.dumps(rec), flush=True)
        log(f"{name}: fused {rec['fused_tflops']} plain {rec['plain_tflops']} "
            f"blas {rec['blas_tflops']} TFLOP/s")
        del w, plain, scratch, B, Bop, fns
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.compare_blas:
        import torch
        import activation_epilogue_gemm_amd as ge
        ge.library()
        torch.cuda.set_device(0)
        compare_blas(args.only)
        return
    if args.mfma_ceiling:
        import torch
        torch.cuda.set_device(0)
        mfma_ceiling()
        return
    if args.profile_traffic or args.profile_decode or args.profile_layouts or args.profile_workloads:
        import torch  # noqa: F401
        import activation_epilogue_gemm_amd as ge
        ge.library()
        if args.profile_traffic:
            profile_traffic()
        elif args.profile_layouts:
            profile_layouts()
        elif args.profile_workloads:
            profile_workloads(args.only)
        else:
            profile_decode()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the fused GEMM shards by output tiles; this benchmark measures one GPU's share)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import activation_epilogue_gemm_amd as ge
    ge.library()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs {props.multi_processor_count}")

    suite = build_suite(args.only)
    extras = build_extras(args.only)
    if not suite:  # --only selected extras alone: they form the step
        suite, extras = extras, []
    for w in suite + extras:
        log(f"{w.name}: {w.fused.info()}")

    # the dominant kernel, the C3 fp16 fused GEMM: each of its launches in the
    # timed steps is bracketed by HIP events on the stream it runs on
    dom = next((w for w in suite if w.name == "c3_relu_aux_f16"), None) or \
        max(suite, key=lambda w: w.flops)
    dom_events = []

    def step(i, timed=False):
        for w in suite:
            if timed and w is dom:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                w.run(False, i)
                e1.record(stream)
                dom_events.append((e0, e1))
            else:
                w.run(False, i)

    # warmup + timed steps (the whole suite, fused)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i, timed=True)
    end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    step_flops = sum(w.flops for w in suite)
    log(f"step {ms_step:.3f} ms (wall {1e3 * wall / args.steps:.3f} ms), "
        f"{step_flops / ms_step / 1e9:.1f} TFLOP/s")

    # per-workload fused / unfused timing
    per = {}
    stream_ref = None
    for w in suite + extras:
        reps = args.reps
        if not reps:
            t = time_region(lambda i: w.run(False, i), 3, stream)
            reps = reps_for(t)
        r = bench_workload(w, reps, stream)
        f_ms, u_ms = r["fused"], r["unfused"]
        entry = {"fused_ms": round(f_ms, 5), "unfused_ms": round(u_ms, 5),
                 "fused_min_ms": round(r["fused_min"], 5), "unfused_min_ms": round(r["unfused_min"], 5),
                 "trials": TRIALS, "rotated_copies": len(w.rotation) if w.rotation else 1,
                 "speedup": round(u_ms / f_ms, 4), "reps": reps,
                 "tflops": round(w.flops / f_ms / 1e9, 2),
                 "frac_mfma_peak": round(w.flops / f_ms / 1e9 / PEAK_TFLOPS, 4),
                 "plan": w.fused.info()}
        if w in extras:
            entry.update({"in_step": False, "gbs_algorithmic": round(w.bytes / f_ms / 1e6, 1)})
        if isinstance(w, NormWorkload):
            import statistics
            w.run(False, 0)
            torch.cuda.synchronize()
            single = ge.norm_pass_status(w.stats, w.case.M) == 1
            for i in range(2):
                w.run(False, i, two_pass=True)
            trials = [time_region(lambda i: w.run(False, i, two_pass=True), reps, stream)
                      for _ in range(TRIALS)]
            t_ms = statistics.median(trials)
            entry.update({"two_pass_ms": round(t_ms, 5), "two_pass_min_ms": round(min(trials), 5),
                          "speedup_vs_two_pass": round(t_ms / f_ms, 4),
                          "single_pass": single})
        if w.name.startswith("c1_"):
            gbs = w.bytes / f_ms / 1e6
            # the practical floor: the fastest launch shape of a plain 128-bit
            # read of the same weight bytes, rotated over the same copies
            wb = w.B.numel() * 2
            if stream_ref is None:
                sweep = sweep_stream_read([r[1] for r in w.rotation], wb, reps, stream)
                best = min(sweep, key=sweep.get)
                stream_ref = {"ms": sweep[best], "shape": best,
                              "sweep_gbs": {f"{t}x{l}{'nt' if nt else ''}": round(wb / v / 1e6, 1)
                                            for (t, l, nt), v in sweep.items()}}
                log(f"stream-read sweep over {wb} bytes: best {best} "
                    f"{wb / stream_ref['ms'] / 1e6:.1f} GB/s; {stream_ref['sweep_gbs']}")
            s_ms = stream_ref["ms"]
            t, l, nt = stream_ref["shape"]
            entry.update({"gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_GBS, 4),
                          "bytes": w.bytes, "stream_read_ms": round(s_ms, 5),
                          "stream_read_gbs": round(wb / s_ms / 1e6, 1),
                          "stream_read_shape": f"{t} threads x {l} loads{' non-temporal' if nt else ''}",
                          "frac_of_stream_read": round(s_ms / f_ms, 4)})
            if w.name == "c1_decode_T1":
                entry["stream_read_sweep_gbs"] = stream_ref["sweep_gbs"]
        per[w.name] = entry
        log(f"{w.name}: fused {f_ms:.4f} ms unfused {u_ms:.4f} ms "
            f"x{u_ms / f_ms:.3f} {entry['tflops']} TFLOP/s" +
            (f" {entry['gbs']} GB/s" if "gbs" in entry else ""))

    # roofline of the dominant kernel: the mean duration of its launches in
    # the timed steps
    ms = sum(e0.elapsed_time(e1) for e0, e1 in dom_events) / len(dom_events)
    achieved = dom.flops / ms / 1e9
    traffic = measured_traffic() if dom.name == "c3_relu_aux_f16" else None
    util = measured_counters().get("mfma_util") if dom.name == "c3_relu_aux_f16" else None
    # the published peak assumes 2400 MHz; the chip runs this kernel at a
    # power-limited clock.  The MFMA busy share per cycle (rocprofv3) is the
    # fraction of the peak at the clock actually run, and with the measured
    # time it gives that clock: FLOPs = util * cycles * peak FLOP per cycle.
    sclk = dom.flops / (util * (PEAK_TFLOPS * 1e12 / 2.4e9) * ms * 1e-3) / 1e6 if util else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": dom.name, "avg_launch_ms": round(ms, 5), "launches": len(dom_events),
                "bracket": ("the workload's execution: the B staging copy, then the GEMM kernel"
                            if "stage_b" in dom.fused.info() else "the GEMM kernel"),
                "algorithmic_bytes": dom.bytes, "kernel_source_sha": kernel_source_hash(),
                "frac_of_clock_adjusted_peak": util,
                "implied_sclk_mhz": round(sclk) if sclk else None}
    log(f"roofline {dom.name}: {achieved:.1f} TFLOP/s = {achieved / PEAK_TFLOPS:.3f} of peak; "
        f"MFMA busy share {util}, implied shader clock {sclk and round(sclk)} MHz")
    # context beside the published peak, measured after the timed steps on
    # this same GPU: the tile's MFMA work alone at the power limit (fp16, normal
    # operands, no memory traffic)
    loop = mfma_loop_rate("f16", "normal", trials=3, launches=3)
    loop_bf16 = mfma_loop_rate("bf16", "normal", trials=3, launches=3)
    roofline["mfma_loop_tflops"] = loop["tflops"]
    roofline["frac_of_mfma_loop"] = round(achieved / loop["tflops"], 4)
    log(f"mfma loop on this GPU: {loop['tflops']} TFLOP/s (bf16 {loop_bf16['tflops']}); the "
        f"roofline kernel at {roofline['frac_of_mfma_loop']} of it")
    # every GEMM workload beside the loop of its own dtype (the decode shapes
    # are bound by HBM and carry their stream-read fraction instead)
    for w in suite + extras:
        e = per[w.name]
        if "gbs" not in e:
            ref = loop_bf16 if w.case.dtype == "bf16" else loop
            e["frac_of_mfma_loop"] = round(e["tflops"] / ref["tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()
        log(f"cpu baseline: {cpu}")

    names = [w.name for w in suite]
    rec = {
        "metric": "fused GEMM+bias/act TFLOP/s (% MFMA peak); decode-shape GB/s (% HBM)",
        "value": round(step_flops / ms_step / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16+bf16 in, fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": "fused-epilogue GEMM suite: " + ", ".join(names),
                   "step_tflop": round(step_flops / 1e12, 4),
                   "frac_mfma_peak": round(step_flops / ms_step / 1e9 / PEAK_TFLOPS, 4),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "workloads": per,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
