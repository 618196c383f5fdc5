#!/usr/bin/env python3
"""Throughput of the fine-grained FP8 block-scaled GEMM path on one MI355X.

One step is one pass of the path over one batch of synthetic input. The
default workload is the dense Fprop projection (X[4096][7168] BF16 quantized
1x128, W[7168][7168] BF16 quantized 128x128, block-scaled FP8 GEMM with FP32
promotion per 128-wide K chunk, BF16 output). Other workloads (--workload)
measure the remaining forms of the path: the backward pair (Dgrad + Wgrad with
the 128x1 transposed quantizer), the grouped MoE expert GEMMs and their
backward (grouped Dgrad, grouped 128x1 transposed quantizers, per-expert
Wgrad), the MoE dispatch with its FP8 payload and the BF16 combine, the
decode-shaped grouped GEMM, the Fprop whose GEMM writes the next layer's
1x128-quantized input directly (fused quantizing epilogue; also with the
transposed 128x1 copy for the backward), and the Fprop with power-of-two
scales applied by the MFMA itself (E8M0 variant).

Prints one JSON line. `value` is whole-step throughput with inputs resident in
HBM; `roofline` describes the dominant kernel, timed live with HIP events (created
without the system-scope fence a default event performs on record) on
the stream the kernels run on; `cpu_baseline` times the CPU oracle on a
bounded sample of the same step (rank 0, one GPU only). Before the warm-up
steps, untimed steps run for --clock-ramp-ms (300 ms by default) so that the
GPU clocks have reached their loaded steady state; `clock_ramp` reports them.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOPS and % of MI355X FP8 MFMA peak; quant GB/s"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "fp8_block_scaled_x1_amd", "csrc", f)
                  for f in ("gemm.hip", "quant.hip", "moe.hip", "device_common.h")]


def _code_only(text):
    """Kernel source without its comments and with whitespace collapsed (the
    sources hold no string literal with a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest():
    """Digest of the kernel sources' code: it changes when the code does, not
    when only comments do."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counters, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(f"{workload}:{kernel}")
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("bytes_per_launch")


class HipTimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence.

    A default HIP event performs a system-scope fence when it is recorded (an
    L2 writeback and invalidation on MI355X), which slows the kernel that
    follows it; the HIP headers recommend this flag for events that only
    measure time. Calls go to the HIP runtime torch has loaded, so torch's
    stream handles are valid here.
    """

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes
        self.ctypes = ctypes
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = self.ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = self.ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(self.ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


class Timer:
    """Timing events around each kernel of a step, on the stream the kernels run on."""

    def __init__(self, torch, names, steps, stream, events):
        self.names = names
        self.stream = stream
        self.events = events
        self.ev = [[events.create() for _ in range(len(names) + 1)] for _ in range(steps)]
        self.i = 0
        self.k = 0

    def mark(self):
        if self.i < len(self.ev):
            self.events.record(self.ev[self.i][self.k], self.stream)
        self.k += 1
        if self.k == len(self.names) + 1:
            self.k = 0
            self.i += 1

    def samples_us(self):
        out = {}
        for j, n in enumerate(self.names):
            out[n] = [self.events.elapsed_ms(row[j], row[j + 1]) * 1e3 for row in self.ev[:self.i]]
        return out

    def averages_us(self):
        return {n: sum(ts) / len(ts) for n, ts in self.samples_us().items()}

    def close(self):
        for row in self.ev:
            for e in row:
                self.events.destroy(e)
        self.ev = []


class ClockSampler:
    """Samples the GPU's shader clock from the SMI on a background thread while
    the workload runs: the mean over the XCDs of amdsmi's current_gfxclks when
    it is available, else torch.cuda.clock_rate.

    The SMI refreshes its clock readings only about once a second, so the
    first readings of a window can still show the clock from before the load
    (an idle ~100-200 MHz). The window therefore lasts longer than one refresh
    period, and the leading readings that repeat the window's first value are
    dropped once a different one has arrived."""

    def __init__(self, torch, period_s=0.02):
        import threading
        self.torch = torch
        self.period = period_s
        self.samples = []
        self.source = None
        self.stop_evt = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            import amdsmi
            handle = self.torch.cuda._get_amdsmi_handler(0)   # the handle torch.cuda.clock_rate(0) reads
            xs = [float(v) for v in (amdsmi.amdsmi_get_gpu_metrics_info(handle).get("current_gfxclks") or [])
                  if isinstance(v, (int, float)) and 0 < v < 10000]
            if xs:
                self.source = "amdsmi current_gfxclks, mean over XCDs"
                return sum(xs) / len(xs)
        except Exception:
            pass
        self.source = "torch.cuda.clock_rate"
        return float(self.torch.cuda.clock_rate(0))

    def _run(self):
        while not self.stop_evt.is_set():
            try:
                mhz = self._read()
            except Exception:
                return
            if mhz > 0:
                self.samples.append(mhz)
            self.stop_evt.wait(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop_evt.set()
        self.thread.join()

    def summary(self):
        return clock_summary(self.samples, self.source)


def clock_summary(samples, source=None):
    """Median, range and count of the clock readings after dropping the stale
    leading run (readings equal to the first one, when a later reading
    differs); None without readings."""
    if not samples:
        return None
    k = 0
    while k < len(samples) and samples[k] == samples[0]:
        k += 1
    used = samples[k:] if k < len(samples) else samples
    xs = sorted(used)
    return {"median_mhz": round(xs[len(xs) // 2], 1), "min_mhz": round(xs[0], 1), "max_mhz": round(xs[-1], 1),
            "samples": len(xs), "stale_dropped": len(samples) - len(used), "source": source}


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return float("nan")
    k = (len(xs) - 1) * q
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


# ---------------------------------------------------------------------------
# workloads: each returns (step(timer), info dict)
# ---------------------------------------------------------------------------

def _rotations(bytes_per_set, target=600e6):
    """Copies of the inputs to cycle through so the working set exceeds the 256 MB
    Infinity Cache (the inputs are then served from HBM, not from the cache)."""
    return max(2, int(-(-target // bytes_per_set)))


def _cast_ceilings(torch, dev, inputs):
    """Streaming ceilings for the quantizers: PyTorch's own elementwise cast of
    the same BF16 input to float8_e4m3fn (the same bytes read and written, no
    amax and no scale). The casts cycle through copies of the input whose
    inputs and outputs together exceed the Infinity Cache, so that, like the
    quantizers in the timed steps, they read from HBM. Returns, per kernel
    name, a function that runs the cast of step i."""
    out = {}
    for name, x in inputs.items():
        n = _rotations(x.numel() * 3)
        xs = [x.clone() for _ in range(n)]
        dst = [torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev) for _ in range(n)]
        out[name] = (lambda xs_, dst_: lambda i: dst_[i % len(xs_)].copy_(xs_[i % len(xs_)]))(xs, dst)
    return out


def _kernel_choice(fb, M, N, K, mode):
    """The kernel fp8_gemm_blockscaled picks for an M x N x K problem."""
    bm, bn, depth, tail = fb.fp8_gemm_blockscaled_tile(M, N, K, mode)
    return {"tile": [bm, bn], "ring_depth": depth, "tail_tiles": tail}


def setup_dense_fprop(torch, fb, dev, M=4096, N=7168, K=7168, fused=False, pow2=False):
    """Quantize X 1x128 and W 128x128, then the GEMM. With fused=True the GEMM
    writes the 1x128 quantization of its result (the next layer's FP8 input)
    instead of the BF16 result. With pow2=True the scales are powers of two
    and the MFMA applies them (E8M0 operand scales)."""
    import workloads
    sets = []
    R = _rotations(M * K * 2 + N * K * 2 + M * K + N * K + M * N * (int(fused) if fused else 2))
    for r in range(R):
        d = workloads.dense_fprop(device=dev, seed=r, M=M, N=N, K=K)
        sets.append({
            "X": d["X"], "W": d["W"],
            "qx": torch.empty((M, K), dtype=torch.uint8, device=dev),
            "sx": torch.empty((K // 128, M), dtype=torch.float32, device=dev),
            "qw": torch.empty((N, K), dtype=torch.uint8, device=dev),
            "sw": torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev),
        })
        if fused:
            sets[-1]["Q"] = torch.empty((M, N), dtype=torch.uint8, device=dev)
            sets[-1]["sQ"] = torch.empty((N // 128, M), dtype=torch.float32, device=dev)
        if fused == 2:
            sets[-1]["QT"] = torch.empty((N, M), dtype=torch.uint8, device=dev)
            sets[-1]["sQT"] = torch.empty((M // 128, N), dtype=torch.float32, device=dev)
        else:
            sets[-1]["C"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ceilings = _cast_ceilings(torch, dev, {"quant_act_1x128": sets[0]["X"], "quant_w_128x128": sets[0]["W"]})
    L = fb.lib()
    qa = L.fp8_quant_act_1x128_pow2 if pow2 else L.fp8_quant_act_1x128
    qw = L.fp8_quant_w_128x128_pow2 if pow2 else L.fp8_quant_w_128x128
    stream = torch.cuda.current_stream(dev).cuda_stream
    state = {"i": 0}

    def step(timer):
        s = sets[state["i"] % R]
        state["i"] += 1
        timer.mark()
        rc = qa(s["X"].data_ptr(), fb.BF16, M, K, s["qx"].data_ptr(), s["sx"].data_ptr(), stream)
        timer.mark()
        rc |= qw(s["W"].data_ptr(), fb.BF16, N, K, s["qw"].data_ptr(), s["sw"].data_ptr(), None, None, stream)
        timer.mark()
        if pow2:
            rc |= L.fp8_gemm_blockscaled_pow2(s["qx"].data_ptr(), s["sx"].data_ptr(), s["qw"].data_ptr(),
                                              s["sw"].data_ptr(), fb.SCALE_BLOCK128, s["C"].data_ptr(), M, N, K,
                                              stream)
        elif fused == 2:
            rc |= L.fp8_gemm_blockscaled_q1x128_q128x1T(s["qx"].data_ptr(), s["sx"].data_ptr(), s["qw"].data_ptr(),
                                                        s["sw"].data_ptr(), fb.SCALE_BLOCK128, s["Q"].data_ptr(),
                                                        s["sQ"].data_ptr(), s["QT"].data_ptr(), s["sQT"].data_ptr(),
                                                        M, N, K, stream)
        elif fused:
            rc |= L.fp8_gemm_blockscaled_q1x128(s["qx"].data_ptr(), s["sx"].data_ptr(), s["qw"].data_ptr(),
                                                s["sw"].data_ptr(), fb.SCALE_BLOCK128, s["Q"].data_ptr(),
                                                s["sQ"].data_ptr(), M, N, K, stream)
        else:
            rc |= L.fp8_gemm_blockscaled(s["qx"].data_ptr(), s["sx"].data_ptr(), s["qw"].data_ptr(),
                                         s["sw"].data_ptr(), fb.SCALE_BLOCK128, s["C"].data_ptr(), M, N, K, stream)
        timer.mark()
        if rc:
            raise RuntimeError(f"libfp8bs call failed ({rc})")

    flops = 2.0 * M * N * K
    gemm = {0: "gemm_blockscaled_pow2" if pow2 else "gemm_blockscaled", 1: "gemm_blockscaled_q1x128",
            2: "gemm_blockscaled_q1x128_q128x1T"}[int(fused)]
    out = {0: f"C[{M}x{N}] bf16" + (", power-of-two scales applied by the MFMA (E8M0)" if pow2 else ""),
           1: f"Q[{M}x{N}] fp8 + sQ[{N // 128}x{M}] (fused 1x128 quantizing epilogue)",
           2: f"Q[{M}x{N}] + sQ and QT[{N}x{M}] + sQT (fused 1x128 and transposed 128x1 quantizing epilogue)"
           }[int(fused)]
    info = {
        "names": ["quant_act_1x128", "quant_w_128x128", gemm],
        "kernel_choice": {} if fused or pow2 else {gemm: _kernel_choice(fb, M, N, K, fb.SCALE_BLOCK128)},
        "step_flops": flops,
        "work": {
            "quant_act_1x128": ("GB/s", M * K * 2 + M * K + M * K // 128 * 4),
            "quant_w_128x128": ("GB/s", N * K * 2 + N * K + N * K // 16384 * 4),
            gemm: ("TFLOP/s", flops),
        },
        "dominant": gemm,
        "ceilings": ceilings,
        "config": {"workload": f"dense Fprop projection X[{M}x{K}] bf16 1x128, W[{N}x{K}] bf16 128x128, "
                               f"{out}", "M": M, "N": N, "K": K, "input_rotations": R},
    }
    return step, info


def setup_tiny_fprop(torch, fb, dev, M=256, N=512, K=1024):
    """The tiny Fprop: X[256x1024] and W[512x1024] float32 quantized 1x128 and
    128x128, then the GEMM (launch-latency bound; reported in microseconds)."""
    import workloads
    d = workloads.tiny_fprop(device=dev, M=M, N=N, K=K)
    X, W = d["X"], d["W"]
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sx = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L = fb.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(timer):
        timer.mark()
        rc = L.fp8_quant_act_1x128(X.data_ptr(), fb.F32, M, K, qx.data_ptr(), sx.data_ptr(), stream)
        timer.mark()
        rc |= L.fp8_quant_w_128x128(W.data_ptr(), fb.F32, N, K, qw.data_ptr(), sw.data_ptr(), None, None, stream)
        timer.mark()
        rc |= L.fp8_gemm_blockscaled(qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), fb.SCALE_BLOCK128,
                                     C.data_ptr(), M, N, K, stream)
        timer.mark()
        if rc:
            raise RuntimeError(f"libfp8bs call failed ({rc})")

    flops = 2.0 * M * N * K
    info = {
        "names": ["quant_act_1x128", "quant_w_128x128", "gemm_blockscaled"],
        "kernel_choice": {"gemm_blockscaled": _kernel_choice(fb, M, N, K, fb.SCALE_BLOCK128)},
        "step_flops": flops,
        "work": {"quant_act_1x128": ("GB/s", M * K * 4 + M * K + M * K // 128 * 4),
                 "quant_w_128x128": ("GB/s", N * K * 4 + N * K + N * K // 16384 * 4),
                 "gemm_blockscaled": ("TFLOP/s", flops)},
        "dominant": "gemm_blockscaled",
        "config": {"workload": f"tiny Fprop X[{M}x{K}] f32 1x128, W[{N}x{K}] f32 128x128, C[{M}x{N}] bf16 "
                               f"(launch-latency bound)", "M": M, "N": N, "K": K},
    }
    return step, info


def setup_fprop_q1x128(torch, fb, dev):
    return setup_dense_fprop(torch, fb, dev, fused=True)


def setup_fprop_qboth(torch, fb, dev):
    return setup_dense_fprop(torch, fb, dev, fused=2)


def setup_fprop_pow2(torch, fb, dev):
    return setup_dense_fprop(torch, fb, dev, pow2=True)


def setup_backward(torch, fb, dev, M=4096, N=7168, K=7168):
    """Dgrad dX = dY W and Wgrad dW = dY^T X, with the quantizers they need."""
    import workloads
    R = _rotations(2 * M * N * 2 + M * K * 2 + N * K * 2)
    sets = []
    for r in range(R):
        d = workloads.backward_pair(device=dev, seed=r, M=M, N=N, K=K)
        qw, sw, qwT, swT = fb.fp8_quant_w_128x128(d["W"], transposed=True)   # weights: quantized in Fprop
        sets.append({
            "dY": d["dY"], "X": d["X"], "qwT": qwT, "swT": swT,
            "qdy": torch.empty((M, N), dtype=torch.uint8, device=dev),
            "sdy": torch.empty((N // 128, M), dtype=torch.float32, device=dev),
            "qdyT": torch.empty((N, M), dtype=torch.uint8, device=dev),
            "sdyT": torch.empty((M // 128, N), dtype=torch.float32, device=dev),
            "qxT": torch.empty((K, M), dtype=torch.uint8, device=dev),
            "sxT": torch.empty((M // 128, K), dtype=torch.float32, device=dev),
            "dX": torch.empty((M, K), dtype=torch.bfloat16, device=dev),
            "dW": torch.empty((N, K), dtype=torch.bfloat16, device=dev),
        })
        del qw, sw
    ceilings = _cast_ceilings(torch, dev, {"quant_act_128x1_T(X)": sets[0]["X"]})
    L = fb.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    state = {"i": 0}

    def step(timer):
        s = sets[state["i"] % R]
        state["i"] += 1
        timer.mark()
        # dY both ways in one pass: 1x128 for Dgrad, 128x1 transposed for Wgrad
        rc = L.fp8_quant_act_1x128_128x1_T(s["dY"].data_ptr(), fb.BF16, M, N, s["qdy"].data_ptr(), s["sdy"].data_ptr(),
                                           s["qdyT"].data_ptr(), s["sdyT"].data_ptr(), stream)
        timer.mark()
        rc |= L.fp8_quant_act_128x1_T(s["X"].data_ptr(), fb.BF16, M, K, s["qxT"].data_ptr(), s["sxT"].data_ptr(), stream)
        timer.mark()
        rc |= L.fp8_gemm_blockscaled(s["qdy"].data_ptr(), s["sdy"].data_ptr(), s["qwT"].data_ptr(), s["swT"].data_ptr(),
                                     fb.SCALE_BLOCK128, s["dX"].data_ptr(), M, K, N, stream)
        timer.mark()
        rc |= L.fp8_gemm_blockscaled(s["qdyT"].data_ptr(), s["sdyT"].data_ptr(), s["qxT"].data_ptr(), s["sxT"].data_ptr(),
                                     fb.SCALE_ROW, s["dW"].data_ptr(), N, K, M, stream)
        timer.mark()
        if rc:
            raise RuntimeError(f"libfp8bs call failed ({rc})")

    flops = 2.0 * M * N * K
    info = {
        "names": ["quant_act_1x128_128x1_T(dY)", "quant_act_128x1_T(X)", "gemm_dgrad", "gemm_wgrad"],
        "kernel_choice": {"gemm_dgrad": _kernel_choice(fb, M, K, N, fb.SCALE_BLOCK128),
                          "gemm_wgrad": _kernel_choice(fb, N, K, M, fb.SCALE_ROW)},
        "step_flops": 2 * flops,
        "work": {
            "quant_act_1x128_128x1_T(dY)": ("GB/s", M * N * 2 + 2 * (M * N + M * N // 128 * 4)),
            "quant_act_128x1_T(X)": ("GB/s", M * K * 2 + M * K + M * K // 128 * 4),
            "gemm_dgrad": ("TFLOP/s", flops),
            "gemm_wgrad": ("TFLOP/s", flops),
        },
        "dominant": "gemm_wgrad",
        "ceilings": ceilings,
        "config": {"workload": f"backward pair: Dgrad dX[{M}x{K}] = dY[{M}x{N}] W, Wgrad dW[{N}x{K}] = dY^T X "
                               f"over {M} tokens", "M": M, "N": N, "K": K, "input_rotations": R},
    }
    return step, info


def _quantized_experts(torch, fb, dev, W):
    E, N, K = W.shape
    qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
    for e in range(E):
        qw[e], sw[e] = fb.fp8_quant_w_128x128(W[e])
    return qw, sw


def setup_moe(torch, fb, dev):
    """Grouped expert GEMMs: up (K=7168 -> N=4096) then down (K=2048 -> N=7168)."""
    import workloads
    d = workloads.grouped_moe(device=dev)
    off = torch.from_numpy(d["offsets"]).to(dev)
    Mt = int(d["offsets"][-1])
    E = len(d["counts"])
    qwu, swu = _quantized_experts(torch, fb, dev, d.pop("W_up"))
    qwd, swd = _quantized_experts(torch, fb, dev, d.pop("W_dn"))
    Nu, Ku = qwu.shape[1:]
    Nd, Kd = qwd.shape[1:]
    bufs = {
        "qa": torch.empty((Mt, Ku), dtype=torch.uint8, device=dev),
        "sa": torch.empty((Ku // 128, Mt), dtype=torch.float32, device=dev),
        "qh": torch.empty((Mt, Kd), dtype=torch.uint8, device=dev),
        "sh": torch.empty((Kd // 128, Mt), dtype=torch.float32, device=dev),
        "Cu": torch.empty((Mt, Nu), dtype=torch.bfloat16, device=dev),
        "Cd": torch.empty((Mt, Nd), dtype=torch.bfloat16, device=dev),
    }
    L = fb.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    A_up, A_dn = d["A_up"], d["A_dn"]
    ceilings = _cast_ceilings(torch, dev, {"quant_act_1x128(up)": A_up, "quant_act_1x128(down)": A_dn})

    def step(timer):
        b = bufs
        timer.mark()
        rc = L.fp8_quant_act_1x128(A_up.data_ptr(), fb.BF16, Mt, Ku, b["qa"].data_ptr(), b["sa"].data_ptr(), stream)
        timer.mark()
        rc |= L.fp8_grouped_gemm_blockscaled(b["qa"].data_ptr(), b["sa"].data_ptr(), qwu.data_ptr(), swu.data_ptr(),
                                             b["Cu"].data_ptr(), off.data_ptr(), E, Mt, Nu, Ku, stream)
        timer.mark()
        rc |= L.fp8_quant_act_1x128(A_dn.data_ptr(), fb.BF16, Mt, Kd, b["qh"].data_ptr(), b["sh"].data_ptr(), stream)
        timer.mark()
        rc |= L.fp8_grouped_gemm_blockscaled(b["qh"].data_ptr(), b["sh"].data_ptr(), qwd.data_ptr(), swd.data_ptr(),
                                             b["Cd"].data_ptr(), off.data_ptr(), E, Mt, Nd, Kd, stream)
        timer.mark()
        if rc:
            raise RuntimeError(f"libfp8bs call failed ({rc})")

    fu, fd = 2.0 * Mt * Nu * Ku, 2.0 * Mt * Nd * Kd
    info = {
        "names": ["quant_act_1x128(up)", "grouped_gemm_up", "quant_act_1x128(down)", "grouped_gemm_down"],
        "step_flops": fu + fd,
        "work": {
            "quant_act_1x128(up)": ("GB/s", Mt * Ku * 3 + Mt * Ku // 32),
            "grouped_gemm_up": ("TFLOP/s", fu),
            "quant_act_1x128(down)": ("GB/s", Mt * Kd * 3 + Mt * Kd // 32),
            "grouped_gemm_down": ("TFLOP/s", fd),
        },
        "dominant": "grouped_gemm_up",
        "ceilings": ceilings,
        "config": {"workload": f"grouped MoE experts: {E} experts, {Mt} routed rows (8192 tokens x top-8, "
                               f"Dirichlet(0.5)), up {Ku}->{Nu}, down {Kd}->{Nd}", "E": E, "rows": Mt},
    }
    return step, info


def setup_moe_backward(torch, fb, dev):
    """Backward of the grouped expert GEMMs, down then up: per projection the
    quantizer of dY into both layouts (1x128 and the experts' 128x1 groups),
    the grouped Dgrad on the weights' transposed copies, the grouped 128x1
    transposed quantizer of the forward input, and the per-expert Wgrad."""
    import workloads
    d = workloads.grouped_moe_backward(device=dev)
    off = torch.from_numpy(d["offsets"]).to(dev)
    Mt = int(d["offsets"][-1])
    E = len(d["counts"])
    ld = fb.grouped_ld(Mt, E)
    L = fb.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    proj = []
    for tag, dy_key, x_key, w_key in (("down", "dY_dn", "A_dn", "W_dn"), ("up", "dY_up", "A_up", "W_up")):
        W = d.pop(w_key)
        _, N, K = W.shape        # forward: C[M][N] = X[M][K] W^T
        qwT = torch.empty((E, K, N), dtype=torch.uint8, device=dev)
        swT = torch.empty((E, K // 128, N // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            _, _, qwT[e], swT[e] = fb.fp8_quant_w_128x128(W[e], transposed=True)   # quantized in the forward pass
        del W
        proj.append({
            "tag": tag, "N": N, "K": K, "dY": d[dy_key], "X": d[x_key], "qwT": qwT, "swT": swT,
            "qdy": torch.empty((Mt, N), dtype=torch.uint8, device=dev),
            "sdy": torch.empty((N // 128, Mt), dtype=torch.float32, device=dev),
            "dX": torch.empty((Mt, K), dtype=torch.bfloat16, device=dev),
            "qdyT": torch.empty((N, ld), dtype=torch.uint8, device=dev),
            "sdyT": torch.empty((ld // 128, N), dtype=torch.float32, device=dev),
            "qxT": torch.empty((K, ld), dtype=torch.uint8, device=dev),
            "sxT": torch.empty((ld // 128, K), dtype=torch.float32, device=dev),
            "dW": torch.empty((E, N, K), dtype=torch.bfloat16, device=dev),
        })
    torch.cuda.empty_cache()

    def step(timer):
        rc = 0
        timer.mark()
        for p in proj:
            N, K = p["N"], p["K"]
            # dY both ways in one pass: 1x128 for the grouped Dgrad, the
            # experts' 128x1 groups for the grouped Wgrad
            rc |= L.fp8_quant_act_1x128_128x1_T_grouped(p["dY"].data_ptr(), fb.BF16, Mt, N, off.data_ptr(), E, ld,
                                                        p["qdy"].data_ptr(), p["sdy"].data_ptr(),
                                                        p["qdyT"].data_ptr(), p["sdyT"].data_ptr(), stream)
            timer.mark()
            rc |= L.fp8_grouped_gemm_blockscaled(p["qdy"].data_ptr(), p["sdy"].data_ptr(), p["qwT"].data_ptr(),
                                                 p["swT"].data_ptr(), p["dX"].data_ptr(), off.data_ptr(), E, Mt, K, N,
                                                 stream)
            timer.mark()
            rc |= L.fp8_quant_act_128x1_T_grouped(p["X"].data_ptr(), fb.BF16, Mt, K, off.data_ptr(), E, ld,
                                                  p["qxT"].data_ptr(), p["sxT"].data_ptr(), stream)
            timer.mark()
            rc |= L.fp8_grouped_gemm_wgrad(p["qdyT"].data_ptr(), p["sdyT"].data_ptr(), p["qxT"].data_ptr(),
                                           p["sxT"].data_ptr(), p["dW"].data_ptr(), off.data_ptr(), E, Mt, N, K, ld,
                                           stream)
            timer.mark()
        if rc:
            raise RuntimeError(f"libfp8bs call failed ({rc})")

    names, work, flops = [], {}, 0.0
    for p in proj:
        N, K, t = p["N"], p["K"], p["tag"]
        f = 2.0 * Mt * N * K
        for n, w in ((f"quant_1x128_128x1_T_grouped(dY_{t})", ("GB/s", Mt * N * 4 + Mt * N // 16)),
                     (f"grouped_dgrad_{t}", ("TFLOP/s", f)),
                     (f"quant_128x1_T_grouped(X_{t})", ("GB/s", Mt * K * 3 + Mt * K // 32)),
                     (f"grouped_wgrad_{t}", ("TFLOP/s", f))):
            names.append(n)
            work[n] = w
        flops += 2 * f
    info = {
        "names": names,
        "step_flops": flops,
        "work": work,
        "dominant": "grouped_wgrad_up",
        "config": {"workload": f"grouped MoE backward: {E} experts, {Mt} routed rows (8192 tokens x top-8, "
                               f"Dirichlet(0.5)); down (dX 7168->2048, dW 7168x2048) then up (dX 4096->7168, "
                               f"dW 4096x7168) per expert", "E": E, "rows": Mt, "ld": ld},
    }
    return step, info


def setup_moe_dispatch(torch, fb, dev):
    """MoE dispatch with the FP8 payload (routing, permute + 1x128 quantize into
    the grouped GEMM's layout) and the BF16 combine of the experts' outputs."""
    import workloads
    d = workloads.moe_dispatch(device=dev)
    T, K = d["X"].shape
    topk, E = d["ids"].shape[1], 32
    P = T * topk
    ids = torch.from_numpy(d["ids"]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    X, Y = d["X"], d["Y"]
    L = fb.lib()
    ws = torch.empty(max(L.fp8_moe_dispatch_workspace_bytes(T, topk, E) // 4, 1), dtype=torch.int32, device=dev)
    q = torch.empty((P, K), dtype=torch.uint8, device=dev)
    s = torch.empty((K // 128, P), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((T, topk), dtype=torch.int32, device=dev)
    src = torch.empty(P, dtype=torch.int32, device=dev)
    out = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(timer):
        timer.mark()
        rc = L.fp8_moe_dispatch(X.data_ptr(), fb.BF16, T, K, ids.data_ptr(), topk, E, q.data_ptr(), s.data_ptr(),
                                off.data_ptr(), pos.data_ptr(), src.data_ptr(), ws.data_ptr(), stream)
        timer.mark()
        rc |= L.fp8_moe_combine(Y.data_ptr(), pos.data_ptr(), w.data_ptr(), T, topk, K, out.data_ptr(), stream)
        timer.mark()
        if rc:
            raise RuntimeError(f"libfp8bs call failed ({rc})")

    disp = T * K * 2 + P * K + P * (K // 128) * 4 + P * 4 * 3     # x in; codes, scales, ids/pos/src
    comb = P * K * 2 + T * K * 2 + P * 8                           # Y in, out, pos + weights
    info = {
        "names": ["moe_dispatch", "moe_combine"],
        "step_flops": 0.0,
        "step_bytes": disp + comb,
        "work": {"moe_dispatch": ("GB/s", disp), "moe_combine": ("GB/s", comb)},
        "dominant": "moe_combine",
        "config": {"workload": f"MoE dispatch + combine: {T} tokens x top-{topk} of {E} experts "
                               f"(Dirichlet(0.5)), d_model {K}; payload FP8 1x128, combine BF16",
                   "tokens": T, "topk": topk, "E": E, "K": K},
    }
    return step, info


def setup_decode(torch, fb, dev):
    """Decode-shaped grouped GEMM: 32 experts, 1..256 rows each, weights pre-quantized."""
    import workloads
    d = workloads.decode_grouped(device=dev)
    off = torch.from_numpy(d["offsets"]).to(dev)
    Mt = int(d["offsets"][-1])
    E, N, K = d["W"].shape
    qw, sw = _quantized_experts(torch, fb, dev, d.pop("W"))
    qa, sa = fb.fp8_quant_act_1x128(d["A"])
    # second weight copy so consecutive steps do not hit the Infinity Cache
    qw2, sw2 = qw.clone(), sw.clone()
    C = torch.empty((Mt, N), dtype=torch.bfloat16, device=dev)
    L = fb.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    state = {"i": 0}

    def step(timer):
        w, s = (qw, sw) if state["i"] % 2 == 0 else (qw2, sw2)
        state["i"] += 1
        timer.mark()
        rc = L.fp8_grouped_gemm_blockscaled(qa.data_ptr(), sa.data_ptr(), w.data_ptr(), s.data_ptr(),
                                            C.data_ptr(), off.data_ptr(), E, Mt, N, K, stream)
        timer.mark()
        if rc:
            raise RuntimeError(f"libfp8bs call failed ({rc})")

    nbytes = E * N * K + Mt * K + Mt * N * 2 + E * (N // 128) * (K // 128) * 4 + (K // 128) * Mt * 4
    info = {
        "names": ["grouped_gemm_decode"],
        "step_flops": 2.0 * Mt * N * K,
        "step_bytes": nbytes,
        "work": {"grouped_gemm_decode": ("GB/s", nbytes)},
        "dominant": "grouped_gemm_decode",
        "config": {"workload": f"decode grouped GEMM: {E} experts, {Mt} rows (1..256 per expert), "
                               f"K={K}, N={N}, weights pre-quantized", "E": E, "rows": Mt},
    }
    return step, info


def setup_copy(torch, fb, dev, nbytes=None):
    """A plain device-to-device copy of known size (calibrates HBM byte counters)."""
    nbytes = nbytes or int(os.environ.get("BENCH_COPY_BYTES", 1 << 30))
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)

    def step(timer):
        timer.mark()
        dst.copy_(src)
        timer.mark()

    info = {"names": ["copy"], "step_flops": 0.0, "step_bytes": 2 * nbytes,
            "work": {"copy": ("GB/s", 2 * nbytes)}, "dominant": "copy",
            "config": {"workload": f"device copy of {nbytes} bytes (counter calibration)", "bytes": nbytes}}
    return step, info


WORKLOADS = {"copy": setup_copy, "tiny_fprop": setup_tiny_fprop, "dense_fprop": setup_dense_fprop,
             "fprop_q1x128": setup_fprop_q1x128,
             "fprop_pow2": setup_fprop_pow2, "fprop_qboth": setup_fprop_qboth,
             "backward": setup_backward, "moe": setup_moe, "moe_backward": setup_moe_backward,
             "moe_dispatch": setup_moe_dispatch, "decode": setup_decode}


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same step)
# ---------------------------------------------------------------------------

def cpu_baseline(workload):
    import numpy as np
    import torch
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info())
    except Exception:
        cores = os.cpu_count()
    g = torch.Generator().manual_seed(0)
    if workload == "copy":
        return None
    if workload == "decode":
        # one expert of the decode GEMM: 256 rows x 4096 x 7168, weights pre-quantized
        M, N, K = 256, 4096, 7168
        A = torch.randn(M, K, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        W = (torch.randn(N, K, generator=g) * 0.01).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        qw, sw = oracle.quant_w_128x128(W)
        qa, sa = oracle.quant_act_1x128(A)
        t0 = time.perf_counter()
        oracle.gemm_ref(qa, sa, qw, sw)
        dt = time.perf_counter() - t0
        nbytes = N * K + M * K + M * N * 2
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"one decode expert: GEMM {M}x{N}x{K} (pre-quantized operands), {dt:.1f} s"}
    if workload == "moe_dispatch":
        # 1024 tokens x top-8 of 32 experts, d_model 7168: route, quantize, permute; combine
        import workloads
        T, K, topk = 1024, 7168, 8
        ids, wts = workloads.moe_topk(0, T, 32, topk)
        X = torch.randn(T, K, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        Y = torch.randn(T * topk, K, generator=g).to(torch.bfloat16).float().numpy()
        t0 = time.perf_counter()
        _, _, _, pos, _ = oracle.dispatch_quant(X, ids, 32)
        oracle.combine_ref(Y, pos, wts)
        dt = time.perf_counter() - t0
        P = T * topk
        nbytes = T * K * 2 + P * K + P * (K // 128) * 4 + P * 12 + P * K * 2 + T * K * 2 + P * 8
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{T} tokens x top-{topk}, K={K}: dispatch (route, quantize, permute) and combine; "
                          f"{dt:.1f} s"}
    if workload == "moe_backward":
        # one expert's Wgrad: 1000 tokens (8 groups, the last one padded), dW 4096 x 7168
        T, N, K = 1000, 4096, 7168
        dY = (torch.randn(T, N, generator=g) * 1e-3).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        X = torch.randn(T, K, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        off = np.array([0, T])
        t0 = time.perf_counter()
        qa, sa = oracle.quant_act_128x1_T_grouped(dY, off)
        qb, sb = oracle.quant_act_128x1_T_grouped(X, off)
        oracle.grouped_wgrad_ref(qa, sa, qb, sb, off)
        dt = time.perf_counter() - t0
        return {"value": 2.0 * T * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"one expert's Wgrad over {T} tokens: grouped 128x1 quantizers of dY[{T}x{N}] and "
                          f"X[{T}x{K}], per-expert Wgrad GEMM; {dt:.1f} s"}
    M, N, K = 1024, 4096, 7168
    X = torch.randn(M, K, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    W = (torch.randn(N, K, generator=g) * 0.006).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    fused = workload == "fprop_q1x128"
    pow2 = workload == "fprop_pow2"
    t0 = time.perf_counter()
    qx, sx = oracle.quant_act_1x128(X, pow2=pow2)
    qw, sw = oracle.quant_w_128x128(W, pow2=pow2)
    C, _ = oracle.gemm_ref(qx, sx, qw, sw)
    if fused:
        oracle.quant_act_1x128(C.astype(np.float32))
    dt = time.perf_counter() - t0
    what = "GEMM, quantize C 1x128" if fused else "GEMM"
    return {"value": 2.0 * M * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"one Fprop step at {M}x{N}x{K}: quantize X 1x128 and W 128x128, {what}; {dt:.1f} s"}


def run_workload(torch, fb, dev, name, steps, warmup, ramp_ms, clock_ms=1500.0):
    """Set up one workload, ramp the clocks, warm up, time `steps` steps.

    Returns the step function's info, the wall-clock ms per step, per-kernel
    statistics (HIP events on the launch stream, one pair per kernel and
    step) and the shader clock sampled while the same steps run on after the
    timed ones."""
    step, info = WORKLOADS[name](torch, fb, dev)
    names = info["names"]
    events = HipTimingEvents(torch)
    stream = torch.cuda.current_stream(dev).cuda_stream
    warm = Timer(torch, names, 0, stream, events)
    # The MI355X raises its clocks over the first ~100 ms under load: a few
    # warm-up steps alone leave the timed steps at ramp-up clocks (the dense
    # GEMM measured 15% slower). Untimed steps for ramp_ms come first.
    ramp_steps, t_ramp = 0, time.perf_counter()
    while (time.perf_counter() - t_ramp) * 1e3 < ramp_ms and ramp_steps < 20000:
        for _ in range(4):
            step(warm)
        ramp_steps += 4
        torch.cuda.synchronize()
    ramp = {"steps": ramp_steps, "ms": round((time.perf_counter() - t_ramp) * 1e3, 1)}
    for _ in range(warmup):
        step(warm)
    torch.cuda.synchronize()
    timer = Timer(torch, names, steps, stream, events)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    samples = timer.samples_us()
    timer.close()
    # The shader clock under this workload's load: the same steps, untimed, for
    # clock_ms more while the clock is sampled (the SMI refreshes its reading
    # about once a second, so the window is longer than that).
    try:
        torch.cuda.clock_rate(0)        # initializes the query before the window
    except Exception:
        pass
    with ClockSampler(torch) as clk:
        t_c = time.perf_counter()
        while (time.perf_counter() - t_c) * 1e3 < clock_ms:
            for _ in range(4):
                step(warm)
            torch.cuda.synchronize()
    ceiling_us = {}
    for n, cast in info.get("ceilings", {}).items():
        for i in range(4):
            cast(i)
        ct = Timer(torch, [n], steps, stream, events)
        for i in range(steps):
            ct.mark()
            cast(i)
            ct.mark()
        torch.cuda.synchronize()
        ceiling_us[n] = percentile(ct.samples_us()[n], 0.5)
        ct.close()
    kernels = {}
    for n in names:
        unit, work = info["work"][n]
        ts = samples[n]
        mean = sum(ts) / len(ts)
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        peak = PEAK_FP8_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBS
        rate = work / (mean * 1e-6) / scale
        kernels[n] = {"us": round(mean, 2), "us_median": round(percentile(ts, 0.5), 2),
                      "us_p10": round(percentile(ts, 0.1), 2), "us_p90": round(percentile(ts, 0.9), 2),
                      unit: round(rate, 1), "frac_of_peak": round(rate / peak, 4)}
        if n in ceiling_us:
            # the same bytes through PyTorch's elementwise BF16 -> FP8 cast
            kernels[n]["cast_ceiling_us_median"] = round(ceiling_us[n], 2)
            kernels[n]["frac_of_cast_ceiling"] = round(ceiling_us[n] / percentile(ts, 0.5), 3)
    for n, choice in info.pop("kernel_choice", {}).items():
        kernels[n]["kernel"] = choice
    info.pop("ceilings", None)
    del step
    return info, ms_per_step, kernels, clk.summary(), ramp


def device_summary(torch, dev, clock):
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    out = {"name": props.name, "compute_units": cus}
    if clock:
        mhz = clock["median_mhz"]
        out["sclk_mhz_under_load"] = clock
        out["fp8_peak_at_that_sclk_tflops"] = round(cus * 8192 * mhz * 1e6 / 1e12, 1)
    return out


# Sub-results measured by the default run besides the headline: every
# workload configuration of the benchmark definition, each its own short run.
EXTRA_CONFIGS = [("1_tiny_fprop", "tiny_fprop"), ("3_moe_grouped", "moe"), ("4_decode_grouped", "decode"),
                 ("5_backward_pair", "backward")]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="dense_fprop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="with the default workload, skip the sub-results of the other configurations")
    ap.add_argument("--config-steps", type=int, default=20, help="timed steps of each other configuration")
    ap.add_argument("--clock-ramp-ms", type=float, default=300.0,
                    help="untimed steps for this long before the warm-up steps, so that the GPU clocks "
                         "reach their loaded steady state (0 to skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_block_scaled_x1_amd as fb
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fb.lib()   # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    info, ms_per_step, kernels, clock, ramp = run_workload(torch, fb, dev, args.workload, args.steps, args.warmup,
                                                           args.clock_ramp_ms)
    torch.cuda.empty_cache()

    dom = info["dominant"]
    unit, work = info["work"][dom]
    achieved = kernels[dom][unit]
    peak = PEAK_FP8_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBS
    roofline = {"bound": "mfma" if unit == "TFLOP/s" else "hbm", "achieved": achieved, "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dom, args.workload), "kernel": dom,
                "work_per_launch": work}

    if "step_bytes" in info:
        value, vunit = info["step_bytes"] / (ms_per_step * 1e-3) / 1e9, "GB/s"
    else:
        value, vunit = info["step_flops"] / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": vunit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": info["config"], "kernels": kernels, "roofline": roofline,
        "device": device_summary(torch, dev, clock), "clock_ramp": ramp,
    }
    if args.workload == "dense_fprop" and not args.no_configs:
        configs = {}
        for key, wl in EXTRA_CONFIGS:
            cinfo, cms, ck, cclk, _ = run_workload(torch, fb, dev, wl, args.config_steps, 3, 100.0, 1200.0)
            configs[key] = {"workload": cinfo["config"]["workload"], "ms_per_step": round(cms, 4),
                            "kernels": ck, "sclk_median_mhz": cclk["median_mhz"] if cclk else None}
            torch.cuda.empty_cache()
        line["configs"] = configs
    if not args.no_cpu_baseline and args.workload != "copy":
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
