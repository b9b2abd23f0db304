#!/usr/bin/env python3
"""Benchmark of the GEMM / implicit-GEMM convolution path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

One step is one call of the workload's entry point over its synthetic inputs,
which are resident in HBM before the timed region starts.  W untimed steps,
then exactly K steps between two synchronizations; rank 0 prints one JSON
line.  The headline workload is the 4096^3 fp16 GEMM (TFLOPS); the other
workloads (c1, c2, c4, c5, the quantized convolution q4 and the
blocked-layout convolution b4) are measured in
the same run the same way, before the headline, each followed by 0.3 s of
its own untimed load, and reported under "workloads" (the u8 x i8 ones in
TOPS).

`value` and `roofline.achieved` are algorithmic operations per launch
(2*M*N*K) divided by the mean launch duration of K back-to-back launches
between two HIP events on the stream the kernel runs on, against the MI355X
dense MFMA peak of its dtype.  After that timed region, untimed for `value`:
each launch alone between two events (median, min, max), for c1 and c2 also
with the caches flushed before every launch (cold) and as replays of 100
launches captured into one HIP graph (no host launch path per kernel; a replay
must reproduce the eager call's outputs bit for bit).  Once every timed region
is over, the shader clock of this GPU is read from the driver while each
workload runs (its reads perturbed the launches timed right after them).  `traffic` (HBM bytes per launch)
comes from the committed rocprofv3 counter summary in profiles/ when that
summary was taken on the current kernel sources, else null.

`cpu_baseline` times the CPU oracle on a bounded sample of the same workload
(whole output rows, or whole output pixels for the convolution) on the host's
cores, with the OpenMP thread count it used, the CPUs available to the
process and the CPU model.
"""
from __future__ import annotations

import argparse
import hashlib
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "GEMM/conv TFLOPS (fp16) & TOPS (int8) on 1 MI355X; % of dense MFMA peak"
# MI355X dense MFMA peaks: 256 CUs x 2.4 GHz x (4096 fp16 FLOP | 8192 int8 OP) per clock per CU.
PEAK_F16_TFLOPS = 2516.6
PEAK_I8_TOPS = 5033.2
HBM_GBPS = 8000.0
SRC_FILES = ("implicit_gemm_convolution_amd/csrc/igc.hip",
             "implicit_gemm_convolution_amd/csrc/igc_kernels.hpp",
             "implicit_gemm_convolution_amd/csrc/igc_host.hpp",
             "implicit_gemm_convolution_amd/csrc/igc_launch.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in SRC_FILES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl) -> int:
    """Bytes the workload must move at least once: inputs read once, outputs written once."""
    d = wl.dims
    M, N, K = d["M"], d["N"], d["K"]
    if wl.kind == "gemm_f16":
        return 2 * (M * K + N * K) + 4 * M * N
    if wl.kind in ("conv_f16", "conv_f16_blk"):
        return wl.arrays["x"].nbytes + wl.arrays["w"].nbytes + 4 * M * N
    if wl.kind == "conv_u8i8":
        return wl.arrays["x"].nbytes + wl.arrays["w"].nbytes + M * N + 8 * N
    out = 0
    for o in wl.params["outputs"]:
        out += {"C_i32": 4, "D_f32": 4, "Q_i8": 1}[o] * M * N
    return M * K + N * K + out + (8 * N if "Q_i8" in wl.params["outputs"] else 0)


class Runner:
    """Device-resident inputs/outputs of one workload and a closure launching it."""

    def __init__(self, wl, igc, torch):
        self.wl = wl
        dev = torch.device("cuda:0")
        self.lib = igc.load()
        self.stream = torch.cuda.current_stream().cuda_stream
        d = wl.dims
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        self.keep = []
        self.outs = []  # output tensors (the GEMMs: checked after graph replays)
        if wl.kind == "gemm_f16":
            A, B = t(wl.arrays["A"]), t(wl.arrays["Bt"])
            C = torch.empty((d["M"], d["N"]), dtype=torch.float32, device=dev)
            M, N, K = d["M"], d["N"], d["K"]
            ws, nws = self._workspace(igc.gemm_f16f32_workspace_size(M, N, K), torch, dev)
            self.keep = [A, B, C, ws]
            self.outs = [C]
            self.call = self._direct("gemm_f16f32", M, N, K, A.data_ptr(), K, B.data_ptr(), K,
                                     C.data_ptr(), N, ws.data_ptr() if nws else None, nws, self.stream)
            self.dtype, self.peak, self.unit = "f16", PEAK_F16_TFLOPS, "TFLOPS"
        elif wl.kind == "gemm_u8i8":
            pr = wl.params
            A, B = t(wl.arrays["A"]), t(wl.arrays["Bt"])
            M, N, K = d["M"], d["N"], d["K"]
            kw = {}
            if "C_i32" in pr["outputs"]:
                C = torch.empty((M, N), dtype=torch.int32, device=dev)
                kw.update(C_i32=C, ldc=N)
            if "D_f32" in pr["outputs"]:
                D = torch.empty((M, N), dtype=torch.float32, device=dev)
                s = float(np.float32(np.float32(pr["sA"]) * np.float32(pr["sB"])))
                kw.update(D_f32=D, ldd=N, dq_scale=s)
            if "Q_i8" in pr["outputs"]:
                Q = torch.empty((M, N), dtype=torch.int8, device=dev)
                S, Bi = t(wl.arrays["scale"]), t(wl.arrays["bias"])
                kw.update(Q_i8=Q, ldq=N, scale_n=S, bias_n=Bi)
            ws, nws = self._workspace(igc.gemm_u8i8_zp_workspace_size(M, N, K), torch, dev)
            self.keep = [A, B, ws] + [v for v in kw.values() if hasattr(v, "data_ptr")]
            self.outs = [kw[k] for k in ("C_i32", "D_f32", "Q_i8") if k in kw]
            zA, zB = pr["zA"], pr["zB"]
            a = lambda k: kw[k].data_ptr() if k in kw else None  # noqa: E731
            self.ep = igc.Epilogue(a("C_i32"), kw.get("ldc", 0), a("D_f32"), kw.get("ldd", 0),
                                   kw.get("dq_scale", 0.0), a("Q_i8"), kw.get("ldq", 0),
                                   a("scale_n"), a("bias_n"), ws.data_ptr() if nws else None, nws)
            self.call = self._direct("gemm_u8i8_zp", M, N, K, A.data_ptr(), K, zA, B.data_ptr(), K, zB,
                                     ctypes.byref(self.ep), self.stream)
            self.dtype, self.peak, self.unit = "i8", PEAK_I8_TOPS, "TOPS"
        elif wl.kind == "conv_u8i8":
            pr = wl.params
            x, w = t(wl.arrays["x"]), t(wl.arrays["w"])
            S, Bi = t(wl.arrays["scale"]), t(wl.arrays["bias"])
            Q = torch.empty((d["M"], d["N"]), dtype=torch.int8, device=dev)
            args = (d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"],
                    d["stride_w"], d["pad_h"], d["pad_w"])
            ws, nws = self._workspace(igc.conv2d_u8i8_zp_workspace_size(*args), torch, dev)
            # the weights are fixed across calls: their column sums are formed
            # once here, outside the timed launches (colsum_B)
            Kd = d["R"] * d["S"] * d["C"]
            cs = torch.empty(d["N"], dtype=torch.int32, device=dev)
            igc.u8i8_colsum(d["N"], Kd, w, Kd, cs)
            self.keep = [x, w, S, Bi, Q, ws, cs]
            self.ep = igc.Epilogue(None, 0, None, 0, 0.0, Q.data_ptr(), d["N"], S.data_ptr(), Bi.data_ptr(),
                                   ws.data_ptr() if nws else None, nws, cs.data_ptr())
            self.call = self._direct("conv2d_u8i8_zp", *args, x.data_ptr(), pr["zA"], w.data_ptr(), pr["zB"],
                                     ctypes.byref(self.ep), self.stream)
            self.dtype, self.peak, self.unit = "i8", PEAK_I8_TOPS, "TOPS"
        elif wl.kind == "conv_f16_blk":
            x, w = t(wl.arrays["x"]), t(wl.arrays["w"])
            P = (d["H"] + 2 * d["pad_h"] - d["R"]) // d["stride_h"] + 1
            Q = (d["W"] + 2 * d["pad_w"] - d["S"]) // d["stride_w"] + 1
            y = torch.empty((d["Nb"] // 16, P, Q, d["Kout"] // 16, 16, 16), dtype=torch.float32, device=dev)
            args = (d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"],
                    d["stride_w"], d["pad_h"], d["pad_w"])
            ws, nws = self._workspace(igc.conv2d_implicit_gemm_nhwcnc_workspace_size(*args), torch, dev)
            self.keep = [x, w, y, ws]
            self.call = self._direct("conv2d_implicit_gemm_nhwcnc", *args, x.data_ptr(), w.data_ptr(),
                                     y.data_ptr(), ws.data_ptr(), nws, self.stream)
            self.dtype, self.peak, self.unit = "f16", PEAK_F16_TFLOPS, "TFLOPS"
        else:
            x, w = t(wl.arrays["x"]), t(wl.arrays["w"])
            P = (d["H"] + 2 * d["pad_h"] - d["R"]) // d["stride_h"] + 1
            Q = (d["W"] + 2 * d["pad_w"] - d["S"]) // d["stride_w"] + 1
            y = torch.empty((d["Nb"], P, Q, d["Kout"]), dtype=torch.float32, device=dev)
            args = (d["Nb"], d["H"], d["W"], d["C"], d["Kout"], d["R"], d["S"], d["stride_h"],
                    d["stride_w"], d["pad_h"], d["pad_w"])
            ws, nws = self._workspace(igc.conv2d_implicit_gemm_workspace_size(*args), torch, dev)
            self.keep = [x, w, y, ws]
            self.call = self._direct("conv2d_implicit_gemm", *args, x.data_ptr(), w.data_ptr(),
                                     y.data_ptr(), ws.data_ptr() if nws else None, nws, self.stream)
            self.dtype, self.peak, self.unit = "f16", PEAK_F16_TFLOPS, "TFLOPS"

    @staticmethod
    def _workspace(nbytes, torch, dev):
        """The caller-owned workspace the library asks for (zero-filled once)."""
        return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev), nbytes

    def _direct(self, name, *args):
        """The C-ABI entry point with its arguments converted once: the timed
        loop pays the library call, not the binding's per-call marshalling."""
        fn = getattr(self.lib, name)

        def call():
            st = fn(*args)
            if st:
                raise RuntimeError(f"{name}: status {st}")
        return call

    def measure(self, torch, steps: int, warmup: int, cold: bool = False, extras: bool = True) -> dict:
        """Time `steps` back-to-back launches on the current stream between two
        HIP events: the average launch duration is the elapsed time / steps
        (no event commands between the launches, as a caller would run them).
        Then, untimed for the headline value: each launch alone between two
        events (median, min, max), and the same with the caches flushed before
        every launch when `cold`.  (The shader clock is read in a pass of its
        own after every workload's timed regions: see `sclk_while_running`.)"""
        if warmup is None:
            # until 0.25 s of work has run (at least 10 launches)
            warmup, t0 = 0, time.perf_counter()
            while warmup < 10 or time.perf_counter() - t0 < 0.25:
                for _ in range(10):
                    self.call()
                warmup += 10
                torch.cuda.synchronize()
        else:
            for _ in range(warmup):
                self.call()
        torch.cuda.synchronize()
        t_all0 = torch.cuda.Event(enable_timing=True)
        t_all1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_all0.record()
        for _ in range(steps):
            self.call()
        t_all1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total = t_all0.elapsed_time(t_all1) * 1e-3
        ops = self.wl.ops()
        step_s = total / steps
        res = dict(
            steps=steps, warmup=warmup, ms_per_step=step_s * 1e3, wall_s=wall,
            value=ops / step_s / 1e12, unit=self.unit, dtype=self.dtype,
            launch_us_mean=step_s * 1e6,
            achieved=ops / step_s / 1e12, peak=self.peak,
            frac_of_peak=ops / step_s / 1e12 / self.peak,
            alg_gbps=algorithmic_bytes(self.wl) / step_s / 1e9,
        )
        if not extras:
            return res
        res.update(self._per_launch(torch, steps, "alone_us"))
        if cold:
            # a 512 MiB write between launches evicts the operands from the
            # 256 MiB last-level cache (MALL) and the L2s
            flush = torch.empty(512 << 18, dtype=torch.float32, device="cuda")
            res.update(self._per_launch(torch, steps, "cold_launch_us", before=lambda: flush.fill_(1.0)))
            res["cold_alg_gbps"] = algorithmic_bytes(self.wl) / (res["cold_launch_us_median"] * 1e-6) / 1e9
            del flush
        return res

    def _per_launch(self, torch, steps, key, before=None) -> dict:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            if before is not None:
                before()
            e0.record()
            self.call()
            e1.record()
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
        return {f"{key}_median": us[len(us) // 2], f"{key}_min": us[0], f"{key}_max": us[-1],
                f"{key}_mean": sum(us) / len(us)}

    def sustain(self, torch, seconds):
        """Back-to-back launches for `seconds` (untimed)."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                self.call()
            torch.cuda.synchronize()

    def sclk_while_running(self, torch, path, seconds=0.3):
        """Shader clock (MHz) read from `path` while back-to-back launches run,
        or None.  Each read of the driver's DPM table queries the GPU's power
        management, and the launches timed shortly after such reads ran
        slower (8192^3 int8 with --warmup 5: 447-459 us per launch against
        368 us without them), so bench takes these readings only after every
        workload's timed regions."""
        import threading

        if path is None:
            return None
        samples, stop = [], threading.Event()

        def poll():
            while not stop.is_set():
                v = read_sclk_mhz(path)
                if v is None:
                    return
                samples.append(v)
                time.sleep(0.01)

        th = threading.Thread(target=poll, daemon=True)
        th.start()
        self.sustain(torch, seconds)
        stop.set()
        th.join()
        if not samples:
            return None
        samples.sort()
        return {"median": samples[len(samples) // 2], "min": samples[0], "max": samples[-1],
                "samples": len(samples)}


def sclk_path(torch):
    """The driver's DPM table (pp_dpm_sclk) of the GPU this process uses,
    matched by PCI address among /sys/class/drm/card*, or None (another
    card's table would give another GPU's clock)."""
    import glob

    try:
        pr = torch.cuda.get_device_properties(torch.cuda.current_device())
        want = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}."
    except (AttributeError, RuntimeError):
        return None
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        if os.path.basename(os.path.realpath(os.path.dirname(path))).lower().startswith(want):
            return path
    return None


def read_sclk_mhz(path=None):
    """Current shader clock (MHz) in a pp_dpm_sclk table (the level marked
    '*'), or None where there is none or it is not readable."""
    if path is None:
        return None
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    tok = [t for t in line.split() if t.lower().endswith("mhz")]
                    if tok:
                        return float(tok[0][:-3])
    except OSError:
        pass
    return None


def host_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "cpus_available": avail}


def graph_launch_us(wl, igc, torch, launches: int = 100, replays: int = 10) -> dict:
    """The workload's launches captured into one HIP graph and replayed: per
    launch = elapsed / (launches x replays).  At the small sizes (c1, c2) the
    host's per-call launch path (a ctypes call and a kernel launch), not the
    kernel, bounds the back-to-back figure; a caller with a launch-bound loop
    would capture it.  Reported only if a replay reproduces the eager call's
    outputs bit for bit."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r = Runner(wl, igc, torch)  # its launches go to the capture stream
        r.call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in r.outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
        for _ in range(launches):
            r.call()
    for o in r.outs:
        o.fill_(7)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    if not r.outs or not all(torch.equal(o, e) for o, e in zip(r.outs, ref)):
        return {"graph_launch_us": None, "graph_note": "a replay did not reproduce the eager call"}
    for _ in range(3):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (launches * replays)
    return {"graph_launch_us": us, "graph_launches": launches, "graph_replays": replays}


def cpu_baseline(wl, budget_s: float) -> dict:
    """Time the oracle on whole output rows (pixels) of the workload for about budget_s."""
    import oracle

    oracle.lib()
    d = wl.dims
    cores = oracle.num_threads()

    done = [0]  # rows (pixels) the last run covered

    def run(nrows):
        done[0] = nrows
        rows = np.arange(nrows)
        t0 = time.perf_counter()
        if wl.kind == "conv_f16_blk":
            # whole groups of 16 images (the blocked layout's unit)
            g = max(1, -(-nrows // (16 * d["M"] // d["Nb"])))
            oracle.conv2d_nhwcnc_direct(wl.arrays["x"][:g], wl.arrays["w"],
                                        (d["stride_h"], d["stride_w"]), (d["pad_h"], d["pad_w"]))
            done[0] = min(d["M"], g * 16 * d["M"] // d["Nb"])
            return time.perf_counter() - t0
        if wl.kind == "gemm_f16":
            oracle.gemm_f16(wl.arrays["A"][rows], wl.arrays["Bt"])
        elif wl.kind == "gemm_u8i8":
            pr = wl.params
            C = oracle.gemm_u8i8_naive(wl.arrays["A"][rows], pr["zA"], wl.arrays["Bt"], pr["zB"])
            if "D_f32" in pr["outputs"]:
                oracle.dequant(C, pr["sA"], pr["sB"])
            if "Q_i8" in pr["outputs"]:
                oracle.requant(C, wl.arrays["scale"], wl.arrays["bias"])
        elif wl.kind == "conv_u8i8":
            pr = wl.params
            C = oracle.conv2d_u8i8_direct_at(wl.arrays["x"], pr["zA"], wl.arrays["w"], pr["zB"], rows,
                                             (d["stride_h"], d["stride_w"]), (d["pad_h"], d["pad_w"]))
            oracle.requant(C, wl.arrays["scale"], wl.arrays["bias"])
        else:
            oracle.conv2d_direct_at(wl.arrays["x"], wl.arrays["w"], rows,
                                    (d["stride_h"], d["stride_w"]), (d["pad_h"], d["pad_w"]))
        return time.perf_counter() - t0

    n = 8
    t = run(n)
    while t < 0.5 and n < d["M"]:
        n = min(d["M"], n * 4)
        t = run(n)
    n = int(min(d["M"], max(n, n * budget_s / max(t, 1e-9))))
    t = run(n)
    n = done[0]
    ops = 2.0 * n * d["N"] * d["K"]
    unit = "TOPS" if wl.kind in ("gemm_u8i8", "conv_u8i8") else "TFLOPS"
    what = "output pixels" if wl.kind.startswith("conv") else "output rows"
    info = host_info()
    return dict(value=ops / t / 1e12, unit=unit, cores=cores, kind="oracle",
                sample=f"first {n} of {d['M']} {what} of {wl.name} (all {d['N']} columns, "
                       f"K={d['K']}), {t:.1f} s on {cores} OpenMP threads",
                cpu_model=info["cpu_model"], cpus_available=info["cpus_available"],
                seconds=t)


def traffic_for(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("kernel_source_hash:"):
            vals["hash"] = line.split(":", 1)[1].strip()
        elif line.startswith("hbm_bytes_per_launch "):
            key, v = line[len("hbm_bytes_per_launch "):].split(":", 1)
            vals[key.strip()] = int(v)
    if vals.get("hash") != kernel_source_hash():
        return None
    return vals.get(workload)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches first (default: as many as take 0.25 s, since the GPU's "
                         "clock reaches its steady state only after ~20 ms of sustained load)")
    ap.add_argument("--workload", default="c3", choices=synth.WORKLOADS)
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the back-to-back launches only: no per-launch, cold-cache or clock passes "
                         "(for profiler runs)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--variant", type=int, default=-1,
                    help="force a tile variant through igc_set_tuning (-1: by shape; 0 256x256, 1 128x128, "
                         "2 64x64, 3 256x128, 4 224x256, 5 fp16 LDS bypass) -- for A/B runs, not the headline")
    ap.add_argument("--streamk", type=int, default=1, help="stream-K mode for igc_set_tuning (0, 1, 2)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                          "launches": 5}))
        return 0

    import implicit_gemm_convolution_amd as igc

    st = igc.device_check()
    if st != igc.IGC_OK:
        print(f"device check failed: {igc.last_error()}", file=sys.stderr)
        return 1
    igc.set_tuning(args.variant, args.streamk)

    # The headline workload runs last: after the others, the GPU is at the
    # steady clock it holds under sustained load (it needs ~20 ms of load to
    # leave its idle clock), whatever --warmup says, provided nothing leaves
    # it idle in between (below).
    # The others run in an order where each follows one of similar power
    # draw: the fp16 convolutions, then the int8 ones (q4 after c5 read
    # 61-62 us per launch with --warmup 5, 58.5 after the fp16 convolutions;
    # c5 right after c2 read 405-411 us, 377-382 after q4).
    order = ("c1", "c2", "c4", "b4", "q4", "c5", "c3")
    assert sorted(order) == sorted(synth.WORKLOADS)
    names = ([] if args.only else [w for w in order if w != args.workload]) + [args.workload]
    # Every workload's inputs are made resident before the first measurement,
    # so the measurements follow one another with no host-to-device copies
    # between them and the headline's timed region starts from the sustained
    # load of the workload before it.
    # Each is launched once here, too: the runtime loads a kernel's code at
    # its first launch (~1.3 ms with the GPU idle), and the launches after
    # such a stall run in a clock transient (4096^3 GEMM with --warmup 5:
    # 107 us per launch instead of ~100).
    wls = {name: synth.workload(name) for name in names}
    runners = {name: Runner(wls[name], igc, torch) for name in names}
    for r in runners.values():
        r.call()
    torch.cuda.synchronize()
    results = {}
    head_wl = None
    for name in names:
        wl = wls[name]
        res = runners[name].measure(torch, args.steps, args.warmup, cold=name in ("c1", "c2"),
                                    extras=not args.no_extras)
        if name in ("c1", "c2") and not args.no_extras:
            res.update(graph_launch_us(wl, igc, torch))
        res["roofline_traffic_bytes"] = traffic_for(name)
        res["config"] = synth.DESCRIPTIONS[name]
        results[name] = res
        if name == args.workload:
            head_wl = wl
        elif not args.no_extras:
            # 0.3 s of this workload's own load, untimed: the next workload's
            # warm-up and timed launches follow sustained load, not a host gap
            runners[name].sustain(torch, 0.3)
    # the shader clock of each workload, read only now that every timed
    # region is over (see Runner.sclk_while_running)
    if not args.no_extras:
        path = sclk_path(torch)
        for name in names:
            results[name]["sclk_mhz"] = runners[name].sclk_while_running(torch, path)
    del runners
    for name in names:
        res = results[name]
        print(f"# {name}: {res['value']:.1f} {res['unit']} ({100 * res['frac_of_peak']:.1f}% of peak), "
              f"{res['launch_us_mean']:.1f} us/launch back to back"
              + (f", {res['alone_us_median']:.1f} us median alone" if "alone_us_median" in res else "")
              + (f", {res['cold_launch_us_median']:.1f} us cold" if "cold_launch_us_median" in res else "")
              + (f", {res['graph_launch_us']:.1f} us/launch as graph replays" if res.get("graph_launch_us") else "")
              + (f", sclk {res['sclk_mhz']['median']:.0f} MHz" if res.get("sclk_mhz") else ""),
              file=sys.stderr, flush=True)

    head = results[args.workload]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head_wl, args.cpu_budget)
        cpu.pop("seconds", None)

    d = head_wl.dims
    line = {
        "metric": METRIC,
        **({"tuning": {"variant": args.variant, "streamk": args.streamk}}
           if (args.variant, args.streamk) != (-1, 1) else {}),
        "value": round(head["value"], 2),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": head["warmup"],
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded numpy inputs with the workload's shapes and distributions)",
        "config": {"workload": f"{args.workload}: {synth.DESCRIPTIONS[args.workload]}",
                   "M": d["M"], "N": d["N"], "K": d["K"], "ops_per_step": head_wl.ops()},
        "roofline": {
            "bound": "mfma",
            "achieved": round(head["achieved"], 2),
            "peak": head["peak"],
            "unit": "TFLOP/s" if head["dtype"] == "f16" else "TOP/s",
            "frac": round(head["frac_of_peak"], 4),
            "traffic": traffic_for(args.workload),
            "launch_us_mean": round(head["launch_us_mean"], 2),
            # each launch alone between two events (after the timed region)
            "alone_us_median": round(head["alone_us_median"], 2) if "alone_us_median" in head else None,
            "alone_us_min": round(head["alone_us_min"], 2) if "alone_us_min" in head else None,
            "alone_us_max": round(head["alone_us_max"], 2) if "alone_us_max" in head else None,
            "sclk_mhz": head.get("sclk_mhz"),
            "kernel_source_hash": kernel_source_hash(),
        },
        "cpu_baseline": cpu,
        "workloads": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in results.items()},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
