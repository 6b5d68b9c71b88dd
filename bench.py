#!/usr/bin/env python3
"""Benchmark of the TQ2_0_g128 ternary matmul on one MI355X.

Headline (one JSON line on stdout): the decode GEMV M=1, K=N=4096 with the
fused residual (out = residual + x . W^T), one ``tq2_gemv`` call per step,
as achieved HBM GB/s of algorithmic bytes (codes + scales + x + residual +
out, each counted once).  The weight of every call comes from a pool of
copies larger than the 256 MB Infinity Cache, so each call streams its
weight from HBM; the calls are replayed back to back from a HIP graph.
Every timed region (the headline's exactly --steps calls after exactly
--warmup untimed ones) is preceded by an untimed run-in of the same calls,
about 20 ms of GPU time, so that it measures them at the clock the GPU
settles to under that load rather than at the idle clock (time_graphs).

Also reported in the same line: the roofline object of the dominant kernel,
the CPU oracle's throughput on a bounded sample of the same workload, and the
large-M GEMM (M=1536, K=N=3072) in TFLOP/s against the f16 matrix-core peak.
"""

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
F16_MFMA_PEAK_TFLOPS = 2516.6    # MI355X dense f16 matrix-core peak (256 CU, 2.4 GHz)
METRIC = "TQ2 GEMV achieved HBM GB/s (M=1); TQ2 GEMM TFLOP/s at M=1536 (% roofline)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=4096)
    p.add_argument("--warmup", type=int, default=512)
    p.add_argument("--pool-mib", type=int, default=1100,
                   help="total size of the rotated weight copies (>> 256 MB Infinity Cache)")
    p.add_argument("--gemm-reps", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-gemm", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-batched", action="store_true",
                   help="skip the batched decode GEMV (16 weights per call)")
    p.add_argument("--no-chain", action="store_true",
                   help="skip the 100-layer M=1536 chain (config 5)")
    p.add_argument("--no-small-batch", action="store_true",
                   help="skip the small-batch prefill GEMM lines (M = 7, 8, 9, 100; K=4096 -> N=11008)")
    p.add_argument("--no-swiglu", action="store_true",
                   help="skip the fused gate/up + SwiGLU lines (K=4096 -> N=11008)")
    p.add_argument("--no-q1", action="store_true",
                   help="skip the Q1_g128 (1-bit) decode GEMV and M=1536 GEMM lines")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the decode GEMV size sweep (N = K = 4096, 8192, 16384)")
    p.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                   help="untimed run-in of the same calls ahead of each timed region (ms of GPU "
                        "time; a profiler run may shorten it to keep its trace small)")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run one device-to-device copy of this size (MiB) so a "
                        "counter run can scale FETCH_SIZE / WRITE_SIZE against known bytes")
    return p.parse_args()


KERNEL_HEADERS = ("gemv_tq2_g128_amd/csrc/tq2_internal.h", "gemv_tq2_g128_amd/csrc/tq2_device.h")


def kernel_source_digest(source):
    """sha256 of a kernel source followed by the headers it includes."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for path in (source,) + KERNEL_HEADERS:
        with open(os.path.join(here, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key, source):
    """HBM bytes per launch of one kernel from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled against a device copy of known size), or
    None when the kernel source or its headers have changed since the
    counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        digest = kernel_source_digest(source)
        with open(os.path.join(here, "profiles", "gemv_k4096_n4096_traffic.md")) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    tag = "machine-readable: %s=" % key
    for line in lines:
        if line.startswith(tag):
            fields = dict(kv.split("=", 1) for kv in line[len("machine-readable: "):].split())
            if fields.get("kernel_source_sha256") == digest:
                return int(fields[key])
    return None


def run_environment(torch):
    """Device, HIP runtime and ROCm version, and the GFX clock levels the
    driver lists (None where a file is not readable).  Files only: no other
    program is started from this process."""
    import glob
    import re
    props = torch.cuda.get_device_properties(0)
    env = {"device": torch.cuda.get_device_name(0) or None,
           "arch": getattr(props, "gcnArchName", None), "hip_runtime": torch.version.hip,
           "rocm": None, "gfx_clock_mhz_max": None, "gfx_clock_mhz_min": None}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip() or None
    except OSError:
        pass
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                mhz = [int(v) for v in re.findall(r"(\d+)\s*Mhz", f.read(), re.I)]
        except OSError:
            continue
        if mhz:
            env["gfx_clock_mhz_max"], env["gfx_clock_mhz_min"] = max(mhz), min(mhz)
            break
    return env


def _sclk_file(torch):
    """The driver's pp_dpm_sclk file of the GPU torch calls cuda:0 (matched
    by PCI address), else the first one found, or None."""
    import glob
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    props = torch.cuda.get_device_properties(0)
    bus = getattr(props, "pci_bus_id", None)
    if bus is not None:
        want = "%04x:%02x:%02x" % (getattr(props, "pci_domain_id", 0), bus,
                                   getattr(props, "pci_device_id", 0))
        for f in files:
            if os.path.basename(os.path.realpath(os.path.dirname(f))).startswith(want):
                return f
    return files[0] if files else None


class ClockSampler:
    """Samples the GFX clock level the driver marks as current ('*' in
    pp_dpm_sclk) from a background thread, about once a millisecond, while
    `with sampler.phase(name):` blocks run; reports MHz per phase."""

    def __init__(self, torch):
        import threading
        self.path = _sclk_file(torch)
        self.samples = {}
        self._name = None
        self._stop = threading.Event()
        self._thread = None
        if self.path:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def _read(self):
        import re
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*Mhz", line, re.I)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.wait(0.001):
            name = self._name
            if name is not None:
                mhz = self._read()
                if mhz is not None:
                    self.samples.setdefault(name, []).append(mhz)

    def phase(self, name):
        sampler = self

        class _Phase:
            def __enter__(self):
                sampler._name = name

            def __exit__(self, *exc):
                sampler._name = None
        return _Phase()

    def report(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=1.0)
        out = {"source": self.path}
        for name, v in self.samples.items():
            v = sorted(v)
            out[name] = {"samples": len(v), "min_mhz": v[0], "median_mhz": v[len(v) // 2],
                         "max_mhz": v[-1]}
        return out


def gemv_bytes(n, k, residual):
    codes_scales = n * (k // 128) * 34
    return codes_scales + 4 * k + 4 * n + (4 * n if residual else 0)


# Untimed run-in ahead of every timed region.  The GPU's clock governor
# takes milliseconds of load to leave the level it idles at (a 20-call GEMV
# region that starts from idle runs at 650-700 MHz, against 1.4-1.6 GHz once
# the same calls have run for a while), so each region is preceded by about
# SETTLE_MS of the same calls, untimed; the region then measures the calls at
# the clock they settle to.
SETTLE_MS = 20.0           # --settle-ms

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence, recorded on
    a torch stream through the HIP runtime torch itself loaded (found by its
    soname; the process maps only one).  HIP documents the flag for events
    used only to time device work: recording skips the system-scope fence and
    its cache writeback, which adds about a microsecond to every timed region
    (two events around nothing: 4.2-4.3 us with torch's events, 3.2 us with
    these).  Elapsed time is read after a device-wide synchronize."""

    _lib = None

    @classmethod
    def _hip(cls):
        if cls._lib is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so.7")
            vp = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [vp, vp]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            lib.hipEventDestroy.argtypes = [vp]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.lib = self._hip()
        self.ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(self.ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)

    def record(self, stream):
        rc = self.lib.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both completed)."""
        ms = self._ct.c_float()
        rc = self.lib.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return float(ms.value)

    def __del__(self):
        if getattr(self, "ev", None) is not None and self.ev.value:
            self.lib.hipEventDestroy(self.ev)


def _replay(graphs):
    for graph, replays in graphs:
        for _ in range(replays):
            graph.replay()


def time_graphs(torch, graphs, stream, warm=()):
    """Time [(graph, replays)] back to back on `stream` with two events
    (TimingEvent).

    Enqueued with no synchronisation in between: a run-in of the timed graphs
    themselves (passes over them until about SETTLE_MS of GPU time, from one
    untimed pass measured beforehand), the untimed `warm` [(graph, replays)],
    the start event, the timed replays and the end event.  The run-in keeps
    the stream busy while the host submits the rest, so the region holds
    exactly the timed calls, at the clock the workload settles to, and not the
    host's submission of them.  Returns (event ms, wall s of the region's
    submission and execution)."""
    torch.cuda.synchronize()
    start = TimingEvent()
    end = TimingEvent()
    with torch.cuda.stream(stream):
        start.record(stream)
        _replay(graphs)
        end.record(stream)
    torch.cuda.synchronize()
    passes = max(1, min(2000, int(math.ceil(SETTLE_MS / max(start.elapsed_time(end), 1e-3)))))
    if SETTLE_MS <= 0:
        passes = 0
    start = TimingEvent()
    end = TimingEvent()
    with torch.cuda.stream(stream):
        for _ in range(passes):
            _replay(graphs)
        _replay(warm)
        t0 = time.perf_counter()
        start.record(stream)
        _replay(graphs)
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end), time.perf_counter() - t0


def time_graph(torch, graph, replays, stream):
    """`replays` timed replays of one graph, after one untimed replay of it
    (see time_graphs); returns (event ms, wall s)."""
    return time_graphs(torch, [(graph, replays)], stream, warm=[(graph, 1)])


def capture(torch, stream, fn, count):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn(0)                                    # one eager call before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(count):
                fn(i)
    torch.cuda.synchronize()
    return g


def exact_graphs(torch, stream, fn, calls, chunk=2048):
    """HIP graphs that together make exactly `calls` calls fn(0), fn(1), ...:
    one graph of `chunk` calls replayed as often as it fits, and one graph
    for the remainder.  Returns [(graph, replays)]."""
    full, rest = divmod(calls, chunk)
    out = []
    if full:
        out.append((capture(torch, stream, fn, chunk), full))
    if rest:
        out.append((capture(torch, stream, lambda i: fn(full * chunk + i), rest), 1))
    return out


def _time_oracle(fn, seconds):
    """Evaluations of fn() for about `seconds` (at least one; an untimed
    call first when seconds > 0); returns (evaluations, seconds per
    evaluation)."""
    if seconds > 0:
        fn()
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return reps, dt / reps


def cpu_baseline(case2, seconds):
    """The oracle as it stands (float64 NumPy dequantise + product), on the
    host, per workload, with 1 BLAS thread and with the host's cores.

    The dequantisation is single-threaded NumPy; the BLAS threads speed up
    only the float64 product.  Workloads: the two GEMVs in full; the
    small-batch prefill at M = 8 and M = 100 in full; the M = 1536 GEMM in
    full; the 100-layer chain on 64 output columns per layer (every layer's
    first 64 weight rows against fixed N(0, 1) inputs: the chain input for
    K = 3072, a seeded draw for K = 12288).  The headline `value` is the
    K = N = 4096 residual GEMV at the host's cores, in the headline's
    unit."""
    from threadpoolctl import threadpool_limits
    import numpy as np
    import oracle
    import tq2_inputs as G
    cores = len(os.sched_getaffinity(0))
    c1, c3_8, c3_100, c4 = G.config1(), G.config3(8), G.config3(100), G.config4()
    chain_x = {3072: G.chain_input(),
               12288: G.make_activations(np.random.default_rng(12288), G.CHAIN_M, 12288)}
    chain_w = [G.chain_layer_weight(layer) for layer in range(G.CHAIN_LAYERS)]
    cols = np.arange(64)

    def full(c):
        return lambda: oracle.matmul(c["aos"], c["x"], c["n"], c["k"], c["residual"])

    def chain():
        for layer, w in enumerate(chain_w):
            k, n = G.chain_layer_shape(layer)
            oracle.matmul_rows(w, chain_x[k], n, k, cols)

    chain_flop = sum(2.0 * G.CHAIN_M * 64 * G.chain_layer_shape(l)[0]
                     for l in range(G.CHAIN_LAYERS))
    legs = [
        ("gemv_m1_k1024_n1024", full(c1), gemv_bytes(1024, 1024, False), "GB/s", seconds / 8),
        ("gemv_m1_k4096_n4096_residual", full(case2), gemv_bytes(4096, 4096, True), "GB/s",
         seconds / 4),
        ("gemm_m8_k4096_n11008", full(c3_8), 2.0 * 8 * 11008 * 4096, "GFLOP/s", 0.0),
        ("gemm_m100_k4096_n11008", full(c3_100), 2.0 * 100 * 11008 * 4096, "GFLOP/s", 0.0),
        ("gemm_m1536_k3072_n3072", full(c4), 2.0 * 1536 * 3072 * 3072, "GFLOP/s", seconds / 8),
        ("chain_100_layers_m1536_64_columns_per_layer", chain, chain_flop, "GFLOP/s", 0.0),
    ]
    per = {}
    for name, fn, work, unit, secs in legs:
        per[name] = {}
        for threads in ((1, cores) if cores > 1 else (1,)):
            if name.startswith("chain") and threads == 1 and cores > 1:
                continue                         # about 5 s per pass: host cores only
            with threadpool_limits(limits=threads):
                reps, dt = _time_oracle(fn, secs)
            per[name]["threads_%d" % threads] = {
                "value": round(work / dt / 1e9, 4), "unit": unit, "s_per_eval": round(dt, 4),
                "evals": reps}
    head = per["gemv_m1_k4096_n4096_residual"]["threads_%d" % cores]
    return {"value": head["value"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d full oracle evaluations of the K=N=4096 residual GEMV (float64 numpy "
                      "dequantise, single-threaded, + product with %d BLAS threads), %.3f s "
                      "each; per-workload figures at 1 thread and %d threads in `workloads` "
                      "(the chain on 64 output columns per layer)" %
                      (head["evals"], cores, head["s_per_eval"], cores),
            "workloads": per}


def chain_bench(torch, tq2, G, dev, stream):
    """Config 5: 100 chained ternary linears at M = 1536 (shapes repeating
    3072->9216, 3072->3072, 3072->12288, 12288->3072), each with its own
    seeded weight; after a 9216-wide layer the next layer takes the first 3072
    columns, and every input is RMS-rescaled per row (plain torch glue).
    Reported: the GEMM kernels alone (graph of the 100 GEMM launches on fixed
    inputs) and the whole chain with the glue."""
    m = G.CHAIN_M
    soas, shapes = [], []
    for layer in range(G.CHAIN_LAYERS):
        k, n = G.chain_layer_shape(layer)
        aos = torch.from_numpy(G.chain_layer_weight(layer)).to(dev)
        soas.append(tq2.reformat_aos_to_soa(aos, n, k))
        shapes.append((k, n))
        del aos
    x0 = torch.from_numpy(G.chain_input()).to(dev)
    xs = {3072: x0.clone(), 12288: torch.randn((m, 12288), device=dev)}
    outs = {n: torch.empty((m, n), dtype=torch.float32, device=dev) for n in (3072, 9216, 12288)}
    flop = sum(2.0 * m * n * k for k, n in shapes)

    def gemms_only(_):
        for (k, n), soa in zip(shapes, soas):
            st = tq2.gemm_ptr(soa.data_ptr(), xs[k].data_ptr(), 0, outs[n].data_ptr(), m, n, k,
                              torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError("tq2_gemm failed: %s" % tq2.status_string(st))

    g = capture(torch, stream, gemms_only, 1)
    time_graph(torch, g, 1, stream)
    ms, _ = time_graph(torch, g, 3, stream)
    kernels_ms = ms / 3

    def full_chain():
        x = x0
        for layer, ((k, n), soa) in enumerate(zip(shapes, soas)):
            y = tq2.gemm(soa, x, n, k)
            nk = G.chain_layer_shape(layer + 1)[0]
            y = y[:, :nk]
            x = (y / torch.sqrt(torch.mean(y * y, dim=1, keepdim=True) + 1e-6)).contiguous()
        return x

    with torch.cuda.stream(stream):
        full_chain()
        torch.cuda.synchronize()
        start = TimingEvent()
        end = TimingEvent()
        start.record(stream)
        full_chain()
        end.record(stream)
    torch.cuda.synchronize()
    chain_ms = start.elapsed_time(end)
    del soas
    return {"layers": G.CHAIN_LAYERS, "tflop": round(flop / 1e12, 4),
            "gemm_kernels_ms": round(kernels_ms, 4),
            "gemm_tflops": round(flop / (kernels_ms * 1e-3) / 1e12, 2),
            "gemm_frac": round(flop / (kernels_ms * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
            "with_glue_ms": round(chain_ms, 4)}


def swiglu_bench(torch, tq2, G, dev, stream, args):
    """Fused gate/up + SwiGLU, K = 4096 -> N = 11008 (half-zero codes):
    decode (M = 1, gate/up pairs rotated over copies larger than the Infinity
    Cache, as for the GEMV) in GB/s of algorithmic bytes, and prefill
    (M = 1536) in TFLOP/s (4 M N K flop per call: two projections)."""
    n, k = G.SWIGLU_N, G.SWIGLU_K
    gate, up = G.swiglu_weights()
    gs = tq2.reformat_aos_to_soa(torch.from_numpy(gate).to(dev), n, k)
    us = tq2.reformat_aos_to_soa(torch.from_numpy(up).to(dev), n, k)
    sb = tq2.soa_bytes(n, k)
    pool = max(1, int(math.ceil(args.pool_mib * 2 ** 20 / (2 * sb))))
    gpool, upool = gs.repeat(pool), us.repeat(pool)
    gb, ub = gpool.data_ptr(), upool.data_ptr()
    x1 = torch.from_numpy(G.swiglu_activations(1)).to(dev)
    out1 = torch.empty((1, n), dtype=torch.float32, device=dev)

    def decode_call(i):
        st = tq2.gate_up_swiglu_ptr(gb + (i % pool) * sb, ub + (i % pool) * sb, x1.data_ptr(),
                                    out1.data_ptr(), 1, n, k,
                                    torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError("tq2_gate_up_swiglu failed: %s" % tq2.status_string(st))

    g1 = capture(torch, stream, decode_call, pool)
    time_graph(torch, g1, 2, stream)
    reps = max(1, int(math.ceil(args.steps / 4 / pool)))
    ms1, _ = time_graph(torch, g1, reps, stream)
    us1 = ms1 * 1e3 / (reps * pool)
    nbytes = 2 * n * (k // 128) * 34 + 4 * k + 4 * n
    gbs = nbytes / (us1 * 1e-6) / 1e9
    del g1, gpool, upool

    m = 1536
    xm = torch.from_numpy(G.swiglu_activations(m)).to(dev)
    outm = torch.empty((m, n), dtype=torch.float32, device=dev)

    def prefill_call(i):
        st = tq2.gate_up_swiglu_ptr(gs.data_ptr(), us.data_ptr(), xm.data_ptr(), outm.data_ptr(),
                                    m, n, k, torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError("tq2_gate_up_swiglu failed: %s" % tq2.status_string(st))

    per_graph = 10
    gm = capture(torch, stream, prefill_call, per_graph)
    time_graph(torch, gm, 1, stream)
    repm = max(1, args.gemm_reps // 40)
    msm, _ = time_graph(torch, gm, repm, stream)
    usm = msm * 1e3 / (repm * per_graph)
    tflops = 4.0 * m * n * k / (usm * 1e-6) / 1e12
    return {
        "swiglu_decode_k4096_n11008": {
            "gbs": round(gbs, 2), "us_per_call": round(us1, 3), "bytes_per_call": nbytes,
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "calls": reps * pool,
            "pairs_rotated": pool},
        "swiglu_prefill_m1536_k4096_n11008": {
            "tflops": round(tflops, 2), "us_per_call": round(usm, 3),
            "peak_tflops": F16_MFMA_PEAK_TFLOPS, "frac": round(tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "path": tq2.gemm_path(m, n, k), "calls": repm * per_graph},
    }


def launch_floor(torch, dev, stream, base, pool, sb, blocks, steps):
    """Reference launches with the decode GEMV's grid (`blocks` blocks of 256
    threads) from libtq2_probe.so: an empty kernel, and a plain streaming read
    of one weight copy's sb bytes (copies rotated as for the GEMV).  Returns
    None when the probe library is not built."""
    import ctypes
    from gemv_tq2_g128_amd import build as B
    path = os.path.join(B.PKG_DIR, B.PROBE_LIB_NAME)
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    lib.tq2_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.tq2_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    sink = torch.zeros(blocks, dtype=torch.int32, device=dev)

    def empty_call(i):
        if lib.tq2_probe_empty(blocks, torch.cuda.current_stream(dev).cuda_stream) != 0:
            raise RuntimeError("tq2_probe_empty failed")

    def read_call(i):
        if lib.tq2_probe_read(base + (i % pool) * sb, sb, sink.data_ptr(), blocks,
                              torch.cuda.current_stream(dev).cuda_stream) != 0:
            raise RuntimeError("tq2_probe_read failed")

    out = {"grid": "%d blocks x 256 threads" % blocks, "read_bytes": sb, "calls": steps}
    for name, fn in (("empty", empty_call), ("read", read_call)):
        warm = exact_graphs(torch, stream, fn, min(steps, 512))
        ms, _ = time_graphs(torch, exact_graphs(torch, stream, fn, steps), stream, warm=warm)
        out[name + "_us_per_launch"] = round(ms * 1e3 / steps, 3)
    out["read_gbs"] = round(sb / (out["read_us_per_launch"] * 1e-6) / 1e9, 2)
    return out


def gemm_shape_bench(torch, tq2, G, dev, stream, m, n, k, args):
    """tq2_gemm at one shape with config 4's distributions (codes uniform over
    {-1, 0, +1}, d ~ U[0.01, 0.1], x ~ N(0, 1) with 1% outliers x20; seed
    from the shape), graph-replayed back to back: TFLOP/s."""
    import numpy as np
    rng = np.random.default_rng(m + 7 * n + 13 * k)
    soa = tq2.reformat_aos_to_soa(torch.from_numpy(G.make_weight(rng, n, k)).to(dev), n, k)
    x = torch.from_numpy(G.make_activations(rng, m, k, outlier_frac=0.01)).to(dev)
    out = torch.empty((m, n), dtype=torch.float32, device=dev)

    def call(i):
        st = tq2.gemm_ptr(soa.data_ptr(), x.data_ptr(), 0, out.data_ptr(), m, n, k,
                          torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError("tq2_gemm failed: %s" % tq2.status_string(st))

    per_graph = 10
    g = capture(torch, stream, call, per_graph)
    reps = max(1, args.gemm_reps // 40)
    ms, _ = time_graph(torch, g, reps, stream)
    us = ms * 1e3 / (reps * per_graph)
    tflops = 2.0 * m * n * k / (us * 1e-6) / 1e12
    del g, soa, x, out
    return {"tflops": round(tflops, 2), "us_per_call": round(us, 3),
            "peak_tflops": F16_MFMA_PEAK_TFLOPS, "frac": round(tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "path": tq2.gemm_path(m, n, k), "calls": reps * per_graph}


def config1_bench(torch, tq2, G, dev, stream, args):
    """The small decode GEMV, M = 1, K = N = 1024 (8192 blocks, 286,720
    algorithmic bytes), weight copies rotated past the Infinity Cache, calls
    replayed back to back; at this size one call is mostly launch cost."""
    c = G.config1()
    n, k = c["n"], c["k"]
    soa = tq2.reformat_aos_to_soa(torch.from_numpy(c["aos"]).to(dev), n, k)
    sb = tq2.soa_bytes(n, k)
    pool = max(2, int(math.ceil(args.pool_mib * 2 ** 20 / sb)))
    buf = soa.repeat(pool)
    del soa
    base = buf.data_ptr()
    x = torch.from_numpy(c["x"]).to(dev).reshape(-1)
    out = torch.empty(n, dtype=torch.float32, device=dev)

    def call(i):
        st = tq2.gemv_ptr(base + (i % pool) * sb, x.data_ptr(), 0, out.data_ptr(), n, k,
                          torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError("tq2_gemv failed: %s" % tq2.status_string(st))

    calls = max(1, args.steps)
    warm = exact_graphs(torch, stream, call, min(calls, 512))
    ms, _ = time_graphs(torch, exact_graphs(torch, stream, call, calls), stream, warm=warm)
    us = ms * 1e3 / calls
    nbytes = gemv_bytes(n, k, False)
    del buf
    return {"gemv_m1_k1024_n1024": {
        "us_per_call": round(us, 3), "bytes_per_call": nbytes,
        "gbs": round(nbytes / (us * 1e-6) / 1e9, 2),
        "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "copies_rotated": pool, "calls": calls}}


def gemv_sweep(torch, tq2, G, dev, stream, args):
    """Decode GEMV with residual at N = K = 4096, 8192 and 16384 (config 2's
    code and scale distributions, seed 20 + N/4096), each weight rotated over
    copies larger than the Infinity Cache and replayed back to back from a HIP
    graph.  The fixed per-launch cost weighs less as the weight grows."""
    import numpy as np
    lines = {}
    for size in (4096, 8192, 16384):
        n = k = size
        rng = np.random.default_rng(20 + size // 4096)
        aos = torch.from_numpy(G.make_weight(rng, n, k)).to(dev)
        x = torch.from_numpy(G.make_activations(rng, 1, k)).to(dev).reshape(-1)
        res = torch.from_numpy(rng.standard_normal(n, dtype=np.float32)).to(dev)
        soa = tq2.reformat_aos_to_soa(aos, n, k)
        del aos
        sb = tq2.soa_bytes(n, k)
        pool = max(2, int(math.ceil(args.pool_mib * 2 ** 20 / sb)))
        buf = soa.repeat(pool)
        del soa
        base = buf.data_ptr()
        out = torch.empty(n, dtype=torch.float32, device=dev)

        def call(i):
            st = tq2.gemv_ptr(base + (i % pool) * sb, x.data_ptr(), res.data_ptr(), out.data_ptr(),
                              n, k, torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError("tq2_gemv failed: %s" % tq2.status_string(st))

        g = capture(torch, stream, call, pool)
        time_graph(torch, g, 1, stream)
        reps = max(1, int(math.ceil(args.steps / 4 / pool)))
        ms, _ = time_graph(torch, g, reps, stream)
        us = ms * 1e3 / (reps * pool)
        nbytes = gemv_bytes(n, k, True)
        del g, buf
        lines["n%d_k%d" % (n, k)] = {
            "us_per_call": round(us, 3), "bytes_per_call": nbytes,
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 2),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "copies_rotated": pool, "calls": reps * pool}
    return {"gemv_size_sweep_residual": lines}


def small_batch_bench(torch, tq2, G, dev, stream, args):
    """Small-batch prefill GEMM, K = 4096 -> N = 11008 (half-zero codes,
    d ~ U[0.005, 0.05]) at the workload's M = 7, 8, 9 and 100; the weight is
    rotated over copies larger than the Infinity Cache, as for the GEMV.
    Reported per M: time per call, algorithmic bytes (weight + x + out) per
    second and the fraction of the HBM peak, and the path taken.  Where
    tq2_gemm_workspace_bytes is nonzero (M = 100) the line times tq2_gemm_ws
    with its workspace (entry "tq2_gemm_ws"), and "m100_tq2_gemm" times
    tq2_gemm itself on the same inputs."""
    import numpy as np
    out_lines = {}
    c = G.config3(100)
    n, k = c["n"], c["k"]
    soa = tq2.reformat_aos_to_soa(torch.from_numpy(c["aos"]).to(dev), n, k)
    sb = tq2.soa_bytes(n, k)
    pool = max(1, int(math.ceil(args.pool_mib * 2 ** 20 / sb)))
    wpool = soa.repeat(pool)
    base = wpool.data_ptr()
    for key, m, use_ws in (("m7", 7, True), ("m8", 8, True), ("m9", 9, True), ("m100", 100, True),
                           ("m100_tq2_gemm", 100, False)):
        # config3(m)'s x is the first m rows of the same 100-row draw
        x = torch.from_numpy(np.ascontiguousarray(c["x"][:m])).to(dev)
        out = torch.empty((m, n), dtype=torch.float32, device=dev)
        need = tq2.gemm_workspace_bytes(m, n, k) if use_ws else 0
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def call(i, x=x, out=out, m=m, ws=ws, need=need):
            if need:
                st = tq2.gemm_ws_ptr(base + (i % pool) * sb, x.data_ptr(), 0, out.data_ptr(), m, n,
                                     k, ws.data_ptr(), need,
                                     torch.cuda.current_stream(dev).cuda_stream)
            else:
                st = tq2.gemm_ptr(base + (i % pool) * sb, x.data_ptr(), 0, out.data_ptr(), m, n, k,
                                  torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError("tq2_gemm failed: %s" % tq2.status_string(st))

        g = capture(torch, stream, call, pool)
        time_graph(torch, g, 1, stream)
        reps = max(1, int(math.ceil(args.steps / 8 / pool)))
        ms, _ = time_graph(torch, g, reps, stream)
        us = ms * 1e3 / (reps * pool)
        nbytes = n * (k // 128) * 34 + 4 * m * k + 4 * m * n
        gbs = nbytes / (us * 1e-6) / 1e9
        tflops = 2.0 * m * n * k / (us * 1e-6) / 1e12
        out_lines[key] = {"us_per_call": round(us, 3), "gbs": round(gbs, 2),
                          "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                          "tflops": round(tflops, 2),
                          "frac_of_f16_peak": round(tflops / F16_MFMA_PEAK_TFLOPS, 4),
                          "path": tq2.gemm_path(m, n, k), "calls": reps * pool,
                          "entry": "tq2_gemm_ws" if need else "tq2_gemm"}
        del g, ws
    del wpool
    return {"gemm_small_batch_k4096_n11008": out_lines}


def q1_bench(torch, tq2, G, dev, stream, args):
    """Q1_g128 (1-bit) sibling format on the same shapes as the TQ2 lines:
    decode GEMV M=1, K=N=4096 with residual (weight copies rotated past the
    Infinity Cache), and the M=1536, K=N=3072 GEMM."""
    c = G.q1_decode(True)
    n, k = c["n"], c["k"]
    soa = tq2.reformat_aos_to_soa(torch.from_numpy(c["aos"]).to(dev), n, k, fmt="q1")
    sb = tq2.q1_soa_bytes(n, k)
    pool = max(1, int(math.ceil(args.pool_mib * 2 ** 20 / sb)))
    pool_buf = soa.repeat(pool)
    base = pool_buf.data_ptr()
    x = torch.from_numpy(c["x"]).to(dev).reshape(-1)
    res = torch.from_numpy(c["residual"]).to(dev).reshape(-1)
    out = torch.empty(n, dtype=torch.float32, device=dev)

    def gemv_call(i):
        st = tq2.q1_gemv_ptr(base + (i % pool) * sb, x.data_ptr(), res.data_ptr(), out.data_ptr(),
                             n, k, torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError("tq2_q1_gemv failed: %s" % tq2.status_string(st))

    gg = capture(torch, stream, gemv_call, pool)
    time_graph(torch, gg, 2, stream)
    reps = max(1, int(math.ceil(args.steps / pool)))
    ms, _ = time_graph(torch, gg, reps, stream)
    us = ms * 1e3 / (reps * pool)
    nbytes = n * (k // 128) * 18 + 4 * k + 8 * n
    gbs = nbytes / (us * 1e-6) / 1e9
    del gg, pool_buf

    c4 = G.q1_gemm()
    m4, n4, k4 = c4["m"], c4["n"], c4["k"]
    soa4 = tq2.reformat_aos_to_soa(torch.from_numpy(c4["aos"]).to(dev), n4, k4, fmt="q1")
    x4 = torch.from_numpy(c4["x"]).to(dev)
    out4 = torch.empty((m4, n4), dtype=torch.float32, device=dev)

    def gemm_call(i):
        st = tq2.q1_gemm_ptr(soa4.data_ptr(), x4.data_ptr(), 0, out4.data_ptr(), m4, n4, k4,
                             torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError("tq2_q1_gemm failed: %s" % tq2.status_string(st))

    per_graph = 20
    g4 = capture(torch, stream, gemm_call, per_graph)
    time_graph(torch, g4, 2, stream)
    reps4 = max(1, args.gemm_reps // per_graph)
    ms4, _ = time_graph(torch, g4, reps4, stream)
    us4 = ms4 * 1e3 / (reps4 * per_graph)
    tflops = 2.0 * m4 * n4 * k4 / (us4 * 1e-6) / 1e12
    return {
        "q1_gemv_k4096_n4096_residual": {
            "gbs": round(gbs, 2), "us_per_call": round(us, 3), "bytes_per_call": nbytes,
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "calls": reps * pool},
        "q1_gemm_m1536_k3072_n3072": {
            "tflops": round(tflops, 2), "us_per_call": round(us4, 3),
            "peak_tflops": F16_MFMA_PEAK_TFLOPS, "frac": round(tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "path": tq2.gemm_path(m4, n4, k4), "calls": reps4 * per_graph},
    }


def main():
    global SETTLE_MS
    args = parse()
    SETTLE_MS = args.settle_ms
    if args.gpus != 1:
        print("bench.py: the library runs and is measured on one GPU; --gpus %d is not supported "
              "(run with --gpus 1)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import tq2_inputs as G
    from gemv_tq2_g128_amd import tq2

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    clock = ClockSampler(torch)

    # ---- decode GEMV, K = N = 4096, fused residual -------------------------
    case = G.config2(with_residual=True)
    n, k = case["n"], case["k"]
    nbytes = gemv_bytes(n, k, True)
    aos = torch.from_numpy(case["aos"]).to(dev)
    soa0 = tq2.reformat_aos_to_soa(aos, n, k)
    sb = tq2.soa_bytes(n, k)
    pool = max(1, int(math.ceil(args.pool_mib * 2 ** 20 / sb)))
    pool_buf = soa0.repeat(pool)                       # pool copies, sb bytes apart
    x = torch.from_numpy(case["x"]).to(dev).reshape(-1)
    res = torch.from_numpy(case["residual"]).to(dev).reshape(-1)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    base = pool_buf.data_ptr()

    def gemv_call(i):
        st = tq2.gemv_ptr(base + (i % pool) * sb, x.data_ptr(), res.data_ptr(), out.data_ptr(),
                          n, k, torch.cuda.current_stream(dev).cuda_stream)
        if st != 0:
            raise RuntimeError("tq2_gemv failed: %s" % tq2.status_string(st))

    # Exactly `warmup` untimed calls, then exactly `steps` timed ones; call i
    # reads weight copy i % pool, so consecutive calls read different copies.
    # The warm-up calls run right before the start event, with the timed calls
    # already queued behind them (time_graphs).
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    warm = exact_graphs(torch, stream, gemv_call, warmup) if warmup else []
    timed = exact_graphs(torch, stream, gemv_call, steps)
    with clock.phase("headline_gemv"):
        ms, wall = time_graphs(torch, timed, stream, warm=warm)
    del timed, warm
    us_per_call = ms * 1e3 / steps
    gbs = nbytes / (us_per_call * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode GEMV M=1 K=4096 N=4096 with fused residual; weight "
                               "rotated over %d copies (%.0f MiB) so every call reads HBM; "
                               "calls replayed back to back from a HIP graph" %
                               (pool, pool * sb / 2 ** 20),
                   "m": 1, "n": n, "k": k, "bytes_per_call": nbytes,
                   "wall_s_timed": round(wall, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gemv_traffic_bytes_per_launch",
                                                 "gemv_tq2_g128_amd/csrc/tq2_gemv.hip"),
                     "traffic_unit": "bytes per launch", "kernel": "gemv_kernel",
                     "us_per_launch": round(us_per_call, 3)},
    }

    # ---- what one launch of the GEMV's grid costs, and a plain read of the
    # same bytes in one such launch (reference kernels, not the library) -------
    floor = launch_floor(torch, dev, stream, base, pool, sb, (n + 7) // 8, steps)
    if floor is not None:
        floor["gemv_us_per_launch"] = round(us_per_call, 3)
        result["launch_floor_k4096_n4096"] = floor

    # ---- batched decode GEMV: 16 K = N = 4096 weights per call ----------------
    if not args.no_batched:
        nb = 16
        calls = max(1, pool // nb)
        outs = torch.empty((nb, n), dtype=torch.float32, device=dev)
        ress = res.repeat(nb).reshape(nb, n)

        def batched_call(i):
            probs = [(base + ((i * nb + j) % pool) * sb, x.data_ptr(), ress[j].data_ptr(),
                      outs[j].data_ptr(), n, k) for j in range(nb)]
            st = tq2.gemv_batched_ptr(probs, torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError("tq2_gemv_batched failed: %s" % tq2.status_string(st))

        gb = capture(torch, stream, batched_call, calls)
        time_graph(torch, gb, 2, stream)
        reps = max(1, int(math.ceil(args.steps / (calls * nb))))
        msb, _ = time_graph(torch, gb, reps, stream)
        usb = msb * 1e3 / (reps * calls)
        gbs_b = nb * nbytes / (usb * 1e-6) / 1e9
        result["gemv_batched_16x4096x4096"] = {
            "gbs": round(gbs_b, 2), "us_per_call": round(usb, 3), "weights_per_call": nb,
            "bytes_per_call": nb * nbytes, "frac_of_hbm_peak": round(gbs_b / HBM_PEAK_GBS, 4),
            "calls": reps * calls,
            "traffic": measured_traffic("gemv_batched_traffic_bytes_per_launch",
                                        "gemv_tq2_g128_amd/csrc/tq2_gemv.hip")}

    # ---- large-M GEMM, M = 1536, K = N = 3072 --------------------------------
    if not args.no_gemm:
        c4 = G.config4()
        m4, n4, k4 = c4["m"], c4["n"], c4["k"]
        soa4 = tq2.reformat_aos_to_soa(torch.from_numpy(c4["aos"]).to(dev), n4, k4)
        x4 = torch.from_numpy(c4["x"]).to(dev)
        out4 = torch.empty((m4, n4), dtype=torch.float32, device=dev)

        def gemm_call(i):
            st = tq2.gemm_ptr(soa4.data_ptr(), x4.data_ptr(), 0, out4.data_ptr(), m4, n4, k4,
                              torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError("tq2_gemm failed: %s" % tq2.status_string(st))

        per_graph = 20
        g4 = capture(torch, stream, gemm_call, per_graph)
        time_graph(torch, g4, 2, stream)
        reps = max(1, args.gemm_reps // per_graph)
        ms4, _ = time_graph(torch, g4, reps, stream)
        us4 = ms4 * 1e3 / (reps * per_graph)
        tflops = 2.0 * m4 * n4 * k4 / (us4 * 1e-6) / 1e12
        def precise_call(i):
            st = tq2.gemm_precise_ptr(soa4.data_ptr(), x4.data_ptr(), 0, out4.data_ptr(), m4, n4,
                                      k4, torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError("tq2_gemm_precise failed: %s" % tq2.status_string(st))

        # The clock level during a long run of the same calls (about 100 ms;
        # the timed region above is too short to sample).
        with clock.phase("gemm_m1536_k3072_n3072"):
            time_graph(torch, g4, max(1, int(0.1 / (us4 * 1e-6) / per_graph)), stream)
        gp = capture(torch, stream, precise_call, per_graph)
        time_graph(torch, gp, 1, stream)
        msp, _ = time_graph(torch, gp, max(1, reps // 2), stream)
        usp = msp * 1e3 / (max(1, reps // 2) * per_graph)
        result["gemm_precise_m1536_k3072_n3072"] = {
            "tflops": round(2.0 * m4 * n4 * k4 / (usp * 1e-6) / 1e12, 2),
            "us_per_call": round(usp, 3), "path": 1, "tolerance": "1e-5 * sum|x w|"}
        result["gemm_m1536_k16384_n3072"] = gemm_shape_bench(torch, tq2, G, dev, stream,
                                                             1536, 3072, 16384, args)
        result["gemm_m1536_k3072_n3072"] = {
            "tflops": round(tflops, 2), "us_per_call": round(us4, 3),
            "peak_tflops": F16_MFMA_PEAK_TFLOPS, "frac": round(tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "path": tq2.gemm_path(m4, n4, k4), "calls": reps * per_graph,
            "traffic": measured_traffic("gemm_traffic_bytes_per_launch",
                                        "gemv_tq2_g128_amd/csrc/tq2_gemm.hip")}

    result.update(config1_bench(torch, tq2, G, dev, stream, args))

    if not args.no_sweep:
        result.update(gemv_sweep(torch, tq2, G, dev, stream, args))

    if not args.no_small_batch:
        result.update(small_batch_bench(torch, tq2, G, dev, stream, args))

    if not args.no_swiglu:
        result.update(swiglu_bench(torch, tq2, G, dev, stream, args))

    if not args.no_q1:
        result.update(q1_bench(torch, tq2, G, dev, stream, args))

    if not args.no_chain:
        with clock.phase("chain_100_layers_m1536"):
            result["chain_100_layers_m1536"] = chain_bench(torch, tq2, G, dev, stream)

    if args.calibrate_copy_mib > 0:
        nb = args.calibrate_copy_mib * 2 ** 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = nb

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)

    result["environment"] = run_environment(torch)
    result["environment"]["gfx_clock_in_use"] = clock.report()

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
