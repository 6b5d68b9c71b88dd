#!/usr/bin/env python3
"""Benchmark of the TQ2_0_g128 ternary matmul on one MI355X.

Headline (one JSON line on stdout): the decode GEMV M=1, K=N=4096 with the
fused residual (out = residual + x . W^T), one ``tq2_gemv`` call per step,
as achieved HBM GB/s of algorithmic bytes (codes + scales + x + residual +
out, each counted once).  The weight of every call comes from a pool of
copies larger than the 256 MB Infinity Cache, so each call streams its
weight from HBM; the calls are replayed back to back from a HIP graph.

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


def gemv_bytes(n, k, residual):
    codes_scales = n * (k // 128) * 34
    return codes_scales + 4 * k + 4 * n + (4 * n if residual else 0)


def time_graph(torch, graph, replays, stream):
    """Replay a captured graph ``replays`` times between two events on the
    stream the kernels run on; returns (event ms, wall s)."""
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(replays):
            graph.replay()
        end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end), wall


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


def time_graphs(torch, graphs, stream):
    """Replay [(graph, replays)] back to back between two events on the stream
    the kernels run on; returns (event ms, wall s)."""
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        for graph, replays in graphs:
            for _ in range(replays):
                graph.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end), time.perf_counter() - t0


def cpu_baseline(case, seconds):
    """The oracle as it stands, on the host, single BLAS thread."""
    from threadpoolctl import threadpool_limits
    import oracle
    n, k = case["n"], case["k"]
    nbytes = gemv_bytes(n, k, case["residual"] is not None)
    with threadpool_limits(limits=1):
        oracle.matmul(case["aos"], case["x"], n, k, case["residual"])    # warm
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            oracle.matmul(case["aos"], case["x"], n, k, case["residual"])
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full oracle evaluations of the K=N=4096 residual GEMV (float64 numpy "
                      "dequantize + product, 1 BLAS thread), %.3f s each" % (reps, dt)}


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
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
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
        time_graphs(torch, exact_graphs(torch, stream, fn, min(steps, 512)), stream)
        ms, _ = time_graphs(torch, exact_graphs(torch, stream, fn, steps), stream)
        out[name + "_us_per_launch"] = round(ms * 1e3 / steps, 3)
    out["read_gbs"] = round(sb / (out["read_us_per_launch"] * 1e-6) / 1e9, 2)
    return out


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
    second and the fraction of the HBM peak, and the path taken."""
    import numpy as np
    out_lines = {}
    c = G.config3(100)
    n, k = c["n"], c["k"]
    soa = tq2.reformat_aos_to_soa(torch.from_numpy(c["aos"]).to(dev), n, k)
    sb = tq2.soa_bytes(n, k)
    pool = max(1, int(math.ceil(args.pool_mib * 2 ** 20 / sb)))
    wpool = soa.repeat(pool)
    base = wpool.data_ptr()
    for m in (7, 8, 9, 100):
        # config3(m)'s x is the first m rows of the same 100-row draw
        x = torch.from_numpy(np.ascontiguousarray(c["x"][:m])).to(dev)
        out = torch.empty((m, n), dtype=torch.float32, device=dev)

        def call(i, x=x, out=out, m=m):
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
        out_lines["m%d" % m] = {"us_per_call": round(us, 3), "gbs": round(gbs, 2),
                                "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                                "tflops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 2),
                                "path": tq2.gemm_path(m, n, k), "calls": reps * pool}
        del g
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
    args = parse()
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
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    if warmup:
        warm = exact_graphs(torch, stream, gemv_call, warmup)
        time_graphs(torch, warm, stream)
        del warm
    timed = exact_graphs(torch, stream, gemv_call, steps)
    ms, wall = time_graphs(torch, timed, stream)
    del timed
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

        gp = capture(torch, stream, precise_call, per_graph)
        time_graph(torch, gp, 1, stream)
        msp, _ = time_graph(torch, gp, max(1, reps // 2), stream)
        usp = msp * 1e3 / (max(1, reps // 2) * per_graph)
        result["gemm_precise_m1536_k3072_n3072"] = {
            "tflops": round(2.0 * m4 * n4 * k4 / (usp * 1e-6) / 1e12, 2),
            "us_per_call": round(usp, 3), "path": 1, "tolerance": "1e-5 * sum|x w|"}
        result["gemm_m1536_k3072_n3072"] = {
            "tflops": round(tflops, 2), "us_per_call": round(us4, 3),
            "peak_tflops": F16_MFMA_PEAK_TFLOPS, "frac": round(tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "path": tq2.gemm_path(m4, n4, k4), "calls": reps * per_graph,
            "traffic": measured_traffic("gemm_traffic_bytes_per_launch",
                                        "gemv_tq2_g128_amd/csrc/tq2_gemm.hip")}

    if not args.no_sweep:
        result.update(gemv_sweep(torch, tq2, G, dev, stream, args))

    if not args.no_small_batch:
        result.update(small_batch_bench(torch, tq2, G, dev, stream, args))

    if not args.no_swiglu:
        result.update(swiglu_bench(torch, tq2, G, dev, stream, args))

    if not args.no_q1:
        result.update(q1_bench(torch, tq2, G, dev, stream, args))

    if not args.no_chain:
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

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
