"""Throughput of the BitLinear (W1.58A8) forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the per-token hot path over one 2B-class decoder layer
at T = 1: for each of its seven projections (q, k, v, o: 2560->2560/640;
gate, up: 2560->6912; down: 6912->2560) the bf16 activation is quantised to
int8 and contracted with the 2-bit packed ternary weights, then rescaled.
The projections run as four launches in the order a decoder layer needs
them -- [q, k, v], [o], [gate, up], [down] -- each one call of
bitlinear_linear_grouped (act-quant fused into the decode GEMV kernel).
Weights are packed once at set-up (step A0 is an offline conversion) and then
copied to L distinct layer sets (> 1 GB in total, four times the 256 MB MALL),
and consecutive steps rotate through them, so every step streams its weights
from HBM.  The timed steps replay a HIP graph of L consecutive steps.  The
same layer as 14 separate launches (act-quant, then forward, per projection)
is reported beside it.

The JSON line reports algorithmic GB/s of the whole step (value), the decode
kernel against the HBM roofline, the CPU oracle timed on a bounded sample,
and, as extra context: the device's measured ceilings (launch floor, HBM read
stream, int8 matrix-core loop), the spread of the step time, the prefill GEMM
(T = 2048) in int8 TOP/s, the batched decode crossover between the decode
kernel and the tiled MFMA kernel, the 70B-class shapes at T = 1 (GB/s)
and T = 256 (TOP/s), and the 3B-class layer (decode GB/s, prefill TOP/s).
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, TOP/s
ROT_BYTES = 1.1e9               # packed weights rotated through per pass


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=4096)
    p.add_argument("--warmup", type=int, default=256)
    p.add_argument("--cpu-budget", type=float, default=6.0,
                   help="seconds of the CPU oracle's headline sample (the per-workload "
                        "breakdown adds about 20-30 s)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extra", action="store_true", help="skip the prefill GEMM context run")
    p.add_argument("--profile-prefill", action="store_true",
                   help="run act-quant + the tiled MFMA kernel on both T=2048 prefill shapes "
                        "five times each (eager), then a 256 MiB device copy, and exit: the "
                        "program that the prefill rocprofv3 summaries profile")
    p.add_argument("--extra", default="all",
                   help="context runs to do: 'all' or a comma list of calib, toy, prefill, "
                        "crossover, 70b, 3b, subln, gated, lut, binary, pack")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (HBM counter calibration)")
    p.add_argument("--fused-only", action="store_true",
                   help="time only the fused layer steps (a kernel trace of this run holds "
                        "nothing but the roofline kernel's launches)")
    p.add_argument("--profile-pass", action="store_true",
                   help="counter runs: two eager passes of the fused steps over the layer "
                        "sets plus the copy calibration, no timing and no JSON")
    return p.parse_args()


def fused_bytes(t, n, k, in_bytes=2):
    """Algorithmic bytes of one problem of a fused launch: packed W, raw x and
    gamma in; fp32 y, int8 x and absmax out."""
    return n * k // 4 + in_bytes * t * k + 4 + 4 * t * n + t * k + 4 * t


def gemv_bytes(t, n, k):
    """Algorithmic bytes of one forward launch: packed W, int8 x, absmax, gamma, fp32 y."""
    return n * k // 4 + t * k + 4 * t + 4 + 4 * t * n


def quant_bytes(t, k, in_bytes=2):
    """Algorithmic bytes of one act-quant launch: x in, int8 x, absmax, rowsum out."""
    return in_bytes * t * k + t * k + 8 * t


def kernel_src_hash(name):
    path = os.path.join(ROOT, "bitlinear_w1_a8_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(kernel_file, key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only
    while the kernel source still hashes to what was profiled."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_src_hash(kernel_file):
        return None
    return rec.get("bytes_per_launch")


class Calls:
    """Direct C-ABI calls with pre-built pointer arguments (no per-call torch work)."""

    def __init__(self, lib):
        self.lib = lib

    def quant(self, x, xq, absmax, t, k, stream, rowsum=None):
        rc = self.lib.bitlinear_quant_act(x, 1, t, k, xq, absmax, rowsum, stream)
        if rc:
            raise RuntimeError(self.lib.bitlinear_last_error().decode())

    def forward(self, packed, gamma, xq, absmax, t, n, k, y, algo, stream, rowsum=None):
        rc = self.lib.bitlinear_forward_algo(packed, gamma, xq, absmax, rowsum, t, n, k, y, None,
                                             algo, stream)
        if rc:
            raise RuntimeError(self.lib.bitlinear_last_error().decode())

    def grouped(self, descs, t, stream):
        rc = self.lib.bitlinear_linear_grouped(descs, len(descs), t, 1, stream)
        if rc:
            raise RuntimeError(self.lib.bitlinear_last_error().decode())


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def decode_setup(torch, binding, wl, dev):
    """Seeded weights and activations of the 2B decode layer, packed on the GPU."""
    wk = wl.WORKLOADS[2]
    mats = []
    pack_ms = []
    for mi, m in enumerate(wk.matrices):
        w = torch.from_numpy(wk.weights(mi)).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        packed, gamma = binding.pack_weights(w)
        torch.cuda.synchronize()
        pack_ms.append((time.perf_counter() - t0) * 1e3)
        del w
        bits = wl.bf16_bits(wk.activations(mi, 1))
        x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        mats.append(dict(m=m, packed=packed, gamma=gamma, x=x,
                         xq=torch.empty((1, m.k), dtype=torch.int8, device=dev),
                         absmax=torch.empty(1, dtype=torch.float32, device=dev),
                         y=torch.empty((1, m.n), dtype=torch.float32, device=dev)))
    layer_bytes = sum(d["packed"].numel() for d in mats)
    n_sets = int(np.ceil(ROT_BYTES / layer_bytes))
    sets = [[d["packed"] for d in mats]]
    for _ in range(n_sets - 1):
        sets.append([d["packed"].clone() for d in mats])
    torch.cuda.synchronize()
    return mats, sets, pack_ms


def capture(torch, fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn(stream)  # one eager pass before capture
    stream.synchronize()
    with torch.cuda.graph(g, stream=stream):
        fn(stream)
    return g


def time_graph(torch, g, reps, warm, stream):
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(reps):
            g.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end)  # ms


def calibration(torch, binding, dev, stream):
    """The device's own ceilings, measured with the library's helper kernels:
    the launch floor (an empty kernel per graph node), the HBM read stream
    (one 70B-class packed matrix per launch over 20 rotated buffers, as the
    decode kernels stream their weights, and one 1 GiB buffer, both read at
    full width, the better of two load layouts) and the
    int8 matrix-core rate (back-to-back v_mfma_i32_32x32x32_i8 on registers,
    four waves per SIMD)."""
    lib = binding.load()
    h = lambda s: ctypes.c_void_p(s.cuda_stream)

    def ok(rc):
        if rc:
            raise RuntimeError(lib.bitlinear_last_error().decode())

    out = {}
    n = 256
    g = capture(torch, lambda s: [ok(lib.bitlinear_calib_empty(h(s))) for _ in range(n)], stream)
    out["empty_kernel_launch_us"] = round(time_graph(torch, g, 8, 2, stream) * 1e3 / (8 * n), 3)
    sink = torch.empty(lib.bitlinear_calib_sink_len(), dtype=torch.int32, device=dev)
    # reads of one 70B-class packed matrix (58.7 MB), rotated over 20 buffers
    # (> 1 GB, four times the MALL) as the decode kernels' weights are, and
    # one read of 1 GiB, each in the helper's two layouts (contiguous chunks
    # per block, grid-stride).  Which layout reads faster depends on the
    # buffer size on this device (a grid-stride loop puts its loads in flight
    # a power of two apart and slows down on buffers of 64 MiB and more), so
    # the ceiling is the better of the two, taken at the size the decode
    # kernels stream.
    for nbytes, copies, key in ((58720256, 20, "hbm_read_stream_70b_matrix_rotated"),
                                (1 << 30, 1, "hbm_read_stream_1gib")):
        bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device=dev) for _ in range(copies)]
        best = 0.0
        for layout, name in ((0, "chunks"), (1, "stride")):
            us = rotated_time_us(
                torch, lambda s, i: ok(lib.bitlinear_calib_read(ptr(bufs[i]), nbytes, layout,
                                                                ptr(sink), h(s))),
                copies, stream, reps=max(2, 20 // copies))
            out[f"{key}_{name}_gb_s"] = round(nbytes / us / 1e3, 1)
            best = max(best, nbytes / us / 1e3)
        out[key + "_gb_s"] = round(best, 1)
        out[key + "_frac_of_peak"] = round(best / HBM_PEAK_GBS, 4)
        del bufs
    iters = 1024
    g = capture(torch, lambda s: ok(lib.bitlinear_calib_mfma(iters, 1, ptr(sink), h(s))), stream)
    us = time_graph(torch, g, 10, 2, stream) * 1e3 / 10
    ops = 2.0 * 4 * iters * 4096 * 32768
    out["int8_mfma_loop_tops"] = round(ops / us / 1e6, 1)
    out["int8_mfma_loop_frac_of_peak"] = round(ops / us / 1e6 / INT8_PEAK_TOPS, 4)
    torch.cuda.empty_cache()
    return out


def time_plan(torch, timed, warm, stream):
    """Milliseconds for replaying the graphs of `timed` in order, after the
    graphs of `warm` (untimed), from HIP events on `stream` bracketed by
    device synchronisations."""
    for g in warm:
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for g in timed:
            g.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def time_graph_chunks(torch, g, reps, chunks, stream):
    """Milliseconds per replay in each of `chunks` consecutive timed runs."""
    per = max(1, reps // chunks)
    out = []
    for _ in range(chunks):
        out.append(time_graph(torch, g, per, 0, stream) / per)
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, min_s):
    """Seconds per call of fn(), repeating until min_s have passed (at least once)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return el / n


def cpu_baseline(oracle, wl, budget_s=12.0):
    """The oracle as it stands, timed on the host per workload and per step.

    Step A0 (pack: exact gamma by math.fsum, ternarise, 2-bit pack) is timed
    on the first rows of each matrix (about 2M weights) and reported per
    weight; step A1 (act-quant) on the workload's full activations; steps
    A2 + A3 (contract in binary64, rescale) on the first rows of the matrix
    (at most 2^25 weights) and reported per 1000 rows and as rates.  The headline value is the 2B decode layer (7 projections,
    T = 1: act-quant + contract + rescale) in algorithmic GB/s on every core
    the process may use, as many whole layers as fit budget_s; the same on
    one core (BLAS limited to one thread) beside it."""
    from threadpoolctl import threadpool_info, threadpool_limits

    cores_avail = len(os.sched_getaffinity(0))
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])

    def layer_prep():
        wk = wl.WORKLOADS[2]
        tern, xs, gammas = [], [], []
        for mi, m in enumerate(wk.matrices):
            w = wk.weights(mi)
            g = oracle.absmean_gamma(w)
            tern.append(oracle.ternarize(w, g))
            gammas.append(g)
            xs.append(wl.bf16_bits(wk.activations(mi, 1)))
        return wk, tern, xs, gammas

    wk, tern, xs, gammas = layer_prep()

    def layer():
        for mi in range(len(wk.matrices)):
            q, a, _ = oracle.quant_act(xs[mi])
            acc = oracle.contract(q, tern[mi])
            oracle.rescale(acc, gammas[mi], a)

    step_bytes = sum(fused_bytes(1, m.n, m.k) for m in wk.matrices)
    layers, t0 = 0, time.perf_counter()
    while True:
        layer()
        layers += 1
        el = time.perf_counter() - t0
        if el >= budget_s or layers >= 200:
            break
    value = step_bytes * layers / el / 1e9
    with threadpool_limits(limits=1):
        s1 = _timed(layer, 2.0)
    value_1 = step_bytes / s1 / 1e9

    # per workload and per step, all cores, on bounded slices: step A0 on
    # about 2M weights of each matrix, steps A1-A3 on the first rows of the
    # matrix (at most 2^25 weights) against the workload's full activations
    by_cfg = {}
    for idx, wkl in sorted(wl.WORKLOADS.items()):
        rec = {}
        for mi, m in enumerate(wkl.matrices):
            seed = wl.seed_of(idx, mi, False)
            rows_pack = min(m.n, max(16, (1 << 21) // m.k))
            w_pack = wl.latent_weights(rows_pack, m.k, wkl.sigma, seed)   # the matrix's first rows
            sp = _timed(lambda: oracle.pack_weights(w_pack), 0.3)
            rows = min(m.n, max(16, (1 << 25) // m.k))
            w = wl.latent_weights(rows, m.k, wkl.sigma, seed)
            g = oracle.absmean_gamma(w_pack)
            t_rows = oracle.ternarize(w, g)
            del w, w_pack
            for t in wkl.tokens:
                x = wkl.activations(mi, t)
                xin = wl.bf16_bits(x) if wkl.x_dtype == "bf16" else x
                sq = _timed(lambda: oracle.quant_act(xin), 0.2)
                q, a, _ = oracle.quant_act(xin)
                sf = _timed(lambda: oracle.rescale(oracle.contract(q, t_rows), g, a), 0.3)
                fb = gemv_bytes(t, rows, m.k)
                rec[f"{m.name}_{m.k}->{m.n}_T{t}"] = {
                    "pack_ns_per_weight": round(sp / (rows_pack * m.k) * 1e9, 2),
                    "act_quant_ms": round(sq * 1e3, 3),
                    "forward_rows_timed": rows,
                    "forward_ms_per_1k_rows": round(sf * 1e3 * 1000 / rows, 3),
                    "forward_gb_s": round(fb / sf / 1e9, 3),
                    "forward_gop_s": round(2.0 * t * rows * m.k / sf / 1e9, 2)}
            del t_rows
        by_cfg[f"{idx}_{wkl.name}"] = rec
    return {"value": value, "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{layers} decode layers (7 projections, T=1, act-quant + contract + "
                      f"rescale) in {el:.1f} s; weights ternarised beforehand; the contraction "
                      f"converts the ternary matrix to binary64 on every call, as the oracle does",
            "cpu_model": _cpu_model(), "cores_available": cores_avail,
            "value_1_core": round(value_1, 4),
            "by_workload_all_cores": by_cfg,
            "context_not_target": {
                "pages_cpu_decode_ms_per_token_2b": 29,
                "pages_cpu_decode_hardware": "Intel i7-13800H, 8 threads (2B4T report summary, "
                                             "section 4.1)",
                "pages_bitnet_cpp_x86_speedup": "2.37-6.17x over llama.cpp "
                                                "(bitnet.cpp post, section 2.3)"}}


def rotated_time_us(torch, body, n, stream, reps=10):
    """Microseconds per call of body(stream, i) for i over n rotated copies,
    from HIP events over graph replays of all n calls."""
    g = capture(torch, lambda s: [body(s, i) for i in range(n)], stream)
    return time_graph(torch, g, reps, 2, stream) * 1e3 / (reps * n)


def pack_extra(torch, binding, dev, stream):
    """Step A0 on the device: bitlinear_pack_weights on seeded fp32 latent
    weights (N(0, 0.02)) of the 2B and 70B-class shapes, microseconds per
    call from HIP events around ten eager calls (the buckets zeroed, the
    exact histogram of |w|, gamma, then ternarise and pack).  GB/s counts one
    read of W plus the packed write against the 8 TB/s peak; gamma has to be
    known before any weight is rounded, so the method reads W twice, and the
    two-read figure is given beside it."""
    lib = binding.load()
    out = {}
    shapes = ((2560, 2560), (2560, 640), (2560, 6912), (6912, 2560), (8192, 28672), (28672, 8192))
    for k, n in shapes:
        gen = torch.Generator(device=dev)
        gen.manual_seed(8000 + n + k)
        w = torch.randn((n, k), device=dev, generator=gen) * 0.02
        packed = torch.empty((n, k // 4), dtype=torch.uint8, device=dev)
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(int(lib.bitlinear_pack_workspace_bytes(n, k)), dtype=torch.uint8, device=dev)
        h = ctypes.c_void_p(stream.cuda_stream)

        def call():
            rc = lib.bitlinear_pack_weights(ptr(w), n, k, ptr(packed), ptr(gamma), ptr(ws), ws.numel(), h)
            if rc:
                raise RuntimeError(lib.bitlinear_last_error().decode())

        with torch.cuda.stream(stream):
            for _ in range(3):
                call()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            best = float("inf")
            for _ in range(3):
                e0.record(stream)
                for _ in range(10):
                    call()
                e1.record(stream)
                e1.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1e3 / 10)
        one = 4.0 * n * k + n * k / 4 + 4
        two = 8.0 * n * k + n * k / 4 + 4
        out[f"{k}->{n}"] = {"pack_us": round(best, 1),
                            "gb_s_one_read": round(one / best / 1e3, 1),
                            "frac_of_hbm_peak_one_read": round(one / best / 1e3 / HBM_PEAK_GBS, 4),
                            "gb_s_two_reads": round(two / best / 1e3, 1)}
        del w, packed
        torch.cuda.empty_cache()
    return out


def subln_extra(torch, binding, dev, stream):
    """The sub-layer norm fused with act-quant against act-quant alone: bf16
    rows of K in {2560, 6912} at T in {1, 2048}, over 64 distinct activation
    buffers per graph; GB/s of algorithmic bytes (x and gain in, int8 codes,
    scale and row sum out) against the 8 TB/s HBM peak."""
    lib = binding.load()
    out = {}
    for t, k in ((1, 2560), (1, 6912), (2048, 2560), (2048, 6912)):
        n = 64 if t == 1 else 8
        gen = torch.Generator(device=dev)
        gen.manual_seed(7000 + t + k)
        xs = [torch.randn((t, k), device=dev, generator=gen).to(torch.bfloat16) for _ in range(n)]
        gain = (1.0 + 0.3 * torch.randn(k, device=dev, generator=gen)).float()
        xq = torch.empty((t, k), dtype=torch.int8, device=dev)
        sc = torch.empty(t, dtype=torch.float32, device=dev)
        rs = torch.empty(t, dtype=torch.int32, device=dev)

        def norm(s, i):
            rc = lib.bitlinear_subln_quant_act(ptr(xs[i]), 1, ptr(gain), 1e-5, t, k, ptr(xq), ptr(sc),
                                               ptr(rs), ctypes.c_void_p(s.cuda_stream))
            if rc:
                raise RuntimeError(lib.bitlinear_last_error().decode())

        def plain(s, i):
            rc = lib.bitlinear_quant_act(ptr(xs[i]), 1, t, k, ptr(xq), ptr(sc), ptr(rs),
                                         ctypes.c_void_p(s.cuda_stream))
            if rc:
                raise RuntimeError(lib.bitlinear_last_error().decode())

        us_n = rotated_time_us(torch, norm, n, stream)
        us_p = rotated_time_us(torch, plain, n, stream)
        byts = 2 * t * k + 4 * k + t * k + 8 * t
        out[f"T{t}_K{k}"] = {"subln_quant_us": round(us_n, 2),
                             "subln_quant_gb_s": round(byts / us_n / 1e3, 1),
                             "subln_frac_of_hbm_peak": round(byts / us_n / 1e3 / HBM_PEAK_GBS, 4),
                             "act_quant_alone_us": round(us_p, 2)}
        del xs
    return out


def toy_extra(torch, binding, wl, dev, stream):
    """The toy workload (T = 4, K = 256 -> N = 512, fp32 activations with
    outliers): the fused grouped call (act-quant inside the decode kernel)
    and act-quant + forward as two launches, over 64 copies of the packed
    matrix (2 MB in all, so the weights stay in the device caches: a latency
    figure, not a bandwidth one)."""
    wk = wl.WORKLOADS[1]
    m = wk.matrices[0]
    t = wk.tokens[0]
    lib = binding.load()
    calls = Calls(lib)
    packed, gamma = binding.pack_weights(torch.from_numpy(wk.weights(0)).to(dev))
    copies = [packed] + [packed.clone() for _ in range(63)]
    x = torch.from_numpy(wk.activations(0, t)).to(dev)
    xq = torch.empty((t, m.k), dtype=torch.int8, device=dev)
    am = torch.empty(t, dtype=torch.float32, device=dev)
    rs = torch.empty(t, dtype=torch.int32, device=dev)
    y = torch.empty((t, m.n), dtype=torch.float32, device=dev)
    descs = []
    for c in copies:
        arr = (binding.BlLinear * 1)()
        arr[0] = binding.BlLinear(x.data_ptr(), c.data_ptr(), gamma.data_ptr(), m.n, m.k,
                                  y.data_ptr(), xq.data_ptr(), am.data_ptr(), None)
        descs.append(arr)

    def fused(s, i):
        rc = lib.bitlinear_linear_grouped(descs[i], 1, t, 0, ctypes.c_void_p(s.cuda_stream))
        if rc:
            raise RuntimeError(lib.bitlinear_last_error().decode())

    def two(s, i):
        h = ctypes.c_void_p(s.cuda_stream)
        rc = lib.bitlinear_quant_act(ptr(x), 0, t, m.k, ptr(xq), ptr(am), ptr(rs), h)
        if rc:
            raise RuntimeError(lib.bitlinear_last_error().decode())
        calls.forward(ptr(copies[i]), ptr(gamma), ptr(xq), ptr(am), t, m.n, m.k, ptr(y), 0, h,
                      ptr(rs))

    us_f = rotated_time_us(torch, fused, len(copies), stream)
    us_2 = rotated_time_us(torch, two, len(copies), stream)
    byts = fused_bytes(t, m.n, m.k, in_bytes=4)
    return {"fused_us": round(us_f, 2), "fused_gb_s": round(byts / us_f / 1e3, 1),
            "act_quant_plus_forward_us": round(us_2, 2), "weights": "64 copies, cache-resident"}


def big_extra(torch, binding, wl, dev, stream):
    """Context: the 70B-class shapes (8192->28672, 28672->8192) at T = 1
    (GB/s of act-quant fused with the decode kernel, and of the decode kernel
    alone on int8 input) and at T = 256 (TOP/s of act-quant + tiled MFMA
    kernel), weights rotated over > 1 GB.  The latent weights are drawn on the
    GPU (N(0, 0.01), seeded) and packed there: only their code distribution
    matters for the timing."""
    wk = wl.WORKLOADS[5]
    lib = binding.load()
    calls = Calls(lib)
    out = {}
    for mi, m in enumerate(wk.matrices):
        gen = torch.Generator(device=dev)
        gen.manual_seed(5000 + mi)
        w = torch.randn((m.n, m.k), device=dev, generator=gen) * 0.01
        packed, gamma = binding.pack_weights(w)
        del w
        copies = [packed] + [packed.clone() for _ in range(int(np.ceil(ROT_BYTES / packed.numel())) - 1)]
        rec = {"rotated_copies": len(copies)}
        for t in (1, 256):
            xg = torch.Generator(device=dev)
            xg.manual_seed(6000 + 10 * mi + t)
            x = torch.randn((t, m.k), device=dev, generator=xg).to(torch.bfloat16)
            xq = torch.empty((t, m.k), dtype=torch.int8, device=dev)
            am = torch.empty(t, dtype=torch.float32, device=dev)
            rs = torch.empty(t, dtype=torch.int32, device=dev)
            y = torch.empty((t, m.n), dtype=torch.float32, device=dev)
            descs = []
            for c in copies:
                arr = (binding.BlLinear * 1)()
                arr[0] = binding.BlLinear(x.data_ptr(), c.data_ptr(), gamma.data_ptr(), m.n, m.k,
                                          y.data_ptr(), xq.data_ptr(), am.data_ptr(), None)
                descs.append(arr)
            P = [ptr(c) for c in copies]
            us_grp = rotated_time_us(
                torch, lambda s, i: calls.grouped(descs[i], t, ctypes.c_void_p(s.cuda_stream)),
                len(copies), stream)
            calls.quant(ptr(x), ptr(xq), ptr(am), t, m.k, ctypes.c_void_p(stream.cuda_stream),
                        ptr(rs))
            us_fwd = rotated_time_us(
                torch, lambda s, i: calls.forward(P[i], ptr(gamma), ptr(xq), ptr(am), t, m.n, m.k,
                                                  ptr(y), 0, ctypes.c_void_p(s.cuda_stream)),
                len(copies), stream)
            # the same with the tokens' row sums handed in (no sum-of-q pass in the kernel)
            us_rs = rotated_time_us(
                torch, lambda s, i: calls.forward(P[i], ptr(gamma), ptr(xq), ptr(am), t, m.n, m.k,
                                                  ptr(y), 0, ctypes.c_void_p(s.cuda_stream),
                                                  ptr(rs)),
                len(copies), stream)
            if t == 1:
                rec["t1_act_quant_plus_forward_us"] = round(us_grp, 2)
                rec["t1_act_quant_plus_forward_gb_s"] = round(fused_bytes(1, m.n, m.k) / us_grp / 1e3, 1)
                rec["t1_forward_us"] = round(us_fwd, 2)
                rec["t1_forward_gb_s"] = round(gemv_bytes(1, m.n, m.k) / us_fwd / 1e3, 1)
                rec["t1_forward_frac_of_hbm_peak"] = round(gemv_bytes(1, m.n, m.k) / us_fwd / 1e3 / HBM_PEAK_GBS, 4)
                rec["t1_forward_rowsum_given_us"] = round(us_rs, 2)
            else:
                ops = 2.0 * t * m.n * m.k
                rec["t256_act_quant_plus_forward_us"] = round(us_grp, 2)
                rec["t256_forward_us"] = round(us_fwd, 2)
                rec["t256_forward_tops"] = round(ops / us_fwd / 1e6, 1)
                rec["t256_forward_frac_of_int8_peak"] = round(ops / us_fwd / 1e6 / INT8_PEAK_TOPS, 4)
                rec["t256_forward_rowsum_given_us"] = round(us_rs, 2)
        # small batches of int8 tokens (the persistent kernel takes up to
        # four over rows of up to 8192; longer rows stage up to 128 KiB)
        for t in (2, 4):
            xq = torch.randint(-127, 128, (t, m.k), dtype=torch.int8, device=dev)
            am = torch.rand(t, device=dev) * 4 + 1
            y = torch.empty((t, m.n), dtype=torch.float32, device=dev)
            P = [ptr(c) for c in copies]
            us = rotated_time_us(
                torch, lambda s, i: calls.forward(P[i], ptr(gamma), ptr(xq), ptr(am), t, m.n, m.k,
                                                  ptr(y), 0, ctypes.c_void_p(s.cuda_stream)),
                len(copies), stream)
            rec[f"t{t}_int8_forward_us"] = round(us, 2)
            rec[f"t{t}_int8_forward_gb_s"] = round(gemv_bytes(t, m.n, m.k) / us / 1e3, 1)
        out[f"{m.k}->{m.n}"] = rec
        del copies, packed
        torch.cuda.empty_cache()
    return out


# 3B-class layer: the BitNet b1.58 3B model (listed among the released models
# on the bitnet.cpp pages) follows the LLaMA-3B layout, hidden 3200, FFN 8640,
# keys and values as wide as the queries; the pages give no dimensions, so
# these are a stated reading.  K = 3200 and 8640 are not multiples of 256
# (short last decode chunks) and 8640 is not one of 128 (the register-staged
# MFMA kernel at T = 2048).
THREE_B = [("q", 3200, 3200), ("k", 3200, 3200), ("v", 3200, 3200), ("o", 3200, 3200),
           ("gate", 3200, 8640), ("up", 3200, 8640), ("down", 8640, 3200)]


def three_b_extra(torch, binding, dev, stream):
    """Context: the 3B-class layer.  Decode, T = 1: the seven projections as
    the headline's four fused launches [q, k, v], [o], [gate, up], [down],
    layer sets rotated over > 1 GB, GB/s of the step.  Prefill, T = 2048:
    act-quant + tiled MFMA kernel on 3200 -> 8640 and 8640 -> 3200, TOP/s.
    Weights N(0, 0.02) and bf16 activations N(0, 1), drawn on the GPU
    (seeded) and packed there."""
    lib = binding.load()
    calls = Calls(lib)
    mats = []
    for mi, (name, k, n) in enumerate(THREE_B):
        gen = torch.Generator(device=dev)
        gen.manual_seed(7000 + mi)
        w = torch.randn((n, k), device=dev, generator=gen) * 0.02
        packed, gamma = binding.pack_weights(w)
        del w
        x = torch.randn((1, k), device=dev, generator=gen).to(torch.bfloat16)
        mats.append(dict(name=name, k=k, n=n, packed=packed, gamma=gamma, x=x,
                         xq=torch.empty((1, k), dtype=torch.int8, device=dev),
                         absmax=torch.empty(1, dtype=torch.float32, device=dev),
                         y=torch.empty((1, n), dtype=torch.float32, device=dev)))
    layer_bytes = sum(d["packed"].numel() for d in mats)
    n_sets = int(np.ceil(ROT_BYTES / layer_bytes))
    sets = [[d["packed"] for d in mats]] + [[d["packed"].clone() for d in mats]
                                            for _ in range(n_sets - 1)]
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    descs = []
    for sp in sets:
        per = []
        for grp in groups:
            arr = (binding.BlLinear * len(grp))()
            for gi, mi in enumerate(grp):
                d = mats[mi]
                arr[gi] = binding.BlLinear(d["x"].data_ptr(), sp[mi].data_ptr(), d["gamma"].data_ptr(),
                                           d["n"], d["k"], d["y"].data_ptr(), d["xq"].data_ptr(),
                                           d["absmax"].data_ptr(), None)
            per.append(arr)
        descs.append(per)

    def steps(s):
        h = ctypes.c_void_p(s.cuda_stream)
        for per in descs:
            for arr in per:
                calls.grouped(arr, 1, h)

    g = capture(torch, steps, stream)
    reps = 16
    ms = time_graph(torch, g, reps, 2, stream)
    us_step = ms * 1e3 / (reps * n_sets)
    step_bytes = sum(fused_bytes(1, d["n"], d["k"]) for d in mats)
    out = {"decode_t1_layer": {"us_per_step": round(us_step, 2),
                               "gb_s": round(step_bytes / us_step / 1e3, 1),
                               "frac_of_hbm_peak": round(step_bytes / us_step / 1e3 / HBM_PEAK_GBS, 4),
                               "step_bytes": int(step_bytes), "layer_sets_rotated": n_sets}}
    del descs, sets, g
    torch.cuda.empty_cache()
    t = 2048
    for mi in (4, 6):
        d = mats[mi]
        k, n = d["k"], d["n"]
        copies = [d["packed"]] + [d["packed"].clone() for _ in range(int(np.ceil(ROT_BYTES / d["packed"].numel())) - 1)]
        gen = torch.Generator(device=dev)
        gen.manual_seed(7100 + mi)
        x = torch.randn((t, k), device=dev, generator=gen).to(torch.bfloat16)
        xq = torch.empty((t, k), dtype=torch.int8, device=dev)
        am = torch.empty(t, dtype=torch.float32, device=dev)
        y = torch.empty((t, n), dtype=torch.float32, device=dev)
        P = [ptr(c) for c in copies]
        calls.quant(ptr(x), ptr(xq), ptr(am), t, k, ctypes.c_void_p(stream.cuda_stream))
        us1 = rotated_time_us(
            torch, lambda s, i: calls.forward(P[i], ptr(d["gamma"]), ptr(xq), ptr(am), t, n, k, ptr(y),
                                              0, ctypes.c_void_p(s.cuda_stream)),
            len(copies), stream, reps=4)

        def both(s, i):
            h = ctypes.c_void_p(s.cuda_stream)
            calls.quant(ptr(x), ptr(xq), ptr(am), t, k, h)
            calls.forward(P[i], ptr(d["gamma"]), ptr(xq), ptr(am), t, n, k, ptr(y), 0, h)

        us2 = rotated_time_us(torch, both, len(copies), stream, reps=4)
        ops = 2.0 * t * n * k
        out[f"prefill_t2048_{k}->{n}"] = {
            "gemm_us": round(us1, 2), "gemm_tops": round(ops / us1 / 1e6, 1),
            "gemm_frac_of_int8_peak": round(ops / us1 / 1e6 / INT8_PEAK_TOPS, 4),
            "quant_plus_gemm_us": round(us2, 2), "quant_plus_gemm_tops": round(ops / us2 / 1e6, 1),
            "rotated_copies": len(copies)}
        del copies
        torch.cuda.empty_cache()
    return out


def crossover_extra(torch, mats, sets, dev, stream, calls):
    """Batched decode: the decode kernel against the tiled MFMA kernel on
    2560->6912 and 6912->2560 for T in {1, 8, 32, 64, 128, 256} (int8 input,
    weights rotated over the layer sets); T* is the largest T at which the
    decode kernel is still the faster."""
    out = {}
    for mi in (4, 6):
        d = mats[mi]
        n, k = d["m"].n, d["m"].k
        rows = {}
        for t in (1, 8, 32, 64, 128, 256):
            xq = torch.randint(-127, 128, (t, k), dtype=torch.int8, device=dev)
            am = torch.rand(t, device=dev) * 4 + 1
            y = torch.empty((t, n), dtype=torch.float32, device=dev)
            P = [ptr(s_[mi]) for s_ in sets]
            us = [rotated_time_us(
                torch, lambda s, i, a=algo: calls.forward(P[i], ptr(d["gamma"]), ptr(xq), ptr(am), t,
                                                          n, k, ptr(y), a, ctypes.c_void_p(s.cuda_stream)),
                len(sets), stream, reps=5) for algo in (1, 2)]
            rows[str(t)] = {"decode_kernel_us": round(us[0], 2), "tiled_mfma_us": round(us[1], 2)}
        tstar = max([int(t) for t, r in rows.items() if r["decode_kernel_us"] <= r["tiled_mfma_us"]] + [0])
        out[f"{k}->{n}"] = {"by_T": rows, "T_star": tstar}
    return out


def prefill_extra(torch, binding, wl, dev, stream):
    """Context: prefill (T = 2048) on both 2B shapes, TOP/s of the tiled MFMA
    kernel alone and of act-quant + kernel, each with the row sums derived in
    the kernel and handed in from act-quant.  As in a model, where every layer
    has its own weights, consecutive calls rotate through 64 copies of the
    packed matrix."""
    wk = wl.WORKLOADS[4]
    lib = binding.load()
    calls = Calls(lib)
    out = {}
    for mi, m in enumerate(wk.matrices):
        t = 2048
        packed, gamma = binding.pack_weights(torch.from_numpy(wk.weights(mi)).to(dev))
        copies = [packed] + [packed.clone() for _ in range(63)]
        bits = wl.bf16_bits(wk.activations(mi, t))
        x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        xq = torch.empty((t, m.k), dtype=torch.int8, device=dev)
        absmax = torch.empty(t, dtype=torch.float32, device=dev)
        y = torch.empty((t, m.n), dtype=torch.float32, device=dev)
        P = [ptr(c) for c in copies]
        Q = [ptr(v) for v in (gamma, xq, absmax, y, x)]
        calls.quant(Q[4], Q[1], Q[2], t, m.k, ctypes.c_void_p(stream.cuda_stream))
        us1 = rotated_time_us(
            torch, lambda s, i: calls.forward(P[i], Q[0], Q[1], Q[2], t, m.n, m.k, Q[3], 2,
                                              ctypes.c_void_p(s.cuda_stream)),
            len(copies), stream, reps=4)

        def both(s, i):
            h = ctypes.c_void_p(s.cuda_stream)
            calls.quant(Q[4], Q[1], Q[2], t, m.k, h)
            calls.forward(P[i], Q[0], Q[1], Q[2], t, m.n, m.k, Q[3], 2, h)

        us2 = rotated_time_us(torch, both, len(copies), stream, reps=4)
        # the same with the tokens' row sums: act-quant writes them, the
        # tiled kernel takes them instead of summing q in its K loop
        rs = torch.empty(t, dtype=torch.int32, device=dev)
        calls.quant(Q[4], Q[1], Q[2], t, m.k, ctypes.c_void_p(stream.cuda_stream), ptr(rs))
        us3 = rotated_time_us(
            torch, lambda s, i: calls.forward(P[i], Q[0], Q[1], Q[2], t, m.n, m.k, Q[3], 2,
                                              ctypes.c_void_p(s.cuda_stream), ptr(rs)),
            len(copies), stream, reps=4)

        def both_rs(s, i):
            h = ctypes.c_void_p(s.cuda_stream)
            calls.quant(Q[4], Q[1], Q[2], t, m.k, h, ptr(rs))
            calls.forward(P[i], Q[0], Q[1], Q[2], t, m.n, m.k, Q[3], 2, h, ptr(rs))

        us4 = rotated_time_us(torch, both_rs, len(copies), stream, reps=4)
        ops = 2.0 * t * m.n * m.k
        out[f"{m.k}->{m.n}"] = {
            "gemm_us": round(us1, 2), "gemm_tops": round(ops / us1 / 1e6, 1),
            "gemm_frac_of_int8_peak": round(ops / us1 / 1e6 / INT8_PEAK_TOPS, 4),
            "quant_plus_gemm_us": round(us2, 2),
            "quant_plus_gemm_tops": round(ops / us2 / 1e6, 1),
            "gemm_rowsum_given_us": round(us3, 2),
            "gemm_rowsum_given_frac_of_int8_peak": round(ops / us3 / 1e6 / INT8_PEAK_TOPS, 4),
            "quant_plus_gemm_rowsum_us": round(us4, 2)}
        del copies, packed
        torch.cuda.empty_cache()
    return out


def gated_extra(torch, binding, dev, stream):
    """The gate/up pair of the 2B FFN (2560 -> 2 x 6912) with the gated
    ReLU^2 epilogue writing bfloat16 h, against the same two projections
    writing binary32 outputs (without the activation): T = 1 (one launch
    each, act-quant fused) and T = 2048 (act-quant, then the tiled MFMA
    kernel; two GEMMs against one).  Weights drawn on the GPU (N(0, 0.02),
    seeded), rotated over > 1 GB at T = 1 and 64 copies at T = 2048."""
    lib = binding.load()
    calls = Calls(lib)
    k, n = 2560, 6912
    gen = torch.Generator(device=dev)
    gen.manual_seed(8100)
    pg, gg = binding.pack_weights(torch.randn((n, k), device=dev, generator=gen) * 0.02)
    pu, gu = binding.pack_weights(torch.randn((n, k), device=dev, generator=gen) * 0.02)
    pgu = binding.interleave_rows(pg, pu)
    out = {}
    for t in (1, 2048):
        ncopy = int(np.ceil(ROT_BYTES / pgu.numel())) if t == 1 else 64
        cg = [pg] + [pg.clone() for _ in range(ncopy - 1)]
        cu = [pu] + [pu.clone() for _ in range(ncopy - 1)]
        cgu = [pgu] + [pgu.clone() for _ in range(ncopy - 1)]
        x = torch.randn((t, k), device=dev, generator=gen).to(torch.bfloat16)
        xq = torch.empty((t, k), dtype=torch.int8, device=dev)
        am = torch.empty(t, dtype=torch.float32, device=dev)
        yg = torch.empty((t, n), dtype=torch.float32, device=dev)
        yu = torch.empty((t, n), dtype=torch.float32, device=dev)
        h = torch.empty((t, n), dtype=torch.bfloat16, device=dev)
        X, XQ, AM, YG, YU, H, GG, GU = (ptr(v) for v in (x, xq, am, yg, yu, h, gg, gu))

        def gated(s, i):
            rc = lib.bitlinear_gated_relu2(X, 1, ptr(cgu[i]), GG, GU, t, n, k, H, XQ, AM, None,
                                           ctypes.c_void_p(s.cuda_stream))
            if rc:
                raise RuntimeError(lib.bitlinear_last_error().decode())

        if t == 1:
            descs = []
            for i in range(ncopy):
                arr = (binding.BlLinear * 2)()
                arr[0] = binding.BlLinear(x.data_ptr(), cg[i].data_ptr(), gg.data_ptr(), n, k,
                                          yg.data_ptr(), xq.data_ptr(), am.data_ptr(), None)
                arr[1] = binding.BlLinear(x.data_ptr(), cu[i].data_ptr(), gu.data_ptr(), n, k,
                                          yu.data_ptr(), xq.data_ptr(), am.data_ptr(), None)
                descs.append(arr)

            def plain(s, i):
                calls.grouped(descs[i], 1, ctypes.c_void_p(s.cuda_stream))
        else:
            def plain(s, i):
                hs = ctypes.c_void_p(s.cuda_stream)
                calls.quant(X, XQ, AM, t, k, hs)
                calls.forward(ptr(cg[i]), GG, XQ, AM, t, n, k, YG, 0, hs)
                calls.forward(ptr(cu[i]), GU, XQ, AM, t, n, k, YU, 0, hs)

        reps = 10 if t == 1 else 4
        us_g = rotated_time_us(torch, gated, ncopy, stream, reps=reps)
        us_p = rotated_time_us(torch, plain, ncopy, stream, reps=reps)
        rec = {"gated_bf16_us": round(us_g, 2), "two_projections_f32_us": round(us_p, 2),
               "rotated_copies": ncopy}
        if t == 1:
            byts = 2 * n * k // 4 + 2 * k + 2 * n + k + 4
            rec["gated_gb_s"] = round(byts / us_g / 1e3, 1)
            rec["gated_frac_of_hbm_peak"] = round(byts / us_g / 1e3 / HBM_PEAK_GBS, 4)
        else:
            ops = 2.0 * t * 2 * n * k
            rec["gated_tops"] = round(ops / us_g / 1e6, 1)
            rec["gated_frac_of_int8_peak"] = round(ops / us_g / 1e6 / INT8_PEAK_TOPS, 4)
            rec["two_projections_tops"] = round(ops / us_p / 1e6, 1)
        out[f"T{t}_K{k}_N2x{n}"] = rec
        del cg, cu, cgu
        torch.cuda.empty_cache()
    return out


def lut_extra(torch, binding, mats, sets, dev, stream, calls):
    """The two comparison designs of the decode step, the table-lookup kernel
    (bitnet.cpp TL1/TL2 style) and the packed-int8-dot (v_dot4) kernel,
    against the matrix-core decode kernel at T = 1 on int8 input: the 2B
    shapes (weights rotated over the layer sets) and 8192 -> 28672 (weights
    drawn on the GPU, rotated over > 1 GB)."""
    out = {}
    for mi in (0, 4, 6):
        d = mats[mi]
        n, k = d["m"].n, d["m"].k
        xq = torch.randint(-127, 128, (1, k), dtype=torch.int8, device=dev)
        am = torch.rand(1, device=dev) * 4 + 1
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        P = [ptr(s_[mi]) for s_ in sets]
        us = [rotated_time_us(
            torch, lambda s, i, a=algo: calls.forward(P[i], ptr(d["gamma"]), ptr(xq), ptr(am), 1, n, k,
                                                      ptr(y), a, ctypes.c_void_p(s.cuda_stream)),
            len(sets), stream, reps=5) for algo in (3, 4, 1)]
        out[f"{k}->{n}"] = {"lut_us": round(us[0], 2), "dot4_us": round(us[1], 2),
                            "decode_kernel_us": round(us[2], 2),
                            "lut_gb_s": round(gemv_bytes(1, n, k) / us[0] / 1e3, 1),
                            "dot4_gb_s": round(gemv_bytes(1, n, k) / us[1] / 1e3, 1)}
    n, k = 28672, 8192
    gen = torch.Generator(device=dev)
    gen.manual_seed(5100)
    packed, gamma = binding.pack_weights(torch.randn((n, k), device=dev, generator=gen) * 0.01)
    copies = [packed] + [packed.clone() for _ in range(int(np.ceil(ROT_BYTES / packed.numel())) - 1)]
    xq = torch.randint(-127, 128, (1, k), dtype=torch.int8, device=dev)
    am = torch.rand(1, device=dev) * 4 + 1
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    P = [ptr(c) for c in copies]
    us = [rotated_time_us(
        torch, lambda s, i, a=algo: calls.forward(P[i], ptr(gamma), ptr(xq), ptr(am), 1, n, k, ptr(y), a,
                                                  ctypes.c_void_p(s.cuda_stream)),
        len(copies), stream, reps=5) for algo in (3, 4, 1)]
    out[f"{k}->{n}"] = {"lut_us": round(us[0], 2), "dot4_us": round(us[1], 2),
                        "decode_kernel_us": round(us[2], 2),
                        "lut_gb_s": round(gemv_bytes(1, n, k) / us[0] / 1e3, 1),
                        "dot4_gb_s": round(gemv_bytes(1, n, k) / us[1] / 1e3, 1)}
    del copies, packed
    torch.cuda.empty_cache()
    return out


def binary_extra(torch, binding, dev, stream):
    """Binary (+1/-1, one bit each) weights against the ternary format on the
    same shapes: T = 1 (decode kernels, int8 input, weights rotated over
    > 1 GB) on 2560->6912, 6912->2560 and 8192->28672, and T = 2048 (tiled
    MFMA kernels, 64 rotated copies) on 2560->6912.  Weights drawn on the GPU
    (N(0, 0.02), seeded)."""
    lib = binding.load()
    calls = Calls(lib)
    out = {}
    for (k, n, t) in ((2560, 6912, 1), (6912, 2560, 1), (8192, 28672, 1), (2560, 6912, 2048)):
        gen = torch.Generator(device=dev)
        gen.manual_seed(9100 + k + t)
        w = torch.randn((n, k), device=dev, generator=gen) * 0.02
        pt, gt = binding.pack_weights(w)
        pb, gb = binding.pack_weights_binary(w)
        del w
        xq = torch.randint(-127, 128, (t, k), dtype=torch.int8, device=dev)
        am = torch.rand(t, device=dev) * 4 + 1
        y = torch.empty((t, n), dtype=torch.float32, device=dev)
        rec = {}
        for name, p, g in (("ternary", pt, gt), ("binary", pb, gb)):
            ncopy = int(np.ceil(ROT_BYTES / p.numel())) if t == 1 else 64
            copies = [p] + [p.clone() for _ in range(ncopy - 1)]
            P = [ptr(c) for c in copies]
            if name == "ternary":
                fn = lambda s, i: calls.forward(P[i], ptr(g), ptr(xq), ptr(am), t, n, k, ptr(y), 0,
                                                ctypes.c_void_p(s.cuda_stream))
            else:
                def fn(s, i):
                    rc = lib.bitlinear_forward_binary(P[i], ptr(g), ptr(xq), ptr(am), t, n, k, ptr(y),
                                                      None, 0, ctypes.c_void_p(s.cuda_stream))
                    if rc:
                        raise RuntimeError(lib.bitlinear_last_error().decode())
            us = rotated_time_us(torch, fn, ncopy, stream, reps=5 if t == 1 else 4)
            wbytes = p.numel()
            if t == 1:
                byts = wbytes + k + 4 + 4 * n + 4
                rec[name] = {"us": round(us, 2), "gb_s": round(byts / us / 1e3, 1),
                             "frac_of_hbm_peak": round(byts / us / 1e3 / HBM_PEAK_GBS, 4)}
            else:
                ops = 2.0 * t * n * k
                rec[name] = {"us": round(us, 2), "tops": round(ops / us / 1e6, 1),
                             "frac_of_int8_peak": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4)}
            del copies
        out[f"T{t}_{k}->{n}"] = rec
        del pt, pb
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(sharding the forward across GPUs is a design note, not code)", file=sys.stderr)
        sys.exit(2)

    import torch
    from bitlinear_w1_a8_amd import binding, workloads as wl

    if not os.path.exists(binding.LIB_PATH):
        from bitlinear_w1_a8_amd import build
        build.build(verbose=False)
    lib = binding.load()
    calls = Calls(lib)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)

    if args.profile_prefill:
        wk = wl.WORKLOADS[4]
        for mi, m in enumerate(wk.matrices):
            packed, gamma = binding.pack_weights(torch.from_numpy(wk.weights(mi)).to(dev))
            bits = wl.bf16_bits(wk.activations(mi, 2048))
            x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
            for _ in range(5):
                xq, absmax, _ = binding.quant_act(x, with_rowsum=False)
                binding.forward(packed, gamma, xq, absmax, m.n, algo="gemm")
            torch.cuda.synchronize()
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print("profile pass done", flush=True)
        return

    mats, sets, pack_ms = decode_setup(torch, binding, wl, dev)
    n_sets = len(sets)
    mp = [dict(x=ptr(d["x"]), xq=ptr(d["xq"]), absmax=ptr(d["absmax"]), y=ptr(d["y"]),
               gamma=ptr(d["gamma"]), n=d["m"].n, k=d["m"].k) for d in mats]
    set_ptrs = [[ptr(p) for p in s] for s in sets]

    def steps(s, with_quant=True, with_gemv=True):
        """The layer as 14 launches: act-quant then forward per projection."""
        h = ctypes.c_void_p(s.cuda_stream)
        for sp in set_ptrs:                      # one step per layer set
            for mi, d in enumerate(mp):
                if with_quant:
                    calls.quant(d["x"], d["xq"], d["absmax"], 1, d["k"], h)
                if with_gemv:
                    calls.forward(sp[mi], d["gamma"], d["xq"], d["absmax"], 1, d["n"], d["k"],
                                  d["y"], 1, h)

    # The layer's dependency order: q, k, v share their input; o needs the
    # attention output; gate, up share their input; down needs their product.
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    group_descs = []
    for sp in set_ptrs:
        per_set = []
        for grp in groups:
            arr = (binding.BlLinear * len(grp))()
            for gi, mi in enumerate(grp):
                d = mats[mi]
                arr[gi] = binding.BlLinear(d["x"].data_ptr(), sp[mi].value,
                                           d["gamma"].data_ptr(), d["m"].n, d["m"].k,
                                           d["y"].data_ptr(), d["xq"].data_ptr(),
                                           d["absmax"].data_ptr(), None)
            per_set.append(arr)
        group_descs.append(per_set)

    def fused_steps(s, first=0, count=None):
        """`count` layer steps (default: one per layer set) from layer set
        `first` on, each as four fused launches in dependency order."""
        h = ctypes.c_void_p(s.cuda_stream)
        for i in range(first, first + (n_sets if count is None else count)):
            for arr in group_descs[i % n_sets]:
                calls.grouped(arr, 1, h)

    if args.profile_pass:
        for _ in range(2):
            fused_steps(stream)
        stream.synchronize()
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print("profile pass done", flush=True)
        return

    step_bytes = sum(fused_bytes(1, d["n"], d["k"]) for d in mp)
    fused_launch_bytes = step_bytes / len(groups)
    unfused_step_bytes = sum(gemv_bytes(1, d["n"], d["k"]) + quant_bytes(1, d["k"]) for d in mp)
    gemv_launch_bytes = sum(gemv_bytes(1, d["n"], d["k"]) for d in mp) / len(mp)

    reps = max(1, args.steps // n_sets)
    warm = max(1, args.warmup // n_sets)
    k_steps = reps * n_sets

    # timed region: exactly --steps layer steps after exactly --warmup
    # untimed ones, as graph replays: whole rotations over the layer sets
    # plus a graph of the remaining steps (each step's weights come from the
    # next layer set, so they stream cold)
    g_fused = capture(torch, fused_steps, stream)
    tails = {}

    def plan(count):
        full, rest = divmod(count, n_sets)
        if rest and rest not in tails:
            tails[rest] = capture(torch, lambda s_: fused_steps(s_, 0, rest), stream)
        return [g_fused] * full + ([tails[rest]] if rest else [])

    warm_plan, timed_plan = plan(args.warmup), plan(args.steps)
    ms = time_plan(torch, timed_plan, warm_plan, stream)
    ms_per_step = ms / args.steps
    fused_us = ms * 1e3 / (args.steps * len(groups))

    extra = {}
    if not args.fused_only:
        # the same layer as 14 separate launches, and its kernels alone
        g_all = capture(torch, lambda s: steps(s), stream)
        ms_unfused = time_graph(torch, g_all, reps, warm, stream)
        g_gemv = capture(torch, lambda s: steps(s, with_quant=False), stream)
        ms_g = time_graph(torch, g_gemv, reps, warm, stream)
        gemv_us = ms_g * 1e3 / (k_steps * len(mp))
        g_quant = capture(torch, lambda s: steps(s, with_gemv=False), stream)
        ms_q = time_graph(torch, g_quant, reps, warm, stream)
        quant_us = ms_q * 1e3 / (k_steps * len(mp))

        # the fused steps launched one by one on the stream, without a graph
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eager_reps = max(1, reps // 4)
        for _ in range(eager_reps):
            fused_steps(stream)
        stream.synchronize()
        eager_ms_per_step = (time.perf_counter() - t0) * 1e3 / (eager_reps * n_sets)
        extra = {"eager_ms_per_step": round(eager_ms_per_step, 4),
                 "unfused_ms_per_step": round(ms_unfused / k_steps, 5),
                 "unfused_gb_s": round(unfused_step_bytes / (ms_unfused / k_steps * 1e-3) / 1e9, 2),
                 "gemv_avg_launch_us": round(gemv_us, 3),
                 "gemv_gb_s": round(gemv_launch_bytes / (gemv_us * 1e-6) / 1e9, 1),
                 "act_quant_avg_launch_us": round(quant_us, 3)}

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()

    achieved = fused_launch_bytes / (fused_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": committed_traffic("gemv.hip", "decode_fused_2b_t1"),
                "kernel": "k_gemv_dec (act-quant fused into the decode GEMV), T=1",
                "avg_launch_us": round(fused_us, 3),
                "algorithmic_bytes_per_launch": int(fused_launch_bytes)}

    if not args.fused_only:
        # spread of the step time: the same graph in 16 shorter timed runs
        chunk_ms = time_graph_chunks(torch, g_fused, reps, 16, stream)
        q = np.percentile(np.array(chunk_ms) / n_sets, [10, 50, 90])
        extra["ms_per_step_p10_p50_p90"] = [round(float(v), 5) for v in q]
    extra.update({"layer_sets_rotated": n_sets,
                  "rotated_packed_bytes": int(sum(p.numel() for p in sets[0]) * n_sets),
                  "pack_ms_per_matrix": [round(v, 3) for v in pack_ms]})
    want = set(args.extra.split(",")) if args.extra != "all" else {
        "calib", "toy", "prefill", "crossover", "70b", "3b", "subln", "gated", "lut", "binary",
        "pack"}
    if not args.no_extra:
        if "calib" in want:
            extra["device_ceilings"] = calibration(torch, binding, dev, stream)
            roofline["measured_read_stream_gb_s"] = \
                extra["device_ceilings"]["hbm_read_stream_70b_matrix_rotated_gb_s"]
        if "toy" in want:
            extra["toy_t4_k256_n512"] = toy_extra(torch, binding, wl, dev, stream)
        if "prefill" in want:
            extra["prefill_t2048"] = prefill_extra(torch, binding, wl, dev, stream)
        if "crossover" in want:
            extra["batched_decode_crossover"] = crossover_extra(torch, mats, sets, dev, stream, calls)
        if "70b" in want:
            extra["70b_class"] = big_extra(torch, binding, wl, dev, stream)
        if "3b" in want:
            extra["3b_class"] = three_b_extra(torch, binding, dev, stream)
        if "subln" in want:
            extra["subln_act_quant"] = subln_extra(torch, binding, dev, stream)
        if "pack" in want:
            extra["a0_pack"] = pack_extra(torch, binding, dev, stream)
        if "gated" in want:
            extra["gated_relu2_ffn"] = gated_extra(torch, binding, dev, stream)
        if "binary" in want:
            extra["binary_weights"] = binary_extra(torch, binding, dev, stream)
        if "lut" in want:
            extra["lut_decode_comparison"] = lut_extra(torch, binding, mats, sets, dev, stream, calls)

    # the same figures against the device's measured ceilings
    ceil = extra.get("device_ceilings")
    if ceil:
        stream_gbs = ceil["hbm_read_stream_70b_matrix_rotated_gb_s"]
        mfma_tops = ceil["int8_mfma_loop_tops"]
        for rec_ in extra.get("70b_class", {}).values():
            rec_["t1_forward_frac_of_measured_read_stream"] = round(
                rec_["t1_forward_gb_s"] / stream_gbs, 4)
            rec_["t256_forward_frac_of_measured_mfma_loop"] = round(
                rec_["t256_forward_tops"] / mfma_tops, 4)
        for rec_ in extra.get("prefill_t2048", {}).values():
            rec_["gemm_frac_of_measured_mfma_loop"] = round(rec_["gemm_tops"] / mfma_tops, 4)

    cpu = None
    if not args.no_cpu:
        import oracle
        cpu = cpu_baseline(oracle, wl, budget_s=args.cpu_budget)

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    rec = {"metric": "BitLinear decode GEMV HBM GB/s (% peak) + prefill GEMM int8 TOPS (% MFMA peak)",
           "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
           "data": "synthetic",
           "config": {"workload": "decode_2b_t1_layer: T=1, bf16 x, 7 projections "
                                  "(q 2560->2560, k/v 2560->640, o 2560->2560, gate/up "
                                  "2560->6912, down 6912->2560) as 4 fused launches "
                                  "[qkv][o][gate,up][down], weights rotated cold",
                      "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
                      "step_bytes": int(step_bytes)},
           "roofline": roofline, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
