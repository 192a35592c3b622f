"""Benchmark of the chunked SSD forward on one MI355X.

Default workload: the BitMamba-1B Mamba-2 layer shape -- batch 2, T 2048,
64 heads, head dim 64, state 128, one B/C group, chunk 256, bf16 x/B/C with
fp32 dt/A/state -- on seeded synthetic inputs.  One step = one call of
ssd_chunk_fwd over the whole batch (every kernel of the call: chunk states,
the state passing between chunks, chunk outputs).

Timing: HIP events bound by the library to each kernel's dispatch on the
launch stream (a start/stop pair per kernel, every timed step); a kernel's
time is the mean of its pair's intervals, ms_per_step the mean interval from
the first kernel's start to the last kernel's stop (gaps between the kernels
included).  Between steps a 512 MiB buffer is read (outside the timed
intervals) so that the 256 MB Infinity Cache and the L2s hold none of the
step's inputs: the number is the rate with inputs resident in HBM.  The flush
reads rather than writes: a written flush would leave the cache full of dirty
lines whose write-back the next step's first kernel would pay for.

Prints one JSON line (rank 0): metric, value (tokens/s), roofline of the
dominant kernel, and the float64 CPU oracle timed on a bounded sample.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/s per layer (H64 P64 N128) + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
# dense MFMA peaks (MI355X datasheet)
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bitmamba_bf16",
                    choices=["bitmamba_bf16", "long_bf16", "mamba3lite_complex", "tiny_f32",
                             "decode_f32", "decode_complex", "conv_bf16", "conv_decode_f32",
                             "bwd_bf16", "bwd_complex", "mamba3lite_packed", "mimo_bf16",
                             "varlen_bf16"])
    ap.add_argument("--no-flush", action="store_true",
                    help="keep the Infinity Cache warm between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run one plain 256 MiB device copy (reference for the HBM "
                         "byte counters)")
    return ap.parse_args()


class Hip:
    """Minimal HIP event API through ctypes (the runtime torch already loaded)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return e

    def record(self, e, stream):
        rc = self.lib.hipEventRecord(e, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value


# Device code behind each workload's kernels: the kernel file and the device
# headers every kernel file includes.  A traffic record stays valid while these
# files hash the same.
DEVICE_HEADERS = ["ssd_chunk_common.h", "ssd_device.h"]
KERNEL_SOURCES = {
    # (ssd_internal.h: the segment length the bf16 forward launches with)
    "bitmamba_bf16": ["ssd_chunk_bf16.hip", "ssd_internal.h"],
    "long_bf16": ["ssd_chunk_bf16.hip", "ssd_internal.h"],
    "tiny_f32": ["ssd_chunk.hip"],
    "mamba3lite_complex": ["ssd_chunk_cplx.hip"],
    "decode_f32": ["ssd_decode.hip"],
    "decode_complex": ["ssd_decode.hip"],
    "conv_bf16": ["ssd_conv.hip"],
    "conv_decode_f32": ["ssd_conv.hip"],
    "bwd_bf16": ["ssd_bwd_bf16.hip", "ssd_chunk_bf16.hip", "ssd_internal.h"],
    "mamba3lite_packed": ["ssd_chunk_cplx.hip"],
    "mimo_bf16": ["ssd_linear.hip"],
    "bwd_complex": ["ssd_bwd_f32.hip", "ssd_chunk.hip"],
    "varlen_bf16": ["ssd_chunk_bf16.hip", "ssd_internal.h"],
}


def source_sha256(workload):
    """Hash of the device sources of a workload's kernels (names and contents)."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "selective_state_space_09_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[workload] + DEVICE_HEADERS):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def copy_counter_reference(torch, dev):
    """One plain 256 MiB device-to-device copy: the reference the HBM byte
    counters are scaled by."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` (FETCH + WRITE, rocprofv3 counters
    scaled by a plain copy of known size) from profiles/traffic_<workload>.json,
    or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_sha256(workload):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["fetch_bytes"] + k["write_bytes"]


def kernel_segments(cfg):
    """Kernels of one chunked-forward call and the event pair bound to each:
    chunk states, the state passing between chunks, then the outputs."""
    if cfg["kind"] == "real" and cfg.get("dtype") == "bf16":
        return {"ssd_state_bf16_kernel": (0, 1), "ssd_pass_bf16_kernel": (2, 3),
                "ssd_scan_bf16_kernel": (4, 5)}
    if cfg["kind"] in ("complex", "complex_packed"):
        return {"ssd_state_cplx_kernel": (0, 1), "ssd_pass_kernel": (2, 3),
                "ssd_scan_cplx_kernel": (4, 5)}
    return {"ssd_state_kernel": (0, 1), "ssd_pass_kernel": (2, 3), "ssd_scan_kernel": (4, 5)}


def own_io_bytes(cfg, dims):
    """Bytes each kernel of one chunked-forward call reads or writes, every
    array once, workspace arrays (chunk states, token tables) included.  This
    is a kernel's own traffic, not the algorithmic figure the roofline uses."""
    Bsz, T, H, P, G, N, Q = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N", "Q"))
    cplx = cfg["kind"] in ("complex", "complex_packed")
    es = 2 if cfg.get("dtype") == "bf16" else 4          # x element
    bs = 8 if cplx else es                                # B/C element
    KC = 2 * N if cplx else N
    nc = -(-T // Q)
    x = Bsz * T * H * P * es
    bc = Bsz * T * G * N * bs
    dt = Bsz * T * H * 4
    states = Bsz * nc * H * P * KC * 4
    decay = Bsz * H * nc * 8
    y = Bsz * T * H * P * (4 if cplx else es)
    st16 = Bsz * nc * H * P * N * 2                       # bf16 chunk / boundary states
    dec = Bsz * H * nc * 4
    tok = Bsz * nc * H * Q * 8                            # per-token (exponent, step) pairs
    return {
        "ssd_state_bf16_kernel": x + bc + dt + st16 + dec + tok,
        "ssd_pass_bf16_kernel": 2 * st16 + dec,
        "ssd_scan_bf16_kernel": x + 2 * bc + tok + st16 + y,
        # complex: the per-token table is (exponent, cos, sin, 0), 16 bytes
        "ssd_state_cplx_kernel": x + bc + dt + states + decay + 2 * tok,
        "ssd_scan_cplx_kernel": x + 2 * bc + 2 * tok + states + y,
        "ssd_state_kernel": x + bc + dt + states + decay,
        "ssd_pass_kernel": 2 * states + decay,
        "ssd_scan_kernel": x + 2 * bc + dt + states + y,
    }


def algorithmic_bytes(cfg, dims):
    """The whole forward's algorithmic HBM bytes: x, dt, B, C read once and y
    written once (17.15 KB per token at the BitMamba layer shape)."""
    Bsz, T, H, P, G, N = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N"))
    cplx = cfg["kind"] in ("complex", "complex_packed")
    es = 2 if cfg.get("dtype") == "bf16" else 4
    bs = 8 if cplx else es
    return (Bsz * T * H * P * es + 2 * Bsz * T * G * N * bs + Bsz * T * H * 4
            + Bsz * T * H * P * (4 if cplx else es))


def algorithmic_flops(cfg, dims):
    """Algorithmic matrix flops of one forward, per kernel: the lower
    triangle of the in-chunk scores C.B^T (once per (batch, chunk, group):
    heads of a group share it) and of (scores o L).(delta x), the chunk
    states (2QNP per (batch, chunk, head)) and the carried-state readout
    C.h_in (2QNP).  Complex, rotation-factored: real products with K = 2N
    features, no delta factor."""
    Bsz, T, H, P, G, N, Q = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N", "Q"))
    KC = 2 * N if cfg["kind"] in ("complex", "complex_packed") else N
    nch = T / Q                                  # chunks (fractional tail as a fraction)
    tri = Q * (Q + 1) / 2
    units = Bsz * nch * H
    gunits = Bsz * nch * G
    state = units * 2 * Q * KC * P
    scan = gunits * 2 * tri * KC + units * (2 * tri * P + 2 * Q * KC * P)
    return {"ssd_state_kernel": state, "ssd_state_bf16_kernel": state, "ssd_state_cplx_kernel": state,
            "ssd_scan_kernel": scan, "ssd_scan_bf16_kernel": scan, "ssd_scan_cplx_kernel": scan,
            "whole_forward": state + scan}


def copy_reference(torch, dev, nbytes, flush, reps=10):
    """A plain device copy moving `nbytes` in all (nbytes/2 read, nbytes/2
    written), cold (the same flush read before each), timed by HIP events on
    the current stream: the achievable-HBM reference at the workload's own
    size.  Returns (median GB/s, bytes moved)."""
    n = max(1 << 20, int(nbytes) // 2) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    times = []
    for _ in range(reps + 2):
        if flush is not None:
            flush.max()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times[2:]))
    del src, dst
    return 2 * n / (ms / 1e3) / 1e9, 2 * n


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (or platform.processor)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(inp, cfg, dims, target_s):
    """The float64 oracle on a bounded sample of the same workload: the first
    k (batch, head) recurrences in full length, k grown until the run takes
    about target_s seconds.  Reported as tokens/s of the whole workload's
    token count scaled by the sampled fraction."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    H = dims["H"]
    Bsz, T = dims["Bsz"], dims["T"]
    total_bh = Bsz * H

    def run(nh):
        sub = dict(inp)
        sub["x"] = np.ascontiguousarray(inp["x"][:1, :, :nh])
        sub["dt"] = np.ascontiguousarray(inp["dt"][:1, :, :nh])
        sub["A"] = np.ascontiguousarray(inp["A"][:nh])
        G, N = dims["G"], dims["N"]
        hpg = H // G
        groups = [h // hpg for h in range(nh)]
        sub["B"] = np.ascontiguousarray(inp["B"][:1, :, groups])
        sub["C"] = np.ascontiguousarray(inp["C"][:1, :, groups])
        for k in ("D", "dt_bias"):
            sub[k] = None if inp[k] is None else np.ascontiguousarray(inp[k][:nh])
        t0 = time.perf_counter()
        if cfg["kind"] in ("complex", "complex_packed"):
            oracle.complex_fwd(sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"],
                               sub["dt_bias"], sub["dt_min"], sub["dt_max"], None)
        else:
            oracle.fwd(sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"], sub["D"],
                       sub["dt_bias"], sub["dt_min"], sub["dt_max"], None)
        return time.perf_counter() - t0

    def run_full():
        t0 = time.perf_counter()
        if cfg["kind"] in ("complex", "complex_packed"):
            oracle.complex_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                               inp["dt_bias"], inp["dt_min"], inp["dt_max"], None)
        else:
            oracle.fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                       inp["dt_bias"], inp["dt_min"], inp["dt_max"], None)
        return time.perf_counter() - t0

    nh = min(H, max(1, threads))
    dt_run = run(nh)
    while dt_run < target_s / 2 and nh < H:
        nh = min(H, nh * 2)
        dt_run = run(nh)
    if nh == H and dt_run < target_s / 2:
        # the whole workload is small for the host: repeated full passes
        reps, total = 0, 0.0
        while total < target_s:
            total += run_full()
            reps += 1
        out = {"value": reps * Bsz * T / total, "unit": "tokens/s",
               "cores": oracle.threads_used(), "kind": "oracle",
               "sample": f"the whole workload ({total_bh} (batch, head) recurrences, T={T}), "
                         f"float64, {reps} passes in {total:.2f} s"}
    else:
        frac = nh / total_bh
        out = {"value": (Bsz * T * frac) / dt_run, "unit": "tokens/s",
               "cores": oracle.threads_used(), "kind": "oracle",
               "sample": f"{nh} of {total_bh} (batch, head) recurrences of the same workload, "
                         f"full length T={T}, float64, {dt_run:.2f} s; tokens/s scaled by the "
                         f"sampled fraction {nh}/{total_bh}"}
    # one thread: (batch, head) recurrences one after another for about a
    # quarter of the target time
    oracle.set_threads(1)
    reps, total = 0, 0.0
    while total < target_s / 4 and reps < 4 * H:
        total += run(1)
        reps += 1
    oracle.set_threads(threads)
    out["cpu_model"] = cpu_model()
    # the workload's Bsz*T tokens take Bsz*H recurrences of T steps: tokens/s
    # = T / (H * seconds per recurrence)
    out["one_thread"] = {"value": reps * T / (H * total), "unit": "tokens/s", "cores": 1,
                         "sample": f"{reps} runs of one (batch, head) recurrence of T={T} "
                                   f"steps in {total:.2f} s; scaled by the workload's {H} "
                                   f"recurrences per token"}
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the scan shards by batch/head with no communication; see DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_09_amd as ssd
    from selective_state_space_09_amd import inputs

    cfg = dict(inputs.WORKLOADS[args.workload])
    if cfg["kind"] in ("decode", "complex_decode"):
        return bench_decode(args, cfg)
    if cfg["kind"] in ("conv", "conv_decode"):
        return bench_conv(args, cfg)
    if cfg["kind"] == "bwd":
        return bench_bwd(args, cfg)
    if cfg["kind"] == "bwd_complex":
        return bench_bwd_complex(args, cfg)
    if cfg["kind"] == "mimo":
        return bench_mimo(args, cfg)
    if cfg["kind"] == "varlen":
        return bench_varlen(args, cfg)
    inp = inputs.make_workload(args.workload, seed=0)
    Q = cfg["chunk"]
    dims = dict(inp["dims"], Q=Q)
    dev = torch.device("cuda:0")

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    Bsz, T, H, P, G, N = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N"))
    cplx = cfg["kind"] in ("complex", "complex_packed")
    packed = cfg["kind"] == "complex_packed"
    y = torch.empty((Bsz, T, H, P), dtype=torch.float32 if cplx else d["x"].dtype, device=dev)
    nbytes = ssd.ssd_workspace_size(Bsz, T, H, P, G, N, Q, cplx)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.int32, device=dev)
    L = ssd.lib()
    hip = Hip()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())

    # timed steps: one event pair around each plain call (the call as a user
    # makes it); kernel breakdown: separate calls of the measurement variant,
    # whose per-kernel events (bound to each dispatch) time the kernels alone
    # but add a few microseconds between them
    n_total = args.warmup + args.steps
    n_kern = max(10, args.steps // 2)
    step_evs = [(hip.event(), hip.event()) for _ in range(n_total)]
    evs = [[hip.event() for _ in range(6)] for _ in range(n_kern)]
    ev_arrays = [(ctypes.c_void_p * 6)(*[e.value for e in row]) for row in evs]

    if packed:
        # x, B, C, dt read in place from the in_proj rows (Bsz, T, H(P+4N+1))
        proj = d["proj"]
        fixed = (P_(proj), proj.shape[2], P_(d["A"]), P_(d["dt_bias"]), float(d["dt_min"]),
                 float(d["dt_max"]), None, P_(y), None, Bsz, T, H, P, N, Q, P_(ws), ws.numel(), sp)
        call = lambda evarr: L.ssd_complex_chunk_fwd_packed_ev(*fixed, evarr)
        plain = lambda: L.ssd_complex_chunk_fwd_packed(*fixed)
        dtype_name = "bf16x3"
        peak_name = "bf16"
    elif cplx:
        fixed = (P_(d["x"]), P_(d["dt"]), P_(d["A"]), P_(d["B"]), P_(d["C"]), P_(d["dt_bias"]),
                 float(d["dt_min"]), float(d["dt_max"]), None, P_(y), None,
                 Bsz, T, H, P, G, N, Q, P_(ws), ws.numel(), sp)
        call = lambda evarr: L.ssd_complex_chunk_fwd_ev(*fixed, evarr)
        plain = lambda: L.ssd_complex_chunk_fwd(*fixed)
        dtype_name = "bf16x3"
        peak_name = "bf16"
    else:
        dcode = ssd.SSD_BF16 if d["x"].dtype == torch.bfloat16 else ssd.SSD_F32
        fixed = (P_(d["x"]), P_(d["dt"]), P_(d["A"]), P_(d["B"]), P_(d["C"]), P_(d["D"]),
                 P_(d["dt_bias"]), float(d["dt_min"]), float(d["dt_max"]), None, P_(y), None,
                 Bsz, T, H, P, G, N, Q, dcode, P_(ws), ws.numel(), sp)
        call = lambda evarr: L.ssd_chunk_fwd_ev(*fixed, evarr)
        plain = lambda: L.ssd_chunk_fwd(*fixed)
        dtype_name = "bf16" if dcode == ssd.SSD_BF16 else "f32"
        peak_name = dtype_name

    def check(rc):
        if rc != 0:
            raise RuntimeError(L.ssd_last_error().decode())

    def step(i):
        if flush is not None:
            flush.max()  # reads 512 MiB: evicts the inputs, leaves clean lines
        a, b = step_evs[i]
        hip.lib.hipEventRecord(a, sp)
        check(plain())
        hip.lib.hipEventRecord(b, sp)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.warmup, n_total):
        step(i)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per_step = [hip.elapsed_ms(*step_evs[i]) for i in range(args.warmup, n_total)]

    for i in range(n_kern):
        if flush is not None:
            flush.max()
        check(call(ev_arrays[i]))
    torch.cuda.synchronize()
    segs = kernel_segments(cfg)
    names = list(segs)
    per_kernel = {n: [] for n in names}
    per_step_ev = []
    for i in range(n_kern):
        e = evs[i]
        per_step_ev.append(hip.elapsed_ms(e[0], e[5]))
        for n, (k0, k1) in segs.items():
            per_kernel[n].append(hip.elapsed_ms(e[k0], e[k1]))
    ms = float(np.mean(per_step))
    tokens = Bsz * T
    value = tokens / (ms / 1e3)
    own = own_io_bytes(cfg, dims)
    kf = algorithmic_flops(cfg, dims)
    alg = algorithmic_bytes(cfg, dims)
    # complex products run as three bf16 products each (split operands)
    flop_mult = 3 if cplx else 1
    kern = {}
    for n in names:
        avg = float(np.mean(per_kernel[n]))
        ent = {"avg_us": avg * 1e3, "own_io_bytes": own[n],
               "own_io_gbs": own[n] / (avg / 1e3) / 1e9}
        if n in kf:
            tf = kf[n] * flop_mult / (avg / 1e3) / 1e12
            ent.update({"alg_flops": kf[n], "mfma_executed_flops": kf[n] * flop_mult,
                        "mfma_tflops": tf, "mfma_frac": tf / MFMA_PEAK_TFLOPS[peak_name]})
        kern[n] = ent
    dom = max(names, key=lambda n: kern[n]["avg_us"])
    dom_s = kern[dom]["avg_us"] / 1e6
    traffic = measured_traffic(args.workload, dom)
    achieved = alg / dom_s / 1e9
    copy_gbs, copy_bytes = copy_reference(torch, dev, alg, flush)
    # the roofline: the whole forward's algorithmic bytes (x, dt, B, C in, y
    # out, once) over the dominant kernel's launch time, against 8 TB/s
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom,
            "alg_bytes": alg, "launch_us": dom_s * 1e6,
            "frac_of_copy": achieved / copy_gbs}
    if dom in kf:
        tf = kf[dom] * flop_mult / dom_s / 1e12
        roof["mfma"] = {"alg_flops": kf[dom], "executed_flops": kf[dom] * flop_mult,
                        "executed_dtype": "bf16x3" if cplx else dtype_name,
                        "tflops": tf, "peak": MFMA_PEAK_TFLOPS[peak_name], "unit": "TFLOP/s",
                        "frac": tf / MFMA_PEAK_TFLOPS[peak_name]}
        if cplx:
            f32e = kf[dom] / dom_s / 1e12
            roof["mfma"]["fp32_equivalent"] = {"tflops": f32e, "peak": MFMA_PEAK_TFLOPS["f32"],
                                               "frac": f32e / MFMA_PEAK_TFLOPS["f32"]}
    e2e = alg / (ms / 1e3) / 1e9
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(np.min(per_step)),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_name, "data": "synthetic",
        "config": {"workload": args.workload, "batch": Bsz, "seq_len": T, "heads": H,
                   "headdim": P, "d_state": N, "ngroups": G, "chunk": Q,
                   "complex": cplx, "inputs": "in_proj rows, read in place" if packed else
                   "separate arrays", "cache": "cold (Infinity Cache flushed between steps)"
                   if flush is not None else "warm"},
        "roofline": roof,
        "end_to_end": {"alg_bytes": alg, "gbs": e2e, "frac": e2e / HBM_PEAK_GBS,
                       "alg_flops": kf["whole_forward"], "frac_of_copy": e2e / copy_gbs},
        "achievable_hbm": {"kernel": "device copy (torch copy_)", "bytes_moved": copy_bytes,
                           "gbs": copy_gbs, "frac_of_peak": copy_gbs / HBM_PEAK_GBS,
                           "cache": "cold" if flush is not None else "warm"},
        "kernels": kern,
        "wall_ms_per_step_incl_flush": t_wall / args.steps * 1e3,
        "ms_per_step_with_kernel_events": float(np.mean(per_step_ev)),
    }
    if args.copy_ref:
        copy_counter_reference(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, cfg, dims, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_varlen(args, cfg):
    """Variable-length prefill: one step = one ssd_chunk_fwd_varlen call over
    the packed batch (its three kernels, the segment-table copy included).
    Roofline over the batch's algorithmic bytes (x, dt, B, C read once, y
    written once for its Ttot tokens) as for the uniform forward."""
    import torch
    import selective_state_space_09_amd as ssd
    from selective_state_space_09_amd import inputs
    inp = inputs.make_workload(args.workload, seed=0, with_h0=True)
    d0 = inp["dims"]
    Q = cfg["chunk"]
    Ttot, H, P, G, N = (d0[k] for k in ("Ttot", "H", "P", "G", "N"))
    dims = dict(Bsz=1, T=Ttot, H=H, P=P, G=G, N=N, Q=Q)
    dev = torch.device("cuda:0")

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {k: (up(v) if isinstance(v, np.ndarray) and k != "cu_seqlens" else v) for k, v in inp.items()}
    cu = np.ascontiguousarray(inp["cu_seqlens"], np.int32)
    nseq = cu.size - 1
    y = torch.empty((Ttot, H, P), dtype=torch.bfloat16, device=dev)
    hf = torch.empty((nseq, H, P, N), dtype=torch.float32, device=dev)
    L = ssd.lib()
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    nbytes = int(L.ssd_varlen_workspace_size(cup, nseq, H, P, G, N, Q))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.int32, device=dev)
    hip = Hip()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    fixed = (P_(d["x"]), P_(d["dt"]), P_(d["A"]), P_(d["B"]), P_(d["C"]), P_(d["D"]), P_(d["dt_bias"]),
             float(d["dt_min"]), float(d["dt_max"]), P_(d["h0"]), P_(y), P_(hf), cup, nseq, H, P, G, N, Q,
             ssd.SSD_BF16, P_(ws), ws.numel(), sp)

    def check(rc):
        if rc != 0:
            raise RuntimeError(L.ssd_last_error().decode())

    n_total = args.warmup + args.steps
    n_kern = max(10, args.steps // 2)
    step_evs = [(hip.event(), hip.event()) for _ in range(n_total)]
    evs = [[hip.event() for _ in range(6)] for _ in range(n_kern)]
    ev_arrays = [(ctypes.c_void_p * 6)(*[e.value for e in row]) for row in evs]
    for i in range(n_total):
        if flush is not None:
            flush.max()
        a, b = step_evs[i]
        hip.lib.hipEventRecord(a, sp)
        check(L.ssd_chunk_fwd_varlen(*fixed))
        hip.lib.hipEventRecord(b, sp)
    torch.cuda.synchronize()
    per_step = [hip.elapsed_ms(*step_evs[i]) for i in range(args.warmup, n_total)]
    for i in range(n_kern):
        if flush is not None:
            flush.max()
        check(L.ssd_chunk_fwd_varlen_ev(*fixed, ev_arrays[i]))
    torch.cuda.synchronize()
    vcfg = dict(kind="real", dtype="bf16")
    segs = kernel_segments(vcfg)
    kern = {}
    for n, (k0, k1) in segs.items():
        avg = float(np.mean([hip.elapsed_ms(evs[i][k0], evs[i][k1]) for i in range(n_kern)]))
        kern[n] = {"avg_us": avg * 1e3}
    ms = float(np.mean(per_step))
    alg = algorithmic_bytes(vcfg, dims)
    dom = max(kern, key=lambda n: kern[n]["avg_us"])
    dom_s = kern[dom]["avg_us"] / 1e6
    achieved = alg / dom_s / 1e9
    copy_gbs, copy_bytes = copy_reference(torch, dev, alg, flush)
    e2e = alg / (ms / 1e3) / 1e9
    out = {
        "metric": METRIC, "value": Ttot / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_median": float(np.median(per_step)), "ms_per_step_min": float(np.min(per_step)),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "sequences": [int(v) for v in np.diff(cu)], "tokens": Ttot,
                   "heads": H, "headdim": P, "d_state": N, "ngroups": G, "chunk": Q,
                   "cache": "cold (Infinity Cache flushed between steps)" if flush is not None else "warm"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload, dom),
                     "kernel": dom, "alg_bytes": alg, "launch_us": dom_s * 1e6,
                     "frac_of_copy": achieved / copy_gbs},
        "end_to_end": {"alg_bytes": alg, "gbs": e2e, "frac": e2e / HBM_PEAK_GBS},
        "achievable_hbm": {"kernel": "device copy (torch copy_)", "bytes_moved": copy_bytes,
                           "gbs": copy_gbs, "frac_of_peak": copy_gbs / HBM_PEAK_GBS},
        "kernels": kern,
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle.set_threads(len(os.sched_getaffinity(0)))
        # the oracle on the first k heads of every sequence, k doubled until a
        # run takes half the target
        nh, t_run = 1, 0.0
        while True:
            hs = list(range(nh))
            sub = {k: inp[k] for k in ("B", "C", "cu_seqlens", "dt_min", "dt_max")}
            t0 = time.perf_counter()
            oracle.fwd_varlen(np.ascontiguousarray(inp["x"][:, hs]), np.ascontiguousarray(inp["dt"][:, hs]),
                              inp["A"][hs], sub["B"], sub["C"], sub["cu_seqlens"], inp["D"][hs],
                              inp["dt_bias"][hs], sub["dt_min"], sub["dt_max"],
                              np.ascontiguousarray(inp["h0"][:, hs]))
            t_run = time.perf_counter() - t0
            if t_run >= args.cpu_seconds / 2 or nh >= H:
                break
            nh = min(H, 2 * nh)
        out["cpu_baseline"] = {"value": Ttot * (nh / H) / t_run, "unit": "tokens/s",
                               "cores": oracle.threads_used(), "kind": "oracle",
                               "sample": f"every sequence, the first {nh} of {H} heads, float64"}
    if args.copy_ref:
        copy_counter_reference(torch, dev)
    print(json.dumps(out), flush=True)


def bench_decode(args, cfg):
    """Decode workloads: one step = one decode call over the whole batch, state
    updated in place (real: 256 x 64 x 64 x 128 fp32; complex: 1024 x 16 x 64
    x 64 complex64, both 537 MB, above the 256 MB Infinity Cache)."""
    import torch
    import selective_state_space_09_amd as ssd
    from selective_state_space_09_amd import inputs
    cplx = cfg["kind"] == "complex_decode"
    inp = inputs.make_workload(args.workload, seed=0, steps=1)
    dev = torch.device("cuda:0")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h = up(inp["h0"])
    st = inp["steps"][0]
    x, dt, B, C = up(st["x"]), up(st["dt"]), up(st["B"]), up(st["C"])
    A = up(inp["A"])
    D = None if inp["D"] is None else up(inp["D"])
    bias = None if inp["dt_bias"] is None else up(inp["dt_bias"])
    Bsz, H, P, N = h.shape[:4]
    G = B.shape[1]
    y = torch.empty((Bsz, H, P), dtype=torch.float32, device=dev)
    L = ssd.lib()
    hip = Hip()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    if cplx:
        fn = L.ssd_complex_step_decode_ev
        args_c = (P_(h), P_(x), P_(dt), P_(A), P_(B), P_(C), P_(bias),
                  float(inp["dt_min"]), float(inp["dt_max"]), P_(y), Bsz, H, P, G, N, sp)
        kernel = "ssd_complex_decode_kernel"
    else:
        fn = L.ssd_step_decode_ev
        args_c = (P_(h), P_(x), P_(dt), P_(A), P_(B), P_(C), P_(D), P_(bias),
                  float(inp["dt_min"]), float(inp["dt_max"]), P_(y), Bsz, H, P, G, N, sp)
        kernel = "ssd_decode_kernel"
    n_total = args.warmup + args.steps
    evs = [(hip.event(), hip.event()) for _ in range(n_total)]
    for i in range(n_total):
        arr = (ctypes.c_void_p * 2)(evs[i][0].value, evs[i][1].value)
        rc = fn(*args_c, arr)
        if rc:
            raise RuntimeError(L.ssd_last_error().decode())
    torch.cuda.synchronize()
    times = [hip.elapsed_ms(a, b) for a, b in evs[args.warmup:]]
    ms = float(np.mean(times))
    # algorithmic bytes: the state read and written once, x and y, dt, and B/C
    nbytes = (2 * h.numel() * 4 + Bsz * H * P * 8 + Bsz * H * 4
              + 2 * Bsz * G * N * (8 if cplx else 4))
    gbs = nbytes / (ms / 1e3) / 1e9
    shape = "B1024 H16 P64 N64 complex" if cplx else "B256 H64 P64 N128"
    out = {"metric": f"SSD {'complex ' if cplx else ''}decode tokens/s ({shape})",
           "value": Bsz / (ms / 1e3),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "c64" if cplx else "f32", "data": "synthetic",
           "config": {"workload": args.workload, "batch": Bsz, "heads": H, "headdim": P,
                      "d_state": N, "ngroups": G},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS,
                        "traffic": measured_traffic(args.workload, kernel),
                        "kernel": kernel},
           "kernels": {kernel: {"avg_us": ms * 1e3, "alg_bytes": nbytes,
                                "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}}}
    if args.copy_ref:
        copy_counter_reference(torch, dev)
    print(json.dumps(out), flush=True)


def bench_conv(args, cfg):
    """Convolution workloads.  conv_bf16: one step = one ssd_conv1d_fwd call
    over the whole batch (B2 T2048, 4352 channels read from 8512-wide rows,
    split into x/B/C).  conv_decode_f32: one step = one ssd_conv1d_step over
    256 sequences, state in place.  The 512 MiB flush read runs between steps
    in both (the step's data would otherwise sit in the Infinity Cache)."""
    import torch
    import selective_state_space_09_amd as ssd
    from selective_state_space_09_amd import inputs
    decode = cfg["kind"] == "conv_decode"
    inp = inputs.make_workload(args.workload, seed=0, **({"steps": 1} if decode else {}))
    dims = inp["dims"]
    Bsz, HP, GN, ld = dims["Bsz"], dims["HP"], dims["GN"], dims["ld"]
    Ch = HP + 2 * GN
    T = 1 if decode else dims["T"]
    dev = torch.device("cuda:0")

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    w, bias = up(inp["w"]), up(inp["bias"])
    L = ssd.lib()
    hip = Hip()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.int32, device=dev)
    if decode:
        state = up(inp["state0"])
        xt = up(inp["steps"][0])
        x = torch.empty((Bsz, HP), dtype=torch.float32, device=dev)
        B = torch.empty((Bsz, GN), dtype=torch.float32, device=dev)
        C = torch.empty_like(B)
        fn = L.ssd_conv1d_step_ev
        args_c = (P_(state), P_(xt), ld, P_(w), P_(bias), 1, P_(x), P_(B), P_(C),
                  Bsz, HP, GN, 4, sp)
        kernel, es = "ssd_conv1d_step_kernel", 4
        # state read and written, the token row's channels read, x|B|C written
        nbytes = 2 * Bsz * 3 * Ch * 4 + 2 * Bsz * Ch * 4 + Ch * 20
        dtype_name = "f32"
    else:
        xbc = up(inp["xbc"])
        si = up(inp["state_in"])
        so = torch.empty_like(si)
        x = torch.empty((Bsz, T, HP), dtype=xbc.dtype, device=dev)
        B = torch.empty((Bsz, T, GN), dtype=xbc.dtype, device=dev)
        C = torch.empty_like(B)
        dcode = ssd.SSD_BF16 if xbc.dtype == torch.bfloat16 else ssd.SSD_F32
        es = 2 if dcode == ssd.SSD_BF16 else 4
        fn = L.ssd_conv1d_fwd_ev
        args_c = (P_(xbc), ld, P_(w), P_(bias), P_(si), 1, P_(x), P_(B), P_(C), P_(so),
                  Bsz, T, HP, GN, 4, dcode, sp)
        kernel = "ssd_conv1d_kernel"
        # the used channels of every row read once, x|B|C written once, taps,
        # bias and both states
        nbytes = 2 * Bsz * T * Ch * es + Ch * 20 + 2 * Bsz * 3 * Ch * 4
        dtype_name = "bf16" if es == 2 else "f32"
    n_total = args.warmup + args.steps
    evs = [(hip.event(), hip.event()) for _ in range(n_total)]
    for i in range(n_total):
        if flush is not None:
            flush.max()
        arr = (ctypes.c_void_p * 2)(evs[i][0].value, evs[i][1].value)
        rc = fn(*args_c, arr)
        if rc:
            raise RuntimeError(L.ssd_last_error().decode())
    torch.cuda.synchronize()
    times = [hip.elapsed_ms(a, b) for a, b in evs[args.warmup:]]
    ms = float(np.mean(times))
    gbs = nbytes / (ms / 1e3) / 1e9
    tokens = Bsz * T
    out = {"metric": (f"conv1d {'decode step' if decode else 'fwd'} tokens/s "
                      f"(k=4 SiLU over x|B|C, {Ch} channels)"),
           "value": tokens / (ms / 1e3),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dtype_name, "data": "synthetic",
           "config": {"workload": args.workload, "batch": Bsz, "seq_len": T, "channels": Ch,
                      "x_channels": HP, "bc_channels": GN, "row_stride": ld, "kernel_size": 4,
                      "cache": "cold (Infinity Cache flushed between steps)"
                      if flush is not None else "warm"},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS,
                        "traffic": measured_traffic(args.workload, kernel),
                        "kernel": kernel},
           "kernels": {kernel: {"avg_us": ms * 1e3, "alg_bytes": nbytes,
                                "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}}}
    if args.copy_ref:
        copy_counter_reference(torch, dev)
    if not decode and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_conv(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_conv(inp, target_s):
    """The float64 oracle convolution over the whole workload, repeated until
    about target_s seconds have passed (one pass takes well under a second)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    dims = inp["dims"]
    Ch = dims["HP"] + 2 * dims["GN"]
    reps, total = 0, 0.0
    while total < target_s:
        t0 = time.perf_counter()
        oracle.conv1d(inp["xbc"], inp["w"], inp["bias"], inp["state_in"], act=1, ch=Ch)
        total += time.perf_counter() - t0
        reps += 1
    return {"value": reps * dims["Bsz"] * dims["T"] / total, "unit": "tokens/s",
            "cores": oracle.threads_used(), "kind": "oracle",
            "sample": f"the whole workload ({dims['Bsz']} x {dims['T']} tokens x {Ch} channels), "
                      f"float64, {reps} passes in {total:.2f} s"}


BWD_KERNELS = ["ssd_state_bf16_kernel", "ssd_pass_bf16_kernel", "ssd_adj_state_kernel",
               "ssd_adj_pass_kernel", "ssd_bwd_dxdb_kernel", "ssd_bwd_dc_kernel",
               None, "ssd_bwd_dt_kernel", None,
               "ssd_bwd_reduce_kernel(dB, dC, dA)", None]


def bwd_kernel_costs(dims, nparts):
    """Algorithmic HBM bytes and MFMA flops of each kernel of one backward
    call (bf16 x/B/C/dy; every array a kernel must read or write counted once;
    flops: the lower-triangle in-chunk products and the boundary products)."""
    Bsz, T, H, P, G, N, Q = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N", "Q"))
    nc = -(-T // Q)
    nb = -(-Q // 64)
    x = Bsz * T * H * P * 2                 # x, dy, dx (bf16)
    bc = Bsz * T * G * N * 2                # B or C (bf16)
    st = Bsz * nc * H * P * N * 4           # fp32 chunk / boundary / adjoint states
    tok = Bsz * nc * H * Q * 8              # (cs, delta) per token
    dec = Bsz * H * nc * 4
    pt = Bsz * T * H * 4                    # one fp32 value per token and head
    part = nparts * Bsz * T * G * N * 4     # fp32 head-group partials of dB or dC
    out = Bsz * T * G * N * 4               # dB or dC
    units = Bsz * nc * H
    tri = Q * (Q + 1) / 2
    return {
        "ssd_state_bf16_kernel": (x + bc + Bsz * T * H * 4 + st + dec + tok, units * 2 * Q * P * N),
        "ssd_pass_bf16_kernel": (2 * st + dec, 0),
        "ssd_adj_state_kernel": (x + bc + tok + st, units * 2 * Q * P * N),
        # G in, R out, h_in in (the chunk constants' shares)
        "ssd_adj_pass_kernel": (3 * st + dec, 0),
        # x, dy, B, C, tok, R in; dx, x.v, dy.x, f2, col, row shares, dB partials out
        "ssd_bwd_dxdb_kernel": (3 * x + 2 * bc + tok + st + 4 * pt + pt * (nb + 1) / 2 + part,
                                units * (2 * tri * P * 2 + 2 * tri * N + 2 * Q * N * P * 2)
                                + Bsz * nc * G * 2 * tri * N),
        # x, dy, B, C, tok, h_in in; f1, dC partials out
        "ssd_bwd_dc_kernel": (2 * x + 2 * bc + tok + st + pt + part,
                              units * (2 * tri * P + 2 * tri * N + 2 * Q * P * N)),
        "ssd_bwd_dt_kernel": (Bsz * T * H * 4 + 6 * pt + pt * (nb + 1) / 2, 0),
        # dB, dC partials in, dB, dC out; the per-head sums of the chunk shares
        "ssd_bwd_reduce_kernel(dB, dC, dA)": (2 * (part + out) + Bsz * H * nc * 24 + H * 12, 0),
        # x, dy in and dx out; B, C in; dt in and ddt out; dB, dC out (fp32)
        "whole_backward": (3 * x + 2 * bc + Bsz * T * H * 8 + 2 * out, 0),
    }


def bench_bwd(args, cfg):
    """Backward workload: one step = one ssd_chunk_bwd call over the whole
    batch (B2 T2048 H64 P64 N128, bf16 x/B/C/dy; the forward's chunk states
    recomputed inside the call), the 512 MiB flush read between steps."""
    import torch
    import selective_state_space_09_amd as ssd
    from selective_state_space_09_amd import inputs
    inp = inputs.make_workload(args.workload, seed=0)
    Q = cfg["chunk"]
    dims = dict(inp["dims"], Q=Q)
    Bsz, T, H, P, G, N = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N"))
    dev = torch.device("cuda:0")

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    f32 = dict(dtype=torch.float32, device=dev)
    dx = torch.empty_like(d["x"])
    ddt = torch.empty((Bsz, T, H), **f32)
    dA, dD, dbias = (torch.empty(H, **f32) for _ in range(3))
    dB = torch.empty((Bsz, T, G, N), **f32)
    dC = torch.empty_like(dB)
    nbytes = ssd.ssd_bwd_workspace_size(Bsz, T, H, P, G, N, Q)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.int32, device=dev)
    L = ssd.lib()
    hip = Hip()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    fixed = (P_(d["x"]), P_(d["dt"]), P_(d["A"]), P_(d["B"]), P_(d["C"]), P_(d["D"]),
             P_(d["dt_bias"]), float(d["dt_min"]), float(d["dt_max"]), None, P_(d["dy"]), None,
             P_(dx), P_(ddt), P_(dA), P_(dB), P_(dC), P_(dD), P_(dbias), None,
             Bsz, T, H, P, G, N, Q, ssd.SSD_BF16, P_(ws), ws.numel(), sp)

    def check(rc):
        if rc != 0:
            raise RuntimeError(L.ssd_last_error().decode())

    n_total = args.warmup + args.steps
    step_evs = [(hip.event(), hip.event()) for _ in range(n_total)]
    for i in range(n_total):
        if flush is not None:
            flush.max()
        a, b = step_evs[i]
        hip.lib.hipEventRecord(a, sp)
        check(L.ssd_chunk_bwd(*fixed))
        hip.lib.hipEventRecord(b, sp)
    torch.cuda.synchronize()
    per_step = [hip.elapsed_ms(*step_evs[i]) for i in range(args.warmup, n_total)]
    n_kern = max(10, args.steps // 2)
    evs = [[hip.event() for _ in range(22)] for _ in range(n_kern)]
    for i in range(n_kern):
        if flush is not None:
            flush.max()
        arr = (ctypes.c_void_p * 22)(*[e.value for e in evs[i]])
        check(L.ssd_chunk_bwd_ev(*fixed, arr))
    torch.cuda.synchronize()
    nparts = (H // G) // max(k for k in range(1, min(4, H // G) + 1) if (H // G) % k == 0)
    costs = bwd_kernel_costs(dims, nparts)
    kern = {}
    for k, name in enumerate(BWD_KERNELS):
        if name is None:  # (a slot whose work runs in another slot's launch)
            continue
        avg = float(np.mean([hip.elapsed_ms(e[2 * k], e[2 * k + 1]) for e in evs]))
        nb_, fl = costs[name]
        ent = {"avg_us": avg * 1e3, "own_io_bytes": nb_, "own_io_gbs": nb_ / (avg / 1e3) / 1e9}
        if fl:
            tf = fl / (avg / 1e3) / 1e12
            ent.update({"alg_flops": fl, "mfma_tflops": tf,
                        "mfma_frac": tf / MFMA_PEAK_TFLOPS["bf16"]})
        kern[name] = ent
    ms = float(np.mean(per_step))
    dom = max(kern, key=lambda n: kern[n]["avg_us"])
    dom_s = kern[dom]["avg_us"] / 1e6
    traffic = measured_traffic(args.workload, dom)
    # the roofline: the whole backward's algorithmic bytes (x, dt, B, C, dy in,
    # dx, ddt, dB, dC out, once) over the dominant kernel's launch time
    whole = costs["whole_backward"][0]
    achieved = whole / dom_s / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom,
            "alg_bytes": whole, "launch_us": dom_s * 1e6}
    if "alg_flops" in kern[dom]:
        roof["mfma"] = {"alg_flops": kern[dom]["alg_flops"], "tflops": kern[dom]["mfma_tflops"],
                        "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                        "frac": kern[dom]["mfma_frac"]}
    out = {
        "metric": "SSD bwd tokens/s per layer (H64 P64 N128, bf16)", "value": Bsz * T / (ms / 1e3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": Bsz, "seq_len": T, "heads": H,
                   "headdim": P, "d_state": N, "ngroups": G, "chunk": Q,
                   "cache": "cold (Infinity Cache flushed between steps)"
                   if flush is not None else "warm"},
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(np.min(per_step)),
        "roofline": roof,
        "end_to_end": {"alg_bytes": whole, "gbs": whole / (ms / 1e3) / 1e9,
                       "frac": whole / (ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "kernels": kern,
    }
    if args.copy_ref:
        copy_counter_reference(torch, dev)
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        reps, total = 0, 0.0
        while total < args.cpu_seconds / 3:
            t0 = time.perf_counter()
            oracle.bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["dy"], inp["D"],
                       inp["dt_bias"], inp["dt_min"], inp["dt_max"], None, None, want_dh0=False)
            total += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = {
            "value": reps * Bsz * T / total, "unit": "tokens/s", "cores": oracle.threads_used(),
            "kind": "oracle",
            "sample": f"the whole workload (float64 adjoint recurrence), {reps} passes in {total:.2f} s"}
    print(json.dumps(out), flush=True)


# the 14 event slots of ssd_complex_chunk_bwd_ev; None: a slot no kernel fills
# (the chunk constants form inside the adjoint passing), and the group sums
# run only when a group holds several heads
CPLX_BWD_KERNELS = ["ssd_cplx_frame_kernel", "ssd_state_kernel(unit scale)", "ssd_pass_kernel",
                    "ssd_state_kernel(adjoint)", "ssd_f32_adj_pass_kernel", "ssd_f32_col_kernel",
                    "ssd_f32_row_kernel", None, "ssd_cplx_tau_kernel",
                    "ssd_cplx_rho_total_kernel", "ssd_f32_dt_kernel", "ssd_f32_dt_sum_kernel",
                    "ssd_f32_group_sum_kernel", "ssd_cplx_dh0_kernel"]


def cplx_bwd_costs(dims):
    """Algorithmic HBM bytes of the whole complex backward (x, dt, B, C, dy in;
    dx, ddt, dB, dC out; complex64 B/C/dB/dC, float32 x/dy/dx) and the fp32
    matrix flops of the two block kernels and the chunk-state kernels, in the
    rotated frame (2N real features), 64-token chunks."""
    Bsz, T, H, P, G, N = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N"))
    Q, NE = 64, 2 * N
    x = Bsz * T * H * P * 4
    bc = Bsz * T * G * N * 8
    units = Bsz * (T / Q) * H
    tri = Q * (Q + 1) / 2
    state = units * 2 * Q * P * NE
    col = units * (2 * Q * Q * NE + 2 * Q * Q * P + 2 * tri * P + 2 * Q * P * NE * 2 + 2 * tri * NE)
    row = units * (2 * Q * Q * NE + 2 * Q * Q * P + 2 * Q * P * NE + 2 * tri * NE)
    return {"whole_backward": 3 * x + 4 * bc + 2 * Bsz * T * H * 4,
            "flops": {"ssd_state_kernel(unit scale)": state, "ssd_state_kernel(adjoint)": state,
                      "ssd_f32_col_kernel": col, "ssd_f32_row_kernel": row}}


def bench_bwd_complex(args, cfg):
    """Complex backward at the Mamba-3-Lite layer shape: one step = one
    ssd_complex_chunk_bwd over the whole batch (B8 T2048 H16 P64 N64, chunk
    64, gradients of every input through y), the 512 MiB flush read between
    steps.  fp32 matrix products: MFMA figures against the fp32 peak."""
    import torch
    import selective_state_space_09_amd as ssd
    from selective_state_space_09_amd import inputs
    inp = inputs.make_workload(args.workload, seed=0)
    dims = dict(inp["dims"])
    Bsz, T, H, P, G, N = (dims[k] for k in ("Bsz", "T", "H", "P", "G", "N"))
    Q = cfg["chunk"]
    dev = torch.device("cuda:0")
    d = {k: (torch.from_numpy(np.ascontiguousarray(v)).to(dev) if isinstance(v, np.ndarray) else v)
         for k, v in inp.items()}
    f32 = dict(dtype=torch.float32, device=dev)
    dx = torch.empty((Bsz, T, H, P), **f32)
    ddt = torch.empty((Bsz, T, H), **f32)
    dA = torch.empty((H, 2), **f32)
    dB = torch.empty((Bsz, T, G, N, 2), **f32)
    dC = torch.empty_like(dB)
    dbias = torch.empty(H, **f32)
    ws = torch.empty(ssd.ssd_complex_bwd_workspace_size(Bsz, T, H, P, G, N), dtype=torch.uint8,
                     device=dev)
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.int32, device=dev)
    L = ssd.lib()
    hip = Hip()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    fixed = (P_(d["x"]), P_(d["dt"]), P_(d["A"]), P_(d["B"]), P_(d["C"]), P_(d["dt_bias"]),
             float(d["dt_min"]), float(d["dt_max"]), None, P_(d["dy"]), None, P_(dx), P_(ddt),
             P_(dA), P_(dB), P_(dC), P_(dbias), None, Bsz, T, H, P, G, N, Q, P_(ws), ws.numel(), sp)

    def check(rc):
        if rc != 0:
            raise RuntimeError(L.ssd_last_error().decode())

    n_total = args.warmup + args.steps
    step_evs = [(hip.event(), hip.event()) for _ in range(n_total)]
    for i in range(n_total):
        if flush is not None:
            flush.max()
        a, b = step_evs[i]
        hip.lib.hipEventRecord(a, sp)
        check(L.ssd_complex_chunk_bwd(*fixed))
        hip.lib.hipEventRecord(b, sp)
    torch.cuda.synchronize()
    per_step = [hip.elapsed_ms(*step_evs[i]) for i in range(args.warmup, n_total)]
    n_kern = max(10, args.steps // 2)
    nev = 2 * len(CPLX_BWD_KERNELS)
    evs = [[hip.event() for _ in range(nev)] for _ in range(n_kern)]
    for i in range(n_kern):
        if flush is not None:
            flush.max()
        arr = (ctypes.c_void_p * nev)(*[e.value for e in evs[i]])
        check(L.ssd_complex_chunk_bwd_ev(*fixed, arr))
    torch.cuda.synchronize()
    costs = cplx_bwd_costs(dims)
    kern = {}
    for k, name in enumerate(CPLX_BWD_KERNELS):
        if name is None or (name == "ssd_f32_group_sum_kernel" and G == H):
            continue
        avg = float(np.mean([hip.elapsed_ms(e[2 * k], e[2 * k + 1]) for e in evs]))
        ent = {"avg_us": avg * 1e3}
        fl = costs["flops"].get(name)
        if fl:
            tf = fl / (avg / 1e3) / 1e12
            ent.update({"alg_flops": fl, "mfma_tflops": tf, "mfma_frac": tf / MFMA_PEAK_TFLOPS["f32"]})
        kern[name] = ent
    ms = float(np.mean(per_step))
    dom = max(kern, key=lambda n: kern[n]["avg_us"])
    dom_s = kern[dom]["avg_us"] / 1e6
    whole = costs["whole_backward"]
    achieved = whole / dom_s / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload, dom),
            "kernel": dom, "alg_bytes": whole, "launch_us": dom_s * 1e6}
    if "alg_flops" in kern[dom]:
        roof["mfma"] = {"alg_flops": kern[dom]["alg_flops"], "tflops": kern[dom]["mfma_tflops"],
                        "executed_dtype": "f32", "peak": MFMA_PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                        "frac": kern[dom]["mfma_frac"]}
    out = {
        "metric": "SSD complex bwd tokens/s per layer (H16 P64 N64 complex64)",
        "value": Bsz * T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "batch": Bsz, "seq_len": T, "heads": H, "headdim": P,
                   "d_state": N, "ngroups": G, "chunk": Q, "complex": True,
                   "cache": "cold (Infinity Cache flushed between steps)" if flush is not None
                   else "warm"},
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(np.min(per_step)),
        "roofline": roof,
        "end_to_end": {"alg_bytes": whole, "gbs": whole / (ms / 1e3) / 1e9,
                       "frac": whole / (ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "kernels": kern,
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        # one sequence (its H recurrences) at a time, repeated to ~cpu_seconds / 3
        one = {k: (np.ascontiguousarray(v[:1]) if isinstance(v, np.ndarray) and v.ndim >= 3 else v)
               for k, v in inp.items()}
        reps, total = 0, 0.0
        while total < args.cpu_seconds / 3:
            t0 = time.perf_counter()
            oracle.complex_bwd(one["x"], one["dt"], one["A"], one["B"], one["C"], one["dy"],
                               one["dt_bias"], one["dt_min"], one["dt_max"], None, None,
                               want_dh0=False)
            total += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = {
            "value": reps * T / total, "unit": "tokens/s", "cores": oracle.threads_used(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"one of the {Bsz} sequences ({H} complex recurrences of T={T}, float64 "
                      f"adjoint), {reps} runs in {total:.2f} s; tokens/s of that sequence"}
    if args.copy_ref:
        copy_counter_reference(torch, dev)
    print(json.dumps(out), flush=True)


def bench_mimo(args, cfg):
    """MIMO head mixer: one step = one ssd_mimo_fwd over the whole batch (B8
    T2048, 1024 features per token, fp32 y in, bf16 W and z), the 512 MiB
    flush read between steps.  Roofline: the matrix cores (2 M K N flops
    against the bf16 dense peak), with the HBM figure beside it."""
    import torch
    import selective_state_space_09_amd as ssd
    from selective_state_space_09_amd import inputs
    inp = inputs.make_workload(args.workload, seed=0)
    d = inp["dims"]
    Bsz, T, H, P = d["Bsz"], d["T"], d["H"], d["P"]
    dev = torch.device("cuda:0")
    y = torch.from_numpy(inp["y"]).to(dev)
    W = torch.from_numpy(inp["W"].view(np.int16)).view(torch.bfloat16).to(dev)
    z = torch.empty((Bsz, T, H, P), dtype=torch.bfloat16, device=dev)
    L = ssd.lib()
    hip = Hip()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.int32, device=dev)
    M, K = Bsz * T, H * P
    n_total = args.warmup + args.steps
    evs = [(hip.event(), hip.event()) for _ in range(n_total)]
    for i in range(n_total):
        if flush is not None:
            flush.max()
        arr = (ctypes.c_void_p * 2)(evs[i][0].value, evs[i][1].value)
        rc = L.ssd_linear_fwd_ev(ctypes.c_void_p(y.data_ptr()), ssd.SSD_F32,
                                 ctypes.c_void_p(W.data_ptr()), ctypes.c_void_p(z.data_ptr()),
                                 ssd.SSD_BF16, M, K, K, sp, arr)
        if rc:
            raise RuntimeError(L.ssd_last_error().decode())
    torch.cuda.synchronize()
    times = [hip.elapsed_ms(a, b) for a, b in evs[args.warmup:]]
    ms = float(np.mean(times))
    flops = 2.0 * M * K * K
    nbytes = M * K * 4 + K * K * 2 + M * K * 2
    tf = flops / (ms / 1e3) / 1e12
    gbs = nbytes / (ms / 1e3) / 1e9
    out = {"metric": "MIMO head mixer tokens/s (B8 T2048 H16 P64, 1024 x 1024 bf16 weight)",
           "value": M / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms,
           "ms_per_step_median": float(np.median(times)), "ms_per_step_min": float(np.min(times)),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": args.workload, "batch": Bsz, "seq_len": T, "heads": H,
                      "headdim": P, "features": K, "x_dtype": "f32", "out_dtype": "bf16",
                      "cache": "cold (Infinity Cache flushed between steps)"
                      if flush is not None else "warm"},
           "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_PEAK_TFLOPS["bf16"],
                        "unit": "TFLOP/s", "frac": tf / MFMA_PEAK_TFLOPS["bf16"],
                        "traffic": measured_traffic(args.workload, "ssd_linear_kernel"),
                        "kernel": "ssd_linear_kernel", "alg_flops": flops,
                        "launch_us": ms * 1e3,
                        "hbm": {"alg_bytes": nbytes, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS}},
           "kernels": {"ssd_linear_kernel": {"avg_us": ms * 1e3, "alg_bytes": nbytes,
                                             "alg_flops": flops}}}
    if args.copy_ref:
        copy_counter_reference(torch, dev)
    if not args.no_cpu_baseline:
        import oracle
        rows = 256
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < args.cpu_seconds / 4:
            oracle.mimo(inp["y"][:1, :rows], inp["W"])
            reps += 1
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": reps * rows / el, "unit": "tokens/s",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "cpu_model": cpu_model(),
                               "sample": f"{reps} passes over {rows} token rows (float64 numpy "
                                         f"matrix product) in {el:.2f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
