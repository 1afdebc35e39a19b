"""Throughput of the expert-gather GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads C2,C3,...]
                    [--no-cpu] [--no-extra]

A step is one qmv_gather_moe call (expert dispatch, weight streaming, decode,
block dots, scale epilogue, cross-lane reduction, store) on the gpt-oss-20b
MoE decode shape: 4 of 32 MXFP4 experts, K = N = 2880, one bf16 token.
Inputs are synthetic and seeded (module ``synth``) and already resident in
HBM.  To measure HBM rather than the 256 MB Infinity Cache, the weights live
in many layer copies (>= 1 GB in total) that successive calls rotate through,
and every call draws fresh expert ids.  The K timed calls are captured once
into a HIP graph (torch.cuda.CUDAGraph) and replayed, so host launch overhead
is not part of the time.  The graph also holds a one-thread kernel before the
first call and after the last that stores the GPU's 100 MHz real-time counter
(qmv_probe_clock); the time per call is their difference over K, so the graph
replay's fixed start-up (6-11 us per replay, whatever K) is not spread over
the calls and a 20-step run reads what a 1000-step run does.  HIP events on
the replay stream around the whole replay are reported beside it
(``us_per_call_replay_events``).  The replay is bracketed by device
synchronizations.

Prints ONE JSON line.  ``value`` is effective weight GB/s (code + scale bytes
of the experts a call reads / time per call).  ``roofline`` relates the
kernel's algorithmic bytes (weights + activations + ids + output) per launch
to the 8 TB/s HBM peak.  ``stream_ceiling`` times a read-only probe kernel
over exactly the same code and scale bytes (no decode, no ids), so the GEMV's
time can also be read against what the memory system delivers for that
transfer.  Each workload also gets a hot-cache time (the same buffers every
call, so the Infinity Cache serves them).  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload on all host cores, and
``cpu_baseline_1thread`` on one.  ``workloads`` lists the
other shapes measured the same way (not the headline), among them the fused
gate/up + SwiGLU calls (qmv_gather_moe_swiglu) C2gu and C3gu and the down
projections with the router-weighted combine (qmv_gather_moe_combine) C4c and
C2c, the 2-bit and 3-bit gathers fed bf16 activations that the kernel
quantizes while staging them, C3q and C4q, and the gpt-oss gather with MXFP4
weights and int8 activations (fp16 scale per 32), C2i, and a gpt-oss prefill
chunk (512 tokens x top-4 of 32 experts) on the expert-batched matrix-core
path, C6, whose entry also carries its MFMA rate against the dense bf16 peak,
and the same chunk's down projection with the router-weighted combine, C6c.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
# int8 dot products on the vector ALU (v_dot4_i32_i8: 4 multiply-adds per lane,
# 16 lanes per SIMD per clock): 256 CUs x 4 SIMDs x 16 x 8 ops x 2.4 GHz
DOT4_I8_PEAK_TOPS = 256 * 4 * 16 * 8 * 2.4e9 / 1e12
WFMT = {"mxfp4": 0, "cb2": 1, "cb3": 2}
HEADLINE = "C2"
METRIC = "effective weight GB/s and µs/call per expert-gather GEMV; % of HBM peak"


def kernel_source_hash():
    """sha256[:16] over the kernel sources (names and code, sorted), with the
    comments and blank space taken out, so that an edit of comments alone
    keeps the hash (and with it the profiled figures) of the same code."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bit_block_quantized_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)       # the sources hold no "//" or "/*" in strings
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE
    (profiles/qmv_traffic_pmc.md), or None if the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "qmv_traffic_pmc.md")
    try:
        with open(path) as f:
            txt = f.read()
    except OSError:
        return None
    vals = dict(line.strip().split(": ", 1) for line in txt.splitlines()
                if line.strip().startswith("traffic_") and ": " in line)
    if vals.get("traffic_source_sha256_16") != kernel_source_hash():
        return None
    v = vals.get(f"traffic_bytes_per_launch_{name}")
    return float(v) if v else None


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def weight_bytes(wl, n_experts):
    import synth
    return n_experts * wl.N * (synth.row_code_bytes(wl.wfmt, wl.K) + synth.row_scale_bytes(wl.wfmt, wl.K))


def other_bytes(wl):
    """Activation, scale, id and output bytes of one call."""
    V = wl.M * wl.top_k if (wl.kind in ("gather", "combine") and wl.x_per_slot) else wl.M
    bf = wl.afmt in ("bf16", "bf16q8")
    xb = V * wl.K * (2 if bf else 1) + (0 if bf else V * (wl.K // 32) * 2)
    routed = wl.kind in ("gather", "gate_up", "combine")
    outs = wl.M * (wl.top_k if wl.kind in ("gather", "gate_up") else 1) * wl.N
    ids = 4 * wl.M * wl.top_k if routed else 0
    route_w = 4 * wl.M * wl.top_k if wl.kind == "combine" else 0
    return xb + ids + route_w + 4 * outs


# Rotation plan: layer copies so that between two reads of the same weights
# more than the 256 MB Infinity Cache of other weights is read.
ROTATION = {"C1": 1, "C2": 32, "C3": 2, "C4": 2, "C5a": 4, "C5b": 40, "C2gu": 4, "C3gu": 1,
            "C4c": 2, "C2c": 32, "C3q": 2, "C4q": 2, "C2i": 32, "C6": 8, "C6gu": 4, "C6d": 40,
            "C7": 1, "C8": 1, "C6c": 8, "C8c": 1}


def merge_regions(regions):
    """(address, bytes) ranges sorted, with touching ranges joined (adjacent
    experts of one tensor are one range), each under 2 GiB."""
    out = []
    for a, n in sorted(regions):
        if out and out[-1][0] + out[-1][1] == a and out[-1][1] + n < (1 << 31):
            out[-1] = (out[-1][0], out[-1][1] + n)
        else:
            out.append((a, n))
    return out


class Prepared:
    """Device-resident inputs of one workload plus per-call raw arguments.

    ``args[i]`` addresses layer copy i % L (cold: the weights rotate through
    more than the Infinity Cache holds); ``args_hot[i]`` always addresses copy
    0 (hot: the same buffers every call).  ``regions[i]`` lists the (address,
    bytes) ranges of codes and scales call i must read, for the stream probe.
    """

    def __init__(self, name, calls, rotate=True):
        import torch

        import bit_block_quantized_amd as q
        import synth
        self.name = name
        self.wl = wl = synth.workload(name)
        gate_up = wl.kind == "gate_up"
        self.inp = inp = synth.make_gate_up(wl) if gate_up else synth.make(wl)
        self.L = ROTATION[name] if rotate else 1
        dev = torch.device("cuda")

        def layers(a):
            a0 = torch.from_numpy(a).to(dev)
            t = torch.empty((self.L,) + tuple(a0.shape), dtype=torch.uint8, device=dev)
            for layer in range(self.L):
                t[layer].copy_(a0)
            return t

        tensors = [(inp.gcodes, inp.gscales), (inp.ucodes, inp.uscales)] if gate_up else \
            [(inp.codes, inp.scales)]
        self.w = [(layers(c), layers(sc)) for c, sc in tensors]
        if wl.afmt in ("bf16", "bf16q8"):
            self.x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
            self.xs = None
        else:
            self.x = torch.from_numpy(inp.x).to(dev)
            self.xs = torch.from_numpy(inp.xs.view(np.float16)).to(dev)
        routed = wl.kind in ("gather", "gate_up", "combine")
        combine = wl.kind == "combine"
        self.rw = torch.from_numpy(inp.extra["weights"]).to(dev) if combine else None
        if routed:
            if name in ("C3", "C4", "C3gu", "C4c", "C3q", "C4q"):
                ids = synth.disjoint_id_stream(wl.seed + 100, calls, wl.top_k, wl.E)
            else:
                ids = synth.id_stream(wl.seed + 100, calls, wl.M, wl.top_k, wl.E)
            self.ids_host = ids
            self.ids = torch.from_numpy(ids).to(dev)
            experts = [np.unique(i) for i in ids]
            self.y = torch.empty((wl.M, wl.N) if combine else (wl.M, wl.top_k, wl.N),
                                 dtype=torch.float32, device=dev)
        else:
            self.ids_host = None
            self.ids = None
            experts = [np.zeros(1, np.int64) for _ in range(calls)]
            self.y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        self.calls = calls
        n_unique = np.array([len(e) for e in experts])
        self.wbytes = np.array([weight_bytes(wl, u) for u in n_unique], np.float64) * len(self.w)
        pairs = (np.array([(i >= 0).sum() for i in ids], np.float64) if routed
                 else np.full(calls, float(wl.M)))
        self.flops = 2.0 * pairs * wl.N * wl.K * len(self.w)
        self.abytes = self.wbytes + other_bytes(wl)
        self.lib = q.lib()
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)
        rcb = synth.row_code_bytes(wl.wfmt, wl.K) * wl.N
        rsb = synth.row_scale_bytes(wl.wfmt, wl.K) * wl.N
        afmt = {"bf16": 0, "q8": 1, "bf16q8": 2}[wl.afmt]
        xs = None if self.xs is None else self.xs.data_ptr()
        self.args, self.args_hot, self.regions = [], [], []
        for i in range(calls):
            for hot in (False, True):
                layer = 0 if hot else i % self.L
                wp = [(c.data_ptr() + layer * c[0].numel(), sc.data_ptr() + layer * sc[0].numel())
                      for c, sc in self.w]
                idp = None if self.ids is None else self.ids.data_ptr() + i * wl.M * wl.top_k * 4
                if gate_up:
                    a = (WFMT[wl.wfmt], wp[0][0], wp[0][1], wp[1][0], wp[1][1], wl.E, idp, wl.M,
                         wl.top_k, afmt, self.x.data_ptr(), xs, self.y.data_ptr(), wl.N, wl.K)
                elif combine:
                    a = (WFMT[wl.wfmt], wp[0][0], wp[0][1], wl.E, idp, self.rw.data_ptr(), wl.M,
                         wl.top_k, afmt, self.x.data_ptr(), xs, int(wl.x_per_slot),
                         self.y.data_ptr(), wl.N, wl.K)
                elif routed:
                    a = (WFMT[wl.wfmt], wp[0][0], wp[0][1], wl.E, idp, wl.M, wl.top_k, afmt,
                         self.x.data_ptr(), xs, int(wl.x_per_slot), self.y.data_ptr(), wl.N, wl.K)
                else:
                    a = (WFMT[wl.wfmt], wp[0][0], wp[0][1], afmt, self.x.data_ptr(), xs,
                         self.y.data_ptr(), wl.M, wl.N, wl.K)
                (self.args_hot if hot else self.args).append(a)
                if not hot:
                    reg = merge_regions([(cp + int(e) * rcb, rcb) for cp, _ in wp for e in experts[i]] +
                                        [(sp + int(e) * rsb, rsb) for _, sp in wp for e in experts[i]])
                    n = len(reg)
                    self.regions.append((n, (ctypes.c_void_p * n)(*[r[0] for r in reg]),
                                         (ctypes.c_longlong * n)(*[r[1] for r in reg])))

    def call(self, i, stream_handle, hot=False):
        a = (self.args_hot if hot else self.args)[i]
        if self.wl.kind == "gate_up":
            s = self.lib.qmv_gather_moe_swiglu(*a, ctypes.c_void_p(stream_handle))
        elif self.wl.kind == "gather":
            s = self.lib.qmv_gather_moe(*a, ctypes.c_void_p(stream_handle))
        elif self.wl.kind == "combine":
            s = self.lib.qmv_gather_moe_combine(*a, ctypes.c_void_p(stream_handle))
        else:
            s = self.lib.qmv_dense(*a, ctypes.c_void_p(stream_handle))
        if s != 0:
            raise RuntimeError(f"{self.name}: status {s}")

    def probe(self, i, stream_handle, variant):
        n, ptrs, sizes = self.regions[i]
        s = self.lib.qmv_probe_stream_read(n, ptrs, sizes, variant, self.sink.data_ptr(),
                                           ctypes.c_void_p(stream_handle))
        if s != 0:
            raise RuntimeError(f"{self.name}: probe status {s}")


_FLUSH = {}


def flush_caches(stream):
    """Read 512 MiB of memory that no workload touches (the stream probe over
    a buffer of its own), so that neither L2 nor the 256 MB Infinity Cache
    holds any weights when a timed replay starts."""
    import torch

    import bit_block_quantized_amd as q
    if "buf" not in _FLUSH:
        _FLUSH["buf"] = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
        _FLUSH["sink"] = torch.zeros(1, dtype=torch.int32, device="cuda")
        base, n = _FLUSH["buf"].data_ptr(), 4
        _FLUSH["regions"] = [(base + r * (128 << 20), 128 << 20) for r in range(n)]
    q.qmv_probe_stream_read(_FLUSH["regions"], 3, _FLUSH["sink"], stream=stream)


class ClockSampler:
    """Polls the shader and memory clock levels (sysfs pp_dpm_sclk and
    pp_dpm_mclk, the level in use marked '*') from a host thread while the
    timed work runs; reports each level seen with its sample count."""

    def __init__(self):
        import glob
        import threading
        self.files = [f for d in sorted(glob.glob("/sys/class/drm/card*/device"))
                      for f in (os.path.join(d, "pp_dpm_sclk"), os.path.join(d, "pp_dpm_mclk"))
                      if os.path.exists(f)]
        self.seen = {}
        self.n = 0
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set() and self.files:
            for f in self.files:
                try:
                    with open(f) as fh:
                        cur = [ln.strip() for ln in fh if ln.strip().endswith("*")]
                except OSError:
                    continue
                key = (os.path.basename(os.path.dirname(os.path.dirname(f))) + ":" +
                       os.path.basename(f), cur[0] if cur else None)
                self.seen[key] = self.seen.get(key, 0) + 1
            self.n += 1

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def report(self):
        if not self.files:
            return None
        out = {}
        for (f, lvl), c in sorted(self.seen.items(), key=lambda kv: str(kv[0])):
            out.setdefault(f, {})[str(lvl)] = c
        return {"sampled_during_timed_replay": out, "polls": self.n}


# The last time_graph call's two measures of the same replay (seconds per call).
LAST_REPLAY = {}
_STAMPS = {}
RTC_HZ = 100e6          # the GPU real-time counter qmv_probe_clock stores


def time_graph(fn, first, count, clocks=None):
    """Capture fn(i, stream) for i in [first, first+count) into one graph,
    with a GPU clock stamp (qmv_probe_clock) before the first call and after
    the last, replay it untimed for at least 30 ms (graph upload, clocks up),
    read 512 MiB of unrelated memory so no cache holds the weights, then
    replay it timed between HIP events.
    Returns seconds per call between the two stamps: the calls and the gaps
    between them, on the GPU's own clock.  The HIP events around the replay
    also hold the replay's fixed start-up (about 6-11 us per replay, which a
    20-call replay would spread over its calls); LAST_REPLAY keeps both.
    ``clocks`` (a ClockSampler) polls the clock levels during the timed replay."""
    import torch

    import bit_block_quantized_amd as q
    if "t" not in _STAMPS:
        _STAMPS["t"] = torch.zeros(2, dtype=torch.int64, device="cuda")
    st = _STAMPS["t"]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for i in range(first, min(first + 3, first + count)):   # eager warm-up on the stream
            fn(i, s.cuda_stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        h = torch.cuda.current_stream()
        q.qmv_probe_clock(st[0:1], stream=h)
        for i in range(first, first + count):
            fn(i, h.cuda_stream)
        q.qmv_probe_clock(st[1:2], stream=h)
    torch.cuda.synchronize()
    # untimed replays for at least 30 ms of GPU time: graph upload, and the
    # clocks ramped up (a short graph replayed for only 3 ms still ran its
    # first timed replay 5% slow)
    t_end = time.perf_counter() + 0.03
    for _ in range(2000):
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if clocks is not None:
        clocks.__enter__()
    with torch.cuda.stream(s):
        # the flush, the start event and the replay are queued back to back:
        # while the GPU reads the flush buffer the host submits the graph
        flush_caches(s)
        e0.record(s)
        g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    if clocks is not None:
        clocks.__exit__(None, None, None)
    ticks = st.cpu().tolist()
    gpu = (ticks[1] - ticks[0]) / RTC_HZ / count
    ev = e0.elapsed_time(e1) * 1e-3 / count
    LAST_REPLAY.clear()
    LAST_REPLAY.update(gpu_clock=gpu, events=ev)
    return gpu


def time_eager(p, first, count):
    """The same calls launched one by one from Python (host-bound reference)."""
    import torch
    s = torch.cuda.current_stream()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(first, first + count):
        p.call(i, s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / count


def stream_ceiling(p, first, count):
    """Best time per call over the probe's launch shapes for reading exactly
    the bytes of calls [first, first+count): the practical read ceiling."""
    import bit_block_quantized_amd as q
    best = None
    for v in range(q.PROBE_VARIANTS):
        t = time_graph(lambda i, h: p.probe(i, h, v), first, count)
        if best is None or t < best[0]:
            best = (t, v)
    return best


def stream_sweep(sizes_mib=(1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024)):
    """Time the read-only stream probe over one region of S bytes for a range
    of S (best of its launch shapes, each call on a fresh part of a 2 GiB
    buffer so no cache holds it), and fit t = t0 + S / BW by least squares
    over S >= 4 MiB: t0 is the fixed cost of one launch (dispatch, first
    request's latency, drain) and BW the streaming bandwidth."""
    import torch

    import bit_block_quantized_amd as q
    total = 2 << 30
    buf = torch.zeros(total, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()
    rows = []
    for mib in sizes_mib:
        size = mib << 20
        slots = total // size
        calls = max(20, min(400, (8 << 30) // size))

        def probe(i, h, v, size=size, slots=slots):
            ptrs = (ctypes.c_void_p * 1)(base + (i % slots) * size)
            sizes = (ctypes.c_longlong * 1)(size)
            s = q.lib().qmv_probe_stream_read(1, ptrs, sizes, v, sink.data_ptr(), ctypes.c_void_p(h))
            if s != 0:
                raise RuntimeError(f"probe status {s}")
        best = None
        for v in range(q.PROBE_VARIANTS):
            t = time_graph(lambda i, h: probe(i, h, v), 0, calls)
            if best is None or t < best[0]:
                best = (t, v)
        rows.append({"MiB": mib, "us": round(best[0] * 1e6, 3),
                     "GBps": round(size / best[0] / 1e9, 1), "variant": best[1]})
        print(f"stream sweep {mib} MiB: {best[0] * 1e6:.3f} us, {size / best[0] / 1e9:.1f} GB/s",
              file=sys.stderr, flush=True)
    fit = [r for r in rows if r["MiB"] >= 4]
    S = np.array([r["MiB"] * 1048576.0 for r in fit])
    T = np.array([r["us"] * 1e-6 for r in fit])
    A = np.stack([np.ones_like(S), S], axis=1)
    (t0, inv_bw), *_ = np.linalg.lstsq(A, T, rcond=None)
    return {"sweep": rows, "fit": {"t0_us": round(t0 * 1e6, 3), "BW_GBps": round(1.0 / inv_bw / 1e9, 1),
                                   "over": "S >= 4 MiB"}}


def measure(name, steps, warmup, hot=True, clocks=None):
    """Cold (rotated) timing of the workload, then the stream ceiling for the
    same calls, the hot-cache timing and the eager-launch timing."""
    import torch
    print(f"bench: {name}: preparing inputs", file=sys.stderr, flush=True)
    p = Prepared(name, warmup + steps)
    print(f"bench: {name}: timing {steps} calls", file=sys.stderr, flush=True)
    if warmup:
        time_graph(p.call, 0, warmup)
    t = time_graph(p.call, warmup, steps, clocks=clocks)
    t_events = LAST_REPLAY["events"]
    sel = slice(warmup, warmup + steps)
    wb = float(p.wbytes[sel].mean())
    ab = float(p.abytes[sel].mean())
    res = {
        "us_per_call": t * 1e6,
        "us_per_call_replay_events": t_events * 1e6,
        "weight_bytes_per_call": wb,
        "algorithmic_bytes_per_call": ab,
        "eff_weight_GBps": wb / t / 1e9,
        "pct_hbm_peak": 100.0 * (ab / t / 1e9) / HBM_PEAK_GBS,
        "layers_rotated": p.L,
    }
    if p.wl.M > 4:
        # many vectors per expert: also a product (2 ops per weight per routed
        # vector), on the matrix cores (MXFP4 x bf16) or as int8 dot products
        # on the vector ALU (int8 activations)
        fl = float(p.flops[sel].mean())
        res["flops_per_call"] = fl
        if p.wl.afmt == "bf16":
            res["mfma_TFLOPs"] = fl / t / 1e12
            res["pct_mfma_bf16_peak"] = 100.0 * fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS
        else:
            res["int8_TOPs"] = fl / t / 1e12
            res["pct_dot4_i8_alu_peak"] = 100.0 * fl / t / 1e12 / DOT4_I8_PEAK_TOPS
    ts, v = stream_ceiling(p, warmup, min(steps, 500))
    wcode = float(p.wbytes[warmup:warmup + min(steps, 500)].mean())
    res["stream_ceiling_us_per_call"] = ts * 1e6
    res["stream_ceiling_GBps"] = wcode / ts / 1e9
    res["pct_of_stream_ceiling"] = 100.0 * ts / t
    res["stream_probe_variant"] = v
    if hot:
        th = time_graph(lambda i, h: p.call(i, h, hot=True), warmup, min(steps, 500))
        res["hot_us_per_call"] = th * 1e6
    te = time_eager(p, warmup, min(steps, 200))
    res["us_per_call_eager_launch"] = te * 1e6
    torch.cuda.synchronize()
    return p, res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, target_s=10.0, threads=None):
    """The oracle (as it stands) on whole calls of the workload, ``threads``
    host threads (default: all cores) over disjoint output slices, for about
    ``target_s`` seconds; the rate and the median time per call."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import oracle_call
    import synth
    wl = p.wl
    cores = threads or host_cores()
    calls = 0
    t0 = time.perf_counter()
    wbytes = 0.0
    per_call = []
    while True:
        i = calls % p.calls
        inp = p.inp
        if p.ids_host is not None:
            inp = synth.Inputs(wl, p.inp.codes, p.inp.scales, p.ids_host[i], p.inp.x, p.inp.xs)
        t1 = time.perf_counter()
        oracle_call(inp, nthreads=cores)
        per_call.append(time.perf_counter() - t1)
        wbytes += float(p.wbytes[i])
        calls += 1
        el = time.perf_counter() - t0
        if el >= target_s or calls >= 10000:
            break
    return {
        "value": wbytes / el / 1e9,
        "unit": "GB/s",
        "us_per_call": el / calls * 1e6,
        "us_per_call_median": float(np.median(per_call)) * 1e6,
        "cores": cores,
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": f"{calls} complete {wl.name} calls (fresh ids, {wl.M} token(s), "
                  f"K={wl.K}, N={wl.N}), fp64 C oracle, {cores} thread(s) over disjoint outputs, "
                  f"{el:.1f} s wall",
    }


def gpu_clocks():
    """Shader and memory clock levels from sysfs after the run: (level marked
    in use, highest level), or None where the driver does not expose them."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for kind in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, kind)) as f:
                    levels = [ln.strip() for ln in f if ln.strip()]
            except OSError:
                continue
            cur = [ln for ln in levels if ln.endswith("*")]
            out[f"{os.path.basename(os.path.dirname(dev))}:{kind}"] = \
                (cur[0] if cur else None, levels[-1] if levels else None)
    return out or None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workloads", default="C1,C3,C4,C5a,C5b,C2gu,C3gu,C4c,C2c,C3q,C4q,C2i,C6,C6c,C7,C8",
                    help="other shapes to measure besides the headline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-hot", action="store_true")
    ap.add_argument("--stream-sweep", action="store_true",
                    help="only time the read-only stream probe over sizes 1 MiB..1 GiB and fit "
                         "t = t0 + bytes/BW (prints its own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library is a single-GPU operator "
              "(a multi-GPU deployment shards experts or rows, each GPU running the same "
              "kernel on its share); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.stream_sweep:
        print(json.dumps({"stream_sweep": stream_sweep()}), flush=True)
        return

    clocks = ClockSampler()
    p, head = measure(HEADLINE, args.steps, args.warmup, hot=not args.no_hot, clocks=clocks)
    extra = {}
    if not args.no_extra:
        for name in [w for w in args.workloads.split(",") if w and w != HEADLINE]:
            pe, r = measure(name, max(50, args.steps // 5), 10, hot=not args.no_hot)
            print(f"bench: {name}: {r['us_per_call']:.3f} us/call, {r['pct_hbm_peak']:.1f}% of HBM peak, "
                  f"stream ceiling {r['stream_ceiling_us_per_call']:.3f} us", file=sys.stderr, flush=True)
            r["desc"] = pe.wl.desc
            extra[name] = r
            del pe
            torch.cuda.empty_cache()

    t = head["us_per_call"] * 1e-6
    out = {
        "metric": METRIC,
        "value": round(head["eff_weight_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_call"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "C2: gpt-oss-20b MoE decode expert-gather GEMV, MXFP4 (e2m1 + E8M0/32) "
                        "x bf16 -> f32, 4 of 32 experts, 1 token, K=N=2880",
            "E": 32, "top_k": 4, "M": 1, "N": 2880, "K": 2880,
            "layers_rotated": head["layers_rotated"],
            "timing": "HIP graph of the K calls between two GPU real-time-counter stamps "
                      "(qmv_probe_clock) captured with them; HIP events on the replay stream "
                      "around the whole replay give us_per_call_replay_events; 512 MiB of "
                      "unrelated memory read just before the timed replay",
        },
        "us_per_call": round(head["us_per_call"], 3),
        "us_per_call_replay_events": round(head["us_per_call_replay_events"], 3),
        "pct_hbm_peak": round(head["pct_hbm_peak"], 2),
        "us_per_call_eager_launch": round(head["us_per_call_eager_launch"], 3),
        "hot_cache_us_per_call": round(head.get("hot_us_per_call", float("nan")), 3),
        "stream_ceiling": {
            "us_per_call": round(head["stream_ceiling_us_per_call"], 3),
            "weight_GBps": round(head["stream_ceiling_GBps"], 2),
            "pct_of_ceiling": round(head["pct_of_stream_ceiling"], 2),
            "what": "qmv_probe_stream_read over exactly the code and scale bytes of the same "
                    "calls (16-byte non-temporal buffer loads, no decode, no ids), best of "
                    "its launch shapes, timed the same way",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["algorithmic_bytes_per_call"] / t / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["algorithmic_bytes_per_call"] / t / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": profiled_traffic(HEADLINE),
            "kernel": "qmv::qmv_kernel, MXFP4 one-vector gather instantiation the launcher picks for K=N=2880",
            "algorithmic_bytes_per_launch": head["algorithmic_bytes_per_call"],
        },
        "workloads": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in extra.items()},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
        out["cpu_baseline_1thread"] = cpu_baseline(p, args.cpu_seconds / 2, threads=1)
    out["gpu_clocks"] = clocks.report()
    out["gpu_clock_levels"] = gpu_clocks()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
