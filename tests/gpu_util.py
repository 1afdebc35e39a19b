"""Helpers shared by the GPU parity tests: move synthetic inputs to the
device, call the HIP path through the binding, evaluate the oracle on the
same inputs (threaded over disjoint output selections) and compare."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

TOL = 1e-3          # |y - y_ref| <= TOL * sum_k |w_k x_k| per output


def threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_dev(inp, device="cuda"):
    d = {}
    d["codes"] = torch.from_numpy(np.ascontiguousarray(inp.codes)).to(device)
    d["scales"] = torch.from_numpy(np.ascontiguousarray(inp.scales)).to(device)
    d["ids"] = None if inp.ids is None else torch.from_numpy(np.ascontiguousarray(inp.ids)).to(device)
    if inp.wl.afmt in ("bf16", "bf16q8"):
        d["x"] = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).to(device).view(torch.bfloat16)
        d["xs"] = None
    else:
        d["x"] = torch.from_numpy(np.ascontiguousarray(inp.x)).to(device)
        d["xs"] = torch.from_numpy(np.ascontiguousarray(inp.xs).view(np.float16)).to(device)
    return d


def gpu_call(inp, dev=None, y=None, stream=None):
    import bit_block_quantized_amd as q
    wl = inp.wl
    dev = dev or to_dev(inp)
    if wl.kind == "dense":
        return q.qmv_dense(wl.wfmt, dev["codes"], dev["scales"], dev["x"], dev["xs"], y=y,
                           stream=stream)
    x = dev["x"]
    xs = dev["xs"]
    if wl.x_per_slot:
        M, top_k = inp.ids.shape
        x = x.view(M, top_k, wl.K)
        xs = None if xs is None else xs.view(M, top_k, wl.K // 32)
    return q.qmv_gather_moe(wl.wfmt, dev["codes"], dev["scales"], dev["ids"], x, xs,
                            x_per_slot=wl.x_per_slot, y=y, stream=stream)


def oracle_call(inp, outs=None, nthreads=None):
    """Oracle (y, A) for the call; flat over ``outs`` when given, else full shape."""
    o = oracle.load()
    wl = inp.wl
    if wl.kind == "dense":
        codes, scales = inp.codes[None], inp.scales[None]
        ids = np.zeros((wl.M, 1), np.int32)
        shape = (wl.M, wl.N)
    else:
        codes, scales, ids = inp.codes, inp.scales, inp.ids
        shape = (wl.M, wl.top_k, wl.N)
    total = int(np.prod(shape))
    sel = np.arange(total, dtype=np.int64) if outs is None else np.asarray(outs, np.int64)
    n = nthreads or threads()
    parts = np.array_split(sel, max(1, min(n, len(sel) // 64 + 1)))

    afmt, x, xs = wl.afmt, inp.x, inp.xs
    if afmt == "bf16q8":                 # the oracle's quantizer, then the int8 definition
        x, xs = o.quantize_q8(np.asarray(x).reshape(-1, wl.K))
        afmt = "q8"

    def run(p):
        return o.gather(wl.wfmt, codes, scales, ids, afmt, x, xs,
                        x_per_slot=wl.x_per_slot, outs=p)

    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(run, parts))
    y = np.concatenate([r[0] for r in res])
    A = np.concatenate([r[1] for r in res])
    if outs is None:
        return y.reshape(shape), A.reshape(shape)
    return y, A


def assert_parity(y_gpu, y_ref, A_ref, what=""):
    """Every output within TOL * A; NaN only where the oracle has NaN."""
    g = np.asarray(y_gpu, np.float64).reshape(-1)
    r = np.asarray(y_ref, np.float64).reshape(-1)
    A = np.asarray(A_ref, np.float64).reshape(-1)
    nan_r = np.isnan(r)
    assert np.array_equal(np.isnan(g), nan_r), f"{what}: NaN pattern differs"
    ok = ~nan_r
    err = np.abs(g[ok] - r[ok])
    bound = TOL * A[ok]
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {ok.sum()} outputs out of tolerance; first at "
                           f"{np.nonzero(ok)[0][bad[0]]}: gpu {g[ok][bad[0]]!r} ref {r[ok][bad[0]]!r} "
                           f"A {A[ok][bad[0]]!r}")
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def assert_exact(y_gpu, y_ref, what=""):
    """Bit-exact: the oracle's fp64 result rounded to fp32 equals the GPU's."""
    g = np.asarray(y_gpu, np.float32).reshape(-1)
    r = np.asarray(y_ref, np.float64).astype(np.float32).reshape(-1)
    bad = np.nonzero(g.view(np.uint32) != r.view(np.uint32))[0]
    # +0 and -0 compare equal
    bad = bad[~((g[bad] == 0) & (r[bad] == 0))]
    assert bad.size == 0, f"{what}: {bad.size} outputs differ; first {bad[0]}: {g[bad[0]]} vs {r[bad[0]]}"
