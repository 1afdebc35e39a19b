"""Fused gate/up gather with the SwiGLU epilogue against the CPU oracle
(needs an MI355X).

The oracle gives g, u (fp64) and their sum |w x| scales Ag, Au.  The GPU's g
and u each carry the gather's error bound, at most 1e-3 * A; silu has slope
at most 1.1 in magnitude, so propagating those errors gives

    E1 = 1e-3 * (1.1 |u| Ag + |silu(g)| Au + 1.1e-3 Ag Au).

On top of that the kernel evaluates silu(g) * u = g / (1 + e^-g) * u in
fp32.  Its exponential is the hardware base-2 exponential of g * log2(e):
rounding that product to fp32 moves the exponent by at most |g| log2(e)
2^-24, a relative error of at most |g| 2^-24 in e^-g, and the instruction
itself is within 1 ulp (2^-23); the add, the IEEE division and the final
product add 2^-24 each.  An error in e^-g reaches 1 + e^-g at most in full,
so the fp32 evaluation is within (|g| + 5) 2^-24 of silu(g') u' in relative
terms.  With a factor 4 of margin the bar is

    |y - y_ref| <= E1 + 2^-22 (|g| + 8) (|y_ref| + E1).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import threads

pytestmark = pytest.mark.gpu

TOL = 1e-3
SILU_SLOPE = 1.1


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.view(dtype)


def gpu_swiglu(inp, y=None):
    import bit_block_quantized_amd as q
    wl = inp.wl
    if wl.afmt in ("bf16", "bf16q8"):
        x = _dev(inp.x.view(np.int16), torch.bfloat16)
        xs = None
    else:
        x = _dev(inp.x)
        xs = _dev(inp.xs.view(np.float16))
    return q.qmv_gather_moe_swiglu(wl.wfmt, _dev(inp.gcodes), _dev(inp.gscales),
                                   _dev(inp.ucodes), _dev(inp.uscales), _dev(inp.ids), x, xs,
                                   y=y)


def oracle_swiglu(inp, outs=None):
    o = oracle.load()
    wl = inp.wl
    shape = inp.ids.shape + (wl.N,)
    total = int(np.prod(shape))
    sel = np.arange(total, dtype=np.int64) if outs is None else np.asarray(outs, np.int64)
    parts = np.array_split(sel, max(1, min(threads(), len(sel) // 64 + 1)))
    afmt, x, xs = wl.afmt, inp.x, inp.xs
    if afmt == "bf16q8":                 # the oracle's quantizer, then the int8 definition
        x, xs = o.quantize_q8(np.asarray(x).reshape(-1, wl.K))
        afmt = "q8"

    def run(p):
        return o.gather_swiglu(wl.wfmt, inp.gcodes, inp.gscales, inp.ucodes, inp.uscales,
                               inp.ids, afmt, x, xs, outs=p)

    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(run, parts))
    out = [np.concatenate([r[i] for r in res]) for i in range(5)]
    if outs is None:
        out = [a.reshape(shape) for a in out]
    return out


def assert_swiglu_parity(y_gpu, ref, what=""):
    y, g, u, Ag, Au = [np.asarray(a, np.float64).reshape(-1) for a in ref]
    yg = np.asarray(y_gpu, np.float64).reshape(-1)
    assert np.isfinite(yg).all(), f"{what}: non-finite output"
    silu = g / (1.0 + np.exp(-np.clip(g, -700, 700)))
    e1 = TOL * (SILU_SLOPE * np.abs(u) * Ag + np.abs(silu) * Au + SILU_SLOPE * TOL * Ag * Au)
    bound = e1 + 2.0 ** -22 * (np.abs(g) + 8.0) * (np.abs(y) + e1)
    err = np.abs(yg - y)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {y.size} outputs out of tolerance; first at "
                           f"{bad[0]}: gpu {yg[bad[0]]!r} ref {y[bad[0]]!r} g {g[bad[0]]!r} "
                           f"u {u[bad[0]]!r}")
    return float((err / np.maximum(bound, 1e-300)).max())


def _wl(base, **kw):
    return synth.WORKLOADS[base].scaled(name=f"{base}-gate-up", **kw)


# real K and N of the gate/up shapes, small expert tables, plus ragged N.  The
# default E8M0 range puts the MXFP4 gate values in the thousands (silu's
# saturated arms); the narrower range keeps them in silu's curved part.
CASES = {
    "mxfp4 K=N=2880": ("C2", dict(E=8)),
    "mxfp4 K=N=2880 small g": ("C2", dict(E=8, e8m0=(115, 120))),
    "mxfp4 ragged": ("C2", dict(E=8, N=87)),
    "cb2 K=7168": ("C3", dict(E=16, N=2048)),
    "cb2 ragged": ("C3", dict(E=16, N=105)),
    "cb3 K=2048": ("C4", dict(E=16, N=1024, x_per_slot=False)),
    "mxfp4 M=4": ("C5a", dict(E=12, N=59)),
    # more than 4 tokens: the batched matrix-core kernel (many pairs per
    # expert), and groups of 4 tokens on the decode kernels (few)
    "mxfp4 batched M=64": ("C2", dict(E=8, N=300, M=64)),
    "mxfp4 batched ragged": ("C2", dict(E=3, N=77, K=416, M=200, top_k=2)),
    "mxfp4 batched one expert": ("C2", dict(E=1, N=130, K=96, M=150, top_k=1)),
    "mxfp4 few pairs M=6": ("C5a", dict(E=64, N=59, M=6)),
    # more than 4 tokens with int8 activations (given, or bf16 quantized in
    # the kernel): the grouped kernel, 4 pairs at a time per expert
    "cb2 grouped M=24": ("C3", dict(E=16, N=130, M=24, K=1024)),
    "cb2 grouped M=40 bf16 x": ("C3", dict(E=6, N=70, M=40, K=2048, x_bf16=True)),
    "cb3 grouped M=12 bf16 x": ("C4", dict(E=10, N=77, M=12, x_per_slot=False, x_bf16=True)),
    "cb3 grouped one expert": ("C4", dict(E=1, N=45, K=512, M=150, top_k=1, x_per_slot=False)),
    "mxfp4 int8 grouped M=20": ("C2", dict(E=8, N=50, M=20, x_q8=True)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_swiglu_matches_oracle(case):
    base, kw = CASES[case]
    inp = synth.make_gate_up(_wl(base, **kw))
    y = gpu_swiglu(inp).cpu().numpy()
    assert y.shape == inp.ids.shape + (inp.wl.N,)
    worst = assert_swiglu_parity(y, oracle_swiglu(inp), case)
    print(f"{case}: worst |err| / bound = {worst:.3e}")


@pytest.mark.parametrize("wfmt,base", [("mxfp4", "C2"), ("cb2", "C3"), ("cb3", "C4")])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9])
def test_swiglu_m_sweep(wfmt, base, M):
    inp = synth.make_gate_up(_wl(base, M=M, E=5, top_k=3, N=45, K=576, x_per_slot=False,
                                 seed=40 + M))
    assert_swiglu_parity(gpu_swiglu(inp).cpu().numpy(), oracle_swiglu(inp), f"{wfmt} M={M}")


@pytest.mark.parametrize("base", ["C2", "C3", "C4"])
def test_swiglu_invalid_and_duplicate_ids(base):
    inp = synth.make_gate_up(_wl(base, M=3, E=6, top_k=4, N=70, K=256, x_per_slot=False, seed=9))
    inp.ids = np.array([[-1, 2, 6, 2], [2 ** 31 - 1, 5, 5, 0], [2, 2, 2, -2 ** 31]], np.int32)
    y = torch.full((3, 4, 70), 7.0, device="cuda")
    gpu_swiglu(inp, y=y)
    y = y.cpu().numpy()
    assert_swiglu_parity(y, oracle_swiglu(inp), base)
    for t, j in [(0, 0), (0, 2), (1, 0), (2, 3)]:
        assert not y[t, j].any(), (t, j)


def test_swiglu_deterministic_and_matches_separate_gathers():
    """Two runs are bit-identical, and the fused result agrees with silu(g) * u
    formed from two plain gather calls on the same device."""
    import bit_block_quantized_amd as q
    inp = synth.make_gate_up(_wl("C2", E=8))
    y1 = gpu_swiglu(inp).cpu().numpy()
    y2 = gpu_swiglu(inp).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    x = _dev(inp.x.view(np.int16), torch.bfloat16)
    ids = _dev(inp.ids)
    g = q.qmv_gather_moe("mxfp4", _dev(inp.gcodes), _dev(inp.gscales), ids, x)
    u = q.qmv_gather_moe("mxfp4", _dev(inp.ucodes), _dev(inp.uscales), ids, x)
    ys = (torch.nn.functional.silu(g) * u).cpu().numpy()
    ref = oracle_swiglu(inp)
    assert_swiglu_parity(ys, ref, "separate gathers")
    scale = np.abs(ref[2]) * ref[3] + ref[4] * np.abs(ref[1]) + 1e-30
    assert (np.abs(y1 - ys) <= 2.2e-3 * scale + 1e-5 * np.abs(ys)).all()


@pytest.mark.slow
@pytest.mark.parametrize("base", ["C2", "C3"])
def test_swiglu_full_size(base):
    """The gate/up shapes at their full expert tables, every output checked."""
    inp = synth.make_gate_up(_wl(base))
    y = gpu_swiglu(inp).cpu().numpy()
    worst = assert_swiglu_parity(y, oracle_swiglu(inp), base)
    print(f"{base} gate/up: worst |err| / bound = {worst:.3e}")


def test_prefill_gate_up_full_size_sampled():
    """The gpt-oss-20b prefill chunk through the fused gate/up projection
    (512 tokens x top-4 of 32, K=N=2880; the batched kernel) as bench.py
    launches it: 4000 sampled outputs and 4 whole (token, slot) rows."""
    inp = synth.make_gate_up(synth.workload("C6gu"))
    y = gpu_swiglu(inp).cpu().numpy().reshape(-1)
    wl = inp.wl
    rng = np.random.default_rng(6)
    rows = rng.choice(wl.M * wl.top_k, size=4, replace=False)
    outs = np.concatenate([rng.choice(y.size, size=4000, replace=False)] +
                          [r * wl.N + np.arange(wl.N) for r in rows])
    worst = assert_swiglu_parity(y[outs], oracle_swiglu(inp, outs=outs), "C6gu sampled")
    print(f"C6gu: worst |err| / bound = {worst:.3e}")
