"""bf16 activations with 2-bit and 3-bit weights: the kernel quantizes each
32-block of x to int8 + fp16 scale while staging it (QMV_A_BF16_Q8).  Needs an
MI355X.

Two checks per case:
  * the integer decisions: the call on bf16 x must equal, bit for bit, the same
    call on the int8 blocks that the CPU oracle's quantizer makes from that x
    (the kernels after staging are the same, so any differing q or scale shows
    up in the outputs);
  * the result: against the oracle (its quantizer, then its literal
    dequantize-then-dot) within 1e-3 * sum |w x| per output.
Edge blocks cover ties to even, scales that round to fp16 subnormals or to
zero, clipping at +-127, all-zero blocks and large magnitudes.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, oracle_call, to_dev

pytestmark = pytest.mark.gpu


def _bf16_x(seed, V, K, edge=False):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((V, K)).astype(np.float32)
    if edge:
        blk = g.reshape(V, K // 32, 32)
        nb = K // 32
        for v in range(V):
            kinds = rng.permutation(nb)[:min(nb, 8)]
            for j, b in enumerate(kinds):
                kind = j % 8
                if kind == 0:
                    blk[v, b] = 0.0                                     # zero block
                elif kind == 1:
                    blk[v, b] *= 2.0 ** -32                             # scale underflows to 0
                elif kind == 2:
                    blk[v, b] = rng.integers(-6, 7, 32) * 2.0 ** -19   # fp16 subnormal scale
                    blk[v, b, 0] = 3 * 2.0 ** -18
                elif kind == 3:
                    blk[v, b] = rng.integers(-3, 4, 32) * 2.0 ** -18   # clipping at 2^-24 scale
                    blk[v, b, 1] = 2.0 ** -17
                elif kind == 4:                                         # ties at d = 1
                    blk[v, b] = rng.integers(-126, 127, 32) + 0.5
                    blk[v, b, 2] = 127.0
                elif kind == 5:
                    blk[v, b] *= 1e4                                    # large magnitudes
                elif kind == 6:
                    blk[v, b] = -0.0
                    blk[v, b, 3] = 1.0
                else:
                    blk[v, b] *= 1e-3
        g = blk.reshape(V, K)
    return synth.bf16_bits(g)


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _gather_pair(inp, xb):
    """(y on bf16 x, y on the oracle-quantized int8 x) for a gather call."""
    import bit_block_quantized_amd as q
    wl = inp.wl
    dev = to_dev(inp)
    qx, d = oracle.load().quantize_q8(xb)
    M, top_k = inp.ids.shape
    shape = (M, top_k, wl.K) if wl.x_per_slot else (M, wl.K)
    xs_shape = shape[:-1] + (wl.K // 32,)
    y_b = q.qmv_gather_moe(wl.wfmt, dev["codes"], dev["scales"], dev["ids"],
                           _dev_bf16(xb).view(shape), x_per_slot=wl.x_per_slot)
    y_q = q.qmv_gather_moe(wl.wfmt, dev["codes"], dev["scales"], dev["ids"],
                           torch.from_numpy(qx).cuda().view(shape),
                           torch.from_numpy(d.view(np.float16)).cuda().view(xs_shape),
                           x_per_slot=wl.x_per_slot)
    return y_b.cpu().numpy(), y_q.cpu().numpy(), qx, d


def _same_bits(a, b, what):
    a = np.ascontiguousarray(a, np.float32).reshape(-1)
    b = np.ascontiguousarray(b, np.float32).reshape(-1)
    bad = np.nonzero(a.view(np.uint32) != b.view(np.uint32))[0]
    assert bad.size == 0, f"{what}: {bad.size} outputs differ"


GATHER_CASES = {
    "cb2 2-bit gate/up shape": ("C3", dict(E=12, N=70)),
    "cb3 3-bit down shape, per slot": ("C4", dict(E=12, N=59)),
    "cb3 M=4 broadcast": ("C4", dict(E=9, N=37, M=4, x_per_slot=False)),
    "cb2 K=96 (32-weight units)": ("C3", dict(E=5, N=33, K=96, M=2)),
    "cb2 M=3 large K": ("C3", dict(E=6, N=20, M=3, K=16384)),
}


@pytest.mark.parametrize("case", list(GATHER_CASES))
@pytest.mark.parametrize("edge", [False, True])
def test_gather_bf16_quantized_in_kernel(case, edge):
    base, kw = GATHER_CASES[case]
    wl = synth.WORKLOADS[base].scaled(**kw)
    inp = synth.make(wl)
    V = inp.x.shape[0]
    xb = _bf16_x(zlib.crc32(case.encode()) % 1000 + edge, V, wl.K, edge)
    y_b, y_q, qx, d = _gather_pair(inp, xb)
    _same_bits(y_b, y_q, case)
    inp.x, inp.xs = qx, d
    yr, A = oracle_call(inp)
    assert_parity(y_b, yr, A, case)


@pytest.mark.parametrize("wfmt", ["cb2", "cb3"])
@pytest.mark.parametrize("M", [1, 4])
def test_dense_bf16_quantized_in_kernel(wfmt, M):
    import bit_block_quantized_amd as q
    wl = synth.Workload("dense-q8", "dense", wfmt, M=M, N=77, K=2048, seed=30 + M)
    inp = synth.make(wl)
    xb = _bf16_x(40 + M, M, wl.K, edge=True)
    qx, d = oracle.load().quantize_q8(xb)
    dev = to_dev(inp)
    y_b = q.qmv_dense(wfmt, dev["codes"], dev["scales"], _dev_bf16(xb)).cpu().numpy()
    y_q = q.qmv_dense(wfmt, dev["codes"], dev["scales"], torch.from_numpy(qx).cuda(),
                      torch.from_numpy(d.view(np.float16)).cuda()).cpu().numpy()
    _same_bits(y_b, y_q, f"dense {wfmt} M={M}")
    inp.x, inp.xs = qx, d
    yr, A = oracle_call(inp)
    assert_parity(y_b, yr, A, f"dense {wfmt} M={M}")


@pytest.mark.parametrize("wfmt,base", [("cb2", "C3"), ("cb3", "C4")])
def test_swiglu_bf16_quantized_in_kernel(wfmt, base):
    import bit_block_quantized_amd as q
    from test_gpu_swiglu import assert_swiglu_parity, oracle_swiglu
    wl = synth.WORKLOADS[base].scaled(name="gu-q8", E=8, N=64, x_per_slot=False)
    inp = synth.make_gate_up(wl)
    xb = _bf16_x(50, wl.M, wl.K, edge=True)
    qx, d = oracle.load().quantize_q8(xb)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    args = (wfmt, dv(inp.gcodes), dv(inp.gscales), dv(inp.ucodes), dv(inp.uscales), dv(inp.ids))
    y_b = q.qmv_gather_moe_swiglu(*args, _dev_bf16(xb)).cpu().numpy()
    y_q = q.qmv_gather_moe_swiglu(*args, dv(qx), dv(d.view(np.float16))).cpu().numpy()
    _same_bits(y_b, y_q, f"swiglu {wfmt}")
    inp.x, inp.xs = qx, d
    assert_swiglu_parity(y_b, oracle_swiglu(inp), f"swiglu {wfmt}")


@pytest.mark.parametrize("wfmt", ["cb2", "cb3"])
def test_combine_bf16_quantized_in_kernel(wfmt):
    import bit_block_quantized_amd as q
    from test_gpu_combine import _combine_wl, oracle_combine
    wl = _combine_wl(wfmt, M=2, N=90, E=10, top_k=6, seed=60)
    inp = synth.make(wl)
    xb = _bf16_x(61, wl.M * wl.top_k, wl.K, edge=True)
    qx, d = oracle.load().quantize_q8(xb)
    dev = to_dev(inp)
    wt = torch.from_numpy(inp.extra["weights"]).cuda()
    shape = (wl.M, wl.top_k, wl.K)
    y_b = q.qmv_gather_moe_combine(wfmt, dev["codes"], dev["scales"], dev["ids"], wt,
                                   _dev_bf16(xb).view(shape)).cpu().numpy()
    y_q = q.qmv_gather_moe_combine(wfmt, dev["codes"], dev["scales"], dev["ids"], wt,
                                   torch.from_numpy(qx).cuda().view(shape),
                                   torch.from_numpy(d.view(np.float16)).cuda().view(
                                       wl.M, wl.top_k, wl.K // 32)).cpu().numpy()
    _same_bits(y_b, y_q, f"combine {wfmt}")
    inp.x, inp.xs = qx, d
    yr, A = oracle_combine(inp)
    assert_parity(y_b, yr, A, f"combine {wfmt}")


def _exact_sum_bf16_x(seed, V, K):
    """bf16 x whose every 32-block has absmax exactly 127 * 2^k, k in {-1, 0}.

    Then d = amax / 127 = 2^k exactly, fp16(d) = 2^k and 1/d is exact, so the
    quantizer's only free decisions are the roundings of x / d (ties at .5
    included).  With unit weight scales every block term 0.5 * 2^k * S_b is a
    multiple of 2^-2 and every partial sum stays below 2^21, so the result is
    exact in fp32 in any summation order: outputs of two calls agree bit for
    bit exactly when their int8 blocks do, whatever launch shapes they take."""
    rng = np.random.default_rng(seed)
    nb = K // 32
    k = rng.integers(-1, 1, (V, nb, 1)).astype(np.float32)
    step = np.float32(2.0) ** k
    blk = np.clip(rng.standard_normal((V, nb, 32)).astype(np.float32) * 40, -126, 126)
    ties = rng.random((V, nb, 32)) < 0.25
    blk = np.where(ties, np.round(blk) + 0.5, blk) * step
    pos = rng.integers(0, 32, (V, nb))
    sign = np.where(rng.random((V, nb)) < 0.5, -1.0, 1.0).astype(np.float32)
    np.put_along_axis(blk, pos[..., None], (sign[..., None] * 127.0 * step), axis=2)
    return synth.bf16_bits(blk.reshape(V, K))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["C3", "C4"])
def test_full_size_bf16_activations(name):
    """The DeepSeek-shaped 2-bit and 3-bit workloads at full size fed bf16
    activations, every output checked.

    Random x: against the oracle within the float tolerance (the bf16-input
    and int8-input calls may take different launch shapes at this size, so
    their float results may differ in rounding).  Exact-sum x with unit weight
    scales: bit for bit against the same call on the oracle's int8 blocks and
    against the oracle rounded to fp32, which pins every integer decision of
    the in-kernel quantizer at the tuned full-size launch."""
    from gpu_util import assert_exact
    inp = synth.make(name)
    wl = inp.wl
    V = inp.x.shape[0]
    xb = _bf16_x(70, V, wl.K)
    y_b, _, qx, d = _gather_pair(inp, xb)
    inp.x, inp.xs = qx, d
    yr, A = oracle_call(inp)
    assert_parity(y_b, yr, A, name)

    unit = np.full(inp.scales.shape[:-1] + (inp.scales.shape[-1] // 2,), 0x3C00, np.uint16)
    inp.scales = unit.view(np.uint8)
    xb = _exact_sum_bf16_x(71, V, wl.K)
    y_b, y_q, qx, d = _gather_pair(inp, xb)
    assert np.all(d.view(np.uint16) & 0x03FF == 0), "exact-sum x: scales must be powers of two"
    _same_bits(y_b, y_q, name + " exact-sum")
    inp.x, inp.xs = qx, d
    yr, _ = oracle_call(inp)
    assert_exact(y_b, yr, name + " exact-sum")


@pytest.mark.parametrize("name", ["C3q", "C4q"])
def test_quant_workloads_small(name):
    """The bench's bf16-activation workloads with small expert tables, through
    the shared helpers (the oracle quantizes, then takes the int8 definition)."""
    from gpu_util import gpu_call
    wl = synth.workload(name).scaled(E=12, N=70)
    inp = synth.make(wl)
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert_parity(y, yr, A, name)
