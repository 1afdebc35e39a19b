"""MXFP4 weights with int8 activations (QMV_A_Q8B32: int8 x, fp16 scale per
32): every entry point against the CPU oracle on the same seeded inputs.
Needs an MI355X.

The kernels stage the int8 activations as exact bf16 and form each 32-block's
sum of e2m1 * 2^(s-127) * q exactly before the activation scale multiplies
it, so at unit scales (E8M0 127, fp16 1.0) every result is an exact fp32
value and must equal the oracle bit for bit (int8 -128 included); elsewhere
every output is within 1e-3 * sum |w x|.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_exact, assert_parity, gpu_call, oracle_call, to_dev

pytestmark = pytest.mark.gpu


def _wl(kind, M, N, K, E=1, top_k=1, x_per_slot=False, seed=0):
    return synth.Workload("mxfp4-int8", kind, "mxfp4", M=M, N=N, K=K, seed=seed, E=E,
                          top_k=top_k, x_per_slot=x_per_slot, x_q8=True)


def _run(inp, what, exact=False):
    assert inp.wl.afmt == "q8" and inp.x.dtype == np.int8
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert y.shape == yr.shape
    if exact:
        assert_exact(y, yr, what)
    return assert_parity(y, yr, A, what)


def _unit(inp, seed=97):
    inp.scales[...] = 127
    inp.xs.view(np.float16)[...] = 1.0
    rng = np.random.default_rng(seed)
    inp.x = rng.integers(-128, 128, size=inp.x.shape, dtype=np.int16).astype(np.int8)
    return inp


def test_workload_small():
    _run(synth.make(synth.workload("C2i").scaled(E=8, N=87)), "C2i small")


@pytest.mark.slow
def test_workload_full_size():
    """The gpt-oss-shaped gather with int8 activations, as bench.py launches
    it, every output checked."""
    _run(synth.make(synth.workload("C2i")), "C2i")


@pytest.mark.parametrize("K", [32, 64, 96, 160, 1056, 2880, 16384])
def test_k_sweep_dense(K):
    _run(synth.make(_wl("dense", 1, 37, K, seed=K)), f"K={K}")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_m_sweep(M):
    _run(synth.make(_wl("dense", M, 45, 576, seed=10 + M)), f"dense M={M}")
    _run(synth.make(_wl("gather", M, 45, 576, E=5, top_k=3, seed=20 + M)), f"gather M={M}")
    _run(synth.make(_wl("gather", M, 45, 576, E=5, top_k=3, x_per_slot=True, seed=30 + M)),
         f"per-slot M={M}")


@pytest.mark.parametrize("case", ["dense1", "dense4", "gather", "per-slot"])
def test_exact_at_unit_scales(case):
    wl = {"dense1": _wl("dense", 1, 61, 2880, seed=41),
          "dense4": _wl("dense", 4, 29, 1056, seed=42),
          "gather": synth.workload("C2i").scaled(E=8, N=87),
          "per-slot": _wl("gather", 2, 33, 2880, E=6, top_k=4, x_per_slot=True, seed=43)}[case]
    _run(_unit(synth.make(wl)), f"unit {case}", exact=True)


def test_invalid_ids_give_zero_rows():
    inp = synth.make(_wl("gather", 2, 40, 512, E=4, top_k=3, seed=50))
    inp.ids = np.array([[1, -1, 3], [4, 2, 7]], np.int32)
    y = gpu_call(inp).cpu().numpy()
    assert (y[0, 1] == 0).all() and (y[1, 0] == 0).all() and (y[1, 2] == 0).all()
    _run(inp, "invalid ids")


def test_e8m0_special_scales():
    inp = synth.make(_wl("dense", 2, 6, 96, seed=7))
    inp.scales[0, :] = 0
    inp.scales[1, :] = 1
    inp.scales[2, :] = 254
    inp.scales[3, 1] = 255
    inp.scales[4, :] = [0, 127, 254]
    inp.scales[5, :] = 127
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert np.isnan(yr[:, 3]).all()
    fin = (A < 3.0e38) | np.isnan(yr)
    assert_parity(y[fin], yr[fin], A[fin], "e8m0 specials")


def test_bitwise_deterministic_and_graph():
    inp = synth.make(synth.workload("C2i").scaled(E=8, N=87))
    dev = to_dev(inp)
    y1 = gpu_call(inp, dev).cpu().numpy()
    out = torch.empty_like(torch.from_numpy(y1)).cuda()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        gpu_call(inp, dev, y=out, stream=s)
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        gpu_call(inp, dev, y=out, stream=torch.cuda.current_stream())
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), y1.view(np.uint32))


def test_swiglu_int8_activations():
    from test_gpu_swiglu import assert_swiglu_parity, gpu_swiglu, oracle_swiglu
    wl = synth.GATE_UP_WORKLOADS["C2gu"].scaled(name="gu-int8", E=8, N=96, x_q8=True)
    inp = synth.make_gate_up(wl)
    assert inp.x.dtype == np.int8
    assert_swiglu_parity(gpu_swiglu(inp).cpu().numpy(), oracle_swiglu(inp), "swiglu int8")


@pytest.mark.parametrize("top_k,per_slot", [(4, True), (6, True), (4, False)])
def test_combine_int8_activations(top_k, per_slot):
    from test_gpu_combine import gpu_combine, oracle_combine
    wl = synth.Workload("combine-int8", "combine", "mxfp4", M=2, N=59, K=2880, seed=60 + top_k,
                        E=10, top_k=top_k, x_per_slot=per_slot, x_q8=True)
    inp = synth.make(wl)
    y = gpu_combine(inp).cpu().numpy()
    yr, A = oracle_combine(inp)
    assert_parity(y, yr, A, f"combine top_k={top_k} per_slot={per_slot}")
