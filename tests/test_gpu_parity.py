"""HIP path against the CPU oracle, element by element (needs an MI355X).

Every test calls the C ABI through the binding and compares each output with
the oracle on the same seeded inputs: |y - y_ref| <= 1e-3 * sum_k |w_k x_k|,
and bit-exact wherever the arithmetic is exact (integer block sums at unit
scales, MXFP4 with unit scales and small-integer activations).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_exact, assert_parity, gpu_call, oracle_call, to_dev

pytestmark = pytest.mark.gpu

# Shrunken versions of the workloads: real K (so the same launch shapes are
# taken), small expert tables, N spanning several row tiles plus a ragged tail.
SMALL = {
    "C1": dict(),
    "C2": dict(E=8, N=87),
    "C3": dict(E=16, N=105),
    "C4": dict(E=16, N=59),
    "C5a": dict(E=12, N=59),      # small table: tokens share experts (2-4 vectors per item)
    "C5b": dict(N=77),
}


def _run(inp, exact=False, what=""):
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert y.shape == yr.shape
    if exact:
        assert_exact(y, yr, what)
    return assert_parity(y, yr, A, what)


@pytest.mark.parametrize("name", list(SMALL))
def test_workload_small(name):
    wl = synth.WORKLOADS[name].scaled(**SMALL[name])
    _run(synth.make(wl), what=name)


@pytest.mark.slow
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_size(name):
    """The full workloads, exactly as the benchmark launches them, every output checked."""
    inp = synth.make(name)
    worst = _run(inp, what=name)
    print(f"{name}: worst |err| / bound = {worst:.3e}")


def _custom(wfmt, kind, M, N, K, E=1, top_k=1, x_per_slot=False, seed=0, ids=None):
    wl = synth.Workload("custom", kind, wfmt, M=M, N=N, K=K, seed=seed, E=E, top_k=top_k,
                        x_per_slot=x_per_slot)
    inp = synth.make(wl)
    if ids is not None:
        inp.ids = np.asarray(ids, np.int32)
    return inp


FMTS = ["mxfp4", "cb2", "cb3"]


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("K", [32, 64, 96, 160, 256, 1056, 4096, 16384])
def test_k_sweep_dense(wfmt, K):
    _run(_custom(wfmt, "dense", M=1, N=37, K=K, seed=K), what=f"{wfmt} K={K}")


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_m_sweep(wfmt, M):
    _run(_custom(wfmt, "dense", M=M, N=45, K=576, seed=10 + M), what=f"dense {wfmt} M={M}")
    _run(_custom(wfmt, "gather", M=M, N=45, K=576, E=5, top_k=3, seed=20 + M),
         what=f"gather {wfmt} M={M}")
    _run(_custom(wfmt, "gather", M=M, N=45, K=576, E=5, top_k=3, x_per_slot=True, seed=30 + M),
         what=f"per-slot {wfmt} M={M}")


@pytest.mark.parametrize("wfmt", FMTS)
def test_invalid_ids_give_zero_rows(wfmt):
    inp = _custom(wfmt, "gather", M=2, N=70, K=256, E=6, top_k=4, seed=3,
                  ids=[[-1, 2, 6, 0], [2 ** 31 - 1, -2 ** 31, 5, 2]])
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert_parity(y, yr, A, wfmt)
    assert not y[0, 0].any() and not y[0, 2].any() and not y[1, 0].any() and not y[1, 1].any()


@pytest.mark.parametrize("wfmt", FMTS)
def test_all_ids_invalid(wfmt):
    inp = _custom(wfmt, "gather", M=1, N=33, K=128, E=4, top_k=2, seed=4, ids=[[4, -7]])
    y = torch.full((1, 2, 33), 7.0, device="cuda")
    gpu_call(inp, y=y)
    assert not y.cpu().numpy().any()


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("per_slot", [False, True])
def test_duplicate_and_shared_experts(wfmt, per_slot):
    # the same expert twice in one token, and shared across tokens
    inp = _custom(wfmt, "gather", M=3, N=41, K=320, E=9, top_k=4, x_per_slot=per_slot, seed=5,
                  ids=[[3, 3, 5, 3], [5, 1, 3, 8], [3, 3, 3, 3]])
    _run(inp, what=f"{wfmt} per_slot={per_slot}")


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("per_slot", [False, True])
def test_64_pairs_few_experts(wfmt, per_slot):
    # M=4, top_k=16: 64 (token, slot) pairs over 3 experts -> experts read by
    # up to 16 vectors, split into items of four
    rng = np.random.default_rng(6)
    ids = rng.integers(-1, 4, size=(4, 16)).astype(np.int32)
    inp = _custom(wfmt, "gather", M=4, N=23, K=192, E=3, top_k=16, x_per_slot=per_slot, seed=6,
                  ids=ids)
    _run(inp, what=f"{wfmt} per_slot={per_slot}")


def _unit_scale(inp):
    wl = inp.wl
    if wl.wfmt == "mxfp4":
        inp.scales[...] = 127
        rng = np.random.default_rng(99)
        g = rng.integers(-8, 9, size=inp.x.shape).astype(np.float32)
        inp.x = synth.bf16_bits(g)
    else:
        inp.scales.view(np.float16)[...] = 1.0
        inp.xs.view(np.float16)[...] = 1.0
        rng = np.random.default_rng(98)
        inp.x = rng.integers(-128, 128, size=inp.x.shape, dtype=np.int16).astype(np.int8)
    return inp


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5a", "C5b"])
def test_exact_at_unit_scales(name):
    """Integer block sums (CB) and e2m1 x small integers (MXFP4) are exact:
    the GPU result must equal the oracle's bit for bit, including int8 -128."""
    wl = synth.WORKLOADS[name].scaled(**SMALL[name])
    inp = _unit_scale(synth.make(wl))
    _run(inp, exact=True, what=name)


def test_e8m0_special_scales():
    inp = _custom("mxfp4", "dense", M=2, N=6, K=96, seed=7)
    inp.scales[0, :] = 0          # 2^-127, subnormal
    inp.scales[1, :] = 1
    inp.scales[2, :] = 254
    inp.scales[3, 1] = 255        # NaN in the middle group only
    inp.scales[4, :] = [0, 127, 254]
    inp.scales[5, :] = 127
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert np.isnan(yr[:, 3]).all()
    # where sum |w x| exceeds the fp32 range, partial sums of any fp32
    # evaluation order can overflow (inf - inf = NaN): those rows have no
    # fp32 answer to compare; every other row must match
    fin = (A < 3.0e38) | np.isnan(yr)
    assert fin[:, 0].all() and fin[:, 1].all() and fin[:, 5].all()
    assert_parity(y[fin], yr[fin], A[fin], "e8m0 specials")


@pytest.mark.parametrize("name", ["C2", "C3", "C4", "C5a"])
def test_bitwise_deterministic(name):
    wl = synth.WORKLOADS[name].scaled(**SMALL[name])
    inp = synth.make(wl)
    dev = to_dev(inp)
    y1 = gpu_call(inp, dev).cpu().numpy()
    y2 = gpu_call(inp, dev).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("name", ["C2", "C4", "C5b"])
def test_writes_nothing_past_y(name):
    wl = synth.WORKLOADS[name].scaled(**SMALL[name])
    inp = synth.make(wl)
    shape = (wl.M, wl.N) if wl.kind == "dense" else (wl.M, wl.top_k, wl.N)
    n = int(np.prod(shape))
    buf = torch.full((n + 4096,), float("nan"), device="cuda")
    buf[n:] = 12345.0
    gpu_call(inp, y=buf[:n].view(shape))
    tail = buf[n:].cpu().numpy()
    assert (tail == 12345.0).all()
    assert not np.isnan(buf[:n].cpu().numpy()).any()


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("M", [1, 2])
def test_dense_equals_single_expert_gather(wfmt, M):
    """A gather whose every token picks expert e is the dense call on W[e]:
    bit for bit where both run the same kernel family; MXFP4 x bf16 with
    M >= 2 runs the dense call on the matrix cores (another summation order),
    so there both are held to the oracle's tolerance on the same inputs."""
    g = _custom(wfmt, "gather", M=M, N=50, K=448, E=4, top_k=1, seed=8, ids=[[2]] * M)
    d = _custom(wfmt, "dense", M=M, N=50, K=448, seed=8)
    d.codes, d.scales, d.x, d.xs = g.codes[2], g.scales[2], g.x, g.xs
    yg = gpu_call(g).cpu().numpy()[:, 0, :]
    yd = gpu_call(d).cpu().numpy()
    if wfmt == "mxfp4" and M >= 2:
        yr, A = oracle_call(d)
        assert_parity(yd, yr, A, "dense")
        assert_parity(yg, yr, A, "gather")
    else:
        assert np.array_equal(yg.view(np.uint32), yd.view(np.uint32))


def test_runs_on_callers_stream():
    inp = synth.make(synth.WORKLOADS["C2"].scaled(**SMALL["C2"]))
    dev = to_dev(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = gpu_call(inp, dev, stream=s)
    s.synchronize()
    yr, A = oracle_call(inp)
    assert_parity(y.cpu().numpy(), yr, A, "side stream")


def test_rejects_misaligned_and_leaves_y():
    import bit_block_quantized_amd as q
    inp = synth.make(synth.WORKLOADS["C1"])
    dev = to_dev(inp)
    y = torch.full((1, 256), 3.0, device="cuda")
    raw = torch.zeros(256 * 128 + 16, dtype=torch.uint8, device="cuda")
    codes = raw[1:1 + 256 * 128].view(256, 128)          # 1-byte offset
    with pytest.raises(q.QmvError) as e:
        q.qmv_dense("mxfp4", codes, dev["scales"], dev["x"], y=y)
    assert e.value.status == 1
    # K = 48 (not a multiple of 32) with buffers sized for it: the binding's
    # size checks pass and the library refuses the shape
    codes48 = dev["codes"][:, :24].contiguous()
    scales48 = dev["scales"][:, :1].contiguous()
    with pytest.raises(q.QmvError) as e:
        q.qmv_dense("mxfp4", codes48, scales48, dev["x"][:, :48].contiguous(), y=y)
    assert e.value.status == 2
    with pytest.raises(ValueError):                    # buffers sized for another K
        q.qmv_dense("mxfp4", dev["codes"], dev["scales"], dev["x"][:, :48], y=y)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_graph_replays_match_eager():
    """Calls captured in a HIP graph give the eager results on every replay,
    with eager work and synchronizations between the replays."""
    cases = [synth.make(synth.WORKLOADS[n].scaled(**SMALL[n])) for n in ("C2", "C3", "C4", "C5a", "C5b")]
    devs = [to_dev(inp) for inp in cases]
    eager = [gpu_call(inp, dev).clone() for inp, dev in zip(cases, devs)]
    outs = [torch.empty_like(e) for e in eager]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for inp, dev, out in zip(cases, devs, outs):
            gpu_call(inp, dev, y=out, stream=torch.cuda.current_stream())
    for rep in range(4):
        for out in outs:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, out in zip(eager, outs):
            assert torch.equal(e.view(torch.int32), out.view(torch.int32)), rep
        gpu_call(cases[0], devs[0])          # eager work between replays
        torch.cuda.synchronize()
