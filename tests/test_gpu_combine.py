"""Down projection with the router-weighted top-k combine against the CPU
oracle (needs an MI355X).

y[t][n] = sum_j w[t][j] * g(t, j, n), with g the per-slot gather output.  The
oracle returns y in fp64 and A[t][n] = sum_j |w[t][j]| * A_gather(t, j, n);
each slot's dot product on the GPU is within the gather's bound and the fp32
weighted sum of at most 16 terms adds a few ulp of sum_j |w_j g_j| <= A, so
the bar stays |y - y_ref| <= 1e-3 * A per output.  Where every product and
partial sum is exact (unit scales, small-integer activations, power-of-two
router weights) the result must be bit-exact.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_exact, assert_parity, gpu_call, threads, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["mxfp4", "cb2", "cb3"]


def gpu_combine(inp, dev=None, y=None, stream=None, weights=None):
    import bit_block_quantized_amd as q
    wl = inp.wl
    dev = dev or to_dev(inp)
    w = inp.extra["weights"] if weights is None else weights
    wt = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    M, top_k = inp.ids.shape
    x, xs = dev["x"], dev["xs"]
    if wl.x_per_slot:
        x = x.view(M, top_k, wl.K)
        xs = None if xs is None else xs.view(M, top_k, wl.K // 32)
    return q.qmv_gather_moe_combine(wl.wfmt, dev["codes"], dev["scales"], dev["ids"], wt, x, xs,
                                    x_per_slot=wl.x_per_slot, y=y, stream=stream)


def oracle_combine(inp, weights=None, outs=None):
    """The oracle's combine at every output ([M][N]), or at the flat output
    indices ``outs`` (1-D)."""
    o = oracle.load()
    wl = inp.wl
    w = inp.extra["weights"] if weights is None else weights
    M = inp.ids.shape[0]
    sel = np.arange(M * wl.N, dtype=np.int64) if outs is None else np.asarray(outs, np.int64)
    parts = np.array_split(sel, max(1, min(threads(), len(sel) // 64 + 1)))

    def run(p):
        return o.combine(wl.wfmt, inp.codes, inp.scales, inp.ids, w, wl.afmt, inp.x, inp.xs,
                         x_per_slot=wl.x_per_slot, outs=p)

    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(run, parts))
    y = np.concatenate([r[0] for r in res])
    A = np.concatenate([r[1] for r in res])
    if outs is None:
        return y.reshape(M, wl.N), A.reshape(M, wl.N)
    return y, A


def _combine_wl(wfmt, M=1, N=59, K=None, E=16, top_k=4, x_per_slot=True, seed=0):
    K = K or {"mxfp4": 2880, "cb2": 7168, "cb3": 2048}[wfmt]
    return synth.Workload("combine-test", "combine", wfmt, M=M, N=N, K=K, seed=seed, E=E,
                          top_k=top_k, x_per_slot=x_per_slot)


def _check(inp, what):
    y = gpu_combine(inp).cpu().numpy()
    yr, A = oracle_combine(inp)
    assert y.shape == yr.shape == (inp.ids.shape[0], inp.wl.N)
    return assert_parity(y, yr, A, what)


# The combine workloads with small expert tables: real K, N over several row
# tiles plus a ragged tail.
SMALL = {
    "C4c": dict(E=16, N=1000),
    "C2c": dict(E=8, N=87),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_workload_small(name):
    inp = synth.make(synth.COMBINE_WORKLOADS[name].scaled(**SMALL[name]))
    _check(inp, name)


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("top_k", [1, 3, 4, 6, 8, 16])
def test_top_k_groups(wfmt, top_k):
    """Slots are taken four at a time: 1 to 4 groups, including partial ones."""
    wl = _combine_wl(wfmt, N=45, K=576, E=20, top_k=top_k, seed=top_k)
    _check(synth.make(wl), f"{wfmt} top_k={top_k}")


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 17, 40])
@pytest.mark.parametrize("per_slot", [True, False])
def test_m_sweep(wfmt, M, per_slot):
    """Up to 4 tokens on the one-launch combine kernel; more as the gather
    (40 tokens x 5 slots over 7 experts: the matrix-core kernels) followed
    by the slot sum."""
    wl = _combine_wl(wfmt, M=M, N=70, K=448, E=7, top_k=5, x_per_slot=per_slot, seed=10 + M)
    _check(synth.make(wl), f"{wfmt} M={M} per_slot={per_slot}")


def test_k_not_multiple_of_64_two_bit():
    """K % 64 != 0 selects the 32-weight 2-bit unit."""
    wl = _combine_wl("cb2", M=2, N=33, K=96, E=5, top_k=3, seed=3)
    _check(synth.make(wl), "cb2 K=96")


@pytest.mark.parametrize("wfmt", FMTS)
def test_invalid_ids_contribute_nothing(wfmt):
    wl = _combine_wl(wfmt, M=3, N=50, K=256, E=6, top_k=5, seed=21)
    inp = synth.make(wl)
    inp.ids = np.array([[-1, 2, 6, 4, 1], [2 ** 31 - 1, 5, 5, 0, -7], [6, 6, 6, 6, 6]], np.int32)
    y = gpu_combine(inp).cpu().numpy()
    yr, A = oracle_combine(inp)
    assert_parity(y, yr, A, wfmt)
    assert not y[2].any()           # every slot invalid: zero row


def _unit_scale(inp):
    wl = inp.wl
    if wl.wfmt == "mxfp4":
        inp.scales[...] = 127
        g = np.random.default_rng(99).integers(-8, 9, size=inp.x.shape).astype(np.float32)
        inp.x = synth.bf16_bits(g)
    else:
        inp.scales.view(np.float16)[...] = 1.0
        inp.xs.view(np.float16)[...] = 1.0
        inp.x = np.random.default_rng(98).integers(-128, 128, size=inp.x.shape,
                                                    dtype=np.int16).astype(np.int8)
    return inp


@pytest.mark.parametrize("wfmt", FMTS)
def test_exact_at_unit_scales(wfmt):
    """Unit scales, small-integer activations and power-of-two router weights:
    every term and partial sum is exact, so the result is bit-exact."""
    wl = _combine_wl(wfmt, M=2, N=77, E=9, top_k=6, seed=5)
    inp = _unit_scale(synth.make(wl))
    w = np.array([[0.5, 0.25, 0.125, 1.0, 2.0, 1.0], [1.0, 0.5, 0.5, 0.25, 0.125, 2.0]],
                 np.float32)
    y = gpu_combine(inp, weights=w).cpu().numpy()
    yr, _ = oracle_combine(inp, weights=w)
    assert_exact(y, yr, wfmt)


@pytest.mark.parametrize("wfmt", FMTS)
def test_one_hot_weights_equal_gather_rows(wfmt):
    """A one-hot weight picks one slot: at unit scales the combine equals the
    per-slot gather's row for that slot bit for bit."""
    wl = _combine_wl(wfmt, M=1, N=91, E=9, top_k=4, seed=6)
    inp = _unit_scale(synth.make(wl))
    dev = to_dev(inp)
    g = gpu_call(synth.Inputs(wl.scaled(kind="gather"), inp.codes, inp.scales, inp.ids, inp.x,
                              inp.xs), dev).cpu().numpy()
    for j in range(4):
        w = np.zeros((1, 4), np.float32)
        w[0, j] = 1.0
        y = gpu_combine(inp, dev, weights=w).cpu().numpy()
        assert np.array_equal(y[0].view(np.uint32), g[0, j].view(np.uint32)), j


@pytest.mark.parametrize("wfmt", FMTS)
def test_signed_and_zero_sum_weights(wfmt):
    """Router weights of either sign (uniform in [-1, 1]) against the oracle;
    at unit scales, a token whose weights are +a and -a on two slots of one
    expert fed the same vector gets exactly the other slots' sum, and negated
    weights give exactly the negated result."""
    wl = _combine_wl(wfmt, M=3, N=66, K=320, E=5, top_k=4, seed=17)
    inp = synth.make(wl)
    w = np.random.default_rng(171).uniform(-1.0, 1.0, size=(3, 4)).astype(np.float32)
    y = gpu_combine(inp, weights=w).cpu().numpy()
    yr, A = oracle_combine(inp, weights=w)
    assert_parity(y, yr, A, f"{wfmt} signed weights")
    # zero-sum: broadcast activations, slots 0 and 1 of token 0 on one expert
    wlb = _combine_wl(wfmt, M=2, N=66, K=320, E=5, top_k=4, x_per_slot=False, seed=18)
    inp = _unit_scale(synth.make(wlb))
    inp.ids[0, :] = [3, 3, 1, 4]
    wz = np.array([[0.75, -0.75, 0.5, -2.0], [-0.25, 1.0, -0.5, 0.125]], np.float32)
    y = gpu_combine(inp, weights=wz).cpu().numpy()
    yr, _ = oracle_combine(inp, weights=wz)
    assert_exact(y, yr, f"{wfmt} zero-sum weights")
    yn = gpu_combine(inp, weights=-wz).cpu().numpy()
    assert np.array_equal(yn, -y)
    only = wz.copy()
    only[0, :2] = 0.0
    y2 = gpu_combine(inp, weights=only).cpu().numpy()
    assert np.array_equal(y[0], y2[0])


@pytest.mark.parametrize("wfmt", FMTS)
def test_many_tokens_one_hot_and_exact(wfmt):
    """More than 4 tokens: a one-hot weight on slot j gives exactly the per-slot
    gather's row j of every token (the gather runs the same kernel into the
    combine's temporary), and at unit scales with power-of-two weights the
    result is bit-exact against the oracle; invalid ids included."""
    M, top_k = 24, 4
    wl = _combine_wl(wfmt, M=M, N=75, K=320, E=6, top_k=top_k, seed=31)
    inp = _unit_scale(synth.make(wl))
    inp.ids[3, 1] = -1
    inp.ids[7, :] = 6
    dev = to_dev(inp)
    g = gpu_call(synth.Inputs(wl.scaled(kind="gather"), inp.codes, inp.scales, inp.ids, inp.x,
                              inp.xs), dev).cpu().numpy()
    for j in range(top_k):
        w = np.zeros((M, top_k), np.float32)
        w[:, j] = 1.0
        y = gpu_combine(inp, dev, weights=w).cpu().numpy()
        assert np.array_equal(y.view(np.uint32), g[:, j].view(np.uint32)), j
    w = np.random.default_rng(32).choice(np.float32([0.125, 0.25, -0.5, 1.0, 2.0, -4.0]),
                                         size=(M, top_k)).astype(np.float32)
    y = gpu_combine(inp, dev, weights=w).cpu().numpy()
    yr, _ = oracle_combine(inp, weights=w)
    assert_exact(y, yr, f"{wfmt} many tokens, unit scales")
    assert not y[7].any()


@pytest.mark.parametrize("name", ["C6c", "C8c"])
def test_prefill_combine_full_size_sampled(name):
    """The prefill chunks' down projections with the combine, as bench.py
    launches them: sampled outputs and 2 whole rows of y against the oracle."""
    inp = synth.make(synth.workload(name))
    y = gpu_combine(inp).cpu().numpy().reshape(-1)
    wl = inp.wl
    rng = np.random.default_rng(11)
    outs = np.concatenate([rng.choice(y.size, size=3000, replace=False),
                           np.arange(wl.N), 301 * wl.N + np.arange(wl.N)])
    yr, A = oracle_combine(inp, outs=outs)
    worst = assert_parity(y[outs], yr, A, f"{name} sampled")
    print(f"{name}: worst |err| / bound = {worst:.3e}")


@pytest.mark.parametrize("wfmt", FMTS)
def test_many_tokens_at_the_pair_limit(wfmt):
    """8192 (token, slot) pairs, the most a call with more than 4 tokens may
    have: 2048 tokens x 4 slots over 24 experts, sampled outputs against the
    oracle."""
    inp = synth.make(_combine_wl(wfmt, M=2048, N=40, K=128, E=24, top_k=4, seed=43))
    y = gpu_combine(inp).cpu().numpy().reshape(-1)
    rng = np.random.default_rng(44)
    outs = np.concatenate([rng.choice(y.size, size=3000, replace=False), np.arange(40),
                           2047 * 40 + np.arange(40)])
    yr, A = oracle_combine(inp, outs=outs)
    assert_parity(y[outs], yr, A, f"{wfmt} 8192 pairs")


def test_many_tokens_on_two_streams_at_once():
    """Many-token combines queued on two streams without synchronizing
    between them: each call takes its temporary from the pool in its own
    stream's order, so the results equal the calls made one at a time."""
    cases = [synth.make(_combine_wl(f, M=48, N=130, K=320, E=6, top_k=4, seed=61 + i))
             for i, f in enumerate(["mxfp4", "cb3"])]
    devs = [to_dev(inp) for inp in cases]
    ref = [gpu_combine(inp, dev).cpu().numpy() for inp, dev in zip(cases, devs)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty((48, 130), device="cuda") for _ in range(6)] for _ in cases]
    torch.cuda.synchronize()
    for rep in range(6):
        for c, (inp, dev) in enumerate(zip(cases, devs)):
            with torch.cuda.stream(streams[c]):
                gpu_combine(inp, dev, y=outs[c][rep], stream=streams[c])
    torch.cuda.synchronize()
    for c in range(2):
        for rep in range(6):
            assert np.array_equal(outs[c][rep].cpu().numpy().view(np.uint32), ref[c].view(np.uint32)), (c, rep)


def test_many_tokens_leaves_nothing_past_y_and_repeats():
    """The many-token combine writes every row of y, nothing past it, and the
    same bits on a second call (its temporary comes back from the pool)."""
    wl = _combine_wl("mxfp4", M=33, N=130, K=256, E=5, top_k=3, seed=41)
    inp = synth.make(wl)
    dev = to_dev(inp)
    n = wl.M * wl.N
    buf = torch.full((n + 4096,), float("nan"), device="cuda")
    buf[n:] = 12345.0
    y1 = gpu_combine(inp, dev, y=buf[:n].view(wl.M, wl.N)).cpu().numpy().copy()
    assert (buf[n:].cpu().numpy() == 12345.0).all()
    assert not np.isnan(y1).any()
    y2 = gpu_combine(inp, dev).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("name", list(SMALL))
def test_bitwise_deterministic(name):
    inp = synth.make(synth.COMBINE_WORKLOADS[name].scaled(**SMALL[name]))
    dev = to_dev(inp)
    y1 = gpu_combine(inp, dev).cpu().numpy()
    y2 = gpu_combine(inp, dev).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_writes_every_row_and_nothing_past_y():
    wl = synth.COMBINE_WORKLOADS["C4c"].scaled(E=16, N=1000, M=2)
    inp = synth.make(wl)
    n = 2 * wl.N
    buf = torch.full((n + 4096,), float("nan"), device="cuda")
    buf[n:] = 12345.0
    gpu_combine(inp, y=buf[:n].view(2, wl.N))
    assert (buf[n:].cpu().numpy() == 12345.0).all()
    assert not np.isnan(buf[:n].cpu().numpy()).any()


def test_rejects_missing_route_weights_and_leaves_y():
    import ctypes

    import bit_block_quantized_amd as q
    wl = _combine_wl("cb3", N=16, K=64, E=2, top_k=2)
    inp = synth.make(wl)
    dev = to_dev(inp)
    y = torch.full((1, 16), 3.0, device="cuda")
    s = q.lib().qmv_gather_moe_combine(2, dev["codes"].data_ptr(), dev["scales"].data_ptr(), 2,
                                       dev["ids"].data_ptr(), None, 1, 2, 1,
                                       dev["x"].data_ptr(), dev["xs"].data_ptr(), 1,
                                       y.data_ptr(), 16, 64,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert s == 1
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_graph_replays_match_eager():
    cases = [synth.make(synth.COMBINE_WORKLOADS[n].scaled(**SMALL[n])) for n in SMALL]
    devs = [to_dev(inp) for inp in cases]
    eager = [gpu_combine(inp, dev).clone() for inp, dev in zip(cases, devs)]
    outs = [torch.empty_like(e) for e in eager]
    wts = [torch.from_numpy(inp.extra["weights"]).cuda() for inp in cases]
    import bit_block_quantized_amd as q
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for inp, dev, out, wt in zip(cases, devs, outs, wts):
            M, top_k = inp.ids.shape
            xs = None if dev["xs"] is None else dev["xs"].view(M, top_k, -1)
            q.qmv_gather_moe_combine(inp.wl.wfmt, dev["codes"], dev["scales"], dev["ids"], wt,
                                     dev["x"].view(M, top_k, -1), xs, x_per_slot=True, y=out,
                                     stream=torch.cuda.current_stream())
    for rep in range(4):
        for out in outs:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, out in zip(eager, outs):
            assert torch.equal(e.view(torch.int32), out.view(torch.int32)), rep


def test_many_tokens_graph_replays_match_eager():
    """A captured many-token combine (its temporary becomes the graph's own
    allocation) replays to the eager result every time."""
    import bit_block_quantized_amd as q
    cases = [synth.make(_combine_wl(f, M=24, N=96, K=320, E=6, top_k=4, seed=51 + i))
             for i, f in enumerate(FMTS)]
    devs = [to_dev(inp) for inp in cases]
    eager = [gpu_combine(inp, dev).clone() for inp, dev in zip(cases, devs)]
    outs = [torch.empty_like(e) for e in eager]
    wts = [torch.from_numpy(inp.extra["weights"]).cuda() for inp in cases]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for inp, dev, out, wt in zip(cases, devs, outs, wts):
            M, top_k = inp.ids.shape
            xs = None if dev["xs"] is None else dev["xs"].view(M, top_k, -1)
            q.qmv_gather_moe_combine(inp.wl.wfmt, dev["codes"], dev["scales"], dev["ids"], wt,
                                     dev["x"].view(M, top_k, -1), xs, x_per_slot=True, y=out,
                                     stream=torch.cuda.current_stream())
    for rep in range(4):
        for out in outs:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, out in zip(eager, outs):
            assert torch.equal(e.view(torch.int32), out.view(torch.int32)), rep


@pytest.mark.slow
@pytest.mark.parametrize("name", list(synth.COMBINE_WORKLOADS))
def test_full_size(name):
    """The combine workloads at their full expert tables, every output checked."""
    inp = synth.make(synth.COMBINE_WORKLOADS[name])
    worst = _check(inp, name)
    print(f"{name}: worst |err| / bound = {worst:.3e}")
