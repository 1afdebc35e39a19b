"""More than 4 activation vectors on the integer-activation paths: 2-bit and
3-bit codebook weights against int8 blocks (given, or bf16 quantized while
staged) and MXFP4 weights against int8 blocks (needs an MI355X).

2-bit and 3-bit weights with at least two vectors per expert on average run
on the int8 matrix-core kernel: each workgroup takes a run of (expert, row
tile) items of equal weighted cost, lists each expert's (token, slot) pairs in
LDS and stages them in chunks of up to 16 (2-bit) or 12 (3-bit) vectors.  The
other calls run on the grouped kernel: one launch, a workgroup per (row tile,
expert), the pairs taken four at a time through the decode kernels' row loop,
so an expert's rows are read once per four of its vectors.  Dense calls are
one expert with every vector.  MXFP4 x bf16 gathers with fewer than two pairs
per expert take the grouped route too (tests in test_gpu_batched.py).

Against the oracle on the same seeded inputs: every output within
1e-3 * sum |w x|; bit-exact at unit scales with int8 activations (integer
block sums, exact in fp32 in any order); zero rows for ids outside [0, E);
experts with far more than 128 vectors; skewed routing that splits one
expert's tiles over many workgroups (NaN-filled output, bit-exact); the
8192-pair and 1023-expert limits; and the DeepSeek-shaped prefill chunk at
full size on sampled outputs.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_exact, assert_parity, gpu_call, oracle_call

pytestmark = pytest.mark.gpu

# (weight format, activation format flag): int8 given, bf16 quantized in the
# kernel (2-/3-bit), int8 against MXFP4
PAIRS = [("cb2", ""), ("cb2", "bf16"), ("cb3", ""), ("cb3", "bf16"), ("mxfp4", "q8")]


def _wl(wfmt, act, kind, M, N, K, E=1, top_k=1, x_per_slot=False, seed=0):
    return synth.Workload("grouped", kind, wfmt, M=M, N=N, K=K, seed=seed, E=E, top_k=top_k,
                          x_per_slot=x_per_slot, x_bf16=act == "bf16", x_q8=act == "q8")


def _check(inp, what, exact=False):
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert y.shape == yr.shape
    if exact:
        assert_exact(y, yr, what)
    return assert_parity(y, yr, A, what)


def _name(p):
    return f"{p[0]}-{p[1] or 'q8'}"


@pytest.mark.parametrize("pair", PAIRS, ids=_name)
@pytest.mark.parametrize("M,N,K", [(5, 37, 64), (9, 130, 544), (24, 301, 2048), (64, 77, 7168)])
def test_dense(pair, M, N, K):
    wfmt, act = pair
    _check(synth.make(_wl(wfmt, act, "dense", M, N, K, seed=M + N)), f"{_name(pair)} dense M={M}")


@pytest.mark.parametrize("pair", PAIRS, ids=_name)
@pytest.mark.parametrize("M,top_k,E,N,K,per_slot", [(5, 4, 8, 45, 576, False),
                                                    (16, 4, 32, 300, 2048, False),
                                                    (64, 4, 256, 96, 1024, False),
                                                    (40, 6, 12, 259, 1440, True),
                                                    (8, 16, 20, 33, 64, True)])
def test_gather(pair, M, top_k, E, N, K, per_slot):
    wfmt, act = pair
    inp = synth.make(_wl(wfmt, act, "gather", M, N, K, E=E, top_k=top_k, x_per_slot=per_slot,
                         seed=7 * M + E))
    _check(inp, f"{_name(pair)} gather M={M} top_k={top_k} E={E}")


@pytest.mark.parametrize("pair", PAIRS, ids=_name)
def test_one_expert_takes_every_pair(pair):
    """300 pairs on one expert: 75 groups of four in each of its workgroups."""
    wfmt, act = pair
    inp = synth.make(_wl(wfmt, act, "gather", 300, 70, 256, E=4, top_k=1, seed=41))
    inp.ids[...] = 2
    _check(inp, f"{_name(pair)} one expert")


@pytest.mark.parametrize("pair", PAIRS, ids=_name)
def test_invalid_ids_give_zero_rows(pair):
    wfmt, act = pair
    inp = synth.make(_wl(wfmt, act, "gather", 24, 50, 256, E=6, top_k=3, seed=42))
    inp.ids[0, 1] = -1
    inp.ids[5, :] = 6
    inp.ids[9, 2] = 2 ** 31 - 1
    y = gpu_call(inp).cpu().numpy()
    assert (y[0, 1] == 0).all() and (y[5] == 0).all() and (y[9, 2] == 0).all()
    _check(inp, f"{_name(pair)} invalid ids")


def _unit(inp, seed=97):
    """Unit weight and activation scales, int8 activations over the full
    range: every block sum is an integer and every partial sum is exact."""
    wl = inp.wl
    if wl.wfmt == "mxfp4":
        inp.scales[...] = 127
    else:
        inp.scales.view(np.float16)[...] = 1.0
    rng = np.random.default_rng(seed)
    inp.x = rng.integers(-128, 128, size=inp.x.shape, dtype=np.int16).astype(np.int8)
    inp.xs = np.full(inp.x.shape[:-1] + (wl.K // 32,), 1.0, np.float16).view(np.uint16)
    return inp


@pytest.mark.parametrize("wfmt", ["cb2", "cb3", "mxfp4"])
@pytest.mark.parametrize("case", ["dense", "gather", "per-slot"])
def test_exact_at_unit_scales(wfmt, case):
    act = "q8" if wfmt == "mxfp4" else ""
    wl = {"dense": _wl(wfmt, act, "dense", 24, 77, 2048, seed=51),
          "gather": _wl(wfmt, act, "gather", 64, 45, 1024, E=32, top_k=4, seed=52),
          "per-slot": _wl(wfmt, act, "gather", 12, 33, 1056, E=5, top_k=4, x_per_slot=True,
                          seed=53)}[case]
    inp = _unit(synth.make(wl))
    _check(inp, f"unit {wfmt} {case}", exact=True)


def test_bf16_quantized_in_kernel_exact_sum():
    """bf16 activations whose every 32-block has absmax 127 * 2^k quantize to
    power-of-two scales, so with unit weight scales the call must equal, bit
    for bit, the same call on the oracle's int8 blocks and the oracle itself
    rounded to fp32: the in-kernel quantizer's integer decisions are pinned
    on the grouped kernel."""
    from test_gpu_quant import _exact_sum_bf16_x
    for wfmt in ("cb2", "cb3"):
        inp = synth.make(_wl(wfmt, "bf16", "gather", 20, 64, 1024, E=6, top_k=4, seed=57))
        inp.scales.view(np.float16)[...] = 1.0
        xb = _exact_sum_bf16_x(58, inp.x.shape[0], inp.wl.K)
        inp.x = xb
        y_b = gpu_call(inp).cpu().numpy()
        qx, d = oracle.load().quantize_q8(xb)
        qi = synth.make(_wl(wfmt, "", "gather", 20, 64, 1024, E=6, top_k=4, seed=57))
        qi.codes, qi.scales, qi.ids = inp.codes, inp.scales, inp.ids
        qi.x, qi.xs = qx, d
        y_q = gpu_call(qi).cpu().numpy()
        assert np.array_equal(y_b.view(np.uint32), y_q.view(np.uint32)), wfmt
        yr, _ = oracle_call(qi)
        assert_exact(y_b, yr, f"{wfmt} exact-sum bf16")


@pytest.mark.parametrize("pair", [("cb2", ""), ("cb3", "bf16"), ("mxfp4", "q8")], ids=_name)
def test_pair_and_expert_limits(pair):
    """8192 (token, slot) pairs (the LDS pair list's limit) and 1023 experts."""
    wfmt, act = pair
    _check(synth.make(_wl(wfmt, act, "gather", 2048, 20, 64, E=16, top_k=4, seed=81)),
           f"{_name(pair)} 8192 pairs")
    _check(synth.make(_wl(wfmt, act, "gather", 300, 24, 96, E=1023, top_k=4, seed=82)),
           f"{_name(pair)} 1023 experts")


def test_every_id_invalid_gives_zeros():
    import torch
    inp = synth.make(_wl("cb3", "", "gather", 40, 77, 128, E=5, top_k=3, seed=111))
    inp.ids[...] = -7
    out = torch.full((40, 3, 77), float("nan"), device="cuda")
    y = gpu_call(inp, y=out).cpu().numpy()
    assert (y == 0).all()


def test_bitwise_deterministic():
    from gpu_util import to_dev
    inp = synth.make(_wl("cb2", "bf16", "gather", 96, 200, 1024, E=16, top_k=4, seed=91))
    dev = to_dev(inp)
    y1 = gpu_call(inp, dev).cpu().numpy()
    y2 = gpu_call(inp, dev).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("name", ["C7", "C8"])
def test_prefill_chunk_full_size_sampled(name):
    """The DeepSeek-shaped prefill chunk (512 tokens x top-4 of 256) as
    bench.py launches it: 2-bit 7168 -> 2048 and 3-bit 2048 -> 7168 per-slot;
    sampled outputs and 4 whole (token, slot) rows against the oracle."""
    inp = synth.make(synth.workload(name))
    y = gpu_call(inp).cpu().numpy().reshape(-1)
    wl = inp.wl
    rng = np.random.default_rng(6)
    rows = rng.choice(wl.M * wl.top_k, size=4, replace=False)
    outs = np.concatenate([rng.choice(y.size, size=4000, replace=False)] +
                          [r * wl.N + np.arange(wl.N) for r in rows])
    yr, A = oracle_call(inp, outs=outs)
    assert_parity(y[outs], yr, A, f"{name} sampled")


@pytest.mark.parametrize("pair", PAIRS + [("mxfp4", "")], ids=lambda p: f"{p[0]}-{p[1] or ('bf16' if p[0] == 'mxfp4' else 'q8')}")
@pytest.mark.parametrize("M,top_k,E,per_slot", [(80, 2, 200, False), (70, 3, 256, True)])
def test_few_pairs_many_tokens(pair, M, top_k, E, per_slot):
    """Fewer than two pairs per expert and more than 64 tokens: one grouped
    launch (slots over the selected experts, balanced runs of row tiles).
    With 64 tokens or fewer the same calls run as token groups of 4 on the
    decode kernels (test_gpu_batched.py, test_gather_few_pairs_per_expert)."""
    wfmt, act = pair
    inp = synth.make(_wl(wfmt, act, "gather", M, 96, 512, E=E, top_k=top_k, x_per_slot=per_slot,
                         seed=3 * M + E))
    inp.ids[3, 0] = -1
    _check(inp, f"{wfmt} few pairs M={M}")


@pytest.mark.parametrize("pair", [("cb2", ""), ("mxfp4", "q8"), ("cb3", "bf16")], ids=_name)
def test_few_pairs_split_groups(pair):
    """At most 64 tokens and fewer than two pairs per expert: token groups of
    up to 4 (the last one ragged), one decode launch each, per-slot x."""
    wfmt, act = pair
    inp = synth.make(_wl(wfmt, act, "gather", 13, 70, 256, E=64, top_k=2, x_per_slot=True, seed=171))
    inp.ids[12, 1] = 64
    y = gpu_call(inp).cpu().numpy()
    assert (y[12, 1] == 0).all()
    _check(inp, f"{wfmt} split groups")


@pytest.mark.parametrize("pair", [("cb2", ""), ("cb2", "bf16"), ("cb3", "")], ids=_name)
def test_int8_matrix_cores_largest_k(pair):
    """K = 16384 (the largest K; 256 staged units per vector) on the int8
    matrix-core kernel: a dense call with 9 vectors and a gather with
    several vectors per expert."""
    wfmt, act = pair
    _check(synth.make(_wl(wfmt, act, "dense", 9, 40, 16384, seed=191)), f"{_name(pair)} K=16384 dense")
    _check(synth.make(_wl(wfmt, act, "gather", 12, 24, 16384, E=5, top_k=3, seed=192)),
           f"{_name(pair)} K=16384 gather")


def test_int8_matrix_cores_many_experts():
    """1023 experts with more than two pairs per expert on average (the
    bitmap's largest expert count) on the int8 matrix-core kernel."""
    _check(synth.make(_wl("cb3", "", "gather", 600, 40, 128, E=1023, top_k=4, seed=193)), "cb3 1023 experts")


def test_int8_matrix_cores_graph_replays():
    """Calls on the int8 matrix-core kernel captured in a HIP graph give the
    eager result bit for bit on every replay."""
    import torch
    from gpu_util import to_dev
    inp = synth.make(_wl("cb2", "", "gather", 64, 130, 1024, E=16, top_k=4, seed=194))
    dev = to_dev(inp)
    y1 = gpu_call(inp, dev).cpu().numpy()
    out = torch.empty(y1.shape, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gpu_call(inp, dev, y=out, stream=s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gpu_call(inp, dev, y=out, stream=torch.cuda.current_stream())
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), y1.view(np.uint32))


@pytest.mark.parametrize("wfmt", ["cb2", "cb3"])
def test_int8_matrix_cores_skewed_routing(wfmt):
    """Workgroups take runs of (expert, row tile) items of equal weighted cost
    (each expert's cost per tile grows with its vector count): one expert
    with most of the pairs (its tiles split over many workgroups, some
    workgroups left with no item), the rest with 1 to 20 vectors (several
    light experts in one workgroup's run, chunks of 1 to 16 vectors).  The
    output starts as NaN so that an item no workgroup takes fails; unit
    scales make the result bit-exact."""
    import torch
    inp = _unit(synth.make(_wl(wfmt, "", "gather", 300, 1000, 512, E=40, top_k=2, seed=195)))
    rng = np.random.default_rng(196)
    ids = np.full((300, 2), -1, np.int32)
    ids[:, 0] = 7
    spread = np.repeat(np.arange(40), rng.integers(1, 21, size=40))
    rng.shuffle(spread)
    ids[:, 1] = np.resize(spread, 300)
    ids[ids[:, 1] == 7, 1] = 8                      # distinct ids per token
    inp.ids = ids
    y = torch.full((300, 2, 1000), float("nan"), dtype=torch.float32, device="cuda")
    gpu_call(inp, y=y)
    yr, _ = oracle_call(inp)
    assert_exact(y.cpu().numpy(), yr, f"{wfmt} skewed routing")
