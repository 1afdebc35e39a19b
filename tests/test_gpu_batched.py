"""MXFP4 x bf16 with more than 4 activation vectors: the expert-batched
matrix-core path (v_mfma_f32_32x32x16_bf16; every workgroup lists its
expert's (token, slot) pairs in LDS, tiles of one expert x up to 128 vectors
x a few 32-row fragments per wave).  Needs an MI355X.

Against the oracle on the same seeded inputs: every output within
1e-3 * sum |w x|; bit-exact at unit scales with small-integer activations
(every partial sum is an exact fp32 integer, so the MFMA's order cannot
show); NaN exactly where the oracle has NaN; zero rows for ids outside
[0, E).  Cases: dense and gather, broadcast and per-slot activations,
experts with more than 128 vectors (chunked), all pairs on one expert,
ragged N and K (partial 128-weight slices), E8M0 bytes outside [2, 252] and
Inf activations, the pair and expert limits, and the full-size prefill chunk
on sampled outputs.

Which kernel a call reaches: dense calls with 5 to 8 vectors run as groups
of up to 4 vectors on the dense 4-vector kernel, dense calls with 9 to 64
vectors on the K-split tiles (the waves of a workgroup split K, partial tiles
summed in LDS; one 32-vector column fragment up to 32 vectors, two above),
gathers with fewer than two (token, slot) pairs per expert as token groups
on the decode kernels (test_gather_few_pairs_*); every other call with more
than 4 vectors runs on the batched kernel.  The special-value cases below use
dense calls with 24 and 40 vectors (K-split), dense calls with 72 vectors
(batched) and gathers with M * top_k >= 2 E (batched).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_exact, assert_parity, gpu_call, oracle_call, to_dev

pytestmark = pytest.mark.gpu


def _wl(kind, M, N, K, E=1, top_k=1, x_per_slot=False, seed=0, e8m0=(122, 132)):
    return synth.Workload("batched", kind, "mxfp4", M=M, N=N, K=K, seed=seed, E=E, top_k=top_k,
                          x_per_slot=x_per_slot, e8m0=e8m0)


def _check(inp, what, exact=False):
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert y.shape == yr.shape
    if exact:
        assert_exact(y, yr, what)
    return assert_parity(y, yr, A, what)


@pytest.mark.parametrize("M,N,K", [(5, 37, 32), (8, 45, 96), (9, 40, 64), (16, 130, 544), (32, 33, 2880),
                                   (64, 301, 2880), (129, 64, 160), (200, 257, 1056), (33, 513, 7168),
                                   (48, 70, 4160), (65, 97, 2080), (40, 35, 96), (64, 40, 16384),
                                   (33, 17, 16384)])
def test_dense(M, N, K):
    _check(synth.make(_wl("dense", M, N, K, seed=M + N + K)), f"dense M={M} N={N} K={K}")


@pytest.mark.parametrize("M,top_k,E,N,K", [(5, 4, 8, 45, 576), (16, 4, 32, 300, 2880),
                                           (64, 4, 32, 96, 2880), (200, 2, 2, 260, 320),
                                           (40, 6, 12, 259, 1440), (8, 16, 20, 33, 64)])
def test_gather(M, top_k, E, N, K):
    _check(synth.make(_wl("gather", M, N, K, E=E, top_k=top_k, seed=7 * M + E)),
           f"gather M={M} top_k={top_k} E={E} N={N} K={K}")


@pytest.mark.parametrize("M,top_k", [(16, 4), (7, 3)])
def test_gather_per_slot(M, top_k):
    inp = synth.make(_wl("gather", M, 140, 1056, E=9, top_k=top_k, x_per_slot=True, seed=31 + M))
    _check(inp, f"per-slot M={M} top_k={top_k}")


def test_one_expert_takes_every_pair():
    """300 pairs on one expert: three chunks of 100 vectors, over three row
    tiles (workgroups that sort the pairs each in their own order)."""
    inp = synth.make(_wl("gather", 300, 300, 352, E=4, top_k=1, seed=41))
    inp.ids[...] = 2
    _check(inp, "one expert")


def test_invalid_ids_give_zero_rows():
    inp = synth.make(_wl("gather", 24, 50, 256, E=6, top_k=3, seed=42))
    inp.ids[0, 1] = -1
    inp.ids[5, :] = 6
    inp.ids[9, 2] = 2 ** 31 - 1
    y = gpu_call(inp).cpu().numpy()
    assert (y[0, 1] == 0).all() and (y[5] == 0).all() and (y[9, 2] == 0).all()
    _check(inp, "invalid ids")


@pytest.mark.parametrize("case", ["dense", "gather", "per-slot"])
def test_exact_at_unit_scales(case):
    wl = {"dense": _wl("dense", 24, 77, 2880, seed=51),
          "gather": _wl("gather", 64, 45, 2880, E=32, top_k=4, seed=52),
          "per-slot": _wl("gather", 12, 33, 1056, E=5, top_k=4, x_per_slot=True, seed=53)}[case]
    inp = synth.make(wl)
    inp.scales[...] = 127
    rng = np.random.default_rng(54)
    vals = rng.integers(-3, 4, size=inp.x.shape).astype(np.float32)
    inp.x = synth.bf16_bits(vals)
    _check(inp, f"unit {case}", exact=True)


def _assert_special(inp, what):
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    # outputs whose |w x| sum passes fp32's range may overflow either way
    m = (A < 3.0e38) | np.isnan(yr)
    assert np.array_equal(np.isnan(y[m]), np.isnan(yr[m])), what
    fin = (A < 3.0e38) & ~np.isnan(yr)
    assert_parity(y[fin], yr[fin], A[fin], what)
    return yr


def test_e8m0_special_scales():
    """Slices holding scale bytes outside [2, 252] take the exact path:
    0 (2^-127, an fp32 subnormal), 1, 253, 254 and 255 (NaN).  A dense call
    with 24 vectors (the batched kernel)."""
    inp = synth.make(_wl("dense", 24, 40, 320, seed=61))
    inp.scales[0, :] = 0
    inp.scales[1, :] = 1
    inp.scales[2, :] = 254
    inp.scales[3, 4] = 255
    inp.scales[4, :] = [0, 127, 254, 127, 1, 253, 2, 252, 127, 127]
    inp.scales[17, 9] = 0                    # one byte in the last (partial) slice
    inp.scales[39, 0] = 255
    yr = _assert_special(inp, "e8m0 specials, dense")
    assert np.isnan(yr[:, 3]).all() and np.isnan(yr[:, 39]).all()


@pytest.mark.parametrize("M", [40, 72])
def test_e8m0_special_scales_dense_batched(M):
    """The same special scale bytes on dense calls with 40 vectors (the
    K-split tiles with two column fragments) and 72 vectors (the batched
    kernel), each through its exact path."""
    inp = synth.make(_wl("dense", M, 40, 320, seed=63))
    inp.scales[0, :] = 0
    inp.scales[2, :] = 254
    inp.scales[3, 4] = 255
    inp.scales[4, :] = [0, 127, 254, 127, 1, 253, 2, 252, 127, 127]
    inp.scales[39, 9] = 1
    yr = _assert_special(inp, f"e8m0 specials, dense M={M}")
    assert np.isnan(yr[:, 3]).all()


def test_e8m0_special_scales_gather_chunked():
    """A special scale byte in an expert that holds more than 128 vectors
    (two chunks), and in another expert's last rows, on a gather."""
    inp = synth.make(_wl("gather", 300, 70, 416, E=3, top_k=1, seed=62))
    inp.ids[:200, 0] = 1                      # expert 1: 200 vectors
    inp.ids[200:, 0] = np.where(np.arange(100) % 2 == 0, 0, 2)
    inp.scales[1, 5, 3] = 0
    inp.scales[1, 6, :] = 254
    inp.scales[1, 69, 12] = 255
    inp.scales[2, 68, 0] = 1
    inp.scales[2, 0, 12] = 253
    yr = _assert_special(inp, "e8m0 specials, gather")
    assert np.isnan(yr[:200, 0, 69]).all()


def test_inf_activation_stays_in_its_column():
    """An Inf activation reaches only the outputs of its own vector (dense,
    24 vectors: the batched kernel)."""
    inp = synth.make(_wl("dense", 24, 36, 480, seed=71))
    inp.x[7, 100] = 0x7F80                   # +Inf
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert np.array_equal(np.isnan(y), np.isnan(yr)) and np.array_equal(np.isinf(y), np.isinf(yr))
    ok = np.isfinite(yr)
    assert ok[np.arange(24) != 7].all()
    assert_parity(y[ok], yr[ok], A[ok], "inf column")


def test_pair_and_expert_limits():
    """8192 (token, slot) pairs (the LDS sort's limit) and 1023 experts."""
    _check(synth.make(_wl("gather", 2048, 20, 64, E=16, top_k=4, seed=81)), "8192 pairs")
    _check(synth.make(_wl("gather", 300, 24, 96, E=1023, top_k=4, seed=82)), "1023 experts")


def test_bitwise_deterministic_and_graph():
    inp = synth.make(_wl("gather", 96, 200, 1440, E=16, top_k=4, seed=91))
    dev = to_dev(inp)
    y1 = gpu_call(inp, dev).cpu().numpy()
    y2 = gpu_call(inp, dev).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    out = torch.empty_like(torch.from_numpy(y1)).cuda()
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


def test_prefill_chunk_full_size_sampled():
    """The gpt-oss-20b prefill chunk (512 tokens x top-4 of 32, K=N=2880) as
    bench.py launches it; 6000 sampled outputs against the oracle, and the
    outputs of 8 whole (token, slot) rows."""
    inp = synth.make(synth.workload("C6"))
    y = gpu_call(inp).cpu().numpy().reshape(-1)
    wl = inp.wl
    rng = np.random.default_rng(5)
    rows = rng.choice(wl.M * wl.top_k, size=8, replace=False)
    outs = np.concatenate([rng.choice(y.size, size=6000, replace=False)] +
                          [r * wl.N + np.arange(wl.N) for r in rows])
    yr, A = oracle_call(inp, outs=outs)
    assert_parity(y[outs], yr, A, "C6 sampled")


def test_dense_wide_full_size_sampled():
    """Dense 7168 x 7168 MXFP4 against 64 vectors (the K-split tiles with two
    column fragments) as bench.py launches it: sampled outputs and 2 whole
    rows of y."""
    inp = synth.make(synth.workload("C6d"))
    y = gpu_call(inp).cpu().numpy().reshape(-1)
    wl = inp.wl
    rng = np.random.default_rng(7)
    outs = np.concatenate([rng.choice(y.size, size=4000, replace=False),
                           np.arange(wl.N), 37 * wl.N + np.arange(wl.N)])
    yr, A = oracle_call(inp, outs=outs)
    assert_parity(y[outs], yr, A, "C6d sampled")


def test_gather_tall_tiles():
    """Enough (expert, row tile) tiles for the 8-wave 256-row kernel (one per
    CU and more), with a ragged last tile and N % 4 != 0 (element-wise
    stores)."""
    _check(synth.make(_wl("gather", 96, 1281, 256, E=48, top_k=4, seed=101)), "256-row tiles")


def test_every_id_invalid_gives_zeros():
    inp = synth.make(_wl("gather", 40, 77, 128, E=5, top_k=3, seed=111))
    inp.ids[...] = -7
    out = torch.full((40, 3, 77), float("nan"), device="cuda")
    y = gpu_call(inp, y=out).cpu().numpy()
    assert (y == 0).all()


def test_pair_limit_per_slot():
    """8192 (token, slot) pairs, one activation vector each."""
    _check(synth.make(_wl("gather", 1024, 12, 64, E=24, top_k=8, x_per_slot=True, seed=121)),
           "8192 per-slot pairs")


@pytest.mark.parametrize("M,top_k,E,per_slot", [(5, 4, 256, False), (8, 4, 256, False),
                                                (6, 2, 64, True), (64, 4, 256, False)])
def test_gather_few_pairs_per_expert(M, top_k, E, per_slot):
    """Fewer than two pairs per expert: groups of up to 4 tokens on the decode
    kernels (a ragged last group included), broadcast and per-slot x."""
    _check(synth.make(_wl("gather", M, 40, 256, E=E, top_k=top_k, x_per_slot=per_slot, seed=131 + M)),
           f"few pairs M={M} top_k={top_k} E={E}")


def test_gather_few_pairs_invalid_ids():
    inp = synth.make(_wl("gather", 7, 33, 160, E=100, top_k=3, seed=141))
    inp.ids[5, 1] = -1
    inp.ids[6, :] = 100
    y = gpu_call(inp).cpu().numpy()
    assert (y[5, 1] == 0).all() and (y[6] == 0).all()
    _check(inp, "few pairs, invalid ids")
