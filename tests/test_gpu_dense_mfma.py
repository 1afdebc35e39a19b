"""Dense MXFP4 x bf16 with 2 to 4 activation vectors: the matrix-core kernel
(v_mfma_f32_4x4x4_16b_bf16, one wave per quad of rows, 16 units of a row per
load).  Needs an MI355X.

Against the oracle on the same seeded inputs: every output within
1e-3 * sum |w x|; bit-exact at unit scales with small-integer activations
(every partial sum is then an exact fp32 integer, so the MFMA's summation
order cannot show); NaN exactly where the oracle has NaN.  Shapes cover both
launch shapes the launcher picks (fewer than 1024 row quads: 4-wave
workgroups; more: 8-wave), partial last unit steps (K not a multiple of
512), ragged row quads (N % 4 != 0) and M = 2, 3.
"""
import numpy as np
import pytest

import synth
from gpu_util import assert_exact, assert_parity, gpu_call, oracle_call

pytestmark = pytest.mark.gpu


def _dense(M, N, K, seed):
    wl = synth.Workload("dense-mfma", "dense", "mxfp4", M=M, N=N, K=K, seed=seed)
    return synth.make(wl)


def _check(inp, what, exact=False):
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert y.shape == yr.shape
    if exact:
        assert_exact(y, yr, what)
    return assert_parity(y, yr, A, what)


@pytest.mark.parametrize("K", [32, 96, 480, 512, 544, 1056, 2880, 7168, 16384])
@pytest.mark.parametrize("M", [2, 3, 4])
def test_k_sweep(M, K):
    _check(_dense(M, 37, K, seed=100 + K + M), f"M={M} K={K}")


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 61, 4093, 4100])
def test_n_ragged(N):
    """N < 4096: 4-wave workgroups; N >= 4096: 8-wave workgroups."""
    _check(_dense(4, N, 7168 if N > 4000 else 1056, seed=200 + N), f"N={N}")


@pytest.mark.parametrize("M,N,K", [(4, 77, 7168), (3, 4100, 7168), (2, 29, 544), (4, 9, 16384)])
def test_exact_at_unit_scales(M, N, K):
    inp = _dense(M, N, K, seed=300 + M)
    inp.scales[...] = 127
    rng = np.random.default_rng(301)
    xs = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    inp.x = synth.bf16_bits(xs)
    _check(inp, f"unit M={M} N={N} K={K}", exact=True)


def test_special_scales_mixed_steps():
    """Scale bytes 0, 1, 253, 254 (outside the in-conversion range) and 255
    (NaN) in some 16-unit steps of a row, ordinary bytes elsewhere: the steps
    of one wave switch between the two decode paths."""
    inp = _dense(4, 12, 2048, seed=400)        # 64 units per row, 4 steps
    sc = inp.scales                            # uint8 [N][64]
    sc[0, 3] = 0
    sc[1, 17] = 1
    sc[2, 40:44] = 253
    sc[3, 63] = 254
    sc[4, 20] = 255                            # NaN row
    sc[5, :] = 0
    sc[6, :16] = 2
    sc[7, 16:32] = 252
    y = gpu_call(inp).cpu().numpy()
    yr, A = oracle_call(inp)
    assert np.isnan(yr[:, 4]).all()
    fin = (A < 3.0e38) | np.isnan(yr)
    assert_parity(y[fin], yr[fin], A[fin], "special scales")


def test_nonfinite_activations_stay_local():
    """An Inf activation reaches the rows that use it and nothing else (a
    partial last step must not pick up stale activation memory)."""
    inp = _dense(3, 21, 544, seed=500)          # 17 units: the second step is 1 of 16
    xf = np.zeros((3, 544), np.float32)
    xf[1, 530] = np.inf
    xf[0, :] = 1.0
    xf[2, 5] = -2.0
    inp.x = synth.bf16_bits(xf)
    _check(inp, "inf activation")


def test_bitwise_deterministic_and_streams():
    import torch
    from gpu_util import to_dev
    inp = _dense(4, 4100, 7168, seed=600)
    dev = to_dev(inp)
    y1 = gpu_call(inp, dev).cpu().numpy()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = gpu_call(inp, dev, stream=s)
    s.synchronize()
    assert np.array_equal(y1.view(np.uint32), y2.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("offset", [1, 3, 8, 15])
@pytest.mark.parametrize("N,K", [(13, 544), (4099, 7168)])
def test_unaligned_scale_array(offset, N, K):
    """MXFP4 scale arrays are plain bytes with no alignment promise: the
    workgroups stage their scale rows in 16-byte chunks from the aligned
    address below, loading a chunk that straddles the array's first or last
    byte one byte at a time.  Results must not depend on where the array
    starts, and nothing outside it may be read (the edge chunks)."""
    import torch
    import bit_block_quantized_amd as q
    from gpu_util import to_dev
    inp = _dense(4, N, K, seed=700 + offset)
    dev = to_dev(inp)
    flat = torch.zeros(inp.scales.size + 64, dtype=torch.uint8, device="cuda")
    base = (-flat.data_ptr()) % 16 + offset                 # 16-byte boundary + offset
    sc = flat[base:base + inp.scales.size].view(inp.scales.shape)
    sc.copy_(torch.from_numpy(inp.scales).cuda())
    assert sc.data_ptr() % 16 == offset
    y = q.qmv_dense("mxfp4", dev["codes"], sc, dev["x"]).cpu().numpy()
    y0 = gpu_call(inp, dev).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    yr, A = oracle_call(inp)
    assert_parity(y, yr, A, f"scales at +{offset}")
