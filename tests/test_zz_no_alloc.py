"""The allocation-free combine entry point, qmv_gather_moe_combine_noalloc,
against the allocating qmv_gather_moe_combine through the C ABI (needs an
MI355X).

Both run the same kernels in the same order (the per-slot gather into a
temporary, then the ordered slot sum; up to 4 tokens the one-launch kernel),
so the outputs must agree bit for bit; the allocating entry point is itself
checked against the CPU oracle in test_gpu_combine.py, and the first case
here is checked against the oracle too.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_parity, to_dev
from test_gpu_combine import oracle_combine

pytestmark = pytest.mark.gpu


def _wl(wfmt, M, N, K, E, top_k, seed):
    return synth.Workload("noalloc-test", "combine", wfmt, M=M, N=N, K=K, seed=seed, E=E,
                          top_k=top_k, x_per_slot=True)


def _both(inp, dev=None):
    """(allocating, allocation-free) outputs of one call; the allocation-free
    output buffer starts as NaN."""
    import bit_block_quantized_amd as q
    dev = dev or to_dev(inp)
    wl = inp.wl
    M, top_k = inp.ids.shape
    wt = torch.from_numpy(np.ascontiguousarray(inp.extra["weights"], np.float32)).cuda()
    x = dev["x"].view(M, top_k, wl.K)
    xs = None if dev["xs"] is None else dev["xs"].view(M, top_k, wl.K // 32)
    ya = q.qmv_gather_moe_combine(wl.wfmt, dev["codes"], dev["scales"], dev["ids"], wt, x, xs,
                                  x_per_slot=True)
    yn = torch.full((M, wl.N), float("nan"), device="cuda")
    q.qmv_gather_moe_combine_noalloc(wl.wfmt, dev["codes"], dev["scales"], dev["ids"], wt, x, yn,
                                     xs, x_per_slot=True)
    torch.cuda.synchronize()
    return ya.cpu().numpy(), yn.cpu().numpy()


def _same(a, b, what):
    assert a.shape == b.shape, what
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


# two calls in a row per format pair, the second with a smaller input (fewer
# tokens, rows and slots): the second reuses the array the first wrote
CASES = {
    "mxfp4": [dict(M=96, N=200, K=512, E=8, top_k=4), dict(M=40, N=130, K=512, E=8, top_k=3)],
    "cb2": [dict(M=64, N=150, K=448, E=6, top_k=4), dict(M=9, N=70, K=448, E=6, top_k=2)],
    "cb3": [dict(M=48, N=260, K=320, E=20, top_k=5), dict(M=7, N=33, K=320, E=20, top_k=4)],
}


@pytest.mark.parametrize("wfmt", list(CASES))
def test_noalloc_equals_allocating_entry_twice(wfmt):
    for i, kw in enumerate(CASES[wfmt]):
        inp = synth.make(_wl(wfmt, seed=60 + i, **kw))
        ya, yn = _both(inp)
        _same(ya, yn, f"{wfmt} call {i} {kw}")
        if i == 0:
            yr, A = oracle_combine(inp)
            assert_parity(yn, yr, A, f"{wfmt} noalloc")


def test_noalloc_few_tokens_and_largest_temporary():
    """Up to 4 tokens (no temporary), then a call whose temporary fills the
    fixed array exactly (512 x 8 x 4096 floats = 64 MiB), then a small one."""
    import bit_block_quantized_amd as q
    inp = synth.make(_wl("mxfp4", M=3, N=90, K=256, E=5, top_k=4, seed=70))
    _same(*_both(inp), "3 tokens")
    M, top_k, N = 512, 8, 4096
    assert M * top_k * N * 4 == q.NOALLOC_SCRATCH_BYTES
    inp = synth.make(_wl("mxfp4", M=M, N=N, K=64, E=16, top_k=top_k, seed=71))
    _same(*_both(inp), "64 MiB temporary")
    inp = synth.make(_wl("cb3", M=6, N=40, K=64, E=3, top_k=2, seed=72))
    _same(*_both(inp), "small after the largest")


def test_noalloc_refuses_a_larger_temporary_and_leaves_y():
    import bit_block_quantized_amd as q
    M, top_k, N, K = 512, 8, 4097, 32
    codes = torch.zeros((1, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.full((1, N, K // 32), 127, dtype=torch.uint8, device="cuda")
    ids = torch.zeros((M, top_k), dtype=torch.int32, device="cuda")
    rw = torch.ones((M, top_k), dtype=torch.float32, device="cuda")
    x = torch.zeros((M, top_k, K), dtype=torch.bfloat16, device="cuda")
    y = torch.full((M, N), 7.0, device="cuda")
    s = q.lib().qmv_gather_moe_combine_noalloc(
        0, codes.data_ptr(), scales.data_ptr(), 1, ids.data_ptr(), rw.data_ptr(), M, top_k, 0,
        x.data_ptr(), None, 1, y.data_ptr(), N, K,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert s == 4, s
    torch.cuda.synchronize()
    assert (y == 7.0).all()
    with pytest.raises(q.QmvError):
        q.qmv_gather_moe_combine_noalloc("mxfp4", codes, scales, ids, rw, x, y)


def test_noalloc_graph_replays_match_eager():
    """Captured with nothing allocated inside the capture: replays reproduce
    the eager result, with eager calls of the same entry point between them
    (they share the array)."""
    import bit_block_quantized_amd as q
    inp = synth.make(_wl("cb2", M=32, N=96, K=256, E=6, top_k=4, seed=80))
    other = synth.make(_wl("mxfp4", M=20, N=64, K=256, E=4, top_k=4, seed=81))
    dev, dev_o = to_dev(inp), to_dev(other)
    ya, _ = _both(inp, dev)
    M, top_k = inp.ids.shape
    wt = torch.from_numpy(inp.extra["weights"]).cuda()
    x = dev["x"].view(M, top_k, -1)
    xs = dev["xs"].view(M, top_k, -1)
    out = torch.empty((M, inp.wl.N), device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q.qmv_gather_moe_combine_noalloc("cb2", dev["codes"], dev["scales"], dev["ids"], wt, x, out,
                                         xs, x_per_slot=True, stream=torch.cuda.current_stream())
    for rep in range(4):
        out.fill_(float("nan"))
        _both(other, dev_o)                     # an eager call in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(ya, out.cpu().numpy(), f"replay {rep}")
