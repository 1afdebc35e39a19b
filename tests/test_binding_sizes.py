"""The Python binding checks every tensor's size against the call's shape
before anything reaches the library (no GPU needed).

The kernels derive buffer extents from N, K, M and top_k alone, so a tensor
smaller than those sizes imply would be read or written out of bounds on the
device.  Each case below passes CPU tensors: a consistent call gets as far as
the device check ("runs on the GPU only"), and each inconsistent one is
rejected with a ValueError naming the tensor.
"""
import pytest
import torch

import bit_block_quantized_amd as q

E, N, K, M, TOPK = 6, 40, 128, 3, 2


def w(fmt, E=E, N=N, K=K):
    rcb, rsb = {"mxfp4": (K // 2, K // 32), "cb2": (K // 4, K // 16), "cb3": (3 * K // 8, K // 8)}[fmt]
    return torch.zeros(E, N, rcb, dtype=torch.uint8), torch.zeros(E, N, rsb, dtype=torch.uint8)


def ids(M=M, top_k=TOPK):
    return torch.zeros(M, top_k, dtype=torch.int32)


def xb(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def x8(*shape):
    return torch.zeros(*shape, dtype=torch.int8), torch.zeros(*shape[:-1], shape[-1] // 32, dtype=torch.float16)


def _gpu_only(fn, *a, **kw):
    with pytest.raises(ValueError, match="GPU only"):
        fn(*a, **kw)


def _bad(what, fn, *a, **kw):
    with pytest.raises(ValueError, match=what):
        fn(*a, **kw)


def test_consistent_calls_reach_the_device_check():
    c, s = w("mxfp4")
    _gpu_only(q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, K))
    _gpu_only(q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, TOPK, K))
    _gpu_only(q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M * TOPK, K), x_per_slot=True)
    _gpu_only(q.qmv_dense, "mxfp4", c[0], s[0], xb(M, K))
    c2, s2 = w("cb2")
    xq, xs = x8(M, TOPK, K)
    _gpu_only(q.qmv_gather_moe, "cb2", c2, s2, ids(), xq, xs)
    _gpu_only(q.qmv_gather_moe_swiglu, "cb2", c2, s2, c2, s2, ids(), xb(M, K))
    _gpu_only(q.qmv_gather_moe_combine, "cb2", c2, s2, ids(), torch.zeros(M, TOPK), xq, xs)
    # float16 scales are accepted as well as their bytes
    c3, s3 = w("cb3")
    _gpu_only(q.qmv_gather_moe, "cb3", c3, s3.view(torch.float16), ids(), *x8(M, K))


def test_weight_sizes():
    c, s = w("mxfp4")
    _bad("w_codes", q.qmv_gather_moe, "mxfp4", c[:, :, :-16], s, ids(), xb(M, K))
    _bad("w_scales", q.qmv_gather_moe, "mxfp4", c, s[:, :, :-1], ids(), xb(M, K))
    _bad("w_scales", q.qmv_gather_moe, "mxfp4", c, s[:-1], ids(), xb(M, K))
    # K from x decides the row bytes: a wider x than the weights is refused
    _bad("w_codes", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, 2 * K))
    _bad("w_codes", q.qmv_dense, "mxfp4", c[0][:, :-1], s[0], xb(M, K))
    c2, s2 = w("cb2")
    _bad("w_scales", q.qmv_gather_moe, "cb2", c2, s2.view(torch.float16)[:, :, :-1], ids(), *x8(M, K))
    _bad("up_codes", q.qmv_gather_moe_swiglu, "cb2", c2, s2, c2[:, :-1], s2, ids(), xb(M, K))
    _bad("gate_scales", q.qmv_gather_moe_swiglu, "cb2", c2, s2[:, :, :-2], c2, s2, ids(), xb(M, K))


def test_activation_sizes():
    c, s = w("mxfp4")
    _bad("x has shape", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M - 1, K))
    # per-slot activations must hold M * top_k vectors
    _bad("x has shape", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, K), x_per_slot=True)
    # a 3-D x is per-slot: it must match [M][top_k] and not be declared broadcast
    _bad("3-D x", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, TOPK, K), x_per_slot=False)
    _bad("x has shape", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, TOPK + 1, K))
    c2, s2 = w("cb2")
    xq, xs = x8(M, K)
    _bad("x_scales", q.qmv_gather_moe, "cb2", c2, s2, ids(), xq, xs[:, :-1])
    _bad("x_scales", q.qmv_gather_moe, "cb2", c2, s2, ids(), xq, None)
    _bad("x_scales", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, K), xs)
    _bad("x_scales", q.qmv_dense, "cb2", c2[0], s2[0], xq, xs[:, :-1])
    _bad("w_codes", q.qmv_dense, "cb2", c2[0], s2[0], xq[:, :-32], xs[:, :-1])


def test_combine_defaults_to_the_shape_of_x():
    """qmv_gather_moe_combine infers per-slot activations from a 3-D x, as
    qmv_gather_moe does; broadcast [M][K] x is no longer read as per-slot."""
    c2, s2 = w("cb2")
    rw = torch.zeros(M, TOPK)
    _gpu_only(q.qmv_gather_moe_combine, "cb2", c2, s2, ids(), rw, *x8(M, K))
    _gpu_only(q.qmv_gather_moe_combine, "cb2", c2, s2, ids(), rw, *x8(M, TOPK, K))
    _bad("x has shape", q.qmv_gather_moe_combine, "cb2", c2, s2, ids(), rw, *x8(M, K), x_per_slot=True)
    _bad("route_weights", q.qmv_gather_moe_combine, "cb2", c2, s2, ids(), torch.zeros(M, TOPK + 1),
         *x8(M, K))


def test_output_sizes():
    c, s = w("mxfp4")
    _bad("y has shape", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, K), y=torch.zeros(M, N))
    _bad("y has shape", q.qmv_gather_moe, "mxfp4", c, s, ids(), xb(M, K),
         y=torch.zeros(M, TOPK, N, dtype=torch.float16))
    _bad("y has shape", q.qmv_dense, "mxfp4", c[0], s[0], xb(M, K), y=torch.zeros(M, N - 1))
    c2, s2 = w("cb2")
    _bad("y has shape", q.qmv_gather_moe_combine, "cb2", c2, s2, ids(), torch.zeros(M, TOPK),
         *x8(M, TOPK, K), y=torch.zeros(M, TOPK, N))


def test_ids_must_be_2d():
    c, s = w("mxfp4")
    _bad("expert_ids", q.qmv_gather_moe, "mxfp4", c, s, torch.zeros(M * TOPK, dtype=torch.int32),
         xb(M, K))
