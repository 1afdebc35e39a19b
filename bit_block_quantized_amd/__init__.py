"""Python binding of libqmv.so: block-quantized GEMV for MoE expert
projections on AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the GEMV runs in the HIP kernels of
``libqmv.so``; PyTorch supplies device memory and the current stream.  There
is no CPU fallback: without the built library every call raises.

    import torch, bit_block_quantized_amd as qmv
    y = qmv.qmv_gather_moe("mxfp4", codes, scales, ids, x)          # [M][top_k][N]
    y = qmv.qmv_dense("cb2", codes, scales, x, x_scales)            # [M][N]

Layouts (C-contiguous device tensors, see include/qmv.h):
    codes   uint8 [E][N][row_code_bytes]  (dense: [N][row_code_bytes])
    scales  uint8 [E][N][row_scale_bytes] (fp16 scales may be passed as
            float16 [E][N][K/32 or K/16] as well)
    ids     int32 [M][top_k]
    x       bfloat16 [M][K] / int8 [M][K]; per-slot: [M][top_k][K]
    x_scales float16 [...][K/32] for int8 activations
bf16 activations with 2-bit or 3-bit weights (x_scales None) are quantized
to int8 per 32 inside the kernel (QMV_A_BF16_Q8); MXFP4 weights take bf16
activations or int8 activations with their scales (QMV_A_Q8B32).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  -- loads the HIP runtime that libqmv.so binds to

__all__ = ["qmv_dense", "qmv_gather_moe", "qmv_gather_moe_swiglu", "qmv_gather_moe_combine",
           "qmv_strerror",
           "qmv_probe_stream_read", "lib", "LIB_PATH",
           "W_MXFP4", "W_CB2", "W_CB3", "A_BF16", "A_Q8B32", "A_BF16_Q8", "QmvError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmv.so")

W_MXFP4, W_CB2, W_CB3 = 0, 1, 2
A_BF16, A_Q8B32, A_BF16_Q8 = 0, 1, 2
_WFMT = {"mxfp4": W_MXFP4, "cb2": W_CB2, "cb3": W_CB3}
_AFMT_OF = {W_MXFP4: A_BF16, W_CB2: A_Q8B32, W_CB3: A_Q8B32}
STATUS = {0: "QMV_OK", 1: "QMV_EINVAL", 2: "QMV_EUNSUPPORTED", 3: "QMV_EHIP"}


class QmvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "or python -m bit_block_quantized_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.qmv_dense.restype = I
    L.qmv_dense.argtypes = [I, P, P, I, P, P, P, I, I, I, P]
    L.qmv_gather_moe.restype = I
    L.qmv_gather_moe.argtypes = [I, P, P, I, P, I, I, I, P, P, I, P, I, I, P]
    L.qmv_gather_moe_swiglu.restype = I
    L.qmv_gather_moe_swiglu.argtypes = [I, P, P, P, P, I, P, I, I, I, P, P, P, I, I, P]
    L.qmv_gather_moe_combine.restype = I
    L.qmv_gather_moe_combine.argtypes = [I, P, P, I, P, P, I, I, I, P, P, I, P, I, I, P]
    L.qmv_probe_stream_read.restype = I
    L.qmv_probe_stream_read.argtypes = [I, P, P, I, P, P]
    L.qmv_strerror.restype = ctypes.c_char_p
    L.qmv_strerror.argtypes = [I]
    _lib = L
    return L


def qmv_strerror(status: int) -> str:
    return lib().qmv_strerror(int(status)).decode()


def _wfmt(w):
    return _WFMT[w] if isinstance(w, str) else int(w)


def _dev_ptr(t, name, dtypes, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status):
    if status != 0:
        raise QmvError(status, qmv_strerror(status))


_SCALE_DT = (torch.uint8, torch.float16)


def _afmt(w, x):
    """Activation format from the weight format and x's dtype: MXFP4 takes
    bf16 or int8 (+ scales); 2-/3-bit weights take int8 (+ scales) or bf16
    (quantized in-kernel)."""
    is_bf16 = isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16
    if w == W_MXFP4:
        return (A_BF16, (torch.bfloat16,)) if is_bf16 else (A_Q8B32, (torch.int8,))
    if is_bf16:
        return A_BF16_Q8, (torch.bfloat16,)
    return A_Q8B32, (torch.int8,)


def qmv_dense(wfmt, w_codes, w_scales, x, x_scales=None, y=None, stream=None):
    """Dense GEMV: y[m][n] = sum_k w(n,k) x(m,k); returns y (float32 [M][N])."""
    w = _wfmt(wfmt)
    dev = w_codes.device
    if dev.type != "cuda":
        raise ValueError("qmv_dense runs on the GPU only; pass device tensors")
    M, K = x.shape
    N = w_codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    a, xd = _afmt(w, x)
    s = lib().qmv_dense(w, _dev_ptr(w_codes, "w_codes", (torch.uint8,), dev),
                        _dev_ptr(w_scales, "w_scales", _SCALE_DT, dev), a,
                        _dev_ptr(x, "x", xd, dev),
                        _dev_ptr(x_scales, "x_scales", (torch.float16,), dev),
                        _dev_ptr(y, "y", (torch.float32,), dev), M, N, K, _stream(dev, stream))
    _check(s)
    return y


def qmv_gather_moe(wfmt, w_codes, w_scales, expert_ids, x, x_scales=None, x_per_slot=False,
                   y=None, stream=None):
    """Expert-gathered GEMV; returns y (float32 [M][top_k][N]).

    ``x`` is [M][K], or [M][top_k][K] with ``x_per_slot=True``.
    """
    w = _wfmt(wfmt)
    dev = w_codes.device
    if dev.type != "cuda":
        raise ValueError("qmv_gather_moe runs on the GPU only; pass device tensors")
    E, N = w_codes.shape[0], w_codes.shape[1]
    M, top_k = expert_ids.shape
    K = x.shape[-1]
    if y is None:
        y = torch.empty((M, top_k, N), dtype=torch.float32, device=dev)
    a, xd = _afmt(w, x)
    s = lib().qmv_gather_moe(w, _dev_ptr(w_codes, "w_codes", (torch.uint8,), dev),
                             _dev_ptr(w_scales, "w_scales", _SCALE_DT, dev), E,
                             _dev_ptr(expert_ids, "expert_ids", (torch.int32,), dev), M, top_k, a,
                             _dev_ptr(x, "x", xd, dev),
                             _dev_ptr(x_scales, "x_scales", (torch.float16,), dev),
                             int(bool(x_per_slot)),
                             _dev_ptr(y, "y", (torch.float32,), dev), N, K, _stream(dev, stream))
    _check(s)
    return y


def qmv_gather_moe_swiglu(wfmt, gate_codes, gate_scales, up_codes, up_scales, expert_ids, x,
                          x_scales=None, y=None, stream=None):
    """Fused gate/up projection with SwiGLU: y = silu(gate x) * (up x);
    returns y (float32 [M][top_k][N]).  ``x`` is the tokens' [M][K]."""
    w = _wfmt(wfmt)
    dev = gate_codes.device
    if dev.type != "cuda":
        raise ValueError("qmv_gather_moe_swiglu runs on the GPU only; pass device tensors")
    E, N = gate_codes.shape[0], gate_codes.shape[1]
    M, top_k = expert_ids.shape
    K = x.shape[-1]
    if y is None:
        y = torch.empty((M, top_k, N), dtype=torch.float32, device=dev)
    a, xd = _afmt(w, x)
    s = lib().qmv_gather_moe_swiglu(
        w, _dev_ptr(gate_codes, "gate_codes", (torch.uint8,), dev),
        _dev_ptr(gate_scales, "gate_scales", _SCALE_DT, dev),
        _dev_ptr(up_codes, "up_codes", (torch.uint8,), dev),
        _dev_ptr(up_scales, "up_scales", _SCALE_DT, dev), E,
        _dev_ptr(expert_ids, "expert_ids", (torch.int32,), dev), M, top_k, a,
        _dev_ptr(x, "x", xd, dev), _dev_ptr(x_scales, "x_scales", (torch.float16,), dev),
        _dev_ptr(y, "y", (torch.float32,), dev), N, K, _stream(dev, stream))
    _check(s)
    return y


def qmv_gather_moe_combine(wfmt, w_codes, w_scales, expert_ids, route_weights, x, x_scales=None,
                           x_per_slot=True, y=None, stream=None):
    """Down projection with the router-weighted top-k combine:
    y[t][n] = sum_j route_weights[t][j] * (w(ids[t][j]) . x(t, j)); returns y
    (float32 [M][N]).  ``x`` is [M][top_k][K] (``x_per_slot=True``) or [M][K]."""
    w = _wfmt(wfmt)
    dev = w_codes.device
    if dev.type != "cuda":
        raise ValueError("qmv_gather_moe_combine runs on the GPU only; pass device tensors")
    E, N = w_codes.shape[0], w_codes.shape[1]
    M, top_k = expert_ids.shape
    if tuple(route_weights.shape) != (M, top_k):
        raise ValueError(f"route_weights has shape {tuple(route_weights.shape)}, expected {(M, top_k)}")
    K = x.shape[-1]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    a, xd = _afmt(w, x)
    s = lib().qmv_gather_moe_combine(
        w, _dev_ptr(w_codes, "w_codes", (torch.uint8,), dev),
        _dev_ptr(w_scales, "w_scales", _SCALE_DT, dev), E,
        _dev_ptr(expert_ids, "expert_ids", (torch.int32,), dev),
        _dev_ptr(route_weights, "route_weights", (torch.float32,), dev), M, top_k, a,
        _dev_ptr(x, "x", xd, dev), _dev_ptr(x_scales, "x_scales", (torch.float16,), dev),
        int(bool(x_per_slot)), _dev_ptr(y, "y", (torch.float32,), dev), N, K,
        _stream(dev, stream))
    _check(s)
    return y


PROBE_VARIANTS = 6


def qmv_probe_stream_read(regions, variant, sink, stream=None):
    """Read-only streaming probe (include/qmv_probe.h): ``regions`` is a list
    of (device address, bytes); ``sink`` a 1-element int32 device tensor."""
    n = len(regions)
    ptrs = (ctypes.c_void_p * n)(*[int(p) for p, _ in regions])
    sizes = (ctypes.c_longlong * n)(*[int(b) for _, b in regions])
    dev = sink.device
    _check(lib().qmv_probe_stream_read(n, ptrs, sizes, int(variant),
                                       _dev_ptr(sink, "sink", (torch.int32,), dev),
                                       _stream(dev, stream)))
