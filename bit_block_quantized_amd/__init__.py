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
           "qmv_gather_moe_combine_noalloc",
           "qmv_strerror",
           "qmv_probe_stream_read", "qmv_probe_clock", "lib", "LIB_PATH",
           "W_MXFP4", "W_CB2", "W_CB3", "A_BF16", "A_Q8B32", "A_BF16_Q8", "QmvError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmv.so")

W_MXFP4, W_CB2, W_CB3 = 0, 1, 2
A_BF16, A_Q8B32, A_BF16_Q8 = 0, 1, 2
_WFMT = {"mxfp4": W_MXFP4, "cb2": W_CB2, "cb3": W_CB3}
_AFMT_OF = {W_MXFP4: A_BF16, W_CB2: A_Q8B32, W_CB3: A_Q8B32}
STATUS = {0: "QMV_OK", 1: "QMV_EINVAL", 2: "QMV_EUNSUPPORTED", 3: "QMV_EHIP", 4: "QMV_ESCRATCH"}
# bytes of the allocation-free combine's fixed temporary per GPU (include/qmv.h)
NOALLOC_SCRATCH_BYTES = 64 << 20


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
    L.qmv_gather_moe_combine_noalloc.restype = I
    L.qmv_gather_moe_combine_noalloc.argtypes = [I, P, P, I, P, P, I, I, I, P, P, I, P, I, I, P]
    L.qmv_probe_stream_read.restype = I
    L.qmv_probe_stream_read.argtypes = [I, P, P, I, P, P]
    L.qmv_probe_clock.restype = I
    L.qmv_probe_clock.argtypes = [P, P]
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


def _row_bytes(w, K):
    """(code bytes, scale bytes) of one weight row of K weights."""
    if w == W_MXFP4:
        return K // 2, K // 32
    if w == W_CB2:
        return K // 4, 2 * (K // 32)
    return 3 * K // 8, 2 * (K // 16)


def _nbytes(t):
    return t.numel() * t.element_size()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_weights(w, codes, scales, lead, K, what=("w_codes", "w_scales")):
    """codes/scales hold exactly the rows the kernel will address: leading
    dimensions ``lead`` ((E, N) or (N,)) and the row bytes of K weights."""
    rcb, rsb = _row_bytes(w, K)
    rows = 1
    for d in lead:
        rows *= d
    for t, name, per_row in ((codes, what[0], rcb), (scales, what[1], rsb)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        _need(tuple(t.shape[:len(lead)]) == tuple(lead) and _nbytes(t) == rows * per_row,
              f"{name} has shape {tuple(t.shape)} ({_nbytes(t)} bytes), expected leading "
              f"dimensions {tuple(lead)} and {per_row} bytes per row for K={K} "
              f"({rows * per_row} bytes)")


def _check_x(x, x_scales, vectors, K, a):
    """x holds ``vectors`` activation vectors of K values, and x_scales (int8
    activations) one fp16 scale per 32 of them."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    _need(x.dim() >= 1 and x.shape[-1] == K and x.numel() == vectors * K,
          f"x has shape {tuple(x.shape)}, expected {vectors} vectors of K={K}")
    if a == A_Q8B32:
        _need(isinstance(x_scales, torch.Tensor), "int8 activations need x_scales (float16, one per 32)")
        _need(x_scales.numel() == vectors * (K // 32),
              f"x_scales has shape {tuple(x_scales.shape)}, expected {vectors} x {K // 32} fp16 scales")
    else:
        _need(x_scales is None, "x_scales is only used with int8 activations")


def _check_y(y, shape):
    n = 1
    for d in shape:
        n *= d
    _need(isinstance(y, torch.Tensor) and y.numel() == n and y.dtype == torch.float32,
          f"y has shape {tuple(y.shape)} and dtype {y.dtype}, expected float32 {tuple(shape)}")


def _check_ids(expert_ids):
    if not isinstance(expert_ids, torch.Tensor):
        raise TypeError("expert_ids must be a torch.Tensor")
    _need(expert_ids.dim() == 2, f"expert_ids has shape {tuple(expert_ids.shape)}, expected [M][top_k]")
    return expert_ids.shape[0], expert_ids.shape[1]


def _per_slot(x, x_per_slot, M, top_k):
    """Per-slot activations: explicit, or [M][top_k][K] when x is 3-D."""
    if x_per_slot is None:
        return isinstance(x, torch.Tensor) and x.dim() == 3
    x_per_slot = bool(x_per_slot)
    if isinstance(x, torch.Tensor) and x.dim() == 3:
        _need(x_per_slot and tuple(x.shape[:2]) == (M, top_k),
              f"x has shape {tuple(x.shape)}: a 3-D x is [M][top_k][K] per-slot activations")
    return x_per_slot


def _gpu(dev, fn):
    if dev.type != "cuda":
        raise ValueError(f"{fn} runs on the GPU only; pass device tensors")


def qmv_dense(wfmt, w_codes, w_scales, x, x_scales=None, y=None, stream=None):
    """Dense GEMV: y[m][n] = sum_k w(n,k) x(m,k); returns y (float32 [M][N]).
    ``x`` is [M][K]."""
    w = _wfmt(wfmt)
    _need(isinstance(x, torch.Tensor) and x.dim() == 2, "x must be a 2-D tensor [M][K]")
    M, K = x.shape
    N = w_codes.shape[0]
    a, xd = _afmt(w, x)
    _check_weights(w, w_codes, w_scales, (N,), K)
    _check_x(x, x_scales, M, K, a)
    if y is not None:
        _check_y(y, (M, N))
    dev = w_codes.device
    _gpu(dev, "qmv_dense")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    s = lib().qmv_dense(w, _dev_ptr(w_codes, "w_codes", (torch.uint8,), dev),
                        _dev_ptr(w_scales, "w_scales", _SCALE_DT, dev), a,
                        _dev_ptr(x, "x", xd, dev),
                        _dev_ptr(x_scales, "x_scales", (torch.float16,), dev),
                        _dev_ptr(y, "y", (torch.float32,), dev), M, N, K, _stream(dev, stream))
    _check(s)
    return y


def qmv_gather_moe(wfmt, w_codes, w_scales, expert_ids, x, x_scales=None, x_per_slot=None,
                   y=None, stream=None):
    """Expert-gathered GEMV; returns y (float32 [M][top_k][N]).

    ``x`` is [M][K] (one vector per token), or [M][top_k][K] per (token,
    slot); ``x_per_slot`` defaults to ``x.dim() == 3``.
    """
    w = _wfmt(wfmt)
    M, top_k = _check_ids(expert_ids)
    E, N = w_codes.shape[0], w_codes.shape[1]
    K = x.shape[-1]
    per_slot = _per_slot(x, x_per_slot, M, top_k)
    a, xd = _afmt(w, x)
    _check_weights(w, w_codes, w_scales, (E, N), K)
    _check_x(x, x_scales, M * top_k if per_slot else M, K, a)
    if y is not None:
        _check_y(y, (M, top_k, N))
    dev = w_codes.device
    _gpu(dev, "qmv_gather_moe")
    if y is None:
        y = torch.empty((M, top_k, N), dtype=torch.float32, device=dev)
    s = lib().qmv_gather_moe(w, _dev_ptr(w_codes, "w_codes", (torch.uint8,), dev),
                             _dev_ptr(w_scales, "w_scales", _SCALE_DT, dev), E,
                             _dev_ptr(expert_ids, "expert_ids", (torch.int32,), dev), M, top_k, a,
                             _dev_ptr(x, "x", xd, dev),
                             _dev_ptr(x_scales, "x_scales", (torch.float16,), dev),
                             int(per_slot),
                             _dev_ptr(y, "y", (torch.float32,), dev), N, K, _stream(dev, stream))
    _check(s)
    return y


def qmv_gather_moe_swiglu(wfmt, gate_codes, gate_scales, up_codes, up_scales, expert_ids, x,
                          x_scales=None, y=None, stream=None):
    """Fused gate/up projection with SwiGLU: y = silu(gate x) * (up x);
    returns y (float32 [M][top_k][N]).  ``x`` is the tokens' [M][K]."""
    w = _wfmt(wfmt)
    M, top_k = _check_ids(expert_ids)
    E, N = gate_codes.shape[0], gate_codes.shape[1]
    K = x.shape[-1]
    a, xd = _afmt(w, x)
    _check_weights(w, gate_codes, gate_scales, (E, N), K, ("gate_codes", "gate_scales"))
    _check_weights(w, up_codes, up_scales, (E, N), K, ("up_codes", "up_scales"))
    _check_x(x, x_scales, M, K, a)
    if y is not None:
        _check_y(y, (M, top_k, N))
    dev = gate_codes.device
    _gpu(dev, "qmv_gather_moe_swiglu")
    if y is None:
        y = torch.empty((M, top_k, N), dtype=torch.float32, device=dev)
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
                           x_per_slot=None, y=None, stream=None):
    """Down projection with the router-weighted top-k combine:
    y[t][n] = sum_j route_weights[t][j] * (w(ids[t][j]) . x(t, j)); returns y
    (float32 [M][N]).  ``x`` is [M][top_k][K] per (token, slot) -- the usual
    down-projection input -- or [M][K]; ``x_per_slot`` defaults to
    ``x.dim() == 3``."""
    return _combine("qmv_gather_moe_combine", wfmt, w_codes, w_scales, expert_ids, route_weights, x,
                    x_scales, x_per_slot, y, stream)


def qmv_gather_moe_combine_noalloc(wfmt, w_codes, w_scales, expert_ids, route_weights, x, y,
                                   x_scales=None, x_per_slot=None, stream=None):
    """qmv_gather_moe_combine into the caller's y ([M][N] float32, required)
    with nothing allocated, by the library or here: a call with more than 4
    tokens keeps its temporary in the library's fixed per-GPU array of
    NOALLOC_SCRATCH_BYTES (larger ones raise QMV_ESCRATCH); calls that overlap
    on one GPU race on that array."""
    if y is None:
        raise ValueError("qmv_gather_moe_combine_noalloc needs the output y")
    return _combine("qmv_gather_moe_combine_noalloc", wfmt, w_codes, w_scales, expert_ids, route_weights,
                    x, x_scales, x_per_slot, y, stream)


def _combine(entry, wfmt, w_codes, w_scales, expert_ids, route_weights, x, x_scales, x_per_slot, y,
             stream):
    w = _wfmt(wfmt)
    M, top_k = _check_ids(expert_ids)
    E, N = w_codes.shape[0], w_codes.shape[1]
    if not isinstance(route_weights, torch.Tensor):
        raise TypeError("route_weights must be a torch.Tensor")
    _need(tuple(route_weights.shape) == (M, top_k),
          f"route_weights has shape {tuple(route_weights.shape)}, expected {(M, top_k)}")
    K = x.shape[-1]
    per_slot = _per_slot(x, x_per_slot, M, top_k)
    a, xd = _afmt(w, x)
    _check_weights(w, w_codes, w_scales, (E, N), K)
    _check_x(x, x_scales, M * top_k if per_slot else M, K, a)
    if y is not None:
        _check_y(y, (M, N))
    dev = w_codes.device
    _gpu(dev, entry)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    s = getattr(lib(), entry)(
        w, _dev_ptr(w_codes, "w_codes", (torch.uint8,), dev),
        _dev_ptr(w_scales, "w_scales", _SCALE_DT, dev), E,
        _dev_ptr(expert_ids, "expert_ids", (torch.int32,), dev),
        _dev_ptr(route_weights, "route_weights", (torch.float32,), dev), M, top_k, a,
        _dev_ptr(x, "x", xd, dev), _dev_ptr(x_scales, "x_scales", (torch.float16,), dev),
        int(per_slot), _dev_ptr(y, "y", (torch.float32,), dev), N, K,
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


def qmv_probe_clock(out, stream=None):
    """Store the GPU's 100 MHz real-time counter into ``out`` (a 1-element
    int64 device tensor) from a one-thread kernel on ``stream``
    (include/qmv_probe.h)."""
    dev = out.device
    _check(lib().qmv_probe_clock(_dev_ptr(out, "out", (torch.int64,), dev), _stream(dev, stream)))
