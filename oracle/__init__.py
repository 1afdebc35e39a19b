"""CPU oracle for the block-quantized expert-gather GEMV (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``bit_block_quantized_amd``) never
does, and the oracle never imports the product: the two share no code.

The arithmetic lives in ``qmv_oracle.c`` (plain C, fp64, a literal
dequantize-then-dot); this module only compiles it with gcc and marshals
numpy arrays into it through ctypes.  ctypes releases the GIL during the
foreign call, so Python threads running disjoint output selections execute
in parallel.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

W_MXFP4, W_CB2, W_CB3 = 0, 1, 2
A_BF16, A_Q8 = 0, 1
WFMT = {"mxfp4": W_MXFP4, "cb2": W_CB2, "cb3": W_CB3}
AFMT = {"bf16": A_BF16, "q8": A_Q8}


def build(out: str = _LIB, mutant: int = 0) -> str:
    """Compile the oracle with gcc -O2 (no SIMD intrinsics) into ``out``."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fno-fast-math",
           f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_L = ctypes.c_long
_I = ctypes.c_int
_D = ctypes.c_double


def _bind(lib):
    lib.oracle_e2m1.restype = _D
    lib.oracle_e2m1.argtypes = [_I]
    lib.oracle_e8m0.restype = _D
    lib.oracle_e8m0.argtypes = [_I]
    lib.oracle_h2d.restype = _D
    lib.oracle_h2d.argtypes = [ctypes.c_uint]
    lib.oracle_bf16.restype = _D
    lib.oracle_bf16.argtypes = [ctypes.c_uint]
    lib.oracle_cb2_value.restype = _D
    lib.oracle_cb2_value.argtypes = [_I]
    lib.oracle_cb3_value.restype = _D
    lib.oracle_cb3_value.argtypes = [_I]
    lib.oracle_code_value.restype = _D
    lib.oracle_code_value.argtypes = [_I, _I]
    lib.oracle_row_code_bytes.restype = _L
    lib.oracle_row_code_bytes.argtypes = [_I, _L]
    lib.oracle_row_scale_bytes.restype = _L
    lib.oracle_row_scale_bytes.argtypes = [_I, _L]
    lib.oracle_code.restype = _I
    lib.oracle_code.argtypes = [_I, _P, _L]
    lib.oracle_dequant_row.restype = None
    lib.oracle_dequant_row.argtypes = [_I, _P, _P, _L, _P]
    lib.oracle_block_sums.restype = _L
    lib.oracle_block_sums.argtypes = [_I, _P, _P, _L, _P]
    lib.oracle_qmv_gather_sel.restype = _I
    lib.oracle_qmv_gather_sel.argtypes = [_I, _P, _P, _L, _P, _L, _L, _I, _P, _P, _I,
                                          _L, _L, _P, _L, _P, _P]
    lib.oracle_qmv_gather.restype = _I
    lib.oracle_qmv_gather.argtypes = [_I, _P, _P, _L, _P, _L, _L, _I, _P, _P, _I,
                                      _L, _L, _P, _P]
    lib.oracle_qmv_dense.restype = _I
    lib.oracle_qmv_dense.argtypes = [_I, _P, _P, _I, _P, _P, _L, _L, _L, _P, _P]
    lib.oracle_qmv_gather_swiglu_sel.restype = _I
    lib.oracle_qmv_gather_swiglu_sel.argtypes = [_I, _P, _P, _P, _P, _L, _P, _L, _L, _I, _P, _P,
                                                 _L, _L, _P, _L, _P, _P, _P, _P, _P]
    lib.oracle_qmv_combine_sel.restype = _I
    lib.oracle_qmv_combine_sel.argtypes = [_I, _P, _P, _L, _P, _P, _L, _L, _I, _P, _P, _I,
                                           _L, _L, _P, _L, _P, _P]
    lib.oracle_f2h.restype = ctypes.c_uint
    lib.oracle_f2h.argtypes = [ctypes.c_float]
    lib.oracle_quantize_q8.restype = _I
    lib.oracle_quantize_q8.argtypes = [_P, _L, _L, _P, _P]
    lib.oracle_mutant_id.restype = _I
    lib.oracle_mutant_id.argtypes = []
    return lib


_cache: dict = {}


def load(mutant: int = 0):
    """Return an ``Oracle`` over the default build (or a freshly built mutant)."""
    if mutant in _cache:
        return _cache[mutant]
    if mutant == 0:
        if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(_LIB)
        path = _LIB
    else:
        d = tempfile.mkdtemp(prefix="oracle_mutant_")
        path = build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant)
    o = Oracle(_bind(ctypes.CDLL(path)))
    assert o.lib.oracle_mutant_id() == mutant
    _cache[mutant] = o
    return o


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """numpy-facing wrapper over the C oracle.

    Layouts (all C-contiguous): codes uint8[E][N][row_code_bytes],
    scales uint8[E][N][row_scale_bytes] (fp16 scales as little-endian byte
    pairs), ids int32[M][top_k], x uint16 bf16 bits [V][K] or int8 [V][K],
    xs uint16 fp16 bits [V][K/32].
    """

    def __init__(self, lib):
        self.lib = lib

    # scalar decoders -------------------------------------------------
    def e2m1(self, c):
        return self.lib.oracle_e2m1(int(c))

    def e8m0(self, s):
        return self.lib.oracle_e8m0(int(s))

    def h2d(self, h):
        return self.lib.oracle_h2d(int(h))

    def bf16(self, b):
        return self.lib.oracle_bf16(int(b))

    def code_value(self, wfmt, c):
        return self.lib.oracle_code_value(WFMT.get(wfmt, wfmt), int(c))

    def row_code_bytes(self, wfmt, K):
        return self.lib.oracle_row_code_bytes(WFMT.get(wfmt, wfmt), K)

    def row_scale_bytes(self, wfmt, K):
        return self.lib.oracle_row_scale_bytes(WFMT.get(wfmt, wfmt), K)

    def code(self, wfmt, row, k):
        row = _c(row, np.uint8)
        return self.lib.oracle_code(WFMT.get(wfmt, wfmt), _ptr(row), int(k))

    def dequant_row(self, wfmt, crow, srow, K):
        crow, srow = _c(crow, np.uint8), _c(srow, np.uint8)
        w = np.empty(K, np.float64)
        self.lib.oracle_dequant_row(WFMT.get(wfmt, wfmt), _ptr(crow), _ptr(srow), K, _ptr(w))
        return w

    def block_sums(self, wfmt, crow, q, K):
        crow, q = _c(crow, np.uint8), _c(q, np.int8)
        bs = 32 if WFMT.get(wfmt, wfmt) == W_CB2 else 16
        S = np.empty(K // bs, np.int64)
        n = self.lib.oracle_block_sums(WFMT.get(wfmt, wfmt), _ptr(crow), _ptr(q), K, _ptr(S))
        assert n == K // bs
        return S

    # GEMV --------------------------------------------------------------
    @staticmethod
    def _xarr(afmt, x):
        return _c(x, np.uint16 if AFMT.get(afmt, afmt) == A_BF16 else np.int8)

    def gather(self, wfmt, codes, scales, ids, afmt, x, xs=None, x_per_slot=False, outs=None):
        """Gather GEMV; returns (y, A) in fp64.

        Without ``outs`` y and A have shape [M][top_k][N]; with ``outs`` (flat
        output indices) they are 1-D over the selection.
        """
        codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
        ids = _c(ids, np.int32)
        E, N = codes.shape[0], codes.shape[1]
        M, top_k = ids.shape
        x = self._xarr(afmt, x)
        K = x.shape[-1]
        xs = _c(xs, np.uint16)
        w, a = WFMT.get(wfmt, wfmt), AFMT.get(afmt, afmt)
        if outs is None:
            y = np.empty((M, top_k, N), np.float64)
            A = np.empty_like(y)
            rc = self.lib.oracle_qmv_gather(w, _ptr(codes), _ptr(scales), E, _ptr(ids), M, top_k,
                                            a, _ptr(x), _ptr(xs), int(bool(x_per_slot)), N, K,
                                            _ptr(y), _ptr(A))
        else:
            outs = _c(outs, np.int64)
            y = np.empty(outs.shape[0], np.float64)
            A = np.empty_like(y)
            rc = self.lib.oracle_qmv_gather_sel(w, _ptr(codes), _ptr(scales), E, _ptr(ids), M,
                                                top_k, a, _ptr(x), _ptr(xs),
                                                int(bool(x_per_slot)), N, K, _ptr(outs),
                                                outs.shape[0], _ptr(y), _ptr(A))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, A

    def gather_swiglu(self, wfmt, gcodes, gscales, ucodes, uscales, ids, afmt, x, xs=None,
                      outs=None):
        """Fused gate/up + SwiGLU; returns (y, g, u, Ag, Au) in fp64, shaped
        [M][top_k][N] (or flat over ``outs``)."""
        gcodes, gscales = _c(gcodes, np.uint8), _c(gscales, np.uint8)
        ucodes, uscales = _c(ucodes, np.uint8), _c(uscales, np.uint8)
        ids = _c(ids, np.int32)
        E, N = gcodes.shape[0], gcodes.shape[1]
        M, top_k = ids.shape
        x = self._xarr(afmt, x)
        K = x.shape[-1]
        xs = _c(xs, np.uint16)
        shape = (M, top_k, N)
        sel = np.arange(M * top_k * N, dtype=np.int64) if outs is None else _c(outs, np.int64)
        res = [np.empty(sel.shape[0], np.float64) for _ in range(5)]
        rc = self.lib.oracle_qmv_gather_swiglu_sel(
            WFMT.get(wfmt, wfmt), _ptr(gcodes), _ptr(gscales), _ptr(ucodes), _ptr(uscales), E,
            _ptr(ids), M, top_k, AFMT.get(afmt, afmt), _ptr(x), _ptr(xs), N, K, _ptr(sel),
            sel.shape[0], *[_ptr(r) for r in res])
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        if outs is None:
            res = [r.reshape(shape) for r in res]
        return tuple(res)

    def combine(self, wfmt, codes, scales, ids, weights, afmt, x, xs=None, x_per_slot=True,
                outs=None):
        """Down projection with the router-weighted combine; returns (y, A) in
        fp64 shaped [M][N] (or flat over ``outs``, indices t * N + n)."""
        codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
        ids = _c(ids, np.int32)
        weights = _c(weights, np.float32)
        E, N = codes.shape[0], codes.shape[1]
        M, top_k = ids.shape
        assert weights.shape == ids.shape
        x = self._xarr(afmt, x)
        K = x.shape[-1]
        xs = _c(xs, np.uint16)
        sel = np.arange(M * N, dtype=np.int64) if outs is None else _c(outs, np.int64)
        y = np.empty(sel.shape[0], np.float64)
        A = np.empty_like(y)
        rc = self.lib.oracle_qmv_combine_sel(
            WFMT.get(wfmt, wfmt), _ptr(codes), _ptr(scales), E, _ptr(ids), _ptr(weights), M,
            top_k, AFMT.get(afmt, afmt), _ptr(x), _ptr(xs), int(bool(x_per_slot)), N, K,
            _ptr(sel), sel.shape[0], _ptr(y), _ptr(A))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        if outs is None:
            return y.reshape(M, N), A.reshape(M, N)
        return y, A

    def quantize_q8(self, x_bf16_bits):
        """bf16 activations (uint16 bit patterns [V][K]) -> (int8 q [V][K],
        fp16 scale bits uint16 [V][K/32]) by the oracle's q8 quantizer."""
        x = _c(x_bf16_bits, np.uint16)
        squeeze = x.ndim == 1
        if squeeze:
            x = x[None]
        V, K = x.shape
        q = np.empty((V, K), np.int8)
        d = np.empty((V, K // 32), np.uint16)
        if self.lib.oracle_quantize_q8(_ptr(x), V, K, _ptr(q), _ptr(d)) != 0:
            raise ValueError("K must be a multiple of 32")
        return (q[0], d[0]) if squeeze else (q, d)

    def dense(self, wfmt, codes, scales, afmt, x, xs=None):
        """Dense GEMV; codes [N][row_code_bytes]; returns (y, A) shaped [M][N]."""
        codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
        N = codes.shape[0]
        x = self._xarr(afmt, x)
        M, K = x.shape
        xs = _c(xs, np.uint16)
        y = np.empty((M, N), np.float64)
        A = np.empty_like(y)
        rc = self.lib.oracle_qmv_dense(WFMT.get(wfmt, wfmt), _ptr(codes), _ptr(scales),
                                       AFMT.get(afmt, afmt), _ptr(x), _ptr(xs), M, N, K,
                                       _ptr(y), _ptr(A))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, A
