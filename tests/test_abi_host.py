"""The C-ABI library on the host (no GPU needed).

Checks that libqmv.so loads, exports every function include/qmv.h declares,
and that the host-side validation returns the documented status before any
launch.  Pointers passed here are fake but aligned: validation must not
dereference them (no compute call is made without a GPU).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, EINVAL, EUNSUP = 0, 1, 2
FAKE = 0x10000          # 64 KiB-aligned, never dereferenced
W_MXFP4, W_CB2, W_CB3 = 0, 1, 2
A_BF16, A_Q8 = 0, 1


@pytest.fixture(scope="module")
def L():
    import bit_block_quantized_amd as q
    return q.lib()


def declared_functions(header=None):
    """qmv_* functions declared in one header, or in every include/*.h."""
    inc = os.path.join(ROOT, "include")
    names = [header] if header else sorted(f for f in os.listdir(inc) if f.endswith(".h"))
    found = set()
    for h in names:
        with open(os.path.join(inc, h)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        found |= set(re.findall(r"\b(qmv_[a-z_]+)\s*\(", src))
    return sorted(found)


def test_header_declares_the_boundary():
    assert declared_functions("qmv.h") == ["qmv_dense", "qmv_gather_moe",
                                           "qmv_gather_moe_combine",
                                           "qmv_gather_moe_combine_noalloc",
                                           "qmv_gather_moe_swiglu", "qmv_strerror"]
    assert declared_functions("qmv_probe.h") == ["qmv_probe_clock", "qmv_probe_stream_read"]


def test_library_exports_every_declared_symbol(L):
    declared = declared_functions()
    assert len(declared) == 8
    for name in declared:
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {ROOT}/bit_block_quantized_amd/libqmv.so").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", out), name
    # nothing but the declared entry points is exported as a function
    exported = set(re.findall(r"\bT (\S+)", out))
    assert exported == set(declared), sorted(exported - set(declared))


def test_strerror_covers_every_status(L):
    for s in range(5):
        txt = L.qmv_strerror(s).decode()
        assert txt and "unknown" not in txt
    assert L.qmv_strerror(99).decode() == "unknown status"


def dense(L, wfmt=W_MXFP4, codes=FAKE, scales=FAKE, afmt=A_BF16, x=FAKE, xs=None, y=FAKE,
          M=1, N=256, K=256):
    return L.qmv_dense(wfmt, codes, scales, afmt, x, xs, y, M, N, K, None)


def gather(L, wfmt=W_MXFP4, codes=FAKE, scales=FAKE, E=32, ids=FAKE, M=1, top_k=4, afmt=A_BF16,
           x=FAKE, xs=None, per_slot=0, y=FAKE, N=2880, K=2880):
    return L.qmv_gather_moe(wfmt, codes, scales, E, ids, M, top_k, afmt, x, xs, per_slot, y, N, K,
                            None)


DENSE_CASES = [
    (dict(codes=None), EINVAL), (dict(scales=None), EINVAL), (dict(x=None), EINVAL),
    (dict(y=None), EINVAL), (dict(M=0), EINVAL), (dict(N=0), EINVAL), (dict(K=0), EINVAL),
    (dict(N=-5), EINVAL), (dict(K=48), EUNSUP), (dict(K=16416), EUNSUP),
    # more than 4 vectors: every format pair, at most 8192 of them
    (dict(M=8193), EUNSUP), (dict(M=8193, afmt=A_Q8, xs=FAKE), EUNSUP),
    (dict(M=9000, wfmt=W_CB2, afmt=A_Q8, xs=FAKE), EUNSUP),
    (dict(M=5, wfmt=W_CB2, afmt=A_Q8, xs=None), EINVAL),
    (dict(afmt=A_Q8, xs=None), EINVAL), (dict(afmt=A_Q8, xs=FAKE + 2), EINVAL),
    (dict(wfmt=W_CB2), EUNSUP), (dict(wfmt=7), EUNSUP),
    (dict(afmt=3), EUNSUP), (dict(afmt=2), EUNSUP), (dict(codes=FAKE + 8), EINVAL),
    (dict(x=FAKE + 2), EINVAL), (dict(wfmt=W_CB2, afmt=2, x=FAKE + 8), EINVAL),
    (dict(wfmt=W_CB3, afmt=2, x=FAKE, codes=FAKE + 2), EINVAL),
    (dict(y=FAKE + 2), EINVAL),
]


@pytest.mark.parametrize("kw,want", DENSE_CASES)
def test_dense_validation(L, kw, want):
    assert dense(L, **kw) == want


GATHER_CASES = [
    (dict(ids=None), EINVAL), (dict(E=0), EINVAL), (dict(top_k=0), EINVAL),
    (dict(top_k=17), EUNSUP), (dict(K=2880 + 16), EUNSUP),
    # more than 4 vectors: every format pair, at most 8192 (token, slot) pairs and 1023 experts
    (dict(M=2049), EUNSUP), (dict(M=5, E=1024), EUNSUP), (dict(M=2049, afmt=A_Q8, xs=FAKE), EUNSUP),
    (dict(M=5, wfmt=W_CB3, afmt=A_Q8, xs=FAKE, E=1024), EUNSUP),
    (dict(M=5, wfmt=W_CB3, afmt=A_Q8, xs=FAKE, codes=FAKE + 2), EINVAL),
    (dict(wfmt=W_CB2, afmt=A_Q8, xs=None), EINVAL),
    (dict(wfmt=W_CB3, afmt=A_BF16), EUNSUP),
    (dict(wfmt=W_CB2, afmt=A_Q8, xs=FAKE, scales=FAKE + 2), EINVAL),
    (dict(wfmt=W_CB3, afmt=A_Q8, xs=FAKE + 2), EINVAL),
    (dict(wfmt=W_CB3, afmt=A_Q8, xs=FAKE, codes=FAKE + 2), EINVAL),
    (dict(ids=FAKE + 1), EINVAL),
    (dict(E=2 ** 31 - 1, N=2 ** 31 - 1, K=16384), EUNSUP),
    (dict(wfmt=W_CB2, afmt=A_Q8, xs=FAKE, codes=FAKE + 4, K=96), EINVAL),
]


@pytest.mark.parametrize("kw,want", GATHER_CASES)
def test_gather_validation(L, kw, want):
    assert gather(L, **kw) == want


def test_cb2_small_k_needs_only_8_byte_codes(L):
    # K % 64 == 32 takes 8-byte units, so 8-byte aligned codes pass validation
    # (the call then needs a GPU, so only the rejection of 4-byte alignment is
    # checked here)
    assert gather(L, wfmt=W_CB2, afmt=A_Q8, xs=FAKE, codes=FAKE + 4, K=96) == EINVAL


def test_binding_rejects_host_tensors():
    import torch
    import bit_block_quantized_amd as q
    codes = torch.zeros(8, 16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        q.qmv_dense("mxfp4", codes, torch.zeros(8, 1, dtype=torch.uint8),
                    torch.zeros(1, 32, dtype=torch.bfloat16))


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "bit_block_quantized_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                with open(os.path.join(dirpath, f)) as fh:
                    src = fh.read()
                assert "oracle" not in src.replace("oracle-", ""), os.path.join(dirpath, f)


def swiglu(L, wfmt=W_MXFP4, gc=FAKE, gs=FAKE, uc=FAKE, us=FAKE, E=32, ids=FAKE, M=1, top_k=4,
           afmt=A_BF16, x=FAKE, xs=None, y=FAKE, N=2880, K=2880):
    return L.qmv_gather_moe_swiglu(wfmt, gc, gs, uc, us, E, ids, M, top_k, afmt, x, xs, y, N, K,
                                   None)


SWIGLU_CASES = [
    (dict(uc=None), EINVAL), (dict(us=None), EINVAL), (dict(gc=None), EINVAL),
    (dict(uc=FAKE + 8), EINVAL), (dict(ids=None), EINVAL),
    # more than 4 tokens: every format pair, at most 8192 pairs and 1023 experts
    (dict(M=5, wfmt=W_CB2, afmt=A_Q8, xs=FAKE, E=1024), EUNSUP), (dict(M=5, E=1024), EUNSUP),
    (dict(M=2049), EUNSUP), (dict(M=2049, afmt=A_Q8, xs=FAKE), EUNSUP),
    (dict(K=100), EUNSUP), (dict(wfmt=W_CB2), EUNSUP),
    (dict(wfmt=W_CB3, afmt=A_Q8, xs=FAKE, us=FAKE + 2), EINVAL),
]


@pytest.mark.parametrize("kw,want", SWIGLU_CASES)
def test_swiglu_validation(L, kw, want):
    assert swiglu(L, **kw) == want


def combine(L, wfmt=W_CB3, codes=FAKE, scales=FAKE, E=256, ids=FAKE, rw=FAKE, M=1, top_k=4,
            afmt=A_Q8, x=FAKE, xs=FAKE, per_slot=1, y=FAKE, N=7168, K=2048):
    return L.qmv_gather_moe_combine(wfmt, codes, scales, E, ids, rw, M, top_k, afmt, x, xs,
                                    per_slot, y, N, K, None)


COMBINE_CASES = [
    (dict(rw=None), EINVAL), (dict(rw=FAKE + 2), EINVAL), (dict(ids=None), EINVAL),
    (dict(codes=None), EINVAL), (dict(y=FAKE + 1), EINVAL), (dict(xs=None), EINVAL),
    (dict(M=2049), EUNSUP), (dict(M=5, E=1024), EUNSUP), (dict(top_k=17), EUNSUP),
    (dict(top_k=0), EINVAL),
    (dict(K=2048 + 16), EUNSUP), (dict(afmt=A_BF16, xs=None), EUNSUP),
    (dict(wfmt=W_MXFP4, afmt=2, xs=None), EUNSUP), (dict(E=0), EINVAL),
]


@pytest.mark.parametrize("kw,want", COMBINE_CASES)
def test_combine_validation(L, kw, want):
    assert combine(L, **kw) == want


def combine_noalloc(L, wfmt=W_CB3, codes=FAKE, scales=FAKE, E=256, ids=FAKE, rw=FAKE, M=1, top_k=4,
                    afmt=A_Q8, x=FAKE, xs=FAKE, per_slot=1, y=FAKE, N=7168, K=2048):
    return L.qmv_gather_moe_combine_noalloc(wfmt, codes, scales, E, ids, rw, M, top_k, afmt, x, xs,
                                            per_slot, y, N, K, None)


@pytest.mark.parametrize("kw,want", COMBINE_CASES + [
    # more than 4 tokens whose temporary (M * top_k * N * 4 bytes) exceeds the
    # fixed 64 MiB: refused after the argument checks, before any HIP call
    (dict(M=512, top_k=8, N=4097, E=1, K=32), 4),
    (dict(M=2048, top_k=4, N=2049, E=1, K=32), 4),
    (dict(M=2048, top_k=4, N=2049, E=1, K=32, rw=None), EINVAL),
    (dict(M=2048, top_k=5, N=2049, E=1, K=32), EUNSUP),
])
def test_combine_noalloc_validation(L, kw, want):
    """The allocation-free combine makes the allocating entry's checks, then
    the size check of its fixed temporary, all on the host."""
    assert combine_noalloc(L, **kw) == want


def probe(L, n=1, ptrs=(FAKE,), sizes=(4096,), variant=0, sink=FAKE):
    P = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    B = (ctypes.c_longlong * max(1, len(sizes)))(*sizes)
    return L.qmv_probe_stream_read(n, P, B, variant, sink, None)


@pytest.mark.parametrize("kw,want", [
    (dict(n=0), EUNSUP), (dict(n=65), EUNSUP), (dict(variant=6), EUNSUP),
    (dict(variant=-1), EUNSUP), (dict(ptrs=(FAKE + 8,)), EINVAL), (dict(ptrs=(0,)), EINVAL),
    (dict(sizes=(0,)), EINVAL), (dict(sizes=(2 ** 31,)), EINVAL), (dict(sink=None), EINVAL),
    (dict(sink=FAKE + 2), EINVAL),
])
def test_probe_validation(L, kw, want):
    assert probe(L, **kw) == want
