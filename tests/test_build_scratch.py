"""The build refuses kernels that use scratch memory (no GPU needed).

Kernels that count their outstanding loads by hand (s_waitcnt vmcnt(N)) rely
on every vector-memory operation of a step being one the code issued; a
register spill would add scratch traffic to that count.  build.py reads the
compiler's per-kernel resource remarks and fails on any scratch use.  Here a
kernel that indexes a large private array at run time (so the compiler must
place it in scratch) is caught, a plain kernel passes, and the library's own
batched kernel compiles with no scratch.
"""
import os
import subprocess

import pytest

from bit_block_quantized_amd import build as b

SPILL = r"""
#include <hip/hip_runtime.h>
__global__ void uses_scratch(int *o, int i)
{
    int a[512];
    for (int k = 0; k < 512; ++k) a[k] = o[k * 7 % 511];
    o[threadIdx.x] = a[(i + threadIdx.x) & 511];
}
__global__ void no_scratch(int *o, int i) { o[threadIdx.x] = i + (int)threadIdx.x; }
"""


def _remarks(tmp_path, src, name="k.hip"):
    p = tmp_path / name
    p.write_text(src)
    r = subprocess.run([b.HIPCC, *b.FLAGS, b.RESOURCE_REMARKS, "-I", os.path.join(b.ROOT, "include"),
                        "-I", b.CSRC, "-c", str(p), "-o", str(tmp_path / "k.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return b.parse_resource_usage(r.stderr)


def test_scratch_kernel_is_flagged(tmp_path):
    k = _remarks(tmp_path, SPILL)
    names = {n: r for n, r in k.items()}
    spill = [n for n in names if "uses_scratch" in n]
    clean = [n for n in names if "no_scratch" in n]
    assert spill and clean, names
    bad = [n for n, _ in b.scratch_violations(k)]
    assert spill[0] in bad and clean[0] not in bad


def test_batched_kernels_use_no_scratch(tmp_path):
    src = os.path.join(b.CSRC, "qmv_k_mxfp4b.hip")
    r = subprocess.run([b.HIPCC, *b.FLAGS, b.RESOURCE_REMARKS, "-I", os.path.join(b.ROOT, "include"),
                        "-I", b.CSRC, "-c", src, "-o", str(tmp_path / "b.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    k = b.parse_resource_usage(r.stderr)
    batched = [n for n in k if "batched" in n]
    assert batched, sorted(k)
    assert b.scratch_violations(k) == []
