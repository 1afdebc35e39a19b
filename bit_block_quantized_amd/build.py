"""Build libqmv.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_block_quantized_amd.build

Each translation unit (the launcher/ABI and one kernel table per weight
format) is compiled in parallel, then linked into one shared library.  The
library is compiled for gfx950 only.  Packed-FP32 VALU forms are switched off
(``-packed-fp32-ops``) so the compiler never emits v_pk_{add,mul,fma}_f32.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
KERNEL_SOURCES = ["qmv_k_mxfp4.hip", "qmv_k_mxfp4i.hip", "qmv_k_cb2.hip", "qmv_k_cb2s.hip", "qmv_k_cb3.hip",
                  "qmv_k_cb2q.hip", "qmv_k_cb2sq.hip", "qmv_k_cb3q.hip"]
# (source, extra flags, object): the launcher, the probe, the matrix-core
# kernels (MXFP4 x bf16 for 2-4 vectors and for more, codebook x int8 for
# more than 4; their workgroup size is a template argument or fixed), and
# every other kernel table twice -- 4 and 8 wave64s per workgroup, in
# namespaces qmv / qmv_w8.
UNITS = ([("qmv.hip", [], "qmv.o"), ("qmv_probe.hip", [], "qmv_probe.o"),
          ("qmv_k_mxfp4m.hip", [], "qmv_k_mxfp4m.o"),
          ("qmv_k_mxfp4b.hip", [], "qmv_k_mxfp4b.o"),
          ("qmv_k_cbm.hip", [], "qmv_k_cbm.o")] +
         [(k, [], k.replace(".hip", ".o")) for k in KERNEL_SOURCES] +
         [(k, ["-DQMV_WAVES=8", "-DQMV_NS=qmv_w8"], k.replace(".hip", "_w8.o")) for k in KERNEL_SOURCES])
SOURCES = [u[0] for u in UNITS]
LIB = os.path.join(HERE, "libqmv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mcode-object-version=5", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
]


# Every kernel's register and memory budget comes out of the compiler as
# remarks (one block per kernel); the build refuses any kernel that uses
# per-lane scratch memory.  Some kernels count their outstanding vector-memory
# loads by hand (an s_waitcnt vmcnt(N) that assumes a fixed number of loads
# per step); a register spill would add scratch loads and stores to that count
# and turn the wait into a silent race, and in the others it would be a
# performance bug.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs Spill|Dynamic Stack|"
                     r"VGPRs|AGPRs|Occupancy \[waves/SIMD\]):\s*(\S+)")


def parse_resource_usage(text: str) -> dict:
    """Per-kernel resource remarks from the compiler's output:
    {kernel symbol: {field: value}}."""
    kernels, cur = {}, None
    for field, value in _REMARK.findall(text):
        if field == "Function Name":
            cur = kernels.setdefault(value, {})
        elif cur is not None:
            cur[field] = value
    return kernels


def scratch_violations(kernels: dict) -> list:
    """Kernels that use scratch memory: scratch bytes, spilled VGPRs or a
    dynamic stack."""
    bad = []
    for name, r in sorted(kernels.items()):
        if (int(r.get("ScratchSize [bytes/lane]", "0")) != 0 or int(r.get("VGPRs Spill", "0")) != 0 or
                r.get("Dynamic Stack", "False") != "False"):
            bad.append((name, r))
    return bad


class ScratchError(RuntimeError):
    pass


def build(out: str = LIB, extra: list | None = None, verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="qmv_build_") as tmp:
        def compile_one(unit):
            src, defs, objname = unit
            obj = os.path.join(tmp, objname)
            cmd = [HIPCC, *FLAGS, RESOURCE_REMARKS, *inc, *defs, *(extra or []), "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                sys.stderr.write(r.stderr)
                raise subprocess.CalledProcessError(r.returncode, cmd)
            return obj, parse_resource_usage(r.stderr)
        jobs = min(len(UNITS), max(1, os.cpu_count() or 1))
        with ThreadPoolExecutor(jobs) as ex:
            res = list(ex.map(compile_one, UNITS))
        objs = [o for o, _ in res]
        kernels = {}
        for _, k in res:
            kernels.update(k)
        bad = scratch_violations(kernels)
        if bad:
            raise ScratchError("kernels using scratch memory: " +
                               "; ".join(f"{n} {r}" for n, r in bad))
        if verbose:
            print(f"{len(kernels)} kernels, none uses scratch memory", flush=True)
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    sys.exit(0)
