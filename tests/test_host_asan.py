"""The library's host-side logic under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

qmv_host.hpp holds everything the entry points do before a launch -- the
argument checks, the launch-shape choice (pick_shape, tuned_shape) and the
status texts -- as plain C++.  This test builds it with the host compiler and
both sanitizers into a small driver (tests/qmv_host_check.cpp), runs every
argument case of the host ABI tests through it, and requires the statuses
the ABI tests require and a clean sanitizer report.
"""
import inspect
import os
import subprocess

import pytest

import test_abi_host as abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_block_quantized_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asan") / "qmv_host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(ROOT, "tests", "qmv_host_check.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


def _line(cmd, fn, kw):
    """The command line for one ABI test case: the helper's defaults with the
    case's overrides, in the helper's argument order (None -> 0)."""
    params = [p for p in inspect.signature(fn).parameters.values() if p.name != "L"]
    vals = [kw.get(p.name, p.default) for p in params]
    return " ".join([cmd] + [str(0 if v is None else int(v)) for v in vals])


def _run(checker, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([checker], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       env=env, timeout=120)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    out = r.stdout.splitlines()
    assert len(out) == len(lines), (len(out), len(lines), r.stdout[-2000:])
    return out


def test_entry_point_checks_under_sanitizers(checker):
    cases = ([("dense", abi.dense, kw, want) for kw, want in abi.DENSE_CASES] +
             [("gather", abi.gather, kw, want) for kw, want in abi.GATHER_CASES] +
             [("swiglu", abi.swiglu, kw, want) for kw, want in abi.SWIGLU_CASES] +
             [("combine", abi.combine, kw, want) for kw, want in abi.COMBINE_CASES])
    # the helpers' defaults themselves are valid calls
    cases += [(c, fn, {}, abi.OK) for c, fn in (("dense", abi.dense), ("gather", abi.gather),
                                                 ("swiglu", abi.swiglu), ("combine", abi.combine))]
    lines = [_line(c, fn, kw) for c, fn, kw, _ in cases]
    out = _run(checker, lines)
    for (c, _, kw, want), got, line in zip(cases, out, lines):
        assert int(got) == want, f"{line}: {got} != {want}"


def test_shape_choice_and_texts_under_sanitizers(checker):
    lines = ["shapes"] + [f"strerror {s}" for s in (0, 1, 2, 3, 4, 99, -1)]
    out = _run(checker, lines)
    int(out[0])
    assert all(t and "unknown" not in t for t in out[1:6])
    assert out[6] == out[7] == "unknown status"


def test_library_agrees_with_the_sanitized_build(checker):
    """The shipped library returns, case by case, what the sanitized build of
    the same checks returns (one source, two compilers)."""
    import bit_block_quantized_amd as q
    L = q.lib()
    # only calls the checks reject: a valid call with these fake pointers
    # would launch a kernel
    cases = ([("dense", abi.dense, kw) for kw, want in abi.DENSE_CASES if want != abi.OK] +
             [("gather", abi.gather, kw) for kw, want in abi.GATHER_CASES if want != abi.OK])
    out = _run(checker, [_line(c, fn, kw) for c, fn, kw in cases])
    for (c, fn, kw), got in zip(cases, out):
        assert fn(L, **kw) == int(got), (c, kw)
