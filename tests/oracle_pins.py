"""Pins of the CPU oracle against facts fixed outside the oracle.

Each ``check_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something the pages, a published standard, a library
routine or exact arithmetic fixes.  ``test_oracle_pins.py`` runs them against
the oracle; ``test_oracle_mutants.py`` runs them against oracle builds with a
planted mistake and requires every mistake to be caught.

Independent sources used here (none of them is the oracle's C code):
  * the pages' fp2/fp3 code tables (``golden/page_code_tables.json``);
  * the OCP MX v1.0 FP4 (E2M1) value table;
  * torch's float8_e8m0fnu and bfloat16 casts, numpy's float16;
  * numpy ``unpackbits`` as a second bit unpacker;
  * exact rational arithmetic (``fractions.Fraction``) and int64 matmuls;
  * the hand-worked blocks in ``golden/hand_worked_blocks.json`` and the
    hand-quantized activation blocks in ``golden/q8_quantizer_blocks.json``.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# OCP Microscaling Formats v1.0, FP4 E2M1 element values for codes 0..7;
# codes 8..15 are the same magnitudes with the sign bit set.
E2M1_TABLE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def page_tables():
    with open(os.path.join(GOLD, "page_code_tables.json")) as f:
        return json.load(f)


def hand_worked():
    with open(os.path.join(GOLD, "hand_worked_blocks.json")) as f:
        return json.load(f)["cases"]


# ---------------------------------------------------------------- independent decoders
def ref_code_values(fmt):
    """Code -> value tables derived from the pages' printed tables."""
    t = page_tables()
    if fmt == "mxfp4":
        return [E2M1_TABLE[c & 7] * (-1 if c & 8 else 1) for c in range(16)]
    if fmt == "cb2":
        return [v - 0.5 for v in t["fp2"]["values"]]
    vals = [0.5 * v for v in t["fp3"]["values"]]
    vals[4] = -3.0       # the table's second zero is the codebook's -3
    return vals


def ref_codes(fmt, rows, K):
    """Unpack codes with numpy.unpackbits (little bit order): [n][K] ints."""
    rows = np.ascontiguousarray(rows, np.uint8)
    bits = np.unpackbits(rows, axis=-1, bitorder="little").astype(np.int64)
    w = {"mxfp4": 4, "cb2": 2, "cb3": 3}[fmt]
    bits = bits.reshape(rows.shape[0], -1, w)[:, :K, :]
    return (bits * (1 << np.arange(w))).sum(axis=-1)


def ref_e8m0(s):
    import torch
    t = torch.tensor(np.asarray(s, np.uint8)).view(torch.float8_e8m0fnu)
    return t.float().double().numpy()


def ref_fp16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def ref_bf16(bits):
    import torch
    t = torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.float().double().numpy()


def ref_dequant(fmt, crows, srows, K):
    """Dequantized weights [n][K] in float64 from the independent decoders."""
    codes = ref_codes(fmt, crows, K)
    vals = np.array(ref_code_values(fmt))[codes]
    srows = np.ascontiguousarray(srows, np.uint8)
    if fmt == "mxfp4":
        sc = ref_e8m0(srows)                       # [n][K/32]
        return vals * np.repeat(sc, 32, axis=1)
    f16 = ref_fp16(srows.view(np.uint16))
    per = 32 if fmt == "cb2" else 16
    return vals * np.repeat(f16, per, axis=1)


def ref_activations(afmt, x, xs, K):
    if afmt == "bf16":
        return ref_bf16(x)
    return np.asarray(x, np.int8).astype(np.float64) * np.repeat(ref_fp16(xs), 32, axis=1)


# ---------------------------------------------------------------- helpers
def _rng(seed):
    return np.random.default_rng(seed)


def _afmt(fmt):
    return "bf16" if fmt == "mxfp4" else "q8"


def _rcb(fmt, K):
    return {"mxfp4": K // 2, "cb2": K // 4, "cb3": 3 * K // 8}[fmt]


def _rsb(fmt, K):
    return {"mxfp4": K // 32, "cb2": K // 16, "cb3": K // 8}[fmt]


def _random_rows(rng, fmt, n, K, unit_scales=False):
    codes = rng.integers(0, 256, size=(n, _rcb(fmt, K)), dtype=np.uint8)
    if fmt == "mxfp4":
        s = np.full((n, K // 32), 127, np.uint8) if unit_scales else \
            rng.integers(118, 137, size=(n, K // 32), dtype=np.uint8)
    else:
        per = K // 32 if fmt == "cb2" else K // 16
        f = np.ones((n, per), np.float16) if unit_scales else \
            (np.abs(rng.standard_normal((n, per))) * 0.02).astype(np.float16)
        s = f.view(np.uint8).reshape(n, 2 * per)
    return codes, s


def _random_x(rng, fmt, V, K, small_ints=False, unit_xs=False):
    if fmt == "mxfp4":
        import torch
        g = rng.integers(-8, 9, size=(V, K)).astype(np.float32) if small_ints else \
            rng.standard_normal((V, K)).astype(np.float32)
        b = torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return b.copy(), None
    q = rng.integers(-128, 128, size=(V, K), dtype=np.int16).astype(np.int8)
    xs = np.ones((V, K // 32), np.float16) if unit_xs else \
        (np.abs(rng.standard_normal((V, K // 32))) * 0.05 + 1e-3).astype(np.float16)
    return q, xs.view(np.uint16)


def _dense_one_expert(o, fmt, codes, scales, x, xs, afmt=None):
    ids = np.zeros((x.shape[0], 1), np.int32)
    y, A = o.gather(fmt, codes[None], scales[None], ids, afmt or _afmt(fmt), x, xs)
    return y[:, 0, :], A[:, 0, :]


# ---------------------------------------------------------------- P1-P3 scalar decoders
def check_e2m1_table(o):
    for c in range(16):
        v = o.e2m1(c)
        want = E2M1_TABLE[c & 7]
        assert abs(v) == want, (c, v, want)
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0), ("sign", c, v)


def check_e8m0_library(o):
    ref = ref_e8m0(np.arange(256))
    for s in range(256):
        v = o.e8m0(s)
        if math.isnan(ref[s]):
            assert math.isnan(v), s
        else:
            assert v == ref[s], (s, v, ref[s])


def check_fp16_exhaustive(o):
    ref = ref_fp16(np.arange(65536))
    got = np.array([o.h2d(h) for h in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_bf16_exhaustive(o):
    ref = ref_bf16(np.arange(65536))
    got = np.array([o.bf16(b) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def check_codebooks_match_pages(o):
    t = page_tables()
    for fmt in ("cb2", "cb3"):
        got = [o.code_value(fmt, c) for c in range(4 if fmt == "cb2" else 8)]
        assert got == ref_code_values(fmt), (fmt, got)
        want_set = sorted(t["workload_%s_set" % fmt]["values"])
        assert sorted(got) == want_set, (fmt, sorted(got), want_set)


# ---------------------------------------------------------------- P4 hand-worked + unpackers
def _build_hw_case(case):
    fmt = case["fmt"]
    K = 32
    crow = np.zeros(_rcb(fmt, K), np.uint8)
    if "all" in case["codes"]:
        crow[:] = int(case["codes"]["all"], 16)
    else:
        for off, hx in case["codes"].items():
            crow[int(off)] = int(hx, 16)
    if fmt == "mxfp4":
        srow = np.array(case["scales"], np.uint8)
        xv = np.zeros(K, np.float32)
        if "all" in case["x"]:
            xv[:] = case["x"]["all"]
        else:
            for i, v in case["x"].items():
                xv[int(i)] = v
        x = (xv.view(np.uint32) >> 16).astype(np.uint16)[None]   # exact values only
        assert np.array_equal((x.astype(np.uint32) << 16).view(np.float32)[0], xv)
        xs = None
    else:
        srow = np.array(case["scales"], np.float16).view(np.uint8)
        q = np.zeros(K, np.int8)
        for i, v in case["q"].items():
            q[int(i)] = v
        x = q[None]
        xs = np.array(case["xs"], np.float16).view(np.uint16)[None]
    return fmt, crow, srow, x, xs


def check_hand_worked(o):
    for case in hand_worked():
        fmt, crow, srow, x, xs = _build_hw_case(case)
        y, A = _dense_one_expert(o, fmt, crow[None], srow[None], x, xs)
        assert y[0, 0] == case["y"], (case["name"], y[0, 0], case["y"])
        if "S" in case:
            S = o.block_sums(fmt, crow, x[0], 32)
            assert list(S[:len(case["S"])]) == case["S"], (case["name"], S)


def check_unpackers_agree(o):
    rng = _rng(11)
    for fmt in ("mxfp4", "cb2", "cb3"):
        K = 256
        codes, scales = _random_rows(rng, fmt, 8, K)
        ref = ref_codes(fmt, codes, K)
        for r in range(codes.shape[0]):
            got = [o.code(fmt, codes[r], k) for k in range(K)]
            assert got == list(ref[r]), (fmt, r)
        want = ref_dequant(fmt, codes, scales, K)
        for r in range(codes.shape[0]):
            w = o.dequant_row(fmt, codes[r], scales[r], K)
            assert np.array_equal(w, want[r]), (fmt, r)


# ---------------------------------------------------------------- P5 brute force on K = 32
def _frac_e2m1(c):
    return Fraction(E2M1_TABLE[c & 7]) * (-1 if c & 8 else 1)


def check_mxfp4_one_hot(o):
    """Every position x every code x every scale byte in [122, 132]: one
    nonzero weight, exact against rational arithmetic."""
    rng = _rng(12)
    K = 32
    rows, expect, xs_list = [], [], []
    x, _ = _random_x(rng, "mxfp4", 1, K)
    xv = ref_bf16(x[0])
    for i in range(K):
        for c in range(16):
            for s in range(122, 133):
                crow = np.zeros(K // 2, np.uint8)
                crow[i // 2] = (c << 4) if (i & 1) else c
                rows.append((crow, np.array([s], np.uint8)))
                expect.append(_frac_e2m1(c) * Fraction(2) ** (s - 127) * Fraction(float(xv[i])))
    codes = np.stack([r[0] for r in rows])
    scales = np.stack([r[1] for r in rows])
    y, _ = _dense_one_expert(o, "mxfp4", codes, scales, x, None)
    for n, want in enumerate(expect):
        assert Fraction(y[0, n]) == want, (n, y[0, n], float(want))


def check_random_blocks_exact(o):
    """Random K=32 rows against an exact rational dot (within 2^-50 * A)."""
    rng = _rng(13)
    K = 32
    for fmt in ("mxfp4", "cb2", "cb3"):
        n = 400
        codes, scales = _random_rows(rng, fmt, n, K)
        x, xs = _random_x(rng, fmt, 1, K)
        y, A = _dense_one_expert(o, fmt, codes, scales, x, xs)
        vals = ref_code_values(fmt)
        cds = ref_codes(fmt, codes, K)
        if fmt == "mxfp4":
            xv = [Fraction(float(v)) for v in ref_bf16(x[0])]
        else:
            d = Fraction(float(ref_fp16(xs[0])[0]))
            xv = [Fraction(int(q)) * d for q in x[0]]
        for r in range(n):
            if fmt == "mxfp4":
                sc = [Fraction(2) ** (int(scales[r, k // 32]) - 127) for k in range(K)]
            else:
                f16 = ref_fp16(scales[r].view(np.uint16))
                per = 32 if fmt == "cb2" else 16
                sc = [Fraction(float(f16[k // per])) for k in range(K)]
            exact = sum(Fraction(vals[cds[r, k]]) * sc[k] * xv[k] for k in range(K))
            assert abs(Fraction(y[0, r]) - exact) <= Fraction(2) ** -50 * Fraction(A[0, r]), \
                (fmt, r, y[0, r], float(exact))


# ---------------------------------------------------------------- P6 dot structure
def check_block_factored(o):
    """Literal y equals the block-factored sum_b scale_b * xs * S_b / 2 built
    from the integer side output (per-block factorization of the dot)."""
    rng = _rng(14)
    for fmt in ("cb2", "cb3"):
        K = 256
        codes, scales = _random_rows(rng, fmt, 16, K)
        q, xs = _random_x(rng, fmt, 1, K)
        y, A = _dense_one_expert(o, fmt, codes, scales, q, xs)
        f16 = ref_fp16(scales.view(np.uint16))
        xsv = ref_fp16(xs[0])
        bs = 32 if fmt == "cb2" else 16
        for r in range(codes.shape[0]):
            S = o.block_sums(fmt, codes[r], q[0], K)
            blk = sum(float(f16[r, b]) * float(xsv[(b * bs) // 32]) * int(S[b]) / 2.0
                      for b in range(K // bs))
            assert abs(blk - y[0, r]) <= 1e-12 * max(A[0, r], 1e-300), (fmt, r, blk, y[0, r])


# ---------------------------------------------------------------- P7 exact special cases
def check_unit_scale_exact(o):
    rng = _rng(15)
    K = 512
    for fmt in ("cb2", "cb3"):
        codes, scales = _random_rows(rng, fmt, 32, K, unit_scales=True)
        q, xs = _random_x(rng, fmt, 1, K, unit_xs=True)
        y, _ = _dense_one_expert(o, fmt, codes, scales, q, xs)
        v2 = (2 * np.array(ref_code_values(fmt))).astype(np.int64)[ref_codes(fmt, codes, K)]
        want = v2 @ q[0].astype(np.int64)               # int64 matmul, exact
        assert np.array_equal(y[0] * 2, want.astype(np.float64)), fmt
        for r in range(codes.shape[0]):
            S = o.block_sums(fmt, codes[r], q[0], K)
            assert int(S.sum()) == int(want[r]), (fmt, r)
    codes, scales = _random_rows(rng, "mxfp4", 32, K, unit_scales=True)
    x, _ = _random_x(rng, "mxfp4", 1, K, small_ints=True)
    y, _ = _dense_one_expert(o, "mxfp4", codes, scales, x, None)
    vals = np.array(ref_code_values("mxfp4"))[ref_codes("mxfp4", codes, K)]
    want = vals @ ref_bf16(x[0])
    assert np.array_equal(y[0], want), "mxfp4 unit scale"
    # MXFP4 weights with int8 activations at unit scales (E8M0 127, fp16 1.0):
    # twice the result is the int64 matmul of the doubled e2m1 values (all
    # integers) with q, int8 -128 included
    codes, scales = _random_rows(rng, "mxfp4", 32, K, unit_scales=True)
    q, xs = _random_x(rng, "cb2", 1, K, unit_xs=True)
    y, A = _dense_one_expert(o, "mxfp4", codes, scales, q, xs, afmt="q8")
    v2 = (2 * np.array(ref_code_values("mxfp4"))).astype(np.int64)[ref_codes("mxfp4", codes, K)]
    want = v2 @ q[0].astype(np.int64)
    assert np.array_equal(y[0] * 2, want.astype(np.float64)), "mxfp4 x int8 unit scale"
    assert np.array_equal(A[0] * 2, (np.abs(v2) @ np.abs(q[0].astype(np.int64))).astype(np.float64))


# ---------------------------------------------------------------- P8 gather semantics
def check_gather_semantics(o):
    rng = _rng(16)
    K, N, E = 64, 24, 6
    for fmt in ("mxfp4", "cb2", "cb3"):
        afmt = _afmt(fmt)
        codes = np.stack([_random_rows(rng, fmt, N, K)[0] for _ in range(E)])
        scales = np.stack([_random_rows(rng, fmt, N, K)[1] for _ in range(E)])
        x, xs = _random_x(rng, fmt, 2, K)
        # one expert == dense on that expert's matrix
        for e in range(E):
            yg, _ = o.gather(fmt, codes, scales, np.array([[e], [e]], np.int32), afmt, x, xs)
            yd, _ = o.dense(fmt, codes[e], scales[e], afmt, x, xs)
            assert np.array_equal(yg[:, 0, :], yd), (fmt, e)
        # invalid ids give zero rows (and zero A)
        ids = np.array([[-1, 2, E, 0], [2 ** 31 - 1, -2 ** 31, 5, 1]], np.int32)
        y, A = o.gather(fmt, codes, scales, ids, afmt, x, xs)
        for t in range(2):
            for j in range(4):
                e = ids[t, j]
                if 0 <= e < E:
                    yd, _ = o.dense(fmt, codes[e], scales[e], afmt, x[t:t + 1],
                                    None if xs is None else xs[t:t + 1])
                    assert np.array_equal(y[t, j], yd[0]), (fmt, t, j)
                else:
                    assert not y[t, j].any() and not A[t, j].any(), (fmt, t, j)
        # relabelling the experts together with the ids leaves y unchanged
        perm = rng.permutation(E)
        inv = np.argsort(perm)
        ids = np.array([[0, 3, 5], [1, 1, 4]], np.int32)
        y0, _ = o.gather(fmt, codes, scales, ids, afmt, x, xs)
        y1, _ = o.gather(fmt, codes[perm], scales[perm], inv[ids].astype(np.int32), afmt, x, xs)
        assert np.array_equal(y0, y1), fmt
        # y is homogeneous in x: doubling x doubles y exactly
        if fmt == "mxfp4":
            x2 = (x.astype(np.uint32) + (1 << 7)).astype(np.uint16)   # exponent + 1
            xs2 = None
        else:
            x2 = x
            xs2 = (xs.view(np.float16) * np.float16(2)).view(np.uint16)
        y2, _ = o.gather(fmt, codes, scales, ids, afmt, x2, xs2)
        assert np.array_equal(y2, 2 * y0), fmt
        # per-slot activations that all equal the token's vector == broadcast
        xp = np.repeat(x, 3, axis=0)
        xsp = None if xs is None else np.repeat(xs, 3, axis=0)
        yp, _ = o.gather(fmt, codes, scales, ids, afmt, xp, xsp, x_per_slot=True)
        assert np.array_equal(yp, y0), fmt


# ---------------------------------------------------------------- P9 fused gate/up SwiGLU
def check_swiglu(o):
    """silu(g) * u against scipy's logistic function, on g and u from the
    (separately pinned) gather; gate and up must not be interchangeable."""
    from scipy.special import expit
    rng = _rng(17)
    K, N, E = 64, 16, 5
    for fmt in ("mxfp4", "cb2", "cb3"):
        afmt = _afmt(fmt)
        gc = np.stack([_random_rows(rng, fmt, N, K)[0] for _ in range(E)])
        gs = np.stack([_random_rows(rng, fmt, N, K)[1] for _ in range(E)])
        uc = np.stack([_random_rows(rng, fmt, N, K)[0] for _ in range(E)])
        us = np.stack([_random_rows(rng, fmt, N, K)[1] for _ in range(E)])
        x, xs = _random_x(rng, fmt, 2, K)
        if fmt == "mxfp4":
            # make the gate pre-activations span silu's range, well past +-10
            gs = np.full_like(gs, 130)
        ids = np.array([[0, 4, E], [3, -1, 4]], np.int32)
        y, g, u, Ag, Au = o.gather_swiglu(fmt, gc, gs, uc, us, ids, afmt, x, xs)
        g2, Ag2 = o.gather(fmt, gc, gs, ids, afmt, x, xs)
        u2, Au2 = o.gather(fmt, uc, us, ids, afmt, x, xs)
        assert np.array_equal(g, g2) and np.array_equal(u, u2), fmt
        assert np.array_equal(Ag, Ag2) and np.array_equal(Au, Au2), fmt
        want = g * expit(g) * u
        assert np.allclose(y, want, rtol=1e-14, atol=1e-300), fmt
        valid = (ids >= 0) & (ids < E)
        assert not y[~valid].any(), fmt
        assert (np.abs(g[valid]) > 0).all(), fmt
        if fmt == "mxfp4":
            assert np.abs(g).max() > 10, "gate range too narrow to test saturation"
        # an all-zero gate weight gives g = 0 and silu(0) = 0 whatever u is
        zc = np.zeros_like(gc)
        if fmt == "cb2":    # 2-bit codes have no zero: take a zero scale instead
            zs = np.zeros_like(gs)
        else:
            zs = gs
            if fmt == "cb3":
                zc = np.zeros_like(gc)          # code 0 means 0 in the 3-bit book
        yz, gz, _, _, _ = o.gather_swiglu(fmt, zc, zs, uc, us, ids, afmt, x, xs)
        assert not gz.any() and not yz.any(), fmt
        # gate and up are not symmetric: swapping them changes y
        ysw, _, _, _, _ = o.gather_swiglu(fmt, uc, us, gc, gs, ids, afmt, x, xs)
        assert not np.array_equal(ysw[valid], y[valid]), fmt


# ---------------------------------------------------------------- P10 router-weighted combine
def check_combine(o):
    """The combine against facts that do not restate its sum: a one-hot weight
    picks one slot's gather row exactly; scaling every weight by a power of two
    scales y exactly; slots reordered together with their weights give the same
    y (to rounding); an out-of-range id adds nothing; two slots of one expert
    equal one slot with the summed weight."""
    rng = _rng(18)
    K, N, E, M, top_k = 64, 12, 5, 2, 4
    for fmt in ("mxfp4", "cb2", "cb3"):
        afmt = _afmt(fmt)
        codes = np.stack([_random_rows(rng, fmt, N, K)[0] for _ in range(E)])
        scales = np.stack([_random_rows(rng, fmt, N, K)[1] for _ in range(E)])
        x, xs = _random_x(rng, fmt, M * top_k, K)            # one vector per (token, slot)
        ids = np.array([[0, 3, 1, 4], [2, 2, 0, 1]], np.int32)
        w = rng.uniform(0.05, 1.0, size=(M, top_k)).astype(np.float32)
        y, A = o.combine(fmt, codes, scales, ids, w, afmt, x, xs)
        g, Ag = o.gather(fmt, codes, scales, ids, afmt, x, xs, x_per_slot=True)
        for t in range(M):
            for j in range(top_k):
                oh = np.zeros_like(w)
                oh[t, j] = 1.0
                y1, _ = o.combine(fmt, codes, scales, ids, oh, afmt, x, xs)
                assert np.array_equal(y1[t], g[t, j]), (fmt, t, j)
        y4, A4 = o.combine(fmt, codes, scales, ids, 4 * w, afmt, x, xs)
        assert np.array_equal(y4, 4 * y) and np.allclose(A4, 4 * A, rtol=1e-15), fmt
        perm = np.array([2, 0, 3, 1])
        xp = x.reshape(M, top_k, -1)[:, perm].reshape(M * top_k, -1)
        xsp = None if xs is None else xs.reshape(M, top_k, -1)[:, perm].reshape(M * top_k, -1)
        yp, _ = o.combine(fmt, codes, scales, ids[:, perm], w[:, perm], afmt, xp, xsp)
        assert np.allclose(yp, y, rtol=1e-12, atol=1e-12 * A.max()), fmt
        bad = ids.copy()
        bad[0, 1] = E
        yb, Ab = o.combine(fmt, codes, scales, bad, w, afmt, x, xs)
        assert np.allclose(yb[0], y[0] - w[0, 1] * g[0, 1], rtol=1e-12, atol=1e-12 * A.max()), fmt
        assert np.array_equal(yb[1], y[1]), fmt
        # token 1 has expert 2 in slots 0 and 1: with broadcast activations the two
        # slots are one slot of summed weight
        xb, xsb = _random_x(rng, fmt, M, K)
        w2 = w.copy()
        w2[1, 0], w2[1, 1] = 0.25, 0.5
        yd, _ = o.combine(fmt, codes, scales, ids, w2, afmt, xb, xsb, x_per_slot=False)
        gb, _ = o.gather(fmt, codes, scales, ids, afmt, xb, xsb)
        want = 0.75 * gb[1, 0] + w2[1, 2] * gb[1, 2] + w2[1, 3] * gb[1, 3]
        assert np.allclose(yd[1], want, rtol=1e-12, atol=1e-12 * np.abs(gb).max()), fmt


def check_combine_signed(o):
    """Router weights of either sign, and weights that sum to zero: a negative
    one-hot weight gives exactly the negated gather row; negating every weight
    negates y exactly and leaves A (which sums |w| |w x|) unchanged; two slots
    of one expert fed the same vector with weights a and -a cancel, leaving
    the other slots' sum."""
    rng = _rng(19)
    K, N, E, M, top_k = 96, 10, 4, 2, 4
    for fmt in ("mxfp4", "cb2", "cb3"):
        afmt = _afmt(fmt)
        codes = np.stack([_random_rows(rng, fmt, N, K)[0] for _ in range(E)])
        scales = np.stack([_random_rows(rng, fmt, N, K)[1] for _ in range(E)])
        x, xs = _random_x(rng, fmt, M * top_k, K)
        ids = np.array([[1, 1, 3, 0], [2, 0, 3, 1]], np.int32)
        w = rng.uniform(-1.0, 1.0, size=(M, top_k)).astype(np.float32)
        w[0, 2] = -abs(w[0, 2])
        y, A = o.combine(fmt, codes, scales, ids, w, afmt, x, xs)
        g, _ = o.gather(fmt, codes, scales, ids, afmt, x, xs, x_per_slot=True)
        oh = np.zeros_like(w)
        oh[1, 2] = -1.0
        y1, _ = o.combine(fmt, codes, scales, ids, oh, afmt, x, xs)
        assert np.array_equal(y1[1], -g[1, 2]) and not y1[0].any(), fmt
        yn, An = o.combine(fmt, codes, scales, ids, -w, afmt, x, xs)
        assert np.array_equal(yn, -y) and np.array_equal(An, A), fmt
        ya, Aa = o.combine(fmt, codes, scales, ids, np.abs(w), afmt, x, xs)
        assert np.array_equal(Aa, A), fmt
        # token 0: expert 1 in slots 0 and 1; with broadcast activations and
        # weights +a / -a the two slots cancel
        xb, xsb = _random_x(rng, fmt, M, K)
        wz = w.copy()
        wz[0, 0], wz[0, 1] = 0.375, -0.375
        yz, _ = o.combine(fmt, codes, scales, ids, wz, afmt, xb, xsb, x_per_slot=False)
        gb, _ = o.gather(fmt, codes, scales, ids, afmt, xb, xsb)
        want = wz[0, 2] * gb[0, 2] + wz[0, 3] * gb[0, 3]
        assert np.allclose(yz[0], want, rtol=1e-12, atol=1e-12 * np.abs(gb).max()), fmt
        if np.abs(gb[0, 0]).max() > 0:
            assert not np.allclose(yz[0], want + 0.75 * gb[0, 0], rtol=1e-9, atol=0), fmt


# ---------------------------------------------------------------- P11 activation quantizer
def check_f2h_library(o):
    """The oracle's binary16 encoder against numpy's float32 -> float16 cast
    (round to nearest even): every bf16 value, random float32 bit patterns,
    and the exact midpoints between neighbouring fp16 values."""
    rng = _rng(31)
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    rnd = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    h = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = ((h[:-1] + h[1:]) / 2).astype(np.float32)            # exact in fp32
    near = np.concatenate([np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))])
    vals = np.concatenate([bf, rnd, mid, -mid, near, -near]).astype(np.float32)
    vals = vals[~np.isnan(vals)]
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([o.lib.oracle_f2h(float(v)) for v in vals], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (vals[bad[0]], hex(got[bad[0]]), hex(want[bad[0]]))


def q8_blocks_golden():
    with open(os.path.join(GOLD, "q8_quantizer_blocks.json")) as f:
        return json.load(f)["cases"]


def check_q8_hand_worked(o):
    """The quantizer against blocks quantized by hand (ties to even, the
    rounded fp16 scale, clipping, zero and underflowing scales)."""
    for case in q8_blocks_golden():
        x = np.zeros(32, np.float32)
        for i, v in case["x"].items():
            x[int(i)] = v
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), x), case["name"]
        q, d = o.quantize_q8(bits[None])
        want = np.zeros(32, np.int64)
        for i, v in case["q"].items():
            want[int(i)] = v
        assert np.array_equal(q[0].astype(np.int64), want), (case["name"], q[0])
        assert int(d[0, 0]) == int(case["d16"], 16), (case["name"], hex(int(d[0, 0])))


def check_q8_invariants(o):
    """Random blocks over twenty decades of magnitude: |q| <= 127; where the
    fp16 scale d16 is normal, the largest |x| maps to +-127 and every q is
    within 1/2 (plus fp32 rounding of x * r) of x / d16; signs are kept;
    d16 is numpy's float16 rounding of the fp32 amax / 127."""
    rng = _rng(32)
    V, K = 64, 32 * 40
    for sigma in [1e-12, 1e-8, 1e-6, 1e-4, 1e-2, 1.0, 1e2, 1e4]:
        g = (rng.standard_normal((V, K)) * sigma).astype(np.float32)
        bits = (g.view(np.uint32) >> 16).astype(np.uint16)        # truncate to bf16
        x = (bits.astype(np.uint32) << 16).view(np.float32).reshape(V, K // 32, 32)
        q, d = o.quantize_q8(bits)
        q = q.reshape(V, K // 32, 32).astype(np.int64)
        amax = np.abs(x).max(axis=2)
        assert np.array_equal(d, (amax / np.float32(127)).astype(np.float16).view(np.uint16))
        d16 = d.view(np.float16).astype(np.float64)[..., None]
        assert (np.abs(q) <= 127).all()
        assert ((q == 0) | (np.sign(q) == np.sign(x))).all()
        normal = (d16 >= 2.0 ** -14)[..., 0]
        if normal.any():
            t = x.astype(np.float64)[normal] / d16[normal]
            assert (np.abs(q[normal] - t) <= 0.5 + 1e-6 * np.abs(t)).all(), sigma
            am = np.abs(x[normal]).argmax(axis=1)
            top = np.take_along_axis(q[normal], am[:, None], axis=1)[:, 0]
            assert (np.abs(top) == 127).all(), sigma
        zero = (d16 == 0)[..., 0]
        assert (q[zero] == 0).all()


ALL_CHECKS = [
    check_e2m1_table,
    check_e8m0_library,
    check_fp16_exhaustive,
    check_bf16_exhaustive,
    check_codebooks_match_pages,
    check_hand_worked,
    check_unpackers_agree,
    check_mxfp4_one_hot,
    check_random_blocks_exact,
    check_block_factored,
    check_unit_scale_exact,
    check_gather_semantics,
    check_swiglu,
    check_combine,
    check_combine_signed,
    check_f2h_library,
    check_q8_hand_worked,
    check_q8_invariants,
]
