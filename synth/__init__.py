"""Seeded synthetic inputs for the block-quantized GEMV workloads.

This module is shared by the tests, the benchmark and the smoke check, and it
is the ONLY thing the CPU oracle and the HIP path have in common.  It holds no
arithmetic of the GEMV itself: it draws random bytes, random scale bit
patterns, expert ids and activation vectors, nothing else.  Every draw comes
from ``numpy.random.default_rng(seed)`` in one fixed order per workload:
codes -> weight scales -> expert ids -> activations -> activation scales.

Workload shapes (the expert-projection GEMVs the pages measure):

* ``C1``  dense MXFP4, M=1, K=N=256, E8M0 scales uniform in [124, 130].
* ``C2``  gpt-oss-20b MoE decode gather: 32 experts, top-4 distinct ids,
  1 token, K=N=2880, MXFP4 group 32, E8M0 uniform in [122, 132], bf16
  activations ~N(0,1) (mlxcel issue "add an mxfp4 arm to the warp-shared
  gather_qmv kernel for gpt-oss decode", Current Behavior).
* ``C3``  DeepSeek-shaped 2-bit MoE gate/up gather: 256 experts, top-4,
  1 token, K=7168, N=2048, fp16 scale per 32 ~|N(0, 0.02)|, int8
  activations with an fp16 scale per 32 (geo-lucebox PR "DS4 H200:
  rocmfp2_mix MoE matvec", "Why this kernel": in=7168, out=2048, top-k 4).
* ``C4``  3-bit down projection gather: 256 experts, top-4, 1 token,
  K=2048, N=7168, fp16 scale per 16-weight half-block, int8 activations per
  expert slot (each slot feeds its own expert's input).
* ``C5a`` verify width 4: 4 tokens x top-4 of 256 (distinct within a token,
  overlaps across tokens allowed), MXFP4, K=7168, N=2048.
* ``C5b`` dense MXFP4, M=4, K=N=7168.
* ``C6``  prefill chunk: 512 tokens x top-4 of 32 (gpt-oss-20b), MXFP4 x bf16,
  K=N=2880 -- the expert-batched path for more than 4 vectors; ``C6gu`` the
  same chunk through the fused gate/up projection with SwiGLU; ``C6d`` a
  dense 7168 x 7168 MXFP4 matrix against 64 vectors.

Activation recipe: bf16 activations are N(0,1) samples rounded to bf16 by
torch's float32 -> bfloat16 cast (round to nearest even).  int8 activations
are N(0,1) samples quantized per 32 with an absmax recipe (d = fp16(amax/127),
q = clip(rint(x/d), -127, 127), q = 0 where d = 0): this only shapes the
synthetic data; the GEMV consumes (q, d) exactly as given.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FORMATS = ("mxfp4", "cb2", "cb3")


def row_code_bytes(wfmt: str, K: int) -> int:
    return {"mxfp4": K // 2, "cb2": K // 4, "cb3": 3 * K // 8}[wfmt]


def row_scale_bytes(wfmt: str, K: int) -> int:
    return {"mxfp4": K // 32, "cb2": 2 * (K // 32), "cb3": 2 * (K // 16)}[wfmt]


def afmt_of(wfmt: str) -> str:
    return "bf16" if wfmt == "mxfp4" else "q8"


@dataclass
class Workload:
    name: str
    kind: str            # "dense" or "gather"
    wfmt: str
    M: int
    N: int
    K: int
    seed: int
    E: int = 1
    top_k: int = 1
    x_per_slot: bool = False
    e8m0: tuple = (122, 132)
    ids: str = "distinct"     # distinct within a token; overlaps across tokens allowed
    desc: str = ""
    x_bf16: bool = False      # 2-/3-bit weights fed bf16 activations (quantized in the kernel)
    x_q8: bool = False        # MXFP4 weights fed int8 activations with a scale per 32

    @property
    def afmt(self) -> str:
        if self.x_bf16 and self.wfmt != "mxfp4":
            return "bf16q8"
        if self.x_q8 and self.wfmt == "mxfp4":
            return "q8"
        return afmt_of(self.wfmt)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "C1": Workload("C1", "dense", "mxfp4", M=1, N=256, K=256, seed=1, e8m0=(124, 130),
                   desc="dense MXFP4 GEMV, M=1, K=N=256"),
    "C2": Workload("C2", "gather", "mxfp4", M=1, N=2880, K=2880, seed=2, E=32, top_k=4,
                   desc="gpt-oss-20b MoE decode gather, 4 of 32 experts, K=N=2880, MXFP4"),
    "C3": Workload("C3", "gather", "cb2", M=1, N=2048, K=7168, seed=3, E=256, top_k=4,
                   desc="DeepSeek-shaped 2-bit MoE gate/up gather, 4 of 256, K=7168, N=2048"),
    "C4": Workload("C4", "gather", "cb3", M=1, N=7168, K=2048, seed=4, E=256, top_k=4,
                   x_per_slot=True,
                   desc="3-bit MoE down-proj gather, 4 of 256, K=2048, N=7168, per-slot int8 x"),
    "C5a": Workload("C5a", "gather", "mxfp4", M=4, N=2048, K=7168, seed=5, E=256, top_k=4,
                    desc="verify width 4: 4 tokens x top-4 of 256, MXFP4, K=7168, N=2048"),
    "C5b": Workload("C5b", "dense", "mxfp4", M=4, N=7168, K=7168, seed=5,
                    desc="dense MXFP4 GEMV, M=4, K=N=7168"),
}

# Fused gate/up projections (two weight tensors of one shape, SwiGLU between
# them): the gpt-oss-20b and DeepSeek-shaped MoE gate/up matrices.
GATE_UP_WORKLOADS = {
    "C2gu": Workload("C2gu", "gate_up", "mxfp4", M=1, N=2880, K=2880, seed=6, E=32, top_k=4,
                     e8m0=(115, 120),
                     desc="gpt-oss-20b MoE decode gate+up with SwiGLU, 4 of 32 experts, "
                          "K=N=2880, MXFP4"),
    "C3gu": Workload("C3gu", "gate_up", "cb2", M=1, N=2048, K=7168, seed=7, E=256, top_k=4,
                     desc="DeepSeek-shaped 2-bit MoE gate+up with SwiGLU, 4 of 256, K=7168, "
                          "N=2048"),
}


# Down projections with the router-weighted top-k combine (one activation
# vector per (token, slot), y[M][N]).
COMBINE_WORKLOADS = {
    "C4c": Workload("C4c", "combine", "cb3", M=1, N=7168, K=2048, seed=8, E=256, top_k=4,
                    x_per_slot=True,
                    desc="3-bit MoE down-proj, 4 of 256, K=2048, N=7168, per-slot int8 x, "
                         "router-weighted combine"),
    "C2c": Workload("C2c", "combine", "mxfp4", M=1, N=2880, K=2880, seed=9, E=32, top_k=4,
                    x_per_slot=True,
                    desc="gpt-oss-20b MoE down-proj, 4 of 32, K=N=2880, MXFP4, per-slot bf16 x, "
                         "router-weighted combine"),
}


# The 2-bit and 3-bit gathers fed bf16 activations, which the kernel quantizes
# to int8 per 32 while staging them (no separate quantize launch); the MXFP4
# gather fed int8 activations.
QUANT_WORKLOADS = {
    "C3q": WORKLOADS["C3"].scaled(name="C3q", x_bf16=True, seed=10,
                                  desc="DeepSeek-shaped 2-bit MoE gate/up gather, 4 of 256, "
                                       "K=7168, N=2048, bf16 x quantized in the kernel"),
    "C4q": WORKLOADS["C4"].scaled(name="C4q", x_bf16=True, seed=11,
                                  desc="3-bit MoE down-proj gather, 4 of 256, K=2048, N=7168, "
                                       "per-slot bf16 x quantized in the kernel"),
    # MXFP4 weights with int8 activations (fp16 scale per 32)
    "C2i": WORKLOADS["C2"].scaled(name="C2i", x_q8=True, seed=12,
                                  desc="gpt-oss-20b MoE decode gather, 4 of 32, K=N=2880, MXFP4 "
                                       "weights x int8 activations with an fp16 scale per 32"),
}


# More than 4 vectors per call (MXFP4 x bf16, the expert-batched matrix-core
# path): a gpt-oss-20b prefill chunk, every token routed to 4 of the 32
# experts, so each expert meets about 64 of the 2048 (token, slot) pairs.
BATCHED_WORKLOADS = {
    "C6": Workload("C6", "gather", "mxfp4", M=512, N=2880, K=2880, seed=13, E=32, top_k=4,
                   desc="gpt-oss-20b MoE prefill chunk: 512 tokens x top-4 of 32 experts, "
                        "K=N=2880, MXFP4 x bf16, expert-batched"),
    "C6gu": Workload("C6gu", "gate_up", "mxfp4", M=512, N=2880, K=2880, seed=14, E=32, top_k=4,
                     e8m0=(115, 120),
                     desc="gpt-oss-20b MoE prefill chunk, fused gate+up with SwiGLU: 512 tokens "
                          "x top-4 of 32 experts, K=N=2880, MXFP4 x bf16, expert-batched"),
    "C6d": Workload("C6d", "dense", "mxfp4", M=64, N=7168, K=7168, seed=15,
                    desc="dense MXFP4 x bf16, 64 vectors, K=N=7168 (K-split matrix-core tiles)"),
    # A DeepSeek-shaped prefill chunk on the codebook formats: 512 tokens, each
    # routed to 4 of 256 experts (about 8 (token, slot) pairs per expert),
    # int8 activations with a scale per 32.
    "C7": Workload("C7", "gather", "cb2", M=512, N=2048, K=7168, seed=16, E=256, top_k=4,
                   desc="DeepSeek-shaped MoE prefill chunk, 2-bit gate/up gather: 512 tokens x "
                        "top-4 of 256, K=7168, N=2048, int8 x"),
    "C8": Workload("C8", "gather", "cb3", M=512, N=7168, K=2048, seed=17, E=256, top_k=4,
                   x_per_slot=True,
                   desc="DeepSeek-shaped MoE prefill chunk, 3-bit down-proj gather: 512 tokens x "
                        "top-4 of 256, K=2048, N=7168, per-slot int8 x"),
    # The same chunks' down projections with the router-weighted combine
    # (y[M][N]): the per-slot gather, then the slot sum.
    "C6c": Workload("C6c", "combine", "mxfp4", M=512, N=2880, K=2880, seed=18, E=32, top_k=4,
                    x_per_slot=True,
                    desc="gpt-oss-20b MoE prefill chunk, down-proj with router-weighted combine: "
                         "512 tokens x top-4 of 32, K=N=2880, MXFP4 x per-slot bf16"),
    "C8c": Workload("C8c", "combine", "cb3", M=512, N=7168, K=2048, seed=19, E=256, top_k=4,
                    x_per_slot=True,
                    desc="DeepSeek-shaped MoE prefill chunk, 3-bit down-proj with router-weighted "
                         "combine: 512 tokens x top-4 of 256, K=2048, N=7168, per-slot int8 x"),
}


def workload(name: str) -> Workload:
    for table in (WORKLOADS, GATE_UP_WORKLOADS, COMBINE_WORKLOADS, QUANT_WORKLOADS,
                  BATCHED_WORKLOADS):
        if name in table:
            return table[name]
    raise KeyError(name)


@dataclass
class Inputs:
    """Host arrays of one call, in the boundary layouts."""
    wl: Workload
    codes: np.ndarray          # uint8 [E][N][row_code_bytes]   (dense: [N][...])
    scales: np.ndarray         # uint8 [E][N][row_scale_bytes]  (fp16 as LE byte pairs)
    ids: np.ndarray | None     # int32 [M][top_k]
    x: np.ndarray              # uint16 bf16 bits or int8; [V][K]
    xs: np.ndarray | None      # uint16 fp16 bits [V][K/32]
    extra: dict = field(default_factory=dict)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 samples -> bf16 bit patterns via torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def q8_blocks(samples: np.ndarray):
    """Per-32 absmax int8 data (q, fp16 scale bits) shaped like ``samples``."""
    s = np.ascontiguousarray(samples, np.float32)
    V, K = s.shape
    blk = s.reshape(V, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d > 0, np.rint(blk / np.where(d > 0, d, 1)), 0)
    q = np.clip(q, -127, 127).astype(np.int8).reshape(V, K)
    return q, d16.view(np.uint16)


def gen_codes(rng, wfmt, E, N, K):
    # uniform bytes give independent uniform codes for all three packings
    return rng.integers(0, 256, size=(E, N, row_code_bytes(wfmt, K)), dtype=np.uint8)


def gen_scales(rng, wfmt, E, N, K, e8m0=(122, 132)):
    if wfmt == "mxfp4":
        lo, hi = e8m0
        return rng.integers(lo, hi + 1, size=(E, N, K // 32), dtype=np.uint8)
    per = K // 32 if wfmt == "cb2" else K // 16
    s = np.abs(rng.standard_normal(size=(E, N, per), dtype=np.float32)) * np.float32(0.02)
    return s.astype(np.float16).view(np.uint8).reshape(E, N, 2 * per)


def gen_ids(rng, M, top_k, E):
    """Top-k ids: distinct within a token (repeats only when top_k > E),
    independent across tokens."""
    ids = np.empty((M, top_k), np.int32)
    for t in range(M):
        ids[t] = rng.choice(E, size=top_k, replace=top_k > E)
    return ids


def gen_activations(rng, afmt, V, K):
    g = rng.standard_normal(size=(V, K), dtype=np.float32)
    if afmt in ("bf16", "bf16q8"):
        return bf16_bits(g), None
    return q8_blocks(g)


def make(name_or_wl, seed: int | None = None, experts: int | None = None) -> Inputs:
    """Draw one call's inputs for a workload.

    ``experts`` overrides E (to shrink the expert table for fast tests; the ids
    are then drawn from the smaller table).
    """
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    if experts is not None:
        wl = wl.scaled(E=experts)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    routed = wl.kind in ("gather", "combine")
    E = wl.E if routed else 1
    codes = gen_codes(rng, wl.wfmt, E, wl.N, wl.K)
    scales = gen_scales(rng, wl.wfmt, E, wl.N, wl.K, wl.e8m0)
    ids = gen_ids(rng, wl.M, wl.top_k, E) if routed else None
    V = wl.M * wl.top_k if (routed and wl.x_per_slot) else wl.M
    x, xs = gen_activations(rng, wl.afmt, V, wl.K)
    if wl.kind == "dense":
        codes, scales = codes[0], scales[0]
    inp = Inputs(wl, codes, scales, ids, x, xs)
    if wl.kind == "combine":
        inp.extra["weights"] = gen_route_weights(rng, wl.M, wl.top_k)
    return inp


def gen_route_weights(rng, M, top_k):
    """Router weights of the selected slots: softmax of N(0,1) logits over each
    token's top_k slots, fp32 [M][top_k] (positive, summing to 1)."""
    z = rng.standard_normal((M, top_k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


@dataclass
class GateUpInputs:
    """Host arrays of one fused gate/up call (broadcast token activations)."""
    wl: Workload
    gcodes: np.ndarray
    gscales: np.ndarray
    ucodes: np.ndarray
    uscales: np.ndarray
    ids: np.ndarray
    x: np.ndarray
    xs: np.ndarray | None


def make_gate_up(wl, seed: int | None = None) -> GateUpInputs:
    """Gate and up weights of the same shape and recipe, drawn in the order
    gate codes -> gate scales -> up codes -> up scales -> ids -> activations."""
    if isinstance(wl, str):
        wl = workload(wl)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    gc = gen_codes(rng, wl.wfmt, wl.E, wl.N, wl.K)
    gs = gen_scales(rng, wl.wfmt, wl.E, wl.N, wl.K, wl.e8m0)
    uc = gen_codes(rng, wl.wfmt, wl.E, wl.N, wl.K)
    us = gen_scales(rng, wl.wfmt, wl.E, wl.N, wl.K, wl.e8m0)
    ids = gen_ids(rng, wl.M, wl.top_k, wl.E)
    x, xs = gen_activations(rng, wl.afmt, wl.M, wl.K)
    return GateUpInputs(wl, gc, gs, uc, us, ids, x, xs)


def id_stream(seed: int, calls: int, M: int, top_k: int, E: int) -> np.ndarray:
    """Fresh ids for ``calls`` successive calls: int32 [calls][M][top_k]."""
    rng = np.random.default_rng(seed)
    out = np.empty((calls, M, top_k), np.int32)
    for c in range(calls):
        out[c] = gen_ids(rng, M, top_k, E)
    return out


def disjoint_id_stream(seed: int, calls: int, top_k: int, E: int) -> np.ndarray:
    """Single-token ids that walk a seeded permutation of the experts in
    disjoint top_k-sets, so a whole pass reads every expert once: [calls][1][top_k]."""
    rng = np.random.default_rng(seed)
    out = np.empty((calls, 1, top_k), np.int32)
    perm = rng.permutation(E)
    pos = 0
    for c in range(calls):
        if pos + top_k > E:
            perm = rng.permutation(E)
            pos = 0
        out[c, 0] = perm[pos:pos + top_k]
        pos += top_k
    return out
