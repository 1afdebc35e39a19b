/*
 * qmv.h -- C ABI of libqmv.so: block-quantized GEMV for MoE expert
 * projections on AMD Instinct MI355X (gfx950): decode (1 to 4 tokens) and
 * many-token calls (a prefill chunk or a wide verify batch).
 *
 * The library computes, for every output it is asked for,
 *
 *     y = sum_k  w(k) * x(k)
 *
 * where w is a dequantized weight (code value times its block scale) and x a
 * dequantized activation.  The operation is the expert-gathered matrix-vector
 * product that MoE decode spends its time in: mlxcel issue #2178 "add an
 * mxfp4 arm to the warp-shared gather_qmv kernel for gpt-oss decode"
 * (Problem / Background and Proposed Solution), lucebox-hub PR #21
 * "optimize ROCMFPX fp3/fp2 MMVQ on RDNA" (Changes) and geo-lucebox PR #31
 * "DS4 H200: rocmfp2_mix MoE matvec 3.31x" (Why this kernel).
 *
 * ------------------------------------------------------------------ formats
 * Weights are row-major and planar: per expert, N rows of K weights; codes and
 * scales are separate arrays.  A dense call has no expert dimension.
 *
 *   QMV_W_MXFP4  codes  uint8 [E][N][K/2]   two e2m1 nibbles per byte; weight
 *                                            k is the low nibble of byte k/2
 *                                            when k is even, the high nibble
 *                                            when k is odd.
 *                scales uint8 [E][N][K/32]  E8M0: byte s means 2^(s-127),
 *                                            s = 255 is NaN.
 *                (mlxcel issue #2178: w_row[k/2], group k/32, E8M0 uint8
 *                scales.)
 *   QMV_W_CB2    codes  uint8 [E][N][K/4]   2-bit codes, weight k in bits
 *                                            2(k%4)..2(k%4)+1 of byte k/4;
 *                                            code c means c - 1.5, i.e. the
 *                                            codebook {-1.5,-0.5,0.5,1.5}.
 *                scales fp16  [E][N][K/32]  one scale per 32 weights.
 *   QMV_W_CB3    codes  uint8 [E][N][3K/8]  3-bit codes in one little-endian
 *                                            bit stream per row: weight k is
 *                                            stream bits 3k..3k+2 (bit 3k least
 *                                            significant; stream bit b is bit
 *                                            b%8 of byte b/8).  Code c means
 *                                            {0,.5,1,2,-3,-.5,-1,-2}[c].
 *                scales fp16  [E][N][K/16]  one scale per 16-weight
 *                                            half-block.
 *                (lucebox-hub PR #21: the fp2 {-1,0,1,2} and fp3
 *                {0,1,2,4,0,-1,-2,-4} tables and the half-block scale split;
 *                these codebooks are those tables minus 0.5, and times 0.5
 *                with the second zero taken as -3.)
 *
 * Activations:
 *   QMV_A_BF16   x   bf16 [V][K], x_scales unused (pass NULL).
 *   QMV_A_Q8B32  x   int8 [V][K] with x_scales fp16 [V][K/32]: activation k
 *                    is x[k] * x_scales[k/32] (the q8_1 blocks of lucebox-hub
 *                    PR #21).  A 3-bit half-block uses the scale of the
 *                    32-block that contains it.
 *   QMV_A_BF16_Q8 x  bf16 [V][K], x_scales unused (pass NULL): the kernel
 *                    quantizes each 32-block of x to the Q8B32 form while
 *                    staging it and then computes exactly as for Q8B32 --
 *                    the separate activation-quantize launch of the pages
 *                    (geo-lucebox PR #31, "What is now hot": quantize_q8_1)
 *                    folded into the matvec.  Per block, in fp32:
 *                      d   = max_k |x[k]| / 127,
 *                      d16 = d rounded to fp16 (nearest even), the scale;
 *                      q[k] = clamp(rint(x[k] * (1 / d16)), -127, 127),
 *                            ties to even; q = 0 where d16 is 0 or Inf.
 *                    Activations must be finite.  The pages name the
 *                    quantizer but print no formula: this is a reading,
 *                    and no page value pins it (parity unpinned against
 *                    the pages; the CPU oracle implements the same
 *                    reading).
 * Supported pairs: (MXFP4, BF16), (MXFP4, Q8B32), (CB2, Q8B32), (CB3, Q8B32),
 * (CB2, BF16_Q8), (CB3, BF16_Q8).  With (MXFP4, Q8B32) every 32-weight block
 * shares one E8M0 weight scale and one activation scale (both are per 32 of
 * k), and the block's sum of e2m1 x int8 products is formed exactly (it is
 * the integer dot product of the 2*e2m1 values with q, times the weight
 * scale / 2) before the activation scale multiplies it.
 *
 * ------------------------------------------------------------- conventions
 * Ownership: every pointer is a device pointer owned by the caller.  A call
 * only enqueues work on `stream` and returns: the library never copies to
 * the host or synchronizes.  It reads only the extents above and writes only
 * y.  The one device memory it takes for itself is the temporary of a
 * combine call with more than 4 tokens (qmv_gather_moe_combine), allocated
 * and freed in stream order on `stream` from a memory pool the library
 * creates per device at first use and keeps (with the memory it has handed
 * out) until the process ends.  Calls may be made concurrently from several
 * host threads and streams.
 *
 * Alignment: codes 16 bytes (8 for CB2 when K % 64 != 0), x 16 bytes,
 * scales, x_scales, expert ids and y 4 bytes.
 *
 * Limits: M >= 1, 1 <= top_k <= 16, K % 32 == 0, 32 <= K <= 16384, N >= 1,
 * E >= 1, M * top_k * N < 2^31.  With M > 4 (a prefill chunk or a wide
 * verify batch), on every entry point and format pair: at most 8192
 * (token, slot) pairs (M for a dense call, M * top_k otherwise) and, for
 * the routed calls, E <= 1023.
 *
 * Errors: arguments are checked on the host before anything is launched; on
 * a failed check the call returns the status, launches nothing and leaves y
 * untouched.  No check needs a device synchronization.  QMV_EHIP (the
 * runtime refused a launch) can come after earlier launches of the same
 * call have run: a dense (MXFP4, BF16) call with 5 to 8 vectors, and a
 * gather or gate/up call with 5 to 64 tokens and fewer than two (token,
 * slot) pairs per expert (M * top_k < 2 E), are one launch per group of up
 * to 4 vectors or tokens, so y may then hold the rows of the groups before
 * the failing one.  A combine call with more than 4 tokens writes y only in
 * its last launch.  Every other call is one launch.  An expert
 * id outside [0, E) is not an error: that (token, slot) output row is
 * written with zeros (mlxcel issue #2178, Implementation Notes, Edge cases).
 *
 * Determinism: results are bitwise identical from run to run (fixed
 * reduction order, no atomics).
 */
#ifndef QMV_H
#define QMV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QMV_W_MXFP4 = 0, QMV_W_CB2 = 1, QMV_W_CB3 = 2 } qmv_wfmt_t;
typedef enum { QMV_A_BF16 = 0, QMV_A_Q8B32 = 1, QMV_A_BF16_Q8 = 2 } qmv_afmt_t;

typedef enum {
    QMV_OK = 0,
    QMV_EINVAL = 1,        /* null or misaligned pointer, size <= 0 */
    QMV_EUNSUPPORTED = 2,  /* M, top_k or K out of range; unsupported format pair */
    QMV_EHIP = 3,          /* the HIP runtime refused the launch */
    QMV_ESCRATCH = 4       /* the call needs more than QMV_NOALLOC_SCRATCH_BYTES of
                              temporary (qmv_gather_moe_combine_noalloc only) */
} qmv_status_t;

/* The fixed device temporary of qmv_gather_moe_combine_noalloc, per GPU. */
#define QMV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * Dense GEMV: y[m][n] = sum_k w(n, k) * x(m, k) for m < M, n < N.
 *   w_codes, w_scales  one weight matrix, layouts above with E omitted
 *   x, x_scales        M activation vectors ([M][K], [M][K/32])
 *   y                  fp32 [M][N]
 * This is the gather below with one expert, top_k = 1 and ids all 0.
 * With (MXFP4, BF16), 5 <= M <= 8 runs as groups of up to 4 vectors on the
 * 4-vector kernel (one launch per group), 9 <= M <= 64 in one launch of
 * 32-row tiles whose K is split over the waves of a workgroup (one or two
 * 32-vector column fragments), and M > 64 on the batched matrix-core kernel
 * described under qmv_gather_moe; 2-bit and 3-bit
 * weights with int8 (or in-kernel quantized bf16) activations and M >= 8 on
 * the int8 matrix-core kernel;
 * every other M > 4 call on the grouped kernel.
 */
qmv_status_t qmv_dense(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales,
                       qmv_afmt_t afmt, const void *x, const void *x_scales,
                       float *y, int M, int N, int K, hipStream_t stream);

/*
 * Expert-gathered GEMV (MoE decode):
 *   y[t][j][n] = sum_k w(e, n, k) * x(t, j, k)     e = expert_ids[t][j]
 *   y[t][j][n] = 0                                  if e is outside [0, E)
 * for t < M tokens, j < top_k slots and n < N rows.
 *   expert_ids  int32 [M][top_k] in device memory
 *   x_per_slot  0: x is [M][K] and token t's vector feeds all its slots;
 *               1: x is [M][top_k][K], one vector per (token, slot), as for a
 *                  down projection whose input differs per expert.
 *   y           fp32 [M][top_k][N]
 * Each distinct expert's weights are streamed from memory once per call and
 * applied to every activation vector routed to it (up to four per pass).
 * With M > 4 (the expert-batched product that prefill takes once many
 * tokens share each expert: mlxcel issue #2178, "Problem / Background"; the
 * verify-batch matmul of lucebox-hub PR #19, "Depends on") every workgroup
 * lists the (token, slot) pairs of its expert in LDS (no host sort, no
 * workspace) and one launch computes the call:
 *   (MXFP4, BF16) with M * top_k >= 2 E: each expert's rows against all of
 *     its vectors, up to 128 at a time, on the 32x32x16 bf16 matrix cores;
 *   (CB2 with K % 64 == 0 or CB3, Q8B32 or BF16_Q8) with M * top_k >= 2 E:
 *     exact int32 block sums on the int8 4x4x4 matrix cores, up to 16
 *     (2-bit) or 12 (3-bit) vectors per staged chunk (bf16 x quantized
 *     while staged), each workgroup a run of (expert, row tile) items of
 *     equal cost with the experts' vector counts weighed in;
 *   at most 64 tokens with fewer than two pairs per expert: groups of up to
 *     4 tokens on the decode kernels, one launch per group;
 *   every other call: the decode kernels' own multiply-adds in one launch,
 *     four of an expert's vectors at a time.
 * The result is the same definition within the same tolerance (bit-exact
 * where the arithmetic is exact) and bitwise repeatable.
 */
qmv_status_t qmv_gather_moe(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales, int E,
                            const int32_t *expert_ids, int M, int top_k,
                            qmv_afmt_t afmt, const void *x, const void *x_scales,
                            int x_per_slot, float *y, int N, int K, hipStream_t stream);

/*
 * Fused gate/up expert projection with the SwiGLU activation:
 *   y[t][j][n] = silu(g) * u,   silu(g) = g / (1 + e^-g),
 *   g = sum_k w_gate(e, n, k) * x(t, k),   u = sum_k w_up(e, n, k) * x(t, k)
 * with e = expert_ids[t][j] (0 where e is outside [0, E)).  Both projections
 * use the weight format and layout above ([E][N][...] each) and the token's
 * activation vector x[M][K]; y is fp32 [M][top_k][N].  One launch streams both
 * weight tensors of the routed experts -- the gate and up expert projections
 * that geo-lucebox PR #31 "DS4 H200: rocmfp2_mix MoE matvec" (Why this kernel)
 * computes in one matvec kernel -- and hands the down projection its input
 * directly.  Arguments, limits and errors as qmv_gather_moe (M > 4
 * included: (MXFP4, BF16) with M * top_k >= 2 E on the batched matrix-core
 * kernel with a gate and an up fragment per output fragment, every other
 * call on the grouped kernel); silu is evaluated in fp32.
 */
qmv_status_t qmv_gather_moe_swiglu(qmv_wfmt_t wfmt, const void *gate_codes, const void *gate_scales,
                                   const void *up_codes, const void *up_scales, int E,
                                   const int32_t *expert_ids, int M, int top_k,
                                   qmv_afmt_t afmt, const void *x, const void *x_scales,
                                   float *y, int N, int K, hipStream_t stream);

/*
 * Down (expert output) projection with the router-weighted top-k combine:
 *   y[t][n] = sum_j  route_weights[t][j] * g(t, j, n)      for t < M, n < N
 *   g(t, j, n) = sum_k w(e, n, k) * x(t, j, k),  e = expert_ids[t][j]
 *   g(t, j, n) = 0                               if e is outside [0, E)
 * The per-slot gather above followed by the weighted sum over each token's
 * slots: the result an MoE layer adds to the residual stream.
 * The pages count gate, up and down expert calls per decoded token (mlxcel
 * issue #2178, Problem / Background) and time the down projection's 3-bit
 * matvec on its own (lucebox-hub PR #21, Summary); the combine is the
 * standard top-k mixture sum that consumes it.
 *   route_weights  fp32 [M][top_k] in device memory (4-byte aligned)
 *   x_per_slot     1: x is [M][top_k][K], the activated gate/up output of
 *                     each (token, slot) -- the usual down-projection input;
 *                  0: x is [M][K] for every slot of a token.
 *   y              fp32 [M][N], overwritten (not accumulated into).
 * The slots of a token are summed in slot order, each slot one fused
 * multiply-add onto a sum that starts at zero; results are bitwise
 * reproducible.  An out-of-range id contributes route_weights[t][j] * 0.
 * Up to 4 tokens: one launch, a workgroup per token and row tile, each lane
 * carrying one row of four of the token's slots.  More than 4 tokens: the
 * gather of qmv_gather_moe (same kernels and routing) writes every (token,
 * slot) row to a temporary of M * top_k * N floats from the library's pool
 * (see Ownership; it can be recorded into a HIP graph as the graph's own
 * allocation), and a second launch forms the slot sums from it; an
 * allocation the pool refuses is QMV_EHIP before anything is launched.
 * Weights, scales and activations, limits and errors as qmv_gather_moe;
 * route_weights may be signed or sum to zero; a null or misaligned
 * route_weights is QMV_EINVAL.
 */
qmv_status_t qmv_gather_moe_combine(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales,
                                    int E, const int32_t *expert_ids, const float *route_weights,
                                    int M, int top_k, qmv_afmt_t afmt, const void *x,
                                    const void *x_scales, int x_per_slot, float *y, int N, int K,
                                    hipStream_t stream);

/*
 * qmv_gather_moe_combine without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture that must record no
 * allocation, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results (bit for bit), limits and errors as
 * qmv_gather_moe_combine, except where the temporary of a call with more
 * than 4 tokens lives: in a fixed array inside the library's device code,
 * QMV_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which each GPU the library
 * runs on holds from the library's load until the process ends.  A call with
 * more than 4 tokens needs M * top_k * N * 4 bytes of it; a larger one
 * returns QMV_ESCRATCH, launches nothing and leaves y untouched (the
 * allocating entry point takes it).  Up to 4 tokens use no temporary.
 * Every call on one GPU uses that GPU's one array, and each call overwrites
 * what it reads back, so nothing needs clearing between calls; but calls
 * whose work overlaps on one GPU (other streams, other host threads) race on
 * it: the caller orders them, e.g. on one stream.  The first call on a device
 * looks up the array's device address (hipGetSymbolAddress), with that device
 * made current for the lookup.
 */
qmv_status_t qmv_gather_moe_combine_noalloc(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales,
                                            int E, const int32_t *expert_ids, const float *route_weights,
                                            int M, int top_k, qmv_afmt_t afmt, const void *x,
                                            const void *x_scales, int x_per_slot, float *y, int N, int K,
                                            hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char *qmv_strerror(qmv_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
