// qmv_k_mxfp4m.hip -- dense MXFP4 x bf16 GEMV for 2 to 4 activation vectors
// on the matrix cores.
//
// With one vector per weight row the product is a plain dot, and the VALU
// kernels (qmv_device.hpp) decode and multiply with v_cvt_scalef32_pk_bf16_fp4
// and v_dot2c_f32_bf16.  With four vectors every decoded weight is used four
// times, and the 64 v_dot2c per 32 weights outweigh the 16 conversions and
// the load: measured on MI355X, the dense 4-vector 7168 x 7168 call spent
// about 59% of each CU's cycles issuing VALU.  v_mfma_f32_4x4x4_16b_bf16 does
// those multiplies as 16 independent 4 x 4 x 4 blocks per wave: block b takes
// 4 k-values of 4 weight rows (lanes 4b..4b+3, A) and the same 4 k-values of
// the 4 vectors (the same lanes, B), and accumulates a 4 x 4 (row, vector)
// tile, one column per lane.  The blocks are independent, so each block can
// own its own stretch of K:
//
//   wave  = one quad of 4 consecutive rows;
//   lane  = 4 * blk + r: row r of the quad (A) and vector r (B);
//   step  = 16 units of 32 weights; unit s*16 + blk belongs to block blk.
//
// One load instruction therefore reads 4 rows x 256 contiguous bytes (the
// same coalescing as the VALU kernels with 16 lanes per row), one 4x4x4
// MFMA replaces 16 wave-wide v_dot2c (1024 MACs in about 8 clocks per SIMD
// against 16 x 4 clocks), and the 16 blocks' tiles are summed once at the
// end.  Measured on MI355X: one 4x4x4 bf16 MFMA issues every ~8 clocks per
// SIMD, v_dot2c_f32_bf16 and the fp4 conversions every 4.  The lane layout
// of the instruction (lane 4b + j holds tile column j, rows 0..3 in its four
// accumulator registers; A row i and B column j come from lanes 4b + i and
// 4b + j) was confirmed on the device.
//
// Activations: every workgroup stages the M vectors once into LDS as bf16,
// interleaved by vector within each (unit, dword) so that one ds_read_b128
// hands each lane its own vector's 8 values; the dword index is xor-ed with
// the unit's low bits so the 16 lanes of one read quarter hit 16 distinct
// 16-byte bank groups (the idea of the Strata PR's query swizzle, fitted to
// this record).  A zeroed unit after the last one serves the lanes of a
// partial last step.
//
// E8M0 scales: as in the VALU kernels, when every scale byte of a step is in
// [2, 252] the scale is applied inside the conversion (e2m1 * 2^(s-127) is
// then an exact bf16 normal); otherwise the step is decoded unscaled, its
// tile multiplied by the exactly built 2^(s-127) per row and added.
//
// Every wave covers the whole of K for its quad, so results are bitwise
// reproducible (splitting K over two waves per quad, for more waves per CU,
// measured slower: every workgroup then stages all of x for half the rows).
#include "qmv_device.hpp"

namespace qmv {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Byte offset in LDS of the 16-byte chunk holding bf16 x[j][32u + 8q .. + 8).
__device__ __forceinline__ int m4_off(int u, int q, int j)
{
    return 16 * (u * 16 + (((q ^ (u & 3)) << 2) | j));
}

constexpr int kM4XReg = 8;          // staging chunks per thread held in registers

__device__ __forceinline__ s16x4 pack4(bf16x2 lo, bf16x2 hi)
{
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    const u32x2v v = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    return __builtin_bit_cast(s16x4, v);
}

__device__ __forceinline__ s16x4 pack4u(uint32_t lo, uint32_t hi)
{
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    const u32x2v v = {lo, hi};
    return __builtin_bit_cast(s16x4, v);
}

template <int CTRL>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// 16 bytes at offset off of a resource whose first `lo` bytes are not to be
// read (they precede the scale array) and whose end the hardware range check
// covers: one byte load each, so no byte outside [lo, end) is read.
__device__ __noinline__ u32x4 load16_edge(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t lo)
{
    u32x4 v = {0u, 0u, 0u, 0u};
    for (int b = 0; b < 16; ++b)
        if (off + b >= lo)
            v[b >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, off + b, 0, 0) << (8 * (b & 3));
    return v;
}

// Chunk c of the workgroup's scale bytes: 16-byte loads inside the array,
// byte loads for a chunk that straddles its start or end.
__device__ __forceinline__ u32x4 load_scale_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t lo,
                                                  uint32_t end)
{
    if (off >= lo && off + 16 <= end) return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    return load16_edge(rs, off, lo);
}

template <int WAVES, int CPL>
__global__ __launch_bounds__(64 * WAVES) void qmv_dense4_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int T = 64 * WAVES;
    constexpr int QPW = WAVES;                     // row quads per workgroup
    const int lane = threadIdx.x & 63;
    const int qw = threadIdx.x >> 6;
    const int blk = lane >> 2;
    const int r = lane & 3;                        // row of the quad (A) and vector (B)
    const int quad = blockIdx.x * QPW + qw;
    const int U = a.units;
    const int s0 = 0;
    const int s1 = (U + 15) >> 4;                  // unit steps over K

    // LDS: activations (U + 1 units of 256 B), then this workgroup's rows of
    // E8M0 scales.
    uint8_t *const lds_sc = lds + 256 * (U + 1);

    // 1. activation and scale chunks into registers, before the weight loads
    //    (loads complete in issue order, so the staging must not queue behind
    //    the weight stream).  The scale rows of the workgroup's row quads are
    //    one contiguous byte range: it is read in 16-byte chunks from the
    //    16-byte-aligned address at or below the scale array (its base need
    //    not be aligned), and each step then reads its scale byte from LDS --
    //    measured on MI355X, a 1-byte global load per lane and step cost the
    //    dense 4-vector 7168 x 7168 call 1.7 us of 9.7.
    const int nch = U * 16;                        // (unit, dword, vector) chunks
    const uint32_t smis = (uint32_t)((uintptr_t)a.scales & 15);
    const __amdgpu_buffer_rsrc_t rss = buffer_rsrc(a.scales - smis, a.expert_sb + smis);
    const uint32_t row0 = (uint32_t)blockIdx.x * (QPW * 4);
    const uint32_t sbyte0 = smis + row0 * (uint32_t)a.rsb;        // (N + 3) * rsb < 2^31
    const int snch = (int)(((sbyte0 & 15) + QPW * 4 * a.rsb + 15) >> 4);
    // Every workgroup reads the same activation bytes at the same moment;
    // starting each one at a different 1 KB-aligned point of the vectors
    // spreads the simultaneous requests over the L2 channels.  Workgroups
    // are dealt to the 8 XCDs in turn, so the rotation follows the index
    // within the XCD (blockIdx / 8).
    const int xrot = ((int)((blockIdx.x >> 3) % 16) * (nch >> 4)) & ~63;
    uint4 xr[kM4XReg];
#pragma unroll
    for (int i = 0; i < kM4XReg; ++i) {
        int c = threadIdx.x + i * T + xrot;
        c = c >= nch ? c - nch : c;
        const int j = c & 3;
        xr[i] = make_uint4(0u, 0u, 0u, 0u);
        if (threadIdx.x + i * T < nch && j < a.M)
            xr[i] = *(const uint4 *)(a.x + (size_t)j * a.x_vec_bytes + (c >> 2) * 16);
    }
    const uint32_t send = smis + (uint32_t)a.expert_sb;
    u32x4 sr = {0u, 0u, 0u, 0u};
    if ((int)threadIdx.x < snch)
        sr = load_scale_chunk(rss, (sbyte0 & ~15u) + threadIdx.x * 16, smis, send);

    // 2. code loads of the first CPL steps.  Rows past N and units past the
    //    row's end read at an offset past the buffer: zeros, no traffic.
    //    Every step slot issues its load whether or not the step exists (a
    //    missing step reads past the buffer), so the loads of a wave form a
    //    fixed sequence and each step waits only for its own bytes.
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.codes, a.expert_cb);
    const uint32_t n = (uint32_t)(quad * 4 + r);   // (N + 3) * rcb < 2^32
    const uint32_t oc = n * (uint32_t)a.rcb + blk * 16;
    constexpr uint32_t kPast = 0x80000000u;        // >= every buffer size
    u32x4 wc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int s = s0 + c;
        const bool ok = s < s1 && s * 16 + blk < U;
        wc[c] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? oc + s * 256 : kPast, 0, kStream);
    }

    // 3. activations and scales to LDS; unit U is zeros
#pragma unroll
    for (int i = 0; i < kM4XReg; ++i) {
        int c = threadIdx.x + i * T + xrot;
        c = c >= nch ? c - nch : c;
        if (threadIdx.x + i * T < nch) {
            const int uq = c >> 2;
            *(uint4 *)(lds + m4_off(uq >> 2, uq & 3, c & 3)) = xr[i];
        }
    }
    if ((int)threadIdx.x < snch) *(u32x4 *)(lds_sc + 16 * threadIdx.x) = sr;
    for (int c0 = threadIdx.x + kM4XReg * T; c0 < nch; c0 += T) {
        const int c = c0 + xrot >= nch ? c0 + xrot - nch : c0 + xrot;
        const int j = c & 3, uq = c >> 2;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (j < a.M) v = *(const uint4 *)(a.x + (size_t)j * a.x_vec_bytes + uq * 16);
        *(uint4 *)(lds + m4_off(uq >> 2, uq & 3, j)) = v;
    }
    for (int c = threadIdx.x + T; c < snch; c += T)
        *(u32x4 *)(lds_sc + 16 * c) = load_scale_chunk(rss, (sbyte0 & ~15u) + c * 16, smis, send);
    if (threadIdx.x < 16)
        *(uint4 *)(lds + 16 * (U * 16 + (int)threadIdx.x)) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();

    // 4. steps: decode + 8 MFMAs per step, next loads CPL steps ahead
    int xo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xo[q] = 64 * (q ^ (blk & 3)) + 16 * r;
    const uint8_t *const lds_srow = lds_sc + (sbyte0 & 15) + (qw * 4 + r) * a.rsb + blk;
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
    for (int sb = s0; sb < s1; sb += CPL) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int s = sb + c;
            if (s < s1) {
                const bool ok = s * 16 + blk < U;
                const uint8_t *xp = lds + min(4096 * s + 256 * blk, 256 * U);
                uint4 xq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) xq[q] = lds_read16(xp + xo[q]);
                const uint32_t sbyte = ok ? (uint32_t)lds_srow[s * 16] : 127u;
                const uint32_t cw[4] = {wc[c].x, wc[c].y, wc[c].z, wc[c].w};
                if (__all((sbyte - 2u) <= 250u)) {
                    const float sc = __uint_as_float(sbyte << 23);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const s16x4 a0 = pack4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 0),
                                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 1));
                        const s16x4 a1 = pack4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 2),
                                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 3));
                        acc0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a0, pack4u(xq[q].x, xq[q].y), acc0, 0, 0, 0);
                        acc1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a1, pack4u(xq[q].z, xq[q].w), acc1, 0, 0, 0);
                    }
                } else {
                    f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const s16x4 a0 = pack4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 0),
                                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 1));
                        const s16x4 a1 = pack4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 2),
                                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 3));
                        t = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a0, pack4u(xq[q].x, xq[q].y), t, 0, 0, 0);
                        t = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a1, pack4u(xq[q].z, xq[q].w), t, 0, 0, 0);
                    }
                    // t[v] is row v of the quad; its scale byte sits in lane 4 * blk + v
                    acc0[0] = __builtin_fmaf(t[0], e8m0_f32(quad_bcast<0x00>(sbyte)), acc0[0]);
                    acc0[1] = __builtin_fmaf(t[1], e8m0_f32(quad_bcast<0x55>(sbyte)), acc0[1]);
                    acc0[2] = __builtin_fmaf(t[2], e8m0_f32(quad_bcast<0xAA>(sbyte)), acc0[2]);
                    acc0[3] = __builtin_fmaf(t[3], e8m0_f32(quad_bcast<0xFF>(sbyte)), acc0[3]);
                }
            }
            const int sn = s + CPL;
            const bool okn = sn < s1 && sn * 16 + blk < U;
            wc[c] = __builtin_amdgcn_raw_buffer_load_b128(rc, okn ? oc + sn * 256 : kPast, 0, kStream);
        }
    }

    // 5. sum the 16 blocks' tiles (butterfly over lane bits 2..5: every lane
    //    of a column ends with the same bits)
    f32x4 acc = acc0 + acc1;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int m = 4; m < 64; m <<= 1) acc[v] += __shfl_xor(acc[v], m);
    }
    // lane 4 * v + j (blk = v < 4) owns row 4 * quad + v of vector j
    const float val = blk == 0 ? acc[0] : blk == 1 ? acc[1] : blk == 2 ? acc[2] : acc[3];
    const int row = quad * 4 + blk;
    if (blk < 4 && r < a.M && row < a.N) a.y[r * a.N + row] = val;
}

// [4 waves, 8 waves], 4 unit steps in flight
extern const void *const kTableDense4[2];
const void *const kTableDense4[2] = {(const void *)&qmv_dense4_kernel<4, 4>,
                                     (const void *)&qmv_dense4_kernel<8, 4>};

}  // namespace qmv
