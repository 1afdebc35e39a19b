// qmv_k_cbm.hip -- 2-bit and 3-bit codebook weights against int8 activations
// with more than 4 vectors per expert, on the int8 matrix cores.
//
// The pages' verify batch runs the low-bit weights through a batched matmul
// (lucebox-hub PR #21 "optimize ROCMFPX fp3/fp2 MMVQ on RDNA", Depends on:
// the batched ROCmFPX MMQ; lucebox-hub PR #19 "speed up fp3 ROCMFPX matvec",
// Depends on: the fp3 verify-batch matmul).  Its arithmetic is the decode
// path's: per 32-weight block (16 for 3-bit scales) an exact integer sum of
// code value x int8 activation, then the block's fp16 weight scale and fp16
// activation scale.  With several vectors per weight row those integer sums
// are a small matrix product, and v_mfma_i32_4x4x4_16b_i8 forms them: 16
// independent 4 x 4 x 4 blocks per wave, block b taking 4 k-values of 4
// weight rows (lanes 4b..4b+3, A) and the same 4 k-values of 4 vectors (the
// same lanes, B), accumulating a 4 (row) x 4 (vector) int32 tile, column j
// in lane 4b + j (layout confirmed on the device).  Each block owns its own
// stretch of K, as in the dense 4-vector MXFP4 kernel:
//
//   wave = one quad of 4 consecutive weight rows;
//   lane = 4 * blk + r: row r of the quad (A) and vector r of a group (B);
//   step = 16 units; unit 16 s + blk belongs to block blk.
//
// A unit is 64 weights for 2-bit codes (16 bytes, two 32-blocks) and 32 for
// 3-bit codes (12 bytes, two 16-weight half-blocks); one load instruction
// reads 4 rows x 256 (192) contiguous bytes.  Each block's int32 tile is
// read after the k-values of one scale block, scaled and added into fp32:
//
//   2-bit: S = sum((2c - 3) q) (the codebook is c - 1.5; a v_perm_b32 LUT
//          turns the codes into the int8 A operand 2c - 3),
//          acc += S * (ws * xs / 2);
//   3-bit: S_h = sum(v * q) per half-block (v = twice the codebook value,
//          from a v_perm_b32 LUT), acc += (ws_0 S_0 + ws_1 S_1) * xs / 2;
//
// the same factors as the decode kernels, so at unit scales every value is
// an exact integer multiple of 1/2 and the result is bit-exact.  The MFMA
// replaces 4 v_dot4 per 16 weights and vector; what remains on the VALU is
// the decode (shared by all vector groups) and 4 multiply-adds per block,
// row and vector.
//
// Vectors: an expert's vectors are taken in chunks of up to 4 * NVG (NVG
// groups of 4); a chunk is staged into LDS once per workgroup and used for
// every row tile of the workgroup's run of that expert.  LDS per unit: the
// NVG groups' records one after another (so a group's place is a constant
// offset from its unit's), each the four vectors' activations in the order
// the selectors need (chunk (q, j) at a swizzled place within the record, so
// the 16 lanes of a read quarter hit distinct banks: gm_chunk_off); after all
// units, the side data xs/2 per 32-block of each vector, in the same order.
// Units past K and vectors past the chunk are staged as zeros.
//
// Work: (expert slot, row tile) items as in the grouped decode-MAC kernel
// (qmv_device.hpp): the y-th selected expert from a bitmap of the ids, the
// expert's (token, slot) pairs listed in index order, contiguous runs of
// items per workgroup, of equal cost when the vector counts are weighed in
// (gm_weighted_run).
#include "qmv_device.hpp"

namespace qmv {

typedef int i32x4g __attribute__((ext_vector_type(4)));

// 2-bit code c (bytes 0..3 of the selector) -> int8 2c - 3: {-3, -1, 1, 3}
constexpr uint32_t kCb2Lut2 = 0x0301FFFDu;

// lane 4 * (lane / 4) + I of v, for every lane (DPP quad permute)
template <int I>
__device__ __forceinline__ uint32_t quad_lane(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, I * 0x55, 0xF, 0xF, false);
}

template <int F> struct GmFmt;
// CH: 16-byte activation chunks per unit and vector; SIDE: side bytes per
// unit and vector; CB: code bytes per unit.
template <> struct GmFmt<kCB2> { static constexpr int W = 64, CH = 4, SIDE = 8, CB = 16; };
template <> struct GmFmt<kCB3> { static constexpr int W = 32, CH = 2, SIDE = 4, CB = 12; };

// Side-data bytes per unit: NVG groups of 4 vectors, and for 2-bit weights
// with 4 groups 32 bytes of padding, so that the 4 units a read quarter
// takes (32 bytes of one group each) start 160 bytes apart and fall on
// distinct banks (128 bytes apart, units u and u + 2 would share them).
template <int F, int NVG>
constexpr int gm_side_stride()
{
    return NVG * 4 * GmFmt<F>::SIDE + (F == kCB2 && NVG == 4 ? 32 : 0);
}

// LDS bytes of the staged vector groups over Up units.
template <int F, int NVG>
__device__ __forceinline__ int gm_stage_bytes(int Up)
{
    return Up * (NVG * GmFmt<F>::CH * 64 + gm_side_stride<F, NVG>());
}

// Activation chunk (q, j) of group g at unit u (units of NVG records).  The
// 16 lanes of a read quarter take units u .. u + 3 (one chunk q each, four
// vectors j): the chunk position within a record is xor-ed with the unit's
// bits above the unit's share of a 256-byte bank row, so those 16 chunks
// fall on 16 distinct 16-byte bank groups (2-bit: 256-byte records,
// q ^ (u & 3); 3-bit: 128-byte records, q ^ ((u >> 1) & 1), units 128 or
// 384 bytes apart for NVG 1 or 3; with NVG 2 two of the four units share
// a half row, a 2-way conflict).
template <int F, int NVG>
__device__ __forceinline__ int gm_chunk_off(int u, int g, int q, int j)
{
    constexpr int CH = GmFmt<F>::CH;
    const int pos = CH == 4 ? q ^ (u & 3) : q ^ ((u >> 1) & 1);
    return 16 * ((u * NVG * CH + pos) * 4 + j) + g * (CH * 64);
}

// Side data of vector j of group g at unit u (past the Up units' records).
template <int F, int NVG>
__device__ __forceinline__ int gm_side_off(int Up, int u, int g, int j)
{
    constexpr int CH = GmFmt<F>::CH, SIDE = GmFmt<F>::SIDE;
    return Up * NVG * CH * 64 + u * gm_side_stride<F, NVG>() + SIDE * j + g * (4 * SIDE);
}

// 3-bit half-block (16 codes: 6 bytes at byte offset OFF of hi:lo) -> four
// dwords of int8 values, twice the codebook, in the cb3_xorder order.
template <int OFF>
__device__ __forceinline__ uint4 cb3_decode_half(uint32_t hi, uint32_t lo)
{
    constexpr uint32_t A0 = OFF, A1 = OFF + 1, A2 = OFF + 2, B0 = OFF + 3, B1 = OFF + 4, B2 = OFF + 5;
    const uint32_t q0 = perm(hi, lo, A0 | (B0 << 8) | (A0 << 16) | (B0 << 24));
    const uint32_t q1 = perm(hi, lo, A1 | (B1 << 8) | (A1 << 16) | (B1 << 24));
    const uint32_t q2 = perm(hi, lo, A2 | (B2 << 8) | (A2 << 16) | (B2 << 24));
    const uint32_t q3 = perm(hi, lo, A0 | (A1 << 8) | (B0 << 16) | (B1 << 24));
    const uint32_t q4 = perm(hi, lo, A1 | (A2 << 8) | (B1 << 16) | (B2 << 24));
    const uint32_t s0 = pk_shr<0, 3>(q0) & 0x07070707u;
    const uint32_t s1 = pk_shr<1, 4>(q1) & 0x07070707u;
    const uint32_t s2 = pk_shr<2, 5>(q2) & 0x07070707u;
    const uint32_t s3 = (pk_shr<6, 6>(q3) & 0x00070007u) | ((pk_shr<7, 7>(q4) & 0x00070007u) << 8);
    uint4 o;
    o.x = perm(kCb3LutHi, kCb3LutLo, s0);
    o.y = perm(kCb3LutHi, kCb3LutLo, s1);
    o.z = perm(kCb3LutHi, kCb3LutLo, s2);
    o.w = perm(kCb3LutHi, kCb3LutLo, s3);
    return o;
}

// Stage vectors [v0, v0 + cc) of the list (pair indices in `pairs`, or the
// vector indices themselves for a dense call) as ng groups of 4.  Q: the
// activations are bf16 and each 32-block is quantized here to int8 and an
// fp16 scale (quant_q8_block, the decode kernels' staging quantizer).
template <int F, int THREADS, bool Q, int NVG>
__device__ __forceinline__ void gm_stage(const Args &a, uint8_t *lds, const uint16_t *pairs, bool gather,
                                         int v0, int cc, int ng, int Up)
{
    constexpr int W = GmFmt<F>::W;
    const int U = a.units;
    const int items = ng * 4 * Up;                   // (vector slot, unit)
    for (int i = threadIdx.x; i < items; i += THREADS) {
        // vector j of group g at unit u, j fastest and then u: the 16 lanes
        // of a write quarter store 4 units x 4 vectors, as a read quarter
        // reads them, on distinct banks
        const int j = i & 3, t = i >> 2;
        const int g = t / Up, u = t - g * Up;
        const int m = 4 * g + j;                    // vector slot m of the chunk
        uint4 c0 = make_uint4(0u, 0u, 0u, 0u), c1 = c0, c2 = c0, c3 = c0;
        float xs0 = 0.0f, xs1 = 0.0f;
        if (m < cc && u < U) {
            const int p = gather ? (int)pairs[v0 + m] : v0 + m;
            const int vec = gather && !a.x_per_slot ? p / a.top_k : p;
            if constexpr (Q) {
                // 32 bf16 (64 bytes) per block
                const uint8_t *xp = a.x + (size_t)vec * a.x_vec_bytes + (size_t)u * W * 2;
                uint4 r[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) r[k] = *(const uint4 *)(xp + 16 * k);
                xs0 = 0.5f * (float)__builtin_bit_cast(_Float16, (uint16_t)quant_q8_block(r, c0, c1));
                if constexpr (F == kCB2) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) r[k] = *(const uint4 *)(xp + 64 + 16 * k);
                    xs1 = 0.5f * (float)__builtin_bit_cast(_Float16, (uint16_t)quant_q8_block(r, c2, c3));
                }
            } else {
                const uint8_t *xp = a.x + (size_t)vec * a.K + (size_t)u * W;
                const uint16_t *sp = a.xs + (size_t)vec * (a.K / 32) + (size_t)u * W / 32;
                c0 = *(const uint4 *)xp;
                c1 = *(const uint4 *)(xp + 16);
                xs0 = 0.5f * (float)__builtin_bit_cast(_Float16, sp[0]);
                if constexpr (F == kCB2) {
                    c2 = *(const uint4 *)(xp + 32);
                    c3 = *(const uint4 *)(xp + 48);
                    xs1 = 0.5f * (float)__builtin_bit_cast(_Float16, sp[1]);
                }
            }
        }
        if constexpr (F == kCB2) {
            *(uint4 *)(lds + gm_chunk_off<F, NVG>(u, g, 0, j)) = cb2_xorder(c0);
            *(uint4 *)(lds + gm_chunk_off<F, NVG>(u, g, 1, j)) = cb2_xorder(c1);
            *(uint4 *)(lds + gm_chunk_off<F, NVG>(u, g, 2, j)) = cb2_xorder(c2);
            *(uint4 *)(lds + gm_chunk_off<F, NVG>(u, g, 3, j)) = cb2_xorder(c3);
            *(uint2 *)(lds + gm_side_off<F, NVG>(Up, u, g, j)) = make_uint2(__float_as_uint(xs0), __float_as_uint(xs1));
        } else {
            *(uint4 *)(lds + gm_chunk_off<F, NVG>(u, g, 0, j)) = cb3_xorder(c0);
            *(uint4 *)(lds + gm_chunk_off<F, NVG>(u, g, 1, j)) = cb3_xorder(c1);
            *(float *)(lds + gm_side_off<F, NVG>(Up, u, g, j)) = xs0;
        }
    }
}

// fp16 halves of a packed scale pair, widened where they are used: as an
// operand of a multiply-add the compiler folds the widening into it
// (v_fma_mix_f32), and a product written as fma(w, x, 0) is the product
// rounded once, as w * x is (a zero may differ in sign only).
__device__ __forceinline__ float h16_lo(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
}
__device__ __forceinline__ float h16_hi(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

// One step (16 units, one per block) of NG vector groups: the int32 tiles
// of each scale block, scaled into acc[g] (rows 0..3 of the quad, vector j
// of group g).  The groups' MFMA chains are interleaved, so NG independent
// accumulators are in flight.
template <int F, int NG, int NVG>
__device__ __forceinline__ void gm_step(const uint8_t *lds, int Up, int u, int j,
                                        const uint32_t (&A)[16], const uint32_t (&sw)[4],
                                        float (&acc)[NG][4])
{
    if constexpr (F == kCB2) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            uint32_t xv[NG][8];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint4 x0 = lds_read16(lds + gm_chunk_off<F, NVG>(u, g, 2 * b, j));
                const uint4 x1 = lds_read16(lds + gm_chunk_off<F, NVG>(u, g, 2 * b + 1, j));
                xv[g][0] = x0.x; xv[g][1] = x0.y; xv[g][2] = x0.z; xv[g][3] = x0.w;
                xv[g][4] = x1.x; xv[g][5] = x1.y; xv[g][6] = x1.z; xv[g][7] = x1.w;
            }
            i32x4g d[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) d[g] = (i32x4g){0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    d[g] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)A[8 * b + t], (int)xv[g][t], d[g], 0, 0, 0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float xsh = *(const float *)(lds + gm_side_off<F, NVG>(Up, u, g, j) + 4 * b);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ws = b == 0 ? h16_lo(sw[i]) : h16_hi(sw[i]);
                    acc[g][i] = __builtin_fmaf((float)d[g][i], __builtin_fmaf(ws, xsh, 0.0f), acc[g][i]);
                }
            }
        }
    } else {
        uint32_t xv[NG][8];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint4 x0 = lds_read16(lds + gm_chunk_off<F, NVG>(u, g, 0, j));
            const uint4 x1 = lds_read16(lds + gm_chunk_off<F, NVG>(u, g, 1, j));
            xv[g][0] = x0.x; xv[g][1] = x0.y; xv[g][2] = x0.z; xv[g][3] = x0.w;
            xv[g][4] = x1.x; xv[g][5] = x1.y; xv[g][6] = x1.z; xv[g][7] = x1.w;
        }
        i32x4g d0[NG], d1[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) d0[g] = d1[g] = (i32x4g){0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                d0[g] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)A[t], (int)xv[g][t], d0[g], 0, 0, 0);
                d1[g] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)A[4 + t], (int)xv[g][4 + t], d1[g], 0, 0, 0);
            }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float xsh = *(const float *)(lds + gm_side_off<F, NVG>(Up, u, g, j));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float t = __builtin_fmaf(h16_hi(sw[i]), (float)d1[g][i],
                                               __builtin_fmaf(h16_lo(sw[i]), (float)d0[g][i], 0.0f));
                acc[g][i] = __builtin_fmaf(t, xsh, acc[g][i]);
            }
        }
    }
}

// v's bits moved under DPP control CTRL into the lanes of the 4-lane banks
// BANKS of every 16-lane row; the other lanes keep `old`.
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_into(float old, float v)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xF, BANKS, false));
}

// The sum over the wave's 16 blocks (lane bits 2..5) of a block's 4 x 4 tile,
// v[i] = row i of the lane's vector (lane bits 0..1).  A reduce-scatter over
// lane bits 3 and 2 -- each lane keeps the rows its side of the pair will
// own, and adds its partner's copy of them (DPP within the 16-lane row; a
// row rotation by n hands lane l the value of lane l - n) -- then a sum over
// bits 4 and 5.  Lane 4 blk + j ends with row blk & 3 of vector j, summed in
// a fixed order.  Against a 4-level shuffle butterfly over all four rows:
// about 100 fewer instructions per tile, C8 686-697 -> 646-656 us on MI355X.
__device__ __forceinline__ float gm_tile_sum(const float (&v)[4])
{
    constexpr int kId = 0xE4, kRor4 = 0x124, kRor8 = 0x128, kRor12 = 0x12C;
    float t[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        // bit 3: banks 0-1 keep row i, banks 2-3 row i + 2; partner l ^ 8
        const float keep = dpp_into<kId, 0x3>(v[i + 2], v[i]);
        const float send = dpp_into<kId, 0x3>(v[i], v[i + 2]);
        t[i] = keep + dpp_into<kRor8, 0xF>(0.0f, send);
    }
    // bit 2: banks 0 and 2 keep t[0] (rows 0, 2), banks 1 and 3 t[1]; the
    // partner is l + 4 (bit 2 clear) or l - 4 (set)
    const float keep = dpp_into<kId, 0x5>(t[1], t[0]);
    const float send = dpp_into<kId, 0x5>(t[0], t[1]);
    float s = keep + dpp_into<kRor4, 0xA>(dpp_into<kRor12, 0x5>(0.0f, send), send);
    s += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(s), 0x401F));   // lane ^ 16
    s += __shfl_xor(s, 32);
    return s;
}

// Codes and scales of flattened step f = (tile ti, step s): this lane's row
// of the wave's quad in row tile tile0 + ti, unit 16 s + blk.
template <int F>
__device__ __forceinline__ void gm_load(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, const Args &a,
                                        int row0, int ti, int s, int steps, int ntiles, int blk, u32x4 &wc,
                                        uint32_t &wsd)
{
    constexpr int CB = GmFmt<F>::CB;
    constexpr uint32_t kPast = 0x80000000u;                 // >= every buffer size
    const bool ok = ti < ntiles && 16 * s + blk < a.units;
    // rows past N read past the buffer: zeros, no traffic
    const uint32_t n = (uint32_t)(row0 + ti * a.rows_per_tile);
    const uint32_t oc = ok ? n * (uint32_t)a.rcb + (uint32_t)((16 * s + blk) * CB) : kPast;
    const uint32_t os = ok ? n * (uint32_t)a.rsb + (uint32_t)((16 * s + blk) * 4) : kPast;
    if constexpr (F == kCB2) {
        wc = __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, kStream);
    } else {
        const u32x3 t = __builtin_amdgcn_raw_buffer_load_b96(rc, oc, 0, kStream);
        wc = (u32x4){t[0], t[1], t[2], 0u};
    }
    wsd = __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0);
}

// A run of ntiles row tiles (from tile0) of one expert against NG staged
// vector groups; each wave streams its quad of every tile as one sequence of
// (tile, step) pairs with CPL steps of loads in flight across tile
// boundaries, and stores the rows of vectors [v0, v0 + cc) after each tile.
template <int F, int WAVES, int CPL, int NG, int NVG>
__device__ __forceinline__ void gm_run(const Args &a, const uint8_t *lds, const uint16_t *pairs, bool gather,
                                       int expert, int tile0, int ntiles, int v0, int cc, int Up)
{
    const int lane = threadIdx.x & 63;
    const int blk = lane >> 2, r = lane & 3;
    const int steps = Up >> 4;
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.codes + (long long)expert * a.expert_cb, a.expert_cb);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.scales + (long long)expert * a.expert_sb, a.expert_sb);
    const int wrow = tile0 * a.rows_per_tile + 4 * (int)(threadIdx.x >> 6);   // the wave's quad, first tile
    const int row0 = wrow + r;
    u32x4 wc[CPL];
    uint32_t wsd[CPL];
    int lt = 0, ls = 0;                                     // next (tile, step) to load
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        gm_load<F>(rc, rs, a, row0, lt, ls, steps, ntiles, blk, wc[c], wsd[c]);
        if (++ls == steps) { ls = 0; ++lt; }
    }
    float acc[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;

    int ct = 0, cs = 0;                                     // (tile, step) to compute
    const int total = ntiles * steps;
    for (int fb = 0; fb < total; fb += CPL) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (fb + c < total) {
                const int u = 16 * cs + blk;
                // the quad's four rows' scales for this block's unit
                const uint32_t sw[4] = {quad_lane<0>(wsd[c]), quad_lane<1>(wsd[c]), quad_lane<2>(wsd[c]),
                                        quad_lane<3>(wsd[c])};
                uint32_t A[16];
                if constexpr (F == kCB2) {
                    // codes c -> int8 2c - 3 (a v_perm_b32 LUT), so the MFMA
                    // forms the block's integer sum sum((2c - 3) q) itself
                    const uint32_t cw[4] = {wc[c][0], wc[c][1], wc[c][2], wc[c][3]};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            A[4 * q + t] = perm(0u, kCb2Lut2, (cw[q] >> (2 * t)) & 0x03030303u);
                } else {
                    const uint4 h0 = cb3_decode_half<0>(wc[c][1], wc[c][0]);
                    const uint4 h1 = cb3_decode_half<2>(wc[c][2], wc[c][1]);
                    A[0] = h0.x; A[1] = h0.y; A[2] = h0.z; A[3] = h0.w;
                    A[4] = h1.x; A[5] = h1.y; A[6] = h1.z; A[7] = h1.w;
#pragma unroll
                    for (int t = 8; t < 16; ++t) A[t] = 0u;
                }
                gm_step<F, NG, NVG>(lds, Up, u, r, A, sw, acc);
                if (cs == steps - 1) {
                    // tile done: sum the 16 blocks' tiles (gm_tile_sum: lane
                    // 4 blk + j ends with row blk & 3 of vector j), and the
                    // lanes 16 (g & 3) .. 16 (g & 3) + 15 store group g's 4 x 4
                    const int row = wrow + ct * a.rows_per_tile + (blk & 3);
#pragma unroll
                    for (int g = 0; g < NG; ++g) {
                        const float val = gm_tile_sum(acc[g]);
                        const int m = 4 * g + r;
                        if ((blk >> 2) == (g & 3) && m < cc && row < a.N) {
                            const int p = gather ? (int)pairs[v0 + m] : v0 + m;
                            a.y[p * a.N + row] = val;       // M * top_k * N < 2^31
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;
                    }
                }
                if (++cs == steps) { cs = 0; ++ct; }
            }
            gm_load<F>(rc, rs, a, row0, lt, ls, steps, ntiles, blk, wc[c], wsd[c]);
            if (++ls == steps) { ls = 0; ++lt; }
        }
    }
}

// The cost of one row tile of an expert with c vectors, in units of the step
// loop's issue slots (from the instruction counts of the step: the decode and
// the loads cost about 1.5 times one vector group's matrix products and
// scale epilogue): each chunk of up to 4 * NVG vectors decodes the weights
// again, each group of 4 vectors adds its own products.
template <int NVG>
__device__ __forceinline__ int gm_tile_cost(int c)
{
    constexpr int kChunk = 3, kGroup = 2;
    if (c <= 0) return 0;
    return kChunk * ((c + 4 * NVG - 1) / (4 * NVG)) + kGroup * ((c + 3) >> 2);
}

// This workgroup's run of (expert slot, row tile) items, [run[0], run[1]),
// weighted by gm_tile_cost: the experts a call selects differ in their vector
// counts, and equal runs of items would leave the workgroups of the busiest
// experts working long after the rest.  Item i = slot * tiles + t starts at
// cost tiles * P_slot + t * cost_slot (P the costs of the slots before it);
// the workgroup takes the items that start in its equal share of the total,
// [total * b / G, total * (b + 1) / G).  ids are counted per expert into
// cnt[0..1024) with LDS atomics; one wave scans the counts, 16 experts per
// lane.  Every workgroup computes the same split.
template <int THREADS, int NVG>
__device__ __forceinline__ void gm_weighted_run(const int32_t *ids, int B, int E, int tiles, int *cnt, int *run,
                                                Ids8 first)
{
    const int tid = threadIdx.x;
    for (int e = tid; e < 1024; e += THREADS) cnt[e] = 0;
    __syncthreads();
    const int rounds = (B + THREADS - 1) / THREADS;
    for (int j0 = 0; j0 < rounds; j0 += 8) {
        const Ids8 idv = j0 == 0 ? first : load_ids8<THREADS>(ids, B, E, j0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = idv.v[j];
            if (tid + (j0 + j) * THREADS < B && (unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    if (tid < 64) {
        long long cost = 0;
        int busy = 0;
        for (int k = 0; k < 16; ++k) {
            const int c = cnt[16 * tid + k];
            cost += gm_tile_cost<NVG>(c);
            busy += c > 0;
        }
        long long cs = cost;                            // inclusive scans over the lanes
        int bs = busy;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const long long tc = __shfl_up(cs, d);
            const int tb = __shfl_up(bs, d);
            if (tid >= d) {
                cs += tc;
                bs += tb;
            }
        }
        const long long total = (long long)tiles * __shfl(cs, 63);
        const int D = __shfl(bs, 63);
        const long long lo = total * blockIdx.x / gridDim.x;
        const long long hi = total * (blockIdx.x + 1) / gridDim.x;
        if (tid == 0) {                                 // a bound at the end: past the last item
            if (lo >= total) run[0] = D * tiles;
            if (hi >= total) run[1] = D * tiles;
        }
        long long p = (long long)tiles * (cs - cost);   // this lane's first expert's start
        int s = bs - busy;                              // and its slot
        for (int k = 0; k < 16; ++k) {
            const int c = cnt[16 * tid + k];
            const int w = gm_tile_cost<NVG>(c);
            if (w > 0) {
                const long long end = p + (long long)tiles * w;
                // items of slot s that start before the bound
                if (lo >= p && lo < end) run[0] = s * tiles + (int)((lo - p + w - 1) / w);
                if (hi >= p && hi < end) run[1] = s * tiles + (int)((hi - p + w - 1) / w);
                p = end;
                ++s;
            }
        }
    }
    __syncthreads();
}

// Work items (expert slot, row tile), slot-major, dealt in contiguous runs of
// equal weighted cost (gm_weighted_run; equal runs of items for a dense
// call); per slot the pairs are listed and taken in chunks of up to 4 * NVG
// vectors, each staged once and streamed against every row tile of the run.
template <int F, int WAVES, int NVG, int CPL, bool Q>
__global__ __launch_bounds__(64 * WAVES) void qmv_gmma_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int THREADS = 64 * WAVES;
    const bool gather = a.ids != nullptr;
    const int Up = (a.units + 15) & ~15;
    uint8_t *tail = lds + gm_stage_bytes<F, NVG>(Up);
    PairList L;
    L.cnt = (int *)tail;
    uint32_t *bm = (uint32_t *)(tail + kPairCountBytes);
    int *ecnt = (int *)(tail + kPairCountBytes + kExpertBitmapBytes);
    L.perm = (uint16_t *)(tail + kPairCountBytes + kExpertBitmapBytes + kExpertCountBytes);
    const int tiles = a.gr_tiles, rpt = a.rows_per_tile;
    const int B = a.M * a.top_k;
    Ids8 id0;
    int D = 1;
    if (gather) {
        id0 = load_ids8<THREADS>(a.ids, B, a.E, 0);
        D = expert_bitmap<THREADS>(a.ids, B, a.E, bm, id0);
        const int z0 = (int)((long long)blockIdx.x * tiles / gridDim.x);
        const int z1 = (int)((long long)(blockIdx.x + 1) * tiles / gridDim.x);
        if (z1 > z0) {                              // zero rows of ids outside [0, E)
            const int ci = list_pairs<THREADS>(a.ids, B, a.E, -1, L, id0);
            const int n0 = z0 * rpt;
            const int rows = min(a.N, z1 * rpt) - n0;
            for (int o = threadIdx.x; o < ci * rows; o += THREADS)
                a.y[(int)L.perm[o / rows] * a.N + n0 + o % rows] = 0.0f;
            __syncthreads();
        }
    }
    int i, i1;
    if (gather) {
        int *run = (int *)(bm + 34);
        gm_weighted_run<THREADS, NVG>(a.ids, B, a.E, tiles, ecnt, run, id0);
        i = run[0];
        i1 = run[1];
    } else {
        i = (int)((long long)blockIdx.x * tiles / gridDim.x);
        i1 = (int)((long long)(blockIdx.x + 1) * tiles / gridDim.x);
    }
    while (i < i1) {
        const int slot = i / tiles;
        const int iend = min(i1, (slot + 1) * tiles);   // this run's items of the slot
        int e = 0, c = a.M;
        if (gather) {
            e = kth_expert(bm, slot);
            c = list_pairs<THREADS>(a.ids, B, a.E, e, L, id0);
        }
        // full chunks of 4 * NVG vectors and the rest, ceil(c / 4) vector
        // groups in all
        for (int v0 = 0; v0 < c;) {
            const int cc = min(4 * NVG, c - v0);
            const int ng = (cc + 3) >> 2;
            gm_stage<F, THREADS, Q, NVG>(a, lds, L.perm, gather, v0, cc, ng, Up);
            __syncthreads();
            const int tile0 = i - slot * tiles, nt = iend - i;
            if constexpr (NVG >= 4) {
                if (ng == 4) gm_run<F, WAVES, CPL, 4, NVG>(a, lds, L.perm, gather, e, tile0, nt, v0, cc, Up);
            }
            if constexpr (NVG >= 3) {
                if (ng == 3) gm_run<F, WAVES, CPL, 3, NVG>(a, lds, L.perm, gather, e, tile0, nt, v0, cc, Up);
            }
            if constexpr (NVG >= 2) {
                if (ng == 2) gm_run<F, WAVES, CPL, 2, NVG>(a, lds, L.perm, gather, e, tile0, nt, v0, cc, Up);
            }
            if (ng == 1) gm_run<F, WAVES, CPL, 1, NVG>(a, lds, L.perm, gather, e, tile0, nt, v0, cc, Up);
            __syncthreads();                            // the next chunk or expert restages
            v0 += cc;
        }
        i = iend;
    }
}

// [workgroup: 8 waves, 12 waves][int8 activations, bf16 quantized in
// staging][format: 2-bit, 3-bit][vector groups per chunk: 1, 2, 3, 4 (at 12
// waves 2-bit only: the 3-bit kernel with four groups needs more than the 168
// registers per lane that three waves per SIMD leave)]; 3 steps of loads in
// flight.
#define QMV_GM(W, F, N, Q) (const void *)&qmv_gmma_kernel<F, W, N, 3, Q>
extern const void *const kTableGmma[2][2][2][4];
const void *const kTableGmma[2][2][2][4] = {
    {{{QMV_GM(8, kCB2, 1, false), QMV_GM(8, kCB2, 2, false), QMV_GM(8, kCB2, 3, false), QMV_GM(8, kCB2, 4, false)},
      {QMV_GM(8, kCB3, 1, false), QMV_GM(8, kCB3, 2, false), QMV_GM(8, kCB3, 3, false), QMV_GM(8, kCB3, 4, false)}},
     {{QMV_GM(8, kCB2, 1, true), QMV_GM(8, kCB2, 2, true), QMV_GM(8, kCB2, 3, true), QMV_GM(8, kCB2, 4, true)},
      {QMV_GM(8, kCB3, 1, true), QMV_GM(8, kCB3, 2, true), QMV_GM(8, kCB3, 3, true), QMV_GM(8, kCB3, 4, true)}}},
    {{{QMV_GM(12, kCB2, 1, false), QMV_GM(12, kCB2, 2, false), QMV_GM(12, kCB2, 3, false), QMV_GM(12, kCB2, 4, false)},
      {QMV_GM(12, kCB3, 1, false), QMV_GM(12, kCB3, 2, false), QMV_GM(12, kCB3, 3, false), nullptr}},
     {{QMV_GM(12, kCB2, 1, true), QMV_GM(12, kCB2, 2, true), QMV_GM(12, kCB2, 3, true), QMV_GM(12, kCB2, 4, true)},
      {QMV_GM(12, kCB3, 1, true), QMV_GM(12, kCB3, 2, true), QMV_GM(12, kCB3, 3, true), nullptr}}}};
#undef QMV_GM

}  // namespace qmv
