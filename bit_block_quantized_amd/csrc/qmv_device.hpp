// qmv_device.hpp -- gfx950 device code of the block-quantized GEMV.
//
// One kernel family serves every call.  A workgroup (4 wave64s) owns one
// "work item" (an expert plus up to four activation vectors routed to it) and
// one tile of consecutive output rows.  Inside a wave, LPR lanes share a row:
// lane li streams the row's 16-byte-aligned "units" li, li+LPR, ... so each
// load instruction reads LPR*unit_bytes contiguous bytes of a row, and each
// lane keeps RT rows in flight.  Weight loads run ahead of the arithmetic that
// consumes them (geo-lucebox PR #31 "DS4 H200: rocmfp2_mix MoE matvec", the
// commit table: hoisting row loads above the FMAs was one of its steps);
// activations are staged once per workgroup into swizzled LDS in the layout
// each decode consumes (the same table's LDS staging step), and the lanes'
// partial sums of a row are combined by a fixed butterfly, so results are
// bitwise reproducible.
//
// The 2-bit and 3-bit kernels are also built with Q = true: activations then
// arrive as bf16 and each staging thread quantizes one 32-block to int8 plus
// an fp16 scale on its way into LDS (quant_q8_block); everything after the
// staging is the int8 kernel unchanged.
//
// Units per format (one unit = what a lane decodes per load):
//   MXFP4  32 weights: 16 B of nibbles + 1 E8M0 byte      (bf16 x, 64 B)
//   CB2    64 weights: 16 B of 2-bit codes + 2 fp16 scales (int8 x, 64 B)
//   CB2S   32 weights:  8 B of 2-bit codes + 1 fp16 scale  (int8 x, 32 B)
//   CB3    32 weights: 12 B of 3-bit codes + 2 fp16 scales (int8 x, 32 B)
//   MXFP4I 32 weights: 16 B of nibbles + 1 E8M0 byte      (int8 x as bf16, 64 B)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_host.hpp"

// The kernels are instantiated twice, with 4 and with 8 wave64s per
// workgroup (a larger workgroup stages the activations once for twice the
// rows); QMV_NS keeps the two sets of names apart.
#ifndef QMV_NS
#define QMV_NS qmv
#endif

namespace QMV_NS {

#ifndef QMV_WAVES
#define QMV_WAVES 4
#endif
constexpr int kWaves = QMV_WAVES;        // wave64s per workgroup
constexpr int kThreads = 64 * kWaves;

using namespace qmv_cfg;      // format kinds, unit sizes, launch menus (qmv_host.hpp)

struct Args {
    const uint8_t *codes;
    const uint8_t *scales;
    const uint8_t *codes2;   // gate/up mode: the up projection (codes is the gate)
    const uint8_t *scales2;
    const int32_t *ids;      // nullptr for a dense call
    const float *route_w;    // combine mode: router weights fp32 [M][top_k]
    const uint8_t *x;
    const uint16_t *xs;      // int8 activation scales (fp16 bits) or nullptr
    float *y;
    long long expert_cb;     // bytes of codes per expert (N * rcb)
    long long expert_sb;     // bytes of scales per expert (N * rsb)
    int rcb, rsb;            // bytes per row of codes / of scales (N * rcb < 2^31)
    int x_vec_bytes;         // bytes per activation vector
    int E, M, top_k, N, K;
    int units;               // units per row
    int x_per_slot;
    int x_early;             // activation vectors known before routing
    int rows_per_tile;
    int lds_vec_bytes;       // LDS bytes per staged activation vector
    // batched kernels (more than 4 vectors): tiles of (expert or vector
    // chunk, row tile), dealt to the 8 XCDs in contiguous runs
    int bt_row_tiles;        // row tiles per expert
    int bt_tiles;            // tiles in the call
    int bt_per_xcd;          // tiles per XCD (ceil(bt_tiles / 8))
    int bt_chunk;            // dense: vectors per tile
    int bt_vmax;             // vectors the activation ring holds (32, 64 or 128)
    // grouped kernel: work items (expert slot, row tile), slot-major
    int gr_tiles;            // row tiles per expert
};

// ------------------------------------------------------------------ helpers
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));


__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Shift the two 16-bit halves of v right by s_lo and s_hi (v_pk_lshrrev_b16).
template <int S_LO, int S_HI>
__device__ __forceinline__ uint32_t pk_shr(uint32_t v)
{
    u16x2 h = __builtin_bit_cast(u16x2, v);
    const u16x2 s = {(unsigned short)S_LO, (unsigned short)S_HI};
    return __builtin_bit_cast(uint32_t, h >> s);
}

__device__ __forceinline__ float f16_lo(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

// E8M0 byte -> float 2^(s-127), built exactly: s = 0 is the subnormal
// 2^-127 and s = 255 is NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t s)
{
    uint32_t bits = s << 23;
    bits |= (((s + 1u) & 0xFEu) == 0u) ? 0x00400000u : 0u;
    return __uint_as_float(bits);
}

// LDS position (in 16-byte chunks) of chunk q of unit u.  The xor keeps the
// 8 (or 16) lanes that one ds_read_b128 serves on distinct bank groups while
// they read consecutive units -- the same trick as the query swizzle of
// Strata PR #1661, fitted to 64- and 32-byte records.
template <int CH> __device__ __forceinline__ int swz(int u);
template <> __device__ __forceinline__ int swz<4>(int u) { return (((u >> 1) ^ (u >> 3)) & 1) | ((u >> 1) & 2); }
template <> __device__ __forceinline__ int swz<2>(int u) { return ((u >> 2) ^ (u >> 3)) & 1; }
template <int CH> __device__ __forceinline__ int chunk_pos(int u, int q) { return u * CH + (q ^ swz<CH>(u)); }

// Chunk position of unit u0 + c * LPR.  The swizzle reads bits 1..3 of the
// unit index only, so for LPR >= 16 a lane's units share it and the position
// advances by a constant (an immediate LDS offset) from one unit to the next.
template <int CH, int LPR>
__device__ __forceinline__ int chunk_at(int u0, int c, int q)
{
    if constexpr (LPR >= 16) return chunk_pos<CH>(u0, q) + c * LPR * CH;
    else return chunk_pos<CH>(u0 + c * LPR, q);
}

// One 16-byte LDS read as a single vector load.  Reading through a HIP
// uint4 lets the compiler split the struct into per-field loads and rebuild
// them as ds_read_b96 + ds_read_b32, whose 4-byte part hits only a quarter
// of the banks at a 16-byte lane stride; a native vector load stays one
// ds_read_b128.
__device__ __forceinline__ uint4 lds_read16(const uint8_t *p)
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = *(const v4u *)__builtin_assume_aligned(p, 16);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ routing
// A work item: one expert and up to four activation vectors that read it.
struct Item {
    int kind;                     // 0: compute, 1: zero rows, -1: nothing to do
    int expert;
    int nv;
    int vec[4];                   // activation vector index (token, or pair)
    unsigned long long dest[4];   // output rows (pair index bits) of each vector
    int pair[4];                  // grouped kernel: the one output row of each vector
};

// Token of pair p (M <= 4 tokens of k slots each), without a division.
__device__ __forceinline__ int token_of(int p, int k)
{
    return (p >= k) + (p >= 2 * k) + (p >= 3 * k);
}

__device__ __forceinline__ int nth_set_bit(unsigned long long m, int n)
{
    for (int i = 0; i < n; ++i) m &= m - 1;
    return __ffsll((long long)m) - 1;
}

// Activation vectors of an item when they are known before routing.
__device__ __forceinline__ Item early_item(const Args &a)
{
    Item it;
    it.kind = 0;
    it.expert = 0;
    it.nv = a.ids == nullptr ? a.M : 1;
#pragma unroll
    for (int m = 0; m < 4; ++m) { it.vec[m] = m; it.dest[m] = 0ull; it.pair[m] = 0; }
    return it;
}

// Routing of a one-vector kernel (dense, or a single broadcast token): the
// items are the distinct valid experts in order of first appearance, each
// read by activation vector 0; out-of-range ids become zero items after them.
__device__ Item route_one(const Args &a, int item_idx)
{
    Item it;
    it.kind = -1;
    it.expert = 0;
    it.nv = 1;
#pragma unroll
    for (int m = 0; m < 4; ++m) { it.vec[m] = 0; it.dest[m] = 0ull; it.pair[m] = 0; }
    if (a.ids == nullptr) {
        if (item_idx == 0) { it.kind = 0; it.dest[0] = 1ull; }
        return it;
    }
    const int lane = threadIdx.x & 63;
    const int P = a.M * a.top_k;
    int e = -1;
    if (lane < P) e = a.ids[lane];
    const bool valid = lane < P && e >= 0 && e < a.E;
    bool dup = false;
    for (int q = 0; q < P; ++q)
        dup = dup || (q < lane && __builtin_amdgcn_readlane(e, q) == e);
    const unsigned long long lead = __ballot(valid && !dup);
    const unsigned long long inval = __ballot(lane < P && !valid);
    const int n_real = __popcll(lead);
    if (item_idx < n_real) {
        const int e_lead = __builtin_amdgcn_readlane(e, nth_set_bit(lead, item_idx));
        it.kind = 0;
        it.expert = e_lead;
        it.dest[0] = __ballot(valid && e == e_lead);
    } else if (item_idx < n_real + __popcll(inval)) {
        it.kind = 1;
        it.dest[0] = 1ull << nth_set_bit(inval, item_idx - n_real);
    }
    return it;
}

// Every wave derives the same item list from the ids on its own (no LDS, no
// barrier).  Pairs p = t*top_k + j live on lanes.  Distinct (expert, vector)
// entries are grouped per expert in order of first appearance, four vectors
// per item; out-of-range ids become "zero" items after the real ones.  With
// M = 1 and broadcast activations this is one item per distinct expert, the
// unsorted decode schedule of mlxcel issue #2178 (Current Behavior).
__device__ Item route(const Args &a, int item_idx)
{
    Item it;
    it.kind = -1;
    it.expert = 0;
    it.nv = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) { it.vec[m] = 0; it.dest[m] = 0ull; it.pair[m] = 0; }

    if (a.ids == nullptr) {                       // dense: one item, M vectors
        if (item_idx == 0) {
            it.kind = 0;
            it.nv = a.M;
#pragma unroll
            for (int m = 0; m < 4; ++m) { it.vec[m] = m; it.dest[m] = (m < a.M) ? (1ull << m) : 0ull; }
        }
        return it;
    }

    const int lane = threadIdx.x & 63;
    const int P = a.M * a.top_k;
    int e = -1;
    if (lane < P) e = a.ids[lane];
    const bool valid = lane < P && e >= 0 && e < a.E;
    const int v = a.x_per_slot ? lane : token_of(lane, a.top_k);

    unsigned long long same_e = 0ull, same_ev = 0ull;
    for (int q = 0; q < P; ++q) {
        const int eq = __builtin_amdgcn_readlane(e, q);
        const int vq = a.x_per_slot ? q : token_of(q, a.top_k);
        const bool hit = valid && eq == e;
        same_e |= hit ? (1ull << q) : 0ull;
        same_ev |= (hit && vq == v) ? (1ull << q) : 0ull;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    const bool uniq = valid && (same_ev & below) == 0ull;
    const unsigned long long uniq_mask = __ballot(uniq);
    const int rank = __popcll(same_e & uniq_mask & below);
    const bool leader = uniq && (rank & 3) == 0;
    const unsigned long long leader_mask = __ballot(leader);
    const unsigned long long inval_mask = __ballot(lane < P && !valid);
    const int n_real = __popcll(leader_mask);
    const int n_zero = __popcll(inval_mask);

    if (item_idx < n_real) {
        const int ll = nth_set_bit(leader_mask, item_idx);
        const int e_lead = __builtin_amdgcn_readlane(e, ll);
        const int r_lead = __builtin_amdgcn_readlane(rank, ll);
        unsigned long long mm = __ballot(uniq && e == e_lead && rank >= r_lead && rank < r_lead + 4);
        it.kind = 0;
        it.expert = e_lead;
        it.nv = __popcll(mm);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m < it.nv) {
                const int ml = __ffsll((long long)mm) - 1;
                mm &= mm - 1ull;
                const int vm = a.x_per_slot ? ml : token_of(ml, a.top_k);
                it.vec[m] = vm;
                it.dest[m] = __ballot(valid && e == e_lead && v == vm);
            }
        }
    } else if (item_idx < n_real + n_zero) {
        it.kind = 1;
        it.dest[0] = 1ull << nth_set_bit(inval_mask, item_idx - n_real);
    }
    return it;
}

// ------------------------------------------------------------------ staging
// The item's activation vectors are written into LDS in the order each
// format's decode consumes them.  Staging is split in two so that its global
// loads can be issued before the weight loads: xload() fetches up to kXReg
// 16-byte chunks per thread into registers, xstore() writes them to LDS once
// the weight loads are in flight, and xrest() moves whatever did not fit
// (large K with several vectors) synchronously.
constexpr int kXReg = 4;

__device__ __forceinline__ int item_vec(const Item &it, int m)
{
    return m == 0 ? it.vec[0] : m == 1 ? it.vec[1] : m == 2 ? it.vec[2] : it.vec[3];
}

// Staging items: MXFP4 -- one 16-byte chunk of bf16; CB2/CB3/MXFP4I -- one
// 32-byte block of int8 (two chunks).
template <int F> struct XItem { static constexpr int chunks = (F == kMXFP4) ? 1 : 2; };

template <int F>
__device__ __forceinline__ int x_items_per_vec(const Args &a) { return F == kMXFP4 ? 4 * a.units : a.K / 32; }

// Staging item i -> (vector m, item c within the vector); nv <= NVMAX <= 4.
template <int NVMAX>
__device__ __forceinline__ int item_m(int i, int per)
{
    if constexpr (NVMAX == 1) return 0;
    else return (i >= per) + (i >= 2 * per) + (i >= 3 * per);
}

// Staging item i's bytes in global memory: Q items are 64-byte bf16 blocks.
template <int F, int NVMAX, bool Q>
__device__ __forceinline__ const uint8_t *x_item_ptr(const Args &a, const Item &it, int i)
{
    const int per = x_items_per_vec<F>(a);
    const int m = item_m<NVMAX>(i, per);
    const int c = i - __umul24(m, per);
    return a.x + __umul24(item_vec(it, m), a.x_vec_bytes) + c * (Q ? 64 : 16 * XItem<F>::chunks);
}

template <int F, int NVMAX, bool Q>
__device__ __forceinline__ void xload(const Args &a, const Item &it, uint4 (&r)[kXReg])
{
    if constexpr (Q) {                                      // one bf16 block per thread
        const int T = __umul24(it.nv, x_items_per_vec<F>(a));
        const uint8_t *p = x_item_ptr<F, NVMAX, true>(a, it, min((int)threadIdx.x, T - 1));
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = *(const uint4 *)(p + 16 * q);
        return;
    }
    constexpr int PER = kXReg / XItem<F>::chunks;          // items held per thread
    const int T = __umul24(it.nv, x_items_per_vec<F>(a));
    const int jn = (T + kThreads - 1) / kThreads;           // items this workgroup needs per thread
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (j < jn) {
            const int i = min((int)threadIdx.x + j * kThreads, T - 1);   // clamped: no divergence
            const uint8_t *p = x_item_ptr<F, NVMAX, false>(a, it, i);
            r[j * XItem<F>::chunks] = *(const uint4 *)p;
            if constexpr (XItem<F>::chunks == 2) r[j * 2 + 1] = *(const uint4 *)(p + 16);
        }
    }
}

// 16 int8 activations -> the 4x4 byte transpose that matches the 2-bit
// selectors (w >> 2j) & 0x03030303: dword j holds x[j], x[4+j], x[8+j], x[12+j].
__device__ __forceinline__ uint4 cb2_xorder(uint4 in)
{
    const uint32_t t0 = perm(in.y, in.x, 0x05010400u);   // x0 x4 x1 x5
    const uint32_t t1 = perm(in.w, in.z, 0x05010400u);   // x8 x12 x9 x13
    const uint32_t t2 = perm(in.y, in.x, 0x07030602u);   // x2 x6 x3 x7
    const uint32_t t3 = perm(in.w, in.z, 0x07030602u);   // x10 x14 x11 x15
    uint4 o;
    o.x = perm(t1, t0, 0x05040100u);                      // x0 x4 x8 x12
    o.y = perm(t1, t0, 0x07060302u);                      // x1 x5 x9 x13
    o.z = perm(t3, t2, 0x05040100u);                      // x2 x6 x10 x14
    o.w = perm(t3, t2, 0x07060302u);                      // x3 x7 x11 x15
    return o;
}

// 16 int8 activations of a 3-bit half-block -> the orders of the four
// selector dwords built in cb3_half: (0,8,1,9) (3,11,4,12) (6,14,7,15) (2,5,10,13).
__device__ __forceinline__ uint4 cb3_xorder(uint4 in)
{
    uint4 o;
    o.x = perm(in.z, in.x, 0x05010400u);                  // x0 x8 x1 x9
    const uint32_t a = perm(in.z, in.x, 0x07030703u);     // x3 x11 . .
    const uint32_t b = perm(in.w, in.y, 0x04000400u);     // x4 x12 . .
    o.y = perm(b, a, 0x05040100u);                        // x3 x11 x4 x12
    const uint32_t c = perm(in.w, in.y, 0x06020602u);     // x6 x14 . .
    const uint32_t d = perm(in.w, in.y, 0x07030703u);     // x7 x15 . .
    o.z = perm(d, c, 0x05040100u);                        // x6 x14 x7 x15
    const uint32_t e = perm(in.y, in.x, 0x05050502u);     // x2 x5 . .
    const uint32_t f = perm(in.w, in.z, 0x05050502u);     // x10 x13 . .
    o.w = perm(f, e, 0x05040100u);                        // x2 x5 x10 x13
    return o;
}

__device__ __forceinline__ int sum_i8x16(uint4 v)
{
    int s = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, 0, false);
    s = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, s, false);
    return __builtin_amdgcn_sdot4((int)v.w, 0x01010101, s, false);
}

// Bytes 2h and 2h+1 of w (int8) -> two bf16 in one dword, the first in the
// low half.  |q| <= 128 has at most 8 significant bits, so the f32 value's
// top 16 bits are the exact bf16.
__device__ __forceinline__ uint32_t i8x2_bf16(uint32_t w, int h)
{
    const float f0 = (float)(int8_t)(w >> (16 * h));
    const float f1 = (float)(int8_t)(w >> (16 * h + 8));
    return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
}

// Write staging item i (already in registers) to its LDS place.
//  MXFP4: chunk c of a vector = bf16 x[8c..8c+7], stored in natural order so
//         byte b of code dword q pairs with bf16 dword b of chunk q.
//  CB2:   block b -> chunks 2b, 2b+1 transposed for the 2-bit selectors, and
//         per-unit side data {0.5*xs, -3*sum(q)} per 32-block (the codebook
//         is c - 1.5, so a block's integer sum is 2*dot(c, q) - 3*sum(q)).
//  CB3:   block b -> its two half-blocks in the cb3_half order; side data
//         0.5*xs per block.
//  MXFP4I: block b -> unit b's four chunks of bf16 (int8 values are exact in
//         bf16), laid out as MXFP4's; side data xs per block.
template <int F, int NVMAX>
__device__ __forceinline__ void xput_blk(const Args &a, const Item &it, uint8_t *lds, int i,
                                         uint4 lo, uint4 hi, uint32_t xsb)
{
    const int per = x_items_per_vec<F>(a);
    const int m = item_m<NVMAX>(i, per);
    const int c = i - __umul24(m, per);
    uint8_t *dst = lds + __umul24(m, a.lds_vec_bytes);
    if constexpr (F == kMXFP4) {
        *(uint4 *)(dst + 16 * chunk_pos<4>(c >> 2, c & 3)) = lo;
    } else if constexpr (F == kMXFP4I) {
        const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *(uint4 *)(dst + 16 * chunk_pos<4>(c, q)) =
                make_uint4(i8x2_bf16(d[2 * q], 0), i8x2_bf16(d[2 * q], 1),
                           i8x2_bf16(d[2 * q + 1], 0), i8x2_bf16(d[2 * q + 1], 1));
        ((float *)(dst + a.units * Fmt<F>::XB))[c] = (float)__builtin_bit_cast(_Float16, (uint16_t)xsb);
    } else {
        constexpr int CH = Fmt<F>::XB / 16;
        const int xbytes = a.units * Fmt<F>::XB;
        const float xsh = 0.5f * (float)__builtin_bit_cast(_Float16, (uint16_t)xsb);
        if constexpr (F == kCB3) {
            *(uint4 *)(dst + 16 * chunk_pos<2>(c, 0)) = cb3_xorder(lo);
            *(uint4 *)(dst + 16 * chunk_pos<2>(c, 1)) = cb3_xorder(hi);
            ((float *)(dst + xbytes))[c] = xsh;
        } else {
            const int c0 = 2 * c, c1 = 2 * c + 1;
            *(uint4 *)(dst + 16 * chunk_pos<CH>(c0 / CH, c0 % CH)) = cb2_xorder(lo);
            *(uint4 *)(dst + 16 * chunk_pos<CH>(c1 / CH, c1 % CH)) = cb2_xorder(hi);
            const int nq = -3 * (sum_i8x16(lo) + sum_i8x16(hi));
            if constexpr (F == kCB2) {
                float *side = (float *)(dst + xbytes + 16 * (c >> 1));
                side[c & 1] = xsh;
                ((int *)side)[2 + (c & 1)] = nq;
            } else {
                float *side = (float *)(dst + xbytes + 8 * c);
                side[0] = xsh;
                ((int *)side)[1] = nq;
            }
        }
    }
}

template <int F, int NVMAX>
__device__ __forceinline__ void xput(const Args &a, const Item &it, uint8_t *lds, int i,
                                     uint4 lo, uint4 hi)
{
    uint32_t xsb = 0;
    if constexpr (F != kMXFP4) {
        const int per = x_items_per_vec<F>(a);
        const int m = item_m<NVMAX>(i, per);
        xsb = a.xs[__umul24(item_vec(it, m), a.K / 32) + (i - __umul24(m, per))];
    }
    xput_blk<F, NVMAX>(a, it, lds, i, lo, hi, xsb);
}

// bf16 activations of one 32-block -> 32 int8 (lo, hi) and the fp16 scale
// bits, all in fp32: d = amax / 127, d16 = fp16(d) (nearest even), then
// q = clamp(rint(x * (1 / d16)), -127, 127) with ties to even, and q = 0
// where d16 is 0 or infinite.  This is the q8 activation block that the
// pages quantize in a launch of its own before every integer matvec
// (geo-lucebox PR #31, "What is now hot": quantize_q8_1); here each staging
// thread quantizes one block on its way into LDS, so there is no separate
// launch and no int8 copy of x in memory.  Division and reciprocal are the
// IEEE (correctly rounded) ones.
__device__ __forceinline__ uint32_t quant_q8_block(const uint4 (&c)[4], uint4 &lo, uint4 &hi)
{
    const uint32_t w[16] = {c[0].x, c[0].y, c[0].z, c[0].w, c[1].x, c[1].y, c[1].z, c[1].w,
                            c[2].x, c[2].y, c[2].z, c[2].w, c[3].x, c[3].y, c[3].z, c[3].w};
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
    }
    const float d = amax / 127.0f;
    const _Float16 h = (_Float16)d;
    const float dd = (float)h;
    const float r = (dd > 0.0f && dd < __builtin_inff()) ? 1.0f / dd : 0.0f;
    uint32_t qd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float t = fminf(fmaxf(__builtin_rintf(v[4 * j + b] * r), -127.0f), 127.0f);
            packed |= ((uint32_t)(int)t & 0xFFu) << (8 * b);
        }
        qd[j] = packed;
    }
    lo = make_uint4(qd[0], qd[1], qd[2], qd[3]);
    hi = make_uint4(qd[4], qd[5], qd[6], qd[7]);
    return (uint32_t)__builtin_bit_cast(unsigned short, h);
}

template <int F, int NVMAX, bool Q>
__device__ __forceinline__ void xstore(const Args &a, const Item &it, uint8_t *lds, const uint4 (&r)[kXReg])
{
    if constexpr (Q) {
        const int i = (int)threadIdx.x;
        if (i < __umul24(it.nv, x_items_per_vec<F>(a))) {
            uint4 lo, hi;
            const uint32_t xsb = quant_q8_block(r, lo, hi);
            xput_blk<F, NVMAX>(a, it, lds, i, lo, hi, xsb);
        }
        return;
    }
    constexpr int CHK = XItem<F>::chunks;
    constexpr int PER = kXReg / CHK;
    const int T = __umul24(it.nv, x_items_per_vec<F>(a));
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = (int)threadIdx.x + j * kThreads;
        if (i < T) xput<F, NVMAX>(a, it, lds, i, r[j * CHK], r[j * CHK + (CHK - 1)]);
    }
}

// Items beyond the register budget, loaded and stored directly.  Returns
// whether there were any (the same answer in every thread).
template <int F, int NVMAX, bool Q>
__device__ __forceinline__ bool xrest(const Args &a, const Item &it, uint8_t *lds)
{
    if constexpr (Q) {
        const int T = __umul24(it.nv, x_items_per_vec<F>(a));
        if (T <= kThreads) return false;
        for (int i = kThreads + (int)threadIdx.x; i < T; i += kThreads) {
            const uint8_t *p = x_item_ptr<F, NVMAX, true>(a, it, i);
            uint4 c[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) c[q] = *(const uint4 *)(p + 16 * q);
            uint4 lo, hi;
            const uint32_t xsb = quant_q8_block(c, lo, hi);
            xput_blk<F, NVMAX>(a, it, lds, i, lo, hi, xsb);
        }
        return true;
    }
    constexpr int PER = kXReg / XItem<F>::chunks;
    const int T = __umul24(it.nv, x_items_per_vec<F>(a));
    if (T <= PER * kThreads) return false;
    for (int i = PER * kThreads + (int)threadIdx.x; i < T; i += kThreads) {
        const uint8_t *p = x_item_ptr<F, NVMAX, false>(a, it, i);
        const uint4 lo = *(const uint4 *)p;
        const uint4 hi = (XItem<F>::chunks == 2) ? *(const uint4 *)(p + 16) : lo;
        xput<F, NVMAX>(a, it, lds, i, lo, hi);
    }
    return true;
}

// ------------------------------------------------------------------ units
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Weights are read through raw buffer resources over one expert's codes (or
// scales): the base sits in SGPRs, each lane carries a 32-bit row offset,
// and a unit's position in the row becomes the instruction's immediate
// offset.  A read at or past the end of the expert returns zeros without
// touching memory, so the rows of a partial last tile need no clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, long long bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

template <int F> struct Unit;
template <> struct Unit<kMXFP4> { u32x4 c; uint32_t s; static constexpr int CB = 16, SB = 1; };
template <> struct Unit<kCB2>   { u32x4 c; uint32_t s; static constexpr int CB = 16, SB = 4; };
template <> struct Unit<kCB2S>  { u32x2 c; uint32_t s; static constexpr int CB = 8, SB = 2; };
template <> struct Unit<kCB3>   { u32x3 c; uint32_t s; static constexpr int CB = 12, SB = 4; };
template <> struct Unit<kMXFP4I> { u32x4 c; uint32_t s; static constexpr int CB = 16, SB = 1; };

// ------------------------------------------------------------------ MAC per unit
// Each mac_* adds the unit's contribution for RT rows and NV vectors.

// MXFP4 x bf16.  Fast path (every E8M0 byte of the unit in [2, 252], so
// e2m1 * 2^(s-127) is an exact bf16 normal): v_cvt_scalef32_pk_bf16_fp4
// decodes two nibbles and applies the scale in one instruction, and
// v_dot2c_f32_bf16 accumulates straight into the row's f32 sum.  Otherwise
// (scale bytes 0, 1, 253..255 anywhere in the wave): decode unscaled, dot the
// group, then one fma with the exactly built 2^(s-127) (subnormal at 0, NaN
// at 255).
template <int LPR, int RT, int NV>
__device__ __forceinline__ void mac_mxfp4(const Unit<kMXFP4> (&w)[RT], const uint8_t *lds,
                                          int vec_bytes, int u0, int cu, bool fast,
                                          float (&acc)[RT][NV])
{
    uint4 xq[NV][4];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xq[v][q] = lds_read16(lds + v * vec_bytes + 16 * chunk_at<4, LPR>(u0, cu, q));
    if (fast) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const uint32_t cw[4] = {w[r].c.x, w[r].c.y, w[r].c.z, w[r].c.w};
            const float sc = __uint_as_float(w[r].s << 23);
            bf16x2 wv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wv[4 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 0);
                wv[4 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 1);
                wv[4 * q + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 2);
                wv[4 * q + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 3);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float s = acc[r][v];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t xd[4] = {xq[v][q].x, xq[v][q].y, xq[v][q].z, xq[v][q].w};
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        s = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + b], __builtin_bit_cast(bf16x2, xd[b]), s, false);
                }
                acc[r][v] = s;
            }
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const uint32_t cw[4] = {w[r].c.x, w[r].c.y, w[r].c.z, w[r].c.w};
        bf16x2 wv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wv[4 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 0);
            wv[4 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 1);
            wv[4 * q + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 2);
            wv[4 * q + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], 1.0f, 3);
        }
        const float sc = e8m0_f32(w[r].s);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t xd[4] = {xq[v][q].x, xq[v][q].y, xq[v][q].z, xq[v][q].w};
                d0 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 0], __builtin_bit_cast(bf16x2, xd[0]), d0, false);
                d1 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 1], __builtin_bit_cast(bf16x2, xd[1]), d1, false);
                d0 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 2], __builtin_bit_cast(bf16x2, xd[2]), d0, false);
                d1 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 3], __builtin_bit_cast(bf16x2, xd[3]), d1, false);
            }
            acc[r][v] = __builtin_fmaf(d0 + d1, sc, acc[r][v]);
        }
    }
}

// MXFP4 x int8 (kMXFP4I).  The activations sit in LDS as exact bf16 in the
// MXFP4 layout, their fp16 block scale as an f32 per unit after them.  Every
// product e2m1 * 2^(s-127) * q carries the block's factor 2^(s-127) and at
// most 10 significant bits, and the 32 of a block sum to below 2^16 of its
// least step, so the block sum the bf16 dot builds is exact in f32 in any
// order -- the integer dot product of the weights' 2*e2m1 values with q,
// scaled -- and the activation scale is applied once per block.  The same
// decode as MXFP4 x bf16 (hardware fp4 conversion, v_dot2c) costs 1 VALU per
// weight here, where decoding nibbles to signed int8 for v_dot4 would take
// about 2 (there is no fp4 -> int8 conversion, and the sign needs its own
// selects).
template <int LPR, int RT, int NV>
__device__ __forceinline__ void mac_mxfp4i(const Unit<kMXFP4I> (&w)[RT], const uint8_t *lds,
                                           int vec_bytes, int xbytes, int u0, int cu, bool fast,
                                           float (&acc)[RT][NV])
{
    uint4 xq[NV][4];
    float xs[NV];
    const int u = u0 + cu * LPR;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xq[v][q] = lds_read16(lds + v * vec_bytes + 16 * chunk_at<4, LPR>(u0, cu, q));
        xs[v] = *(const float *)(lds + v * vec_bytes + xbytes + 4 * u);
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const uint32_t cw[4] = {w[r].c.x, w[r].c.y, w[r].c.z, w[r].c.w};
        const float sc = fast ? __uint_as_float(w[r].s << 23) : 1.0f;
        bf16x2 wv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wv[4 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 0);
            wv[4 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 1);
            wv[4 * q + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 2);
            wv[4 * q + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[q], sc, 3);
        }
        const float ws = fast ? 1.0f : e8m0_f32(w[r].s);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t xd[4] = {xq[v][q].x, xq[v][q].y, xq[v][q].z, xq[v][q].w};
                d0 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 0], __builtin_bit_cast(bf16x2, xd[0]), d0, false);
                d1 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 1], __builtin_bit_cast(bf16x2, xd[1]), d1, false);
                d0 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 2], __builtin_bit_cast(bf16x2, xd[2]), d0, false);
                d1 = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * q + 3], __builtin_bit_cast(bf16x2, xd[3]), d1, false);
            }
            // slow path: the activation scale first, the power of two last, so
            // a tiny weight scale does not underflow a product of two scales
            acc[r][v] = fast ? __builtin_fmaf(d0 + d1, xs[v], acc[r][v])
                             : __builtin_fmaf((d0 + d1) * xs[v], ws, acc[r][v]);
        }
    }
}

// CB2 x int8: selectors (w >> 2j) & 0x03030303 hold raw codes; v_dot4 with
// the transposed activations gives dot(c, q) exactly in int32, and the
// block's integer sum is 2*dot + (-3*sum q).
template <int F, int LPR, int RT, int NV>
__device__ __forceinline__ void mac_cb2(const Unit<F> (&w)[RT], const uint8_t *lds,
                                        int vec_bytes, int xbytes, int u0, int cu, float (&acc)[RT][NV])
{
    const int u = u0 + cu * LPR;
    constexpr int NB = (F == kCB2) ? 2 : 1;      // 32-blocks per unit
    constexpr int CH = 2 * NB;                   // 16-byte chunks per unit
    uint4 xq[NV][CH];
    float xsh[NV][NB];
    int nq[NV][NB];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint8_t *base = lds + v * vec_bytes;
#pragma unroll
        for (int q = 0; q < CH; ++q)
            xq[v][q] = lds_read16(base + 16 * chunk_at<CH, LPR>(u0, cu, q));
        if constexpr (NB == 2) {
            const uint4 sd = lds_read16(base + xbytes + 16 * u);
            xsh[v][0] = __uint_as_float(sd.x);
            xsh[v][1] = __uint_as_float(sd.y);
            nq[v][0] = (int)sd.z;
            nq[v][1] = (int)sd.w;
        } else {
            const uint2 sd = *(const uint2 *)(base + xbytes + 8 * u);
            xsh[v][0] = __uint_as_float(sd.x);
            nq[v][0] = (int)sd.y;
        }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        uint32_t cw[CH];
        if constexpr (NB == 2) { cw[0] = w[r].c.x; cw[1] = w[r].c.y; cw[2] = w[r].c.z; cw[3] = w[r].c.w; }
        else { cw[0] = w[r].c.x; cw[1] = w[r].c.y; }
        uint32_t sel[CH][4];
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            sel[q][0] = cw[q] & 0x03030303u;
            sel[q][1] = (cw[q] >> 2) & 0x03030303u;
            sel[q][2] = (cw[q] >> 4) & 0x03030303u;
            sel[q][3] = (cw[q] >> 6) & 0x03030303u;
        }
        float ws[NB];
        ws[0] = f16_lo(w[r].s);
        if constexpr (NB == 2) ws[1] = f16_hi(w[r].s);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint4 x0 = xq[v][2 * b], x1 = xq[v][2 * b + 1];
                int d0 = __builtin_amdgcn_sdot4((int)sel[2 * b][0], (int)x0.x, 0, false);
                int d1 = __builtin_amdgcn_sdot4((int)sel[2 * b + 1][0], (int)x1.x, 0, false);
                d0 = __builtin_amdgcn_sdot4((int)sel[2 * b][1], (int)x0.y, d0, false);
                d1 = __builtin_amdgcn_sdot4((int)sel[2 * b + 1][1], (int)x1.y, d1, false);
                d0 = __builtin_amdgcn_sdot4((int)sel[2 * b][2], (int)x0.z, d0, false);
                d1 = __builtin_amdgcn_sdot4((int)sel[2 * b + 1][2], (int)x1.z, d1, false);
                d0 = __builtin_amdgcn_sdot4((int)sel[2 * b][3], (int)x0.w, d0, false);
                d1 = __builtin_amdgcn_sdot4((int)sel[2 * b + 1][3], (int)x1.w, d1, false);
                const int S = 2 * (d0 + d1) + nq[v][b];
                acc[r][v] = __builtin_fmaf((float)S, ws[b] * xsh[v][b], acc[r][v]);
            }
        }
    }
}

// CB3 x int8: the 16 codes of a half-block (two 24-bit triples A, B) become
// four selector dwords with one byte permute of the code bytes, one packed
// 16-bit shift and a mask each (straddling codes take two); a byte-permute
// lookup of {0,1,2,4,-6,-1,-2,-4} (twice the codebook) turns selectors into
// int8 values (lucebox-hub PR #21, Changes 'fp3' item 1: v_perm_b32 over an
// 8-byte LUT), and v_dot4 sums them exactly per half-block.
constexpr uint32_t kCb3LutLo = 0x04020100u;   // codes 0..3 -> 0, 1, 2, 4
constexpr uint32_t kCb3LutHi = 0xFCFEFFFAu;   // codes 4..7 -> -6, -1, -2, -4

template <int OFF>   // byte offset of triple A inside the (hi:lo) dword pair
__device__ __forceinline__ int cb3_half(uint32_t hi, uint32_t lo, uint4 x)
{
    constexpr uint32_t A0 = OFF, A1 = OFF + 1, A2 = OFF + 2, B0 = OFF + 3, B1 = OFF + 4, B2 = OFF + 5;
    const uint32_t q0 = perm(hi, lo, A0 | (B0 << 8) | (A0 << 16) | (B0 << 24));
    const uint32_t q1 = perm(hi, lo, A1 | (B1 << 8) | (A1 << 16) | (B1 << 24));
    const uint32_t q2 = perm(hi, lo, A2 | (B2 << 8) | (A2 << 16) | (B2 << 24));
    const uint32_t q3 = perm(hi, lo, A0 | (A1 << 8) | (B0 << 16) | (B1 << 24));
    const uint32_t q4 = perm(hi, lo, A1 | (A2 << 8) | (B1 << 16) | (B2 << 24));
    const uint32_t s0 = pk_shr<0, 3>(q0) & 0x07070707u;            // codes 0 8 1 9
    const uint32_t s1 = pk_shr<1, 4>(q1) & 0x07070707u;            // codes 3 11 4 12
    const uint32_t s2 = pk_shr<2, 5>(q2) & 0x07070707u;            // codes 6 14 7 15
    const uint32_t s3 = (pk_shr<6, 6>(q3) & 0x00070007u) |
                        ((pk_shr<7, 7>(q4) & 0x00070007u) << 8);   // codes 2 5 10 13
    int d = __builtin_amdgcn_sdot4((int)perm(kCb3LutHi, kCb3LutLo, s0), (int)x.x, 0, false);
    d = __builtin_amdgcn_sdot4((int)perm(kCb3LutHi, kCb3LutLo, s1), (int)x.y, d, false);
    d = __builtin_amdgcn_sdot4((int)perm(kCb3LutHi, kCb3LutLo, s2), (int)x.z, d, false);
    return __builtin_amdgcn_sdot4((int)perm(kCb3LutHi, kCb3LutLo, s3), (int)x.w, d, false);
}

template <int LPR, int RT, int NV>
__device__ __forceinline__ void mac_cb3(const Unit<kCB3> (&w)[RT], const uint8_t *lds,
                                        int vec_bytes, int xbytes, int u0, int cu, float (&acc)[RT][NV])
{
    const int u = u0 + cu * LPR;
    uint4 xq[NV][2];
    float xsh[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint8_t *base = lds + v * vec_bytes;
        xq[v][0] = lds_read16(base + 16 * chunk_at<2, LPR>(u0, cu, 0));
        xq[v][1] = lds_read16(base + 16 * chunk_at<2, LPR>(u0, cu, 1));
        xsh[v] = ((const float *)(base + xbytes))[u];
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const float ws0 = f16_lo(w[r].s), ws1 = f16_hi(w[r].s);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int S0 = cb3_half<0>(w[r].c.y, w[r].c.x, xq[v][0]);
            const int S1 = cb3_half<2>(w[r].c.z, w[r].c.y, xq[v][1]);
            const float t = __builtin_fmaf(ws1, (float)S1, ws0 * (float)S0);
            acc[r][v] = __builtin_fmaf(t, xsh[v], acc[r][v]);
        }
    }
}

// ------------------------------------------------------------------ row body
// Sum a value over the LPR lanes of a row (lane groups aligned to LPR) with a
// fixed butterfly: DPP quad permutes and row mirrors within 16 lanes,
// ds_swizzle across 16, readlane across 32.  After each step every lane of a
// group holds the same bits (a + b == b + a), so the result is reproducible.
template <int CTRL>
__device__ __forceinline__ float dpp_step(float v)
{
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int LPR>
__device__ __forceinline__ float group_sum(float v)
{
    v = dpp_step<0xB1>(v);                          // quad_perm [1,0,3,2]
    v = dpp_step<0x4E>(v);                          // quad_perm [2,3,0,1]
    v = dpp_step<0x141>(v);                         // row_half_mirror
    if constexpr (LPR >= 16) v = dpp_step<0x140>(v);  // row_mirror
    if constexpr (LPR >= 32)
        v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // lane ^ 16
    if constexpr (LPR >= 64)
        v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return v;
}

// Code bytes are read exactly once per call, in whole cache lines per wave
// instruction, so they are streamed with the non-temporal cache policy (aux
// bit 1, "nt"): on MI355X this lifts a cold 17 MB gather read from about 3.9
// to 4.4 TB/s.  Scale loads touch only part of a line per instruction and
// the next unit step reads the rest, so they keep the default policy.
constexpr int kStream = 2;

template <int F>
__device__ __forceinline__ uint32_t load_scale(__amdgpu_buffer_rsrc_t rs, uint32_t os)
{
    if constexpr (F == kMXFP4 || F == kMXFP4I) return __builtin_amdgcn_raw_buffer_load_b8(rs, os, 0, 0);
    else if constexpr (F == kCB2S) return __builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0);
}

template <int F>
__device__ __forceinline__ void load_codes(Unit<F> &w, __amdgpu_buffer_rsrc_t rc, uint32_t oc)
{
    if constexpr (F == kMXFP4 || F == kCB2 || F == kMXFP4I) w.c = __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, kStream);
    else if constexpr (F == kCB2S) w.c = __builtin_amdgcn_raw_buffer_load_b64(rc, oc, 0, kStream);
    else w.c = __builtin_amdgcn_raw_buffer_load_b96(rc, oc, 0, kStream);
}

// Loads of one segment: every scale first (1/17 to 1/4 of the bytes), then
// the codes of unit steps c (all RT rows of step c) on demand.
// Offsets are relative to the lane's first unit (oc/os include li * bytes);
// a unit past the row end is redirected to the row's last unit, which another
// lane of the same instruction reads anyway, so it costs no extra traffic.
template <int F, int LPR, int CPL, int RT>
__device__ __forceinline__ void load_scales(Unit<F> (&w)[CPL][RT], const __amdgpu_buffer_rsrc_t (&rs)[RT],
                                            const uint32_t (&os)[RT], int seg_unit, int li, int U)
{
    constexpr int SB = Unit<F>::SB;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int du = min(seg_unit + c * LPR, U - 1 - li);
#pragma unroll
        for (int r = 0; r < RT; ++r) w[c][r].s = load_scale<F>(rs[r], os[r] + du * SB);
    }
}

template <int F, int LPR, int CPL, int RT>
__device__ __forceinline__ void load_step(Unit<F> (&w)[CPL][RT], const __amdgpu_buffer_rsrc_t (&rc)[RT],
                                          const uint32_t (&oc)[RT], int seg_unit, int li, int U, int c)
{
    constexpr int CB = Unit<F>::CB;
    const int du = min(seg_unit + c * LPR, U - 1 - li);
#pragma unroll
    for (int r = 0; r < RT; ++r) load_codes<F>(w[c][r], rc[r], oc[r] + du * CB);
}

// Unit steps whose code loads are in flight ahead of the step being computed.
// Vector-memory loads of a wave complete in issue order, so a long lead makes
// early steps wait behind later requests, and a short one exposes more of
// each request's latency.  Measured on MI355X (weights rotated past the
// Infinity Cache), A/B in one process: the MXFP4 x bf16 gather/dense kernel
// is fastest with 3 steps of lead (the gpt-oss gather, 3 units per lane:
// 5.94 -> 5.78 us; the 4-token gather, 7 units per lane: 23.9 -> 23.4 us;
// the fused gate/up and the tiny dense call unchanged); every other kernel
// with 1: 2-bit and 3-bit weights +2-3% at lead 2 or 3, MXFP4 x int8 +4.6%,
// and the combine kernel, whose lanes carry 4 slots' rows, +14% at lead 3.
template <int F, int CPL> struct Lead {
    static constexpr int want = F == kMXFP4 ? 3 : 1;
    static constexpr int v = want < CPL ? want : CPL;
};
template <int CPL> struct Lead1 {                  // the combine kernel
    static constexpr int v = 1 < CPL ? 1 : CPL;
};

template <int F, int LPR, int CPL, int RT, int NV>
__device__ __forceinline__ void mac_seg(Unit<F> (&w)[CPL][RT], const Args &a, const uint8_t *lds,
                                        const __amdgpu_buffer_rsrc_t (&rc)[RT], const uint32_t (&oc)[RT],
                                        int seg_unit, int u0, int U, float (&acc)[RT][NV])
{
    constexpr int LEAD = Lead<F, CPL>::v;
    const int xbytes = U * Fmt<F>::XB;
    bool fast = true;              // MXFP4: every scale byte of the segment in [2, 252]
    if constexpr (F == kMXFP4 || F == kMXFP4I) {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int r = 0; r < RT; ++r) fast = fast && (w[c][r].s - 2u) <= 250u;
        fast = __all(fast);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (c + LEAD < CPL) load_step<F, LPR, CPL, RT>(w, rc, oc, seg_unit, u0 - seg_unit, U, c + LEAD);
        if (u0 + c * LPR < U) {
            if constexpr (F == kMXFP4) mac_mxfp4<LPR, RT, NV>(w[c], lds, a.lds_vec_bytes, u0, c, fast, acc);
            else if constexpr (F == kMXFP4I) mac_mxfp4i<LPR, RT, NV>(w[c], lds, a.lds_vec_bytes, xbytes, u0, c, fast, acc);
            else if constexpr (F == kCB3) mac_cb3<LPR, RT, NV>(w[c], lds, a.lds_vec_bytes, xbytes, u0, c, acc);
            else mac_cb2<F, LPR, RT, NV>(w[c], lds, a.lds_vec_bytes, xbytes, u0, c, acc);
        }
    }
}

// y = silu(g) * u with silu(g) = g / (1 + e^-g), in f32 (SwiGLU, the gated
// activation between an MoE expert's gate/up and down projections).
__device__ __forceinline__ float swiglu(float g, float u)
{
    return g / (1.0f + __expf(-g)) * u;
}

// One workgroup, one item, one tile of rows.  Order of work per lane:
//   1. activation staging loads (registers)
//   2. all scale loads, then code loads one unit step ahead (load_step)
//   3. activations to LDS, barrier (waits only for the staging loads)
//   4. per unit, as its bytes arrive: decode and dot (progressive vmcnt)
//   5. further segments when K needs them; butterfly; store.
// MODE 0: the lane's RT rows are RT consecutive output rows.  MODE 1 (gate/up,
// RT == 2): the lane's two rows are row n of the gate and row n of the up
// projection, and the store writes swiglu(gate, up).
// STAGE = false: the activations of `it` are already in LDS (the grouped
// kernel's next row tile of the same vectors): no loads, no barrier.
template <int F, int LPR, int CPL, int RT, int NV, int NVMAX, int MODE, bool Q, bool GR = false,
          bool STAGE = true>
__device__ __forceinline__ void rows_body(const Args &a, const Item &it, uint8_t *lds, int row_base,
                                          uint4 (&xr)[kXReg])
{
    static_assert(MODE == 0 || RT == 2, "gate/up rows come in pairs");
    constexpr int SLOTS = 64 / LPR;
    constexpr int SEG = LPR * CPL;
    constexpr int NROW = MODE == 0 ? RT : 1;                  // output rows per lane
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane / LPR;
    const int li = lane % LPR;
    const int row0 = row_base + (wave * SLOTS + slot) * NROW;
    const int U = a.units;
    __amdgpu_buffer_rsrc_t rc[RT], rs[RT];
    uint32_t oc[RT], os[RT];           // rows past N land past the expert's end: zeros
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const bool up = MODE == 1 && r == 1;
        rc[r] = buffer_rsrc((up ? a.codes2 : a.codes) + (long long)it.expert * a.expert_cb, a.expert_cb);
        rs[r] = buffer_rsrc((up ? a.scales2 : a.scales) + (long long)it.expert * a.expert_sb, a.expert_sb);
        const int n = row0 + (MODE == 0 ? r : 0);
        oc[r] = (uint32_t)__umul24(n, a.rcb) + li * Unit<F>::CB;
        os[r] = (uint32_t)__umul24(n, a.rsb) + li * Unit<F>::SB;
    }

    if constexpr (STAGE) {
        if (!a.x_early) xload<F, NVMAX, Q>(a, it, xr);
    }
    Unit<F> w[CPL][RT];
    load_scales<F, LPR, CPL, RT>(w, rs, os, 0, li, U);
#pragma unroll
    for (int c = 0; c < Lead<F, CPL>::v; ++c) load_step<F, LPR, CPL, RT>(w, rc, oc, 0, li, U, c);
    if constexpr (STAGE) {
        xstore<F, NVMAX, Q>(a, it, lds, xr);
        __syncthreads();
        if (xrest<F, NVMAX, Q>(a, it, lds)) __syncthreads();
    }

    float acc[RT][NV];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[r][v] = 0.0f;

    const int nseg = (U + SEG - 1) / SEG;
    for (int seg = 0;;) {
        mac_seg<F, LPR, CPL, RT, NV>(w, a, lds, rc, oc, seg * SEG, seg * SEG + li, U, acc);
        if (++seg >= nseg) break;
        load_scales<F, LPR, CPL, RT>(w, rs, os, seg * SEG, li, U);
#pragma unroll
        for (int c = 0; c < Lead<F, CPL>::v; ++c) load_step<F, LPR, CPL, RT>(w, rc, oc, seg * SEG, li, U, c);
    }

#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[r][v] = group_sum<LPR>(acc[r][v]);

    // Lane li < NROW stores row row0 + li for every vector and destination.
    if (li < NROW) {
        const int n = row0 + li;
        if (n < a.N) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float val;
                if constexpr (MODE == 1) {
                    val = swiglu(acc[0][v], acc[1][v]);
                } else {
                    val = acc[0][v];
#pragma unroll
                    for (int r = 1; r < RT; ++r) val = (li == r) ? acc[r][v] : val;
                }
                if constexpr (GR) {
                    a.y[it.pair[v] * a.N + n] = val;            // M * top_k * N < 2^31
                } else {
                    unsigned long long d = it.dest[v];
                    while (d) {
                        const int p = __ffsll((long long)d) - 1;
                        d &= d - 1ull;
                        a.y[p * a.N + n] = val;                 // M * top_k * N < 2^31
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ kernel
// F: format kind; LPR: lanes per row; CPL: units per lane and row in flight;
// RT: rows per lane; NVMAX: most activation vectors one item may carry;
// Q: bf16 activations quantized to int8 blocks while staged.
template <int F, int LPR, int CPL, int RT, int NVMAX, int MODE, bool Q>
__global__ __launch_bounds__(kThreads) void qmv_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint4 xr[kXReg];
    if (a.x_early) xload<F, NVMAX, Q>(a, early_item(a), xr);   // in flight while the ids arrive
    Item it;
    if constexpr (NVMAX == 1) it = route_one(a, blockIdx.y);
    else it = route(a, blockIdx.y);
    if (it.kind < 0) return;
    const int row_base = blockIdx.x * a.rows_per_tile;
    if (it.kind == 1) {
        const int p = __ffsll((long long)it.dest[0]) - 1;
        const int end = min(a.N, row_base + a.rows_per_tile);
        for (int n = row_base + threadIdx.x; n < end; n += kThreads)
            a.y[p * a.N + n] = 0.0f;
        return;
    }
    if constexpr (NVMAX == 1) {
        rows_body<F, LPR, CPL, RT, 1, 1, MODE, Q>(a, it, lds, row_base, xr);
    } else {
        switch (it.nv) {
        case 1: rows_body<F, LPR, CPL, RT, 1, NVMAX, MODE, Q>(a, it, lds, row_base, xr); break;
        case 2: rows_body<F, LPR, CPL, RT, 2, NVMAX, MODE, Q>(a, it, lds, row_base, xr); break;
        case 3: rows_body<F, LPR, CPL, RT, 3, NVMAX, MODE, Q>(a, it, lds, row_base, xr); break;
        default: rows_body<F, LPR, CPL, RT, 4, NVMAX, MODE, Q>(a, it, lds, row_base, xr); break;
        }
    }
}

// ------------------------------------------------------------------ grouped
// More than 4 tokens (a prefill chunk, a wide verify batch) for every format
// pair: the expert-batched gather of the pages (mlxcel issue #2178, "Problem /
// Background"; lucebox-hub PR #19, "Depends on": the verify-batch matmul),
// taken as groups of up to four of an expert's vectors through the decode
// kernel's own staging, decode, integer block dots and scale epilogue.
//
// The grid is (row tile, expert slot), with min(E, pairs) slots: slot y
// takes the y-th smallest expert id the call selects (a bitmap of the
// selected experts in LDS; no device-wide sort) and leaves at once when the
// call selects fewer.  A workgroup lists its expert's (token, slot) pairs in
// index order with ballots (the same list in every workgroup, no atomics),
// then streams its rows once per group of four vectors (the first pass from
// memory, the later ones mostly from L2).  The tiles of slot 0 also write
// the zero rows of pairs whose id is outside [0, E).  A dense call is one
// expert with the vectors in index order.

// Pair listing: with B <= 8192 pairs and workgroups of 64 to 512 threads
// there are at most 8192 / 64 + 7 = 135 (round, wave) counts; the scan takes
// up to 4 per lane.
constexpr int kMaxCounts = kPairCounts;

// LDS past a workgroup's activation area: the (round, wave) counts and their
// total (kPairCountBytes) and the expert's pair list (16-bit pair indices).
struct PairList {
    int *cnt;
    uint16_t *perm;
};

// Eight rounds of ids: v[j] = ids[tid + (j0 + j) * THREADS] (index clamped to
// B - 1 so every lane loads; rounds past the last hold E).  A workgroup loads
// the first eight rounds once and hands them to every scan below, so calls
// with up to 8 * THREADS pairs read their ids once per workgroup.
struct Ids8 {
    int v[8];
};

template <int THREADS>
__device__ __forceinline__ Ids8 load_ids8(const int32_t *ids, int B, int E, int j0)
{
    const int rounds = (B + THREADS - 1) / THREADS;
    Ids8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        r.v[j] = E;
        if (j0 + j < rounds) r.v[j] = ids[min((int)threadIdx.x + (j0 + j) * THREADS, B - 1)];
    }
    return r;
}

// Bits j of the result: pair tid + (j0 + j) * THREADS (id idv.v[j]) exists
// and is in bucket `bucket` (an expert, or -1 for ids outside [0, E)).
template <int THREADS>
__device__ __forceinline__ uint32_t match8(Ids8 idv, int B, int E, int bucket, int j0)
{
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const bool inb = (int)threadIdx.x + (j0 + j) * THREADS < B;
        const int e = idv.v[j];
        const bool hit = inb && (bucket >= 0 ? e == bucket : (unsigned)e >= (unsigned)E);
        m |= (uint32_t)hit << j;
    }
    return m;
}

// The pairs of bucket `bucket` in index order, written to L.perm; returns
// their number.  Thread tid looks at the ids i = tid + j * THREADS (the first
// eight rounds from `first`, later ones loaded here): a ballot per round j
// gives each wave's matches, one wave turns the (round, wave) counts into
// offsets, and a second pass writes each match at its rank.  The list is the
// same in every workgroup and needs no atomics.  Needs B <= 8192.
// (The ids, pair count and expert count come by value: a reference to the
// kernel's argument block would make the compiler copy it to scratch.)
template <int THREADS>
__device__ __forceinline__ int list_pairs(const int32_t *ids, int B, int E, int bucket, PairList L, Ids8 first)
{
    constexpr int W = THREADS / 64;
    static_assert((8192 + THREADS - 1) / THREADS * W <= kMaxCounts, "pair-list counts");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rounds = (B + THREADS - 1) / THREADS;
    for (int j0 = 0; j0 < rounds; j0 += 8) {
        const Ids8 idv = j0 == 0 ? first : load_ids8<THREADS>(ids, B, E, j0);
        const uint32_t m8 = match8<THREADS>(idv, B, E, bucket, j0);
        for (int j = 0; j < 8 && j0 + j < rounds; ++j) {
            const unsigned long long bal = __ballot((m8 >> j) & 1u);
            if (lane == 0) L.cnt[(j0 + j) * W + w] = __popcll(bal);
        }
    }
    __syncthreads();
    if (w == 0) {                                   // exclusive scan of the counts, 4 per lane
        const int n = rounds * W;
        int v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = 4 * lane + q < n ? L.cnt[4 * lane + q] : 0;
        const int mine = v[0] + v[1] + v[2] + v[3];
        int s = mine;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(s, d);
            if (lane >= d) s += t;
        }
        int ex = s - mine;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (4 * lane + q < n) L.cnt[4 * lane + q] = ex;
            ex += v[q];
        }
        if (lane == 63) L.cnt[kMaxCounts] = s;
    }
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j0 = 0; j0 < rounds; j0 += 8) {
        const Ids8 idv = j0 == 0 ? first : load_ids8<THREADS>(ids, B, E, j0);
        const uint32_t m8 = match8<THREADS>(idv, B, E, bucket, j0);
        for (int j = 0; j < 8 && j0 + j < rounds; ++j) {
            const bool m = (m8 >> j) & 1u;
            const unsigned long long bal = __ballot(m);
            if (m)
                L.perm[L.cnt[(j0 + j) * W + w] + __popcll(bal & below)] =
                    (uint16_t)(threadIdx.x + (j0 + j) * THREADS);
        }
    }
    const int total = L.cnt[kMaxCounts];
    __syncthreads();
    return total;
}

// bm[0..32) = the set of expert ids in [0, E) that occur in ids[0..B)
// (E <= 1024), in LDS; returns the set's size.
template <int THREADS>
__device__ __forceinline__ int expert_bitmap(const int32_t *ids, int B, int E, uint32_t *bm, Ids8 first)
{
    const int tid = threadIdx.x;
    const int rounds = (B + THREADS - 1) / THREADS;
    if (tid < 32) bm[tid] = 0u;
    __syncthreads();
    for (int j0 = 0; j0 < rounds; j0 += 8) {
        const Ids8 idv = j0 == 0 ? first : load_ids8<THREADS>(ids, B, E, j0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = idv.v[j];
            if (tid + (j0 + j) * THREADS < B && (unsigned)e < (unsigned)E)
                atomicOr(&bm[e >> 5], 1u << (e & 31));
        }
    }
    __syncthreads();
    if (tid < 64) {
        int c = tid < 32 ? __popc(bm[tid]) : 0;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
        if (tid == 0) bm[33] = (uint32_t)c;
    }
    __syncthreads();
    return (int)bm[33];
}

// The y-th smallest id in the bitmap, or -1 when it holds fewer than y + 1;
// bm[32] carries the answer to every wave.  Every thread reads it before the
// next barrier, so the next call cannot overwrite it early.
__device__ __forceinline__ int kth_expert(uint32_t *bm, int y)
{
    const int tid = threadIdx.x;
    if (tid < 64) {                                 // wave 0: 32 bitmap words
        const uint32_t word = tid < 32 ? bm[tid] : 0u;
        const int c = __popc(word);
        int s = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(s, d);
            if (tid >= d) s += t;
        }
        if (y >= s - c && y < s) {                  // the word that holds it
            uint32_t w = word;
            for (int k = y - (s - c); k > 0; --k) w &= w - 1u;
            bm[32] = (uint32_t)(32 * tid + __builtin_ctz(w));
        } else if (tid == 63 && y >= s) {
            bm[32] = 0xFFFFFFFFu;
        }
    }
    __syncthreads();
    return (int)bm[32];
}

// One group of up to four of an expert's vectors over one row tile.
template <int F, int LPR, int CPL, int MODE, bool Q, bool STAGE>
__device__ __forceinline__ void grouped_rows(const Args &a, const Item &it, uint8_t *lds, int row_base)
{
    constexpr int RT = 2;
    uint4 xr[kXReg];
    switch (it.nv) {
    case 1: rows_body<F, LPR, CPL, RT, 1, 4, MODE, Q, true, STAGE>(a, it, lds, row_base, xr); break;
    case 2: rows_body<F, LPR, CPL, RT, 2, 4, MODE, Q, true, STAGE>(a, it, lds, row_base, xr); break;
    case 3: rows_body<F, LPR, CPL, RT, 3, 4, MODE, Q, true, STAGE>(a, it, lds, row_base, xr); break;
    default: rows_body<F, LPR, CPL, RT, 4, 4, MODE, Q, true, STAGE>(a, it, lds, row_base, xr); break;
    }
}

// Work items are (expert slot, row tile) in slot-major order, over the D
// distinct experts the call selects (counted in every workgroup from the
// bitmap); workgroup b takes the contiguous run [b T / G, (b + 1) T / G) of
// the T = D * tiles items (G workgroups, at most one round of the chip), so
// every workgroup gets the same number of row tiles within one, and a run
// changes expert at most a few times.  Per expert the pair list is rebuilt; per row tile the groups
// of four vectors are streamed, and when the expert has at most four vectors
// they stay staged in LDS from one row tile to the next.
template <int F, int LPR, int CPL, int MODE, bool Q>
__global__ __launch_bounds__(kThreads) void qmv_grouped_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const bool gather = a.ids != nullptr;
    uint8_t *tail = lds + 4 * a.lds_vec_bytes;
    PairList L;
    L.cnt = (int *)tail;
    uint32_t *bm = (uint32_t *)(tail + kPairCountBytes);
    L.perm = (uint16_t *)(tail + kPairCountBytes + kExpertBitmapBytes);
    const int tiles = a.gr_tiles, rpt = a.rows_per_tile;
    const int B = a.M * a.top_k;
    Ids8 id0;
    int D = 1;
    if (gather) {
        id0 = load_ids8<kThreads>(a.ids, B, a.E, 0);
        D = expert_bitmap<kThreads>(a.ids, B, a.E, bm, id0);
    }
    const long long T = (long long)D * tiles;
    const int i0 = (int)((long long)blockIdx.x * T / gridDim.x);
    const int i1 = (int)((long long)(blockIdx.x + 1) * T / gridDim.x);
    if (gather) {
        // the zero rows of pairs whose id is outside [0, E), row tiles dealt
        // in runs like the items
        const int z0 = (int)((long long)blockIdx.x * tiles / gridDim.x);
        const int z1 = (int)((long long)(blockIdx.x + 1) * tiles / gridDim.x);
        if (z1 > z0) {
            const int ci = list_pairs<kThreads>(a.ids, B, a.E, -1, L, id0);
            const int n0 = z0 * rpt;
            const int rows = min(a.N, z1 * rpt) - n0;
            for (int o = threadIdx.x; o < ci * rows; o += kThreads)
                a.y[(int)L.perm[o / rows] * a.N + n0 + o % rows] = 0.0f;
            __syncthreads();
        }
    }
    int cur = -1, c = 0, e = 0;
    bool staged = false;
    for (int i = i0; i < i1; ++i) {
        const int slot = i / tiles;
        const int row_base = (i - slot * tiles) * rpt;
        if (slot != cur) {
            cur = slot;
            staged = false;
            if (gather) {
                e = kth_expert(bm, slot);           // slot < D: a selected expert
                c = list_pairs<kThreads>(a.ids, B, a.E, e, L, id0);
            } else {
                c = a.M;
            }
        }
        for (int g = 0; g < c; g += 4) {
            Item it;
            it.kind = 0;
            it.expert = e;
            it.nv = min(4, c - g);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // the pair list is the same in every lane: scalar registers
                const int p = __builtin_amdgcn_readfirstlane(
                    gather ? (int)L.perm[g + (m < it.nv ? m : 0)] : g + (m < it.nv ? m : 0));
                it.pair[m] = p;
                it.vec[m] = gather && !a.x_per_slot ? p / a.top_k : p;
                it.dest[m] = 0ull;
            }
            if (staged && c <= 4)
                grouped_rows<F, LPR, CPL, MODE, Q, false>(a, it, lds, row_base);
            else
                grouped_rows<F, LPR, CPL, MODE, Q, true>(a, it, lds, row_base);
            if (c > 4) __syncthreads();             // the next group restages the activations
        }
        staged = true;
    }
}

// ------------------------------------------------------------------ combine
// Down projection with the router-weighted top-k combine:
//     y[t][n] = sum_j  w[t][j] * g(t, j, n),   g = the gather output of slot j
// (zero for an expert id outside [0, E)).  A workgroup owns token t
// (blockIdx.y) and a tile of rows; each lane keeps row n of up to four of the
// token's slots in flight at once (the four slots' experts are four buffer
// resources), so the slots' dot products of a row end in the same lane group
// and the weighted sum is formed in registers, in slot order, with no second
// pass over memory and no atomics.  Slots beyond the fourth are taken four at
// a time by the same workgroup.  The activation vector of slot j is x[t][j]
// (or x[t] for every slot when x_per_slot == 0), known before the ids arrive,
// so its staging loads are issued first.
constexpr int kCombineRT = 4;        // slots per pass

__device__ __forceinline__ Item combine_item(const Args &a, int t, int g)
{
    Item it;
    it.kind = 0;
    it.expert = 0;
    it.nv = a.x_per_slot ? min(4, a.top_k - 4 * g) : 1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        it.vec[m] = a.x_per_slot ? t * a.top_k + 4 * g + m : t;
        it.dest[m] = 0ull;
        it.pair[m] = 0;
    }
    return it;
}

// One unit step of the combine: row r (slot 4g + r) is dotted with its own
// staged vector (vo[r] bytes into LDS) only; rows of invalid slots are
// skipped (wave-uniform) and keep a zero sum.
template <int F, int LPR, int CPL, int RT>
__device__ __forceinline__ void mac_seg_diag(Unit<F> (&w)[CPL][RT], const Args &a, const uint8_t *lds,
                                             const __amdgpu_buffer_rsrc_t (&rc)[RT], const uint32_t (&oc)[RT],
                                             const int (&vo)[RT], const bool (&valid)[RT],
                                             int seg_unit, int u0, int U, float (&acc)[RT])
{
    constexpr int LEAD = Lead1<CPL>::v;
    const int xbytes = U * Fmt<F>::XB;
    bool fast = true;
    if constexpr (F == kMXFP4 || F == kMXFP4I) {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int r = 0; r < RT; ++r) fast = fast && (!valid[r] || (w[c][r].s - 2u) <= 250u);
        fast = __all(fast);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (c + LEAD < CPL) load_step<F, LPR, CPL, RT>(w, rc, oc, seg_unit, u0 - seg_unit, U, c + LEAD);
        if (u0 + c * LPR < U) {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                if (!valid[r]) continue;
                const Unit<F>(&w1)[1] = *reinterpret_cast<const Unit<F>(*)[1]>(&w[c][r]);
                float(&a1)[1][1] = *reinterpret_cast<float(*)[1][1]>(&acc[r]);
                const uint8_t *l = lds + vo[r];
                if constexpr (F == kMXFP4) mac_mxfp4<LPR, 1, 1>(w1, l, 0, u0, c, fast, a1);
                else if constexpr (F == kMXFP4I) mac_mxfp4i<LPR, 1, 1>(w1, l, 0, xbytes, u0, c, fast, a1);
                else if constexpr (F == kCB3) mac_cb3<LPR, 1, 1>(w1, l, 0, xbytes, u0, c, a1);
                else mac_cb2<F, LPR, 1, 1>(w1, l, 0, xbytes, u0, c, a1);
            }
        }
    }
}

template <int F, int LPR, int CPL, bool Q>
__global__ __launch_bounds__(kThreads) void qmv_combine_kernel(const Args a)
{
    constexpr int RT = kCombineRT;
    constexpr int SLOTS = 64 / LPR;
    constexpr int SEG = LPR * CPL;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane % LPR;
    const int n = blockIdx.x * a.rows_per_tile + wave * SLOTS + lane / LPR;
    const int U = a.units;
    const int ngroups = (a.top_k + RT - 1) / RT;

    Item it = combine_item(a, t, 0);
    uint4 xr[kXReg];
    xload<F, 4, Q>(a, it, xr);                     // in flight while the ids arrive
    int e_l = -1;
    float w_l = 0.0f;
    if (lane < a.top_k) {
        e_l = a.ids[t * a.top_k + lane];
        w_l = a.route_w[t * a.top_k + lane];
    }

    float y = 0.0f;
    for (int g = 0; g < ngroups; ++g) {
        __amdgpu_buffer_rsrc_t rc[RT], rs[RT];
        uint32_t oc[RT], os[RT];
        bool valid[RT];
        int vo[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int j = RT * g + r;
            const int e = __builtin_amdgcn_readlane(e_l, j);          // lane j < 16 < 64
            valid[r] = j < a.top_k && e >= 0 && e < a.E;
            const long long eo = valid[r] ? (long long)e : 0ll;      // invalid: empty resource, reads 0
            rc[r] = buffer_rsrc(a.codes + eo * a.expert_cb, valid[r] ? a.expert_cb : 0);
            rs[r] = buffer_rsrc(a.scales + eo * a.expert_sb, valid[r] ? a.expert_sb : 0);
            oc[r] = (uint32_t)__umul24(n, a.rcb) + li * Unit<F>::CB;
            os[r] = (uint32_t)__umul24(n, a.rsb) + li * Unit<F>::SB;
            vo[r] = a.x_per_slot ? r * a.lds_vec_bytes : 0;
        }
        const bool restage = g > 0 && a.x_per_slot;
        if (restage) {
            it = combine_item(a, t, g);
            xload<F, 4, Q>(a, it, xr);
        }
        Unit<F> w[CPL][RT];
        load_scales<F, LPR, CPL, RT>(w, rs, os, 0, li, U);
#pragma unroll
        for (int c = 0; c < Lead1<CPL>::v; ++c) load_step<F, LPR, CPL, RT>(w, rc, oc, 0, li, U, c);
        if (g == 0 || restage) {
            if (restage) __syncthreads();          // every wave is done with the last group's vectors
            xstore<F, 4, Q>(a, it, lds, xr);
            __syncthreads();
            if (xrest<F, 4, Q>(a, it, lds)) __syncthreads();
        }

        float acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = 0.0f;
        const int nseg = (U + SEG - 1) / SEG;
        for (int seg = 0;;) {
            mac_seg_diag<F, LPR, CPL, RT>(w, a, lds, rc, oc, vo, valid, seg * SEG, seg * SEG + li, U, acc);
            if (++seg >= nseg) break;
            load_scales<F, LPR, CPL, RT>(w, rs, os, seg * SEG, li, U);
#pragma unroll
            for (int c = 0; c < Lead1<CPL>::v; ++c) load_step<F, LPR, CPL, RT>(w, rc, oc, seg * SEG, li, U, c);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int j = RT * g + r;
            const float s = group_sum<LPR>(acc[r]);
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), j));
            if (j < a.top_k) y = __builtin_fmaf(wj, valid[r] ? s : 0.0f, y);
        }
    }
    if (li == 0 && n < a.N) a.y[t * a.N + n] = y;      // M * N < 2^31
}

// Kernel tables, one per format kind (qmv_k_*.hip): [variant][lpr][cpl].
extern const void *const kTable_mxfp4[3][4][5];
extern const void *const kTable_cb2[3][4][5];
extern const void *const kTable_cb2s[3][4][5];
extern const void *const kTable_cb3[3][4][5];
// Gate/up (SwiGLU) kernels: [variant 0 or 1][lpr][cpl].
extern const void *const kTableGU_mxfp4[2][4][5];
extern const void *const kTableGU_cb2[2][4][5];
extern const void *const kTableGU_cb2s[2][4][5];
extern const void *const kTableGU_cb3[2][4][5];
// Combine kernels: [lpr][cpl in {1, 2, 3, 4}].
extern const void *const kTableCB_mxfp4[4][4];
extern const void *const kTableCB_cb2[4][4];
extern const void *const kTableCB_cb2s[4][4];
extern const void *const kTableCB_cb3[4][4];
extern const void *const kTable_mxfp4i[3][4][5];
extern const void *const kTableGU_mxfp4i[2][4][5];
extern const void *const kTableCB_mxfp4i[4][4];
// Grouped kernels (more than 4 tokens): [mode 0 or 1][lpr][cpl]; built with
// 4-wave workgroups only.
extern const void *const kTableGR_mxfp4[2][4][5];
extern const void *const kTableGR_mxfp4i[2][4][5];
extern const void *const kTableGR_cb2[2][4][5];
extern const void *const kTableGR_cb2s[2][4][5];
extern const void *const kTableGR_cb3[2][4][5];
extern const void *const kTableQGR_cb2[2][4][5];
extern const void *const kTableQGR_cb2s[2][4][5];
extern const void *const kTableQGR_cb3[2][4][5];
// The same for bf16 activations quantized in staging (2-bit and 3-bit only).
extern const void *const kTableQ_cb2[3][4][5];
extern const void *const kTableQ_cb2s[3][4][5];
extern const void *const kTableQ_cb3[3][4][5];
extern const void *const kTableQGU_cb2[2][4][5];
extern const void *const kTableQGU_cb2s[2][4][5];
extern const void *const kTableQGU_cb3[2][4][5];
extern const void *const kTableQCB_cb2[4][4];
extern const void *const kTableQCB_cb2s[4][4];
extern const void *const kTableQCB_cb3[4][4];

}  // namespace QMV_NS

// Instantiate one format's kernel tables: [variant][lpr index][cpl index];
// Q selects bf16 activations quantized in staging.
#define QMV_K(F, V, L, C, MODE, Q) \
    (const void *)&::QMV_NS::qmv_kernel<F, L, C, ((V) == 2 ? 4 : 2), ((V) == 0 ? 1 : 4), MODE, Q>
#define QMV_ROW01(F, V, L, MODE, Q) \
    { QMV_K(F, V, L, 1, MODE, Q), QMV_K(F, V, L, 2, MODE, Q), QMV_K(F, V, L, 3, MODE, Q), \
      QMV_K(F, V, L, 4, MODE, Q), QMV_K(F, V, L, 7, MODE, Q) }
#define QMV_ROW2(F, V, L, Q) \
    { QMV_K(F, V, L, 1, 0, Q), QMV_K(F, V, L, 2, 0, Q), QMV_K(F, V, L, 4, 0, Q), nullptr, nullptr }
#define QMV_NOROW { nullptr, nullptr, nullptr, nullptr, nullptr }
#define QMV_TABLE(F, Q) \
    { { QMV_ROW01(F, 0, 8, 0, Q), QMV_ROW01(F, 0, 16, 0, Q), QMV_ROW01(F, 0, 32, 0, Q), QMV_ROW01(F, 0, 64, 0, Q) }, \
      { QMV_ROW01(F, 1, 8, 0, Q), QMV_ROW01(F, 1, 16, 0, Q), QMV_ROW01(F, 1, 32, 0, Q), QMV_ROW01(F, 1, 64, 0, Q) }, \
      { QMV_NOROW, QMV_ROW2(F, 2, 16, Q), QMV_ROW2(F, 2, 32, Q), QMV_ROW2(F, 2, 64, Q) } }
#define QMV_KC(F, L, C, Q) (const void *)&::QMV_NS::qmv_combine_kernel<F, L, C, Q>
#define QMV_ROWC(F, L, Q) { QMV_KC(F, L, 1, Q), QMV_KC(F, L, 2, Q), QMV_KC(F, L, 3, Q), QMV_KC(F, L, 4, Q) }
#define QMV_TABLE_CB(F, Q) { QMV_ROWC(F, 8, Q), QMV_ROWC(F, 16, Q), QMV_ROWC(F, 32, Q), QMV_ROWC(F, 64, Q) }
#define QMV_TABLE_GU(F, Q) \
    { { QMV_ROW01(F, 0, 8, 1, Q), QMV_ROW01(F, 0, 16, 1, Q), QMV_ROW01(F, 0, 32, 1, Q), QMV_ROW01(F, 0, 64, 1, Q) }, \
      { QMV_ROW01(F, 1, 8, 1, Q), QMV_ROW01(F, 1, 16, 1, Q), QMV_ROW01(F, 1, 32, 1, Q), QMV_ROW01(F, 1, 64, 1, Q) } }
#define QMV_KG(F, L, C, MODE, Q) (const void *)&::QMV_NS::qmv_grouped_kernel<F, L, C, MODE, Q>
#define QMV_ROWG(F, L, MODE, Q) \
    { QMV_KG(F, L, 1, MODE, Q), QMV_KG(F, L, 2, MODE, Q), QMV_KG(F, L, 3, MODE, Q), \
      QMV_KG(F, L, 4, MODE, Q), QMV_KG(F, L, 7, MODE, Q) }
#define QMV_TABLE_GR(F, Q) \
    { { QMV_ROWG(F, 8, 0, Q), QMV_ROWG(F, 16, 0, Q), QMV_ROWG(F, 32, 0, Q), QMV_ROWG(F, 64, 0, Q) }, \
      { QMV_ROWG(F, 8, 1, Q), QMV_ROWG(F, 16, 1, Q), QMV_ROWG(F, 32, 1, Q), QMV_ROWG(F, 64, 1, Q) } }
