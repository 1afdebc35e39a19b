// qmv_k_mxfp4b.hip -- MXFP4 x bf16 products with more than 4 activation
// vectors: the expert-batched gather (a prefill chunk, a wide verify batch)
// and the dense call, on the 16x16x32 bf16 matrix cores.
//
// With many vectors per expert the work is a grouped matrix product: each
// expert's weight rows meet every vector routed to it (mlxcel issue,
// "Problem / Background": the expert-batched gather_qmm path that prefill
// takes once enough tokens share each expert).  Every workgroup first sorts
// the call's (token, slot) pairs by expert in LDS (a counting sort over the
// ids: count, prefix-sum, place), so nothing is allocated and no second
// launch is needed.  The sorted list defines the tiles:
//
//   tile = (expert, 16 * RF * WAVES weight rows);
//
// the workgroup multiplies the tile's rows with all of the expert's vectors,
// in chunks of at most 128 (equal chunks when an expert has more).  The LDS
// atomics order an expert's pairs differently in each workgroup, so a chunk
// must never be a tile of its own: two workgroups would cut different sets.
// A dense call has one bucket in index order, and there each chunk is a tile
// (more tiles for the same rows).  Workgroups take the list's tiles in an
// XCD-aware order until it ends.
//
// Inside a tile, wave w owns 16*RF rows as RF fragments of 16.  The K axis is
// walked in 128-weight slices.  Lane 16q + r loads row r's 32-weight block
// 4s + q of slice s (16 contiguous bytes), so one load instruction reads 16
// rows x 64 bytes.  The MFMA's 32-long k axis is then the lane's own block in
// four 8-weight steps t: in step t, lane group q supplies k = 32(4s + q) + 8t
// .. + 7 of its row (A) and the matching 8 activations of column r (B).  The
// dot product does not care which physical k sits in which MFMA slot as long
// as A and B agree, so this layout costs nothing.
//
// Decode: v_cvt_scalef32_pk_bf16_fp4 turns 8 nibbles into the A operand with
// the E8M0 scale folded in; e2m1 * 2^(s-127) is an exact bf16 normal for
// s in [2, 252].  A chunk whose weights hold any other scale byte (never in
// real weights: they are 2^-127, 2^-126, 2^126, 2^127 and NaN) is recomputed
// by a plain exact path after the loop, which keeps the loop itself to one
// path.
//
// Activations: per slice, every workgroup stages the tile's vectors' 128
// bf16 values into LDS (256 bytes per vector; chunk index xor-ed with the
// vector's low 4 bits so that the 16 lanes of one ds_read_b128 quarter hit
// 16 distinct bank groups), with direct global-to-LDS loads into a ring of
// four slice buffers.  Loads complete in issue order per wave, so a load's
// lead can be no longer than that of the loads waited on after it: the
// activations and the weights of a slice are issued together, three slices
// ahead, each slice starts with one wait on the wave's own loads and a
// barrier, and no register holds staged activations.
//
// Every output element is one MFMA column's dot product over the whole of K
// in a fixed order, so results do not depend on where a vector lands in the
// sorted list (the LDS counting sort's order within an expert may vary) and
// are bitwise reproducible.
#include "qmv_device.hpp"

namespace qmv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBVecMax = 128;           // vectors per tile: 8 column fragments of 16
constexpr int kBXBytes = kBVecMax * 256;     // one activation slice buffer
constexpr int kBAhead = 3;                     // slices loaded ahead of the one multiplied
constexpr int kBRing = kBAhead + 1;            // activation slice buffers in LDS

// s_waitcnt immediate (gfx9 layout) that waits for vmcnt <= N only.
template <int N> struct kVmcnt {
    static constexpr int enc = (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);
};
constexpr uint32_t kBPast = 0x80000000u;   // >= every buffer size: reads zeros

// LDS offset of 16-byte chunk pos (k = 8 pos .. 8 pos + 7 of the slice) of tile vector v.
__device__ __forceinline__ int bx_off(int v, int pos)
{
    return v * 256 + 16 * (pos ^ (v & 15));
}

__device__ __forceinline__ bf16x8 dec8(uint32_t w, float sc)
{
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                   __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Tiles of a bucket with c pairs: row tiles, times chunks when chunks are tiles.
__device__ __forceinline__ int tiles_of(int c, int nt, bool chunk_tiles)
{
    return c == 0 ? 0 : (chunk_tiles ? (c + kBVecMax - 1) / kBVecMax : 1) * nt;
}

// The outputs of one chunk of vectors over rows [row_lo, row_lo + rows),
// computed exactly as the per-block definition reads: each 32-weight block's
// sum of e2m1 * x in fp32, times 2^(s-127) built exactly (so scale bytes 0,
// 1, 253, 254 and 255 come out as they should).  One output per thread at a
// time, plain loads: slow, and only run for chunks whose weights hold a scale
// byte outside [2, 252].
__device__ __forceinline__ void batched_chunk_exact(const Args &a, const uint8_t *codes, const uint8_t *scales,
                                                 const uint16_t *vecs, int nv, int row_lo, int rows)
{
    const bool gather = a.ids != nullptr;
    for (int o = threadIdx.x; o < rows * nv; o += blockDim.x) {
        const int n = row_lo + o % rows;
        const int i = vecs[o / rows];
        const int xrow = gather && a.x_per_slot ? i : (gather ? i / a.top_k : i);
        const uint16_t *xv = (const uint16_t *)(a.x + (size_t)xrow * a.x_vec_bytes);
        const uint8_t *cw = codes + (size_t)n * a.rcb;
        float acc = 0.0f;
        for (int blk = 0; blk < a.units; ++blk) {
            float part = 0.0f;
            for (int j = 0; j < 16; ++j) {
                const uint32_t byte = cw[16 * blk + j];
                const bf16x2 w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte, 1.0f, 0);
                part = __builtin_fmaf((float)w[0], __uint_as_float((uint32_t)xv[32 * blk + 2 * j] << 16), part);
                part = __builtin_fmaf((float)w[1], __uint_as_float((uint32_t)xv[32 * blk + 2 * j + 1] << 16), part);
            }
            acc = __builtin_fmaf(part, e8m0_f32(scales[(size_t)n * a.rsb + blk]), acc);
        }
        a.y[(size_t)i * a.N + n] = acc;
    }
}

template <int RF, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void qmv_batched_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int kBThreads = 64 * WAVES;
    constexpr int TR = 16 * RF * WAVES;            // rows per tile
    constexpr int BPT = 1024 / kBThreads;          // scan buckets per thread
    constexpr int XJ = 32 / WAVES;                 // staging instructions (4 vectors each) per wave and slice
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int r = lane & 15;
    const int q = lane >> 4;
    const bool gather = a.ids != nullptr;
    const int B = gather ? a.M * a.top_k : a.M;    // (token, slot) pairs
    const int nb = gather ? a.E + 1 : 1;           // buckets: experts, then invalid ids
    const int NT = (a.N + TR - 1) / TR;
    const int U = a.units;                         // 32-weight blocks per row
    const int S = (U + 3) >> 2;                    // 128-weight slices

    int *const cnt = (int *)(lds + kBRing * kBXBytes);
    int *const voff = cnt + (nb + 1);
    int *const toff = voff + (nb + 1);
    int *const wsum = toff + (nb + 1);             // 2 x 8 wave totals
    uint16_t *const perm = (uint16_t *)(wsum + 16);
    uint32_t *const tmp = (uint32_t *)lds;         // (bucket << 16 | rank) per pair, in the x area

    // 1. counting sort of the pairs by expert (a dense call: one bucket, index order)
    for (int b = tid; b < nb; b += kBThreads) cnt[b] = gather ? 0 : B;
    __syncthreads();
    for (int i = tid; i < B; i += kBThreads) {
        int b = 0, rank = i;
        if (gather) {
            const int e = a.ids[i];
            b = (unsigned)e < (unsigned)a.E ? e : a.E;
            rank = atomicAdd(&cnt[b], 1);
        }
        tmp[i] = ((uint32_t)b << 16) | (uint32_t)rank;
    }
    __syncthreads();
    {
        int c[BPT], sv = 0, st = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = BPT * tid + j;
            c[j] = b < nb ? cnt[b] : 0;
            sv += c[j];
            st += tiles_of(c[j], NT, !gather);
        }
        const int ov = sv, ot = st;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int tv = __shfl_up(sv, d), tt = __shfl_up(st, d);
            if (lane >= d) { sv += tv; st += tt; }
        }
        if (lane == 63) { wsum[w] = sv; wsum[8 + w] = st; }
        __syncthreads();
        int ev = sv - ov, et = st - ot;
        for (int k = 0; k < w; ++k) { ev += wsum[k]; et += wsum[8 + k]; }
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = BPT * tid + j;
            if (b < nb) { voff[b] = ev; toff[b] = et; }
            ev += c[j];
            et += tiles_of(c[j], NT, !gather);
        }
        if (tid == kBThreads - 1) { voff[nb] = ev; toff[nb] = et; }
    }
    __syncthreads();
    for (int i = tid; i < B; i += kBThreads) {
        const uint32_t v = tmp[i];
        perm[voff[v >> 16] + (v & 0xFFFFu)] = (uint16_t)i;
    }
    __syncthreads();
    const int total = toff[nb];

    const int x_bytes = (gather && a.x_per_slot ? B : a.M) * a.x_vec_bytes;   // < 2^31
    const bool vec4 = (a.N & 3) == 0 && ((uintptr_t)a.y & 15) == 0;

    // Workgroups are dealt to the 8 XCDs in turn (workgroup b to XCD b % 8;
    // the grid is a multiple of 8).  Each XCD takes one contiguous eighth of
    // the expert-major tile list, so its L2 holds the activation rows of a
    // few experts only, shared by the row tiles of one expert that its CUs
    // stream at the same time.
    const int per = (total + 7) >> 3;
    const int xcd = blockIdx.x & 7;
    for (int xl = blockIdx.x >> 3; xl < per; xl += gridDim.x >> 3) {
        const int t = xcd * per + xl;
        if (t >= total) break;
        // 2. the tile: bucket, row tile (and chunk, for a dense call)
        int lo = 0, hi = nb;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (toff[mid] <= t) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int local = t - toff[b];
        const int c = voff[b + 1] - voff[b];
        const int nch = (c + kBVecMax - 1) / kBVecMax;
        const int cs = (c + nch - 1) / nch;
        const int ct = gather ? 0 : local / NT;    // the tile's chunk, if chunks are tiles
        const int rt = local - ct * NT;
        const int row0 = rt * TR + 16 * RF * w;    // this wave's first row
        for (int chunk = ct; chunk < (gather ? nch : ct + 1); ++chunk) {
            const int vstart = voff[b] + chunk * cs;
            const int nv = min(cs, c - chunk * cs);
            int nf = (nv + 15) >> 4;

            f32x4 acc[RF][8];
#pragma unroll
            for (int f = 0; f < RF; ++f)
#pragma unroll
                for (int g = 0; g < 8; ++g) acc[f][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

            if (b < a.E || !gather) {
                const int e = gather ? b : 0;
                const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.codes + (long long)e * a.expert_cb, a.expert_cb);
                const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.scales + (long long)e * a.expert_sb, a.expert_sb);
                uint32_t oc[RF], os[RF];
#pragma unroll
                for (int f = 0; f < RF; ++f) {
                    const int n = row0 + 16 * f + r;
                    oc[f] = n < a.N ? (uint32_t)n * (uint32_t)a.rcb + 16u * q : kBPast;
                    os[f] = n < a.N ? (uint32_t)n * (uint32_t)a.rsb + q : kBPast;
                }
                // Activation staging: direct loads from global memory into a ring
                // of kBRing LDS slice buffers (each lane's 16 bytes land at the
                // instruction's LDS base + 16 * lane).  One instruction fills 4
                // vectors x 256 bytes; wave w issues the vector quads w + WAVES j.
                // Lane 16 h + p of quad d fills slot p of vector 4 d + h with the
                // chunk the swizzle puts there, k-chunk p ^ (vector & 15).
                const int wv = __builtin_amdgcn_readfirstlane(w);
                uint32_t xo[XJ];
                int xpos[XJ];
#pragma unroll
                for (int j = 0; j < XJ; ++j) {
                    const int v = 4 * (wv + WAVES * j) + (lane >> 4);
                    xpos[j] = (lane & 15) ^ (v & 15);
                    uint32_t o = kBPast;
                    if (v < nv) {
                        const int i = perm[vstart + v];
                        const int row = gather && a.x_per_slot ? i : (gather ? i / a.top_k : i);
                        o = (uint32_t)row * (uint32_t)a.x_vec_bytes;
                    }
                    xo[j] = o;
                }
                auto issue_x = [&](int s) {
                    // (built here from kernel arguments, so it stays in scalar registers)
                    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, x_bytes);
                    uint8_t *const buf = lds + (s % kBRing) * kBXBytes;
#pragma unroll
                    for (int j = 0; j < XJ; ++j) {
                        const int k = 128 * s + 8 * xpos[j];
                        const uint32_t o = (k < a.K && xo[j] != kBPast) ? xo[j] + 2u * k : kBPast;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rx, (__attribute__((address_space(3))) void *)(buf + 1024 * (wv + WAVES * j)), 16, o, 0, 0, 0);
                    }
                };
                auto load_w = [&](int s, u32x4 (&wc)[RF], uint8_t (&sb)[RF]) {
                    const bool ok = s < S && 4 * s + q < U;
#pragma unroll
                    for (int f = 0; f < RF; ++f) {
                        const bool okf = ok && oc[f] != kBPast;
                        wc[f] = __builtin_amdgcn_raw_buffer_load_b128(rc, okf ? oc[f] + 64u * s : kBPast, 0, kStream);
                        sb[f] = __builtin_amdgcn_raw_buffer_load_b8(rs, okf ? os[f] + 4u * s : kBPast, 0, 0);
                    }
                };
                // A slice whose scale bytes are all in [2, 252] (every real
                // weight) is exact with the scale folded into the convert; any
                // other byte only marks the chunk for the exact recomputation
                // below, which keeps this loop free of a second path (and the
                // accumulators out of the VALU).
                int slow = 0;
                auto compute = [&](int s, const u32x4 (&wc)[RF], const uint8_t (&sbr)[RF]) {
                    const bool ok = 4 * s + q < U;
                    const uint8_t *const buf = lds + (s % kBRing) * kBXBytes;
                    bf16x8 A[RF][4];
#pragma unroll
                    for (int f = 0; f < RF; ++f) {
                        const uint32_t sb = (ok && oc[f] != kBPast) ? (uint32_t)sbr[f] : 127u;
                        slow |= (sb - 2u) > 250u;
                        const float sc = __uint_as_float(sb << 23);
#pragma unroll
                        for (int k = 0; k < 4; ++k) A[f][k] = dec8(wc[f][k], sc);
                    }
#pragma unroll
                    for (int g = 0; g < 8; ++g) {
                        if (g < nf) {
                            bf16x8 Bv[4];
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                Bv[k] = __builtin_bit_cast(bf16x8, lds_read16(buf + bx_off(16 * g + r, 4 * q + k)));
#pragma unroll
                            for (int f = 0; f < RF; ++f)
#pragma unroll
                                for (int k = 0; k < 4; ++k)
                                    acc[f][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[f][k], Bv[k], acc[f][g], 0, 0, 0);
                        }
                    }
                };
                // Top of slice s: this wave's loads of slice s are done once at
                // most kAfter of its later loads are outstanding (loads complete
                // in issue order, and every slice issues the same number); the
                // barrier then covers the other waves' parts of the buffer.
                constexpr int kAfter = 2 * RF + (kBAhead - 1) * (XJ + 2 * RF);
                static_assert(kAfter < 64, "vmcnt holds at most 63");
                auto slice_ready = [&]() {
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(kVmcnt<kAfter>::enc);
                    __syncthreads();
                };

                // 3. slices, kBAhead (3) ahead for activations and weights alike;
                //    the slice count is padded to a multiple of 3 (the padding
                //    reads past the buffers: zeros).
                u32x4 wc0[RF], wc1[RF], wc2[RF];
                uint8_t sb0[RF], sb1[RF], sb2[RF];   // widened only where used
                issue_x(0);
                load_w(0, wc0, sb0);
                issue_x(1);
                load_w(1, wc1, sb1);
                issue_x(2);
                load_w(2, wc2, sb2);
                for (int s = 0; s < S; s += 3) {
                    slice_ready();
                    issue_x(s + 3);
                    compute(s, wc0, sb0);
                    load_w(s + 3, wc0, sb0);
                    slice_ready();
                    issue_x(s + 4);
                    compute(s + 1, wc1, sb1);
                    load_w(s + 4, wc1, sb1);
                    slice_ready();
                    issue_x(s + 5);
                    compute(s + 2, wc2, sb2);
                    load_w(s + 5, wc2, sb2);
                }
                // the ring's last loads land before the next chunk reuses it
                __builtin_amdgcn_s_waitcnt(kVmcnt<0>::enc);
                if (__syncthreads_or(slow)) {
                    const int e = gather ? b : 0;
                    batched_chunk_exact(a, a.codes + (long long)e * a.expert_cb, a.scales + (long long)e * a.expert_sb,
                                        perm + vstart, nv, rt * TR, min(TR, a.N - rt * TR));
                    nf = 0;                        // stored: nothing left for step 4
                }
            }

            // 4. store: lane 16 (row quad) + column; invalid ids give zero rows
#pragma unroll
            for (int f = 0; f < RF; ++f) {
                const int n0 = row0 + 16 * f + 4 * q;
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    const int col = 16 * g + r;
                    if (g < nf && col < nv && n0 < a.N) {
                        const int i = perm[vstart + col];
                        float *yp = a.y + (size_t)i * a.N + n0;
                        if (vec4) {
                            *(float4 *)yp = make_float4(acc[f][g][0], acc[f][g][1], acc[f][g][2], acc[f][g][3]);
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                if (n0 + v < a.N) yp[v] = acc[f][g][v];
                        }
                    }
                }
            }
            __syncthreads();                           // the next chunk restages x
        }
    }
}

// [4 waves x 2 fragments: 128 rows per tile, 8 waves x 2 fragments: 256 rows
// per tile (two waves per SIMD)]
extern const void *const kTableBatched[2];
const void *const kTableBatched[2] = {(const void *)&qmv_batched_kernel<2, 4>,
                                      (const void *)&qmv_batched_kernel<2, 8>};

}  // namespace qmv
