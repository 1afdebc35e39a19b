// qmv_k_mxfp4b.hip -- MXFP4 x bf16 products with more than 4 activation
// vectors: the expert-batched gather (a prefill chunk, a wide verify batch)
// and the dense call, on the 16x16x32 bf16 matrix cores.
//
// With many vectors per expert the work is a grouped matrix product: each
// expert's weight rows meet every vector routed to it (mlxcel issue,
// "Background": the expert-batched gather_qmm path that prefill takes once
// enough tokens share each expert).  Every workgroup first sorts the call's
// (token, slot) pairs by expert in LDS (a counting sort over the ids: count,
// prefix-sum, place), so nothing is allocated and no second launch is needed.
// The sorted list defines the tiles:
//
//   tile = (expert, 64*RF weight rows);
//
// the workgroup multiplies the tile's rows with all of the expert's vectors,
// in chunks of at most 128 (equal chunks when an expert has more).  The LDS
// atomics order an expert's pairs differently in each workgroup, so a chunk
// must never be a tile of its own: two workgroups would cut different sets.
// A dense call has one bucket in index order, and there each chunk is a tile
// (more tiles for the same rows).  Workgroups take tiles blockIdx.x,
// blockIdx.x + gridDim.x, ... until the list ends.
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
// s in [2, 252].  A slice with any other scale byte (rare) is decoded
// unscaled and multiplied one lane group at a time (the other groups' A set
// to zero), each group's partial tile then scaled by its exactly built
// 2^(s-127) per row.
//
// Activations: per slice, every workgroup stages the tile's vectors' 128
// bf16 values into LDS (256 bytes per vector; chunk index xor-ed with the
// vector's low 4 bits so that the 16 lanes of one ds_read_b128 quarter hit
// 16 distinct bank groups).  Weight loads run two slices ahead; the next
// slice's activations are loaded into registers while the current slice
// multiplies.  Loads complete in issue order, so each slice issues its
// activation loads before the weight loads of two slices later: waiting for
// the activations never waits for weights not yet needed.
//
// Every output element is one MFMA column's dot product over the whole of K
// in a fixed order, so results do not depend on where a vector lands in the
// sorted list (the LDS counting sort's order within an expert may vary) and
// are bitwise reproducible.
#include "qmv_device.hpp"

namespace qmv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBThreads = 256;          // 4 wave64s
constexpr int kBVecMax = 128;           // vectors per tile: 8 column fragments of 16
constexpr int kBXBytes = kBVecMax * 256;
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

template <int RF>
__global__ __launch_bounds__(kBThreads) void qmv_batched_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int TR = 64 * RF;                    // rows per tile
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

    int *const cnt = (int *)(lds + kBXBytes);
    int *const voff = cnt + (nb + 1);
    int *const toff = voff + (nb + 1);
    int *const wsum = toff + (nb + 1);             // 2 x 4 wave totals
    uint16_t *const perm = (uint16_t *)(wsum + 8);
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
        int c[4], sv = 0, st = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * tid + j;
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
        if (lane == 63) { wsum[w] = sv; wsum[4 + w] = st; }
        __syncthreads();
        int ev = sv - ov, et = st - ot;
        for (int k = 0; k < w; ++k) { ev += wsum[k]; et += wsum[4 + k]; }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * tid + j;
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

    const long long x_bytes = (long long)(gather && a.x_per_slot ? B : a.M) * a.x_vec_bytes;
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, x_bytes);
    const bool vec4 = (a.N & 3) == 0 && ((uintptr_t)a.y & 15) == 0;

    for (int t = blockIdx.x; t < total; t += gridDim.x) {
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
            const int nf = (nv + 15) >> 4;

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
                // activation rows of this thread's staging chunks: vectors tid/16 + 16j, k-chunk tid%16
                const int pos = tid & 15;
                uint32_t xo[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int v = (tid >> 4) + 16 * j;
                    uint32_t o = kBPast;
                    if (v < nv) {
                        const int i = perm[vstart + v];
                        const int row = gather && a.x_per_slot ? i : (gather ? i / a.top_k : i);
                        o = (uint32_t)row * (uint32_t)a.x_vec_bytes;
                    }
                    xo[j] = o;
                }

                uint4 xr[8];
                auto load_x = [&](int s) {
                    const int k = 128 * s + 8 * pos;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t o = (k < a.K && xo[j] != kBPast) ? xo[j] + 2u * k : kBPast;
                        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
                        xr[j] = make_uint4(v[0], v[1], v[2], v[3]);
                    }
                };
                auto put_x = [&]() {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int v = (tid >> 4) + 16 * j;
                        if (v < nf * 16) *(uint4 *)(lds + bx_off(v, pos)) = xr[j];
                    }
                };
                auto load_w = [&](int s, u32x4 (&wc)[RF], uint32_t (&sb)[RF]) {
                    const bool ok = s < S && 4 * s + q < U;
#pragma unroll
                    for (int f = 0; f < RF; ++f) {
                        const bool okf = ok && oc[f] != kBPast;
                        wc[f] = __builtin_amdgcn_raw_buffer_load_b128(rc, okf ? oc[f] + 64u * s : kBPast, 0, kStream);
                        sb[f] = __builtin_amdgcn_raw_buffer_load_b8(rs, okf ? os[f] + 4u * s : kBPast, 0, 0);
                    }
                };
                auto compute = [&](int s, const u32x4 (&wc)[RF], const uint32_t (&sbr)[RF]) {
                    const bool ok = 4 * s + q < U;
                    bf16x8 A[RF][4];
                    uint32_t sb[RF];
                    bool fast[RF];
#pragma unroll
                    for (int f = 0; f < RF; ++f) {
                        sb[f] = (ok && oc[f] != kBPast) ? sbr[f] : 127u;
                        fast[f] = __all((sb[f] - 2u) <= 250u);
                        const float sc = fast[f] ? __uint_as_float(sb[f] << 23) : 1.0f;
#pragma unroll
                        for (int k = 0; k < 4; ++k) A[f][k] = dec8(wc[f][k], sc);
                    }
#pragma unroll
                    for (int g = 0; g < 8; ++g) {
                        if (g < nf) {
                            bf16x8 Bv[4];
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                Bv[k] = __builtin_bit_cast(bf16x8, lds_read16(lds + bx_off(16 * g + r, 4 * q + k)));
#pragma unroll
                            for (int f = 0; f < RF; ++f) {
                                if (fast[f]) {
#pragma unroll
                                    for (int k = 0; k < 4; ++k)
                                        acc[f][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[f][k], Bv[k], acc[f][g], 0, 0, 0);
                                } else {
                                    // one lane group (one 32-weight block per row) at a time
                                    const bf16x8 z = {};
#pragma unroll
                                    for (int qq = 0; qq < 4; ++qq) {
                                        f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                                        for (int k = 0; k < 4; ++k)
                                            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q == qq ? A[f][k] : z, Bv[k], p, 0, 0, 0);
                                        // p[v] is row 4 (lane / 16) + v of the fragment; its block's
                                        // scale byte sits in lane 16 qq + 4 (lane / 16) + v
#pragma unroll
                                        for (int v = 0; v < 4; ++v) {
                                            const uint32_t sv = (uint32_t)__shfl((int)sb[f], 16 * qq + 4 * q + v);
                                            acc[f][g][v] = __builtin_fmaf(p[v], e8m0_f32(sv), acc[f][g][v]);
                                        }
                                    }
                                }
                            }
                        }
                    }
                };

                // 3. slices: weights two ahead, activations one ahead (one LDS buffer)
                u32x4 wc0[RF], wc1[RF];
                uint32_t sb0[RF], sb1[RF];
                load_x(0);
                load_w(0, wc0, sb0);
                load_w(1, wc1, sb1);
                put_x();
                __syncthreads();
                for (int s = 0; s < S; s += 2) {
                    load_x(s + 1);
                    compute(s, wc0, sb0);
                    load_w(s + 2, wc0, sb0);
                    __syncthreads();
                    put_x();
                    __syncthreads();
                    if (s + 1 < S) {
                        load_x(s + 2);
                        compute(s + 1, wc1, sb1);
                        load_w(s + 3, wc1, sb1);
                        __syncthreads();
                        put_x();
                        __syncthreads();
                    }
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

// Rows per tile: 128 (RF 2), 256 (RF 4).
extern const void *const kTableBatched[2];
const void *const kTableBatched[2] = {(const void *)&qmv_batched_kernel<2>,
                                      (const void *)&qmv_batched_kernel<4>};

}  // namespace qmv
