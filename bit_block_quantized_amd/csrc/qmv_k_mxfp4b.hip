// qmv_k_mxfp4b.hip -- MXFP4 x bf16 products with more than 4 activation
// vectors: the expert-batched gather (a prefill chunk, a wide verify batch),
// the fused gate/up gather with SwiGLU, and the dense call, on the 32x32x16
// bf16 matrix cores.
//
// With many vectors per expert the work is a grouped matrix product: each
// expert's weight rows meet every vector routed to it (mlxcel issue,
// "Problem / Background": the expert-batched gather_qmm path that prefill
// takes once enough tokens share each expert).
//
// Tiles.  A tile is (expert, R consecutive weight rows), R = 32 * RF * WAVES
// (for the gate/up kernel R = 16 * RF * WAVES output rows: each holds a gate
// and an up row).  The grid has one workgroup per tile of every expert, whether or not
// any pair selects it, so the tiling needs no device-wide knowledge of the
// ids and no sort: a workgroup lists its own expert's (token, slot) pairs in
// index order by scanning the ids with ballots (deterministic, no atomics),
// and leaves at once when there are none.  The tiles of expert 0 also write
// the zero rows of pairs whose id is outside [0, E).  Workgroup b runs on XCD
// b % 8 (the dispatcher deals workgroups round robin); the tiles are dealt to
// XCDs in contiguous, expert-major runs, so each XCD's L2 holds the
// activation rows of a few experts, shared by the row tiles that stream them
// side by side.  A dense call is one expert whose vectors come in index
// order; there the vectors are split into chunks and each (chunk, row tile)
// is a tile, so even a single weight matrix gives enough tiles.
//
// Inside a tile, wave w owns RF fragments of 32 rows, multiplied on the
// 32x32x16 bf16 MFMA (measured on MI355X: about twice the rate per flop of
// the 16x16x32 form).  K is walked in 128-weight slices.  Lane (r, h) =
// lane 32 h + r loads row r's 32-weight blocks 2 h and 2 h + 1 of slice s
// (32 contiguous code bytes, and their two scale bytes in one 16-bit load;
// one byte load per block made the scale loads a large part of the gpt-oss
// prefill chunk's time: dropping them altogether ran 25% faster, pairing them
// 4% -- 12% with gate/up).  The MFMA's 16-long k axis is
// split between the lane halves h: in step (jb, t), half h supplies weights
// 8t .. 8t + 7 of block 2 h + jb of its row (A) and the same 8 activations
// of vector r (B).
// The dot product does not care which physical k sits in which MFMA slot as
// long as A and B agree, so this layout costs nothing.  An expert's vectors
// are taken up to VCAP at a time (equal chunks when it has more), and the
// kernel body is compiled for 32, 64, 96 and 128 vectors so that a tile with
// few vectors loads and multiplies no empty fragments.
//
// Decode: v_cvt_scalef32_pk_bf16_fp4 turns 8 nibbles into the A operand with
// the E8M0 scale folded in; e2m1 * 2^(s-127) is an exact bf16 normal for
// s in [2, 252].  A chunk whose weights hold any other scale byte (never in
// real weights: they are 2^-127, 2^-126, 2^126, 2^127 and NaN) is recomputed
// by a plain exact path after the loop, which keeps the loop itself to one
// path.
//
// Activations: per slice, the tile's vectors' 128 bf16 values are loaded
// into registers three slices ahead and written into one of two LDS slice
// buffers one slice ahead (256 bytes per vector; the 16-byte chunk index
// xor-ed with the vector's low 4 bits, so the 16 lanes of one ds_read_b128
// quarter hit 16 distinct bank groups); one barrier per slice.  Weights go
// straight to registers, three slices ahead.  Every load is an ordinary
// register load, so the compiler's waits cover exactly what each step uses
// (direct global-to-LDS loads were measured slower here: the compiler's wait
// counts do not account for them, which cut the prefetch depth).
//
// Every output element is one MFMA column's dot product over the whole of K
// in a fixed order, so results are bitwise reproducible.
#include "qmv_device.hpp"

namespace qmv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBVecMax = 128;                  // vectors per chunk
constexpr int kBRing = 2;                      // activation slice buffers in LDS
constexpr int kBatchedMenu = 6;                // kernel shapes (kBatchedShapes)
constexpr uint32_t kBPast = 0x80000000u;       // >= every buffer size: reads zeros

// LDS offset of 16-byte chunk pos (k = 8 pos .. 8 pos + 7 of the slice) of ring vector v.
__device__ __forceinline__ int bx_off(int v, int pos)
{
    return v * 256 + 16 * (pos ^ (v & 15));
}

// The E8M0 bytes of blocks 4 s + 2 h and 4 s + 2 h + 1 of a row (the two
// blocks lane half h takes in 128-weight slice s) in bits 0-7 and 8-15: one
// 16-bit load at os = the row's scale offset + 2 h (always even: a row's
// scales start at an even byte and hold an even count in every slice but the
// last of an odd count).  A byte past the row's end reads as 0; only the last
// slice of an odd-length row has a lone block, and there (a wave-uniform
// branch) the two bytes are loaded one at a time.
__device__ __forceinline__ uint32_t load_scale_pair(__amdgpu_buffer_rsrc_t rs, uint32_t os, int s, int U, int h,
                                                    bool valid)
{
    const int b0 = 4 * s + 2 * h;
    const uint32_t o = os + 4u * (uint32_t)s;
    if ((U & 1) && 4 * s + 4 > U) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b8(rs, valid && b0 < U ? o : kBPast, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b8(rs, valid && b0 + 1 < U ? o + 1u : kBPast, 0, 0);
        return lo | hi << 8;
    }
    return __builtin_amdgcn_raw_buffer_load_b16(rs, valid && b0 < U ? o : kBPast, 0, 0);
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

// The outputs of one chunk of vectors over rows [row_lo, row_lo + rows),
// computed exactly as the per-block definition reads: each 32-weight block's
// sum of e2m1 * x in fp32, times 2^(s-127) built exactly (so scale bytes 0,
// 1, 253, 254 and 255 come out as they should).  One output per thread at a
// time, plain loads: slow, and only run for chunks whose weights hold a scale
// byte outside [2, 252].  MODE 1 forms the gate and up sums and stores
// silu(gate) * up.
template <int MODE>
__device__ __forceinline__ void batched_chunk_exact(const Args &a, int e, const uint16_t *vecs, int vstart,
                                                    int nv, int row_lo, int rows)
{
    const bool gather = a.ids != nullptr;
    for (int o = threadIdx.x; o < rows * nv; o += blockDim.x) {
        const int n = row_lo + o % rows;
        const int i = gather ? (int)vecs[o / rows] : vstart + o / rows;
        const int xrow = gather && a.x_per_slot ? i : (gather ? i / a.top_k : i);
        const uint16_t *xv = (const uint16_t *)(a.x + (size_t)xrow * a.x_vec_bytes);
        float acc[2] = {0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < (MODE == 1 ? 2 : 1); ++h) {
            const uint8_t *codes = (h ? a.codes2 : a.codes) + (long long)e * a.expert_cb;
            const uint8_t *scales = (h ? a.scales2 : a.scales) + (long long)e * a.expert_sb;
            const uint8_t *cw = codes + (size_t)n * a.rcb;
            for (int blk = 0; blk < a.units; ++blk) {
                float part = 0.0f;
                for (int j = 0; j < 16; ++j) {
                    const uint32_t byte = cw[16 * blk + j];
                    const bf16x2 wv = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte, 1.0f, 0);
                    part = __builtin_fmaf((float)wv[0], __uint_as_float((uint32_t)xv[32 * blk + 2 * j] << 16), part);
                    part = __builtin_fmaf((float)wv[1], __uint_as_float((uint32_t)xv[32 * blk + 2 * j + 1] << 16), part);
                }
                acc[h] = __builtin_fmaf(part, e8m0_f32(scales[(size_t)n * a.rsb + blk]), acc[h]);
            }
        }
        a.y[(size_t)i * a.N + n] = MODE == 1 ? swiglu(acc[0], acc[1]) : acc[0];
    }
}

// One chunk of nv <= VMAX vectors (ring slots 0..nv-1) against this tile's
// rows.  vecs: the chunk's pair indices (gather), or nullptr with the
// vectors vstart .. vstart + nv - 1 (dense).
template <int RF, int WAVES, int MODE, int VMAX>
__device__ __forceinline__ void batched_chunk(const Args &a, uint8_t *lds, int e, int row_base,
                                              const uint16_t *vecs, int vstart, int nv)
{
    constexpr int TR = 32 * RF * WAVES / (MODE == 1 ? 2 : 1);   // output rows per tile
    constexpr int XJ = VMAX / (4 * WAVES);          // staging loads (4 vectors each) per wave and slice
    constexpr int CF = VMAX / 32;                   // column fragments of 32 vectors
    constexpr int RH = MODE == 1 ? RF / 2 : RF;      // output row fragments per wave
    static_assert(XJ >= 1 && (MODE == 0 || RF % 2 == 0), "batched kernel shape");
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r = lane & 31;                        // row (A) / vector (B) within a fragment
    const int h = lane >> 5;                        // k half of an MFMA step
    const bool gather = a.ids != nullptr;
    const int U = a.units;                          // 32-weight blocks per row
    const int S = (U + 3) >> 2;                     // 128-weight slices
    const int row0 = row_base + 32 * RH * w;        // this wave's first output row
    const int nf = (nv + 31) >> 5;                  // column fragments in use

    f32x16 acc[RF][CF];
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int g = 0; g < CF; ++g)
#pragma unroll
            for (int k = 0; k < 16; ++k) acc[f][g][k] = 0.0f;

    // lane (r, h) streams blocks 2 h and 2 h + 1 of each 128-weight slice of
    // its fragments' row r (32 contiguous code bytes, two adjacent scale bytes)
    __amdgpu_buffer_rsrc_t rc[RF], rs[RF];
    uint32_t oc[RF], os[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        const bool up = MODE == 1 && f >= RH;
        rc[f] = buffer_rsrc((up ? a.codes2 : a.codes) + (long long)e * a.expert_cb, a.expert_cb);
        rs[f] = buffer_rsrc((up ? a.scales2 : a.scales) + (long long)e * a.expert_sb, a.expert_sb);
        const int n = row0 + 32 * (MODE == 1 ? f % RH : f) + r;
        oc[f] = n < a.N ? (uint32_t)n * (uint32_t)a.rcb + 32u * h : kBPast;
        os[f] = n < a.N ? (uint32_t)n * (uint32_t)a.rsb + 2u * h : kBPast;
    }
    // Activation staging: lane 16 c + p of load j holds chunk p (k = 8 p ..
    // 8 p + 7 of the slice) of ring vector 4 (w + WAVES j) + c, and writes it
    // where the swizzle puts it.  The loads go through registers (not direct
    // to LDS), so the compiler's own waits track every load in flight.
    const int x_bytes = (gather && a.x_per_slot ? a.M * a.top_k : a.M) * a.x_vec_bytes;   // < 2^31
    uint32_t xo[XJ];
    int xdst[XJ];
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
        const int v = 4 * (w + WAVES * j) + (lane >> 4);
        xdst[j] = bx_off(v, lane & 15);
        uint32_t o = kBPast;
        if (v < nv) {
            const int i = gather ? (int)vecs[v] : vstart + v;
            const int row = gather && a.x_per_slot ? i : (gather ? i / a.top_k : i);
            o = (uint32_t)row * (uint32_t)a.x_vec_bytes + 16u * (lane & 15);
        }
        xo[j] = o;
    }
    // (the lambdas below capture no kernel argument: taking the argument
    // block's address would make the compiler copy it to scratch memory)
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, x_bytes);
    const int K = a.K;
    auto load_x = [&](int s, u32x4 (&xr)[XJ]) {
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const bool ok = s < S && 128 * s + 8 * (lane & 15) < K && xo[j] != kBPast;
            xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? xo[j] + 256u * s : kBPast, 0, 0);
        }
    };
    auto store_x = [&](int s, const u32x4 (&xr)[XJ]) {
        uint8_t *const buf = lds + (s % kBRing) * (VMAX * 256);
#pragma unroll
        for (int j = 0; j < XJ; ++j) *(u32x4 *)(buf + xdst[j]) = xr[j];
    };
    // (the scales two bytes at a time: a row's scales start at any even
    // byte, and an unaligned dword load is far slower than 16-bit loads)
    auto load_w = [&](int s, u32x4 (&wc)[RF][2], uint32_t (&sb)[RF]) {
#pragma unroll
        for (int f = 0; f < RF; ++f) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const bool okf = s < S && 4 * s + 2 * h + jb < U && oc[f] != kBPast;
                wc[f][jb] = __builtin_amdgcn_raw_buffer_load_b128(rc[f], okf ? oc[f] + 64u * s + 16u * jb : kBPast, 0, 0);
            }
            sb[f] = load_scale_pair(rs[f], os[f], s, U, h, s < S && oc[f] != kBPast);
        }
    };
    // A slice whose scale bytes are all in [2, 252] (every real weight) is
    // exact with the scale folded into the convert; any other byte only marks
    // the chunk for the exact recomputation below, which keeps this loop free
    // of a second path (and the accumulators out of the VALU).
    int slow = 0;
    auto compute = [&](int s, const u32x4 (&wc)[RF][2], const uint32_t (&sbr)[RF]) {
        const uint8_t *const buf = lds + (s % kBRing) * (VMAX * 256);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const bool ok = 4 * s + 2 * h + jb < U;
            float sc[RF];
#pragma unroll
            for (int f = 0; f < RF; ++f) {
                const uint32_t sb = (ok && oc[f] != kBPast) ? (sbr[f] >> (8 * jb)) & 0xffu : 127u;
                slow |= (sb - 2u) > 250u;
                sc[f] = __uint_as_float(sb << 23);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // step (jb, t): lane half h supplies weights 8t .. 8t + 7 of
                // block 2 h + jb of the slice, and the same 8 activations;
                // every fragment's activations are read before the MFMAs
                bf16x8 Bv[CF];
#pragma unroll
                for (int g = 0; g < CF; ++g)
                    if (g < nf) Bv[g] = __builtin_bit_cast(bf16x8, lds_read16(buf + bx_off(32 * g + r, 4 * (2 * h + jb) + t)));
                bf16x8 A[RF];
#pragma unroll
                for (int f = 0; f < RF; ++f) A[f] = dec8(wc[f][jb][t], sc[f]);
#pragma unroll
                for (int g = 0; g < CF; ++g) {
                    if (g < nf) {
#pragma unroll
                        for (int f = 0; f < RF; ++f)
                            acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[f], Bv[g], acc[f][g], 0, 0, 0);
                    }
                }
            }
        }
    };

    // Slices: weights are loaded 3 slices ahead and activations 2 (register
    // sets rotating over 3 and 2 slices; the loop is unrolled 6 times), the
    // activations of slice s + 1 are written to the LDS ring (2 slice
    // buffers) while slice s is multiplied; one barrier per slice publishes
    // the buffer just written and frees the one the next write reuses.  The
    // slice count is padded to a multiple of 6 (the padding reads past the
    // buffers: zeros).
    u32x4 wc0[RF][2], wc1[RF][2], wc2[RF][2];
    uint32_t sb0[RF], sb1[RF], sb2[RF];
    u32x4 xr0[XJ], xr1[XJ];
    load_w(0, wc0, sb0);
    load_x(0, xr0);
    load_w(1, wc1, sb1);
    load_x(1, xr1);
    load_w(2, wc2, sb2);
    store_x(0, xr0);
    load_x(2, xr0);
    // step s: x(s + 1) sits in register set (s + 1) % 2 (loaded two slices
    // ago); it is written to LDS and the set refilled with x(s + 3)
    auto step = [&](int s, u32x4 (&wc)[RF][2], uint32_t (&sb)[RF], u32x4 (&xn)[XJ]) {
        __syncthreads();
        store_x(s + 1, xn);
        load_x(s + 3, xn);
        compute(s, wc, sb);
        load_w(s + 3, wc, sb);
    };
    for (int s = 0; s < S; s += 6) {
        step(s, wc0, sb0, xr1);
        step(s + 1, wc1, sb1, xr0);
        step(s + 2, wc2, sb2, xr1);
        step(s + 3, wc0, sb0, xr0);
        step(s + 4, wc1, sb1, xr1);
        step(s + 5, wc2, sb2, xr0);
    }
    if (__syncthreads_or(slow)) {
        batched_chunk_exact<MODE>(a, e, vecs, vstart, nv, row_base, min(TR, a.N - row_base));
        __syncthreads();
        return;
    }

    // store: lane (vector r, half h) holds rows 8 i + 4 h .. + 3 of each
    // fragment, four consecutive rows of one vector per i
    const bool vec4 = (a.N & 3) == 0 && ((uintptr_t)a.y & 15) == 0;
#pragma unroll
    for (int g = 0; g < CF; ++g) {
        const int col = 32 * g + r;
        if (g < nf && col < nv) {
            const int i = gather ? (int)vecs[col] : vstart + col;
            float *const yrow = a.y + (size_t)i * a.N;
#pragma unroll
            for (int f = 0; f < RH; ++f) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int n0 = row0 + 32 * f + 8 * ii + 4 * h;
                    if (n0 < a.N) {
                        float v[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            v[k] = MODE == 1 ? swiglu(acc[f][g][4 * ii + k], acc[f + RH][g][4 * ii + k])
                                             : acc[f][g][4 * ii + k];
                        if (vec4) {
                            *(float4 *)(yrow + n0) = make_float4(v[0], v[1], v[2], v[3]);
                        } else {
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                if (n0 + k < a.N) yrow[n0 + k] = v[k];
                        }
                    }
                }
            }
        }
    }
    __syncthreads();                                // the next chunk refills the ring
}

// VCAP: the most vectors one chunk holds (register budget: RF * VCAP / 4
// accumulators per lane).
template <int RF, int WAVES, int MODE, int VCAP>
__global__ __launch_bounds__(64 * WAVES, 1) void qmv_batched_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int THREADS = 64 * WAVES;
    constexpr int TR = 32 * RF * WAVES / (MODE == 1 ? 2 : 1);
    // the tile: XCD b % 8 takes the contiguous run of tiles
    // [xcd * per_xcd, (xcd + 1) * per_xcd)
    const int b = blockIdx.x;
    const int t = (b & 7) * a.bt_per_xcd + (b >> 3);
    if (t >= a.bt_tiles) return;
    const int bucket = t / a.bt_row_tiles;            // expert (gather) or vector chunk (dense)
    const int rt = t - bucket * a.bt_row_tiles;
    const int row_base = rt * TR;
    const bool gather = a.ids != nullptr;
    PairList L;
    L.cnt = (int *)(lds + kBRing * a.bt_vmax * 256);
    L.perm = (uint16_t *)(L.cnt + kMaxCounts + 4);

    int e = 0, c = 0, vstart = 0;
    const uint16_t *vecs = nullptr;
    if (gather) {
        const Ids8 id0 = load_ids8<THREADS>(a.ids, a.M * a.top_k, a.E, 0);
        if (bucket == 0) {
            // the tiles of expert 0 also write the zero rows of invalid ids
            const int ci = list_pairs<THREADS>(a.ids, a.M * a.top_k, a.E, -1, L, id0);
            const int rows = min(TR, a.N - row_base);
            for (int o = threadIdx.x; o < ci * rows; o += THREADS)
                a.y[(size_t)L.perm[o / rows] * a.N + row_base + o % rows] = 0.0f;
            __syncthreads();
        }
        e = bucket;
        c = list_pairs<THREADS>(a.ids, a.M * a.top_k, a.E, bucket, L, id0);
        if (c == 0) return;
        vecs = L.perm;
    } else {
        vstart = bucket * a.bt_chunk;
        c = min(a.bt_chunk, a.M - vstart);
    }
    // an expert's vectors in equal chunks of at most VCAP (dense: one chunk);
    // the ring holds bt_vmax >= every chunk's vectors
    const int nch = (c + VCAP - 1) / VCAP;
    const int cs = (c + nch - 1) / nch;
    for (int ch = 0; ch < nch; ++ch) {
        const int nv = min(cs, c - ch * cs);
        const uint16_t *cv = vecs ? vecs + ch * cs : nullptr;
        const int vs = vstart + ch * cs;
        if (nv <= 32)
            batched_chunk<RF, WAVES, MODE, 32>(a, lds, e, row_base, cv, vs, nv);
        else if (nv <= 64 || VCAP == 64)
            batched_chunk<RF, WAVES, MODE, (VCAP < 64 ? 32 : 64)>(a, lds, e, row_base, cv, vs, nv);
        else if (nv <= 96 || VCAP == 96)
            batched_chunk<RF, WAVES, MODE, (VCAP < 96 ? 32 : 96)>(a, lds, e, row_base, cv, vs, nv);
        else
            batched_chunk<RF, WAVES, MODE, (VCAP < 128 ? 32 : 128)>(a, lds, e, row_base, cv, vs, nv);
    }
}

// Dense calls with few vectors per weight matrix (a wide verify batch, a
// short prompt): one 32-row tile of a single matrix has too little work for
// a workgroup of waves that each own other rows, and too few tiles fill the
// GPU.  Here the waves of a workgroup split the tile's K instead: wave w
// takes the 128-weight slices w, w + WAVES, w + 2 WAVES, ... of the tile
// (32 rows x a chunk of at most VMAX vectors: 32, or 64 in 32-vector column
// fragments), stages their activations in an LDS ring of its own (two
// slices; one with 64 vectors) with no workgroup barrier in the loop, and
// the waves' partial tiles are summed in LDS in wave order at the end, so
// the result is bitwise reproducible.  The loads, decode and MFMA steps are
// the batched kernel's (lane (r, h): blocks 2 h and 2 h + 1 of row r per
// slice).
template <int WAVES, int VMAX>
__global__ __launch_bounds__(64 * WAVES) void qmv_batched_ks_kernel(const Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int XJ = VMAX / 4;                    // staging loads (4 vectors each) per lane and slice
    constexpr int CF = VMAX / 32;                   // column fragments of 32 vectors
    // activation slices per wave's LDS ring: two, or one with 64 vectors
    // (8 waves x 64 vectors x 256 bytes: 128 KB of LDS)
    constexpr int RING = VMAX == 64 ? 1 : kBRing;
    const int b = blockIdx.x;
    const int t = (b & 7) * a.bt_per_xcd + (b >> 3);
    if (t >= a.bt_tiles) return;
    const int chunk = t / a.bt_row_tiles;
    const int row_base = (t - chunk * a.bt_row_tiles) * 32;
    const int vstart = chunk * a.bt_chunk;
    const int nv = min(a.bt_chunk, a.M - vstart);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r = lane & 31;                        // row (A) / vector (B)
    const int h = lane >> 5;                        // k half of an MFMA step
    const int U = a.units;
    const int S = (U + 3) >> 2;                     // 128-weight slices
    const int KS = S > w ? (S - w + WAVES - 1) / WAVES : 0;   // this wave's slices
    uint8_t *const ring = lds + w * (RING * VMAX * 256);

    const int nf = (nv + 31) >> 5;                  // column fragments in use
    f32x16 acc[CF];
#pragma unroll
    for (int g = 0; g < CF; ++g)
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[g][k] = 0.0f;
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.codes, a.expert_cb);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.scales, a.expert_sb);
    const int n = row_base + r;
    const uint32_t oc = n < a.N ? (uint32_t)n * (uint32_t)a.rcb + 32u * h : kBPast;
    const uint32_t os = n < a.N ? (uint32_t)n * (uint32_t)a.rsb + 2u * h : kBPast;
    // activation staging: lane 16 c + p of load j holds chunk p of vector
    // 4 j + c of the chunk (offsets formed per load, not kept in registers)
    const int vl = lane >> 4, pl = lane & 15;
    const uint32_t xvb = (uint32_t)a.x_vec_bytes;
    const uint32_t xbase = (uint32_t)(vstart + vl) * xvb + 16u * pl;
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(a.x, a.M * a.x_vec_bytes);   // < 2^31
    const int K = a.K;
    auto slice = [&](int k) { return w + WAVES * k; };
    auto load_x = [&](int k, u32x4 (&xr)[XJ]) {
        const int s = slice(k);
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const bool ok = k < KS && 128 * s + 8 * pl < K && 4 * j + vl < nv;
            xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? xbase + 4u * j * xvb + 256u * s : kBPast, 0, 0);
        }
    };
    auto store_x = [&](int k, const u32x4 (&xr)[XJ]) {
        uint8_t *const buf = ring + (k % RING) * (VMAX * 256);
#pragma unroll
        for (int j = 0; j < XJ; ++j) *(u32x4 *)(buf + bx_off(4 * j + vl, pl)) = xr[j];
    };
    auto load_w = [&](int k, u32x4 (&wc)[2], uint32_t &sb) {
        const int s = slice(k);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const bool ok = k < KS && 4 * s + 2 * h + jb < U && oc != kBPast;
            wc[jb] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? oc + 64u * s + 16u * jb : kBPast, 0, 0);
        }
        sb = load_scale_pair(rs, os, s, U, h, k < KS && oc != kBPast);
    };
    int slow = 0;
    auto compute = [&](int k, const u32x4 (&wc)[2], uint32_t sbr) {
        const int s = slice(k);
        const uint8_t *const buf = ring + (k % RING) * (VMAX * 256);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const bool ok = k < KS && 4 * s + 2 * h + jb < U && oc != kBPast;
            const uint32_t sb = ok ? (sbr >> (8 * jb)) & 0xffu : 127u;
            slow |= (sb - 2u) > 250u;
            const float sc = __uint_as_float(sb << 23);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                bf16x8 Bv[CF];
#pragma unroll
                for (int g = 0; g < CF; ++g)
                    if (g < nf)
                        Bv[g] = __builtin_bit_cast(bf16x8, lds_read16(buf + bx_off(32 * g + r, 4 * (2 * h + jb) + tt)));
                const bf16x8 A = dec8(wc[jb][tt], sc);
#pragma unroll
                for (int g = 0; g < CF; ++g)
                    if (g < nf) acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bv[g], acc[g], 0, 0, 0);
            }
        }
    };
    u32x4 wc0[2], wc1[2], wc2[2];
    uint32_t sb0, sb1, sb2;
    if constexpr (RING == 1) {
        // two waves per SIMD hide each other's latency, so less is kept in
        // flight: weights two of this wave's slices ahead, activations one
        // (one register set, one LDS slice buffer: this wave's reads of slice
        // k are issued before its writes of slice k + 1, and a wave's LDS
        // operations complete in order); the slice count is padded to a
        // multiple of 2 (the padding reads past the buffers: zeros).  Three
        // weight slices ahead measured slower at 7168 x 7168 (27.7 -> 29.5 us)
        u32x4 xr[XJ];
        load_w(0, wc0, sb0);
        load_x(0, xr);
        load_w(1, wc1, sb1);
        store_x(0, xr);
        load_x(1, xr);
        auto step = [&](int k, u32x4 (&wc)[2], uint32_t &sb) {
            compute(k, wc, sb);
            store_x(k + 1, xr);
            load_x(k + 2, xr);
            load_w(k + 2, wc, sb);
        };
        for (int k = 0; k < KS; k += 2) {
            step(k, wc0, sb0);
            step(k + 1, wc1, sb1);
        }
        (void)wc2;
        (void)sb2;
    } else {
        // weights three of this wave's slices ahead, activations two; the
        // LDS ring is this wave's alone (a wave's LDS operations complete in
        // order, so writing slice k + 1's buffer after slice k - 1's reads of
        // it needs no barrier); the slice count is padded to a multiple of 6
        // (the padding reads past the buffers: zeros)
        u32x4 xr0[XJ], xr1[XJ];
        load_w(0, wc0, sb0);
        load_x(0, xr0);
        load_w(1, wc1, sb1);
        load_x(1, xr1);
        load_w(2, wc2, sb2);
        store_x(0, xr0);
        load_x(2, xr0);
        auto step = [&](int k, u32x4 (&wc)[2], uint32_t &sb, u32x4 (&xn)[XJ]) {
            store_x(k + 1, xn);
            load_x(k + 3, xn);
            compute(k, wc, sb);
            load_w(k + 3, wc, sb);
        };
        for (int k = 0; k < KS; k += 6) {
            step(k, wc0, sb0, xr1);
            step(k + 1, wc1, sb1, xr0);
            step(k + 2, wc2, sb2, xr1);
            step(k + 3, wc0, sb0, xr0);
            step(k + 4, wc1, sb1, xr1);
            step(k + 5, wc2, sb2, xr0);
        }
    }
    if (__syncthreads_or(slow)) {
        batched_chunk_exact<0>(a, 0, nullptr, vstart, nv, row_base, min(32, a.N - row_base));
        return;
    }
    // the waves' partial tiles, summed in wave order (every ring is free now)
    float *const red = (float *)lds;
    if (w > 0) {
#pragma unroll
        for (int g = 0; g < CF; ++g)
#pragma unroll
            for (int k = 0; k < 16; ++k) red[(((w - 1) * CF + g) * 16 + k) * 64 + lane] = acc[g][k];
    }
    __syncthreads();
    if (w != 0) return;
    // (one wave's partial tile at a time: reading every wave's at once
    // would take more registers than two waves per SIMD leave)
#pragma unroll 1
    for (int ww = 1; ww < WAVES; ++ww)
#pragma unroll
        for (int g = 0; g < CF; ++g)
#pragma unroll
            for (int k = 0; k < 16; ++k) acc[g][k] += red[(((ww - 1) * CF + g) * 16 + k) * 64 + lane];
    // lane (vector r, half h) of fragment g holds rows 8 i + 4 h .. + 3 of
    // the tile for vector 32 g + r
#pragma unroll
    for (int g = 0; g < CF; ++g) {
    const int col = 32 * g + r;
    if (col < nv) {
        float *const yrow = a.y + (size_t)(vstart + col) * a.N;
        const bool vec4 = (a.N & 3) == 0 && ((uintptr_t)a.y & 15) == 0;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int n0 = row_base + 8 * ii + 4 * h;
            if (n0 < a.N) {
                if (vec4) {
                    *(float4 *)(yrow + n0) = make_float4(acc[g][4 * ii], acc[g][4 * ii + 1], acc[g][4 * ii + 2],
                                                         acc[g][4 * ii + 3]);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (n0 + k < a.N) yrow[n0 + k] = acc[g][4 * ii + k];
                }
            }
        }
    }
    }
}

// [4 waves x 32 vectors, 8 waves x 32 vectors, 8 waves x 64 vectors]
extern const void *const kTableBatchedKS[3];
const void *const kTableBatchedKS[3] = {(const void *)&qmv_batched_ks_kernel<4, 32>,
                                        (const void *)&qmv_batched_ks_kernel<8, 32>,
                                        (const void *)&qmv_batched_ks_kernel<8, 64>};

// Instantiations: (waves per workgroup, 32-row fragments per wave, most
// vectors per chunk), the chunk capacity as large as the register budget
// allows without scratch memory.  Gate/up kernels hold a gate and an up
// fragment per output fragment.
#define QMV_BK(RF, W, MODE, VCAP) (const void *)&qmv_batched_kernel<RF, W, MODE, VCAP>
extern const int kBatchedShapes[kBatchedMenu][3];
// (waves, 32-row fragments per wave, most vectors per chunk); the 1- and
// 2-wave shapes give a single weight matrix (a dense call) enough tiles.
const int kBatchedShapes[kBatchedMenu][3] = {{4, 1, 128}, {4, 2, 96}, {4, 3, 96}, {8, 1, 128}, {1, 1, 32}, {2, 1, 64}};
extern const void *const kTableBatched[kBatchedMenu];
const void *const kTableBatched[kBatchedMenu] = {QMV_BK(1, 4, 0, 128), QMV_BK(2, 4, 0, 96), QMV_BK(3, 4, 0, 96),
                                                 QMV_BK(1, 8, 0, 128), QMV_BK(1, 1, 0, 32), QMV_BK(1, 2, 0, 64)};
extern const int kBatchedShapesGU[kBatchedMenu][3];
const int kBatchedShapesGU[kBatchedMenu][3] = {{4, 2, 128}, {4, 4, 64}, {4, 6, 32}, {8, 2, 64}, {1, 2, 32}, {2, 2, 64}};
extern const void *const kTableBatchedGU[kBatchedMenu];
const void *const kTableBatchedGU[kBatchedMenu] = {QMV_BK(2, 4, 1, 128), QMV_BK(4, 4, 1, 64), QMV_BK(6, 4, 1, 32),
                                                   QMV_BK(2, 8, 1, 64), QMV_BK(2, 1, 1, 32), QMV_BK(2, 2, 1, 64)};
#undef QMV_BK

}  // namespace qmv
