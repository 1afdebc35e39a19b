// qmv.hip -- launcher and C ABI of libqmv.so (declared in include/qmv.h).
//
// The host side validates arguments, picks a kernel instantiation from the
// call's shape, and enqueues the call's launches on the caller's stream.  It
// never synchronizes or touches device memory itself; the one allocation is
// the combine's per-slot rows for more than 4 tokens, stream-ordered from a
// pool of the library's (launch_combine).
#include "qmv_device.hpp"
#include "qmv.h"

#include <mutex>
#include <stdint.h>

// The same kernel tables built with 8 wave64s per workgroup (qmv_device.hpp).
namespace qmv_w8 {
extern const void *const kTable_mxfp4[3][4][5];
extern const void *const kTable_cb2[3][4][5];
extern const void *const kTable_cb2s[3][4][5];
extern const void *const kTable_cb3[3][4][5];
extern const void *const kTableGU_mxfp4[2][4][5];
extern const void *const kTableGU_cb2[2][4][5];
extern const void *const kTableGU_cb2s[2][4][5];
extern const void *const kTableGU_cb3[2][4][5];
extern const void *const kTableCB_mxfp4[4][4];
extern const void *const kTableCB_cb2[4][4];
extern const void *const kTableCB_cb2s[4][4];
extern const void *const kTableCB_cb3[4][4];
extern const void *const kTableQ_cb2[3][4][5];
extern const void *const kTableQ_cb2s[3][4][5];
extern const void *const kTableQ_cb3[3][4][5];
extern const void *const kTableQGU_cb2[2][4][5];
extern const void *const kTableQGU_cb2s[2][4][5];
extern const void *const kTableQGU_cb3[2][4][5];
extern const void *const kTableQCB_cb2[4][4];
extern const void *const kTableQCB_cb2s[4][4];
extern const void *const kTableQCB_cb3[4][4];
extern const void *const kTable_mxfp4i[3][4][5];
extern const void *const kTableGU_mxfp4i[2][4][5];
extern const void *const kTableCB_mxfp4i[4][4];
}  // namespace qmv_w8

// Dense MXFP4 x bf16 with 2 to 4 vectors on the matrix cores (qmv_k_mxfp4m.hip):
// [4 waves, 8 waves] per workgroup.
namespace qmv {
extern const void *const kTableDense4[2];
}

// MXFP4 x bf16 with more than 4 vectors: expert-batched gather, fused
// gate/up gather and dense calls on the 32x32x16 bf16 matrix cores
// (qmv_k_mxfp4b.hip): a menu of kernel shapes, each (waves per workgroup,
// 32-row fragments per wave, most vectors per chunk); gate/up kernels hold a
// gate and an up fragment per output fragment.
// 2-bit and 3-bit codebook weights x int8 activations with more than 4
// vectors per expert on the int8 4x4x4 matrix cores (qmv_k_cbm.hip):
// [int8 x, bf16 x quantized in staging][2-bit, 3-bit][vector groups of 4 per
// staged chunk: 1, 2, 3, 4]; [8 waves, 12 waves] per workgroup.
namespace qmv {
extern const void *const kTableGmma[2][2][2][4];
}

// Dense MXFP4 x bf16 with 9 to 64 vectors: 32-row tiles with K split over
// the waves of a workgroup (qmv_k_mxfp4b.hip): [4 waves x 32 vectors, 8 waves
// x 32 vectors, 8 waves x 64 vectors].
namespace qmv {
extern const void *const kTableBatchedKS[3];
}

namespace qmv {
constexpr int kBatchedMenu = 6;
extern const int kBatchedShapes[kBatchedMenu][3];
extern const void *const kTableBatched[kBatchedMenu];
extern const int kBatchedShapesGU[kBatchedMenu][3];
extern const void *const kTableBatchedGU[kBatchedMenu];
}

namespace {

using namespace qmv;
using namespace qmv_host;

// Kernels for bf16 activations quantized in staging (2-bit and 3-bit weights).
const void *kernel_for_q8(int wi, int kind, int variant, int li, int ci, bool gate_up)
{
    if (wi == 1) {
        if (gate_up) {
            switch (kind) {
            case kCB2: return qmv_w8::kTableQGU_cb2[variant][li][ci];
            case kCB2S: return qmv_w8::kTableQGU_cb2s[variant][li][ci];
            default: return qmv_w8::kTableQGU_cb3[variant][li][ci];
            }
        }
        switch (kind) {
        case kCB2: return qmv_w8::kTableQ_cb2[variant][li][ci];
        case kCB2S: return qmv_w8::kTableQ_cb2s[variant][li][ci];
        default: return qmv_w8::kTableQ_cb3[variant][li][ci];
        }
    }
    if (gate_up) {
        switch (kind) {
        case kCB2: return kTableQGU_cb2[variant][li][ci];
        case kCB2S: return kTableQGU_cb2s[variant][li][ci];
        default: return kTableQGU_cb3[variant][li][ci];
        }
    }
    switch (kind) {
    case kCB2: return kTableQ_cb2[variant][li][ci];
    case kCB2S: return kTableQ_cb2s[variant][li][ci];
    default: return kTableQ_cb3[variant][li][ci];
    }
}

const void *kernel_for(int wi, int kind, int variant, int li, int ci, bool gate_up, bool q8)
{
    if (q8)
        return kernel_for_q8(wi, kind, variant, li, ci, gate_up);
    if (wi == 1) {
        if (gate_up) {
            switch (kind) {
            case kMXFP4: return qmv_w8::kTableGU_mxfp4[variant][li][ci];
            case kMXFP4I: return qmv_w8::kTableGU_mxfp4i[variant][li][ci];
            case kCB2: return qmv_w8::kTableGU_cb2[variant][li][ci];
            case kCB2S: return qmv_w8::kTableGU_cb2s[variant][li][ci];
            default: return qmv_w8::kTableGU_cb3[variant][li][ci];
            }
        }
        switch (kind) {
        case kMXFP4: return qmv_w8::kTable_mxfp4[variant][li][ci];
        case kMXFP4I: return qmv_w8::kTable_mxfp4i[variant][li][ci];
        case kCB2: return qmv_w8::kTable_cb2[variant][li][ci];
        case kCB2S: return qmv_w8::kTable_cb2s[variant][li][ci];
        default: return qmv_w8::kTable_cb3[variant][li][ci];
        }
    }
    if (gate_up) {
        switch (kind) {
        case kMXFP4: return kTableGU_mxfp4[variant][li][ci];
        case kMXFP4I: return kTableGU_mxfp4i[variant][li][ci];
        case kCB2: return kTableGU_cb2[variant][li][ci];
        case kCB2S: return kTableGU_cb2s[variant][li][ci];
        default: return kTableGU_cb3[variant][li][ci];
        }
    }
    switch (kind) {
    case kMXFP4: return kTable_mxfp4[variant][li][ci];
    case kMXFP4I: return kTable_mxfp4i[variant][li][ci];
    case kCB2: return kTable_cb2[variant][li][ci];
    case kCB2S: return kTable_cb2s[variant][li][ci];
    default: return kTable_cb3[variant][li][ci];
    }
}

// Grouped kernels (more than 4 tokens through the decode kernels' MACs), all
// with 4-wave workgroups.
const void *grouped_kernel_for(int kind, int mode, int li, int ci, bool q8)
{
    if (q8) {
        switch (kind) {
        case kCB2: return kTableQGR_cb2[mode][li][ci];
        case kCB2S: return kTableQGR_cb2s[mode][li][ci];
        default: return kTableQGR_cb3[mode][li][ci];
        }
    }
    switch (kind) {
    case kMXFP4: return kTableGR_mxfp4[mode][li][ci];
    case kMXFP4I: return kTableGR_mxfp4i[mode][li][ci];
    case kCB2: return kTableGR_cb2[mode][li][ci];
    case kCB2S: return kTableGR_cb2s[mode][li][ci];
    default: return kTableGR_cb3[mode][li][ci];
    }
}

const void *combine_kernel_for(int wi, int kind, int li, int ci, bool q8)
{
    if (q8) {
        if (wi == 1) {
            switch (kind) {
            case kCB2: return qmv_w8::kTableQCB_cb2[li][ci];
            case kCB2S: return qmv_w8::kTableQCB_cb2s[li][ci];
            default: return qmv_w8::kTableQCB_cb3[li][ci];
            }
        }
        switch (kind) {
        case kCB2: return kTableQCB_cb2[li][ci];
        case kCB2S: return kTableQCB_cb2s[li][ci];
        default: return kTableQCB_cb3[li][ci];
        }
    }
    if (wi == 1) {
        switch (kind) {
        case kMXFP4: return qmv_w8::kTableCB_mxfp4[li][ci];
        case kMXFP4I: return qmv_w8::kTableCB_mxfp4i[li][ci];
        case kCB2: return qmv_w8::kTableCB_cb2[li][ci];
        case kCB2S: return qmv_w8::kTableCB_cb2s[li][ci];
        default: return qmv_w8::kTableCB_cb3[li][ci];
        }
    }
    switch (kind) {
    case kMXFP4: return kTableCB_mxfp4[li][ci];
    case kMXFP4I: return kTableCB_mxfp4i[li][ci];
    case kCB2: return kTableCB_cb2[li][ci];
    case kCB2S: return kTableCB_cb2s[li][ci];
    default: return kTableCB_cb3[li][ci];
    }
}

std::once_flag g_attr_once[2][2][2][5][3][4][5];        // [q8][waves][gate_up][kind][variant][lpr][cpl]
hipError_t g_attr_err[2][2][2][5][3][4][5];
std::once_flag g_cattr_once[2][2][5][4][4];             // [q8][waves][kind][lpr][cpl]
hipError_t g_cattr_err[2][2][5][4][4];

// Arguments common to every kernel of a call (Args in qmv_device.hpp).
Args base_args(int wfmt, int afmt, int kind, const void *codes, const void *scales, int E,
               const int32_t *ids, int M, int top_k, const void *x, const void *xs,
               int x_per_slot, float *y, int N, int K)
{
    Args a;
    a.codes = (const uint8_t *)codes;
    a.scales = (const uint8_t *)scales;
    a.codes2 = nullptr;
    a.scales2 = nullptr;
    a.ids = ids;
    a.route_w = nullptr;
    a.x = (const uint8_t *)x;
    a.xs = (const uint16_t *)xs;
    a.y = y;
    a.rcb = (int)row_code_bytes(wfmt, K);
    a.rsb = (int)row_scale_bytes(wfmt, K);
    a.expert_cb = (long long)N * a.rcb;
    a.expert_sb = (long long)N * a.rsb;
    a.x_vec_bytes = (afmt == QMV_A_Q8B32) ? K : 2 * K;      // int8, or bf16
    a.E = E;
    a.M = M;
    a.top_k = top_k;
    a.N = N;
    a.K = K;
    a.units = K / kUnitWeights[kind];
    a.x_per_slot = x_per_slot;
    a.x_early = 0;
    a.rows_per_tile = 0;
    const int vec_bytes = a.units * (kUnitXB[kind] + kUnitAB[kind]);
    a.lds_vec_bytes = (vec_bytes + 15) & ~15;
    return a;
}

// Batched MXFP4 x bf16 (M > 4): LDS of one workgroup = a ring of 2
// activation slice buffers (128 weights of vmax vectors, 256 B each), the
// pair scan's counts and the tile's pair list: at most 64 + 1 + 16 KB.
size_t batched_lds(int vmax, int pairs)
{
    return (size_t)2 * vmax * 256 + kPairCountBytes + (((size_t)2 * pairs + 15) & ~(size_t)15);
}

std::once_flag g_b_once[2][kBatchedMenu];
hipError_t g_b_err[2][kBatchedMenu];

int g_cu_count[64];
std::once_flag g_cu_once[64];

int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::call_once(g_cu_once[dev], [&] {
        int n = 0;
        const bool ok = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
        g_cu_count[dev] = ok && n > 0 ? n : 256;
    });
    return g_cu_count[dev];
}

// Tiles: (expert, R rows) for a gather, (chunk of vectors, R rows) for a
// dense call, one workgroup each; R = 32 x fragments x waves.  The choice
// minimizes the estimated time of the call: every CU streams, per weight,
// R * 0.53 bytes of its tile's codes and scales (twice for gate/up) and
// 2 bytes per vector of activations, one tile after another, so the time is
// the number of rounds of tiles over the CUs times that per-tile stream; ties
// go to taller tiles (fewer re-reads of the activations).  A gather's busy
// tiles are its experts that some pair selects, estimated as min(E, pairs).
// Dense calls also choose the vector chunk: a single weight matrix of a few
// thousand rows gives too few row tiles to fill the GPU, and two chunks of
// 32 vectors give twice the tiles for twice the weight reads (L2 serves the
// second).
struct BatchedPlan { int shape, waves, rows, chunk, row_tiles, tiles, cap; };

BatchedPlan plan_batched(bool gather, bool gate_up, int E, int pairs, int N)
{
    const int cus = cu_count();
    BatchedPlan best = {0, 0, 0, 0, 0, 0, 0};
    double best_cost = 0.0;
    const int busy = gather ? (pairs < E ? pairs : E) : 1;
    const double vbar = gather ? (double)pairs / busy : 0.0;
    for (int sh = 0; sh < kBatchedMenu; ++sh)
        for (int ci = 0; ci < (gather ? 1 : 3); ++ci) {
            const int *const m = gate_up ? kBatchedShapesGU[sh] : kBatchedShapes[sh];
            const int waves = m[0], cap = m[2];
            const int rows = 32 * m[1] * waves / (gate_up ? 2 : 1);
            int chunk = 0;
            if (!gather) {
                chunk = ci == 0 ? (pairs < cap ? pairs : cap) : ci == 1 ? 64 : 32;
                if (chunk > cap || (ci > 0 && chunk >= pairs)) continue;
            }
            const int rt = (N + rows - 1) / rows;
            const long long tiles = (long long)rt * (gather ? busy : (pairs + chunk - 1) / chunk);
            const long long rounds = (tiles + cus - 1) / cus;
            // a gather tile takes its expert's vectors in passes of at most cap
            const double passes = gather ? (vbar > cap ? vbar / cap + 1.0 : 1.0) : 1.0;
            const double v = gather ? vbar : (double)chunk;
            const double cost = (double)rounds * (passes * rows * 0.53125 * (gate_up ? 2 : 1) + 2.0 * v);
            if (best.rows == 0 || cost < best_cost * 0.999) {
                best = {sh, waves, rows, chunk, rt, 0, cap};
                best_cost = cost;
            }
        }
    best.tiles = best.row_tiles * (gather ? E : (pairs + best.chunk - 1) / best.chunk);
    return best;
}

// Grid: one workgroup per tile, dealt to the XCDs in contiguous runs (the
// kernel maps workgroup b to tile (b % 8) * per_xcd + b / 8).  Measured on
// the 512-token gpt-oss prefill chunk (32 experts, K = N = 2880): see the
// kernel's header for the tile shapes.
qmv_status_t launch_batched(const void *codes, const void *scales, const void *codes2, const void *scales2,
                            int E, const int32_t *ids, int M, int top_k, const void *x, int x_per_slot,
                            float *y, int N, int K, hipStream_t stream)
{
    const bool gather = ids != nullptr;
    const bool gate_up = codes2 != nullptr;
    Args a = base_args(QMV_W_MXFP4, QMV_A_BF16, kMXFP4, codes, scales, gather ? E : 1, ids, M,
                       gather ? top_k : 1, x, nullptr, gather ? x_per_slot : 0, y, N, K);
    a.codes2 = (const uint8_t *)codes2;
    a.scales2 = (const uint8_t *)scales2;
    const int pairs = gather ? M * top_k : M;
    const BatchedPlan pl = plan_batched(gather, gate_up, gather ? E : 1, pairs, N);
    a.rows_per_tile = pl.rows;
    a.bt_row_tiles = pl.row_tiles;
    a.bt_tiles = pl.tiles;
    a.bt_per_xcd = (pl.tiles + 7) / 8;
    a.bt_chunk = pl.chunk;
    // the activation ring holds the most vectors one chunk can have
    int vmost = gather ? pairs : pl.chunk;
    vmost = vmost < pl.cap ? vmost : pl.cap;
    a.bt_vmax = vmost <= 32 ? 32 : vmost <= 64 ? 64 : vmost <= 96 ? 96 : 128;
    const int gu = gate_up ? 1 : 0;
    const void *fn = gate_up ? kTableBatchedGU[pl.shape] : kTableBatched[pl.shape];
    std::call_once(g_b_once[gu][pl.shape], [&] {
        g_b_err[gu][pl.shape] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    batched_lds(128, kMaxPairsBatched));
    });
    if (g_b_err[gu][pl.shape] != hipSuccess)
        return QMV_EHIP;
    void *kargs[] = {&a};
    const size_t lds = batched_lds(a.bt_vmax, gather ? pairs : 0);
    if (hipLaunchKernel(fn, dim3((unsigned)(8 * a.bt_per_xcd)), dim3(64 * pl.waves), kargs, lds, stream) !=
        hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

std::once_flag g_gr_once[2][2][5][4][5];                // [q8][mode][kind][lpr][cpl]
hipError_t g_gr_err[2][2][5][4][5];
int g_gr_occ[2][2][5][4][5];                            // workgroups per CU by registers

// LDS of a grouped workgroup: four staged activation vectors, the pair
// scan's counts, the expert bitmap and the pair list.
size_t grouped_lds(int vec_bytes, int pairs)
{
    return (size_t)4 * vec_bytes + kPairCountBytes + kExpertBitmapBytes + (((size_t)2 * pairs + 15) & ~(size_t)15);
}

// More than 4 tokens on the decode kernels' MACs (every format pair; MXFP4 x
// bf16 when few pairs share an expert): one launch of 4-wave workgroups, each
// taking a run of (expert slot, row tile) items (plan_grouped).
qmv_status_t launch_grouped(int wfmt, int afmt, const void *codes, const void *scales, const void *codes2,
                            const void *scales2, int E, const int32_t *ids, int M, int top_k, const void *x,
                            const void *xs, int x_per_slot, float *y, int N, int K, hipStream_t stream)
{
    const bool gather = ids != nullptr;
    const bool gate_up = codes2 != nullptr;
    const int kind = kind_of(wfmt, afmt, K);
    const bool q8 = afmt == QMV_A_BF16_Q8;
    const int mode = gate_up ? 1 : 0;
    const int pairs = gather ? M * top_k : M;
    const int busy = gather ? (pairs < E ? pairs : E) : 1;
    const int units = K / kUnitWeights[kind];
    Args a = base_args(wfmt, afmt, kind, codes, scales, gather ? E : 1, ids, M, gather ? top_k : 1, x, xs,
                       gather ? x_per_slot : 0, y, N, K);
    a.codes2 = (const uint8_t *)codes2;
    a.scales2 = (const uint8_t *)scales2;
    const size_t lds = grouped_lds(a.lds_vec_bytes, gather ? pairs : 0);
    // per kernel, once: the largest LDS any call may ask for, and how many
    // workgroups a CU holds by the kernel's registers
    auto prepare = [&](int li, int ci) -> hipError_t {
        std::call_once(g_gr_once[q8][mode][kind][li][ci], [&] {
            const void *f = grouped_kernel_for(kind, mode, li, ci, q8);
            const int umax = kMaxK / kUnitWeights[kind];
            const int vmax = (umax * (kUnitXB[kind] + kUnitAB[kind]) + 15) & ~15;
            hipError_t err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 grouped_lds(vmax, kMaxPairsBatched));
            int n = 0;
            if (err == hipSuccess)
                err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 64 * kWaveMenu[0], 0);
            g_gr_err[q8][mode][kind][li][ci] = err;
            g_gr_occ[q8][mode][kind][li][ci] = n > 0 ? n : 1;
        });
        return g_gr_err[q8][mode][kind][li][ci];
    };
    bool failed = false;
    const long long row_bytes = row_code_bytes(wfmt, K) + row_scale_bytes(wfmt, K);
    const GroupedPlan p = plan_grouped(units, row_bytes, N, busy, gate_up, cu_count(),
                                       (long long)lds, [&](int li, int ci) {
                                           if (prepare(li, ci) != hipSuccess) failed = true;
                                           return g_gr_occ[q8][mode][kind][li][ci];
                                       });
    if (failed)
        return QMV_EHIP;
    a.rows_per_tile = p.rows_per_tile;
    a.gr_tiles = p.tiles;
    const void *fn = grouped_kernel_for(kind, mode, p.sh.li, p.sh.ci, q8);
    void *kargs[] = {&a};
    if (hipLaunchKernel(fn, dim3((unsigned)p.grid), dim3(64 * kWaveMenu[0]), kargs, lds, stream) != hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

std::once_flag g_gm_once[2][2][2][4];
hipError_t g_gm_err[2][2][2][4];
int g_gm_occ[2][2][2][4];                               // workgroups per CU by registers
// Workgroups of 12 waves (three per SIMD, which cover each other's latency,
// with up to 168 registers per lane: 4 vector groups of 2-bit weights, 3 of
// 3-bit ones) for calls with many (expert, 48-row tile) items, 8 waves
// (32-row tiles, up to 4 groups) for the others, whose tiles would not fill
// the chip.  Measured on MI355X, 12 against 8 waves: C7 421 -> 408 us, C8
// 745 -> 667 us (4 waves: 500-640 and 700-806 us); 2-bit with 4 groups
// against 3 at 12 waves: C7 400 -> 384-391 us; dense 16 and 64 vectors of
// 7168 x 7168 2-bit, 16 of 7168 x 2048 3-bit: 15.3, 53 and 10.3 us at 8
// waves against 17.9, 62 and 14.4 at 12.
constexpr int kGmWaveMenu[2] = {8, 12};
constexpr int kGmNvg[4] = {1, 2, 3, 4};

// Codebook weights x int8 activations, more than 4 vectors, several per
// expert: one launch of the int8 matrix-core kernel.  A workgroup's LDS:
// the staged vector groups (per group of 4 and unit: the activations in
// selector order and the per-block side data), the pair scan and bitmap,
// the pair list, the per-expert counts.  The groups per chunk cover the
// average expert's vectors (with room for a few more) as far as the LDS
// allows; the grid is at most one round of the chip, each workgroup a run of
// (expert, row tile) items of equal cost with each expert's vector count
// weighed in, so one staging of a chunk serves many row tiles.
qmv_status_t launch_gmma(int wfmt, int afmt, int kind, const void *codes, const void *scales, int E,
                         const int32_t *ids, int M, int top_k, const void *x, const void *xs, int x_per_slot,
                         float *y, int N, int K, hipStream_t stream)
{
    const bool gather = ids != nullptr;
    const int qi = afmt == QMV_A_BF16_Q8 ? 1 : 0;
    const int fi = kind == kCB2 ? 0 : 1;
    const int pairs = gather ? M * top_k : M;
    const int busy = gather ? (pairs < E ? pairs : E) : 1;
    const int U = K / kUnitWeights[kind];
    const int Up = (U + 15) & ~15;
    const size_t group_bytes = (size_t)Up * (fi == 0 ? 256 + 32 : 128 + 16);
    const size_t tail =
        kPairCountBytes + kExpertBitmapBytes + kExpertCountBytes + (((size_t)2 * (gather ? pairs : 0) + 15) & ~(size_t)15);
    // groups of 4 for twice the average expert's vectors (the counts spread
    // around the average, and every further chunk decodes the weights again),
    // as far as one workgroup's LDS allows
    const int avg = (pairs + busy - 1) / busy;
    const int want = (2 * avg + 3) / 4;
    // 12 waves when the 48-row tiles give at least two items per CU
    const int wv = (long long)busy * ((N + 47) / 48) >= 2LL * cu_count() ? 1 : 0;
    const int waves = kGmWaveMenu[wv];
    const int nimax = wv == 1 && fi == 1 ? 2 : 3;
    int ni = want < 1 ? 0 : want - 1 > nimax ? nimax : want - 1;
    // the staged groups (2-bit with 4 groups: 32 bytes of padding per unit
    // in the side data), then the tail
    auto staged = [&](int k) { return kGmNvg[k] * group_bytes + (fi == 0 && kGmNvg[k] == 4 ? (size_t)Up * 32 : 0); };
    while (ni > 0 && staged(ni) + tail > (size_t)kLdsPerCU) --ni;
    const size_t lds = staged(ni) + tail;
    if (lds > (size_t)kLdsPerCU)
        return QMV_EUNSUPPORTED;
    const void *fn = kTableGmma[wv][qi][fi][ni];
    std::call_once(g_gm_once[wv][qi][fi][ni], [&] {
        hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsPerCU);
        int n = 0;
        if (err == hipSuccess)
            err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64 * waves, 0);
        g_gm_err[wv][qi][fi][ni] = err;
        g_gm_occ[wv][qi][fi][ni] = n > 0 ? n : 1;
    });
    if (g_gm_err[wv][qi][fi][ni] != hipSuccess)
        return QMV_EHIP;
    Args a = base_args(wfmt, afmt, kind, codes, scales, gather ? E : 1, ids, M, gather ? top_k : 1, x, xs,
                       gather ? x_per_slot : 0, y, N, K);
    a.rows_per_tile = 4 * waves;
    a.gr_tiles = (N + a.rows_per_tile - 1) / a.rows_per_tile;
    const long long items = (long long)busy * a.gr_tiles;
    long long per_cu = g_gm_occ[wv][qi][fi][ni];
    const long long by_lds = (long long)kLdsPerCU / (long long)lds;
    if (per_cu > by_lds) per_cu = by_lds;
    if (per_cu < 1) per_cu = 1;
    const long long slots = per_cu * cu_count();
    const unsigned grid = (unsigned)(items < slots ? items : slots);
    void *kargs[] = {&a};
    if (hipLaunchKernel(fn, dim3(grid), dim3(64 * waves), kargs, lds, stream) != hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

std::once_flag g_ks_once[3];
hipError_t g_ks_err[3];
constexpr int kKsMaxM = 64;

// Dense MXFP4 x bf16, 9 to 64 vectors: one launch of K-split tiles, 32 rows
// by all the call's vectors.  Up to 32 vectors: 8 waves per workgroup when K
// has at least 32 slices of 128 weights, else 4, each wave with a two-slice
// activation ring in LDS; 33 to 64 vectors: two 32-vector column fragments,
// 8 waves (two per SIMD, which cover each other's latency), a one-slice
// ring per wave (128 KB of LDS).  Measured on MI355X against the batched
// kernel (two 32-vector chunks of 64-row tiles): 7168 x 7168 with 64
// vectors 31.9 -> 23.6 us, 40 vectors 31.9 -> 22.3; 2880 x 2880 with 64
// vectors 16.7 -> 14.4; 7168 rows x K = 2048, 64 vectors, 12.9 -> 12.3;
// 2048 rows x K = 7168, 64 vectors, 35.1 -> 22.3 us.  A 4-wave version with
// a two-slice ring (one wave per SIMD) took 33 us at 7168 x 7168.
qmv_status_t launch_batched_ks(const void *codes, const void *scales, const void *x, float *y, int M, int N,
                               int K, hipStream_t stream)
{
    Args a = base_args(QMV_W_MXFP4, QMV_A_BF16, kMXFP4, codes, scales, 1, nullptr, M, 1, x, nullptr, 0, y, N,
                       K);
    const int slices = (K + 127) / 128;
    const int vecs = M > 32 ? 64 : 32;
    const int wi = M > 32 ? 2 : slices >= 32 ? 1 : 0;
    const int waves = wi ? 8 : 4;
    const int ring = vecs == 64 ? 1 : 2;
    a.bt_chunk = M;
    a.bt_row_tiles = (N + 31) / 32;
    a.bt_tiles = a.bt_row_tiles;
    a.bt_per_xcd = (a.bt_tiles + 7) / 8;
    a.bt_vmax = vecs;
    const size_t lds = (size_t)waves * ring * vecs * 256;
    const void *fn = kTableBatchedKS[wi];
    std::call_once(g_ks_once[wi], [&] {
        g_ks_err[wi] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    });
    if (g_ks_err[wi] != hipSuccess)
        return QMV_EHIP;
    void *kargs[] = {&a};
    if (hipLaunchKernel(fn, dim3(8 * a.bt_per_xcd), dim3(64 * waves), kargs, lds, stream) != hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

std::once_flag g_d4_once[2];
hipError_t g_d4_err[2];

qmv_status_t launch_dense4(const void *codes, const void *scales, const void *x, float *y, int M,
                           int N, int K, hipStream_t stream)
{
    Args a = base_args(QMV_W_MXFP4, QMV_A_BF16, kMXFP4, codes, scales, 1, nullptr, M, 1, x, nullptr,
                       0, y, N, K);
    const int waves = dense4_waves(N);
    const int wi = waves == 8 ? 1 : 0;
    const void *fn = kTableDense4[wi];
    std::call_once(g_d4_once[wi], [&] {
        g_d4_err[wi] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           dense4_lds(kMaxK, waves));
    });
    if (g_d4_err[wi] != hipSuccess)
        return QMV_EHIP;
    const unsigned quads = (unsigned)((N + 3) / 4);
    const dim3 grid((quads + waves - 1) / waves);
    void *kargs[] = {&a};
    if (hipLaunchKernel(fn, grid, dim3(64 * waves), kargs, dense4_lds(K, waves), stream) != hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

// codes2/scales2 non-null selects the gate/up mode: codes/scales are the gate
// projection, codes2/scales2 the up projection, y = swiglu(gate x, up x).
qmv_status_t launch(int wfmt, int afmt, const void *codes, const void *scales, const void *codes2,
                    const void *scales2, int E, const int32_t *ids,
                    int M, int top_k, const void *x, const void *xs, int x_per_slot,
                    float *y, int N, int K, hipStream_t stream)
{
    const bool gather = ids != nullptr;
    const bool gate_up = codes2 != nullptr;
    const int kind = kind_of(wfmt, afmt, K);
    // Dense MXFP4 x bf16 with 9 to 64 vectors: K-split tiles, one launch.
    // Measured on 7168 x 7168: 16 vectors 34.3 us as four 4-vector launches,
    // 20.8 us here; 24 vectors 34.5 (batched) against 21.0; 5 vectors 16.6
    // as two launches against 20.7 here; 64 vectors 31.9 (batched) against
    // 23.6.  Every tile restages all of x through L2 (up to 64 vectors x K
    // bf16 per 32-row tile: eight times the tile's weight bytes at
    // K = 7168), which bounds this shape.
    if (!gather && !gate_up && kind == kMXFP4 && afmt == QMV_A_BF16 && M > kDenseGroupsMaxM && M <= kKsMaxM)
        return launch_batched_ks(codes, scales, x, y, M, N, K, stream);
    if (!gather && !gate_up && kind == kMXFP4 && afmt == QMV_A_BF16 && M > kMaxM && M <= kDenseGroupsMaxM) {
        // A dense call with a few more than 4 vectors: groups of up to 4 on
        // the dense 4-vector kernel, each a launch over its own rows of x
        // and y (7168 x 7168: 4 vectors 8.75 us; 5 vectors 16.6 us).
        for (int m0 = 0; m0 < M; m0 += kMaxM) {
            const int mg = M - m0 < kMaxM ? M - m0 : kMaxM;
            const qmv_status_t st = launch(wfmt, afmt, codes, scales, nullptr, nullptr, 1, nullptr, mg, 1,
                                           (const uint8_t *)x + (size_t)m0 * K * 2, nullptr, 0,
                                           y + (size_t)m0 * N, N, K, stream);
            if (st != QMV_OK)
                return st;
        }
        return QMV_OK;
    }
    if (M > kMaxM) {
        // More than 4 tokens: MXFP4 x bf16 on the batched matrix-core kernel
        // when experts are shared (at least two pairs per expert), every
        // other case on the grouped kernel.  A gather with fewer than two
        // (token, slot) pairs per expert reuses almost no weights, and the
        // decode kernels' MACs stream them faster than the matrix-core tiles
        // (4 of 256 experts, K = 7168, N = 2048: 5 tokens 105 us and 16
        // tokens 175 us batched, 32 and 94 us as groups of 4 tokens).
        if (kind == kMXFP4 && afmt == QMV_A_BF16 && (!gather || (long long)M * top_k >= 2LL * E))
            return launch_batched(codes, scales, codes2, scales2, E, ids, M, top_k, x, x_per_slot, y, N, K, stream);
        // codebook weights x int8 with at least two vectors per expert on
        // average: the int8 matrix-core kernel
        if ((kind == kCB2 || kind == kCB3) && (afmt == QMV_A_Q8B32 || afmt == QMV_A_BF16_Q8) && !gate_up &&
            (gather ? (long long)M * top_k >= 2LL * E : M >= 8))
            return launch_gmma(wfmt, afmt, kind, codes, scales, E, ids, M, top_k, x, xs, x_per_slot, y, N, K,
                               stream);
        // A gather of at most 64 tokens with fewer than two pairs per expert
        // (a verify batch over many experts) reuses almost no weights: as
        // token groups of up to 4 on the decode kernels, one launch per
        // group, it measured 10-20% faster than one grouped launch (MXFP4,
        // 4 of 256, 7168 -> 2048: 5 tokens 31.8 against 37.9 us, 16 tokens
        // 95.5 against 114.6 us; 2-bit, 8 tokens 34.6 against 37.8 us).
        if (gather && (long long)M * top_k < 2LL * E && M <= kSplitMaxM) {
            const size_t xe = afmt == QMV_A_Q8B32 ? 1 : 2;                 // bytes per activation
            const size_t xv = x_per_slot ? (size_t)top_k : 1;             // vectors per token
            for (int m0 = 0; m0 < M; m0 += kMaxM) {
                const int mg = M - m0 < kMaxM ? M - m0 : kMaxM;
                const qmv_status_t st = launch(
                    wfmt, afmt, codes, scales, codes2, scales2, E, ids + (size_t)m0 * top_k, mg, top_k,
                    (const uint8_t *)x + (size_t)m0 * xv * K * xe,
                    xs ? (const void *)((const uint16_t *)xs + (size_t)m0 * xv * (K / 32)) : nullptr, x_per_slot,
                    y + (size_t)m0 * top_k * N, N, K, stream);
                if (st != QMV_OK)
                    return st;
            }
            return QMV_OK;
        }
        return launch_grouped(wfmt, afmt, codes, scales, codes2, scales2, E, ids, M, top_k, x, xs, x_per_slot, y,
                              N, K, stream);
    }
    if (!gather && !gate_up && kind == kMXFP4 && afmt == QMV_A_BF16 && M >= 2)
        return launch_dense4(codes, scales, x, y, M, N, K, stream);
    const int units = K / kUnitWeights[kind];
    const int nv_needed = !gather ? M : (x_per_slot ? (M * top_k < 4 ? M * top_k : 4) : M);
    int variant, rt;
    if (nv_needed == 1) { variant = 0; rt = 2; }
    else if (gather)    { variant = 1; rt = 2; }
    else                { variant = 2; rt = 4; }
    const int nvmax = variant == 0 ? 1 : 4;
    const long long rows_total = (long long)N * (gather ? M * top_k : 1) * (gate_up ? 2 : 1);
    Shape sh;
    const bool q8 = afmt == QMV_A_BF16_Q8;
    int wi = q8 ? 1 : 0;
    if (!tuned_shape(kind, variant, gate_up, q8, K, N, gather ? M * top_k : 1, wi, sh))
        sh = pick_shape(variant, units, rows_total, rt);
    Args a = base_args(wfmt, afmt, kind, codes, scales, gather ? E : 1, ids, M, gather ? top_k : 1, x, xs,
                       gather ? x_per_slot : 0, y, N, K);
    a.codes2 = (const uint8_t *)codes2;
    a.scales2 = (const uint8_t *)scales2;
    a.x_early = (!gather || (M == 1 && !x_per_slot)) ? 1 : 0;
    const int waves = kWaveMenu[wi];
    a.rows_per_tile = waves * (64 / sh.lpr) * (gate_up ? 1 : rt);
    const size_t lds = (size_t)nvmax * a.lds_vec_bytes;

    const void *fn = kernel_for(wi, kind, variant, sh.li, sh.ci, gate_up, q8);
    // Largest dynamic LDS this kernel can ask for (K = kMaxK, all vectors).
    std::call_once(g_attr_once[q8][wi][gate_up][kind][variant][sh.li][sh.ci], [&] {
        const int umax = kMaxK / kUnitWeights[kind];
        const int vmax = (umax * (kUnitXB[kind] + kUnitAB[kind]) + 15) & ~15;
        g_attr_err[q8][wi][gate_up][kind][variant][sh.li][sh.ci] = hipFuncSetAttribute(
            fn, hipFuncAttributeMaxDynamicSharedMemorySize, nvmax * vmax);
    });
    if (g_attr_err[q8][wi][gate_up][kind][variant][sh.li][sh.ci] != hipSuccess)
        return QMV_EHIP;

    const dim3 grid((unsigned)((N + a.rows_per_tile - 1) / a.rows_per_tile),
                    (unsigned)(gather ? M * top_k : 1));
    void *kargs[] = {&a};
    if (hipLaunchKernel(fn, grid, dim3(64 * waves), kargs, lds, stream) != hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

// The router-weighted sum over each token's slots of the per-slot rows g
// ([M][top_k][N], fp32): y[t][n] = w[t][0] g[t][0][n] + ... in slot order,
// each slot one fused multiply-add onto a sum that starts at zero -- the
// order and rounding of the single-launch combine kernel.  A thread owns
// four consecutive rows of one token and loads four slots' rows at a time.
// VEC: N % 4 == 0 and y, g 16-byte aligned (float4 loads and stores).
template <bool VEC>
__device__ __forceinline__ float4 slot_rows(const float *p, int n0, int N)
{
    if (VEC) return *(const float4 *)p;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (n0 < N) v.x = p[0];
    if (n0 + 1 < N) v.y = p[1];
    if (n0 + 2 < N) v.z = p[2];
    if (n0 + 3 < N) v.w = p[3];
    return v;
}

template <bool VEC>
__global__ __launch_bounds__(256) void qmv_slot_sum_kernel(const float *__restrict__ g,
                                                           const float *__restrict__ route_w,
                                                           float *__restrict__ y, int M, int top_k, int N)
{
    const int nq = (N + 3) >> 2;
    const int q = blockIdx.x * 256 + threadIdx.x;    // M * N < 2^31
    if (q >= M * nq) return;
    const int t = q / nq;
    const int n0 = 4 * (q - t * nq);
    const float *gt = g + (size_t)t * top_k * N + n0;
    const float *wt = route_w + t * top_k;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto add = [&](float w, float4 v) {
        s.x = __builtin_fmaf(w, v.x, s.x);
        s.y = __builtin_fmaf(w, v.y, s.y);
        s.z = __builtin_fmaf(w, v.z, s.z);
        s.w = __builtin_fmaf(w, v.w, s.w);
    };
    int j = 0;
    for (; j + 4 <= top_k; j += 4) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = slot_rows<VEC>(gt + (size_t)(j + u) * N, n0, N);
#pragma unroll
        for (int u = 0; u < 4; ++u) add(wt[j + u], v[u]);
    }
    for (; j < top_k; ++j) add(wt[j], slot_rows<VEC>(gt + (size_t)j * N, n0, N));
    float *yt = y + (size_t)t * N + n0;
    if (VEC) {
        *(float4 *)yt = s;
    } else {
        if (n0 < N) yt[0] = s.x;
        if (n0 + 1 < N) yt[1] = s.y;
        if (n0 + 2 < N) yt[2] = s.z;
        if (n0 + 3 < N) yt[3] = s.w;
    }
}

// The combine of more than 4 tokens: the gather above (whatever kernel its
// shape takes) writes every (token, slot) row into g, zeros for ids outside
// [0, E), and the slot sum reads them back.  g holds M * top_k * N floats
// (4-byte aligned at least; float4 accesses only when it and y are 16-byte
// aligned); y is written only by the last launch.
qmv_status_t launch_combine_via(int wfmt, int afmt, const void *codes, const void *scales, int E,
                                const int32_t *ids, const float *route_w, int M, int top_k, const void *x,
                                const void *xs, int x_per_slot, float *g, float *y, int N, int K,
                                hipStream_t stream)
{
    const qmv_status_t st = launch(wfmt, afmt, codes, scales, nullptr, nullptr, E, ids, M, top_k, x, xs,
                                   x_per_slot, g, N, K, stream);
    if (st != QMV_OK)
        return st;
    const long long quads = (long long)M * ((N + 3) / 4);
    const unsigned blocks = (unsigned)((quads + 255) / 256);
    const bool vec = (N & 3) == 0 && (((uintptr_t)y | (uintptr_t)g) & 15) == 0;
    const void *fn = vec ? (const void *)&qmv_slot_sum_kernel<true> : (const void *)&qmv_slot_sum_kernel<false>;
    const float *gc = g;
    void *kargs[] = {&gc, &route_w, &y, &M, &top_k, &N};
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), kargs, 0, stream) == hipSuccess ? QMV_OK : QMV_EHIP;
}

// The per-slot rows of a many-token combine come from a memory pool of the
// library's, one per device, that keeps what it has handed out (release
// threshold: no limit): a call allocates and frees them in stream order
// (hipMallocFromPoolAsync / hipFreeAsync on the caller's stream), and calls
// after the first of their size reuse the pool's memory.
constexpr int kPoolDevices = 64;
std::once_flag g_pool_once[kPoolDevices];
hipMemPool_t g_pool[kPoolDevices];
hipError_t g_pool_err[kPoolDevices];

hipError_t combine_pool(int dev, hipMemPool_t &pool)
{
    std::call_once(g_pool_once[dev], [&] {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipError_t e = hipMemPoolCreate(&g_pool[dev], &props);
        if (e == hipSuccess) {
            uint64_t keep = ~0ull;
            e = hipMemPoolSetAttribute(g_pool[dev], hipMemPoolAttrReleaseThreshold, &keep);
        }
        g_pool_err[dev] = e;
    });
    pool = g_pool[dev];
    return g_pool_err[dev];
}

// The allocation-free combine's temporary: one array per GPU in the device
// code, held from the library's load until the process ends.  In host code
// `scratch` is only a host-side stand-in, never a device address: the
// address is looked up once per device (scratch_on) and only that is used.
static __device__ __align__(256) float scratch[QMV_NOALLOC_SCRATCH_BYTES / sizeof(float)];

std::once_flag g_scratch_once[kPoolDevices];
float *g_scratch_ptr[kPoolDevices];
hipError_t g_scratch_err[kPoolDevices];

// The device address of device dev's `scratch`, looked up at the first call
// on that device with the device made current for the lookup.
hipError_t scratch_on(int dev, float *&ptr)
{
    std::call_once(g_scratch_once[dev], [&] {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        const bool other = e == hipSuccess && cur != dev;
        if (other) e = hipSetDevice(dev);
        void *p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (other) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        g_scratch_ptr[dev] = (float *)p;
        g_scratch_err[dev] = e == hipSuccess && p == nullptr ? hipErrorInvalidSymbol : e;
    });
    ptr = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

// Down projection with the router-weighted combine: one launch, grid (row
// tiles, tokens); each lane carries row n of four of the token's slots.
qmv_status_t launch_combine(int wfmt, int afmt, const void *codes, const void *scales, int E,
                            const int32_t *ids, const float *route_w, int M, int top_k,
                            const void *x, const void *xs, int x_per_slot, float *y, int N, int K,
                            hipStream_t stream)
{
    if (M > kMaxM) {
        // Many tokens: gather into pool memory, then the slot sum (the
        // one-launch kernel below re-reads each expert's weights per token).
        hipDevice_t dev = 0;                         // the stream's device
        hipMemPool_t pool;
        if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kPoolDevices ||
            combine_pool(dev, pool) != hipSuccess)
            return QMV_EHIP;
        void *g = nullptr;
        if (hipMallocFromPoolAsync(&g, (size_t)M * top_k * N * sizeof(float), pool, stream) != hipSuccess)
            return QMV_EHIP;
        const qmv_status_t st = launch_combine_via(wfmt, afmt, codes, scales, E, ids, route_w, M, top_k, x, xs,
                                                   x_per_slot, (float *)g, y, N, K, stream);
        const hipError_t fe = hipFreeAsync(g, stream);
        if (st != QMV_OK)
            return st;
        return fe == hipSuccess ? QMV_OK : QMV_EHIP;
    }
    const int kind = kind_of(wfmt, afmt, K);
    Args a = base_args(wfmt, afmt, kind, codes, scales, E, ids, M, top_k, x, xs, x_per_slot, y, N, K);
    a.route_w = route_w;
    a.x_early = 1;
    Shape sh;
    int wi = 1;
    constexpr int RT = 4;
    const bool q8 = afmt == QMV_A_BF16_Q8;
    if (!tuned_shape(kind, 3, false, q8, K, N, M * top_k, wi, sh))
        sh = pick_shape(3, a.units, (long long)N * M * RT, RT);
    const int waves = kWaveMenu[wi];
    a.rows_per_tile = waves * (64 / sh.lpr);
    const int nv = x_per_slot ? (top_k < 4 ? top_k : 4) : 1;
    const size_t lds = (size_t)nv * a.lds_vec_bytes;

    const void *fn = combine_kernel_for(wi, kind, sh.li, sh.ci, q8);
    std::call_once(g_cattr_once[q8][wi][kind][sh.li][sh.ci], [&] {
        const int umax = kMaxK / kUnitWeights[kind];
        const int vmax = (umax * (kUnitXB[kind] + kUnitAB[kind]) + 15) & ~15;
        g_cattr_err[q8][wi][kind][sh.li][sh.ci] = hipFuncSetAttribute(
            fn, hipFuncAttributeMaxDynamicSharedMemorySize, 4 * vmax);
    });
    if (g_cattr_err[q8][wi][kind][sh.li][sh.ci] != hipSuccess)
        return QMV_EHIP;
    const dim3 grid((unsigned)((N + a.rows_per_tile - 1) / a.rows_per_tile), (unsigned)M);
    void *kargs[] = {&a};
    if (hipLaunchKernel(fn, grid, dim3(64 * waves), kargs, lds, stream) != hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

}  // namespace

extern "C" {

#define QMV_API __attribute__((visibility("default")))

QMV_API qmv_status_t qmv_dense(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales,
                       qmv_afmt_t afmt, const void *x, const void *x_scales,
                       float *y, int M, int N, int K, hipStream_t stream)
{
    const qmv_status_t s = check_dense(wfmt, w_codes, w_scales, afmt, x, x_scales, y, M, N, K);
    if (s != QMV_OK)
        return s;
    return launch(wfmt, afmt, w_codes, w_scales, nullptr, nullptr, 1, nullptr, M, 1, x,
                  afmt == QMV_A_Q8B32 ? x_scales : nullptr, 0, y, N, K, stream);
}

QMV_API qmv_status_t qmv_gather_moe(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales, int E,
                            const int32_t *expert_ids, int M, int top_k,
                            qmv_afmt_t afmt, const void *x, const void *x_scales,
                            int x_per_slot, float *y, int N, int K, hipStream_t stream)
{
    const qmv_status_t s = check_gather(wfmt, w_codes, w_scales, E, expert_ids, M, top_k, afmt, x, x_scales,
                                        y, N, K);
    if (s != QMV_OK)
        return s;
    return launch(wfmt, afmt, w_codes, w_scales, nullptr, nullptr, E, expert_ids, M, top_k, x,
                  afmt == QMV_A_Q8B32 ? x_scales : nullptr, x_per_slot ? 1 : 0, y, N, K, stream);
}

QMV_API qmv_status_t qmv_gather_moe_swiglu(qmv_wfmt_t wfmt, const void *gate_codes, const void *gate_scales,
                                   const void *up_codes, const void *up_scales, int E,
                                   const int32_t *expert_ids, int M, int top_k,
                                   qmv_afmt_t afmt, const void *x, const void *x_scales,
                                   float *y, int N, int K, hipStream_t stream)
{
    const void *xs = used_xs(afmt, x_scales);
    const qmv_status_t s = check_swiglu(wfmt, gate_codes, gate_scales, up_codes, up_scales, E, expert_ids, M,
                                        top_k, afmt, x, x_scales, y, N, K);
    if (s != QMV_OK)
        return s;
    return launch(wfmt, afmt, gate_codes, gate_scales, up_codes, up_scales, E, expert_ids, M, top_k, x,
                  xs, 0, y, N, K, stream);
}

QMV_API qmv_status_t qmv_gather_moe_combine(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales,
                                    int E, const int32_t *expert_ids, const float *route_weights,
                                    int M, int top_k, qmv_afmt_t afmt, const void *x,
                                    const void *x_scales, int x_per_slot, float *y, int N, int K,
                                    hipStream_t stream)
{
    const void *xs = used_xs(afmt, x_scales);
    const qmv_status_t s = check_combine(wfmt, w_codes, w_scales, E, expert_ids, route_weights, M, top_k, afmt,
                                         x, x_scales, y, N, K);
    if (s != QMV_OK)
        return s;
    return launch_combine(wfmt, afmt, w_codes, w_scales, E, expert_ids, route_weights, M, top_k, x, xs,
                          x_per_slot ? 1 : 0, y, N, K, stream);
}

QMV_API qmv_status_t qmv_gather_moe_combine_noalloc(qmv_wfmt_t wfmt, const void *w_codes, const void *w_scales,
                                            int E, const int32_t *expert_ids, const float *route_weights,
                                            int M, int top_k, qmv_afmt_t afmt, const void *x,
                                            const void *x_scales, int x_per_slot, float *y, int N, int K,
                                            hipStream_t stream)
{
    const void *xs = used_xs(afmt, x_scales);
    const qmv_status_t s = check_combine(wfmt, w_codes, w_scales, E, expert_ids, route_weights, M, top_k, afmt,
                                         x, x_scales, y, N, K);
    if (s != QMV_OK)
        return s;
    if (M <= kMaxM)                                  // the one-launch kernel: no temporary
        return launch_combine(wfmt, afmt, w_codes, w_scales, E, expert_ids, route_weights, M, top_k, x, xs,
                              x_per_slot ? 1 : 0, y, N, K, stream);
    if ((size_t)M * top_k * N * sizeof(float) > QMV_NOALLOC_SCRATCH_BYTES)
        return QMV_ESCRATCH;
    hipDevice_t dev = 0;                             // the stream's device
    float *g = nullptr;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kPoolDevices ||
        scratch_on(dev, g) != hipSuccess)
        return QMV_EHIP;
    return launch_combine_via(wfmt, afmt, w_codes, w_scales, E, expert_ids, route_weights, M, top_k, x, xs,
                              x_per_slot ? 1 : 0, g, y, N, K, stream);
}

QMV_API const char *qmv_strerror(qmv_status_t status)
{
    return status_text(status);
}

}  // extern "C"
