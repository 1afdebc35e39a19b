// qmv_host.hpp -- host-side logic of libqmv.so that needs no GPU: argument
// checks of every entry point (include/qmv.h), the launch-shape choice and
// the format constants the kernels share with it.
//
// Plain C++17: nothing here calls HIP or dereferences a caller's pointer, so
// the same code is also built with the host compiler under AddressSanitizer
// and UndefinedBehaviorSanitizer (qmv_host_check.cpp) and driven over the
// argument cases of the host tests.
#pragma once

#include <stdint.h>

#include "qmv.h"

namespace qmv_cfg {

// kMXFP4I: MXFP4 codes with int8 activations (fp16 scale per 32), staged as
// exact bf16 so that the MXFP4 decode and bf16 dot serve both.
enum Kind : int { kMXFP4 = 0, kCB2 = 1, kCB2S = 2, kCB3 = 3, kMXFP4I = 4 };

// Units per format (one unit = what a decode-kernel lane takes per load):
// W weights; XB LDS bytes of activations per unit and vector; AB LDS bytes of
// per-unit activation side data (scales, sums).
template <int F> struct Fmt;
template <> struct Fmt<kMXFP4> { static constexpr int W = 32, XB = 64, AB = 0; };
template <> struct Fmt<kCB2>   { static constexpr int W = 64, XB = 64, AB = 16; };
template <> struct Fmt<kCB2S>  { static constexpr int W = 32, XB = 32, AB = 8; };
template <> struct Fmt<kCB3>   { static constexpr int W = 32, XB = 32, AB = 4; };
template <> struct Fmt<kMXFP4I> { static constexpr int W = 32, XB = 64, AB = 4; };

// Decode-kernel menus.  Variant 0: one vector per item, 2 rows per lane.
// Variant 1: up to four vectors per item (gather with M > 1 or per-slot
// activations), 2 rows per lane.  Variant 2: dense with M > 1, 4 rows per
// lane.  Variant 3: the combine kernel.
constexpr int kMenuLpr[4] = {8, 16, 32, 64};
constexpr int kMenuCpl01[5] = {1, 2, 3, 4, 7};
constexpr int kMenuCpl2[3] = {1, 2, 4};
constexpr int kMenuCplC[4] = {1, 2, 3, 4};

// Pair lists of the grouped and batched kernels (more than 4 tokens): room
// for this many (round, wave) counts plus a total in LDS, ahead of the list.
constexpr int kPairCounts = 256;
constexpr int kPairCountBytes = 4 * (kPairCounts + 4);
// The grouped kernel's bitmap of the experts a call selects (E <= 1024), the
// word that hands one of them to every wave, the count of them, and two words
// that hand a workgroup's run of items to every wave.
constexpr int kExpertBitmapBytes = 4 * 36;
// The int8 matrix-core kernel's count of pairs per expert (E <= 1024), from
// which each workgroup finds its share of the call's weighted work.
constexpr int kExpertCountBytes = 4 * 1024;

}  // namespace qmv_cfg

namespace qmv_host {

using namespace qmv_cfg;

constexpr int kWaveMenu[2] = {4, 8};     // wave64s per workgroup: qmv, qmv_w8

constexpr int kMaxK = 16384;
constexpr int kMaxM = 4;
constexpr int kMaxTopK = 16;
// More than 4 tokens (the batched and grouped kernels): every workgroup lists
// its expert's (token, slot) pairs in LDS as 16-bit indices, scanning the ids
// in at most 32 rounds of 256 threads; the grid covers every expert.
constexpr int kMaxPairsBatched = 8192;
// Dense MXFP4 x bf16 calls with 5..20 vectors run as groups of 4 on the
// decode kernels (one expert gives the batched kernel too few tiles).
constexpr int kDenseGroupsMaxM = 8;
constexpr int kSplitMaxM = 64;           // few-pairs gathers split into token groups up to this M
constexpr int kMaxEBatched = 1023;

constexpr int kUnitWeights[5] = {Fmt<kMXFP4>::W, Fmt<kCB2>::W, Fmt<kCB2S>::W, Fmt<kCB3>::W, Fmt<kMXFP4I>::W};
constexpr int kUnitXB[5] = {Fmt<kMXFP4>::XB, Fmt<kCB2>::XB, Fmt<kCB2S>::XB, Fmt<kCB3>::XB, Fmt<kMXFP4I>::XB};
constexpr int kUnitAB[5] = {Fmt<kMXFP4>::AB, Fmt<kCB2>::AB, Fmt<kCB2S>::AB, Fmt<kCB3>::AB, Fmt<kMXFP4I>::AB};

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline long long row_code_bytes(int wfmt, long long K)
{
    return wfmt == QMV_W_MXFP4 ? K / 2 : wfmt == QMV_W_CB2 ? K / 4 : 3 * K / 8;
}
inline long long row_scale_bytes(int wfmt, long long K)
{
    return wfmt == QMV_W_MXFP4 ? K / 32 : wfmt == QMV_W_CB2 ? K / 16 : K / 8;
}

inline int kind_of(int wfmt, int afmt, int K)
{
    if (wfmt == QMV_W_MXFP4)
        return afmt == QMV_A_Q8B32 ? kMXFP4I : kMXFP4;
    return wfmt == QMV_W_CB3 ? kCB3 : (K % 64 == 0 ? kCB2 : kCB2S);
}

// Argument checks shared by the entry points (no HIP call, no pointer
// dereference).  batched_ok: the entry point takes M > 4.
inline qmv_status_t validate(int wfmt, const void *codes, const void *scales, long long E,
                             const int32_t *ids, bool gather, int M, int top_k, int afmt,
                             const void *x, const void *xs, const float *y, int N, int K,
                             bool batched_ok = false)
{
    if (!codes || !scales || !x || !y || (gather && !ids))
        return QMV_EINVAL;
    if (afmt == QMV_A_Q8B32 && !xs)
        return QMV_EINVAL;
    if (M <= 0 || N <= 0 || K <= 0 || E <= 0 || top_k <= 0)
        return QMV_EINVAL;
    if (wfmt < QMV_W_MXFP4 || wfmt > QMV_W_CB3 || afmt < QMV_A_BF16 || afmt > QMV_A_BF16_Q8)
        return QMV_EUNSUPPORTED;
    // pairs: (MXFP4, BF16), (MXFP4, Q8B32), (CB2 or CB3, Q8B32), (CB2 or CB3, BF16_Q8)
    if ((wfmt == QMV_W_MXFP4) ? afmt == QMV_A_BF16_Q8 : afmt == QMV_A_BF16)
        return QMV_EUNSUPPORTED;
    if (top_k > kMaxTopK || K % 32 != 0 || K > kMaxK)
        return QMV_EUNSUPPORTED;
    if (M > kMaxM) {
        // more than 4 vectors: at most 8192 (token, slot) pairs and 1023 experts
        if (!batched_ok || (long long)M * (gather ? top_k : 1) > kMaxPairsBatched ||
            (gather && E > kMaxEBatched))
            return QMV_EUNSUPPORTED;
    }
    const uintptr_t calign = (wfmt == QMV_W_CB2 && K % 64 != 0) ? 8 : (wfmt == QMV_W_CB3 ? 4 : 16);
    if (!aligned(codes, calign) || !aligned(x, 16) || !aligned(y, 4) ||
        (wfmt != QMV_W_MXFP4 && !aligned(scales, 4)) || (xs && !aligned(xs, 4)) ||
        (ids && !aligned(ids, 4)))
        return QMV_EINVAL;
    // in-expert row offsets and output indices are 32-bit on the device
    const long long per_expert = (long long)N * row_code_bytes(wfmt, K);
    if (N >= (1 << 24) || per_expert >= (1LL << 31) || (long long)M * top_k * N >= (1LL << 31))
        return QMV_EUNSUPPORTED;
    if (E > (1LL << 62) / per_expert)
        return QMV_EUNSUPPORTED;
    return QMV_OK;
}

// The checks of each entry point, in the order the entry point makes them.
// x_scales is used only with QMV_A_Q8B32.
inline const void *used_xs(int afmt, const void *x_scales)
{
    return afmt == QMV_A_Q8B32 ? x_scales : nullptr;
}

inline qmv_status_t check_dense(int wfmt, const void *codes, const void *scales, int afmt, const void *x,
                                const void *x_scales, const float *y, int M, int N, int K)
{
    return validate(wfmt, codes, scales, 1, nullptr, false, M, 1, afmt, x, used_xs(afmt, x_scales), y, N, K,
                    true);
}

inline qmv_status_t check_gather(int wfmt, const void *codes, const void *scales, int E, const int32_t *ids,
                                 int M, int top_k, int afmt, const void *x, const void *x_scales,
                                 const float *y, int N, int K)
{
    return validate(wfmt, codes, scales, E, ids, true, M, top_k, afmt, x, used_xs(afmt, x_scales), y, N, K,
                    true);
}

inline qmv_status_t check_swiglu(int wfmt, const void *gate_codes, const void *gate_scales,
                                 const void *up_codes, const void *up_scales, int E, const int32_t *ids,
                                 int M, int top_k, int afmt, const void *x, const void *x_scales,
                                 const float *y, int N, int K)
{
    const void *xs = used_xs(afmt, x_scales);
    const qmv_status_t s = validate(wfmt, gate_codes, gate_scales, E, ids, true, M, top_k, afmt, x, xs, y, N, K,
                                    true);
    if (s != QMV_OK)
        return s;
    return validate(wfmt, up_codes, up_scales, E, ids, true, M, top_k, afmt, x, xs, y, N, K, true);
}

inline qmv_status_t check_combine(int wfmt, const void *codes, const void *scales, int E, const int32_t *ids,
                                  const float *route_weights, int M, int top_k, int afmt, const void *x,
                                  const void *x_scales, const float *y, int N, int K)
{
    const qmv_status_t s = validate(wfmt, codes, scales, E, ids, true, M, top_k, afmt, x,
                                    used_xs(afmt, x_scales), y, N, K, true);
    if (s != QMV_OK)
        return s;
    if (!route_weights || !aligned(route_weights, 4))
        return QMV_EINVAL;
    return QMV_OK;
}

// Launch shape: lanes per row (LPR) and units per lane step (CPL) from the
// variant's menu.  Measured on MI355X over the C2..C5 shapes: the kernel is
// fastest with 8 to 14 waves per CU in total (enough to cover memory latency,
// few enough that per-wave set-up stays small), with few lane slots wasted on
// the row's padding, and with as many units in flight per lane as possible.
// So: keep shapes within 85% of the best lane efficiency, prefer total waves
// in [8, 14] x 256 (else the nearest), then the larger CPL, then more waves.
struct Shape { int li, ci, lpr, cpl; };

inline const int *cpl_menu(int variant, int &n)
{
    n = variant == 3 ? 4 : variant == 2 ? 3 : 5;
    return variant == 3 ? kMenuCplC : variant == 2 ? kMenuCpl2 : kMenuCpl01;
}

inline Shape pick_shape(int variant, int units, long long rows_total, int rt)
{
    int ncpl = 0;
    const int *cmenu = cpl_menu(variant, ncpl);
    const bool no_lpr8 = variant == 2;
    double best_eff = 0.0;
    for (int li = 0; li < 4; ++li)
        for (int ci = 0; ci < ncpl; ++ci) {
            const int lpr = kMenuLpr[li];
            if (no_lpr8 && lpr == 8) continue;
            const long long seg = (long long)lpr * cmenu[ci];
            const double eff = (double)units / (double)(((units + seg - 1) / seg) * seg);
            if (eff > best_eff) best_eff = eff;
        }
    const long long lo = 8LL * 256, hi = 14LL * 256;
    Shape best = {0, 0, 0, 0};
    long long best_key[3] = {-1, -1, -1};
    for (int li = 0; li < 4; ++li)
        for (int ci = 0; ci < ncpl; ++ci) {
            const int lpr = kMenuLpr[li];
            if (no_lpr8 && lpr == 8) continue;
            const int cpl = cmenu[ci];
            const long long seg = (long long)lpr * cpl;
            const double eff = (double)units / (double)(((units + seg - 1) / seg) * seg);
            if (eff < 0.85 * best_eff) continue;
            const long long rows_per_wave = (64 / lpr) * rt;
            const long long waves = (rows_total + rows_per_wave - 1) / rows_per_wave;
            const long long miss = waves < lo ? lo - waves : waves > hi ? waves - hi : 0;
            const long long key[3] = {-miss, cpl, waves};      // larger is better
            bool better = best_key[0] == -1 && best_key[1] == -1;
            for (int k = 0; k < 3 && !better; ++k) {
                if (key[k] > best_key[k]) { better = true; break; }
                if (key[k] < best_key[k]) break;
            }
            if (better) {
                best = {li, ci, lpr, cpl};
                for (int k = 0; k < 3; ++k) best_key[k] = key[k];
            }
        }
    return best;
}

// Grouped kernel (more than 4 tokens on the decode kernels' MACs): the
// launch shape and the number of workgroups.  Work items are (expert slot,
// row tile) for `busy` slots; G workgroups take equal contiguous runs of
// them.  With up to 4 rounds of work G is one round of the chip and the
// slowest workgroup streams ceil(items / G) row tiles; with more, G = items.  Each row tile costs its
// weight rows plus a fixed start-up (the first loads' latency, about the
// time to stream 24 KB at one workgroup's share of the bandwidth).  Among the
// shapes with little padding of K, take the cheapest slowest workgroup, then
// the most units in flight.  row_bytes: code and scale bytes of one weight
// row; occ(li, ci): workgroups per CU the shape's kernel can hold by its
// registers; lds: bytes of LDS per workgroup.
struct GroupedPlan {
    Shape sh;
    int rows_per_tile;   // output rows per row tile
    int tiles;           // row tiles per expert
    int items;           // busy * tiles
    int grid;            // workgroups
};

constexpr int kLdsPerCU = 160 * 1024;

template <class Occ>
inline GroupedPlan plan_grouped(int units, long long row_bytes, int N, int busy, bool gate_up, int cus,
                                long long lds, Occ occ)
{
    const int *cmenu = kMenuCpl01;
    const int ncpl = 5;
    double best_eff = 0.0;
    for (int li = 0; li < 4; ++li)
        for (int ci = 0; ci < ncpl; ++ci) {
            const long long seg = (long long)kMenuLpr[li] * cmenu[ci];
            const double eff = (double)units / (double)(((units + seg - 1) / seg) * seg);
            if (eff > best_eff) best_eff = eff;
        }
    const double startup_rows = 2.0 + 24576.0 / (double)(row_bytes > 0 ? row_bytes : 1);
    const long long by_lds = lds > 0 ? kLdsPerCU / lds : 1;
    GroupedPlan best = {{0, 0, kMenuLpr[0], cmenu[0]}, 0, 0, 0, 0};
    double best_cost = -1.0;
    for (int li = 0; li < 4; ++li)
        for (int ci = 0; ci < ncpl; ++ci) {
            const int lpr = kMenuLpr[li], cpl = cmenu[ci];
            const long long seg = (long long)lpr * cpl;
            const double eff = (double)units / (double)(((units + seg - 1) / seg) * seg);
            if (eff < 0.85 * best_eff) continue;
            const int rpt = 4 * (64 / lpr) * (gate_up ? 1 : 2);
            const int wrows = 4 * (64 / lpr) * 2;
            const int tiles = (N + rpt - 1) / rpt;
            const long long items = (long long)busy * tiles;
            long long per_cu = occ(li, ci);
            if (per_cu > by_lds) per_cu = by_lds;
            if (per_cu < 1) per_cu = 1;
            const long long slots = per_cu * cus;
            // up to 4 rounds of the chip: one round of workgroups, each a run
            // of row tiles (balanced runs beat a partial last round); more:
            // one row tile per workgroup (a workgroup that starts as another
            // retires overlaps its first loads with the other's last ones,
            // which a run of tiles in one workgroup does not)
            const long long grid = items > 4 * slots ? items : items < slots ? items : slots;
            const long long run = (items + grid - 1) / grid;
            const long long rounds = (grid + slots - 1) / slots;
            const double cost = (double)(run * rounds) * ((double)wrows / eff + startup_rows);
            if (best_cost < 0.0 || cost < best_cost * 0.999 ||
                (cost <= best_cost * 1.001 && cpl > best.sh.cpl)) {
                best_cost = cost;
                best = {{li, ci, lpr, cpl}, rpt, tiles, (int)items, (int)grid};
            }
        }
    return best;
}

// Launch shapes measured best on MI355X for the MoE expert shapes this library
// is tuned on (sweeps of every menu shape at 4 and 8 waves per workgroup, HBM-
// resident weights rotated past the Infinity Cache).  Other shapes use
// pick_shape() with 4 waves (8 for the combine kernel and for bf16
// activations quantized in staging, whose tuned shapes all prefer it: each
// workgroup quantizes the whole activation vector, so fewer, larger
// workgroups repeat that less).  An entry matches on format kind, variant (3: combine),
// gate/up mode, K, N and the number of (token, slot) pairs.
struct Tuned { int kind, variant, gate_up, K, N, pairs, waves, lpr, cpl, q8; };
constexpr Tuned kTuned[] = {
    {kMXFP4, 0, 0, 2880, 2880, 4, 4, 32, 3, 0},     // gpt-oss-20b expert projection
    {kMXFP4, 0, 1, 2880, 2880, 4, 4, 32, 3, 0},     // gpt-oss-20b gate+up, SwiGLU
    {kCB2,   0, 0, 7168, 2048, 4, 4, 64, 2, 0},     // DeepSeek-shaped 2-bit gate/up
    {kCB2,   0, 1, 7168, 2048, 4, 4, 16, 7, 0},     // ... fused gate+up, SwiGLU
    {kCB3,   1, 0, 2048, 7168, 4, 8, 16, 2, 0},     // DeepSeek-shaped 3-bit down
    {kMXFP4, 1, 0, 7168, 2048, 16, 4, 8, 7, 0},     // 4 tokens x top-4 of 256
    {kMXFP4, 2, 0, 7168, 7168, 1, 8, 64, 4, 0},     // dense, 4 tokens
    {kCB3,   3, 0, 2048, 7168, 4, 8, 32, 1, 0},     // 3-bit down + router-weighted combine
    {kMXFP4, 3, 0, 2880, 2880, 4, 8, 32, 3, 0},     // gpt-oss down + router-weighted combine
    {kMXFP4I, 0, 0, 2880, 2880, 4, 4, 32, 3, 0},    // gpt-oss expert projection, int8 x
    // bf16 activations quantized in staging: larger workgroups quantize the
    // activation vector fewer times over (C3 7.10 -> 6.48 us, C4 10.04 -> 9.17 us)
    {kCB2,   0, 0, 7168, 2048, 4, 8, 32, 4, 1},     // 2-bit gate/up, bf16 x
    {kCB3,   1, 0, 2048, 7168, 4, 8, 16, 4, 1},     // 3-bit down, per-slot bf16 x
};

inline bool tuned_shape(int kind, int variant, bool gate_up, bool q8, int K, int N, int pairs, int &wi,
                        Shape &sh)
{
    for (const Tuned &t : kTuned) {
        if (t.kind != kind || t.variant != variant || t.gate_up != (gate_up ? 1 : 0) || t.K != K ||
            t.N != N || t.pairs != pairs || t.q8 != (q8 ? 1 : 0))
            continue;
        wi = t.waves == 8 ? 1 : 0;
        int ncpl = 0;
        const int *cmenu = cpl_menu(variant, ncpl);
        for (int li = 0; li < 4; ++li)
            for (int ci = 0; ci < ncpl; ++ci)
                if (kMenuLpr[li] == t.lpr && cmenu[ci] == t.cpl) {
                    sh = {li, ci, t.lpr, t.cpl};
                    return true;
                }
    }
    return false;
}

// Dense MXFP4 x bf16, 2 <= M <= 4: one wave per quad of rows, 16 units of a
// row per load instruction, the 4x4x4 bf16 MFMA for the multiplies, 4 unit
// steps in flight.  Measured on the 4-vector 7168 x 7168 call (MI355X,
// weights rotated past the Infinity Cache): 8-wave workgroups 8.6 us, 4-wave
// 10.7 us -- every workgroup stages all of x, so fewer, larger workgroups
// stage it fewer times -- and 7 steps in flight or K split over two waves
// per quad were slower still.  Calls with fewer than 1024 row quads (128
// 8-wave workgroups) use 4-wave workgroups so that more CUs get work.
inline int dense4_waves(int N)
{
    return (N + 3) / 4 >= 1024 ? 8 : 4;
}

// LDS of one dense 4-vector workgroup: activations (K/32 + 1 units of 256 B),
// then the scale rows of its row quads (+ up to 15 bytes of alignment, in
// 16-byte chunks).
inline unsigned long dense4_lds(int K, int waves)
{
    const unsigned long rsb = (unsigned long)K / 32;
    return 256 * (rsb + 1) + 16 * ((waves * 4 * rsb + 30) / 16);
}

// Static English text for a status code (never null).
inline const char *status_text(int status)
{
    switch (status) {
    case QMV_OK: return "success";
    case QMV_EINVAL: return "invalid argument (null or misaligned pointer, or a size <= 0)";
    case QMV_EUNSUPPORTED: return "unsupported shape or format (more than 4 tokens: at most 8192 "
                                  "(token, slot) pairs and E <= 1023; top_k in [1,16], "
                                  "K % 32 == 0 and K <= 16384; "
                                  "pairs MXFP4+BF16, MXFP4+Q8B32, CB2/CB3+Q8B32, CB2/CB3+BF16_Q8)";
    case QMV_EHIP: return "the HIP runtime rejected the kernel launch";
    case QMV_ESCRATCH: return "the call needs more temporary memory than the allocation-free entry point's "
                              "fixed 64 MiB per GPU (M * top_k * N * 4 bytes with more than 4 tokens)";
    }
    return "unknown status";
}

}  // namespace qmv_host
