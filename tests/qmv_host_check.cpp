// qmv_host_check.cpp -- drives the library's host-side logic (qmv_host.hpp:
// the argument checks of every entry point, the launch-shape choice and the
// status texts) from a CPU-only build, so that it can run under
// AddressSanitizer and UndefinedBehaviorSanitizer.  No GPU and no HIP runtime
// call: the checks never dereference the pointers they are given, so fake
// addresses stand in for device memory.
//
// Reads one command per line on stdin and prints one result line each:
//   dense   wfmt codes scales afmt x xs y M N K                   -> status
//   gather  wfmt codes scales E ids M top_k afmt x xs per_slot y N K -> status
//   swiglu  wfmt gc gs uc us E ids M top_k afmt x xs y N K        -> status
//   combine wfmt codes scales E ids rw M top_k afmt x xs per_slot y N K -> status
//   strerror s                                                   -> text
//   shapes                                                       -> checksum of every pick_shape /
//                                                                   tuned_shape / plan_grouped result
//                                                                   over a grid
// Pointers are decimal addresses (0 = null).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "qmv_host.hpp"

using namespace qmv_host;

namespace {

const void *P(long long v) { return (const void *)(uintptr_t)v; }

unsigned long long shapes_checksum()
{
    unsigned long long h = 0;
    const int units[] = {1, 2, 3, 7, 8, 9, 45, 56, 64, 90, 112, 128, 224, 256, 512};
    const long long rows[] = {1, 16, 255, 1024, 2880, 8192, 11520, 28672, 65536, 1LL << 24};
    for (int variant = 0; variant < 4; ++variant)
        for (int u : units)
            for (long long r : rows)
                for (int rt : {1, 2, 4}) {
                    const Shape s = pick_shape(variant, u, r, rt);
                    if (s.li < 0 || s.li > 3 || s.lpr != kMenuLpr[s.li]) {
                        printf("bad shape\n");
                        exit(3);
                    }
                    h = h * 1000003 + (s.li * 7 + s.ci) * 131 + s.lpr + s.cpl;
                }
    for (const Tuned &t : kTuned) {
        int wi = -1;
        Shape s = {0, 0, 0, 0};
        if (!tuned_shape(t.kind, t.variant, t.gate_up != 0, t.q8 != 0, t.K, t.N, t.pairs, wi, s) ||
            s.lpr != t.lpr || s.cpl != t.cpl || kWaveMenu[wi] != t.waves) {
            printf("tuned entry not found\n");
            exit(3);
        }
        h = h * 1000003 + wi * 31 + s.li * 7 + s.ci;
    }
    int wi = 0;
    Shape s = {0, 0, 0, 0};
    if (tuned_shape(kMXFP4, 0, false, false, 4096, 4096, 4, wi, s)) {
        printf("untuned shape matched\n");
        exit(3);
    }
    // grouped-kernel plans: the grid never exceeds the items, the row tiles
    // cover N, and the tile matches the shape
    for (int u : {1, 7, 45, 90, 112, 224, 512})
        for (int N : {1, 33, 2048, 2880, 7168, 100000})
            for (int busy : {1, 4, 20, 256, 1023})
                for (bool gu : {false, true})
                    for (int occ : {1, 3})
                        for (long long lds : {0LL, 40000LL, 150000LL}) {
                            const GroupedPlan p = plan_grouped(u, 48LL * u, N, busy, gu, 256, lds,
                                                               [&](int, int) { return occ; });
                            const int rpt = 4 * (64 / p.sh.lpr) * (gu ? 1 : 2);
                            if (p.grid < 1 || p.grid > p.items || p.rows_per_tile != rpt ||
                                (long long)p.tiles * p.rows_per_tile < N ||
                                (long long)(p.tiles - 1) * p.rows_per_tile >= N ||
                                p.items != (long long)busy * p.tiles || p.sh.lpr != kMenuLpr[p.sh.li]) {
                                printf("bad grouped plan\n");
                                exit(3);
                            }
                            h = h * 1000003 + (unsigned long long)p.grid * 7 + p.sh.li * 5 + p.sh.ci;
                        }
    for (int N : {1, 4, 1023, 4096, 4097, 1 << 20})
        h = h * 1000003 + dense4_waves(N);
    for (int K : {32, 2880, 7168, kMaxK})
        h = h * 1000003 + dense4_lds(K, 4) + dense4_lds(K, 8);
    return h;
}

}  // namespace

int main()
{
    char line[4096];
    while (fgets(line, sizeof line, stdin)) {
        std::vector<std::string> tok;
        for (char *t = strtok(line, " \t\r\n"); t; t = strtok(nullptr, " \t\r\n"))
            tok.emplace_back(t);
        if (tok.empty())
            continue;
        std::vector<long long> v;
        for (size_t i = 1; i < tok.size(); ++i)
            v.push_back(strtoll(tok[i].c_str(), nullptr, 10));
        const std::string &cmd = tok[0];
        auto need = [&](size_t n) {
            if (v.size() != n) {
                printf("bad arity for %s\n", cmd.c_str());
                exit(2);
            }
        };
        if (cmd == "dense") {
            need(10);
            printf("%d\n", (int)check_dense((int)v[0], P(v[1]), P(v[2]), (int)v[3], P(v[4]), P(v[5]),
                                            (const float *)P(v[6]), (int)v[7], (int)v[8], (int)v[9]));
        } else if (cmd == "gather") {
            need(14);
            printf("%d\n", (int)check_gather((int)v[0], P(v[1]), P(v[2]), (int)v[3], (const int32_t *)P(v[4]),
                                             (int)v[5], (int)v[6], (int)v[7], P(v[8]), P(v[9]),
                                             (const float *)P(v[11]), (int)v[12], (int)v[13]));
        } else if (cmd == "swiglu") {
            need(15);
            printf("%d\n", (int)check_swiglu((int)v[0], P(v[1]), P(v[2]), P(v[3]), P(v[4]), (int)v[5],
                                             (const int32_t *)P(v[6]), (int)v[7], (int)v[8], (int)v[9],
                                             P(v[10]), P(v[11]), (const float *)P(v[12]), (int)v[13],
                                             (int)v[14]));
        } else if (cmd == "combine") {
            need(15);
            printf("%d\n", (int)check_combine((int)v[0], P(v[1]), P(v[2]), (int)v[3], (const int32_t *)P(v[4]),
                                              (const float *)P(v[5]), (int)v[6], (int)v[7], (int)v[8],
                                              P(v[9]), P(v[10]), (const float *)P(v[12]), (int)v[13],
                                              (int)v[14]));
        } else if (cmd == "strerror") {
            need(1);
            printf("%s\n", status_text((int)v[0]));
        } else if (cmd == "shapes") {
            need(0);
            printf("%llu\n", shapes_checksum());
        } else {
            printf("unknown command %s\n", cmd.c_str());
            return 2;
        }
        fflush(stdout);
    }
    return 0;
}
