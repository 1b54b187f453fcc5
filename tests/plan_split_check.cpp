// Host check of the windowed kernel's work split (window_split in plan.cpp),
// built with the host compiler by tests/test_plan_host.py.  For many sizes it
// checks the invariants the kernel relies on and, on small sizes, that the
// largest range cost equals the optimum of a brute-force search over every
// contiguous split.  Prints "ok <cases>" or the first failure.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "plan.h"

namespace {

int64_t cost(int64_t u0, int64_t u1, int64_t nch, int64_t seg_x4)
{
    if (u1 <= u0)
        return 0;
    const int64_t touched = (u1 - 1) / nch - u0 / nch + 1;
    return 4 * (u1 - u0) + seg_x4 * touched;
}

// Smallest possible largest cost of `per` contiguous ranges over [0, U).
int64_t best_split(int64_t U, int64_t nch, int64_t per, int64_t seg_x4)
{
    const int64_t INF = INT64_MAX / 4;
    std::vector<int64_t> f(size_t(U + 1), INF), g(size_t(U + 1), INF);
    f[0] = 0;
    for (int64_t k = 0; k < per; ++k) {
        std::fill(g.begin(), g.end(), INF);
        for (int64_t e = 0; e <= U; ++e)
            for (int64_t s = 0; s <= e; ++s)
                if (f[size_t(s)] < INF)
                    g[size_t(e)] = std::min(g[size_t(e)],
                                            std::max(f[size_t(s)], cost(s, e, nch, seg_x4)));
        f.swap(g);
    }
    return f[size_t(U)];
}

int check(int64_t tiles, int64_t nch, int64_t ncta, int64_t seg_x4, bool brute)
{
    uint32_t b[mdcn::kWindowSlots + 1];
    if (!mdcn::window_split(tiles, nch, ncta, seg_x4, b)) {
        std::printf("split refused: tiles %lld nch %lld ncta %lld\n", (long long)tiles,
                    (long long)nch, (long long)ncta);
        return 1;
    }
    const int64_t ngrp = (ncta % 8 == 0 && tiles >= ncta) ? 8 : 1;
    const int64_t per = ncta / ngrp;
    if (b[0] != 0 || int64_t(b[ncta]) != tiles * nch) {
        std::printf("ends: tiles %lld nch %lld ncta %lld\n", (long long)tiles, (long long)nch,
                    (long long)ncta);
        return 1;
    }
    for (int64_t grp = 0; grp < ngrp; ++grp) {
        const int64_t tg0 = grp * tiles / ngrp, tg1 = (grp + 1) * tiles / ngrp;
        // a run starts on a tile boundary (its first workgroup never waits)
        if (int64_t(b[grp * per]) != tg0 * nch) {
            std::printf("run start: grp %lld\n", (long long)grp);
            return 1;
        }
        bool empty_seen = false;
        int64_t worst = 0;
        for (int64_t k = 0; k < per; ++k) {
            const int64_t j = grp * per + k;
            if (b[j + 1] < b[j]) {
                std::printf("not monotone at %lld\n", (long long)j);
                return 1;
            }
            const bool empty = b[j + 1] == b[j];
            // a range after an empty one would wait on a workgroup that
            // publishes nothing
            if (!empty && empty_seen) {
                std::printf("range after an empty one: tiles %lld nch %lld ncta %lld j %lld\n",
                            (long long)tiles, (long long)nch, (long long)ncta, (long long)j);
                return 1;
            }
            empty_seen = empty_seen || empty;
            worst = std::max(worst, cost(b[j], b[j + 1], nch, seg_x4));
        }
        if (int64_t(b[grp * per + per]) != tg1 * nch) {
            std::printf("run end: grp %lld\n", (long long)grp);
            return 1;
        }
        if (brute) {
            const int64_t opt = best_split((tg1 - tg0) * nch, nch, per, seg_x4);
            if (worst != opt) {
                std::printf("not optimal: tiles %lld nch %lld ncta %lld seg %lld: %lld vs %lld\n",
                            (long long)tiles, (long long)nch, (long long)ncta,
                            (long long)seg_x4, (long long)worst, (long long)opt);
                return 1;
            }
        }
    }
    return 0;
}

}  // namespace

int main()
{
    int cases = 0;
    // small sizes against the brute-force optimum
    for (int64_t tiles = 1; tiles <= 12; ++tiles)
        for (int64_t nch : {1, 2, 3, 5})
            for (int64_t ncta = 1; ncta <= std::min<int64_t>(tiles, 9); ++ncta)
                for (int64_t seg : {0, 4, 12, 40}) {
                    if (check(tiles, nch, ncta, seg, true))
                        return 1;
                    ++cases;
                }
    // the benchmark shapes and ragged large ones: invariants only
    const int64_t big[][3] = {{400, 16, 256}, {224, 32, 224}, {400, 16, 200}, {36, 2, 36},
                              {1000, 16, 256}, {257, 7, 256}, {9, 64, 8}, {100000, 3, 256}};
    for (const auto &t : big)
        for (int64_t seg : {0, 12, 100}) {
            if (check(t[0], t[1], t[2], seg, false))
                return 1;
            ++cases;
        }
    std::printf("ok %d\n", cases);
    return 0;
}
