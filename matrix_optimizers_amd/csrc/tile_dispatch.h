// Host-side dispatch of GEMM tiles to the eight XCDs, shared by the work
// lists of the Muon and Shampoo steps.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <vector>

#include "mo_worklist.h"

// One product of a grouped GEMM launch: tm x tn tiles of 256 x 256 (only the
// upper triangle when `upper`), each a K loop of klen elements; `idx` is the
// record index written into its items.
struct mo_gemm_job {
    uint32_t idx;
    uint32_t tm, tn;
    bool upper;
    uint64_t klen;
};

// Appends the dispatch list of one launch to `out`.  A workgroup's XCD is its
// block index mod 8 (the hardware deals consecutive workgroups round-robin
// over the 8 XCDs), and each XCD runs its share in block order on its 32 CUs.
// The tiles of one product are grouped into super-blocks of SB_R tile-rows x
// SB_C tile-columns (super-blocks row-major, tiles row-major inside), so one
// super-block is what an XCD runs at once and its tiles share 4 row panels
// and 8 column panels of the operands in that XCD's L2.  Super-blocks (jobs
// in the given order, normally descending work) go to the XCD with the least
// work so far (K-length x tiles; ties to the lowest XCD), split where that
// XCD would pass an even share of the total, and the list interleaves the 8
// queues: entry 8 j + x is the j-th tile of XCD x, or a pad entry (record
// index MO_WL_PAD) where that queue is shorter.
inline void mo_dispatch_tiles(const std::vector<mo_gemm_job>& jobs, std::vector<mo_wl_item>& out,
                              uint32_t max_split = 4) {
    constexpr uint32_t SB_R = 4, SB_C = 8, NXCD = 8, CU_PER_XCD = 32;
    struct Blk { std::vector<mo_wl_item> tiles; uint64_t klen; };
    std::vector<Blk> blocks;
    uint64_t total = 0;
    for (const mo_gemm_job& k : jobs) {
        const uint32_t tm = k.tm, tn = k.upper ? k.tm : k.tn;
        const uint64_t klen = k.klen;
        for (uint32_t bi = 0; bi < tm; bi += SB_R)
            for (uint32_t bj = 0; bj < tn; bj += SB_C) {
                Blk b{{}, klen};
                for (uint32_t a = bi; a < std::min(bi + SB_R, tm); ++a)
                    for (uint32_t c = bj; c < std::min(bj + SB_C, tn); ++c)
                        if (!k.upper || a <= c) b.tiles.push_back({k.idx, a, c, 4u});
                if (b.tiles.empty()) continue;
                total += klen * b.tiles.size();
                blocks.push_back(std::move(b));
            }
    }
    // A block goes whole to the least-loaded queue while that queue stays
    // under the even share; otherwise the queue takes only what fills it
    // (at least one tile) and the rest moves on to the next least-loaded.
    const uint64_t target = (total + NXCD - 1) / NXCD;
    std::vector<std::vector<mo_wl_item>> q(NXCD);
    uint64_t load[NXCD] = {0};
    for (const Blk& b : blocks) {
        size_t i = 0;
        while (i < b.tiles.size()) {
            uint32_t x = 0;
            for (uint32_t y = 1; y < NXCD; ++y)
                if (load[y] < load[x]) x = y;
            const size_t rest = b.tiles.size() - i;
            size_t take = rest;
            if (load[x] < target) {
                const uint64_t fit = (target - load[x] + b.klen - 1) / b.klen;
                take = std::min<size_t>(rest, std::max<uint64_t>(1, fit));
            }
            q[x].insert(q[x].end(), b.tiles.begin() + i, b.tiles.begin() + i + take);
            load[x] += b.klen * take;
            i += take;
        }
    }
    // Narrow tiles where full ones would leave an XCD's CUs idle: a queue of
    // n <= 32 tiles (one partial round) has every tile split, and a longer
    // queue the n % 32 tiles of its last round, into S = 4 quarter-width
    // or S = 2 half-width tiles, the largest S up to max_split (the widths
    // the launch's kernels run) that still fits the 32 CUs (none if even
    // halves do not).  Split tiles keep their place in the queue, the S parts
    // in column order.
    for (auto& v : q) {
        const size_t n = v.size();
        if (n == 0) continue;
        const size_t first = n <= CU_PER_XCD ? 0 : n - n % CU_PER_XCD;
        const size_t r = n - first;
        const uint32_t S = r == 0 ? 1
                         : (max_split >= 4 && 4 * r <= CU_PER_XCD) ? 4
                         : (max_split >= 2 && 2 * r <= CU_PER_XCD) ? 2 : 1;
        if (S == 1) continue;
        std::vector<mo_wl_item> w(v.begin(), v.begin() + first);
        for (size_t k = first; k < n; ++k)
            for (uint32_t p = 0; p < S; ++p) w.push_back({v[k].mat, v[k].ti, v[k].tj * S + p, 4 / S});
        v.swap(w);
    }
    size_t len = 0;
    for (const auto& v : q) len = std::max(len, v.size());
    for (size_t j = 0; j < len; ++j)
        for (uint32_t x = 0; x < NXCD; ++x)
            out.push_back(j < q[x].size() ? q[x][j] : mo_wl_item{MO_WL_PAD, 0, 0, 0});
}
