// Checks the persistent NS loop's host list scheduler (ns_schedule.cpp) on
// fixed and seeded random sets of block batches.  For every queue set built:
// each (block, iteration, product, tile) appears exactly once; item fields
// are in range (tile runs inside the product's tile count, the tile decodes
// to an upper-triangle tile or a B X tile); every block's items are in one
// queue; and within a queue every item comes after all tiles of the block's
// earlier products (what the kernel waits for, counted as it counts).
// Prints one line per set and "ALL OK", or the first violation; exit code 0
// only when every set passes.
#include <cstdio>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "ns_schedule.hpp"

using muon::LoopDims;
using muon::ScheduleItem;

static LoopDims dims_of(int mp, int np) {
    const uint32_t T = uint32_t(mp / 256), Tn = uint32_t(np / 256);
    return LoopDims{mp, np, T * (T + 1) / 2, T * Tn};
}

static int check(const std::vector<LoopDims>& dims, const std::vector<int64_t>& nbs, int steps, int workers,
                 bool local_ok) {
    std::vector<ScheduleItem> items;
    uint32_t qbase[9];
    int nq = 0;
    muon::schedule_items(dims, nbs, steps, workers, local_ok, items, qbase, nq);
    std::vector<uint32_t> first;
    uint32_t blocks = 0;
    for (int64_t nb : nbs) {
        first.push_back(blocks);
        blocks += uint32_t(nb);
    }
    auto problem = [&](uint32_t g) {
        size_t p = 0;
        for (size_t i = 1; i < first.size(); ++i)
            if (g >= first[i]) p = i;
        return p;
    };
    uint64_t expect = 0;
    for (size_t p = 0; p < dims.size(); ++p) expect += uint64_t(nbs[p]) * steps * (2 * dims[p].nsym + dims[p].nbx);
    if (nq != 1 && nq != 8) { std::printf("FAIL: nq %d\n", nq); return 1; }
    if (qbase[8] != items.size()) { std::printf("FAIL: qbase[8] %u vs %zu items\n", qbase[8], items.size()); return 1; }
    for (int q = 0; q < 8; ++q)
        if (qbase[q] > qbase[q + 1]) { std::printf("FAIL: qbase not ordered\n"); return 1; }
    if (nq == 1 && qbase[1] != qbase[8]) { std::printf("FAIL: one queue but qbase[1] != qbase[8]\n"); return 1; }
    std::set<std::tuple<uint32_t, uint32_t, uint32_t, uint32_t>> seen;
    std::vector<int> queue_of(blocks, -1);
    uint64_t tiles = 0;
    for (int q = 0; q < nq; ++q) {
        std::vector<uint32_t> done(blocks, 0);   // tiles of each block listed so far in this queue
        for (uint32_t i = qbase[q]; i < qbase[q + 1]; ++i) {
            const uint32_t g = items[i].x & 0x0fffffffu, cnt = (items[i].x >> 28) + 1;
            const uint32_t id = items[i].y & 0x3fffffu, ph = (items[i].y >> 22) & 3u, t = items[i].y >> 24;
            if (g >= blocks || ph > 2 || t >= uint32_t(steps)) { std::printf("FAIL: item %u out of range\n", i); return 1; }
            const LoopDims& d = dims[problem(g)];
            if (id + cnt > (ph == 2 ? d.nbx : d.nsym)) { std::printf("FAIL: item %u tile run\n", i); return 1; }
            if (queue_of[g] == -1) queue_of[g] = q;
            if (queue_of[g] != q) { std::printf("FAIL: block %u in two queues\n", g); return 1; }
            const uint32_t need = t * (2 * d.nsym + d.nbx) + (ph >= 1 ? d.nsym : 0u) + (ph >= 2 ? d.nsym : 0u);
            if (done[g] < need) {
                std::printf("FAIL: item %u (queue %d) listed before its dependencies (%u of %u tiles)\n", i, q, done[g], need);
                return 1;
            }
            const int T = d.mp / 256, Tn = d.np / 256;
            for (uint32_t c = 0; c < cnt; ++c) {
                const int tile = int(id + c);
                if (ph < 2) {
                    int r = 0, len = T, x = tile;
                    while (x >= len) { x -= len; ++r; --len; }
                    if (!(r + x < T)) { std::printf("FAIL: symmetric tile %d decodes outside\n", tile); return 1; }
                } else if (!(tile % T < T && tile / T < Tn)) {
                    std::printf("FAIL: B X tile %d decodes outside\n", tile);
                    return 1;
                }
                if (!seen.insert(std::make_tuple(g, t, ph, uint32_t(tile))).second) {
                    std::printf("FAIL: tile listed twice\n");
                    return 1;
                }
            }
            done[g] += cnt;
            tiles += cnt;
        }
    }
    if (tiles != expect) { std::printf("FAIL: %llu tiles listed, %llu expected\n", (unsigned long long)tiles, (unsigned long long)expect); return 1; }
    std::printf("ok: %zu items, %u blocks, %d queue(s)\n", items.size(), blocks, nq);
    return 0;
}

int main() {
    int bad = 0;
    bad |= check({dims_of(768, 3072)}, {32}, 5, 256, true);                          // the 32 x 768x3072 batch
    bad |= check({dims_of(768, 768), dims_of(768, 3072)}, {40, 22}, 5, 256, true);   // 124M attn + mlp
    bad |= check({dims_of(256, 512)}, {3}, 5, 256, true);
    bad |= check({dims_of(256, 256)}, {2}, 2, 256, false);
    bad |= check({dims_of(4096, 4096), dims_of(4096, 14336)}, {8, 8}, 5, 256, true);
    bad |= check({dims_of(512, 1536)}, {3}, 1, 256, false);
    bad |= check({dims_of(768, 3072)}, {32}, 5, 80, true);                           // fewer workgroups
    std::mt19937 rng(12345);
    for (int trial = 0; trial < 150 && !bad; ++trial) {
        std::vector<LoopDims> d;
        std::vector<int64_t> nb;
        const int n = 1 + int(rng() % 4);
        for (int i = 0; i < n; ++i) {
            d.push_back(dims_of(256 * (1 + int(rng() % 4)), 256 * (1 + int(rng() % 8))));
            nb.push_back(1 + int64_t(rng() % 12));
        }
        bad |= check(d, nb, 1 + int(rng() % 6), (rng() % 2) ? 256 : 8 * (1 + int(rng() % 40)), (rng() % 2) != 0);
    }
    std::printf(bad ? "FAILED\n" : "ALL OK\n");
    return bad;
}
