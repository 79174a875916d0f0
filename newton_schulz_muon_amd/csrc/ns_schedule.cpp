// Host list scheduler of the persistent NS loop: see ns_schedule.hpp.
#include "ns_schedule.hpp"

#include <algorithm>
#include <functional>
#include <queue>
#include <set>
#include <tuple>
#include <utility>

namespace muon {
namespace {

// Estimated cycles of one 256-wide tile of product ph (0 Gram, 1 polynomial,
// 2 B X): the measured loop time per 32-deep K step (the Gram's k-contiguous
// operand rows cost more) plus prologue, epilogue (the symmetric products
// also store the mirror tile, the polynomial reads A) and the barrier between
// tiles.
double item_cycles(int ph, const LoopDims& d) {
    const double K = ph == 0 ? d.np : (ph == 2 && d.split ? 3.0 * d.mp : d.mp);
    // the split products store a second plane (B': and its mirror; X': through the fp32 epilogue)
    const double epi = ph == 0 ? 12700.0 : ph == 1 ? (d.split ? 24000.0 : 16300.0) : (d.split ? 12000.0 : 7500.0);
    return (ph == 0 ? 1424.0 : 1216.0) * (K / 32) + epi;
}

// Measured cost of one item boundary beyond a tile boundary (store drain,
// counter release, item read and a satisfied dependency poll), in cycles:
// with the counters synchronised within one XCD, and at device scope (an L2
// write-back and invalidate per item).
constexpr double kItemOverheadLocal = 2000.0;
constexpr double kItemOverheadDevice = 15000.0;

struct SimBlock {
    int prob;
    uint32_t g;        // global block index
};

// Tiles per queue item: symmetric products, B X.
struct Grouping {
    uint32_t sym = 1, bx = 1;
};

// List schedule of the blocks' items over `workers` workgroups.  An item is
// a run of up to `grp` consecutive tiles of one product of one block.  A
// free workgroup takes an item of the ready product with the highest
// priority: with gram_first, Gram products first (they are the longest, and
// every later product of the block waits for them), then the earliest
// product, then the lowest block; otherwise the earliest product, then the
// lowest block.  A block's next product becomes ready when every item of its
// current one has finished.  Appends the items in the order they start
// (which respects every dependency) and returns the estimated makespan.
double list_schedule(const std::vector<SimBlock>& blocks, const std::vector<LoopDims>& dims, int steps, int workers,
                     const Grouping& grp, bool gram_first, double overhead, std::vector<ScheduleItem>* out) {
    const size_t nb = blocks.size();
    std::vector<int> k(nb, 0);
    std::vector<uint32_t> issued(nb, 0), running(nb, 0);   // tiles issued / items running
    auto tiles = [&](size_t i, int kk) { return kk % 3 == 2 ? dims[blocks[i].prob].nbx : dims[blocks[i].prob].nsym; };
    std::set<std::tuple<int, int, size_t>> ready;
    for (size_t i = 0; i < nb; ++i) ready.insert({0, 0, i});
    typedef std::pair<double, size_t> Ev;
    std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> finish;
    double t = 0.0;
    int free = workers;
    for (;;) {
        while (free > 0 && !ready.empty()) {
            const auto it = ready.begin();
            const size_t i = std::get<2>(*it);
            const int ph = k[i] % 3, iter = k[i] / 3;
            const uint32_t n = tiles(i, k[i]);
            const uint32_t cnt = std::min(n - issued[i], ph == 2 ? grp.bx : grp.sym);
            if (out)
                out->push_back(ScheduleItem{blocks[i].g | ((cnt - 1) << 28),
                                     issued[i] | (uint32_t(ph) << 22) | (uint32_t(iter) << 24)});
            finish.push({t + cnt * item_cycles(ph, dims[blocks[i].prob]) + overhead, i});
            issued[i] += cnt;
            ++running[i];
            --free;
            if (issued[i] == n) ready.erase(it);
        }
        if (finish.empty()) break;
        const Ev e = finish.top();
        finish.pop();
        t = e.first;
        ++free;
        const size_t i = e.second;
        --running[i];
        if (issued[i] == tiles(i, k[i]) && running[i] == 0) {
            ++k[i];
            issued[i] = 0;
            if (k[i] < 3 * steps) ready.insert({gram_first && k[i] % 3 != 0, k[i], i});
        }
    }
    return t;
}

}  // namespace

// Builds the item lists (host only): with 8 queues each block's tiles stay in
// one queue (blocks dealt largest first to the least loaded queue), so a
// block's operands are shared in one XCD's L2; a single queue is used instead
// when that balances clearly better.
void schedule_items(const std::vector<LoopDims>& dims, const std::vector<int64_t>& nbs, int steps, int workers,
                    bool local_ok, std::vector<ScheduleItem>& items, uint32_t (&qbase)[9], int& nq) {
    std::vector<SimBlock> all;
    std::vector<double> work;
    uint32_t g = 0;
    for (size_t p = 0; p < dims.size(); ++p) {
        const double w = steps * (dims[p].nsym * (item_cycles(0, dims[p]) + item_cycles(1, dims[p])) +
                                  dims[p].nbx * item_cycles(2, dims[p]));
        for (int64_t b = 0; b < nbs[p]; ++b) {
            all.push_back({int(p), g++});
            work.push_back(w);
        }
    }
    std::vector<std::vector<SimBlock>> qb(8);
    const bool can8 = workers % 8 == 0 && all.size() >= 8;
    if (can8) {
        std::vector<size_t> order(all.size());
        for (size_t i = 0; i < order.size(); ++i) order[i] = i;
        std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return work[x] > work[y]; });
        double load[8] = {};
        for (size_t i : order) {
            const int q = int(std::min_element(load, load + 8) - load);
            load[q] += work[i];
            qb[q].push_back(all[i]);
        }
        for (auto& v : qb)
            std::sort(v.begin(), v.end(), [](const SimBlock& x, const SimBlock& y) { return x.g < y.g; });
    }
    // Tiles per item, priority rule and queue count by the estimated makespan
    // (8 queues preferred within 5%: they keep a block's operands in one L2,
    // and with local_ok they synchronise within the XCD).
    const double ov8 = local_ok ? kItemOverheadLocal : kItemOverheadDevice;
    Grouping best;
    bool best_gram_first = true;
    bool use8 = false;
    double best_score = 0.0;
    for (int gf = 1; gf >= 0; --gf)
        for (uint32_t gs = 1; gs <= 2; ++gs)
            for (uint32_t gb = 1; gb <= 4; ++gb) {
                const Grouping grp{gs, gb};
                const double m1 =
                    1.05 * list_schedule(all, dims, steps, workers, grp, gf != 0, kItemOverheadDevice, nullptr);
                if (best_score == 0.0 || m1 < best_score) {
                    best_score = m1;
                    best = grp;
                    best_gram_first = gf != 0;
                    use8 = false;
                }
                if (can8) {
                    double m8 = 0.0;
                    for (const auto& v : qb)
                        m8 = std::max(m8, list_schedule(v, dims, steps, workers / 8, grp, gf != 0, ov8, nullptr));
                    if (m8 < best_score) {
                        best_score = m8;
                        best = grp;
                        best_gram_first = gf != 0;
                        use8 = true;
                    }
                }
            }
    items.clear();
    if (use8) {
        for (int q = 0; q < 8; ++q) {
            qbase[q] = uint32_t(items.size());
            list_schedule(qb[q], dims, steps, workers / 8, best, best_gram_first, ov8, &items);
        }
        nq = 8;
    } else {
        list_schedule(all, dims, steps, workers, best, best_gram_first, kItemOverheadDevice, &items);
        for (int q = 0; q < 8; ++q) qbase[q] = 0;
        nq = 1;
    }
    qbase[8] = uint32_t(items.size());
    if (nq == 1)
        for (int q = 1; q < 8; ++q) qbase[q] = qbase[8];
}

}  // namespace muon
