// Host list scheduler of the persistent NS loop (host code only, no HIP).
//
// The loop (k_ns_loop in ns_gemm.hip) runs every NS iteration of a set of
// block batches in one launch; its workgroups take items from queues built
// here.  An item is a run of 1..16 consecutive 256-wide tiles of one product
// (Gram, polynomial or B X) of one NS iteration of one block:
//   x = global block index | (tiles - 1) << 28
//   y = first tile | product << 22 | iteration << 24
// Symmetric products (Gram, polynomial) enumerate a block's upper-triangle
// tiles row by row; B X tiles are numbered with the tile row fastest.  Each
// queue lists items so that every item depends only on items listed before
// it in the same queue (a block's products of an iteration in order), and
// every block's items are in one queue.
#pragma once

#include <cstdint>
#include <vector>

namespace muon {

// One block batch: padded sides (multiples of 256) and tiles per block.
struct LoopDims {
    int mp, np;
    uint32_t nsym, nbx;    // symmetric products' upper tiles; B X tiles
    bool split = false;    // ACCURATE: B X reduces over 3 mp (Bh Xh, Bh Xl, Bl Xh), B' has two planes
};

struct ScheduleItem {
    uint32_t x, y;
};

// Builds the queues for nbs[p] blocks of dims[p] over `steps` iterations and
// `workers` workgroups: either 8 queues (qbase[q]..qbase[q + 1], a block's
// items all in one queue; preferred, and with local_ok modelled with the
// cheaper XCD-local synchronisation) or 1 queue (qbase[0] = 0, qbase[1..8] =
// items.size()).  The run lengths, the priority rule (Gram products first, or
// the earliest product first) and the queue count are those with the lowest
// simulated makespan.
void schedule_items(const std::vector<LoopDims>& dims, const std::vector<int64_t>& nbs, int steps, int workers,
                    bool local_ok, std::vector<ScheduleItem>& items, uint32_t (&qbase)[9], int& nq);

}  // namespace muon
