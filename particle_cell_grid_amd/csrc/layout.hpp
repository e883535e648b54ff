// layout.hpp -- work decomposition over a tile layout, shared by the deposit
// and the incremental sort: each tile slice [off[t], off[t+1]) (clipped to the
// partitioned prefix) is split into ceil(len / chunk) balanced chunks; a
// prefix over tiles numbers the chunks so that one work-group takes one chunk.
#pragma once

#include <algorithm>
#include <climits>

#include "common.hpp"

namespace pcg {
namespace {

// Work items per tile: ceil(len/chunk) (0 for an empty tile), exclusive prefix
// over tiles into cum[0..ntiles]; one work-group of 1024 threads.
__global__ __launch_bounds__(1024) void k_chunk_cum(const uint32_t *__restrict__ off,
                                                    uint32_t ntiles, int64_t n_part,
                                                    uint32_t chunk, uint32_t *__restrict__ cum,
                                                    const uint32_t *gate, uint32_t gate_run)
{
    if (gate && *gate != gate_run)
        return;
    __shared__ uint32_t wsum[1024 / WAVE];
    const uint32_t per = (ntiles + 1023) / 1024;
    const uint32_t t0 = threadIdx.x * per;
    const uint32_t t1 = min(t0 + per, ntiles);
    auto items = [&](uint32_t t) -> uint32_t {
        const uint64_t p0 = std::min<uint64_t>(off[t], (uint64_t)n_part);
        const uint64_t p1 = std::min<uint64_t>(off[t + 1], (uint64_t)n_part);
        return p1 > p0 ? (uint32_t)((p1 - p0 + chunk - 1) / chunk) : 0u;
    };
    uint32_t s = 0;
    for (uint32_t t = t0; t < t1; ++t)
        s += items(t);
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    uint32_t inc = s;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t u = __shfl_up(inc, o, WAVE);
        if (lane >= o)
            inc += u;
    }
    if (lane == WAVE - 1)
        wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < 1024 / WAVE; ++w) {
        before += w < wave ? wsum[w] : 0u;
        all += wsum[w];
    }
    uint32_t run = before + inc - s;
    for (uint32_t t = t0; t < t1; ++t) {
        cum[t] = run;
        run += items(t);
    }
    if (threadIdx.x == 0)
        cum[ntiles] = all;
}

struct ChunkRange {
    uint32_t tile;   // UINT_MAX: no work
    uint32_t chunk;  // global chunk number (= the work item)
    uint32_t lo, hi;
};

// Decode work item `item` (one thread calls this): the tile whose chunk range
// holds it, and the item's share of that tile's slice.
__device__ inline ChunkRange find_chunk(uint32_t item, const uint32_t *cum, uint32_t ntiles,
                                        const uint32_t *off, int64_t n_part)
{
    ChunkRange r{UINT_MAX, item, 0, 0};
    if (item >= cum[ntiles])
        return r;
    // largest t with cum[t] <= item (empty tiles own no items)
    uint32_t lo = 0, hi = ntiles - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (cum[mid] <= item)
            lo = mid;
        else
            hi = mid - 1;
    }
    const uint32_t t = lo;
    const uint32_t nch = cum[t + 1] - cum[t];
    const uint32_t c = item - cum[t];
    const uint64_t p0 = std::min<uint64_t>(off[t], (uint64_t)n_part);
    const uint64_t p1 = std::min<uint64_t>(off[t + 1], (uint64_t)n_part);
    const uint64_t len = p1 > p0 ? p1 - p0 : 0;
    r.tile = t;
    r.lo = (uint32_t)(p0 + len * c / nch);
    r.hi = (uint32_t)(p0 + len * (c + 1) / nch);
    return r;
}

}  // namespace
}  // namespace pcg
