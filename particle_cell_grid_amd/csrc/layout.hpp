// layout.hpp -- work decomposition over a tile layout, shared by the deposit
// and the incremental sort: each tile slice [off[t], off[t+1]) (clipped to the
// partitioned prefix) is split into ceil(len / chunk) balanced chunks; a
// prefix over tiles numbers the chunks so that one work-group takes one chunk,
// and a map from chunk number to (tile, first, end) lets a work-group find its
// chunk with one read.
#pragma once

#include <algorithm>
#include <climits>

#include "common.hpp"

namespace pcg {
namespace {

constexpr int CHUNK_SCAN_BLOCK = 1024;  // tiles per block of the chunk prefix

// Writes the n map entries of tile t (chunks c0 .. c0 + n - 1, the balanced
// split of its clipped slice), those below map_len.
__device__ inline void write_tile_chunks(ChunkEntry *map, uint32_t map_len, uint32_t c0,
                                         uint32_t n, uint32_t t, const uint32_t *off,
                                         int64_t n_part)
{
    const uint64_t p0 = std::min<uint64_t>(off[t], (uint64_t)n_part);
    const uint64_t p1 = std::min<uint64_t>(off[t + 1], (uint64_t)n_part);
    const uint64_t len = p1 > p0 ? p1 - p0 : 0;
    for (uint32_t j = 0; j < n && (uint64_t)c0 + j < map_len; ++j)
        map[c0 + j] = ChunkEntry{t, (uint32_t)(p0 + len * j / n), (uint32_t)(p0 + len * (j + 1) / n),
                                 0u};
}

// Work items of tile t: ceil(len / chunk), 0 for an empty tile.
__device__ inline uint32_t tile_items(const uint32_t *__restrict__ off, uint32_t t, int64_t n_part,
                                      uint32_t chunk)
{
    const uint64_t p0 = std::min<uint64_t>(off[t], (uint64_t)n_part);
    const uint64_t p1 = std::min<uint64_t>(off[t + 1], (uint64_t)n_part);
    return p1 > p0 ? (uint32_t)((p1 - p0 + chunk - 1) / chunk) : 0u;
}

// Exclusive prefix of v over the block (1024 threads); *total gets the sum.
__device__ inline uint32_t block_exclusive_1024(uint32_t v, uint32_t *total)
{
    __shared__ uint32_t wsum[CHUNK_SCAN_BLOCK / WAVE];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    uint32_t inc = v;
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
    for (int w = 0; w < CHUNK_SCAN_BLOCK / WAVE; ++w) {
        before += w < wave ? wsum[w] : 0u;
        all += wsum[w];
    }
    *total = all;
    return before + inc - v;
}

// Pass 1, one block per CHUNK_SCAN_BLOCK tiles: block-local exclusive prefix of
// the work items into cum[], the block's total into part[block].
__global__ __launch_bounds__(CHUNK_SCAN_BLOCK) void k_chunk_scan1(
    const uint32_t *__restrict__ off, uint32_t ntiles, int64_t n_part, uint32_t chunk,
    uint32_t *__restrict__ cum, uint32_t *__restrict__ part, const uint32_t *gate,
    uint32_t gate_run)
{
    if (gate && *gate != gate_run)
        return;
    const uint32_t t = blockIdx.x * CHUNK_SCAN_BLOCK + threadIdx.x;
    const uint32_t v = t < ntiles ? tile_items(off, t, n_part, chunk) : 0u;
    uint32_t total;
    const uint32_t ex = block_exclusive_1024(v, &total);
    if (t < ntiles)
        cum[t] = ex;
    if (threadIdx.x == 0)
        part[blockIdx.x] = total;
}

// Pass 2, one block: exclusive prefix of the nb block totals (in place); the
// grand total goes to cum[ntiles].
__global__ __launch_bounds__(CHUNK_SCAN_BLOCK) void k_chunk_scan2(uint32_t *__restrict__ part,
                                                                 uint32_t nb,
                                                                 uint32_t *__restrict__ cum,
                                                                 uint32_t ntiles,
                                                                 const uint32_t *gate,
                                                                 uint32_t gate_run)
{
    if (gate && *gate != gate_run)
        return;
    uint32_t carry = 0;
    for (uint32_t base = 0; base < nb; base += CHUNK_SCAN_BLOCK) {
        const uint32_t i = base + threadIdx.x;
        const uint32_t v = i < nb ? part[i] : 0u;
        uint32_t total;
        const uint32_t ex = block_exclusive_1024(v, &total);
        if (i < nb)
            part[i] = carry + ex;
        carry += total;
        __syncthreads();  // wsum is reused by the next round
    }
    if (threadIdx.x == 0)
        cum[ntiles] = carry;
}

// Pass 3: global prefix (cum[t] += block offset) and the map entries of the
// tile's items cum[t] .. cum[t] + items(t) - 1.
// Entries past map_len are not written (offsets that are not a partition
// could ask for more); their work items are never launched.
__global__ __launch_bounds__(CHUNK_SCAN_BLOCK) void k_chunk_scan3(
    const uint32_t *__restrict__ off, uint32_t ntiles, int64_t n_part, uint32_t chunk,
    uint32_t *__restrict__ cum, const uint32_t *__restrict__ part, ChunkEntry *__restrict__ map,
    uint32_t map_len, const uint32_t *gate, uint32_t gate_run)
{
    if (gate && *gate != gate_run)
        return;
    const uint32_t t = blockIdx.x * CHUNK_SCAN_BLOCK + threadIdx.x;
    if (t >= ntiles)
        return;
    const uint32_t c0 = cum[t] + part[blockIdx.x];
    cum[t] = c0;
    write_tile_chunks(map, map_len, c0, tile_items(off, t, n_part, chunk), t, off, n_part);
}

// Tiles up to which the whole layout is computed in one launch.
constexpr uint32_t CHUNK_PAR_MAX = 8192;
constexpr int CHUNK_PAR_TPT = CHUNK_PAR_MAX / CHUNK_SCAN_BLOCK;  // tiles per thread
constexpr uint32_t CHUNK_PAR_BLOCKS = 64;  // most work-groups of that launch

// The whole layout in one launch (ntiles <= CHUNK_PAR_MAX), on several
// work-groups.  Each work-group computes the prefix of the tiles' work items
// into LDS (the same prefix in every work-group: a few KB of offsets each),
// then writes its share of the map entries, finding each entry's tile by
// binary search in the prefix.  Work-group 0 also writes cum[] and, if `flag`
// is given, whether off is a partition of [0, n_part): *flag = 0 if off[0] = 0,
// off is non-decreasing and off[ntiles] = n_part, else 1.
__global__ __launch_bounds__(CHUNK_SCAN_BLOCK) void k_chunk_layout_par(
    const uint32_t *__restrict__ off, uint32_t ntiles, int64_t n_part, uint32_t chunk,
    uint32_t *__restrict__ cum, ChunkEntry *__restrict__ map, uint32_t map_len,
    const uint32_t *gate, uint32_t gate_run, uint32_t *flag)
{
    if (gate && *gate != gate_run)
        return;
    __shared__ uint32_t s_cum[CHUNK_PAR_MAX + 1];
    __shared__ uint32_t s_bad;
    if (threadIdx.x == 0)
        s_bad = 0;
    const bool check = flag && blockIdx.x == 0;
    const uint32_t t0 = threadIdx.x * CHUNK_PAR_TPT;
    uint32_t items[CHUNK_PAR_TPT], sum = 0;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < CHUNK_PAR_TPT; ++j) {
        const uint32_t t = t0 + j;
        items[j] = t < ntiles ? tile_items(off, t, n_part, chunk) : 0u;
        sum += items[j];
        if (check && t < ntiles)
            bad = bad || (t == 0 ? off[0] != 0u : off[t] < off[t - 1]);
    }
    __syncthreads();  // s_bad is cleared
    if (bad)
        atomicOr(&s_bad, 1u);
    uint32_t total;
    uint32_t c = block_exclusive_1024(sum, &total);
#pragma unroll
    for (int j = 0; j < CHUNK_PAR_TPT; ++j) {
        const uint32_t t = t0 + j;
        if (t < ntiles)
            s_cum[t] = c;
        c += items[j];
    }
    if (threadIdx.x == 0)
        s_cum[ntiles] = total;
    __syncthreads();
    if (blockIdx.x == 0) {
        for (uint32_t t = threadIdx.x; t <= ntiles; t += CHUNK_SCAN_BLOCK)
            cum[t] = s_cum[t];
        if (check && threadIdx.x == 0) {
            bool b = s_bad != 0u || (int64_t)off[ntiles] != n_part;
            b = b || (ntiles == 0 ? off[0] != 0u : off[ntiles] < off[ntiles - 1]);
            *flag = b ? 1u : 0u;
        }
    }
    const uint32_t nent = min(total, map_len);
    for (uint32_t e = blockIdx.x * CHUNK_SCAN_BLOCK + threadIdx.x; e < nent;
         e += gridDim.x * CHUNK_SCAN_BLOCK) {
        // the tile t with s_cum[t] <= e < s_cum[t + 1] (s_cum[0] = 0 <= e < total)
        uint32_t lo = 0, hi = ntiles;
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) / 2;
            if (s_cum[mid] <= e)
                lo = mid;
            else
                hi = mid;
        }
        const uint32_t n = s_cum[lo + 1] - s_cum[lo], j = e - s_cum[lo];
        const uint64_t p0 = std::min<uint64_t>(off[lo], (uint64_t)n_part);
        const uint64_t p1 = std::min<uint64_t>(off[lo + 1], (uint64_t)n_part);
        const uint64_t len = p1 > p0 ? p1 - p0 : 0;
        map[e] = ChunkEntry{lo, (uint32_t)(p0 + len * j / n), (uint32_t)(p0 + len * (j + 1) / n),
                            0u};
    }
}

// Work-groups of the one-launch layout for a map of map_len entries.
inline uint32_t chunk_par_blocks(uint32_t map_len)
{
    return std::max<uint32_t>(1u, std::min<uint32_t>(CHUNK_PAR_BLOCKS,
                                                     (map_len + CHUNK_SCAN_BLOCK - 1) /
                                                         CHUNK_SCAN_BLOCK));
}

// Enqueues the layout: cum[0..ntiles] and map[0..min(cum[ntiles], map_len)),
// in one launch for up to CHUNK_PAR_MAX tiles, else in three passes
// (part needs ceil(ntiles / CHUNK_SCAN_BLOCK) entries).  With a gate, the
// kernels return at once unless *gate == gate_run.
inline pcg_status launch_chunk_layout(const char *name, const uint32_t *off, uint32_t ntiles,
                                      int64_t n_part, uint32_t chunk, uint32_t *cum,
                                      uint32_t *part, ChunkEntry *map, uint32_t map_len,
                                      const uint32_t *gate, uint32_t gate_run, hipStream_t st)
{
    if (ntiles <= CHUNK_PAR_MAX)
        return launch(name, k_chunk_layout_par, dim3(chunk_par_blocks(map_len)),
                      dim3(CHUNK_SCAN_BLOCK), 0, st, off, ntiles, n_part, chunk, cum, map,
                      map_len, gate, gate_run, (uint32_t *)nullptr);
    const uint32_t nb = (ntiles + CHUNK_SCAN_BLOCK - 1) / CHUNK_SCAN_BLOCK;
    PCG_TRY(launch(name, k_chunk_scan1, dim3(nb), dim3(CHUNK_SCAN_BLOCK), 0, st, off, ntiles,
                   n_part, chunk, cum, part, gate, gate_run));
    PCG_TRY(launch(name, k_chunk_scan2, dim3(1), dim3(CHUNK_SCAN_BLOCK), 0, st, part, nb, cum,
                   ntiles, gate, gate_run));
    return launch(name, k_chunk_scan3, dim3(nb), dim3(CHUNK_SCAN_BLOCK), 0, st, off, ntiles,
                  n_part, chunk, cum, (const uint32_t *)part, map, map_len, gate, gate_run);
}

// Entries of part[] launch_chunk_layout needs for ntiles tiles.
inline size_t chunk_part_len(uint32_t ntiles)
{
    return (ntiles + CHUNK_SCAN_BLOCK - 1) / CHUNK_SCAN_BLOCK + 1;
}

struct ChunkRange {
    uint32_t tile;   // UINT_MAX: no work
    uint32_t chunk;  // global chunk number (= the work item)
    uint32_t lo, hi;
};

// Decode work item `item` (item < the map's length): its tile and particle
// range, from one map entry (entries past the total are stale: checked first).
__device__ inline ChunkRange find_chunk(uint32_t item, const uint32_t *cum, const ChunkEntry *map,
                                        uint32_t ntiles)
{
    ChunkRange r{UINT_MAX, item, 0, 0};
    const uint32_t total = cum[ntiles];
    if (item >= total)
        return r;
    const ChunkEntry e = map[item];
    if (e.tile >= ntiles || e.hi <= e.lo)
        return r;
    r.tile = e.tile;
    r.lo = e.lo;
    r.hi = e.hi;
    return r;
}

}  // namespace
}  // namespace pcg
