// sort.hip -- stable tile sort of particles ([TD] Entity wiki "Tiled current
// deposit", section "The tile-based spatial sort"; with T = 1 the cell sort the
// mass-matrix paper's §3.1 assumes).
//
// The result is the unique stable permutation by tile key; two paths reach it.
//
// Incremental path (the input was tile-sorted by `prev` and its particles have
// since moved at most one tile -- [TD] "Halo sizing": at most one cell per
// un-sorted step under CFL).  Every particle's new tile is then one of the 27
// (fewer on a thin grid) neighbours of the tile whose slice holds it, so the
// stable order is a counting sort over (source chunk, direction):
//   k_inc_validate  prev is a partition of [0, count) (else fall back);
//   k_chunk_scan*   source slices split into balanced chunks (prefix and a
//                   chunk-to-tile map);
//   k_inc_count     per chunk, particles per direction (a particle that moved
//                   further raises the fall-back flag);
//   k_inc_totals    per new tile, the sum over its source (chunk, direction)s;
//   scan            -> tile offsets;
//   k_inc_bases     per new tile, running prefix over its sources in source
//                   order -> output base of every (chunk, direction);
//   k_inc_scatter   per chunk, stable ranks by direction (wave ballots), one
//                   coalesced read and one write of every SoA array.
// General path (no `prev`, or the flag is raised):
//   k_tile_keys; LSD radix sort of (key, index) in ceil(bits/8) passes of
//   <= 8 bits (per-block digit histograms, a scan, a stable scatter ranking
//   each wave's keys with ballot peer masks); k_tile_offsets from key
//   transitions; k_permute moves the SoA arrays to their slots, by gather
//   through the permutation, or (an input mostly in tile order, as counted by
//   the first histogram pass) by scatter through its inverse, which the last
//   scatter pass writes.
// Both paths are enqueued when `prev` is given; a device flag makes the kernels
// of the path not taken return at once, so the call stays asynchronous.
#include <algorithm>

#include "common.hpp"
#include "layout.hpp"
#include "regroup.hpp"

namespace pcg {
namespace {

constexpr int SORT_BLOCK = 256;
constexpr int SORT_IPT = 16;
constexpr int SORT_TILE = SORT_BLOCK * SORT_IPT;            // items per block
constexpr int SORT_SLOTS = SORT_IPT * (SORT_BLOCK / WAVE);  // wave-slots per block
constexpr int SCAN_BLOCK = 256;
constexpr int SCAN_IPT = 16;
constexpr int SCAN_TILE = SCAN_BLOCK * SCAN_IPT;

// ----------------------------------------------------------------- keys

template <int DIM, int ORDER>
__global__ __launch_bounds__(256) void k_tile_keys(int64_t count, const float *__restrict__ x0,
                                                   const float *__restrict__ x1,
                                                   const float *__restrict__ x2, KeyGeom g,
                                                   uint32_t *__restrict__ keys,
                                                   uint32_t *__restrict__ same, Gate gate)
{
    if (gated_off(gate))
        return;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *same = 0u;  // counted by the first histogram pass
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const float *xs[3] = {x0, x1, x2};
        uint32_t key = 0, mul = 1;
#pragma unroll
        for (int k = 0; k < DIM; ++k) {
            key += mul * (uint32_t)tile_coord<ORDER>(xs[k][i], g, k);
            mul *= (uint32_t)g.nt[k];
        }
        keys[i] = key;
    }
}

// ----------------------------------------------------------------- radix

template <int BITS>
__global__ __launch_bounds__(SORT_BLOCK) void k_radix_hist(const uint32_t *__restrict__ keys,
                                                           int64_t count, int shift,
                                                           uint32_t *__restrict__ counts,
                                                           uint32_t nblocks,
                                                           uint32_t *__restrict__ same, Gate gate)
{
    if (gated_off(gate))
        return;
    constexpr uint32_t R = 1u << BITS;
    __shared__ uint32_t hist[R];
    // same (first pass only): particles whose key equals that of the particle
    // before them in the input (within a wave), the input's measure of order
    uint32_t eq = 0;
    // the launch may have fewer work-groups than key blocks: each takes every
    // gridDim.x-th block (a small grid keeps a gated-off launch cheap)
    for (uint32_t vb = blockIdx.x; vb < nblocks; vb += gridDim.x) {
        for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK)
            hist[d] = 0;
        __syncthreads();
        const int64_t base = (int64_t)vb * SORT_TILE;
#pragma unroll 4
        for (int j = 0; j < SORT_IPT; ++j) {
            const int64_t idx = base + (int64_t)j * SORT_BLOCK + threadIdx.x;
            const bool valid = idx < count;
            const uint32_t key = valid ? keys[idx] : 0u;
            const uint32_t digit = (key >> shift) & (R - 1);
            if (same) {
                const uint32_t before = __shfl_up(key, 1, WAVE);
                const bool vb = __shfl_up((int)valid, 1, WAVE) != 0;
                eq += (lane_id() > 0 && valid && vb && before == key) ? 1u : 0u;
            }
            const uint64_t peers = peer_mask<BITS>(digit, valid);
            // the lowest lane of each peer group adds the group's size
            if (valid && (peers & lanemask_lt()) == 0)
                atomicAdd(&hist[digit], (uint32_t)__popcll(peers));
        }
        __syncthreads();
        for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK)
            counts[(size_t)d * nblocks + vb] = hist[d];
        __syncthreads();  // hist is cleared for the next block
    }
    if (same) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            eq += (uint32_t)__shfl_xor((int)eq, o, WAVE);
        if (lane_id() == 0 && eq)
            atomicAdd(same, eq);
    }
}

// The arrays are moved by scatter (out[rank[i]] = in[i]) when at least half
// of the input's neighbours share a key (a re-sort of nearly ordered
// particles: reads and most writes consecutive), else by gather (out[i] =
// in[perm[i]]: an unordered input would scatter its writes over whole lines).
__device__ inline bool permute_by_scatter(const uint32_t *same, int64_t count)
{
    return 2 * (int64_t)*same >= count;
}

template <int BITS>
__global__ __launch_bounds__(SORT_BLOCK) void k_radix_scatter(
    const uint32_t *__restrict__ keys_in, const uint32_t *__restrict__ vals_in,
    uint32_t *__restrict__ keys_out, uint32_t *__restrict__ vals_out, int64_t count, int shift,
    const uint32_t *__restrict__ offsets, uint32_t nblocks, uint32_t *__restrict__ rank_out,
    const uint32_t *__restrict__ same, Gate gate)
{
    if (gated_off(gate))
        return;
    if (rank_out && !permute_by_scatter(same, count))
        rank_out = nullptr;
    constexpr uint32_t R = 1u << BITS;
    __shared__ uint16_t cnt[SORT_SLOTS][R];  // items of digit d in wave-slot s, then prefix
    __shared__ uint32_t gbase[R];
    // virtual blocks, as in k_radix_hist
    for (uint32_t vb = blockIdx.x; vb < nblocks; vb += gridDim.x) {
    __syncthreads();  // the previous block is done with cnt and gbase
    {
        uint32_t *c32 = reinterpret_cast<uint32_t *>(&cnt[0][0]);
        constexpr int words = SORT_SLOTS * R / 2;
        for (int i = threadIdx.x; i < words; i += SORT_BLOCK)
            c32[i] = 0;
    }
    for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK)
        gbase[d] = offsets[(size_t)d * nblocks + vb];
    __syncthreads();

    const int wave = threadIdx.x / WAVE;
    const int64_t base = (int64_t)vb * SORT_TILE;
    uint32_t key[SORT_IPT], val[SORT_IPT];
    uint16_t rank[SORT_IPT];
#pragma unroll
    for (int j = 0; j < SORT_IPT; ++j) {
        const int64_t idx = base + (int64_t)j * SORT_BLOCK + threadIdx.x;
        const bool valid = idx < count;
        key[j] = valid ? keys_in[idx] : 0u;
        val[j] = valid ? (vals_in ? vals_in[idx] : (uint32_t)idx) : 0u;
        const uint32_t digit = (key[j] >> shift) & (R - 1);
        const uint64_t peers = peer_mask<BITS>(digit, valid);
        rank[j] = (uint16_t)__popcll(peers & lanemask_lt());
        if (valid && rank[j] == 0)
            cnt[j * (SORT_BLOCK / WAVE) + wave][digit] = (uint16_t)__popcll(peers);
    }
    __syncthreads();
    // exclusive prefix over wave-slots, per digit (slot order = item order)
    for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK) {
        uint32_t run = 0;
        for (int s = 0; s < SORT_SLOTS; ++s) {
            const uint32_t c = cnt[s][d];
            cnt[s][d] = (uint16_t)run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SORT_IPT; ++j) {
        const int64_t idx = base + (int64_t)j * SORT_BLOCK + threadIdx.x;
        if (idx < count) {
            const uint32_t digit = (key[j] >> shift) & (R - 1);
            const uint32_t dst =
                gbase[digit] + cnt[j * (SORT_BLOCK / WAVE) + wave][digit] + rank[j];
            if (dst < (uint64_t)count) {  // always true for a consistent histogram
                keys_out[dst] = key[j];
                vals_out[dst] = val[j];
                // the last pass: where each input element goes
                if (rank_out && val[j] < (uint64_t)count)
                    rank_out[val[j]] = dst;
            }
        }
    }
    }
}

// ----------------------------------------------------------------- scan

__device__ inline uint32_t wave_inclusive_scan(uint32_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t o = __shfl_up(v, off, WAVE);
        if (lane >= off)
            v += o;
    }
    return v;
}

// Exclusive scan of one value per thread across the block; returns the
// exclusive prefix and writes the block total to *total.
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t *total)
{
    __shared__ uint32_t wsum[NT / WAVE];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == WAVE - 1)
        wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / WAVE; ++w) {
        const uint32_t s = wsum[w];
        before += (w < wave) ? s : 0u;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_reduce(const uint32_t *__restrict__ in,
                                                            size_t len,
                                                            uint32_t *__restrict__ partial,
                                                            Gate gate)
{
    if (gated_off(gate))
        return;
    const uint32_t nparts = (uint32_t)((len + SCAN_TILE - 1) / SCAN_TILE);
    for (uint32_t part = blockIdx.x; part < nparts; part += gridDim.x) {
        const size_t base = (size_t)part * SCAN_TILE;
        uint32_t s = 0;
        for (int j = 0; j < SCAN_IPT; ++j) {
            const size_t idx = base + (size_t)j * SCAN_BLOCK + threadIdx.x;
            if (idx < len)
                s += in[idx];
        }
        uint32_t total;
        block_exclusive_scan<SCAN_BLOCK>(s, &total);
        if (threadIdx.x == 0)
            partial[part] = total;
    }
}

// Single work-group exclusive scan of the partial sums (in place).
__global__ __launch_bounds__(1024) void k_scan_partials(uint32_t *__restrict__ partial,
                                                        uint32_t nparts, Gate gate)
{
    if (gated_off(gate))
        return;
    const uint32_t per = (nparts + 1023) / 1024;
    const uint32_t lo = threadIdx.x * per;
    const uint32_t hi = min(lo + per, nparts);
    uint32_t s = 0;
    for (uint32_t i = lo; i < hi; ++i)
        s += partial[i];
    uint32_t total;
    uint32_t run = block_exclusive_scan<1024>(s, &total);
    for (uint32_t i = lo; i < hi; ++i) {
        const uint32_t v = partial[i];
        partial[i] = run;
        run += v;
    }
}

__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_down(uint32_t *__restrict__ data, size_t len,
                                                          const uint32_t *__restrict__ partial,
                                                          Gate gate)
{
    if (gated_off(gate))
        return;
    const uint32_t nparts = (uint32_t)((len + SCAN_TILE - 1) / SCAN_TILE);
    for (uint32_t part = blockIdx.x; part < nparts; part += gridDim.x) {
        // thread t owns SCAN_IPT consecutive elements of the part
        const size_t base = (size_t)part * SCAN_TILE + (size_t)threadIdx.x * SCAN_IPT;
        uint32_t v[SCAN_IPT];
        uint32_t s = 0;
#pragma unroll
        for (int j = 0; j < SCAN_IPT; ++j) {
            v[j] = (base + j < len) ? data[base + j] : 0u;
            s += v[j];
        }
        uint32_t total;
        uint32_t run = block_exclusive_scan<SCAN_BLOCK>(s, &total) + partial[part];
#pragma unroll
        for (int j = 0; j < SCAN_IPT; ++j) {
            if (base + j < len)
                data[base + j] = run;
            run += v[j];
        }
    }
}

// The whole scan in one work-group, for short arrays: rounds of SCAN_ONE_IPT
// consecutive elements per thread, carried from round to round.
constexpr int SCAN_ONE_IPT = 16;
constexpr size_t SCAN_ONE_MAX = 65536;

__global__ __launch_bounds__(1024) void k_scan_one(uint32_t *__restrict__ data, size_t len,
                                                   Gate gate)
{
    if (gated_off(gate))
        return;
    __shared__ uint32_t s_carry;
    if (threadIdx.x == 0)
        s_carry = 0;
    __syncthreads();
    for (size_t base = 0; base < len; base += (size_t)1024 * SCAN_ONE_IPT) {
        const size_t i0 = base + (size_t)threadIdx.x * SCAN_ONE_IPT;
        uint32_t v[SCAN_ONE_IPT], s = 0;
#pragma unroll
        for (int j = 0; j < SCAN_ONE_IPT; ++j) {
            v[j] = i0 + j < len ? data[i0 + j] : 0u;
            s += v[j];
        }
        uint32_t total;
        uint32_t run = s_carry + block_exclusive_scan<1024>(s, &total);
#pragma unroll
        for (int j = 0; j < SCAN_ONE_IPT; ++j) {
            if (i0 + j < len)
                data[i0 + j] = run;
            run += v[j];
        }
        __syncthreads();  // every thread has read s_carry
        if (threadIdx.x == 0)
            s_carry += total;
        __syncthreads();
    }
}

// Work-groups of a general-path launch over n blocks of work: the kernels
// loop over their blocks, so a launch behind the incremental path (gated,
// nearly always returning at once) stays small; an ungated one fills the chip.
inline uint32_t general_grid(int64_t n, const Gate &gate)
{
    const int64_t cap = (int64_t)device_cus() * (gate.flag ? 2 : 8);
    return (uint32_t)std::max<int64_t>(1, std::min<int64_t>(n, cap));
}

pcg_status exclusive_scan(uint32_t *data, size_t len, uint32_t *partial, Gate gate,
                          hipStream_t st)
{
    if (len <= SCAN_ONE_MAX)
        return launch("sort_scan", k_scan_one, dim3(1), dim3(1024), 0, st, data, len, gate);
    const uint32_t nparts = (uint32_t)((len + SCAN_TILE - 1) / SCAN_TILE);
    PCG_TRY(launch("sort_scan_reduce", k_scan_reduce, dim3(general_grid(nparts, gate)),
                   dim3(SCAN_BLOCK), 0, st,
                   (const uint32_t *)data, len, partial, gate));
    PCG_TRY(launch("sort_scan_partials", k_scan_partials, dim3(1), dim3(1024), 0, st, partial,
                   nparts, gate));
    PCG_TRY(launch("sort_scan_down", k_scan_down, dim3(general_grid(nparts, gate)),
                   dim3(SCAN_BLOCK), 0, st, data,
                   len, (const uint32_t *)partial, gate));
    return PCG_OK;
}

// ----------------------------------------------------------------- offsets, permute

__global__ __launch_bounds__(256) void k_tile_offsets(const uint32_t *__restrict__ sk,
                                                      int64_t count, uint32_t ntiles,
                                                      uint32_t *__restrict__ off, Gate gate)
{
    if (gated_off(gate))
        return;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i <= count; i += stride) {
        // tiles t in (sk[i-1], sk[i]] start at slot i (sk[-1] = -1, sk[count] = ntiles)
        const uint32_t lo = (i == 0) ? 0u : sk[i - 1] + 1u;
        const uint32_t hi = (i == count) ? ntiles : sk[i];
        for (uint32_t t = lo; t <= hi && t <= ntiles; ++t)
            off[t] = (uint32_t)i;
    }
}

constexpr int PERM_EPT = 4;  // elements per thread: all rank loads, then the arrays

// The sort's permutation applied to the SoA arrays, in one of two forms
// chosen on the device (permute_by_scatter): out[k][rank[i]] = in[k][i], each
// array read in order, rank the inverse permutation from the last radix pass;
// or out[k][i] = in[k][perm[i]].  Where most particles keep their order (a
// re-sort), the first reads and writes consecutive words but for the few
// movers, while a gather would read every particle that changed tile from its
// old tile's range; for an unordered input the gather's scattered reads cost
// less than scattered writes.
__global__ __launch_bounds__(256) void k_permute(PermArgs a, const uint32_t *__restrict__ perm,
                                                 const uint32_t *__restrict__ rank,
                                                 const uint32_t *__restrict__ same, int64_t count,
                                                 Gate gate)
{
    if (gated_off(gate))
        return;
    const bool scatter = permute_by_scatter(same, count);
    const uint32_t *__restrict__ idx = scatter ? rank : perm;
    for (int64_t blk = blockIdx.x; blk * 256 * PERM_EPT < count; blk += gridDim.x) {
    const int64_t i0 = (blk * PERM_EPT) * 256 + threadIdx.x;
    uint32_t r[PERM_EPT];
#pragma unroll
    for (int e = 0; e < PERM_EPT; ++e) {
        const int64_t i = i0 + e * 256;
        // a permutation of [0, count); the clamp only keeps a broken one in bounds
        r[e] = i < count ? min(idx[i], (uint32_t)(count - 1)) : 0u;
    }
    for (int k = 0; k < a.n; ++k) {
        float v[PERM_EPT];
#pragma unroll
        for (int e = 0; e < PERM_EPT; ++e) {
            const int64_t i = i0 + e * 256;
            v[e] = i < count ? a.in[k][scatter ? i : r[e]] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < PERM_EPT; ++e) {
            const int64_t i = i0 + e * 256;
            if (i < count)
                a.out[k][scatter ? r[e] : i] = v[e];
        }
    }
    }
}

// ----------------------------------------------------------------- incremental path

__global__ void k_set_flag(uint32_t *flag, uint32_t v)
{
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *flag = v;
}

// prev must be a partition of [0, count): off[0] = 0, non-decreasing,
// off[ntiles] = count.  Anything else falls back to the general path.
__global__ __launch_bounds__(256) void k_inc_validate(const uint32_t *__restrict__ off,
                                                      uint32_t ntiles, int64_t count,
                                                      uint32_t *flag)
{
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t > ntiles)
        return;
    bool bad = false;
    if (t == 0)
        bad = off[0] != 0u;
    else
        bad = off[t] < off[t - 1];
    if (t == ntiles)
        bad = bad || (int64_t)off[ntiles] != count;
    if (bad)
        atomicOr(flag, 1u);
}

// One work-group per chunk: every particle's direction (the new tile relative
// to the source tile), the chunk's per-direction counts, and the device flag
// if a particle moved further than one tile.  The work-group's lanes read
// consecutive particles (COUNT_EPT per lane in flight, the next batch loading
// while this one is classified); counts are per wave (ballots) and then per
// work-group (LDS).  Launched with 256 threads and 4 particles per lane for
// chunks of thousands of particles, with one wave and one particle per lane
// for small ones.
template <int DIM, int ORDER, int COUNT_EPT, bool POW2>
__global__ __launch_bounds__(256) void k_inc_count(IncGeom a, const float *x0, const float *x1,
                                                   const float *x2)
{
    if (*a.flag != 0u)
        return;
    __shared__ uint32_t s_tile, s_lo, s_hi;
    __shared__ uint32_t s_cnt[32];
    if (threadIdx.x == 0) {
        const ChunkRange r = find_chunk(blockIdx.x, a.cum, a.map, a.ntiles);
        s_tile = r.tile;
        s_lo = r.lo;
        s_hi = r.hi;
    }
    if (threadIdx.x < 32)
        s_cnt[threadIdx.x] = 0;
    __syncthreads();
    if (s_tile == UINT_MAX)
        return;
    int sc[3];
    tile_coords(s_tile, a.g, sc);
    const uint32_t lo = s_lo, hi = s_hi, stride = blockDim.x;
    // clamped loads: no branch around them, so the next batch stays in flight;
    // addressed from the chunk's first particle (uniform) by a 32-bit offset,
    // which needs no 64-bit address arithmetic per lane
    const float *c0 = x0 + lo, *c1 = DIM > 1 ? x1 + lo : nullptr, *c2 = DIM > 2 ? x2 + lo : nullptr;
    const uint32_t last = hi - 1 - lo;
    float c[COUNT_EPT][3], nc[COUNT_EPT][3];
    auto at = [](const float *base, uint32_t q) {
        return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + q * 4u);
    };
    auto load = [&](uint32_t b, float (*dst)[3]) {
#pragma unroll
        for (int e = 0; e < COUNT_EPT; ++e) {
            const uint32_t q = min(b - lo + e * stride, last);  // below a chunk's length
            dst[e][0] = at(c0, q);
            dst[e][1] = DIM > 1 ? at(c1, q) : 0.f;
            dst[e][2] = DIM > 2 ? at(c2, q) : 0.f;
        }
    };
    bool far = false;
    auto classify = [&](uint32_t b, float (*cx)[3]) {
#pragma unroll
        for (int e = 0; e < COUNT_EPT; ++e) {
            const bool valid = b + e * stride < hi;
            // the geometry test is a template argument here: a per-particle
            // uniform branch would split the batch's straight-line code
            const int dir = POW2 ? particle_dir_pow2<DIM, ORDER>(cx[e][0], cx[e][1], cx[e][2], a.g, sc)
                                 : particle_dir<DIM, ORDER>(cx[e][0], cx[e][1], cx[e][2], a.g, sc);
            far |= valid && dir < 0;
            const bool ok = valid && dir >= 0;
            // most particles stay in their tile: one ballot counts those, and
            // each leaver adds itself
            const uint64_t stay = __ballot(ok && dir == DIR_STAY);
            if (lane_id() == 0 && stay)
                atomicAdd(&s_cnt[DIR_STAY], (uint32_t)__popcll(stay));
            if (ok && dir != DIR_STAY)
                atomicAdd(&s_cnt[dir], 1u);
        }
    };
    // two batch buffers in turn (no register copies): the next batch loads
    // while this one is classified
    const uint32_t step = COUNT_EPT * stride;
    load(lo + threadIdx.x, c);
    for (uint32_t b = lo + threadIdx.x; b - threadIdx.x < hi; b += 2 * step) {
        load(b + step, nc);
        classify(b, c);
        if (b + step - threadIdx.x >= hi)
            break;
        load(b + 2 * step, c);
        classify(b + step, nc);
    }
    if (__ballot(far))
        if (lane_id() == 0)
            atomicOr(a.flag, 1u);
    __syncthreads();
    if (threadIdx.x < NDIR)
        a.cnt[(size_t)blockIdx.x * NDIR + threadIdx.x] = s_cnt[threadIdx.x];
}

// Per (source tile, direction): exclusive prefix of the counts over the tile's
// chunks (in place) and the tile's total.  A work-group takes PREFIX_TILES
// tiles: the prefixes run tile-major (consecutive threads on one chunk's
// consecutive counts), the totals go through LDS and out direction-major
// (consecutive threads on consecutive tiles).  8 tiles (one item per thread)
// where tiles hold several chunks, 16 where most hold one.
template <int PREFIX_TILES>
__global__ __launch_bounds__(256) void k_inc_chunk_prefix(IncGeom a)
{
    if (*a.flag != 0u)
        return;
    __shared__ uint32_t tot[NDIR][PREFIX_TILES];
    const uint32_t s0 = blockIdx.x * PREFIX_TILES;
    const uint32_t nt = min((uint32_t)PREFIX_TILES, a.ntiles - s0);
    for (uint32_t i = threadIdx.x; i < nt * NDIR; i += blockDim.x) {
        const uint32_t sl = i / NDIR, d = i % NDIR, s = s0 + sl;
        uint32_t run = 0;
        for (uint32_t c = a.cum[s]; c < a.cum[s + 1]; ++c) {
            const size_t j = (size_t)c * NDIR + d;
            const uint32_t v = a.cnt[j];
            a.cnt[j] = run;
            run += v;
        }
        tot[d][sl] = run;
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nt * NDIR; i += blockDim.x) {
        const uint32_t d = i / nt, sl = i % nt;
        a.tcnt[(size_t)d * a.ntiles + s0 + sl] = tot[d][sl];
    }
}

// The distinct source coordinates of new-tile coordinate tc on one axis of nt
// tiles, ascending, with the direction index (0, 1, 2 for -1, 0, +1) that
// leads from each to tc.  Returns how many (1, 2 or 3).
__device__ inline int axis_sources(int tc, int nt, int *c, int *d)
{
    if (nt == 1) {
        c[0] = tc;
        d[0] = 1;
        return 1;
    }
    // source tc - delta for delta = +1, 0 (and -1 when nt >= 3)
    int n = 0;
    int cc[3], dd[3];
    cc[n] = wrap_index(tc - 1, nt);
    dd[n++] = 2;
    cc[n] = tc;
    dd[n++] = 1;
    if (nt >= 3) {
        cc[n] = wrap_index(tc + 1, nt);
        dd[n++] = 0;
    }
    // sort <= 3 entries by coordinate
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if (cc[j] < cc[i]) {
                int t = cc[i];
                cc[i] = cc[j];
                cc[j] = t;
                t = dd[i];
                dd[i] = dd[j];
                dd[j] = t;
            }
    for (int i = 0; i < n; ++i) {
        c[i] = cc[i];
        d[i] = dd[i];
    }
    return n;
}

// Thread per new tile: its particle count (scan input) and, in source order
// (ascending linear index = lexicographic in z, y, x), the prefix of every
// source's share.
__global__ __launch_bounds__(256) void k_inc_tiles(IncGeom a, uint32_t *__restrict__ totals)
{
    if (*a.flag != 0u)
        return;
    // blocks are dealt to the 8 XCDs in turn: give each XCD a contiguous run
    // of new tiles, so that the rows of their shared source tiles are read
    // through one L2 (the grid is a multiple of 8 blocks)
    const uint32_t per = gridDim.x / 8;
    const uint32_t blk = (blockIdx.x % 8) * per + blockIdx.x / 8;
    const uint32_t t = blk * blockDim.x + threadIdx.x;
    if (t > a.ntiles)
        return;
    if (t == a.ntiles) {
        totals[t] = 0;
        return;
    }
    int tc[3];
    tile_coords(t, a.g, tc);
    int cx[3], dx[3], cy[3], dy[3], cz[3], dz[3];
    const int nx = axis_sources(tc[0], a.g.nt[0], cx, dx);
    const int ny = axis_sources(tc[1], a.g.nt[1], cy, dy);
    const int nz = axis_sources(tc[2], a.g.nt[2], cz, dz);
    // all (up to 27) source counts are read first, then prefixed in source
    // order; the loops have fixed bounds so that the reads issue together
    size_t jj[27];
    uint32_t v[27];
#pragma unroll
    for (int iz = 0; iz < 3; ++iz)
#pragma unroll
        for (int iy = 0; iy < 3; ++iy)
#pragma unroll
            for (int ix = 0; ix < 3; ++ix) {
                const int q = ix + 3 * iy + 9 * iz;
                const bool ok = ix < nx && iy < ny && iz < nz;
                const int c[3] = {cx[ok ? ix : 0], cy[ok ? iy : 0], cz[ok ? iz : 0]};
                jj[q] = (size_t)(dx[ok ? ix : 0] + 3 * dy[ok ? iy : 0] + 9 * dz[ok ? iz : 0]) *
                            a.ntiles +
                        tile_index(c, a.g);
                v[q] = ok ? a.tcnt[jj[q]] : 0u;
            }
    uint32_t run = 0;
#pragma unroll
    for (int iz = 0; iz < 3; ++iz)
#pragma unroll
        for (int iy = 0; iy < 3; ++iy)
#pragma unroll
            for (int ix = 0; ix < 3; ++ix) {
                const int q = ix + 3 * iy + 9 * iz;
                if (ix < nx && iy < ny && iz < nz) {
                    a.tpre[jj[q]] = run;
                    run += v[q];
                }
            }
    totals[t] = run;
}

// One wave per chunk (four per work-group), walking it in order EPT * 64
// particles at a time: each particle's direction again from its position, its
// slot from the wave's running slot per direction (stable), then every array
// moved.
constexpr int MOVE_WAVES = 4;
constexpr int MOVE_GROUP = 8;  // arrays whose loads the move issues together

template <int DIM, int ORDER, int EPT>
__global__ __launch_bounds__(MOVE_WAVES * WAVE) void k_inc_move(
    IncGeom a, const uint32_t *off, const float *x0, const float *x1, const float *x2,
    PermArgs arr, uint32_t *perm, uint32_t *keys, uint32_t nwork)
{
    if (*a.flag != 0u)
        return;
    __shared__ uint32_t s_run[MOVE_WAVES][32];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    const uint32_t item = blockIdx.x * MOVE_WAVES + wave;
    if (item >= nwork)
        return;
    const ChunkRange r = find_chunk(item, a.cum, a.map, a.ntiles);
    if (r.tile == UINT_MAX)
        return;
    int sc[3];
    tile_coords(r.tile, a.g, sc);
    uint32_t *run = s_run[wave];
    if (lane < NDIR)
        run[lane] = move_base(a, off, r.tile, r.chunk, lane);
    __builtin_amdgcn_wave_barrier();
    for (uint32_t b = r.lo; b < r.hi; b += WAVE * EPT) {
        uint32_t p[EPT], pc[EPT], pos[EPT];
        int dir[EPT];
        bool ok[EPT];
        float c[EPT][3];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            p[e] = b + e * WAVE + lane;
            pc[e] = min(p[e], r.hi - 1);  // clamped: loads without a branch
            c[e][0] = x0[pc[e]];
            c[e][1] = DIM > 1 ? x1[pc[e]] : 0.f;
            c[e][2] = DIM > 2 ? x2[pc[e]] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            dir[e] = tile_dir<DIM, ORDER>(c[e][0], c[e][1], c[e][2], a.g, sc);
            ok[e] = p[e] < r.hi && dir[e] >= 0;  // dir < 0 cannot occur: the flag is clear
            pos[e] = walk_slot(run, dir[e], ok[e]);
            ok[e] = ok[e] && pos[e] < (uint64_t)a.count;
        }
        if (keys) {
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (ok[e])
                    keys[pos[e]] = dest_tile(sc, dir[e], a.g);
        }
        if (perm) {
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (ok[e])
                    perm[pos[e]] = p[e];
        }
        // up to MOVE_GROUP arrays are loaded before any is stored, so that
        // their loads are in flight together (a store may alias a later load,
        // which would otherwise keep each array's round trip apart)
        for (int k0 = 0; k0 < arr.n; k0 += MOVE_GROUP) {
            float v[MOVE_GROUP][EPT];
#pragma unroll
            for (int j = 0; j < MOVE_GROUP; ++j) {
                if (k0 + j >= arr.n)
                    continue;
                // an array that is one of the keyed positions is already in
                // registers (a wave-uniform pointer test): not fetched twice
                const float *src = arr.in[k0 + j];
                if (src == x0) {
#pragma unroll
                    for (int e = 0; e < EPT; ++e)
                        v[j][e] = c[e][0];
                } else if (DIM > 1 && src == x1) {
#pragma unroll
                    for (int e = 0; e < EPT; ++e)
                        v[j][e] = c[e][1];
                } else if (DIM > 2 && src == x2) {
#pragma unroll
                    for (int e = 0; e < EPT; ++e)
                        v[j][e] = c[e][2];
                } else {
#pragma unroll
                    for (int e = 0; e < EPT; ++e)
                        v[j][e] = src[pc[e]];
                }
            }
#pragma unroll
            for (int j = 0; j < MOVE_GROUP; ++j)
                if (k0 + j < arr.n)
#pragma unroll
                    for (int e = 0; e < EPT; ++e)
                        if (ok[e])
                            arr.out[k0 + j][pos[e]] = v[j][e];
        }
    }
}

// The move for small chunks (a few dozen particles, e.g. cells): each wave
// takes MOVE_SMALL_K consecutive chunks and issues every stage's reads for all
// of them at once -- the chunk lookups, the 27 slot bases of each, then one
// 64-particle step of each chunk's positions and arrays -- instead of paying
// the round trips once per chunk.  Ranks, slots and stores are those of
// k_inc_move.
constexpr int MOVE_SMALL_K = 4;

template <int DIM, int ORDER>
__global__ __launch_bounds__(MOVE_WAVES * WAVE) void k_inc_move_small(
    IncGeom a, const uint32_t *off, const float *x0, const float *x1, const float *x2,
    PermArgs arr, uint32_t *perm, uint32_t *keys, uint32_t nwork)
{
    constexpr int K = MOVE_SMALL_K;
    static_assert(K * NDIR <= 2 * WAVE, "two slot bases per lane");
    if (*a.flag != 0u)
        return;
    __shared__ uint32_t s_run[MOVE_WAVES][K][32];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    const uint32_t item0 = (blockIdx.x * MOVE_WAVES + wave) * K;
    if (item0 >= nwork)
        return;
    // the K chunks, one per lane
    uint32_t ct = UINT_MAX, cc = 0, clo = 0, chi = 0;
    if (lane < K && item0 + lane < nwork) {
        const ChunkRange r = find_chunk(item0 + lane, a.cum, a.map, a.ntiles);
        ct = r.tile;
        cc = r.chunk;
        clo = r.lo;
        chi = r.hi;
    }
    // their slot bases, (chunk j, direction d) at lane j * NDIR + d (two rounds of lanes)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = lane + WAVE * h;
        const int j = min(idx / NDIR, K - 1), d = idx % NDIR;
        const uint32_t tj = __shfl(ct, j), cj = __shfl(cc, j);
        if (idx < K * NDIR && tj != UINT_MAX)
            s_run[wave][j][d] = move_base(a, off, tj, cj, d);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t tile[K], lo[K], hi[K], len = 0;
    int sc[K][3];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        tile[j] = __builtin_amdgcn_readlane(ct, j);
        lo[j] = __builtin_amdgcn_readlane(clo, j);
        hi[j] = __builtin_amdgcn_readlane(chi, j);
        if (tile[j] == UINT_MAX)
            hi[j] = lo[j];
        tile_coords(tile[j] == UINT_MAX ? 0u : tile[j], a.g, sc[j]);
        len = max(len, hi[j] - lo[j]);
    }
    for (uint32_t st = 0; st < len; st += WAVE) {
        uint32_t p[K], pc[K], pos[K];
        int dir[K];
        bool ok[K];
        float c[K][3];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            p[j] = lo[j] + st + lane;
            // clamped into the chunk (or to particle 0 for an empty one): no branch
            pc[j] = hi[j] > lo[j] ? min(p[j], hi[j] - 1) : 0u;
            c[j][0] = x0[pc[j]];
            c[j][1] = DIM > 1 ? x1[pc[j]] : 0.f;
            c[j][2] = DIM > 2 ? x2[pc[j]] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            dir[j] = tile_dir<DIM, ORDER>(c[j][0], c[j][1], c[j][2], a.g, sc[j]);
            ok[j] = p[j] < hi[j] && dir[j] >= 0;  // dir < 0 cannot occur: the flag is clear
            pos[j] = walk_slot(s_run[wave][j], dir[j], ok[j]);
            ok[j] = ok[j] && pos[j] < (uint64_t)a.count;
        }
        if (keys) {
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (ok[j])
                    keys[pos[j]] = dest_tile(sc[j], dir[j], a.g);
        }
        if (perm) {
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (ok[j])
                    perm[pos[j]] = p[j];
        }
        // every array's values first (one round trip), then the stores
        // (a keyed position array is taken from registers, as in k_inc_move)
        float v[MAX_ARRAYS][K];
#pragma unroll
        for (int k = 0; k < MAX_ARRAYS; ++k) {
            const float *src = k < arr.n ? arr.in[k] : nullptr;
            if (src == nullptr) {
#pragma unroll
                for (int j = 0; j < K; ++j)
                    v[k][j] = 0.f;
            } else if (src == x0) {
#pragma unroll
                for (int j = 0; j < K; ++j)
                    v[k][j] = c[j][0];
            } else if (DIM > 1 && src == x1) {
#pragma unroll
                for (int j = 0; j < K; ++j)
                    v[k][j] = c[j][1];
            } else if (DIM > 2 && src == x2) {
#pragma unroll
                for (int j = 0; j < K; ++j)
                    v[k][j] = c[j][2];
            } else {
#pragma unroll
                for (int j = 0; j < K; ++j)
                    v[k][j] = src[pc[j]];
            }
        }
#pragma unroll
        for (int k = 0; k < MAX_ARRAYS; ++k) {
            if (k < arr.n) {
#pragma unroll
                for (int j = 0; j < K; ++j)
                    if (ok[j])
                        arr.out[k][pos[j]] = v[k][j];
            }
        }
    }
}

// ----------------------------------------------------------------- host

struct SortPlan {
    int64_t count = 0;
    uint32_t ntiles = 1;
    int key_bits = 0;
    int passes = 1;
    int bits = 1;
    uint32_t nblocks = 0;
    size_t counts_len = 0;
    uint32_t nchunks_max = 0;
};

SortPlan make_plan(const pcg_grid *grid, int64_t count, int T)
{
    SortPlan p;
    p.count = count;
    uint64_t nt = 1;
    for (int k = 0; k < grid->dim; ++k)
        nt *= (uint64_t)(grid->n[k] / T);
    p.ntiles = (uint32_t)nt;
    int kb = 0;
    while ((uint64_t(1) << kb) < nt)
        ++kb;
    p.key_bits = kb;
    p.passes = kb == 0 ? 1 : (kb + 7) / 8;
    p.bits = kb == 0 ? 1 : (kb + p.passes - 1) / p.passes;
    p.nblocks = (uint32_t)((count + SORT_TILE - 1) / SORT_TILE);
    p.counts_len = (size_t)(1u << p.bits) * p.nblocks;
    p.nchunks_max = p.ntiles + (uint32_t)((count + INC_CHUNK - 1) / INC_CHUNK);
    return p;
}

struct SortBuffers {
    uint32_t *k0, *ak, *av, *bv, *fk, *pm, *counts, *partial;
    uint32_t *flag, *cum, *cnt, *tcnt, *tpre, *cpart;
    uint32_t *same;  // general path: neighbouring particles with equal keys
    ChunkEntry *cmap;
};

size_t carve(const SortPlan &p, void *ws, SortBuffers *b)
{
    Carver c(ws);
    const size_t n = (size_t)p.count;
    b->k0 = c.take<uint32_t>(n);
    b->ak = c.take<uint32_t>(n);
    b->av = c.take<uint32_t>(n);
    b->bv = c.take<uint32_t>(n);
    b->fk = c.take<uint32_t>(n);
    b->pm = c.take<uint32_t>(n);
    b->counts = c.take<uint32_t>(p.counts_len);
    const size_t scan_len = std::max(p.counts_len, (size_t)p.ntiles + 1);
    b->partial = c.take<uint32_t>((scan_len + SCAN_TILE - 1) / SCAN_TILE + 1);
    b->flag = c.take<uint32_t>(1);
    b->same = c.take<uint32_t>(1);
    b->cum = c.take<uint32_t>((size_t)p.ntiles + 1);
    b->cnt = c.take<uint32_t>((size_t)p.nchunks_max * NDIR);
    b->tcnt = c.take<uint32_t>((size_t)p.ntiles * NDIR);
    b->tpre = c.take<uint32_t>((size_t)p.ntiles * NDIR);
    b->cpart = c.take<uint32_t>(chunk_part_len(p.ntiles));
    b->cmap = c.take<ChunkEntry>(p.nchunks_max);
    return c.used;
}

pcg_status check_sort_args(const pcg_grid *grid, int64_t count, int T, const char *who)
{
    PCG_TRY(check_grid(grid, who));
    if (T < 1)
        return fail(PCG_EINVAL, "%s: T = %d < 1", who, T);
    for (int k = 0; k < grid->dim; ++k)
        if (grid->n[k] % T)
            return fail(PCG_EINVAL, "%s: n[%d] = %d is not a multiple of T = %d", who, k,
                        grid->n[k], T);
    if (count < 0 || count >= (int64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^31)", who, (long long)count);
    return PCG_OK;
}

template <int BITS>
pcg_status radix_pass(const SortPlan &p, int shift, const uint32_t *kin, const uint32_t *vin,
                      uint32_t *kout, uint32_t *vout, uint32_t *rank, const SortBuffers &b,
                      Gate gate, hipStream_t st)
{
    PCG_TRY(launch("sort_hist", k_radix_hist<BITS>, dim3(general_grid(p.nblocks, gate)),
                   dim3(SORT_BLOCK), 0, st,
                   kin, p.count, shift, b.counts, p.nblocks, shift == 0 ? b.same : nullptr, gate));
    PCG_TRY(exclusive_scan(b.counts, p.counts_len, b.partial, gate, st));
    PCG_TRY(launch("sort_scatter", k_radix_scatter<BITS>, dim3(general_grid(p.nblocks, gate)),
                   dim3(SORT_BLOCK), 0,
                   st, kin, vin, kout, vout, p.count, shift, (const uint32_t *)b.counts,
                   p.nblocks, rank, (const uint32_t *)b.same, gate));
    return PCG_OK;
}

pcg_status radix_pass_dispatch(int bits, const SortPlan &p, int shift, const uint32_t *kin,
                               const uint32_t *vin, uint32_t *kout, uint32_t *vout,
                               uint32_t *rank, const SortBuffers &b, Gate gate, hipStream_t st)
{
    switch (bits) {
    case 1: return radix_pass<1>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    case 2: return radix_pass<2>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    case 3: return radix_pass<3>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    case 4: return radix_pass<4>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    case 5: return radix_pass<5>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    case 6: return radix_pass<6>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    case 7: return radix_pass<7>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    case 8: return radix_pass<8>(p, shift, kin, vin, kout, vout, rank, b, gate, st);
    default: return fail(PCG_EUNSUPPORTED, "radix pass of %d bits", bits);
    }
}

template <int DIM, int ORDER>
pcg_status launch_keys(int64_t count, const float *const x[3], const KeyGeom &g, uint32_t *keys,
                       uint32_t *same, Gate gate, hipStream_t st)
{
    return launch("sort_keys", k_tile_keys<DIM, ORDER>, dim3(general_grid((count + 255) / 256, gate)),
                  dim3(256), 0, st, count, x[0], DIM > 1 ? x[1] : nullptr,
                  DIM > 2 ? x[2] : nullptr, g, keys, same, gate);
}

pcg_status general_path(const pcg_grid *grid, int order, const SortPlan &p, const KeyGeom &g,
                        const float *const key_x[3], const PermArgs &arr, uint32_t *perm,
                        uint32_t *sorted_keys, uint32_t *tile_offsets, const SortBuffers &b,
                        Gate gate, hipStream_t st)
{
    const int64_t count = p.count;
    const int key = grid->dim * 10 + order;
    pcg_status s = PCG_OK;
    switch (key) {
    case 11: s = launch_keys<1, 1>(count, key_x, g, b.k0, b.same, gate, st); break;
    case 12: s = launch_keys<1, 2>(count, key_x, g, b.k0, b.same, gate, st); break;
    case 21: s = launch_keys<2, 1>(count, key_x, g, b.k0, b.same, gate, st); break;
    case 22: s = launch_keys<2, 2>(count, key_x, g, b.k0, b.same, gate, st); break;
    case 31: s = launch_keys<3, 1>(count, key_x, g, b.k0, b.same, gate, st); break;
    case 32: s = launch_keys<3, 2>(count, key_x, g, b.k0, b.same, gate, st); break;
    }
    PCG_TRY(s);
    uint32_t *final_keys = sorted_keys ? sorted_keys : b.fk;
    if (!perm)
        perm = b.pm;  // the last radix pass needs somewhere to put the permutation
    const uint32_t *kin = b.k0;
    const uint32_t *vin = nullptr;  // pass 0 ranks input indices
    // the inverse permutation, written by the last pass (where the arrays will
    // be moved by scatter) into the value buffer that pass does not read (b.bv
    // after an even number of passes, else b.av)
    uint32_t *rank = arr.n > 0 ? (p.passes % 2 == 0 ? b.bv : b.av) : nullptr;
    for (int pass = 0; pass < p.passes; ++pass) {
        const bool last = pass == p.passes - 1;
        uint32_t *kout = last ? final_keys : (pass % 2 == 0 ? b.ak : b.k0);
        uint32_t *vout = last ? perm : (pass % 2 == 0 ? b.av : b.bv);
        PCG_TRY(radix_pass_dispatch(p.bits, p, pass * p.bits, kin, vin, kout, vout,
                                    last ? rank : nullptr, b, gate, st));
        kin = kout;
        vin = vout;
    }
    PCG_TRY(launch("sort_offsets", k_tile_offsets, dim3(general_grid((count + 1 + 255) / 256, gate)),
                   dim3(256), 0, st,
                   (const uint32_t *)final_keys, count, p.ntiles, tile_offsets, gate));
    if (arr.n > 0) {
        const int64_t blocks = (count + 256 * PERM_EPT - 1) / (256 * PERM_EPT);
        PCG_TRY(launch("sort_permute", k_permute, dim3(general_grid(blocks, gate)), dim3(256), 0,
                       st, arr, (const uint32_t *)perm, (const uint32_t *)rank,
                       (const uint32_t *)b.same, count, gate));
    }
    return PCG_OK;
}

template <int DIM, int ORDER>
pcg_status incremental_launch(const IncGeom &a, const float *const key_x[3], uint32_t nwork,
                              const PermArgs &arr, uint32_t *perm, uint32_t *keys,
                              uint32_t *tile_offsets, const SortBuffers &b, const MoveHook *hook,
                              hipStream_t st)
{
    const float *x1 = DIM > 1 ? key_x[1] : nullptr, *x2 = DIM > 2 ? key_x[2] : nullptr;
    // a work-group per chunk: 256 threads when a tile's slice averages a
    // chunk or more, one wave when chunks are small
    const bool big = a.count / std::max<int64_t>(1, a.ntiles) >= (int64_t)INC_CHUNK;
    auto kern = big ? (a.g.pow2 ? k_inc_count<DIM, ORDER, 4, true> : k_inc_count<DIM, ORDER, 4, false>)
                    : (a.g.pow2 ? k_inc_count<DIM, ORDER, 1, true> : k_inc_count<DIM, ORDER, 1, false>);
    PCG_TRY(launch("sort_inc_count", kern, dim3(nwork), dim3(big ? 256 : 64), 0, st, a, key_x[0],
                   x1, x2));
    PCG_TRY(launch("sort_inc_chunk_prefix", big ? k_inc_chunk_prefix<8> : k_inc_chunk_prefix<16>,
                   dim3((a.ntiles + (big ? 8 : 16) - 1) / (big ? 8 : 16)), dim3(256), 0, st, a));
    PCG_TRY(launch("sort_inc_tiles", k_inc_tiles, dim3((a.ntiles + 1 + 2047) / 2048 * 8),
                   dim3(256), 0, st, a, tile_offsets));
    PCG_TRY(exclusive_scan(tile_offsets, (size_t)a.ntiles + 1, b.partial, Gate{b.flag, 0u}, st));
    if (hook)
        return hook->launch(hook->ctx, a, tile_offsets, nwork, arr, st);
    // 8 x 64 particles per step of a wave's walk through its chunk (eight
    // arrays of them in flight at once; four per step ran 10% slower); where
    // chunks are small, several chunks per wave
    if (a.count / std::max<int64_t>(1, a.ntiles) >= (int64_t)INC_CHUNK)
        PCG_TRY(launch("sort_inc_move", k_inc_move<DIM, ORDER, 8>,
                       dim3((nwork + MOVE_WAVES - 1) / MOVE_WAVES), dim3(MOVE_WAVES * WAVE), 0, st,
                       a, (const uint32_t *)tile_offsets, key_x[0], x1, x2, arr, perm, keys,
                       nwork));
    else
        PCG_TRY(launch("sort_inc_move", k_inc_move_small<DIM, ORDER>,
                       dim3((nwork + MOVE_WAVES * MOVE_SMALL_K - 1) / (MOVE_WAVES * MOVE_SMALL_K)),
                       dim3(MOVE_WAVES * WAVE), 0, st, a, (const uint32_t *)tile_offsets, key_x[0],
                       x1, x2, arr, perm, keys, nwork));
    return PCG_OK;
}

}  // namespace

size_t sort_workspace_bytes(const pcg_grid *grid, int64_t count, int32_t T)
{
    if (check_sort_args(grid, count, T, "pcg_sort_workspace_bytes") != PCG_OK)
        return 0;
    SortPlan p = make_plan(grid, count, T);
    SortBuffers b;
    return std::max<size_t>(carve(p, nullptr, &b), 256);
}

pcg_status tile_sort_impl(const pcg_grid *grid, int32_t order, int32_t T, int64_t count,
                          const float *const key_x[3], int32_t n_arrays,
                          const float *const in_arrays[], float *const out_arrays[],
                          uint32_t *perm, uint32_t *sorted_keys, uint32_t *tile_offsets,
                          const pcg_tile *prev, void *workspace, size_t workspace_bytes,
                          hipStream_t st, const MoveHook *hook, bool *incremental_taken)
{
    const char *who = "pcg_tile_sort";
    if (incremental_taken)
        *incremental_taken = false;
    PCG_TRY(check_sort_args(grid, count, T, who));
    if (order != 1 && order != 2)
        return fail(PCG_EUNSUPPORTED, "%s: order %d not in {1,2}", who, order);
    if (count > 0 && !key_x)
        return fail(PCG_EINVAL, "%s: key_x is NULL", who);
    for (int k = 0; k < grid->dim && count > 0; ++k)
        if (!key_x[k])
            return fail(PCG_EINVAL, "%s: key_x[%d] is NULL", who, k);
    if (n_arrays < 0 || n_arrays > MAX_ARRAYS)
        return fail(PCG_EINVAL, "%s: n_arrays = %d not in [0, %d]", who, n_arrays, MAX_ARRAYS);
    if (n_arrays > 0 && (!in_arrays || !out_arrays))
        return fail(PCG_EINVAL, "%s: array lists are NULL", who);
    for (int i = 0; i < n_arrays && count > 0; ++i) {
        if (!in_arrays[i] || !out_arrays[i])
            return fail(PCG_EINVAL, "%s: array %d is NULL", who, i);
        if ((const void *)in_arrays[i] == (const void *)out_arrays[i])
            return fail(PCG_EINVAL, "%s: array %d is permuted in place (out == in)", who, i);
    }
    if (!tile_offsets)
        return fail(PCG_EINVAL, "%s: tile_offsets is NULL", who);
    if (prev) {
        if (prev->T != T || prev->order != order)
            return fail(PCG_EINVAL, "%s: prev layout has T = %d, order = %d; sorting with T = %d,"
                        " order = %d", who, prev->T, prev->order, T, order);
        if (!prev->tile_offsets)
            return fail(PCG_EINVAL, "%s: prev->tile_offsets is NULL", who);
        if ((const void *)prev->tile_offsets == (const void *)tile_offsets)
            return fail(PCG_EINVAL, "%s: prev->tile_offsets must differ from tile_offsets", who);
    }
    SortPlan p = make_plan(grid, count, T);
    SortBuffers b;
    const size_t need = carve(p, nullptr, &b);
    if (!workspace || workspace_bytes < need)
        return fail(PCG_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(PCG_EWORKSPACE, "%s: workspace must be 256-byte aligned", who);
    carve(p, workspace, &b);
    const Gate always{nullptr, 0u};

    if (count == 0) {
        return launch("sort_offsets", k_tile_offsets, dim3(1), dim3(256), 0, st,
                      (const uint32_t *)nullptr, count, p.ntiles, tile_offsets, always);
    }

    KeyGeom g;
    for (int k = 0; k < 3; ++k) {
        g.n[k] = grid->n[k];
        g.nf[k] = (float)grid->n[k];
        g.nt[k] = k < grid->dim ? grid->n[k] / T : 1;
    }
    g.T = T;
    g.T_shift = -1;
    for (int s = 0; s < 31; ++s)
        if ((1 << s) == T)
            g.T_shift = s;
    auto is_pow2 = [](int v) { return v > 0 && (v & (v - 1)) == 0; };
    g.pow2 = g.T_shift >= 0;
    for (int k = 0; k < grid->dim; ++k)
        g.pow2 = g.pow2 && is_pow2(grid->n[k]) && is_pow2(g.nt[k]) && g.nt[k] >= 4;
    PermArgs arr{};
    for (int i = 0; i < n_arrays; ++i) {
        arr.in[i] = in_arrays[i];
        arr.out[i] = out_arrays[i];
    }
    arr.n = n_arrays;

    // the incremental path needs a layout that covers every particle
    const bool incremental = prev && prev->n_partitioned == count;
    if (incremental_taken)
        *incremental_taken = incremental;
    Gate gate = always;
    if (incremental) {
        IncGeom a;
        a.g = g;
        a.ntiles = p.ntiles;
        a.prev_off = prev->tile_offsets;
        a.count = count;
        a.cum = b.cum;
        a.map = b.cmap;
        a.cnt = b.cnt;
        a.tcnt = b.tcnt;
        a.tpre = b.tpre;
        a.flag = b.flag;
        const uint32_t chunk = INC_CHUNK;
        const uint32_t nwork = p.nchunks_max;  // >= ntiles + ceil(count / chunk)
        if (p.ntiles <= CHUNK_PAR_MAX) {
            // one launch: the chunk layout, and the flag set from the check
            // that prev is a partition
            PCG_TRY(launch("sort_inc_chunks", k_chunk_layout_par,
                           dim3(chunk_par_blocks(p.nchunks_max)), dim3(CHUNK_SCAN_BLOCK), 0, st,
                           prev->tile_offsets, p.ntiles, count, chunk, b.cum, b.cmap,
                           p.nchunks_max, (const uint32_t *)nullptr, 0u, b.flag));
        } else {
            PCG_TRY(launch("sort_inc_flag", k_set_flag, dim3(1), dim3(64), 0, st, b.flag, 0u));
            PCG_TRY(launch("sort_inc_validate", k_inc_validate,
                           dim3((p.ntiles + 1 + 255) / 256), dim3(256), 0, st,
                           prev->tile_offsets, p.ntiles, count, b.flag));
            PCG_TRY(launch_chunk_layout("sort_inc_chunks", prev->tile_offsets, p.ntiles, count,
                                        chunk, b.cum, b.cpart, b.cmap, p.nchunks_max,
                                        (const uint32_t *)b.flag, 0u, st));
        }
        const int key = grid->dim * 10 + order;
        pcg_status s = PCG_OK;
        switch (key) {
        case 11: s = incremental_launch<1, 1>(a, key_x, nwork, arr, perm, sorted_keys, tile_offsets, b, hook, st); break;
        case 12: s = incremental_launch<1, 2>(a, key_x, nwork, arr, perm, sorted_keys, tile_offsets, b, hook, st); break;
        case 21: s = incremental_launch<2, 1>(a, key_x, nwork, arr, perm, sorted_keys, tile_offsets, b, hook, st); break;
        case 22: s = incremental_launch<2, 2>(a, key_x, nwork, arr, perm, sorted_keys, tile_offsets, b, hook, st); break;
        case 31: s = incremental_launch<3, 1>(a, key_x, nwork, arr, perm, sorted_keys, tile_offsets, b, hook, st); break;
        case 32: s = incremental_launch<3, 2>(a, key_x, nwork, arr, perm, sorted_keys, tile_offsets, b, hook, st); break;
        }
        PCG_TRY(s);
        gate = Gate{b.flag, 1u};  // the general path runs only if the flag was raised
    }
    return general_path(grid, order, p, g, key_x, arr, perm, sorted_keys, tile_offsets, b, gate,
                        st);
}

}  // namespace pcg

using namespace pcg;

extern "C" {

size_t pcg_sort_workspace_bytes(const pcg_grid *grid, int64_t count, int32_t T)
{
    return sort_workspace_bytes(grid, count, T);
}

pcg_status pcg_tile_sort(const pcg_grid *grid, int32_t order, int32_t T, int64_t count,
                         const float *const key_x[3], int32_t n_arrays,
                         const float *const in_arrays[], float *const out_arrays[],
                         uint32_t *perm, uint32_t *sorted_keys, uint32_t *tile_offsets,
                         const pcg_tile *prev, void *workspace, size_t workspace_bytes,
                         void *stream)
{
    clear_error();
    return tile_sort_impl(grid, order, T, count, key_x, n_arrays, in_arrays, out_arrays, perm,
                          sorted_keys, tile_offsets, prev, workspace, workspace_bytes,
                          static_cast<hipStream_t>(stream), nullptr, nullptr);
}

}  // extern "C"
