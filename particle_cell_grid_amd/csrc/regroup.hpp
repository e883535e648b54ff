// regroup.hpp -- what the tile sort's incremental path shares with the kernel
// that deposits and regroups in one pass over the particle data: the tile
// geometry, the per-chunk direction/rank bookkeeping, and the host entry of the
// sort with a hook for the move stage.
#pragma once

#include "common.hpp"

namespace pcg {

constexpr int MAX_ARRAYS = 16;        // SoA arrays a sort carries along
constexpr int NDIR = 27;              // neighbour directions of the incremental path
constexpr uint32_t INC_CHUNK = 2048;  // particles per chunk of the incremental path
constexpr int DIR_STAY = NDIR / 2;    // direction (0, 0, 0): the same tile

// A kernel runs only if `flag` is NULL or *flag == run.
struct Gate {
    const uint32_t *flag;
    uint32_t run;
};
__device__ inline bool gated_off(const Gate &g) { return g.flag && *g.flag != g.run; }

struct KeyGeom {
    int n[3];
    float nf[3];
    int nt[3];
    int T;
    int T_shift;  // log2(T) if T is a power of two, else -1
    int pow2;     // every used axis has n and n / T >= 4 powers of two (and T too)
};

// Tile coordinate of a particle along one axis: the tile holding its first
// support node (wrapped).
template <int ORDER>
__device__ inline int tile_coord(float xraw, const KeyGeom &g, int k)
{
    const float xf = clamp_coord(xraw, g.nf[k]);
    const float fl = floorf(xf);
    int b = (int)fl;
    if (ORDER == 2 && (xf - fl) < 0.5f)
        b -= 1;
    // b is in [-1, n] (the coordinate is clamped into [0, n]): two selects wrap it
    const int n = g.n[k];
    b += b < 0 ? n : 0;
    b -= b >= n ? n : 0;
    return g.T_shift >= 0 ? (b >> g.T_shift) : (b / g.T);
}

struct PermArgs {
    const float *in[MAX_ARRAYS];
    float *out[MAX_ARRAYS];
    int n;
};

// State of the incremental path between its planning and its move.
struct IncGeom {
    KeyGeom g;
    uint32_t ntiles;
    const uint32_t *prev_off;
    int64_t count;
    const uint32_t *cum;  // [ntiles + 1] chunk numbering of the source slices
    const ChunkEntry *map;  // [nchunks] source tile and range of each chunk
    uint32_t *cnt;        // [nchunks][NDIR] particles per direction; then prefix over chunks
    // per tile, direction-major, so that threads of consecutive tiles touch
    // consecutive words:
    uint32_t *tcnt;       // [NDIR][ntiles] per source tile
    uint32_t *tpre;       // [NDIR][ntiles] prefix over a new tile's sources
    uint32_t *flag;       // non-zero: the general path takes over
};

__device__ inline void tile_coords(uint32_t t, const KeyGeom &g, int *c)
{
    c[0] = (int)(t % (uint32_t)g.nt[0]);
    c[1] = (int)((t / (uint32_t)g.nt[0]) % (uint32_t)g.nt[1]);
    c[2] = (int)(t / ((uint32_t)g.nt[0] * (uint32_t)g.nt[1]));
}

__device__ inline uint32_t tile_index(const int *c, const KeyGeom &g)
{
    return (uint32_t)c[0] + (uint32_t)g.nt[0] * ((uint32_t)c[1] + (uint32_t)g.nt[1] * (uint32_t)c[2]);
}

// New tile reached from source coordinates sc by direction dir.
__device__ inline uint32_t dest_tile(const int *sc, int dir, const KeyGeom &g)
{
    int c[3];
    c[0] = wrap_index(sc[0] + dir % 3 - 1, g.nt[0]);
    c[1] = wrap_index(sc[1] + (dir / 3) % 3 - 1, g.nt[1]);
    c[2] = wrap_index(sc[2] + dir / 9 - 1, g.nt[2]);
    return tile_index(c, g);
}

// Lanes of this wave whose `bits`-bit digit equals mine (among valid lanes).
template <int BITS>
__device__ inline uint64_t peer_mask(uint32_t digit, bool valid)
{
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
        const bool bit = (digit >> b) & 1u;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

// Direction index of the new tile coordinate t relative to source s on one
// axis of nt tiles: 0, 1, 2 for -1, 0, +1; -1 if further.  On an axis of two
// tiles only 0 and +1 are distinct, on an axis of one tile only 0.
__device__ inline int axis_dir(int t, int s, int nt)
{
    int d = t - s;  // in (-nt, nt)
    d += d < 0 ? nt : 0;
    // selects, not branches: 0 wins over 1 and 1 over nt - 1 (nt <= 2)
    int r = d == nt - 1 ? 0 : -1;
    r = d == 1 ? 2 : r;
    return d == 0 ? 1 : r;
}

template <int DIM, int ORDER>
__device__ inline int particle_dir(float x0, float x1, float x2, const KeyGeom &g, const int *sc)
{
    const float xs[3] = {x0, x1, x2};
    int dir = 0, mul = 1;
    bool far = false;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        int d = 1;  // unused axes: direction 0
        if (k < DIM) {
            d = axis_dir(tile_coord<ORDER>(xs[k], g, k), sc[k], g.nt[k]);
            far |= d < 0;
        }
        dir += mul * (d < 0 ? 0 : d);
        mul *= 3;
    }
    return far ? -1 : dir;
}

// particle_dir where n, T and n / T >= 4 are powers of two on every used axis
// (KeyGeom::pow2; four tiles or more keep -1, 0, +1 apart): the periodic wraps of the node and of the tile difference
// are masks, some 28 vector instructions per particle instead of about 66.
// The first support node is floor(x) (CIC) or floor(x - 1/2) (TSC: the node
// below when the fraction is under 1/2; x - 1/2 is exact or rounds only for
// x < 1/4, where the floor is -1 either way), x clamped into [0, n] as in
// tile_coord, so both give the same tile.
template <int DIM, int ORDER>
__device__ inline int particle_dir_pow2(float x0, float x1, float x2, const KeyGeom &g,
                                        const int *sc)
{
    const float xs[3] = {x0, x1, x2};
    int dir = 0, mul = 1;
    uint32_t worst = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        uint32_t d = 1;  // unused axes: direction 0
        if (k < DIM) {
            const float xf = clamp_coord(xs[k], g.nf[k]);
            const int b = (int)floorf(ORDER == 2 ? xf - 0.5f : xf);
            const uint32_t t = ((uint32_t)b & (uint32_t)(g.n[k] - 1)) >> g.T_shift;
            d = (t - (uint32_t)sc[k] + 1u) & (uint32_t)(g.nt[k] - 1);
            worst = max(worst, d);
        }
        dir += mul * (int)d;
        mul *= 3;
    }
    return worst > 2u ? -1 : dir;
}

// The direction of a particle: particle_dir_pow2 where the geometry allows.
template <int DIM, int ORDER>
__device__ inline int tile_dir(float x0, float x1, float x2, const KeyGeom &g, const int *sc)
{
    return g.pow2 ? particle_dir_pow2<DIM, ORDER>(x0, x1, x2, g, sc)
                  : particle_dir<DIM, ORDER>(x0, x1, x2, g, sc);
}

// One 64-particle step of a wave's in-order walk through a chunk: the new
// slot of each lane's particle (lanes with ok set; dir in [0, NDIR)), from the
// wave's next free slot per direction run[] in LDS, advanced past this step.
// Particles keep their order within each direction, so the slots are those of
// a stable counting sort.  Most particles stay in their tile: one ballot ranks
// those, and the few leavers are ranked one direction at a time (a loop over
// the distinct directions present, wave-uniform).  Wave-uniform control flow
// only.
__device__ inline uint32_t walk_slot(uint32_t *run, int dir, bool ok)
{
    const uint64_t lt = lanemask_lt();
    const bool stays = ok && dir == DIR_STAY;
    const uint64_t stay = __ballot(stays);
    uint64_t left = __ballot(ok && dir != DIR_STAY);
    const uint32_t stay_base = run[DIR_STAY];
    uint32_t pos = stay_base + (uint32_t)__popcll(stay & lt);
    while (left) {
        const int l = __builtin_amdgcn_readfirstlane(__ffsll((long long)left) - 1);
        const int d0 = __builtin_amdgcn_readlane(dir, l);
        const bool mine = ok && dir == d0;
        const uint64_t m = __ballot(mine);
        const uint32_t b = run[d0];
        if (mine)
            pos = b + (uint32_t)__popcll(m & lt);
        __builtin_amdgcn_wave_barrier();
        if (lane_id() == l)
            run[d0] = b + (uint32_t)__popcll(m);
        __builtin_amdgcn_wave_barrier();
        left &= ~m;
    }
    if (lane_id() == 0 && stay)
        run[DIR_STAY] = stay_base + (uint32_t)__popcll(stay);
    __builtin_amdgcn_wave_barrier();
    return pos;
}

// Start of chunk c of a tile slice of L particles split into nch balanced
// chunks (the split of the incremental sort).
__device__ inline uint32_t chunk_start(uint32_t c, uint32_t L, uint32_t nch)
{
    return (uint32_t)(((uint64_t)L * c) / nch);
}

// Output slot base of every direction of incremental chunk `chunk` (global
// chunk number) of source tile `tile`: off[new tile] + the tile's prefix among
// the new tile's sources + the chunk's prefix among the tile's chunks.
__device__ inline uint32_t move_base(const IncGeom &a, const uint32_t *off, uint32_t tile,
                                     uint32_t chunk, int dir)
{
    int sc[3];
    tile_coords(tile, a.g, sc);
    const uint32_t t = dest_tile(sc, dir, a.g);
    return off[t] + a.tpre[(size_t)dir * a.ntiles + tile] + a.cnt[(size_t)chunk * NDIR + dir];
}

// The move stage of the incremental path, replaceable by a caller of
// tile_sort_impl: launched after the new tile offsets exist, in place of the
// plain move kernel.  `off` holds the new offsets; `nwork` is the launch size
// of the incremental kernels (chunks, some without work).
struct MoveHook {
    pcg_status (*launch)(void *ctx, const IncGeom &a, const uint32_t *off, uint32_t nwork,
                         const PermArgs &arr, hipStream_t st);
    void *ctx;
};

// pcg_tile_sort with an optional hook for the incremental path's move stage.
// `incremental_taken` (may be NULL) reports whether the incremental path was
// enqueued (its device flag may still hand the work to the general path).
pcg_status tile_sort_impl(const pcg_grid *grid, int32_t order, int32_t T, int64_t count,
                          const float *const key_x[3], int32_t n_arrays,
                          const float *const in_arrays[], float *const out_arrays[],
                          uint32_t *perm, uint32_t *sorted_keys, uint32_t *tile_offsets,
                          const pcg_tile *prev, void *workspace, size_t workspace_bytes,
                          hipStream_t st, const MoveHook *hook, bool *incremental_taken);

// Bytes of sort workspace (the same as pcg_sort_workspace_bytes; 0 if invalid).
size_t sort_workspace_bytes(const pcg_grid *grid, int64_t count, int32_t T);

}  // namespace pcg
