// deposit.hip -- current deposit J_c += q w v_c W(x - x_g) ([TD] Entity wiki
// "Tiled current deposit"; B-spline weights from the mass-matrix paper §2.3
// Eq.(12)).
//
// Tiled path ([TD] "How a tile deposit runs"): one work-group per tile (or per
// chunk of a heavy tile) zeroes an LDS scratch window of TE = T + order + 2D
// nodes per used axis (D nodes of drift below the tile origin, D + order
// above), adds every particle of its slice into it with LDS atomics (exact
// integer fixed-point sums, see k_deposit_tiled), then adds each non-zero
// scratch value to J with one global atomic, wrapping node indices
// periodically.  A particle whose support does not fit the window is deposited
// directly to J with global atomics (the escape valve, [TD] "Correctness is
// independent of the halo"), from a queue the work-group drains after its
// chunk.
// Flat path ([TD] "The two paths", flat column): one thread per particle,
// (order+1)^dim x 3 global atomics -- used with no layout and for the tail.
#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "layout.hpp"
#include "regroup.hpp"

namespace pcg {
namespace {

constexpr size_t LDS_LIMIT = 160 * 1024;

// Particles each thread of the tiled kernel keeps in flight.
#ifndef DEPOSIT_UNROLL
#define DEPOSIT_UNROLL 4
#endif

struct DepArgs {
    int n[3];
    float nf[3];
    int T, D, TE;
    int nt[3];
    uint32_t ntiles;
    int vol;  // TE^dim
    const float *x[3];
    const float *v[3];
    const float *q;
    const float *w;
    float *J;
    int64_t ng;
    const uint32_t *tile_offsets;
    int64_t n_part;
    const uint32_t *chunk_cum;   // [ntiles + 1] work items before each tile
    const ChunkEntry *chunk_map;  // [nwork] tile and range of each work item
    uint32_t *chunk_part;        // scratch of the chunk prefix
    uint32_t chunk;
    unsigned long long *n_escaped;
    int fb64;  // tiled: the packed scratch falls back to 64-bit sums (else fp32)
    uint32_t qoff, qcap;  // tiled: byte offset and capacity of the LDS queue of
                          // particles deposited with global atomics
    uint32_t moff, mcap;  // fused pass: the same for the queue of particles
                          // that change tile
    uint32_t xcd_run;     // work items per XCD run (xcd_item); 0: plain order
};

// The regrouping half of the fused pass: every particle the deposit loads is
// also written to its slot in the next tile layout, as the incremental tile
// sort's move stage would (same slots, so the same result).
constexpr uint32_t MOVE_DEPOSIT_CHUNK = 32768;  // largest deposit chunk when moving
constexpr int MAX_WAVES = 8;                    // waves of a tiled work-group (512 threads)

struct MoveArgs {
    IncGeom inc;
    const uint32_t *off;  // the new tile offsets
    float *out[8];        // new arrays of x[0..dim), v[0..3), q, w
    uint32_t group;       // incremental chunks per deposit work item
};

// One axis of the shape: first support node b, unwrapped (in [-1, n] for a
// coordinate clamped into [0, n]), and order+1 weights.
template <int ORDER>
__device__ inline int shape_axis_raw(float xraw, float nf, float *W)
{
    const float x = clamp_coord(xraw, nf);
    const float fl = floorf(x);
    const float xi = x - fl;
    int b = (int)fl;
    if (ORDER == 1) {
        W[0] = 1.0f - xi;
        W[1] = xi;
    } else {
        float d;
        if (xi < 0.5f) {
            b -= 1;
            d = xi;
        } else {
            d = xi - 1.0f;
        }
        const float lo = 0.5f - d, hi = 0.5f + d;
        W[0] = 0.5f * lo * lo;
        W[1] = 0.75f - d * d;
        W[2] = 0.5f * hi * hi;
    }
    return b;
}

// v mod n for v in (-n, 2n).
__device__ inline int wrap_once(int v, int n)
{
    v += v < 0 ? n : 0;
    return v - (v >= n ? n : 0);
}

// One axis of the shape: first support node b (wrapped) and order+1 weights.
template <int ORDER>
__device__ inline int shape_axis(float xraw, float nf, int n, float *W)
{
    const float x = clamp_coord(xraw, nf);
    const float fl = floorf(x);
    const float xi = x - fl;
    int b = (int)fl;
    if (ORDER == 1) {
        W[0] = 1.0f - xi;
        W[1] = xi;
    } else {
        float d;
        if (xi < 0.5f) {
            b -= 1;
            d = xi;
        } else {
            d = xi - 1.0f;
        }
        const float lo = 0.5f - d, hi = 0.5f + d;
        W[0] = 0.5f * lo * lo;
        W[1] = 0.75f - d * d;
        W[2] = 0.5f * hi * hi;
    }
    return wrap_once(b, n);  // b in [-1, n]
}

// All (order+1)^dim global atomics of one particle; b[k] is wrapped into
// [0, n_k) and order < n_k, so each node index wraps with one subtraction.
template <int DIM, int ORDER>
__device__ __attribute__((always_inline)) inline void deposit_global(const DepArgs &a, const int *b,
                                                                     float W[3][ORDER + 1],
                                                                     const float *amp)
{
    auto wrap_up = [](int v, int n) { return v - (v >= n ? n : 0); };
    constexpr int M = ORDER + 1;
    constexpr int MY = DIM > 1 ? M : 1, MZ = DIM > 2 ? M : 1;
#pragma unroll
    for (int az = 0; az < MZ; ++az) {
        const int gz = DIM > 2 ? wrap_up(b[2] + az, a.n[2]) : 0;
#pragma unroll
        for (int ay = 0; ay < MY; ++ay) {
            const int gy = DIM > 1 ? wrap_up(b[1] + ay, a.n[1]) : 0;
            const float wyz = (DIM > 1 ? W[1][ay] : 1.0f) * (DIM > 2 ? W[2][az] : 1.0f);
#pragma unroll
            for (int ax = 0; ax < M; ++ax) {
                const int gx = wrap_up(b[0] + ax, a.n[0]);
                const int64_t g = gx + (int64_t)a.n[0] * (gy + (int64_t)a.n[1] * gz);
                const float wt = W[0][ax] * wyz;
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    atomic_add_f32(&a.J[c * a.ng + g], amp[c] * wt);
            }
        }
    }
}

template <int DIM, int ORDER>
__global__ __launch_bounds__(1024) void k_deposit_flat(DepArgs a, int64_t begin, int64_t end)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < end; p += stride) {
        float W[3][ORDER + 1];
        int b[3] = {0, 0, 0};
#pragma unroll
        for (int k = 0; k < DIM; ++k)
            b[k] = shape_axis<ORDER>(a.x[k][p], a.nf[k], a.n[k], W[k]);
        const float qw = a.q[p] * a.w[p];
        const float amp[3] = {qw * a.v[0][p], qw * a.v[1][p], qw * a.v[2][p]};
        deposit_global<DIM, ORDER>(a, b, W, amp);
    }
}

// Accumulator of the LDS scratch tile.  LDS float atomics (ds_add_f32) are
// about 30x slower than integer LDS atomics on gfx950, so the scratch holds
// integer fixed-point sums: a work-group picks a power-of-two scale 2^S, every
// product q w v_c W 2^S is rounded once to the nearest integer and added with
// integer atomics.  The in-tile sums are then exact
// and independent of the order of the adds.
//   ACC_PACKED  two 32-bit sums per 64-bit word: x in the low half, y in the
//               high half (added as y 2^32 + x, so a negative x borrows from y
//               and the flush undoes it), z in a 32-bit word.  16 atomics per
//               CIC particle instead of 24 64-bit ones.  A per-cell particle
//               count proves afterwards that no 32-bit sum can have
//               overflowed; a work-group that cannot prove it runs its chunk
//               again at a scale the counts allow (or, if that scale would be
//               too coarse, into ACC_FIXED, or ACC_FLOAT if that does not fit).
//   ACC_FIXED   three 64-bit sums.
//   ACC_FLOAT   fp32 LDS atomics (order-dependent rounding).
enum AccMode { ACC_PACKED = 0, ACC_FIXED = 1, ACC_FLOAT = 2 };

// a*b (formed in fp32) rounded to the nearest integer, ties to even; valid
// for |a*b| < 2^31.
__device__ inline int round_prod(float a, float b)
{
    return __float2int_rn(a * b);
}

// a*b rounded to the nearest integer, ties to even, with one FMA: a*b + 1.5 2^23
// is formed exactly and rounded once to a float whose unit is 1; valid for
// |a*b| < 2^22.
__device__ inline int round_prod_fma(float a, float b)
{
    return __float_as_int(__builtin_fmaf(a, b, 12582912.0f)) - 0x4B400000;
}

// The packed sums of CIC scratch keep every product below 2^22 and round with
// round_prod_fma; TSC (smaller weights, more rounding per node) allows up to
// 2^24 and rounds with round_prod.
template <int ORDER>
__device__ inline int round_packed(float a, float b)
{
    return ORDER == 1 ? round_prod_fma(a, b) : round_prod(a, b);
}

// Per work-group constants of a chunk.
struct TileCtx {
    int origin[3];
    int TE, vol, cedge;     // scratch edge and volume, cells per axis in the window
    float scale, inv_scale; // 2^S and 2^-S
    float lo_ok, hi_ok;     // admitted range of the largest scaled |q w v_c|
};

// LDS views of the scratch tile (all start at the dynamic LDS base), and the
// queue of particles that take global atomics (after the scratch).
struct Scratch {
    unsigned long long *xy;  // PACKED [vol]
    uint32_t *z;             // PACKED [vol]
    uint32_t *cnt;           // PACKED [cedge^dim] particles per base cell
    unsigned long long *acc64;  // FIXED [3][vol]
    float *acc32;               // FLOAT [3][vol]
    float *queue;               // [qcap][QUEUE_FLOATS]: raw x[3], q w v[3]
    uint32_t *qn;               // entries claimed (may exceed qcap)
    uint32_t qcap;
    float *mq;                  // [mcap][MQ_WORDS]: new slot, then the fields
    uint32_t *mn;
    uint32_t mcap;
};

// A queued particle: its raw coordinates and its amplitude q w v_c.
constexpr int QUEUE_FLOATS = 6;
constexpr uint32_t QUEUE_MAX = 512;  // entries per work-group (12 KiB)
// A particle of the fused pass that changes tile: its slot in the new layout
// and its x[dim], v[3], q, w.
constexpr int MQ_WORDS = 9;
constexpr uint32_t MOVE_QUEUE_MAX = 1024;  // entries per work-group (36 KiB)

// A particle's support in a work-group's window: its first support node b
// (unwrapped), the weights, the scratch start s (periodic offset of b from the
// window's low edge) and whether the stencil leaves the window.
template <int ORDER>
struct Support {
    float W[3][ORDER + 1];
    int b[3];
    int s[3];
    bool esc;
};

template <int DIM, int ORDER>
__device__ __attribute__((always_inline)) inline Support<ORDER> support_of(const DepArgs &a,
                                                                           const TileCtx &c,
                                                                           const float *xs)
{
    Support<ORDER> sp;
    const int last = a.T - 1 + 2 * a.D;  // largest scratch start that keeps the stencil inside
    sp.esc = false;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        sp.b[k] = 0;
        sp.s[k] = 0;
    }
#pragma unroll
    for (int k = 0; k < DIM; ++k) {
        sp.b[k] = shape_axis_raw<ORDER>(xs[k], a.nf[k], sp.W[k]);
        // b in [-1, n], origin in [0, n - T], so one wrap suffices
        sp.s[k] = wrap_once(sp.b[k] - c.origin[k] + a.D, a.n[k]);
        sp.esc |= sp.s[k] > last;
    }
    return sp;
}

// Direction (0..26) of the tile holding a particle's first support node,
// relative to the work-group's tile, from the support's scratch start: along
// each axis the tile below (0), the same (1) or above (2).  Valid when every
// used axis has at least three tiles and D < T and the particle moved at most
// one tile: then s < D or s >= n - T + D means the tile below (the second
// after a periodic wrap), s < D + T the same tile, else the tile above.
template <int DIM, int ORDER>
__device__ inline int support_dir(const DepArgs &a, const Support<ORDER> &sp)
{
    int dir = 0, mul = 1;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        int d = 1;
        if (k < DIM) {
            const int sk = sp.s[k];
            d = (sk < a.D || sk >= a.n[k] - a.T + a.D) ? 0 : (sk < a.D + a.T ? 1 : 2);
        }
        dir += mul * d;
        mul *= 3;
    }
    return dir;
}

// One particle: its support, then either the LDS scratch (mode MODE) or, if
// its stencil leaves the window or its amplitude is outside the admitted
// range, global atomics.  `again` marks the fallback pass: particles that
// went to global memory in the first pass are skipped.  Returns 1 for an
// escape (stencil outside the window) on the first pass.
template <int DIM, int ORDER, int MODE, int TEC>
__device__ __attribute__((always_inline)) inline uint32_t deposit_supported(
    const DepArgs &a, const TileCtx &c, const Scratch &sc, const Support<ORDER> &sp,
    const float *xs, const float *vv, float cq, float cw, bool again)
{
    constexpr int M = ORDER + 1;
    constexpr int MY = DIM > 1 ? M : 1, MZ = DIM > 2 ? M : 1;
    const int TE = TEC > 0 ? TEC : c.TE;
    const int vol = TEC > 0 ? (DIM == 3 ? TEC * TEC * TEC : (DIM == 2 ? TEC * TEC : TEC)) : c.vol;
    const float qw = cq * cw;
    float W[3][M];
    int b[3], s[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        b[k] = sp.b[k];
        s[k] = sp.s[k];
#pragma unroll
        for (int j = 0; j < M; ++j)
            W[k][j] = k < DIM ? sp.W[k][j] : 1.0f;
    }
    const bool esc = sp.esc;
    const float qws = qw * c.scale;
    float amp[3] = {qws * vv[0], qws * vv[1], qws * vv[2]};
    const float amax = fmaxf(fabsf(amp[0]), fmaxf(fabsf(amp[1]), fabsf(amp[2])));
    if (amax == 0.0f)  // deposits nothing, but an escape is still an escape
        return (esc && !again) ? 1u : 0u;
    const bool in_lds = !esc && amax >= c.lo_ok && amax < c.hi_ok;
    if (!in_lds) {
        if (again)
            return 0u;
#pragma unroll
        for (int k = 0; k < 3; ++k)
            amp[k] *= c.inv_scale;  // exact: power-of-two scale
        // queue it for the work-group's global pass after the chunk (a wave
        // would otherwise run this particle's global atomics with every other
        // lane idle); straight to global memory when the queue is full
        const uint32_t slot = sc.qcap ? atomicAdd(sc.qn, 1u) : 0u;
        if (slot < sc.qcap) {
            float *e = sc.queue + (size_t)slot * QUEUE_FLOATS;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                e[k] = k < DIM ? xs[k] : 0.0f;
                e[3 + k] = amp[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < DIM; ++k)
                b[k] = wrap_once(b[k], a.n[k]);
            deposit_global<DIM, ORDER>(a, b, W, amp);
        }
        return esc ? 1u : 0u;
    }
    // amp_c * W_x first, then one product per (node, component)
    float ampx[3][M];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int ax = 0; ax < M; ++ax)
            ampx[k][ax] = amp[k] * W[0][ax];
    // window offsets: in [0, TE) on this path
    const int sbase = DIM == 3 ? mad24(mad24(s[2], TE, s[1]), TE, s[0])
                               : (DIM == 2 ? mad24(s[1], TE, s[0]) : s[0]);
    if (MODE == ACC_PACKED) {
        const int cell = DIM == 3 ? mad24(mad24(s[2], c.cedge, s[1]), c.cedge, s[0])
                                  : (DIM == 2 ? mad24(s[1], c.cedge, s[0]) : s[0]);
        __hip_atomic_fetch_add(&sc.cnt[cell], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
#pragma unroll
    for (int az = 0; az < MZ; ++az) {
#pragma unroll
        for (int ay = 0; ay < MY; ++ay) {
            const int row = sbase + (DIM == 3 ? (az * TE + ay) * TE : ay * TE);
            const float wyz = (DIM > 1 ? W[1][ay] : 1.0f) * (DIM > 2 ? W[2][az] : 1.0f);
#pragma unroll
            for (int ax = 0; ax < M; ++ax) {
                const int idx = row + ax;
                if (MODE == ACC_PACKED) {
                    const int ix = round_packed<ORDER>(ampx[0][ax], wyz);
                    const int iy = round_packed<ORDER>(ampx[1][ax], wyz);
                    const int iz = round_packed<ORDER>(ampx[2][ax], wyz);
                    const uint32_t hi = (uint32_t)(iy + (ix >> 31));
                    const unsigned long long v = ((unsigned long long)hi << 32) | (uint32_t)ix;
                    __hip_atomic_fetch_add(&sc.xy[idx], v, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_fetch_add(&sc.z[idx], (uint32_t)iz, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                } else {
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        if (MODE == ACC_FIXED) {
                            const long long f = (long long)round_prod(ampx[k][ax], wyz);
                            __hip_atomic_fetch_add(&sc.acc64[k * vol + idx], (unsigned long long)f,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        } else {
                            __hip_atomic_fetch_add(&sc.acc32[k * vol + idx],
                                                   ampx[k][ax] * wyz * c.inv_scale,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        }
                    }
                }
            }
        }
    }
    return 0u;
}

template <int DIM, int ORDER, int MODE, int TEC>
__device__ __attribute__((always_inline)) inline uint32_t deposit_one(const DepArgs &a, const TileCtx &c, const Scratch &sc,
                                       const float *xs, const float *vv, float cq, float cw,
                                       bool again)
{
    const Support<ORDER> sp = support_of<DIM, ORDER>(a, c, xs);
    return deposit_supported<DIM, ORDER, MODE, TEC>(a, c, sc, sp, xs, vv, cq, cw, again);
}

// Global node index of scratch node i of the window (periodic wrap).
template <int DIM>
__device__ inline int64_t window_node(const DepArgs &a, const TileCtx &c, int i)
{
    int sx = i, sy = 0, sz = 0;
    if (DIM > 1) {
        sx = i % c.TE;
        const int r = i / c.TE;
        sy = DIM > 2 ? r % c.TE : r;
        sz = DIM > 2 ? r / c.TE : 0;
    }
    // origin - D + s lies in [-D, n + order + D) and D + order < n
    const int gx = wrap_once(c.origin[0] - a.D + sx, a.n[0]);
    const int gy = DIM > 1 ? wrap_once(c.origin[1] - a.D + sy, a.n[1]) : 0;
    const int gz = DIM > 2 ? wrap_once(c.origin[2] - a.D + sz, a.n[2]) : 0;
    return gx + (int64_t)a.n[0] * (gy + (int64_t)a.n[1] * gz);
}

// Flush: one global atomic per non-zero scratch value.
template <int DIM, int MODE>
__device__ __attribute__((always_inline)) inline void flush_scratch(const DepArgs &a, const TileCtx &c, const Scratch &sc)
{
    for (int i = threadIdx.x; i < c.vol; i += blockDim.x) {
        float val[3];
        if (MODE == ACC_PACKED) {
            const unsigned long long p = sc.xy[i];
            const int ix = (int)(uint32_t)p;
            const int iy = (int)(uint32_t)((p - (unsigned long long)(long long)ix) >> 32);
            const int iz = (int)sc.z[i];
            val[0] = (float)ix * c.inv_scale;
            val[1] = (float)iy * c.inv_scale;
            val[2] = (float)iz * c.inv_scale;
        } else {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (MODE == ACC_FIXED)
                    val[k] = (float)((double)(long long)sc.acc64[k * c.vol + i] * (double)c.inv_scale);
                else
                    val[k] = sc.acc32[k * c.vol + i];
            }
        }
        if (val[0] == 0.0f && val[1] == 0.0f && val[2] == 0.0f)
            continue;
        const int64_t g = window_node<DIM>(a, c, i);
#pragma unroll
        for (int k = 0; k < 3; ++k)
            if (val[k] != 0.0f)
                atomic_add_f32(&a.J[k * a.ng + g], val[k]);
    }
}

// The queued particles' global atomics, one (particle, stencil node) pair per
// thread: the same weights and products as deposit_global.  Call after a
// barrier that follows the last queue write.
template <int DIM, int ORDER>
__device__ __attribute__((always_inline)) inline void drain_queue(const DepArgs &a,
                                                                  const Scratch &sc)
{
    constexpr int M = ORDER + 1;
    constexpr int NS = DIM == 3 ? M * M * M : (DIM == 2 ? M * M : M);
    auto wrap_up = [](int v, int n) { return v - (v >= n ? n : 0); };
    const uint32_t n = min(*sc.qn, sc.qcap);
    for (uint32_t i = threadIdx.x; i < n * NS; i += blockDim.x) {
        const float *e = sc.queue + (size_t)(i / NS) * QUEUE_FLOATS;
        const int node = (int)(i % NS);
        const int off[3] = {node % M, (node / M) % M, node / (M * M)};
        int g[3] = {0, 0, 0};
        float wk[3] = {1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int k = 0; k < DIM; ++k) {
            float W[M];
            const int b = shape_axis<ORDER>(e[k], a.nf[k], a.n[k], W);
            float w = W[0];
#pragma unroll
            for (int j = 1; j < M; ++j)
                w = off[k] == j ? W[j] : w;
            wk[k] = w;
            g[k] = wrap_up(b + off[k], a.n[k]);
        }
        const int64_t gi = g[0] + (int64_t)a.n[0] * (g[1] + (int64_t)a.n[1] * g[2]);
        const float wt = wk[0] * ((DIM > 1 ? wk[1] : 1.0f) * (DIM > 2 ? wk[2] : 1.0f));
#pragma unroll
        for (int c = 0; c < 3; ++c)
            atomic_add_f32(&a.J[c * a.ng + gi], e[3 + c] * wt);
    }
}

// The staged particles of the fused pass, one per thread, to their new slots.
// Call after a barrier that follows the last staging write.
template <int DIM>
__device__ __attribute__((always_inline)) inline void drain_moves(const MoveArgs &m,
                                                                  const Scratch &sc)
{
    const uint32_t n = min(*sc.mn, sc.mcap);
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
        const float *e = sc.mq + (size_t)i * MQ_WORDS;
        const uint32_t pos = reinterpret_cast<const uint32_t *>(e)[0];
#pragma unroll
        for (int k = 0; k < DIM + 5; ++k)
            m.out[k][pos] = e[1 + k];
    }
}

// One unconditional wait for a group of N particles' values (loaded an
// iteration ago), placed before any branch: the per-particle branches then need
// no waits of their own, and counter-based waits placed after stores there
// would also drain the next group's loads.
template <int N>
__device__ __attribute__((always_inline)) inline void wait_values(float (*x)[3], float (*v)[3],
                                                                  float *q, float *w)
{
#pragma unroll
    for (int u = 0; u < N; ++u)
        asm volatile("" ::"v"(x[u][0]), "v"(x[u][1]), "v"(x[u][2]), "v"(v[u][0]), "v"(v[u][1]),
                     "v"(v[u][2]), "v"(q[u]), "v"(w[u]));
}

// Bytes of LDS the packed scratch and its fallback need.
__host__ __device__ constexpr size_t packed_bytes(size_t vol, size_t ncell)
{
    return vol * 12 + ncell * 4;
}

// Tiled deposit of one chunk per work-group.  ACC is ACC_PACKED (falling back
// per work-group to ACC_FIXED when a.fb64, else ACC_FLOAT) or ACC_FLOAT.
template <int DIM, int ORDER, int ACC, int TEC, bool MOVE>
__global__ __launch_bounds__(512) void k_deposit_tiled(DepArgs a, MoveArgs m)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ uint32_t s_tile, s_lo, s_hi, s_esc, s_maxbits, s_move, s_maxcnt, s_qn, s_mn;
    // MOVE: output slot base per (incremental chunk overlapped, direction), and
    // the end slot of each of those chunks
    // MOVE: each wave's next free slot per direction in the chunk it walks;
    // the work item's first incremental chunk (within the tile) and count
    __shared__ uint32_t s_run[MOVE ? MAX_WAVES : 1][32];
    __shared__ uint32_t s_c0, s_nsub;

    if (threadIdx.x == 0) {
        ChunkRange r = find_chunk(xcd_item(blockIdx.x, a.xcd_run), a.chunk_cum, a.chunk_map, a.ntiles);
        s_esc = 0;
        s_qn = 0;
        s_mn = 0;
        s_maxbits = 0;
        s_maxcnt = 0;
        s_move = MOVE && *m.inc.flag == 0u;
        s_c0 = 0;
        s_nsub = 0;
        if (MOVE && s_move && r.tile != UINT_MAX) {
            // the work item is `group` whole chunks of the incremental sort's
            // split of the tile (the same number of items per tile), so that
            // each wave can walk whole chunks in order
            const uint32_t t = r.tile;
            const uint32_t item = r.chunk - a.chunk_cum[t];
            const uint32_t nch = m.inc.cum[t + 1] - m.inc.cum[t];
            const uint32_t c0 = item * m.group, c1 = min(c0 + m.group, nch);
            const uint32_t p0 = (uint32_t)min((int64_t)m.inc.prev_off[t], m.inc.count);
            const uint32_t L = (uint32_t)min((int64_t)m.inc.prev_off[t + 1], m.inc.count) - p0;
            if (c0 < c1) {
                r.lo = p0 + chunk_start(c0, L, nch);
                r.hi = p0 + chunk_start(c1, L, nch);
                s_c0 = c0;
                s_nsub = c1 - c0;
            } else {
                r.tile = UINT_MAX;
            }
        }
        s_tile = r.tile;
        s_lo = r.lo;
        s_hi = r.hi;
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile == UINT_MAX)
        return;
    const uint32_t lo = s_lo, hi = s_hi;
    TileCtx c;
    {
        uint32_t t = tile;
#pragma unroll
        for (int k = 0; k < 3; ++k)
            c.origin[k] = 0;
#pragma unroll
        for (int k = 0; k < DIM; ++k) {
            c.origin[k] = (int)(t % (uint32_t)a.nt[k]) * a.T;
            t /= (uint32_t)a.nt[k];
        }
    }
    c.TE = TEC > 0 ? TEC : a.TE;
    c.vol = TEC > 0 ? (DIM == 3 ? TEC * TEC * TEC : (DIM == 2 ? TEC * TEC : TEC)) : a.vol;
    c.cedge = a.T + 2 * a.D;
    int ncell = 1;
#pragma unroll
    for (int k = 0; k < DIM; ++k)
        ncell *= c.cedge;
    Scratch sc;
    sc.xy = reinterpret_cast<unsigned long long *>(smem);
    sc.z = reinterpret_cast<uint32_t *>(smem + (size_t)c.vol * 8);
    sc.cnt = reinterpret_cast<uint32_t *>(smem + (size_t)c.vol * 12);
    sc.acc64 = reinterpret_cast<unsigned long long *>(smem);
    sc.acc32 = reinterpret_cast<float *>(smem);
    sc.queue = reinterpret_cast<float *>(smem + a.qoff);
    sc.qn = &s_qn;
    sc.qcap = a.qcap;
    sc.mq = reinterpret_cast<float *>(smem + a.moff);
    sc.mn = &s_mn;
    sc.mcap = MOVE ? a.mcap : 0u;

    const bool move = MOVE && s_move != 0u;

    // zero the scratch; scale from the first batch: largest |q w v_c|
    if (ACC == ACC_PACKED) {
        const int words = c.vol * 3 + ncell;  // xy (2 words each), z, cnt
        uint32_t *w32 = reinterpret_cast<uint32_t *>(smem);
        for (int i = threadIdx.x; i < words; i += blockDim.x)
            w32[i] = 0u;
    } else {
        for (int i = threadIdx.x; i < 3 * c.vol; i += blockDim.x)
            sc.acc32[i] = 0.0f;
    }
    {
        float mx = 0.0f;
        const uint32_t p = lo + threadIdx.x;
        if (p < hi) {
            const float qw = fabsf(a.q[p] * a.w[p]);
            mx = qw * fmaxf(fabsf(a.v[0][p]), fmaxf(fabsf(a.v[1][p]), fabsf(a.v[2][p])));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
        if (lane_id() == 0 && mx > 0.0f && mx <= 3.0e38f)
            atomicMax(&s_maxbits, __float_as_uint(mx));  // non-negative: int order = float order
    }
    __syncthreads();
    // Scale.  Packed sums: the largest scaled product stays below 2^h, the
    // first batch's largest in [2^(h-1), 2^h); h leaves room for the particles
    // of (order+1)^dim cells at twice the chunk's mean density in a 32-bit sum
    // (the count check below turns this into a guarantee), at most 22 (CIC,
    // see round_packed) or 24 (TSC).  When
    // that leaves fewer than PACKED_MIN_BITS bits for the rounding (dense
    // chunks; the TSC weights are small, so it needs more), the chunk takes
    // 64-bit sums from the start if they fit: first batch's largest in
    // [2^23, 2^24), products below 2^30.
    constexpr int PACKED_MIN_BITS = ORDER == 1 ? 21 : 23;
    bool fixed_first = false;
    {
        int h = 24;
        if (ACC == ACC_PACKED) {
            int tcells = 1;
            for (int k = 0; k < DIM; ++k)
                tcells *= a.T;
            constexpr int NS = DIM == 3 ? (ORDER + 1) * (ORDER + 1) * (ORDER + 1)
                                        : (DIM == 2 ? (ORDER + 1) * (ORDER + 1) : ORDER + 1);
            const uint64_t nb = (uint64_t)NS * ((2ull * (hi - lo)) / tcells + 1) + 1;
            const int lg = 64 - __clzll((long long)(nb - 1));  // ceil(log2(nb))
            h = max(10, min(ORDER == 1 ? 22 : 24, 31 - lg));
            fixed_first = h < PACKED_MIN_BITS && a.fb64;
        }
        const float mx = __uint_as_float(s_maxbits);
        int S = 0;
        if (mx > 0.0f)
            S = (fixed_first ? 24 : h) - 1 - ilogbf(mx);
        S = max(-100, min(100, S));
        c.scale = ldexpf(1.0f, S);
        c.inv_scale = ldexpf(1.0f, -S);
        c.hi_ok = ldexpf(1.0f, fixed_first ? 30 : h);
        c.lo_ok = ldexpf(1.0f, fixed_first ? 8 : h - 16);
    }
    if (fixed_first) {
        // the 64-bit scratch reaches into the queues' LDS: no queues here
        sc.qcap = 0;
        sc.mcap = 0;
        for (int i = threadIdx.x; i < 3 * c.vol; i += blockDim.x)
            sc.acc64[i] = 0ull;
        __syncthreads();
    }

    // Each thread keeps U particles in flight: the next group's values load
    // while this group is weighed (and moved) and accumulated.
    constexpr int U = DEPOSIT_UNROLL;
    // Loads of particle p (clamped into the slice by the caller): a 32-bit
    // byte offset from each array's base (counts are below 2^30).
    auto load_one = [&](uint32_t p, float *x, float *v, float &q, float &w)
        __attribute__((always_inline)) {
        const uint32_t off = p * 4u;
        auto at = [off](const float *base) {
            return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + off);
        };
        x[0] = x[1] = x[2] = 0.f;
#pragma unroll
        for (int k = 0; k < DIM; ++k)
            x[k] = at(a.x[k]);
#pragma unroll
        for (int k = 0; k < 3; ++k)
            v[k] = at(a.v[k]);
        q = at(a.q);
        w = at(a.w);
    };
    // The chunk in an order of no consequence to the deposit: thread t takes
    // particles lo + t, lo + t + blockDim.x, ... (no moves).
    auto pass = [&](auto mode_tag, const TileCtx &cx, bool again) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_tag)::value;
        const uint32_t stride = blockDim.x;
        float nx[U][3], nv[U][3], nq[U], nw[U];
        // no branch around the loads: a lane past the slice reloads the
        // slice's last particle (never used), so the number of loads in flight
        // is fixed and the wait for one group leaves the next group's loads
        // outstanding
        auto load_group = [&](uint32_t base) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                load_one(min(base + u * stride, hi - 1), nx[u], nv[u], nq[u], nw[u]);
        };
        uint32_t esc_count = 0;
        load_group(lo + threadIdx.x);
        for (uint32_t base = lo + threadIdx.x; base < hi; base += U * stride) {
            float gx[U][3], gv[U][3], gq[U], gw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    gx[u][k] = nx[u][k];
                    gv[u][k] = nv[u][k];
                }
                gq[u] = nq[u];
                gw[u] = nw[u];
            }
            load_group(base + U * stride);
            wait_values<U>(gx, gv, gq, gw);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t p = base + u * stride;
                if (p >= hi)
                    break;
                esc_count += deposit_one<DIM, ORDER, MODE, TEC>(a, cx, sc, gx[u], gv[u], gq[u],
                                                                gw[u], again);
            }
        }
        if (esc_count)
            atomicAdd(&s_esc, esc_count);
    };

    // Particles per lane in flight in the walk (its slot bookkeeping needs
    // registers the plain pass does not).
    constexpr int UW = DIM == 3 && ORDER == 2 ? 2 : 3;
    // MOVE, first pass: the work item's incremental chunks (or, without the
    // incremental layout, balanced pieces of [lo, hi)) go to the waves in
    // turn; a wave walks each of its chunks in order, 64 U particles at a
    // time, so that it can give every particle its slot in the new layout
    // from its direction and its running count (as the incremental sort's
    // move does), deposits it, and stores it (or stages it, if it changes
    // tile).
    auto walk = [&](auto mode_tag, const TileCtx &cx) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_tag)::value;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
        const int nwaves = blockDim.x / WAVE;
        const uint32_t nsub = move ? s_nsub : (hi - lo + INC_CHUNK - 1) / INC_CHUNK;
        uint32_t p0 = 0, L = 0, nch = 0, g0 = 0;
        int tsc[3] = {0, 0, 0};
        if (move) {
            p0 = (uint32_t)min((int64_t)m.inc.prev_off[tile], m.inc.count);
            L = (uint32_t)min((int64_t)m.inc.prev_off[tile + 1], m.inc.count) - p0;
            g0 = m.inc.cum[tile];
            nch = m.inc.cum[tile + 1] - g0;
            tile_coords(tile, m.inc.g, tsc);
        }
        uint32_t *run = s_run[MOVE ? wave : 0];
        uint32_t esc_count = 0;
        // the direction from the support's window position (support_dir)
        // where every used axis has three tiles or more
        bool fastdir = a.D < a.T;
#pragma unroll
        for (int k = 0; k < DIM; ++k)
            fastdir = fastdir && a.nt[k] >= 3;
        for (uint32_t j = wave; j < nsub; j += nwaves) {
            uint32_t clo, chi;
            if (move) {
                clo = p0 + chunk_start(s_c0 + j, L, nch);
                chi = p0 + chunk_start(s_c0 + j + 1, L, nch);
                if (lane < NDIR)
                    run[lane] = move_base(m.inc, m.off, tile, g0 + s_c0 + j, lane);
                __builtin_amdgcn_wave_barrier();
            } else {
                clo = lo + (uint32_t)((uint64_t)(hi - lo) * j / nsub);
                chi = lo + (uint32_t)((uint64_t)(hi - lo) * (j + 1) / nsub);
            }
            float nx[UW][3], nv[UW][3], nq[UW], nw[UW];
            auto load_group = [&](uint32_t base) {
#pragma unroll
                for (int u = 0; u < UW; ++u)
                    load_one(min(base + u * WAVE + lane, chi - 1), nx[u], nv[u], nq[u], nw[u]);
            };
            load_group(clo);
            for (uint32_t base = clo; base < chi; base += UW * WAVE) {
                float gx[UW][3], gv[UW][3], gq[UW], gw[UW];
#pragma unroll
                for (int u = 0; u < UW; ++u) {
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        gx[u][k] = nx[u][k];
                        gv[u][k] = nv[u][k];
                    }
                    gq[u] = nq[u];
                    gw[u] = nw[u];
                }
                load_group(base + UW * WAVE);
                wait_values<UW>(gx, gv, gq, gw);
#pragma unroll
                for (int u = 0; u < UW; ++u) {
                    const uint32_t p = base + u * WAVE + lane;
                    const bool valid = p < chi;
                    const Support<ORDER> sp = support_of<DIM, ORDER>(a, cx, gx[u]);
                    if (move) {
                        // wave-uniform: the slot comes from the whole wave's
                        // directions
                        const int d = fastdir ? support_dir<DIM, ORDER>(a, sp)
                                              : tile_dir<DIM, ORDER>(gx[u][0], gx[u][1], gx[u][2],
                                                                     m.inc.g, tsc);
                        const bool ok = valid && d >= 0;  // d < 0 cannot occur: flag clear
                        const uint32_t pos = walk_slot(run, d, ok);
                        if (ok && pos < (uint64_t)m.inc.count) {
                            // a particle that changes tile is staged in LDS and
                            // written with the rest of its chunk's leavers after
                            // the pass: stored here, its lines would be written
                            // back piecemeal
                            bool staged = false;
                            if (d != DIR_STAY && sc.mcap) {
                                const uint32_t slot = atomicAdd(sc.mn, 1u);
                                if (slot < sc.mcap) {
                                    float *e = sc.mq + (size_t)slot * MQ_WORDS;
                                    reinterpret_cast<uint32_t *>(e)[0] = pos;
#pragma unroll
                                    for (int k = 0; k < DIM; ++k)
                                        e[1 + k] = gx[u][k];
#pragma unroll
                                    for (int k = 0; k < 3; ++k)
                                        e[1 + DIM + k] = gv[u][k];
                                    e[DIM + 4] = gq[u];
                                    e[DIM + 5] = gw[u];
                                    staged = true;
                                }
                            }
                            if (!staged) {
#pragma unroll
                                for (int k = 0; k < DIM; ++k)
                                    m.out[k][pos] = gx[u][k];
#pragma unroll
                                for (int k = 0; k < 3; ++k)
                                    m.out[DIM + k][pos] = gv[u][k];
                                m.out[DIM + 3][pos] = gq[u];
                                m.out[DIM + 4][pos] = gw[u];
                            }
                        }
                    }
                    if (valid)
                        esc_count += deposit_supported<DIM, ORDER, MODE, TEC>(
                            a, cx, sc, sp, gx[u], gv[u], gq[u], gw[u], false);
                }
            }
        }
        if (esc_count)
            atomicAdd(&s_esc, esc_count);
    };
    // the first pass of a kernel
    auto first = [&](auto mode_tag, const TileCtx &cx) __attribute__((always_inline)) {
        if constexpr (MOVE)
            walk(mode_tag, cx);
        else
            pass(mode_tag, cx, false);
    };

    if (ACC == ACC_PACKED && fixed_first) {
        first(std::integral_constant<int, ACC_FIXED>{}, c);
        __syncthreads();
        flush_scratch<DIM, ACC_FIXED>(a, c, sc);
        if (threadIdx.x == 0 && s_esc && a.n_escaped)
            atomicAdd(a.n_escaped, (unsigned long long)s_esc);
        return;
    }
    first(std::integral_constant<int, ACC>{}, c);
    __syncthreads();
    // the queues lie past the packed scratch, where a 64-bit rerun would
    // write: drain them now (the barrier of the count check below separates
    // the drains from any rerun)
    if (MOVE)
        drain_moves<DIM>(m, sc);
    drain_queue<DIM, ORDER>(a, sc);

    bool redo = false;
    uint32_t maxcnt = 0;
    constexpr int NS = DIM == 3 ? (ORDER + 1) * (ORDER + 1) * (ORDER + 1)
                                : (DIM == 2 ? (ORDER + 1) * (ORDER + 1) : ORDER + 1);
    if (ACC == ACC_PACKED) {
        // no 32-bit sum can have overflowed if every node's contributing cells
        // hold few enough particles: a node sums at most NS * maxcnt products,
        // each at most 2^h in magnitude after rounding
        uint32_t mc = 0;
        for (int i = threadIdx.x; i < ncell; i += blockDim.x)
            mc = max(mc, sc.cnt[i]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            mc = max(mc, (uint32_t)__shfl_xor((int)mc, o, WAVE));
        if (lane_id() == 0 && mc)
            atomicMax(&s_maxcnt, mc);
        __syncthreads();
        maxcnt = s_maxcnt;
        redo = (double)NS * (double)maxcnt * (double)c.hi_ok > 2147483647.0;
    }
    if (ACC == ACC_PACKED && redo) {
        // the chunk again, with the scale lowered so that the counts just
        // measured fit (the same particles are admitted: the range moves with
        // the scale); if that would cost too much precision, into 64-bit sums
        // at the first scale (or, where those do not fit the LDS, fp32 sums
        // once even the coarser packed pass would lose too much)
        const int h2 = min(ORDER == 1 ? 22 : 24,
                           (int)floor(log2(2147483647.0 / ((double)NS * (double)maxcnt))));
        const int h = ilogbf(c.hi_ok);
        // without room for 64-bit sums, a coarser packed pass still beats fp32
        // LDS atomics by far
        if (h2 >= PACKED_MIN_BITS || (!a.fb64 && h2 >= PACKED_MIN_BITS - 3)) {
            TileCtx c2 = c;
            c2.scale = ldexpf(c.scale, h2 - h);
            c2.inv_scale = ldexpf(c.inv_scale, h - h2);
            c2.hi_ok = ldexpf(1.0f, h2);
            c2.lo_ok = ldexpf(c.lo_ok, h2 - h);
            uint32_t *w32 = reinterpret_cast<uint32_t *>(smem);
            for (int i = threadIdx.x; i < c.vol * 3 + ncell; i += blockDim.x)
                w32[i] = 0u;
            __syncthreads();
            pass(std::integral_constant<int, ACC_PACKED>{}, c2, true);
            __syncthreads();
            flush_scratch<DIM, ACC_PACKED>(a, c2, sc);
        } else if (a.fb64) {
            for (int i = threadIdx.x; i < 3 * c.vol; i += blockDim.x)
                sc.acc64[i] = 0ull;
            __syncthreads();
            pass(std::integral_constant<int, ACC_FIXED>{}, c, true);
            __syncthreads();
            flush_scratch<DIM, ACC_FIXED>(a, c, sc);
        } else {
            for (int i = threadIdx.x; i < 3 * c.vol; i += blockDim.x)
                sc.acc32[i] = 0.0f;
            __syncthreads();
            pass(std::integral_constant<int, ACC_FLOAT>{}, c, true);
            __syncthreads();
            flush_scratch<DIM, ACC_FLOAT>(a, c, sc);
        }
    } else {
        flush_scratch<DIM, ACC == ACC_PACKED ? ACC_PACKED : ACC_FLOAT>(a, c, sc);
    }
    if (threadIdx.x == 0 && s_esc && a.n_escaped)
        atomicAdd(a.n_escaped, (unsigned long long)s_esc);
}

template <int DIM, int ORDER>
pcg_status launch_flat(const DepArgs &a, int64_t begin, int64_t end, hipStream_t st)
{
    if (end <= begin)
        return PCG_OK;
    const int64_t blocks = std::min<int64_t>((end - begin + 255) / 256, (int64_t)device_cus() * 32);
    return launch("deposit_flat", k_deposit_flat<DIM, ORDER>, dim3((unsigned)blocks), dim3(256), 0,
                  st, a, begin, end);
}

template <int DIM, int ORDER, int ACC, int TEC, bool MOVE>
pcg_status launch_tiled_impl(const DepArgs &a, const MoveArgs &m, uint32_t nwork, int block,
                             size_t lds, hipStream_t st)
{
    auto kern = k_deposit_tiled<DIM, ORDER, ACC, TEC, MOVE>;
    if (lds > 65536) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return fail(PCG_EHIP, "deposit_currents: cannot raise dynamic LDS to %zu bytes", lds);
    }
    return launch(MOVE ? "deposit_regroup" : "deposit_tiled", kern, dim3(xcd_grid(nwork, a.xcd_run)),
                  dim3(block), lds, st, a, m);
}

// Static LDS of a tiled kernel (its __shared__ variables), so that the dynamic
// part plus this stays within the CU's LDS.
template <int DIM, int ORDER, int ACC, int TEC, bool MOVE>
size_t static_lds()
{
    static const size_t bytes = [] {
        hipFuncAttributes fa{};
        if (hipFuncGetAttributes(&fa, (const void *)k_deposit_tiled<DIM, ORDER, ACC, TEC, MOVE>) !=
            hipSuccess)
            return (size_t)8192;  // above what the kernels declare
        return (size_t)fa.sharedSizeBytes;
    }();
    return bytes;
}

// The scratch mode and LDS size of a layout: packed 32-bit sums (64-bit
// fallback when three 64-bit sums per node fit) when the packed scratch fits,
// else fp32 scratch.
template <int DIM, int ORDER, int TEC, bool MOVE>
pcg_status launch_tiled_mode(DepArgs a, const MoveArgs &m, uint32_t nwork, int block,
                             hipStream_t st)
{
    const size_t vol = (size_t)a.vol;
    size_t ncell = 1;
    for (int k = 0; k < DIM; ++k)
        ncell *= (size_t)(a.T + 2 * a.D);
    const size_t packed = packed_bytes(vol, ncell), fixed = vol * 24, flt = vol * 12;
    // The queues (globally deposited particles; in the fused pass, particles
    // that change tile) follow the first pass's scratch, as large as the LDS
    // left allows (none: no queue) and in proportion to the work-group's
    // waves (64 and 128 entries per wave), so that work-groups of one or two
    // waves over small tiles keep their LDS small and many of them fit a CU.
    // They may reach into the 64-bit scratch, which is used only after they
    // are drained, or instead of them.
    const size_t waves = (size_t)std::max(1, block / WAVE);
    auto with_queues = [&](size_t first, size_t rest, size_t limit) {
        size_t at = (first + 15) / 16 * 16;
        auto room = [&](size_t bytes) { return limit > at ? (limit - at) / bytes : 0; };
        a.qoff = (uint32_t)at;
        a.qcap = (uint32_t)std::min<size_t>(std::min<size_t>(QUEUE_MAX, 64 * waves),
                                            room(QUEUE_FLOATS * 4));
        at += (size_t)a.qcap * QUEUE_FLOATS * 4;
        a.moff = (uint32_t)at;
        a.mcap = MOVE ? (uint32_t)std::min<size_t>(std::min<size_t>(MOVE_QUEUE_MAX, 128 * waves),
                                                   room(MQ_WORDS * 4))
                      : 0u;
        at += (size_t)a.mcap * MQ_WORDS * 4;
        return std::max(at, rest);
    };
    const size_t lim_p = LDS_LIMIT - static_lds<DIM, ORDER, ACC_PACKED, TEC, MOVE>();
    if (packed <= lim_p) {
        a.fb64 = fixed <= lim_p ? 1 : 0;
        const size_t lds = with_queues(packed, a.fb64 ? fixed : flt, lim_p);
        return launch_tiled_impl<DIM, ORDER, ACC_PACKED, TEC, MOVE>(a, m, nwork, block, lds, st);
    }
    a.fb64 = 0;
    const size_t lim_f = LDS_LIMIT - static_lds<DIM, ORDER, ACC_FLOAT, TEC, MOVE>();
    if (flt > lim_f)
        return fail(PCG_ELDS, "deposit_currents: scratch of %zu bytes exceeds the LDS", flt);
    const size_t lds = with_queues(flt, flt, lim_f);
    return launch_tiled_impl<DIM, ORDER, ACC_FLOAT, TEC, MOVE>(a, m, nwork, block, lds, st);
}

template <int DIM, int ORDER, bool MOVE>
pcg_status launch_tiled(const DepArgs &a, const MoveArgs &m, uint32_t nwork, int block,
                        size_t lds, hipStream_t st)
{
    (void)lds;
    // the window shapes of tiles 4, 8, 16 with drift 1 are compiled with a
    // constant edge; any other shape uses the runtime-edge kernel
    if (DIM >= 2 && a.D == 1) {
        switch (a.TE) {
        case ORDER == 1 ? 7 : 8: return launch_tiled_mode<DIM, ORDER, ORDER == 1 ? 7 : 8, MOVE>(a, m, nwork, block, st);
        case ORDER == 1 ? 11 : 12: return launch_tiled_mode<DIM, ORDER, ORDER == 1 ? 11 : 12, MOVE>(a, m, nwork, block, st);
        case ORDER == 1 ? 19 : 20: return launch_tiled_mode<DIM, ORDER, ORDER == 1 ? 19 : 20, MOVE>(a, m, nwork, block, st);
        default: break;
        }
    }
    return launch_tiled_mode<DIM, ORDER, 0, MOVE>(a, m, nwork, block, st);
}

template <bool MOVE>
pcg_status dispatch_tiled(int dim, int order, const DepArgs &a, const MoveArgs &m, uint32_t nwork,
                          int block, size_t lds, hipStream_t st)
{
    switch (dim * 10 + order) {
    case 11: return launch_tiled<1, 1, MOVE>(a, m, nwork, block, lds, st);
    case 12: return launch_tiled<1, 2, MOVE>(a, m, nwork, block, lds, st);
    case 21: return launch_tiled<2, 1, MOVE>(a, m, nwork, block, lds, st);
    case 22: return launch_tiled<2, 2, MOVE>(a, m, nwork, block, lds, st);
    case 31: return launch_tiled<3, 1, MOVE>(a, m, nwork, block, lds, st);
    case 32: return launch_tiled<3, 2, MOVE>(a, m, nwork, block, lds, st);
    }
    return fail(PCG_EUNSUPPORTED, "deposit_currents: dim %d order %d", dim, order);
}

pcg_status dispatch(int dim, int order, bool tiled, const DepArgs &a, int64_t begin, int64_t end,
                    uint32_t nwork, int block, size_t lds, hipStream_t st)
{
    const int key = dim * 10 + order;
    if (tiled) {
        return dispatch_tiled<false>(dim, order, a, MoveArgs{}, nwork, block, lds, st);
    } else {
        switch (key) {
        case 11: return launch_flat<1, 1>(a, begin, end, st);
        case 12: return launch_flat<1, 2>(a, begin, end, st);
        case 21: return launch_flat<2, 1>(a, begin, end, st);
        case 22: return launch_flat<2, 2>(a, begin, end, st);
        case 31: return launch_flat<3, 1>(a, begin, end, st);
        case 32: return launch_flat<3, 2>(a, begin, end, st);
        }
    }
    return fail(PCG_EUNSUPPORTED, "deposit_currents: dim %d order %d", dim, order);
}

uint32_t tile_count(const pcg_grid *grid, int T)
{
    uint64_t nt = 1;
    for (int k = 0; k < grid->dim; ++k)
        nt *= (uint64_t)(grid->n[k] / T);
    return (uint32_t)nt;
}

// Smallest chunk a tiled deposit splits a tile into.
constexpr int64_t MIN_DEPOSIT_CHUNK = 2048;

// Work items of a tiled deposit over `ntiles` tiles and n_part particles:
// at most one per tile plus one per MIN_DEPOSIT_CHUNK particles.
uint64_t max_deposit_work(uint32_t ntiles, int64_t n_part)
{
    return (uint64_t)ntiles + (uint64_t)(std::max<int64_t>(n_part, 0) / MIN_DEPOSIT_CHUNK) + 1;
}

// Workspace: chunk prefix, its block totals and the work-item map.
size_t carve_deposit(uint32_t ntiles, int64_t n_part, void *ws, DepArgs *a)
{
    Carver c(ws);
    uint32_t *cum = c.take<uint32_t>((size_t)ntiles + 1);
    uint32_t *part = c.take<uint32_t>(chunk_part_len(ntiles));
    ChunkEntry *map = c.take<ChunkEntry>(max_deposit_work(ntiles, n_part));
    if (a) {
        a->chunk_cum = cum;
        a->chunk_part = part;
        a->chunk_map = map;
    }
    return c.used;
}

size_t deposit_workspace_bytes(const pcg_grid *grid, const pcg_tile *tile)
{
    if (!tile || !grid || check_grid(grid, "pcg_deposit_workspace_bytes") != PCG_OK || tile->T < 1)
        return 0;
    for (int k = 0; k < grid->dim; ++k)
        if (grid->n[k] % tile->T)
            return 0;
    return carve_deposit(tile_count(grid, tile->T), tile->n_partitioned, nullptr, nullptr);
}

// A validated tiled deposit, ready to launch.
struct TiledPlan {
    DepArgs a{};
    uint32_t nwork = 0;
    int block = 256;
    size_t lds = 0;  // fp32 scratch bytes
    bool tiled = false;
};

// Validates the arguments of deposit_currents and fills `plan` (plan->tiled is
// false when there is no layout: the flat path).  `max_chunk` bounds the
// particles one work-group takes (0: no bound).
pcg_status prepare_deposit(const char *who, const pcg_grid *grid, const pcg_particles *particles,
                           int32_t order, const pcg_tile *tile, float *J,
                           unsigned long long *n_escaped, void *workspace,
                           size_t workspace_bytes, uint32_t max_chunk, TiledPlan *plan)
{
    PCG_TRY(check_grid(grid, who));
    if (!particles)
        return fail(PCG_EINVAL, "%s: particles is NULL", who);
    if (order != 1 && order != 2)
        return fail(PCG_EUNSUPPORTED, "%s: order %d not in {1,2}", who, order);
    const int64_t count = particles->count;
    if (count < 0 || count >= (int64_t(1) << 30))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^30)", who, (long long)count);
    if (!J)
        return fail(PCG_EINVAL, "%s: J is NULL", who);
    if (count > 0) {
        for (int k = 0; k < grid->dim; ++k)
            if (!particles->x[k])
                return fail(PCG_EINVAL, "%s: x[%d] is NULL", who, k);
        for (int c = 0; c < 3; ++c)
            if (!particles->v[c])
                return fail(PCG_EINVAL, "%s: v[%d] is NULL", who, c);
        if (!particles->q || !particles->w)
            return fail(PCG_EINVAL, "%s: q or w is NULL", who);
    }
    DepArgs &a = plan->a;
    for (int k = 0; k < 3; ++k) {
        a.n[k] = grid->n[k];
        a.nf[k] = (float)grid->n[k];
        a.x[k] = k < grid->dim ? particles->x[k] : nullptr;
        a.v[k] = particles->v[k];
        a.nt[k] = 1;
    }
    a.q = particles->q;
    a.w = particles->w;
    a.J = J;
    a.ng = (int64_t)grid->n[0] * grid->n[1] * grid->n[2];
    a.n_escaped = n_escaped;
    plan->tiled = tile != nullptr;
    if (!tile)  // no layout yet: flat path ([TD] "First step / tiny species")
        return PCG_OK;

    const int T = tile->T, D = tile->drift;
    if (T < 1)
        return fail(PCG_EINVAL, "%s: tile T = %d < 1", who, T);
    if (tile->order != order)
        return fail(PCG_EINVAL, "%s: layout keyed with order %d, deposit order %d", who,
                    tile->order, order);
    if (D < 0)
        return fail(PCG_EINVAL, "%s: drift %d < 0", who, D);
    for (int k = 0; k < grid->dim; ++k) {
        if (grid->n[k] % T)
            return fail(PCG_EINVAL, "%s: n[%d] = %d is not a multiple of T = %d", who, k,
                        grid->n[k], T);
        if (D + order >= grid->n[k])
            return fail(PCG_EINVAL, "%s: drift %d + order %d must be < n[%d] = %d", who, D,
                        order, k, grid->n[k]);
    }
    if (tile->n_partitioned < 0 || tile->n_partitioned > count)
        return fail(PCG_EINVAL, "%s: n_partitioned %lld outside [0, count]", who,
                    (long long)tile->n_partitioned);
    if (!tile->tile_offsets)
        return fail(PCG_EINVAL, "%s: tile_offsets is NULL", who);
    const int TE = T + order + 2 * D;
    int64_t vol = 1;
    for (int k = 0; k < grid->dim; ++k)
        vol *= TE;
    const size_t lds = (size_t)vol * 3 * sizeof(float);
    if (lds > 160 * 1024)
        return fail(PCG_ELDS, "%s: scratch tile %d^%d x 3 fp32 = %zu bytes exceeds 160 KiB", who,
                    TE, grid->dim, lds);
    const size_t need = deposit_workspace_bytes(grid, tile);
    if (!workspace || workspace_bytes < need)
        return fail(PCG_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace_bytes);
    int block = tile->block;
    if (block <= 0)
        block = 512;  // one scratch tile (up to ~36 KB) shared by 8 waves
    block = std::max(64, std::min(512, block)) / 64 * 64;

    a.T = T;
    a.D = D;
    a.TE = TE;
    a.vol = (int)vol;
    for (int k = 0; k < grid->dim; ++k)
        a.nt[k] = grid->n[k] / T;
    a.ntiles = tile_count(grid, T);
    a.tile_offsets = tile->tile_offsets;
    a.n_part = tile->n_partitioned;
    carve_deposit(a.ntiles, a.n_part, workspace, &a);
    // a tile holding more than `chunk` particles is split over several
    // work-groups (each with its own scratch and flush) to balance load
    const int64_t target = (count + (int64_t)device_cus() * 4 - 1) / ((int64_t)device_cus() * 4);
    int64_t chunk = std::max<int64_t>(MIN_DEPOSIT_CHUNK, target);
    if (max_chunk)
        chunk = std::min<int64_t>(chunk, max_chunk);
    {
        // Where the 64-bit sums do not fit the LDS (no exact fallback for a
        // dense chunk), chunks are kept small enough that the packed 32-bit
        // sums get their full rounding precision (2^PACKED_MIN_BITS) at twice
        // a chunk's mean density: (order+1)^dim (2 c + 1) + 1 <= 2^(31 - bits)
        // particles per cell c.
        int64_t tcells = 1, ns = 1;
        for (int k = 0; k < grid->dim; ++k) {
            tcells *= T;
            ns *= order + 1;
        }
        if ((size_t)vol * 24 > LDS_LIMIT) {
            const int bits = order == 1 ? 21 : 23;
            const int64_t per_cell = std::max<int64_t>(1, (((int64_t)1 << (31 - bits)) - 1 - ns) / (2 * ns));
            chunk = std::min<int64_t>(chunk, std::max<int64_t>(MIN_DEPOSIT_CHUNK, per_cell * tcells));
        }
    }
    if (max_chunk) {
        // the fused pass: whole chunks of the incremental sort per work item
        chunk = std::max<int64_t>(INC_CHUNK, chunk / INC_CHUNK * INC_CHUNK);
        if (tile->block <= 0) {
            // one wave per incremental chunk of an average tile's work item
            const int64_t per_tile = a.n_part / std::max<int64_t>(1, a.ntiles);
            const int64_t chunks = std::min<int64_t>(chunk / INC_CHUNK,
                                                     (per_tile + INC_CHUNK - 1) / INC_CHUNK);
            block = 64 * (int)std::max<int64_t>(1, std::min<int64_t>(MAX_WAVES, chunks));
        }
    }
    a.chunk = (uint32_t)chunk;
    // Where a tile's window holds more sums than the tile has particles (TSC
    // tiles of edge 4: 1536 sums for about 1024 particles), the flush's
    // device atomics dominate and the windows of neighbouring tiles overlap
    // eightfold; runs of neighbouring tiles per XCD then cut the time by a
    // fifth.  For larger tiles the plain order measured as fast or faster.
    a.xcd_run = 3 * vol > a.n_part / std::max<int64_t>(1, a.ntiles) ? 32u : 0u;
    const uint64_t nwork = (uint64_t)a.ntiles + ((uint64_t)a.n_part + a.chunk - 1) / a.chunk;
    if (nwork > max_deposit_work(a.ntiles, a.n_part))
        return fail(PCG_EINVAL, "%s: internal: work items exceed the map", who);
    if (nwork >= (uint64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: too many work-groups", who);
    plan->nwork = (uint32_t)nwork;
    plan->block = block;
    plan->lds = lds;
    return PCG_OK;
}

pcg_status launch_chunks(const DepArgs &a, hipStream_t st)
{
    return launch_chunk_layout("deposit_chunks", a.tile_offsets, a.ntiles, a.n_part, a.chunk,
                               const_cast<uint32_t *>(a.chunk_cum), a.chunk_part,
                               const_cast<ChunkEntry *>(a.chunk_map),
                               (uint32_t)max_deposit_work(a.ntiles, a.n_part), nullptr, 0u, st);
}

// The fused pass's move hook: it replaces the incremental sort's move kernel.
struct RegroupCtx {
    const TiledPlan *plan;
    int dim, order;
};

pcg_status regroup_hook(void *ctx, const IncGeom &inc, const uint32_t *off, uint32_t,
                        const PermArgs &arr, hipStream_t st)
{
    const RegroupCtx &c = *static_cast<const RegroupCtx *>(ctx);
    MoveArgs m{};
    m.inc = inc;
    m.off = off;
    for (int k = 0; k < arr.n && k < 8; ++k)
        m.out[k] = arr.out[k];
    m.group = c.plan->a.chunk / INC_CHUNK;
    PCG_TRY(launch_chunks(c.plan->a, st));
    return dispatch_tiled<true>(c.dim, c.order, c.plan->a, m, c.plan->nwork, c.plan->block,
                                c.plan->lds, st);
}

}  // namespace

// Scratch of deposit_currents_noalloc: its work-item map, in a file-scope
// device array (every GPU the library runs on holds its own copy until the
// process ends).  Calls on one GPU share it, so calls that overlap on one GPU
// race.
constexpr size_t NOALLOC_SCRATCH_BYTES = PCG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device with that device current (the host-side name is not an address).
pcg_status noalloc_scratch(const char *who, void **out)
{
    static std::mutex mu;
    static void *ptr[64] = {nullptr};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(PCG_EHIP, "%s: no current HIP device", who);
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PCG_EHIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", who,
                        dev, hipGetErrorString(e));
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return PCG_OK;
}

}  // namespace
}  // namespace pcg

using namespace pcg;

extern "C" {

size_t pcg_deposit_workspace_bytes(const pcg_grid *grid, const pcg_tile *tile)
{
    return deposit_workspace_bytes(grid, tile);
}

pcg_status deposit_currents(const pcg_grid *grid, const pcg_particles *particles, int32_t order,
                            const pcg_tile *tile, float *J, unsigned long long *n_escaped,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    const char *who = "deposit_currents";
    clear_error();
    TiledPlan plan;
    PCG_TRY(prepare_deposit(who, grid, particles, order, tile, J, n_escaped, workspace,
                            workspace_bytes, 0, &plan));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t count = particles->count;
    if (count == 0)
        return PCG_OK;
    if (!plan.tiled)
        return dispatch(grid->dim, order, false, plan.a, 0, count, 0, 0, 0, st);
    PCG_TRY(launch_chunks(plan.a, st));
    PCG_TRY(dispatch(grid->dim, order, true, plan.a, 0, 0, plan.nwork, plan.block, plan.lds, st));
    // tail pass ([TD] "Coverage: the tail pass")
    return dispatch(grid->dim, order, false, plan.a, tile->n_partitioned, count, 0, 0, 0, st);
}

// The entry point that allocates nothing: the workspace deposit_currents would
// take comes from a file-scope device array instead.  In host code the array's
// name is only a stand-in for the symbol; its device address (one per GPU) is
// looked up once per device and used everywhere host code passes the array.
pcg_status deposit_currents_noalloc(const pcg_grid *grid, const pcg_particles *particles,
                                    int32_t order, const pcg_tile *tile, float *J,
                                    unsigned long long *n_escaped, void *stream)
{
    const char *who = "deposit_currents_noalloc";
    clear_error();
    void *ws = nullptr;
    if (tile) {
        const size_t need = deposit_workspace_bytes(grid, tile);
        if (need > NOALLOC_SCRATCH_BYTES)
            return fail(PCG_EWORKSPACE,
                        "%s: the layout needs %zu bytes of scratch, above the static %zu bytes "
                        "(fewer tiles or particles, or deposit_currents with a workspace)",
                        who, need, (size_t)NOALLOC_SCRATCH_BYTES);
        // every argument check before the first HIP call (the workspace
        // pointer stands in for the scratch; nothing reads it here)
        TiledPlan probe;
        PCG_TRY(prepare_deposit(who, grid, particles, order, tile, J, n_escaped,
                                reinterpret_cast<void *>(uintptr_t(256)), NOALLOC_SCRATCH_BYTES, 0,
                                &probe));
        PCG_TRY(noalloc_scratch(who, &ws));
    }
    // the rest is deposit_currents with the static scratch as its workspace
    return deposit_currents(grid, particles, order, tile, J, n_escaped, ws,
                            ws ? (size_t)NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t pcg_deposit_regroup_workspace_bytes(const pcg_grid *grid, const pcg_tile *tile,
                                           int64_t count)
{
    if (!tile)
        return 0;
    const size_t d = deposit_workspace_bytes(grid, tile);
    const size_t s = sort_workspace_bytes(grid, count, tile->T);
    return d && s ? d + s : 0;
}

pcg_status deposit_currents_regroup(const pcg_grid *grid, const pcg_particles *particles,
                                    int32_t order, const pcg_tile *tile, float *J,
                                    unsigned long long *n_escaped, int32_t n_arrays,
                                    const float *const in_arrays[], float *const out_arrays[],
                                    uint32_t *tile_offsets, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    const char *who = "deposit_currents_regroup";
    clear_error();
    if (!tile)
        return fail(PCG_EINVAL, "%s: tile is NULL (the pass needs the current layout)", who);
    const size_t need = pcg_deposit_regroup_workspace_bytes(grid, tile, particles ? particles->count : 0);
    if (!workspace || workspace_bytes < need || need == 0)
        return fail(PCG_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(PCG_EWORKSPACE, "%s: workspace must be 256-byte aligned", who);
    const size_t dbytes = deposit_workspace_bytes(grid, tile);
    void *sort_ws = static_cast<char *>(workspace) + dbytes;
    TiledPlan plan;
    PCG_TRY(prepare_deposit(who, grid, particles, order, tile, J, n_escaped, workspace, dbytes,
                            MOVE_DEPOSIT_CHUNK, &plan));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t count = particles->count;
    const int dim = grid->dim;
    // the sort's own checks, before anything is enqueued
    if (!tile_offsets)
        return fail(PCG_EINVAL, "%s: tile_offsets is NULL", who);
    if ((const void *)tile_offsets == (const void *)tile->tile_offsets)
        return fail(PCG_EINVAL, "%s: tile_offsets must differ from the layout's offsets", who);
    if (n_arrays < 0 || n_arrays > MAX_ARRAYS)
        return fail(PCG_EINVAL, "%s: n_arrays = %d not in [0, %d]", who, n_arrays, MAX_ARRAYS);
    for (int i = 0; i < n_arrays && count > 0; ++i) {
        if (!in_arrays || !out_arrays || !in_arrays[i] || !out_arrays[i])
            return fail(PCG_EINVAL, "%s: array %d is NULL", who, i);
        if ((const void *)in_arrays[i] == (const void *)out_arrays[i])
            return fail(PCG_EINVAL, "%s: array %d is moved in place (out == in)", who, i);
    }
    if (tile->n_partitioned != count) {
        // a tail: the layout does not cover every particle, so there is no
        // incremental regroup to fuse with -- deposit, then sort
        PCG_TRY(deposit_currents(grid, particles, order, tile, J, n_escaped, workspace, dbytes,
                                 stream));
        return tile_sort_impl(grid, order, tile->T, count, particles->x, n_arrays, in_arrays,
                              out_arrays, nullptr, nullptr, tile_offsets, tile, sort_ws,
                              workspace_bytes - dbytes, st, nullptr, nullptr);
    }
    bool canon = in_arrays && n_arrays == dim + 5;
    for (int k = 0; canon && k < dim; ++k)
        canon = in_arrays[k] == particles->x[k];
    for (int c = 0; canon && c < 3; ++c)
        canon = in_arrays[dim + c] == particles->v[c];
    canon = canon && in_arrays[dim + 3] == particles->q && in_arrays[dim + 4] == particles->w;
    if (!canon) {
        // other arrays than exactly (x, v, q, w): the deposit, then the
        // incremental sort's own move of every array
        PCG_TRY(deposit_currents(grid, particles, order, tile, J, n_escaped, workspace, dbytes,
                                 stream));
        return tile_sort_impl(grid, order, tile->T, count, particles->x, n_arrays, in_arrays,
                              out_arrays, nullptr, nullptr, tile_offsets, tile, sort_ws,
                              workspace_bytes - dbytes, st, nullptr, nullptr);
    }
    RegroupCtx ctx{&plan, dim, order};
    const MoveHook hook{regroup_hook, &ctx};
    bool taken = false;
    PCG_TRY(tile_sort_impl(grid, order, tile->T, count, particles->x, n_arrays, in_arrays,
                           out_arrays, nullptr, nullptr, tile_offsets, tile, sort_ws,
                           workspace_bytes - dbytes, st, &hook, &taken));
    if (!taken && count > 0)  // cannot happen with n_partitioned == count; never skip the deposit
        return fail(PCG_EINVAL, "%s: the incremental regroup was not enqueued", who);
    return PCG_OK;
}

}  // extern "C"
