// zigzag.hip -- charge-conserving zigzag current deposit ([TD] Entity wiki,
// "Tiled current deposit": "Halo sizing" names the zigzag deposit, which writes
// up to two cells above min(i, i_prev); "How a tile deposit runs" for the
// tiled form).
//
// A move from xp to x (less than one cell per axis) is split at the relay
// point xr_k = min(min(i1_k, i2_k) + 1, max(max(i1_k, i2_k), (xp_k + x_k) / 2)),
// i1 = floor(xp), i2 = floor(x), into two segments that each stay in one cell.
// Each segment deposits the exact current of a straight path inside its cell:
// with F = q w (end - start) and W = midpoint - cell per axis, component c gets
//   F_c [w(d1, W_k1) w(d2, W_k2) +/- F'_k1 F'_k2 / 12]
// at cell + d1 e_k1 + d2 e_k2 (k1, k2 the other axes, + when d1 = d2).  J_c[g]
// sits at g + e_c / 2, so that the CIC charge density obeys the discrete
// continuity equation to round-off.  24 contributions per particle.
//
// Tiled: one work-group per tile of a layout keyed on either end of the move
// (the order-1 tile sort); its LDS window per axis starts D + 1 nodes below
// the tile origin and spans TE = T + 2 D + 3 nodes, which holds the stencil
// min(i1, i2) .. max(i1, i2) + 1 of every particle whose layout is at most D
// cells stale and whose move stays within neighbouring cells.  Others take the
// escape valve (global atomics, counted).  The window is added to J with one
// atomic per non-zero slot.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "regroup.hpp"

namespace pcg {
namespace {

// Dynamic LDS available to the tiled kernel (its static part is a few words).
constexpr size_t ZZ_LDS_MAX = 160 * 1024 - 256;

struct ZzArgs {
    int n[3];
    const float *x[3];
    const float *xp[3];
    const float *q;
    const float *w;
    float *J;  // [3][n_z][n_y][n_x]
    const uint32_t *offsets;
    int64_t n_part;
    int T, D, TE;
    int nt[3];  // tiles per axis
    unsigned long long *n_escaped;
};

__device__ inline int wrapn(int64_t i, int n)
{
    const int64_t r = i % n;
    return (int)(r < 0 ? r + n : r);
}

// The particle's move: relay point, cells and midpoints of both segments.
struct Move {
    int cell[2][3];
    float F[2][3];  // end - start of each segment
    float W[2][3];  // midpoint - cell
    float qw;
    int lo[3];       // min(i1, i2): the first node of the stencil per axis
    int64_t ext[3];  // max(i1, i2) + 1 - lo: its last node (2 for a move under a cell)
};

// A particle's inputs: previous and new position, charge, weight.
struct Raw {
    float a[3], b[3], q, w;
};

__device__ inline Raw load_raw(const ZzArgs &m, int64_t p)
{
    Raw r;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        r.a[k] = m.xp[k][p];
        r.b[k] = m.x[k][p];
    }
    r.q = m.q[p];
    r.w = m.w[p];
    return r;
}

// Positions are taken relative to lo = min(i1, i2) first: a - lo and b - lo
// lie in [0, 2) for a move within neighbouring cells and are exact (or within
// an ulp of 1 for |a| < 1), so the segment lengths and midpoints keep fp32's
// relative precision wherever the particle sits on the grid.
// WHOLE: a move that crosses no cell boundary is one segment (the relay point
// at its end, the second segment empty).  The exact current of a straight
// path is additive along it, so this is the sum of the two halves the split
// at the midpoint would give, in one set of adds.
template <bool WHOLE = false>
__device__ inline Move make_move(const Raw &r)
{
    Move mv;
    mv.qw = r.q * r.w;
    bool same = true;
    if (WHOLE)
#pragma unroll
        for (int k = 0; k < 3; ++k)
            same = same && floorf(r.a[k]) == floorf(r.b[k]);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float a = r.a[k], b = r.b[k];
        const float fa = floorf(a), fb = floorf(b);
        const float flo = fminf(fa, fb);
        const float A = a - flo, B = b - flo;   // in cell units above lo
        const float ca = fa - flo, cb = fb - flo;  // 0 or 1 (or more for a long move)
        const float relay = fminf(1.0f, fmaxf(fmaxf(ca, cb), 0.5f * (A + B)));
        const float xr = WHOLE && same ? B : relay;
        mv.cell[0][k] = (int)fa;
        mv.cell[1][k] = (int)fb;
        mv.F[0][k] = xr - A;
        mv.F[1][k] = B - xr;
        mv.W[0][k] = 0.5f * (A + xr) - ca;
        mv.W[1][k] = 0.5f * (xr + B) - cb;
        mv.lo[k] = (int)flo;
        mv.ext[k] = (int64_t)(int)fmaxf(fa, fb) + 1 - mv.lo[k];
    }
    return mv;
}

__device__ inline Move make_move(const ZzArgs &m, int64_t p)
{
    return make_move(load_raw(m, p));
}

// Calls f(c, j, g[3] (unwrapped node), value) for the 12 contributions of
// segment s (j = d1 + 2 d2 numbers the node of component c).
template <typename Fn>
__device__ inline void for_each_in_segment(const Move &mv, int s, Fn &&f)
{
    // value = (F_c w1) w2 +/- F_c cross: one FMA per contribution
    float wm[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        wm[k] = 1.0f - mv.W[s][k];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const int k1 = c == 0 ? 1 : 0, k2 = c == 2 ? 1 : 2;
        const float fc = mv.qw * mv.F[s][c];
        const float fx = fc * (mv.F[s][k1] * mv.F[s][k2] * (1.0f / 12.0f));
        const float a[2] = {fc * wm[k1], fc * mv.W[s][k1]};
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
            for (int d1 = 0; d1 < 2; ++d1) {
                int g[3] = {mv.cell[s][0], mv.cell[s][1], mv.cell[s][2]};
                g[k1] += d1;
                g[k2] += d2;
                f(c, d1 + 2 * d2, g,
                  fmaf(a[d1], d2 ? mv.W[s][k2] : wm[k2], d1 == d2 ? fx : -fx));
            }
    }
}

// The 24 contributions of both segments.
template <typename Fn>
__device__ inline void for_each_contribution(const Move &mv, Fn &&f)
{
#pragma unroll
    for (int s = 0; s < 2; ++s)
        for_each_in_segment(mv, s, [&](int c, int, const int *g, float v) { f(c, g, v); });
}

__device__ inline void deposit_global(const ZzArgs &m, const Move &mv)
{
    const int64_t ng = (int64_t)m.n[0] * m.n[1] * m.n[2];
    for_each_contribution(mv, [&](int c, const int *g, float v) {
        const int64_t idx = wrapn(g[0], m.n[0]) +
                            (int64_t)m.n[0] * (wrapn(g[1], m.n[1]) +
                                               (int64_t)m.n[1] * wrapn(g[2], m.n[2]));
        atomic_add_f32(&m.J[c * ng + idx], v);
    });
}

__global__ __launch_bounds__(256) void k_zigzag_flat(ZzArgs m, int64_t begin, int64_t end)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < end; p += stride)
        deposit_global(m, make_move(m, p));
}

// Per-axis window coordinate of a stencil's first node: lo - ws, brought into
// [0, n) by at most one period each way (enough for positions within a period
// of the grid; anything else fails the fit test and takes the valve).
__device__ inline int64_t window_coord(int lo, int ws, int n)
{
    int64_t d = (int64_t)lo - ws;
    d += d < 0 ? n : 0;
    d -= d >= n ? n : 0;
    return d;
}

// The largest of the work-group's values v (one per thread).  Ends with a
// barrier, so red may be written again afterwards.
__device__ inline float block_max(float v, float *red)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i)
        v = fmaxf(v, red[i]);
    __syncthreads();
    return v;
}

// The fixed-point scale exponent k for particles whose |q w| is at most qmax:
// 2^k 2.17 qmax < 2^31, so every scaled contribution fits an int32.
__device__ inline int fixed_scale(float qmax)
{
    const float bound = 2.17f * qmax;
    int e = 0;
    frexpf(bound, &e);  // bound < 2^e
    return bound > 0.0f ? 31 - e : 0;
}

// x (|x| < 2^31, already scaled) as a two's-complement int64, rounded toward
// zero (an error below one unit of 2^-k, some 5e-10 of max|q w|).
__device__ inline unsigned long long to_fixed(float x)
{
    return (unsigned long long)(long long)(int32_t)x;
}

// One particle's 24 contributions into the window (ws: its first node per
// axis, unwrapped; TE nodes per axis), scaled by 2^k_scale when FIXED; a
// particle whose stencil does not fit (a move over more than a neighbouring
// cell, or a layout more than D cells stale) goes to global memory on the
// first pass and is skipped on a second.  Returns 1 for such an escape on the
// first pass.  When FIXED, a particle with |q w| above qlim (the bound the
// scale was chosen for) adds nothing: its contributions might not fit an int32,
// and the tile is deposited again at a scale that holds it.
template <bool FIXED, typename Acc>
__device__ __attribute__((always_inline)) inline uint32_t window_add(
    const ZzArgs &m, Acc *win, int TE, int vol, const int *ws, Move mv, int k_scale, bool first,
    float qlim)
{
    const int stride[3] = {1, TE, TE * TE};
    // the stencil fits if its last node lies in the window
    int l0[3];
    bool fits = true;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int64_t d = window_coord(mv.lo[k], ws[k], m.n[k]);
        l0[k] = (int)d;
        fits = fits && d >= 0 && mv.ext[k] >= 1 && mv.ext[k] <= 2 && d + mv.ext[k] < TE;
    }
    if (!fits) {
        if (first)
            deposit_global(m, mv);
        return first ? 1u : 0u;
    }
    if (FIXED && !(fabsf(mv.qw) <= qlim))
        return 0u;
    if (FIXED)
        mv.qw = ldexpf(mv.qw, k_scale);  // every contribution comes out scaled
    // window slot of each segment's cell corner
    int base[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        // every term is in [0, TE) once the stencil fits: 24-bit multiplies
        // (full rate; a 32-bit one issues at a quarter of it)
        base[s] = (int)((unsigned)(l0[0] + mv.cell[s][0] - mv.lo[0]) +
                        __umul24((unsigned)TE,
                                 (unsigned)(l0[1] + mv.cell[s][1] - mv.lo[1]) +
                                     __umul24((unsigned)TE,
                                              (unsigned)(l0[2] + mv.cell[s][2] - mv.lo[2]))));
    auto add = [&](int s, int c, int j, float v) {
        const int k1 = c == 0 ? 1 : 0, k2 = c == 2 ? 1 : 2;
        Acc *a = &win[base[s] + c * vol + (j & 1) * stride[k1] + (j >> 1) * stride[k2]];
        if constexpr (FIXED)
            atomicAdd(a, to_fixed(v));
        else
            atomicAdd(a, v);
    };
    // a move that crosses no cell boundary is one segment when FIXED
    // (make_move<true>); its second, empty one is not added
    const bool same = mv.cell[0][0] == mv.cell[1][0] && mv.cell[0][1] == mv.cell[1][1] &&
                      mv.cell[0][2] == mv.cell[1][2];
    for_each_in_segment(mv, 0, [&](int c, int j, const int *, float v) { add(0, c, j, v); });
    if (!(FIXED && same))
        for_each_in_segment(mv, 1, [&](int c, int j, const int *, float v) { add(1, c, j, v); });
    return 0u;
}

// Adds the window to J (one atomic per non-zero slot, periodic wrap).
template <bool FIXED, typename Acc>
__device__ inline void flush_window(const ZzArgs &m, const Acc *win, int TE, int vol,
                                    const int *ws, int k_scale)
{
    const int64_t ng = (int64_t)m.n[0] * m.n[1] * m.n[2];
    for (int i = threadIdx.x; i < 3 * vol; i += blockDim.x) {
        const Acc a = win[i];
        if (a == 0)
            continue;
        float v;
        if constexpr (FIXED)
            v = (float)ldexp((double)(long long)a, -k_scale);
        else
            v = a;
        const int c = i / vol, r = i - c * vol;
        const int lx = r % TE, ly = (r / TE) % TE, lz = r / (TE * TE);
        const int64_t idx = wrapn(ws[0] + lx, m.n[0]) +
                            (int64_t)m.n[0] * (wrapn(ws[1] + ly, m.n[1]) +
                                               (int64_t)m.n[1] * wrapn(ws[2] + lz, m.n[2]));
        atomic_add_f32(&m.J[c * ng + idx], v);
    }
}

// One work-group per tile.  FIXED: the window holds int64 sums of the
// contributions scaled by 2^k (exact and independent of the order of the adds;
// LDS integer atomics run over twenty times the rate of float ones on this
// chip).  A particle whose move stays within neighbouring cells on every axis
// has |F'| <= 1 and 0 <= w <= 1 per segment, so one segment adds at most
// (13/12) |q w| to a node, and a move within one cell (its two segments merged
// into one add) at most twice that; k is chosen so that 2 (13/12) |q w|,
// scaled, is below 2^31, and particles above the assumed max|q w| add nothing
// until the tile runs again.  Each add then converts one int32, and a node
// sum of fewer than 2^31 particles' adds stays below 2^62.  max|q w| is taken
// as twice the largest of the first particle of every thread, and checked
// after the pass against every particle seen; a tile that breaks it is cleared
// and deposited again with its true maximum (escapes, already deposited, are
// skipped then).  Longer moves take the valve.  Not
// FIXED: fp32 sums (the window in int64 does not fit the LDS).  TEC: the
// window edge when fixed at compile time (0: m.TE), so that every slot a
// segment adds to is its base plus a constant.
template <bool FIXED, int TEC>
__global__ __launch_bounds__(512) void k_zigzag_tiled(ZzArgs m)
{
    using Acc = typename std::conditional<FIXED, unsigned long long, float>::type;
    extern __shared__ __align__(8) unsigned char lds_raw[];
    Acc *win = reinterpret_cast<Acc *>(lds_raw);  // [3][TE][TE][TE]
    __shared__ float red[8];  // one per wave
    const int TE = TEC ? TEC : m.TE;
    const int vol = TE * TE * TE;
    const uint32_t t = blockIdx.x;
    const int tc[3] = {(int)(t % (uint32_t)m.nt[0]), (int)((t / (uint32_t)m.nt[0]) % (uint32_t)m.nt[1]),
                       (int)(t / ((uint32_t)m.nt[0] * (uint32_t)m.nt[1]))};
    int ws[3];  // window start (unwrapped node index)
#pragma unroll
    for (int k = 0; k < 3; ++k)
        ws[k] = tc[k] * m.T - m.D - 1;
    const int64_t lo = std::min<int64_t>(m.offsets[t], m.n_part);
    const int64_t hi = std::max<int64_t>(lo, std::min<int64_t>(m.offsets[t + 1], m.n_part));
    uint32_t escaped = 0;

    // one pass over the tile's particles at scale 2^k_scale; returns the
    // largest |q w| this thread saw
    auto deposit_pass = [&](int k_scale, bool first, float qlim) -> float {
        for (int i = threadIdx.x; i < 3 * vol; i += blockDim.x)
            win[i] = 0;
        __syncthreads();
        float seen = 0.0f;
        // the next particle's inputs are loaded while this one is deposited
        Raw next = {};
        if (lo + (int64_t)threadIdx.x < hi)
            next = load_raw(m, lo + threadIdx.x);
        for (int64_t p = lo + threadIdx.x; p < hi; p += blockDim.x) {
            const Raw cur = next;
            if (p + blockDim.x < hi)
                next = load_raw(m, p + blockDim.x);
            const Move mv = make_move<FIXED>(cur);
            seen = fmaxf(seen, fabsf(mv.qw));
            escaped += window_add<FIXED>(m, win, TE, vol, ws, mv, k_scale, first, qlim);
        }
        __syncthreads();
        return seen;
    };

    int k_scale = 0;
    float assumed = 0.0f;
    if (FIXED) {
        float first_qw = 0.0f;
        if (lo + (int64_t)threadIdx.x < hi)
            first_qw = fabsf(m.q[lo + threadIdx.x] * m.w[lo + threadIdx.x]);
        assumed = 2.0f * block_max(first_qw, red);
        k_scale = fixed_scale(assumed);
    }
    // at most two passes: the second runs with the true maximum, which holds
    for (bool first = true;; first = false) {
        const float seen_here = deposit_pass(k_scale, first, assumed);
        if (!FIXED)
            break;
        const float seen = block_max(seen_here, red);
        if (!first || seen <= assumed)
            break;
        assumed = seen;  // the bound may not have held: deposit again
        k_scale = fixed_scale(seen);
    }

    flush_window<FIXED>(m, win, TE, vol, ws, k_scale);
    if (m.n_escaped && escaped)
        atomicAdd(m.n_escaped, (unsigned long long)escaped);
}

// ------------------------------------------------------------------ fused pass

// The regrouping half of the fused pass: every particle the deposit loads is
// also written to its slot in the next layout (keyed on the new positions),
// the slot the incremental tile sort's move stage would give it.
struct ZzMoveArgs {
    IncGeom inc;
    const uint32_t *off;  // the new tile offsets
    float *out[8];        // new arrays of x[0..3), x_prev[0..3), q, w
    uint32_t mcap;        // entries of the LDS queue of particles that change tile
};

#ifndef PCG_ZZ_MQ
#define PCG_ZZ_MQ 1024
#endif
#ifndef PCG_ZZ_UW
#define PCG_ZZ_UW 2
#endif
#ifndef PCG_ZZ_WAVES
#define PCG_ZZ_WAVES 8
#endif
constexpr int ZZ_MQ_WORDS = 9;                     // new slot, then the eight fields
constexpr uint32_t ZZ_MOVE_QUEUE_MAX = PCG_ZZ_MQ;  // entries per work-group (36 KiB)
constexpr int ZZ_WAVES = PCG_ZZ_WAVES;             // most waves of a work-group
constexpr int ZZ_UW = PCG_ZZ_UW;                   // particles per lane in flight in the walk

// One work-group per tile of the layout the particles are grouped by; its
// waves walk the tile's incremental chunks in order (wave j takes chunks j,
// j + waves, ...), 64 ZZ_UW particles at a time.  Each particle gets its slot
// in the new layout from its direction and the wave's running count per
// direction (walk_slot, a stable counting sort), is stored there (or staged in
// LDS if it changes tile, and written with the work-group's other leavers
// after the walk), and is deposited into the window as k_zigzag_tiled<true>
// does.  If the device flag says the incremental path does not hold, the
// kernel deposits only (the general sort then regroups).  The scale check and
// rerun are those of k_zigzag_tiled; the rerun deposits without moving.
template <int TEC, bool FAST>
__global__ __launch_bounds__(ZZ_WAVES * WAVE) void k_zigzag_regroup(ZzArgs m, ZzMoveArgs mv)
{
    using Acc = unsigned long long;
    extern __shared__ __align__(8) unsigned char lds_raw[];
    Acc *win = reinterpret_cast<Acc *>(lds_raw);  // [3][TE][TE][TE]
    const int TE = TEC ? TEC : m.TE;
    const int vol = TE * TE * TE;
    float *mq = reinterpret_cast<float *>(lds_raw + (size_t)3 * vol * sizeof(Acc));
    __shared__ float red[ZZ_WAVES];
    __shared__ uint32_t s_run[ZZ_WAVES][32];
    __shared__ uint32_t s_mn;
    const uint32_t t = blockIdx.x;
    int tc[3];
    tile_coords(t, mv.inc.g, tc);
    int ws[3];  // window start (unwrapped node index)
#pragma unroll
    for (int k = 0; k < 3; ++k)
        ws[k] = tc[k] * m.T - m.D - 1;
    const int64_t lo = std::min<int64_t>(m.offsets[t], m.n_part);
    const int64_t hi = std::max<int64_t>(lo, std::min<int64_t>(m.offsets[t + 1], m.n_part));
    const bool move = *mv.inc.flag == 0u;  // the same value in every lane
    if (threadIdx.x == 0)
        s_mn = 0;
    // the scale: twice the largest |q w| of the first particle of every thread
    float first_qw = 0.0f;
    if (lo + (int64_t)threadIdx.x < hi)
        first_qw = fabsf(m.q[lo + threadIdx.x] * m.w[lo + threadIdx.x]);
    const float assumed = 2.0f * block_max(first_qw, red);
    int k_scale = fixed_scale(assumed);
    for (int i = threadIdx.x; i < 3 * vol; i += blockDim.x)
        win[i] = 0;
    __syncthreads();

    uint32_t escaped = 0;
    float seen = 0.0f;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    const int nwaves = blockDim.x / WAVE;
    const uint32_t p0 = (uint32_t)lo, L = (uint32_t)(hi - lo);
    uint32_t nch = (L + INC_CHUNK - 1) / INC_CHUNK, g0 = 0;
    if (move) {
        g0 = mv.inc.cum[t];
        nch = mv.inc.cum[t + 1] - g0;
    }
    uint32_t *run = s_run[wave];
    for (uint32_t j = wave; j < nch; j += nwaves) {
        const uint32_t clo = p0 + chunk_start(j, L, nch), chi = p0 + chunk_start(j + 1, L, nch);
        if (clo >= chi)
            continue;
        if (move) {
            if (lane < NDIR)
                run[lane] = move_base(mv.inc, mv.off, t, g0 + j, lane);
            __builtin_amdgcn_wave_barrier();
        }
        // no branch around the loads: a lane past the chunk reloads its last
        // particle (never used).  FAST: every array is under 4 GiB, so each
        // element is a 32-bit byte offset from its array's (uniform) base, with
        // no 64-bit address arithmetic per lane
        auto load_one = [&](uint32_t p) __attribute__((always_inline)) {
            if constexpr (FAST) {
                auto at = [p](const float *base) {
                    return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) +
                                                            p * 4u);
                };
                Raw r;
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    r.a[k] = at(m.xp[k]);
                    r.b[k] = at(m.x[k]);
                }
                r.q = at(m.q);
                r.w = at(m.w);
                return r;
            } else {
                return load_raw(m, p);
            }
        };
        auto load_group = [&](uint32_t base, Raw *dst) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < ZZ_UW; ++u)
                dst[u] = load_one(min(base + u * WAVE + lane, chi - 1));
        };
        auto group = [&](uint32_t base, Raw *cur) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < ZZ_UW; ++u)
                asm volatile("" ::"v"(cur[u].a[0]), "v"(cur[u].a[1]), "v"(cur[u].a[2]),
                             "v"(cur[u].b[0]), "v"(cur[u].b[1]), "v"(cur[u].b[2]), "v"(cur[u].q),
                             "v"(cur[u].w));
#pragma unroll
            for (int u = 0; u < ZZ_UW; ++u) {
                const uint32_t p = base + u * WAVE + lane;
                const bool valid = p < chi;
                if (move) {
                    // wave-uniform: the slot comes from the whole wave's directions
                    const int d =
                        FAST ? particle_dir_pow2<3, 1>(cur[u].b[0], cur[u].b[1], cur[u].b[2],
                                                       mv.inc.g, tc)
                             : tile_dir<3, 1>(cur[u].b[0], cur[u].b[1], cur[u].b[2], mv.inc.g, tc);
                    const bool ok = valid && d >= 0;  // d < 0 cannot occur: the flag is clear
                    const uint32_t pos = walk_slot(run, d, ok);
                    if (ok && pos < (uint64_t)mv.inc.count) {
                        const float f[8] = {cur[u].b[0], cur[u].b[1], cur[u].b[2], cur[u].a[0],
                                            cur[u].a[1], cur[u].a[2], cur[u].q, cur[u].w};
                        bool staged = false;
                        if (d != DIR_STAY && mv.mcap) {
                            const uint32_t slot = atomicAdd(&s_mn, 1u);
                            if (slot < mv.mcap) {
                                float *e = mq + (size_t)slot * ZZ_MQ_WORDS;
                                reinterpret_cast<uint32_t *>(e)[0] = pos;
#pragma unroll
                                for (int k = 0; k < 8; ++k)
                                    e[1 + k] = f[k];
                                staged = true;
                            }
                        }
                        if (!staged) {
#pragma unroll
                            for (int k = 0; k < 8; ++k) {
                                if constexpr (FAST)
                                    *reinterpret_cast<float *>(reinterpret_cast<char *>(mv.out[k]) +
                                                               pos * 4u) = f[k];
                                else
                                    mv.out[k][pos] = f[k];
                            }
                        }
                    }
                }
                if (valid) {
                    const Move mm = make_move<true>(cur[u]);
                    seen = fmaxf(seen, fabsf(mm.qw));
                    escaped += window_add<true>(m, win, TE, vol, ws, mm, k_scale, true, assumed);
                }
            }
        };
        // two groups of registers in turn (no copies): the next group loads
        // while this one is deposited
        Raw ga[ZZ_UW], gb[ZZ_UW];
        constexpr uint32_t STEP = ZZ_UW * WAVE;
        load_group(clo, ga);
        for (uint32_t base = clo; base < chi; base += 2 * STEP) {
            load_group(base + STEP, gb);
            group(base, ga);
            if (base + STEP >= chi)
                break;
            load_group(base + 2 * STEP, ga);
            group(base + STEP, gb);
        }
    }
    __syncthreads();
    // the staged leavers, one per thread
    {
        const uint32_t n = min(s_mn, mv.mcap);
        for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
            const float *e = mq + (size_t)i * ZZ_MQ_WORDS;
            const uint32_t pos = reinterpret_cast<const uint32_t *>(e)[0];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                mv.out[k][pos] = e[1 + k];
        }
    }
    const float seen_all = block_max(seen, red);
    if (seen_all > assumed) {
        // the bound may not have held: deposit again with the true maximum
        // (no moves: those are done; escapes, already deposited, skipped)
        k_scale = fixed_scale(seen_all);
        for (int i = threadIdx.x; i < 3 * vol; i += blockDim.x)
            win[i] = 0;
        __syncthreads();
        for (int64_t p = lo + threadIdx.x; p < hi; p += blockDim.x)
            window_add<true>(m, win, TE, vol, ws, make_move<true>(load_raw(m, p)), k_scale, false,
                             seen_all);
        __syncthreads();
    }
    flush_window<true>(m, win, TE, vol, ws, k_scale);
    if (m.n_escaped && escaped)
        atomicAdd(m.n_escaped, (unsigned long long)escaped);
}

// The fused pass's move hook: it replaces the incremental sort's move kernel.
struct ZzRegroupCtx {
    ZzArgs m;
    size_t lds;       // window bytes
    uint32_t ntiles;
};

pcg_status zz_regroup_hook(void *ctx, const IncGeom &inc, const uint32_t *off, uint32_t,
                           const PermArgs &arr, hipStream_t st)
{
    const ZzRegroupCtx &c = *static_cast<const ZzRegroupCtx *>(ctx);
    ZzMoveArgs mv{};
    mv.inc = inc;
    mv.off = off;
    for (int k = 0; k < 8 && k < arr.n; ++k)
        mv.out[k] = arr.out[k];
    // one wave per incremental chunk of an average tile, up to ZZ_WAVES
    const int64_t per_tile = c.m.n_part / std::max<int64_t>(1, c.ntiles);
    const int waves = (int)std::max<int64_t>(
        1, std::min<int64_t>(ZZ_WAVES, (per_tile + INC_CHUNK - 1) / INC_CHUNK));
    // the fast variant: power-of-two geometry (masked tile directions) and
    // arrays under 4 GiB (32-bit byte offsets)
    const bool fast = inc.g.pow2 && inc.count <= ((int64_t)1 << 30);
    auto pick = [fast](auto k_fast, auto k_gen) { return fast ? k_fast : k_gen; };
    auto kern = c.m.TE == 7    ? pick(k_zigzag_regroup<7, true>, k_zigzag_regroup<7, false>)
                : c.m.TE == 9  ? pick(k_zigzag_regroup<9, true>, k_zigzag_regroup<9, false>)
                : c.m.TE == 11 ? pick(k_zigzag_regroup<11, true>, k_zigzag_regroup<11, false>)
                : c.m.TE == 13 ? pick(k_zigzag_regroup<13, true>, k_zigzag_regroup<13, false>)
                               : pick(k_zigzag_regroup<0, true>, k_zigzag_regroup<0, false>);
    size_t stat = 2048;  // above the kernel's static LDS (run counts, reductions)
    {
        hipFuncAttributes fa{};
        if (hipFuncGetAttributes(&fa, (const void *)kern) == hipSuccess)
            stat = (size_t)fa.sharedSizeBytes;
    }
    const size_t limit = 160 * 1024 - stat;
    const size_t at = (c.lds + 15) / 16 * 16;
    // 128 entries per wave at most, so that small work-groups over small
    // tiles keep their LDS small and many fit a CU
    mv.mcap = at < limit ? (uint32_t)std::min<size_t>(
                               std::min<size_t>(ZZ_MOVE_QUEUE_MAX, 128 * (size_t)waves),
                               (limit - at) / (ZZ_MQ_WORDS * 4))
                         : 0u;
    const size_t lds = at + (size_t)mv.mcap * ZZ_MQ_WORDS * 4;
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
        return fail(PCG_EHIP, "deposit_currents_zigzag_regroup: cannot raise dynamic LDS to %zu "
                    "bytes", lds);
    return launch("zigzag_regroup", kern, dim3(c.ntiles), dim3(waves * WAVE), lds, st, c.m, mv);
}

}  // namespace
}  // namespace pcg

using namespace pcg;

namespace pcg {
namespace {

// A validated zigzag deposit: its arguments, and for a layout the window's
// LDS bytes and accumulator kind.
struct ZzPlan {
    ZzArgs m{};
    size_t lds = 0;
    bool fixed = true;
    bool tiled = false;
};

pcg_status prepare_zigzag(const char *who, const pcg_grid *grid, const pcg_particles *particles,
                          const float *const x_prev[3], const pcg_tile *tile, float *J,
                          unsigned long long *n_escaped, ZzPlan *plan)
{
    PCG_TRY(check_grid(grid, who));
    if (grid->dim != 3)
        return fail(PCG_EUNSUPPORTED, "%s: only 3-D grids (dim = %d)", who, grid->dim);
    if (!particles || !J)
        return fail(PCG_EINVAL, "%s: particles or J is NULL", who);
    const int64_t count = particles->count;
    if (count < 0 || count >= (int64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^31)", who, (long long)count);
    if (count > 0) {
        for (int k = 0; k < 3; ++k)
            if (!particles->x[k] || !x_prev || !x_prev[k])
                return fail(PCG_EINVAL, "%s: x[%d] or x_prev[%d] is NULL", who, k, k);
        if (!particles->q || !particles->w)
            return fail(PCG_EINVAL, "%s: q or w is NULL", who);
    }
    ZzArgs &m = plan->m;
    for (int k = 0; k < 3; ++k) {
        m.n[k] = grid->n[k];
        m.x[k] = particles->x[k];
        m.xp[k] = x_prev ? x_prev[k] : nullptr;
    }
    m.q = particles->q;
    m.w = particles->w;
    m.J = J;
    m.n_escaped = n_escaped;
    plan->tiled = tile != nullptr;
    if (tile) {
        if (tile->order != 1)
            return fail(PCG_EINVAL, "%s: the layout must be keyed on CIC cells (order 1, not %d)",
                        who, tile->order);
        if (tile->T < 1 || tile->drift < 0 || !tile->tile_offsets)
            return fail(PCG_EINVAL, "%s: bad layout (T = %d, drift = %d, offsets %p)", who,
                        tile->T, tile->drift, (const void *)tile->tile_offsets);
        for (int k = 0; k < 3; ++k)
            if (grid->n[k] % tile->T)
                return fail(PCG_EINVAL, "%s: n[%d] = %d is not a multiple of T = %d", who, k,
                            grid->n[k], tile->T);
        if (tile->n_partitioned < 0 || tile->n_partitioned > count)
            return fail(PCG_EINVAL, "%s: n_partitioned outside [0, count]", who);
        const int64_t te = (int64_t)tile->T + 2 * (int64_t)tile->drift + 3;
        if (te > 64)  // 3 * 64^3 fp32 sums already exceed the LDS
            return fail(PCG_ELDS, "%s: window edge %lld exceeds the LDS (T = %d, D = %d)", who,
                        (long long)te, tile->T, tile->drift);
        m.T = tile->T;
        m.D = tile->drift;
        m.TE = (int)te;
        plan->lds = (size_t)3 * m.TE * m.TE * m.TE * sizeof(unsigned long long);
        plan->fixed = plan->lds <= ZZ_LDS_MAX;
        if (!plan->fixed)
            plan->lds /= 2;  // fp32 sums
        if (plan->lds > ZZ_LDS_MAX)
            return fail(PCG_ELDS, "%s: window of %zu bytes exceeds the LDS (T = %d, D = %d)",
                        who, plan->lds, tile->T, tile->drift);
        for (int k = 0; k < 3; ++k)
            m.nt[k] = grid->n[k] / tile->T;
        if ((int64_t)m.nt[0] * m.nt[1] * m.nt[2] >= (int64_t(1) << 31))
            return fail(PCG_EINVAL, "%s: %lld tiles exceed one launch", who,
                        (long long)m.nt[0] * m.nt[1] * m.nt[2]);
        m.offsets = tile->tile_offsets;
        m.n_part = tile->n_partitioned;
    }
    return PCG_OK;
}

pcg_status launch_zigzag_flat(const ZzArgs &m, int64_t begin, int64_t end, hipStream_t st)
{
    if (end <= begin)
        return PCG_OK;
    const int64_t blocks = std::min<int64_t>((end - begin + 255) / 256, (int64_t)device_cus() * 32);
    return launch("zigzag_flat", k_zigzag_flat, dim3((unsigned)blocks), dim3(256), 0, st, m, begin,
                  end);
}

pcg_status launch_zigzag_tiled(const ZzPlan &p, hipStream_t st)
{
    const ZzArgs &m = p.m;
    if (m.n_part <= 0)
        return PCG_OK;
    // window edges of tiles 4 and 8 with drift 0 and 1 are compiled in
    auto kern = !p.fixed       ? k_zigzag_tiled<false, 0>
                : m.TE == 7  ? k_zigzag_tiled<true, 7>
                : m.TE == 9  ? k_zigzag_tiled<true, 9>
                : m.TE == 11 ? k_zigzag_tiled<true, 11>
                : m.TE == 13 ? k_zigzag_tiled<true, 13>
                             : k_zigzag_tiled<true, 0>;
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.lds) != hipSuccess)
        return fail(PCG_EHIP, "deposit_currents_zigzag: cannot raise dynamic LDS to %zu bytes",
                    p.lds);
    const int64_t ntiles = (int64_t)m.nt[0] * m.nt[1] * m.nt[2];
    // a window that leaves room for few work-groups per CU gets wider ones
    const unsigned block = p.lds > 32 * 1024 ? 512 : 256;
    return launch(p.fixed ? "zigzag_tiled" : "zigzag_tiled_f32", kern, dim3((unsigned)ntiles),
                  dim3(block), p.lds, st, m);
}

}  // namespace
}  // namespace pcg

extern "C" pcg_status deposit_currents_zigzag(const pcg_grid *grid, const pcg_particles *particles,
                                              const float *const x_prev[3], const pcg_tile *tile,
                                              float *J, unsigned long long *n_escaped,
                                              void *stream)
{
    const char *who = "deposit_currents_zigzag";
    clear_error();
    ZzPlan plan;
    PCG_TRY(prepare_zigzag(who, grid, particles, x_prev, tile, J, n_escaped, &plan));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t count = particles->count;
    if (count == 0)
        return PCG_OK;
    if (!tile)
        return launch_zigzag_flat(plan.m, 0, count, st);
    PCG_TRY(launch_zigzag_tiled(plan, st));
    return launch_zigzag_flat(plan.m, tile->n_partitioned, count, st);
}

extern "C" pcg_status deposit_currents_zigzag_regroup(
    const pcg_grid *grid, const pcg_particles *particles, const float *const x_prev[3],
    const pcg_tile *tile, float *J, unsigned long long *n_escaped, int32_t n_arrays,
    const float *const in_arrays[], float *const out_arrays[], uint32_t *tile_offsets,
    void *workspace, size_t workspace_bytes, void *stream)
{
    const char *who = "deposit_currents_zigzag_regroup";
    clear_error();
    if (!tile)
        return fail(PCG_EINVAL, "%s: tile is NULL (the pass needs the current layout)", who);
    ZzPlan plan;
    PCG_TRY(prepare_zigzag(who, grid, particles, x_prev, tile, J, n_escaped, &plan));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t count = particles->count;
    // the sort's own checks, before anything is enqueued
    const size_t need = sort_workspace_bytes(grid, count, tile->T);
    if (!workspace || workspace_bytes < need || need == 0)
        return fail(PCG_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace_bytes);
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
    bool canon = in_arrays && n_arrays == 8 && plan.fixed && tile->n_partitioned == count;
    for (int k = 0; canon && k < 3; ++k)
        canon = in_arrays[k] == particles->x[k] && in_arrays[3 + k] == x_prev[k];
    canon = canon && in_arrays[6] == particles->q && in_arrays[7] == particles->w;
    if (!canon) {
        // a tail, fp32 window sums, or other arrays than exactly (x, x_prev,
        // q, w): the deposit, then the sort with its own move
        PCG_TRY(deposit_currents_zigzag(grid, particles, x_prev, tile, J, n_escaped, stream));
        return tile_sort_impl(grid, 1, tile->T, count, particles->x, n_arrays, in_arrays,
                              out_arrays, nullptr, nullptr, tile_offsets, tile, workspace,
                              workspace_bytes, st, nullptr, nullptr);
    }
    ZzRegroupCtx ctx{plan.m, plan.lds, (uint32_t)((int64_t)plan.m.nt[0] * plan.m.nt[1] *
                                                  plan.m.nt[2])};
    const MoveHook hook{zz_regroup_hook, &ctx};
    bool taken = false;
    PCG_TRY(tile_sort_impl(grid, 1, tile->T, count, particles->x, n_arrays, in_arrays, out_arrays,
                           nullptr, nullptr, tile_offsets, tile, workspace, workspace_bytes, st,
                           &hook, &taken));
    if (!taken && count > 0)  // cannot happen with n_partitioned == count; never skip the deposit
        return deposit_currents_zigzag(grid, particles, x_prev, tile, J, n_escaped, stream);
    return PCG_OK;
}
