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

// One work-group per tile.  FIXED: the window holds int64 sums of the
// contributions scaled by 2^k (exact and independent of the order of the adds;
// LDS integer atomics run over twenty times the rate of float ones on this
// chip).  A particle whose move stays within neighbouring cells on every axis
// has |F'| <= 1 and 0 <= w <= 1 per segment, so it adds at most 2 (13/12) |q w|
// to any node (both segments, summed before the add); k is chosen so that this
// bound, scaled, is below 2^31.  Each add then converts one int32, and a node
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
    const int stride[3] = {1, TE, TE * TE};
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
    auto deposit_pass = [&](int k_scale, bool first) -> float {
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
            Move mv = make_move<FIXED>(cur);
            seen = fmaxf(seen, fabsf(mv.qw));
            // the stencil fits if its last node lies in the window (a move over
            // more than a neighbouring cell is sent to global memory)
            int l0[3];
            bool fits = true;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int64_t d = window_coord(mv.lo[k], ws[k], m.n[k]);
                l0[k] = (int)d;
                fits = fits && d >= 0 && mv.ext[k] >= 1 && mv.ext[k] <= 2 && d + mv.ext[k] < TE;
            }
            if (!fits) {
                if (first) {
                    deposit_global(m, mv);
                    ++escaped;
                }
                continue;
            }
            if (FIXED)
                mv.qw = ldexpf(mv.qw, k_scale);  // every contribution comes out scaled
            // window slot of each segment's cell corner
            int base[2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
                base[s] = (l0[0] + mv.cell[s][0] - mv.lo[0]) +
                          TE * ((l0[1] + mv.cell[s][1] - mv.lo[1]) +
                                TE * (l0[2] + mv.cell[s][2] - mv.lo[2]));
            auto add = [&](int s, int c, int j, float v) {
                const int k1 = c == 0 ? 1 : 0, k2 = c == 2 ? 1 : 2;
                Acc *a = &win[base[s] + c * vol + (j & 1) * stride[k1] + (j >> 1) * stride[k2]];
                if constexpr (FIXED)
                    atomicAdd(a, to_fixed(v));
                else
                    atomicAdd(a, v);
            };
            // a move that crosses no cell boundary is one segment when FIXED
            // (above); its second, empty one is not added
            const bool same = mv.cell[0][0] == mv.cell[1][0] && mv.cell[0][1] == mv.cell[1][1] &&
                              mv.cell[0][2] == mv.cell[1][2];
            for_each_in_segment(mv, 0, [&](int c, int j, const int *, float v) { add(0, c, j, v); });
            if (!(FIXED && same))
                for_each_in_segment(mv, 1, [&](int c, int j, const int *, float v) {
                    add(1, c, j, v);
                });
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
        const float seen_here = deposit_pass(k_scale, first);
        if (!FIXED)
            break;
        const float seen = block_max(seen_here, red);
        if (!first || seen <= assumed)
            break;
        assumed = seen;  // the bound may not have held: deposit again
        k_scale = fixed_scale(seen);
    }

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
    if (m.n_escaped && escaped)
        atomicAdd(m.n_escaped, (unsigned long long)escaped);
}

}  // namespace
}  // namespace pcg

using namespace pcg;

extern "C" pcg_status deposit_currents_zigzag(const pcg_grid *grid, const pcg_particles *particles,
                                              const float *const x_prev[3], const pcg_tile *tile,
                                              float *J, unsigned long long *n_escaped,
                                              void *stream)
{
    const char *who = "deposit_currents_zigzag";
    clear_error();
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
    ZzArgs m{};
    for (int k = 0; k < 3; ++k) {
        m.n[k] = grid->n[k];
        m.x[k] = particles->x[k];
        m.xp[k] = x_prev ? x_prev[k] : nullptr;
    }
    m.q = particles->q;
    m.w = particles->w;
    m.J = J;
    m.n_escaped = n_escaped;
    size_t lds = 0;
    bool fixed = true;
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
        lds = (size_t)3 * m.TE * m.TE * m.TE * sizeof(unsigned long long);
        fixed = lds <= ZZ_LDS_MAX;
        if (!fixed)
            lds /= 2;  // fp32 sums
        if (lds > ZZ_LDS_MAX)
            return fail(PCG_ELDS, "%s: window of %zu bytes exceeds the LDS (T = %d, D = %d)",
                        who, lds, tile->T, tile->drift);
        for (int k = 0; k < 3; ++k)
            m.nt[k] = grid->n[k] / tile->T;
        if ((int64_t)m.nt[0] * m.nt[1] * m.nt[2] >= (int64_t(1) << 31))
            return fail(PCG_EINVAL, "%s: %lld tiles exceed one launch", who,
                        (long long)m.nt[0] * m.nt[1] * m.nt[2]);
        m.offsets = tile->tile_offsets;
        m.n_part = tile->n_partitioned;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (count == 0)
        return PCG_OK;
    auto flat = [&](int64_t begin, int64_t end) -> pcg_status {
        if (end <= begin)
            return PCG_OK;
        const int64_t blocks =
            std::min<int64_t>((end - begin + 255) / 256, (int64_t)device_cus() * 32);
        return launch("zigzag_flat", k_zigzag_flat, dim3((unsigned)blocks), dim3(256), 0, st, m,
                      begin, end);
    };
    if (!tile)
        return flat(0, count);
    if (m.n_part > 0) {
        // window edges of tiles 4 and 8 with drift 0 and 1 are compiled in
        auto kern = !fixed         ? k_zigzag_tiled<false, 0>
                    : m.TE == 7  ? k_zigzag_tiled<true, 7>
                    : m.TE == 9  ? k_zigzag_tiled<true, 9>
                    : m.TE == 11 ? k_zigzag_tiled<true, 11>
                    : m.TE == 13 ? k_zigzag_tiled<true, 13>
                                 : k_zigzag_tiled<true, 0>;
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return fail(PCG_EHIP, "%s: cannot raise dynamic LDS to %zu bytes", who, lds);
        const int64_t ntiles = (int64_t)m.nt[0] * m.nt[1] * m.nt[2];
        // a window that leaves room for few work-groups per CU gets wider ones
        const unsigned block = lds > 32 * 1024 ? 512 : 256;
        PCG_TRY(launch(fixed ? "zigzag_tiled" : "zigzag_tiled_f32", kern, dim3((unsigned)ntiles),
                       dim3(block), lds, st, m));
    }
    return flat(tile->n_partitioned, count);
}
