// deposit.hip -- current deposit J_c += q w v_c W(x - x_g) ([TD] Entity wiki
// "Tiled current deposit"; B-spline weights from the mass-matrix paper §2.3
// Eq.(12)).
//
// Tiled path ([TD] "How a tile deposit runs"): one work-group per tile (or per
// chunk of a heavy tile) zeroes an LDS scratch window of TE = T + order + 2D
// nodes per used axis (D nodes of drift below the tile origin, D + order
// above), adds every particle of its slice into it with LDS atomics (exact
// int64 fixed-point sums, see k_deposit_tiled), then adds each non-zero scratch
// value to J with one global atomic, wrapping node indices periodically.  A particle whose support does not fit the window is
// deposited directly to J with global atomics (the escape valve, [TD]
// "Correctness is independent of the halo").
// Flat path ([TD] "The two paths", flat column): one thread per particle,
// (order+1)^dim x 3 global atomics -- used with no layout and for the tail.
#include <algorithm>
#include <climits>

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
    const uint32_t *chunk_cum;
    uint32_t chunk;
    unsigned long long *n_escaped;
};

// The regrouping half of the fused pass: every particle the deposit loads is
// also written to its slot in the next tile layout, as the incremental tile
// sort's move stage would (same slots, so the same result).
constexpr int MOVE_MAX_CHUNKS = 40;          // incremental chunks one deposit chunk can overlap
constexpr uint32_t MOVE_DEPOSIT_CHUNK = 32768;  // largest deposit chunk when moving

struct MoveArgs {
    IncGeom inc;
    const uint32_t *off;  // the new tile offsets
    PermArgs arr;
    int canon;            // arr.in[] are exactly x[0..dim), v[0..3), q, w: store from registers
};

// Incremental chunk (0-based within the tile) holding slot r of a tile slice of
// L particles split into nch balanced chunks (chunk c starts at floor(L c / nch)).
__device__ inline uint32_t chunk_of(uint32_t r, uint32_t L, uint32_t nch)
{
    return (uint32_t)(((uint64_t)(r + 1) * nch + L - 1) / L) - 1u;
}

__device__ inline uint32_t chunk_start(uint32_t c, uint32_t L, uint32_t nch)
{
    return (uint32_t)(((uint64_t)L * c) / nch);
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
    return wrap_index(b, n);
}

// All (order+1)^dim global atomics of one particle.
template <int DIM, int ORDER>
__device__ inline void deposit_global(const DepArgs &a, const int *b, float W[3][ORDER + 1],
                                      const float *amp)
{
    constexpr int M = ORDER + 1;
    constexpr int MY = DIM > 1 ? M : 1, MZ = DIM > 2 ? M : 1;
#pragma unroll
    for (int az = 0; az < MZ; ++az) {
        const int gz = DIM > 2 ? wrap_index(b[2] + az, a.n[2]) : 0;
#pragma unroll
        for (int ay = 0; ay < MY; ++ay) {
            const int gy = DIM > 1 ? wrap_index(b[1] + ay, a.n[1]) : 0;
            const float wyz = (DIM > 1 ? W[1][ay] : 1.0f) * (DIM > 2 ? W[2][az] : 1.0f);
#pragma unroll
            for (int ax = 0; ax < M; ++ax) {
                const int gx = wrap_index(b[0] + ax, a.n[0]);
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

// LDS float atomics (ds_add_f32) are ~30x slower than integer LDS atomics on
// gfx950, so the scratch tile normally holds int64 fixed-point sums: a
// work-group picks a power-of-two scale 2^S from the largest |q w v_c| of its
// first 256 particles (S puts that value near 2^23), every product
// q w v_c W * 2^S is rounded once to an integer and added with ds_add_u64.
// The sums are then exact and independent of the order of the adds.  A
// particle whose largest |q w v_c| * 2^S is outside [2^8, 2^30) would overflow
// or lose precision there, so it takes the escape valve like a particle that
// left the window (only the latter are counted as escapes).  When the int64
// scratch does not fit the LDS, FIXED = false keeps fp32 LDS atomics.
template <int DIM, int ORDER, bool FIXED, int TEC, bool MOVE>
__global__ __launch_bounds__(1024) void k_deposit_tiled(DepArgs a, MoveArgs m)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned long long *acc64 = reinterpret_cast<unsigned long long *>(smem);  // [3][vol]
    float *acc32 = reinterpret_cast<float *>(smem);                          // [3][vol]
    __shared__ uint32_t s_tile, s_lo, s_hi, s_esc, s_maxbits, s_move;
    // MOVE: output slot base per (incremental chunk overlapped, direction), and
    // the end slot of each of those chunks
    __shared__ uint32_t s_base[MOVE ? MOVE_MAX_CHUNKS * NDIR : 1];
    __shared__ uint32_t s_cend[MOVE ? MOVE_MAX_CHUNKS : 1];
    constexpr int M = ORDER + 1;
    constexpr int MY = DIM > 1 ? M : 1, MZ = DIM > 2 ? M : 1;

    if (threadIdx.x == 0) {
        const ChunkRange r = find_chunk(blockIdx.x, a.chunk_cum, a.ntiles, a.tile_offsets,
                                        a.n_part);
        s_tile = r.tile;
        s_lo = r.lo;
        s_hi = r.hi;
        s_esc = 0;
        s_maxbits = 0;
        s_move = MOVE && *m.inc.flag == 0u;
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile == UINT_MAX)
        return;
    const uint32_t lo = s_lo, hi = s_hi;
    int origin[3] = {0, 0, 0};
    {
        uint32_t t = tile;
#pragma unroll
        for (int k = 0; k < DIM; ++k) {
            origin[k] = (int)(t % (uint32_t)a.nt[k]) * a.T;
            t /= (uint32_t)a.nt[k];
        }
    }
    // TEC > 0: the scratch edge is a compile-time constant, so every node offset
    // folds into the LDS instruction's immediate offset
    const int TE = TEC > 0 ? TEC : a.TE;
    const int vol = TEC > 0 ? (DIM == 3 ? TEC * TEC * TEC : (DIM == 2 ? TEC * TEC : TEC)) : a.vol;
    const int D = a.D;

    // MOVE: the incremental chunks of this tile's slice that [lo, hi) overlaps
    const bool move = MOVE && s_move != 0u;
    uint32_t p0 = 0, L = 1, nch = 1, c_first = 0;
    if (move) {
        p0 = (uint32_t)min((int64_t)m.inc.prev_off[tile], m.inc.count);
        const uint32_t p1 = (uint32_t)min((int64_t)m.inc.prev_off[tile + 1], m.inc.count);
        L = p1 - p0;  // >= hi - lo > 0
        const uint32_t g0 = m.inc.cum[tile];
        nch = m.inc.cum[tile + 1] - g0;
        c_first = chunk_of(lo - p0, L, nch);
        const uint32_t c_last = chunk_of(hi - 1 - p0, L, nch);
        const uint32_t nc = min(c_last - c_first + 1, (uint32_t)MOVE_MAX_CHUNKS);
        for (uint32_t i = threadIdx.x; i < nc * NDIR; i += blockDim.x)
            s_base[i] = move_base(m.inc, m.off, tile, g0 + c_first + i / NDIR, (int)(i % NDIR));
        for (uint32_t i = threadIdx.x; i < nc; i += blockDim.x)
            s_cend[i] = p0 + chunk_start(c_first + i + 1, L, nch);
    }

    if (FIXED) {
        for (int i = threadIdx.x; i < 3 * vol; i += blockDim.x)
            acc64[i] = 0ull;
        // scale from the first batch: largest |q w v_c|
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
    } else {
        for (int i = threadIdx.x; i < 3 * vol; i += blockDim.x)
            acc32[i] = 0.0f;
    }
    __syncthreads();
    float scale = 1.0f, inv_scale = 1.0f;
    if (FIXED) {
        const float mx = __uint_as_float(s_maxbits);
        int S = 0;
        if (mx > 0.0f)
            S = 23 - ilogbf(mx);
        S = max(-100, min(100, S));
        scale = ldexpf(1.0f, S);
        inv_scale = ldexpf(1.0f, -S);
    }
    const float lo_ok = 256.0f, hi_ok = 1073741824.0f;  // 2^8 and 2^30 (scaled)

    const int last = a.T - 1 + 2 * D;  // largest scratch start that keeps the stencil inside
    // Each thread keeps U particles (stride blockDim.x apart) in flight: the
    // next group's values (and move codes) load while this group is weighed,
    // moved and accumulated.
    constexpr int U = DEPOSIT_UNROLL;
    const uint32_t stride = blockDim.x;
    float nx[U][3], nv[U][3], nq[U], nw[U];
    uint32_t ncode[U];
    auto load_group = [&](uint32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p = base + u * stride;
            nx[u][0] = nx[u][1] = nx[u][2] = 0.f;
            nv[u][0] = nv[u][1] = nv[u][2] = 0.f;
            nq[u] = nw[u] = 0.f;
            ncode[u] = 0;
            if (p < hi) {
#pragma unroll
                for (int k = 0; k < DIM; ++k)
                    nx[u][k] = a.x[k][p];
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    nv[u][c] = a.v[c][p];
                nq[u] = a.q[p];
                nw[u] = a.w[p];
                if (move)
                    ncode[u] = m.inc.code[p];
            }
        }
    };
    uint32_t ci = 0, c_end = 0;  // MOVE: this thread's chunk (relative to c_first) and its end
    if (move) {
        const uint32_t p = min(lo + threadIdx.x, hi - 1);
        ci = min(chunk_of(p - p0, L, nch) - c_first, (uint32_t)MOVE_MAX_CHUNKS - 1);
        c_end = s_cend[ci];
    }
    load_group(lo + threadIdx.x);

    for (uint32_t base = lo + threadIdx.x; base < hi; base += U * stride) {
        float gx[U][3], gv[U][3], gq[U], gw[U];
        uint32_t gcode[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                gx[u][k] = nx[u][k];
                gv[u][k] = nv[u][k];
            }
            gq[u] = nq[u];
            gw[u] = nw[u];
            gcode[u] = ncode[u];
        }
        load_group(base + U * stride);

#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p = base + u * stride;
            if (p >= hi)
                break;
            const float *xs = gx[u], *vv = gv[u];
            const float cq = gq[u], cw = gw[u];
            if (move) {
                // slot in the new layout: the (chunk, direction) base plus the rank
                while (p >= c_end && ci + 1 < (uint32_t)MOVE_MAX_CHUNKS) {
                    ++ci;
                    c_end = s_cend[ci];
                }
                const uint32_t code = gcode[u];
                const uint32_t d = min(code >> 27, (uint32_t)NDIR - 1);
                const uint32_t pos = s_base[ci * NDIR + d] + (code & RANK_MASK);
                if (pos < (uint64_t)m.inc.count) {
                    if (m.canon) {
#pragma unroll
                        for (int k = 0; k < DIM; ++k)
                            m.arr.out[k][pos] = xs[k];
#pragma unroll
                        for (int c = 0; c < 3; ++c)
                            m.arr.out[DIM + c][pos] = vv[c];
                        m.arr.out[DIM + 3][pos] = cq;
                        m.arr.out[DIM + 4][pos] = cw;
                    } else {
                        for (int i = 0; i < m.arr.n; ++i)
                            m.arr.out[i][pos] = m.arr.in[i][p];
                    }
                }
            }
            const float qw = cq * cw;

            float W[3][M];
            int b[3] = {0, 0, 0};
            int s[3] = {0, 0, 0};
            bool esc = false;
#pragma unroll
            for (int k = 0; k < DIM; ++k) {
                b[k] = shape_axis<ORDER>(xs[k], a.nf[k], a.n[k], W[k]);
                // scratch start: periodic offset of the base node from the window's low edge
                s[k] = wrap_index(b[k] - origin[k] + D, a.n[k]);
                esc |= s[k] > last;
            }
            float amp[3] = {qw * vv[0], qw * vv[1], qw * vv[2]};
            bool in_lds = !esc;
            if (FIXED) {
                const float amax =
                    fmaxf(fabsf(amp[0]), fmaxf(fabsf(amp[1]), fabsf(amp[2]))) * scale;
                if (amax == 0.0f) {  // deposits nothing, but an escape is still an escape
                    if (esc)
                        atomicAdd(&s_esc, 1u);
                    continue;
                }
                in_lds = in_lds && amax >= lo_ok && amax < hi_ok;
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    amp[c] *= scale;
            }
            if (in_lds) {
                // amp_c * W_x first, then one multiply per (node, component)
                float ampx[3][M];
#pragma unroll
                for (int c = 0; c < 3; ++c)
#pragma unroll
                    for (int ax = 0; ax < M; ++ax)
                        ampx[c][ax] = amp[c] * W[0][ax];
                const int sbase = DIM == 3 ? (s[2] * TE + s[1]) * TE + s[0]
                                           : (DIM == 2 ? s[1] * TE + s[0] : s[0]);
#pragma unroll
                for (int az = 0; az < MZ; ++az) {
#pragma unroll
                    for (int ay = 0; ay < MY; ++ay) {
                        const int row = sbase + (DIM == 3 ? (az * TE + ay) * TE : ay * TE);
                        const float wyz =
                            (DIM > 1 ? W[1][ay] : 1.0f) * (DIM > 2 ? W[2][az] : 1.0f);
#pragma unroll
                        for (int ax = 0; ax < M; ++ax) {
                            const int idx = row + ax;
#pragma unroll
                            for (int c = 0; c < 3; ++c) {
                                const float val = ampx[c][ax] * wyz;
                                if (FIXED) {
                                    const long long f = (long long)__float2int_rn(val);
                                    __hip_atomic_fetch_add(&acc64[c * vol + idx],
                                                           (unsigned long long)f,
                                                           __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                                } else {
                                    __hip_atomic_fetch_add(&acc32[c * vol + idx], val,
                                                           __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                                }
                            }
                        }
                    }
                }
            } else {
                if (FIXED) {
#pragma unroll
                    for (int c = 0; c < 3; ++c)
                        amp[c] *= inv_scale;  // exact: power-of-two scale
                }
                deposit_global<DIM, ORDER>(a, b, W, amp);
                if (esc)
                    atomicAdd(&s_esc, 1u);
            }
        }
    }
    __syncthreads();

    // flush: one global atomic per non-zero scratch value, node indices wrapped
    for (int i = threadIdx.x; i < vol; i += blockDim.x) {
        int sx = i, sy = 0, sz = 0;
        if (DIM > 1) {
            sx = i % TE;
            const int r = i / TE;
            sy = DIM > 2 ? r % TE : r;
            sz = DIM > 2 ? r / TE : 0;
        }
        const int gx = wrap_index(origin[0] - D + sx, a.n[0]);
        const int gy = DIM > 1 ? wrap_index(origin[1] - D + sy, a.n[1]) : 0;
        const int gz = DIM > 2 ? wrap_index(origin[2] - D + sz, a.n[2]) : 0;
        const int64_t g = gx + (int64_t)a.n[0] * (gy + (int64_t)a.n[1] * gz);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            float val;
            if (FIXED)
                val = (float)((double)(long long)acc64[c * vol + i] * (double)inv_scale);
            else
                val = acc32[c * vol + i];
            if (val != 0.0f)
                atomic_add_f32(&a.J[c * a.ng + g], val);
        }
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

template <int DIM, int ORDER, bool FIXED, int TEC, bool MOVE>
pcg_status launch_tiled_impl(const DepArgs &a, const MoveArgs &m, uint32_t nwork, int block,
                             size_t lds, hipStream_t st)
{
    auto kern = k_deposit_tiled<DIM, ORDER, FIXED, TEC, MOVE>;
    if (lds > 65536) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return fail(PCG_EHIP, "deposit_currents: cannot raise dynamic LDS to %zu bytes", lds);
    }
    return launch(MOVE ? "deposit_regroup" : "deposit_tiled", kern, dim3(nwork), dim3(block), lds,
                  st, a, m);
}

constexpr size_t scratch_bytes(int dim, int te, int elem)
{
    return (size_t)3 * elem * (dim == 3 ? te * te * te : (dim == 2 ? te * te : te));
}

// A compile-time scratch edge: int64 fixed-point scratch when it fits the LDS.
template <int DIM, int ORDER, int TEC, bool MOVE>
pcg_status launch_tiled_te(const DepArgs &a, const MoveArgs &m, uint32_t nwork, int block,
                           hipStream_t st)
{
    constexpr bool fixed = scratch_bytes(DIM, TEC, 8) <= LDS_LIMIT;
    return launch_tiled_impl<DIM, ORDER, fixed, TEC, MOVE>(
        a, m, nwork, block, scratch_bytes(DIM, TEC, fixed ? 8 : 4), st);
}

template <int DIM, int ORDER, bool MOVE>
pcg_status launch_tiled(const DepArgs &a, const MoveArgs &m, uint32_t nwork, int block,
                        size_t lds, hipStream_t st)
{
    // the window shapes of tiles 4, 8, 16 with drift 1 are compiled with a
    // constant edge; any other shape uses the runtime-edge kernel
    if (DIM >= 2 && a.D == 1) {
        switch (a.TE) {
        case ORDER == 1 ? 7 : 8: return launch_tiled_te<DIM, ORDER, ORDER == 1 ? 7 : 8, MOVE>(a, m, nwork, block, st);
        case ORDER == 1 ? 11 : 12: return launch_tiled_te<DIM, ORDER, ORDER == 1 ? 11 : 12, MOVE>(a, m, nwork, block, st);
        case ORDER == 1 ? 19 : 20: return launch_tiled_te<DIM, ORDER, ORDER == 1 ? 19 : 20, MOVE>(a, m, nwork, block, st);
        default: break;
        }
    }
    // int64 fixed-point scratch when it fits, else fp32 scratch (lds is the fp32 size)
    if (2 * lds <= LDS_LIMIT)
        return launch_tiled_impl<DIM, ORDER, true, 0, MOVE>(a, m, nwork, block, 2 * lds, st);
    return launch_tiled_impl<DIM, ORDER, false, 0, MOVE>(a, m, nwork, block, lds, st);
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

size_t deposit_workspace_bytes(const pcg_grid *grid, const pcg_tile *tile)
{
    if (!tile || !grid || check_grid(grid, "pcg_deposit_workspace_bytes") != PCG_OK || tile->T < 1)
        return 0;
    for (int k = 0; k < grid->dim; ++k)
        if (grid->n[k] % tile->T)
            return 0;
    return align_up(((size_t)tile_count(grid, tile->T) + 1) * sizeof(uint32_t), 256);
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
    if (count < 0 || count >= (int64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^31)", who, (long long)count);
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
    block = std::max(64, std::min(1024, block)) / 64 * 64;

    a.T = T;
    a.D = D;
    a.TE = TE;
    a.vol = (int)vol;
    for (int k = 0; k < grid->dim; ++k)
        a.nt[k] = grid->n[k] / T;
    a.ntiles = tile_count(grid, T);
    a.tile_offsets = tile->tile_offsets;
    a.n_part = tile->n_partitioned;
    a.chunk_cum = static_cast<const uint32_t *>(workspace);
    // a tile holding more than `chunk` particles is split over several
    // work-groups (each with its own scratch and flush) to balance load
    const int64_t target = (count + (int64_t)device_cus() * 4 - 1) / ((int64_t)device_cus() * 4);
    int64_t chunk = std::max<int64_t>(2048, target);
    if (max_chunk)
        chunk = std::min<int64_t>(chunk, max_chunk);
    a.chunk = (uint32_t)chunk;
    const uint64_t nwork = (uint64_t)a.ntiles + ((uint64_t)a.n_part + a.chunk - 1) / a.chunk;
    if (nwork >= (uint64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: too many work-groups", who);
    plan->nwork = (uint32_t)nwork;
    plan->block = block;
    plan->lds = lds;
    return PCG_OK;
}

pcg_status launch_chunks(const DepArgs &a, hipStream_t st)
{
    return launch("deposit_chunks", k_chunk_cum, dim3(1), dim3(1024), 0, st, a.tile_offsets,
                  a.ntiles, a.n_part, a.chunk, const_cast<uint32_t *>(a.chunk_cum),
                  (const uint32_t *)nullptr, 0u);
}

// The fused pass's move hook: it replaces the incremental sort's move kernel.
struct RegroupCtx {
    const TiledPlan *plan;
    int dim, order;
    int canon;
};

pcg_status regroup_hook(void *ctx, const IncGeom &inc, const uint32_t *off, uint32_t,
                        const PermArgs &arr, hipStream_t st)
{
    const RegroupCtx &c = *static_cast<const RegroupCtx *>(ctx);
    MoveArgs m{};
    m.inc = inc;
    m.off = off;
    m.arr = arr;
    m.canon = c.canon;
    PCG_TRY(launch_chunks(c.plan->a, st));
    return dispatch_tiled<true>(c.dim, c.order, c.plan->a, m, c.plan->nwork, c.plan->block,
                                c.plan->lds, st);
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
    if (tile->n_partitioned != count) {
        // a tail: the layout does not cover every particle, so there is no
        // incremental regroup to fuse with -- deposit, then sort
        PCG_TRY(deposit_currents(grid, particles, order, tile, J, n_escaped, workspace, dbytes,
                                 stream));
        return tile_sort_impl(grid, order, tile->T, count, particles->x, n_arrays, in_arrays,
                              out_arrays, nullptr, nullptr, tile_offsets, tile, sort_ws,
                              workspace_bytes - dbytes, st, nullptr, nullptr);
    }
    RegroupCtx ctx{&plan, dim, order, 0};
    if (in_arrays && n_arrays == dim + 5) {
        bool canon = true;
        for (int k = 0; k < dim; ++k)
            canon = canon && in_arrays[k] == particles->x[k];
        for (int c = 0; c < 3; ++c)
            canon = canon && in_arrays[dim + c] == particles->v[c];
        canon = canon && in_arrays[dim + 3] == particles->q && in_arrays[dim + 4] == particles->w;
        ctx.canon = canon ? 1 : 0;
    }
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
