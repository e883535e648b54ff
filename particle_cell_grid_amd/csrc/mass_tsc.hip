// mass_tsc.hip -- scalar mass matrix with TSC weights ([MM] Pennati & Markidis,
// "Mass Matrix Assembly on Tensor Cores for Implicit PIC": §2.1 Eq.(6) in the
// scalar case, §2.3 Eq.(12) at order 2, §3.2-§3.4; the paper's TSC runs, §4.1
// Fig. 8).
//
// Each particle has 27 support nodes; its node pairs span offsets -2..2 per
// axis, so a node row of M holds 125 values, o = (dx+2) + 5 (dy+2) + 25 (dz+2).
// Particles sorted by their TSC support base (pcg_tile_sort with T = 1,
// order = 2) form groups that share all 27 nodes ([MM] §3.3 "support groups";
// the key already is the group, so one pass suffices).  Per group the 27 x 27
// block T[a][b] = sum_p c_p W_a(p) W_b(p) (c = q w) is one product over the
// group's particles: rows padded to 32 and computed as the three tiles (0,0),
// (0,1), (1,1) of v_mfma_f32_16x16x4_f32 per 4 particles (T is symmetric, so
// tile (1,0) is tile (0,1) transposed).  [MM] §3.4 adds each block to M with
// device atomics, 729 per group; the MFMA variant here sums the blocks of a
// brick of 4 x 4 x 2 groups in an LDS patch of fixed-point node rows first and
// adds the patch to M once (about 250 atomics per group, each node row of 125
// floats by consecutive lanes).
//
// Variants: MFMA (bricks), VALU (one wave per group, each lane summing its
// node pairs over the staged particles, 729 atomics per group) and FLAT (one
// thread per particle, 729 atomics; also the unsorted tail).  A particle found in a slice whose group it does not belong to (a
// stale layout) is deposited by its own lane with the flat path.
//
// The tensor (ECSIM) matrix with TSC weights ([MM] Eq.(4)-(5); §4.1 Fig. 9):
// M^ij = sum_p c_p alpha'^ij_p W_a W_b with c = q w / (1 + |omega|^2) and
// alpha' = I + omega omega^T + the rotation terms.  Each of the nine
// components is a symmetric 27 x 27 block per group, so the MFMA variant runs
// three 16x16x4 tiles per component (27 matrix instructions per 4 particles)
// and sums the upper triangles of a brick of 2 x 2 x 2 groups in an LDS patch
// that keeps one entry per unordered node pair (see the brick kernel).  The
// VALU variant forms the ten moments u_k u_l (u = (1, omega)) per lane and
// node pair and adds each group's 6561 values to M itself.
#include <algorithm>

#include "common.hpp"

namespace pcg {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int TSC_NODES = 27;
constexpr int TSC_OFFS = 125;
constexpr int TSC_WAVES = 4;

struct TscArgs {
    int n[3];
    float nf[3];
    const float *x[3];
    const float *q;
    const float *w;
    const float *B[3];  // tensor matrix only
    const float *beta;
    float *M;  // [n_z][n_y][n_x][125] (scalar) or [..][125][3][3] (tensor)
    const uint32_t *offsets;
    int64_t n_part;
    uint32_t ngroups;
    uint32_t nbricks;  // brick kernels: bricks of the grid
    uint32_t xcd_run;  // brick kernels: bricks per XCD run (xcd_item); 0: plain order
};

// One particle's TSC support: wrapped base node per axis and the 27 weights,
// node a = ax + 3 ay + 9 az.  The base is the node below the nearest one
// (fraction < 1/2: floor - 1, else floor), decided exactly in fp32; with
// t = x - (base + 1) in [-1/2, 1/2) the three weights are (1/2 - t)^2 / 2,
// 3/4 - t^2 and (1/2 + t)^2 / 2 ([MM] §2.3 Eq.(12) at order 2).
struct TscParticle {
    int base[3];
    float W[TSC_NODES];
    float c;
};

// Axis k of a particle's support: the wrapped base node and the three weights.
__device__ inline int tsc_axis(const TscArgs &m, float xk, int k, float *wk)
{
    const float x = clamp_coord(xk, m.nf[k]);
    const float fl = floorf(x);
    const bool low = x - fl < 0.5f;
    const float b = low ? fl - 1.0f : fl;
    const float t = x - (b + 1.0f);
    const int bi = (int)b;  // in [-1, n]
    wk[0] = 0.5f * (0.5f - t) * (0.5f - t);
    wk[1] = 0.75f - t * t;
    wk[2] = 0.5f * (0.5f + t) * (0.5f + t);
    return bi < 0 ? bi + m.n[k] : (bi >= m.n[k] ? bi - m.n[k] : bi);
}

__device__ inline TscParticle tsc_particle(const TscArgs &m, float x0, float x1, float x2,
                                           float q, float w)
{
    TscParticle P;
    const float xs[3] = {x0, x1, x2};
    float wk[3][3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        P.base[k] = tsc_axis(m, xs[k], k, wk[k]);
#pragma unroll
    for (int a = 0; a < TSC_NODES; ++a)
        P.W[a] = wk[0][a % 3] * wk[1][(a / 3) % 3] * wk[2][a / 9];
    P.c = q * w;
    return P;
}

__device__ inline int wrap_add(int b, int d, int n)
{
    const int i = b + d;
    return i >= n ? i - n : i;
}

// Node a of a support whose base is `base` (wrapped), as a linear index.
__device__ inline int64_t tsc_node(const TscArgs &m, const int *base, int a)
{
    const int gx = wrap_add(base[0], a % 3, m.n[0]);
    const int gy = wrap_add(base[1], (a / 3) % 3, m.n[1]);
    const int gz = wrap_add(base[2], a / 9, m.n[2]);
    return gx + (int64_t)m.n[0] * (gy + (int64_t)m.n[1] * gz);
}

// Offset of node b seen from node a of one support.
__device__ inline int tsc_offset(int a, int b)
{
    return (b % 3 - a % 3 + 2) + 5 * ((b / 3) % 3 - (a / 3) % 3 + 2) + 25 * (b / 9 - a / 9 + 2);
}

// The particle's whole 27 x 27 contribution with global atomics.
__device__ inline void tsc_deposit_global(const TscArgs &m, const TscParticle &P)
{
    for (int a = 0; a < TSC_NODES; ++a) {
        float *row = m.M + (size_t)tsc_node(m, P.base, a) * TSC_OFFS;
        const float ca = P.c * P.W[a];
        for (int b = 0; b < TSC_NODES; ++b)
            atomic_add_f32(&row[tsc_offset(a, b)], ca * P.W[b]);
    }
}

__device__ inline float ld(const float *base, int64_t p) { return base[p]; }

__global__ __launch_bounds__(256) void k_mass_tsc_flat(TscArgs m, int64_t begin, int64_t end)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < end; p += stride)
        tsc_deposit_global(m, tsc_particle(m, ld(m.x[0], p), ld(m.x[1], p), ld(m.x[2], p),
                                           ld(m.q, p), ld(m.w, p)));
}

// Per-wave LDS: one staged 64-particle batch (rows padded to 32 nodes, the pads
// zero; 36 floats apart, so that the lanes' 16-byte writes of their rows, and
// the reads of four rows at a time, spread over the banks).
struct TscStage {
    float W[64][36];
    float c[64];
};
struct TscScratch {
    TscStage s;
};

__device__ inline void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The 27 x 27 block of one group (support base gb, wrapped; slice [lo, hi)),
// one wave.  MFMA: the three 16x16 tiles (0,0), (0,1), (1,1) on the matrix
// cores, left in acc00, acc01, acc11 (register i of a lane holds entry
// (4 (lane / 16) + i, lane % 16) of its tile); VALU: each lane sums its node
// pairs pr = lane + 64 k into tv.  A particle of the slice that does not belong
// to the group (a stale layout) is deposited by its own lane with global
// atomics.
constexpr int TSC_PAIRS = (TSC_NODES * TSC_NODES + WAVE - 1) / WAVE;  // pairs per lane

// A particle's five inputs, as loaded (slot lo + lane of a slice, clamped).
struct TscRaw {
    float x[3], q, w;
};

__device__ inline TscRaw tsc_load(const TscArgs &m, int64_t lo, int64_t hi, int lane)
{
    const int64_t p = std::min<int64_t>(lo + lane, hi - 1);  // clamped
    TscRaw r;
#pragma unroll
    for (int k = 0; k < 3; ++k)
        r.x[k] = ld(m.x[k], p);
    r.q = ld(m.q, p);
    r.w = ld(m.w, p);
    return r;
}

template <bool MFMA>
__device__ inline void tsc_group_block(const TscArgs &m, TscScratch &ws, int lane, const int *gb,
                                       int64_t lo, int64_t hi, float *tv, floatx4 &acc00,
                                       floatx4 &acc01, floatx4 &acc11,
                                       const TscRaw *ahead = nullptr)
{
    const int r = lane & 15, kk = lane >> 4;
    acc00 = floatx4{0, 0, 0, 0};
    acc01 = floatx4{0, 0, 0, 0};
    acc11 = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < TSC_PAIRS; ++k)
        tv[k] = 0.0f;

    for (int64_t base = lo; base < hi; base += 64) {
        const bool valid = base + lane < hi;
        // the first two batches may come loaded by the caller (ahead[0], [1])
        const TscRaw in = (ahead && base == lo)        ? ahead[0]
                          : (ahead && base == lo + 64) ? ahead[1]
                                                       : tsc_load(m, base, hi, lane);
        const TscParticle P = tsc_particle(m, in.x[0], in.x[1], in.x[2], in.q, in.w);
        const bool home = P.base[0] == gb[0] && P.base[1] == gb[1] && P.base[2] == gb[2];
        const bool take = valid && home;
        if (valid && !home)
            tsc_deposit_global(m, P);  // stale layout: this lane deposits it alone
        wave_sync();
#pragma unroll
        for (int a = 0; a < 32; a += 4) {
            float4 v4;
            v4.x = a + 0 < TSC_NODES ? P.W[a + 0] : 0.0f;
            v4.y = a + 1 < TSC_NODES ? P.W[a + 1] : 0.0f;
            v4.z = a + 2 < TSC_NODES ? P.W[a + 2] : 0.0f;
            v4.w = a + 3 < TSC_NODES ? P.W[a + 3] : 0.0f;
            *reinterpret_cast<float4 *>(&ws.s.W[lane][a]) = v4;
        }
        // only c is zeroed for a slot outside the group: every product takes
        // c once, and the weights of a loaded particle are finite
        ws.s.c[lane] = take ? P.c : 0.0f;
        wave_sync();
        const int nb = (int)std::min<int64_t>(64, hi - base);
        if (MFMA) {
            // four 4-particle steps at a time: their operands are read first
            // (one LDS round trip), then the products, then the twelve matrix
            // instructions back to back; rows past the slice are staged as
            // zero, so a group's steps past nb add nothing
            const int steps = (nb + 3) >> 2;
            for (int i0 = 0; i0 < steps; i0 += 4) {
                float a0[4], a1[4], cq[4], b0[4], b1[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int q = 4 * (i0 + j) + kk;
                    a0[j] = ws.s.W[q][r];
                    a1[j] = ws.s.W[q][16 + r];
                    cq[j] = ws.s.c[q];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    b0[j] = cq[j] * a0[j];
                    b1[j] = cq[j] * a1[j];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc00 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b0[j], acc00, 0, 0, 0);
                    acc01 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b1[j], acc01, 0, 0, 0);
                    acc11 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j], b1[j], acc11, 0, 0, 0);
                }
            }
        } else {
            for (int q = 0; q < nb; ++q) {
                const float cq = ws.s.c[q];
#pragma unroll
                for (int k = 0; k < TSC_PAIRS; ++k) {
                    const int pr = lane + WAVE * k;
                    if (pr < TSC_NODES * TSC_NODES)
                        tv[k] += cq * ws.s.W[q][pr / TSC_NODES] * ws.s.W[q][pr % TSC_NODES];
                }
            }
        }
    }
    wave_sync();  // the staging area is free for the next group
}

// Group coordinates of linear group index g (gx + n_x (gy + n_y gz)).
__device__ inline void group_coords(const TscArgs &m, uint32_t g, int *gb)
{
    gb[0] = (int)(g % (uint32_t)m.n[0]);
    gb[1] = (int)((g / (uint32_t)m.n[0]) % (uint32_t)m.n[1]);
    gb[2] = (int)(g / ((uint32_t)m.n[0] * (uint32_t)m.n[1]));
}

// VALU variant, one wave per group: group = the wave's global index (groups
// are the support base nodes, linear index gx + n_x (gy + n_y gz)); its 729
// node pairs go to M with device atomics.
__global__ __launch_bounds__(TSC_WAVES * WAVE) void k_mass_tsc_valu(TscArgs m)
{
    __shared__ TscScratch scratch[TSC_WAVES];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    TscScratch &ws = scratch[wave];
    // neighbouring groups (which share M rows) on one XCD: blocks are dealt to
    // the 8 XCDs round-robin
    const uint32_t nblocks = (m.ngroups + TSC_WAVES - 1) / TSC_WAVES;
    const uint32_t per = (nblocks + 7) / 8;
    const uint32_t blk = (blockIdx.x % 8) * per + blockIdx.x / 8;
    const uint32_t g = blk * TSC_WAVES + wave;
    if (blk >= nblocks || g >= m.ngroups)
        return;
    const int64_t lo = std::min<int64_t>(m.offsets[g], m.n_part);
    const int64_t hi = std::min<int64_t>(m.offsets[g + 1], m.n_part);
    if (hi <= lo)
        return;
    int gb[3];
    group_coords(m, g, gb);
    float tv[TSC_PAIRS];
    floatx4 unused[3];
    tsc_group_block<false>(m, ws, lane, gb, lo, hi, tv, unused[0], unused[1], unused[2]);
#pragma unroll
    for (int k = 0; k < TSC_PAIRS; ++k) {
        const int pr = lane + WAVE * k;
        if (pr < TSC_NODES * TSC_NODES) {
            const int a = pr / TSC_NODES, b = pr % TSC_NODES;
            atomic_add_f32(&m.M[(size_t)tsc_node(m, gb, a) * TSC_OFFS + tsc_offset(a, b)],
                           tv[k]);
        }
    }
}

// The same matrix with the groups of a brick of TB_X x TB_Y x TB_Z bases per
// work-group: each group's block is added into an LDS patch of the brick's
// (TB + 2)^3 nodes x 125 offsets in 32-bit fixed point (integer LDS atomics,
// exact and order-independent), and the patch goes to M once, each node row of
// 125 floats by consecutive lanes: some 36 cache-line atomics per group instead
// of about 240 when every group adds its 729 values to M itself.  The scale
// 2^k keeps every partial sum of a patch entry below 2^30: a particle adds at
// most (3/4)^2 |q w| to an entry, so 2^k (9/16) sum|q w| over the brick's
// particles < 2^30 bounds them all (products are rounded to the nearest unit,
// 2^-k, so the error of an entry is at most half a unit per particle).
constexpr int TB_X = 4, TB_Y = 4, TB_Z = 2;
constexpr int TP_X = TB_X + 2, TP_Y = TB_Y + 2, TP_Z = TB_Z + 2;
constexpr int TP_NODES = TP_X * TP_Y * TP_Z;
constexpr size_t TSC_PATCH_BYTES = (size_t)TP_NODES * TSC_OFFS * 4;
constexpr int TSC_BRICK_WAVES = 8;

// The patch entries a brick's groups can reach: node pairs at most 2 apart on
// every axis (5 b + 4 per axis for b groups), as (row, offset) in row-major
// order, so consecutive entries are consecutive floats of M.  Entry: patch
// index | lx << 15 | ly << 18 | lz << 21 | o << 23 (the row's local node, the
// offset).
constexpr int TS_FULL = (5 * TB_X + 4) * (5 * TB_Y + 4) * (5 * TB_Z + 4);
struct TsTable {
    uint32_t e[TS_FULL];
    int count;
};
constexpr TsTable ts_table()
{
    TsTable t{};
    for (int lz = 0; lz < TP_Z; ++lz)
        for (int ly = 0; ly < TP_Y; ++ly)
            for (int lx = 0; lx < TP_X; ++lx)
                for (int o = 0; o < TSC_OFFS; ++o) {
                    const int mx = lx + o % 5 - 2, my = ly + (o / 5) % 5 - 2, mz = lz + o / 25 - 2;
                    if (mx < 0 || mx >= TP_X || my < 0 || my >= TP_Y || mz < 0 || mz >= TP_Z)
                        continue;
                    const int ln = lx + TP_X * (ly + TP_Y * lz);
                    if (t.count < TS_FULL)
                        t.e[t.count] = (uint32_t)(ln * TSC_OFFS + o) | (uint32_t)lx << 15 |
                                       (uint32_t)ly << 18 | (uint32_t)lz << 21 |
                                       (uint32_t)o << 23;
                    ++t.count;
                }
    return t;
}
static_assert(ts_table().count == TS_FULL, "reachable patch entries");
static_assert(TP_NODES * TSC_OFFS <= (1 << 15) && TP_X <= 8 && TP_Y <= 8 && TP_Z <= 4,
              "fields of a patch entry");
__device__ constexpr TsTable TS = ts_table();

__global__ __launch_bounds__(TSC_BRICK_WAVES * WAVE) void k_mass_tsc_brick(TscArgs m)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int *patch = reinterpret_cast<int *>(smem);  // [TP_NODES][125]
    __shared__ TscScratch scratch[TSC_BRICK_WAVES];
    __shared__ float red[TSC_BRICK_WAVES];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    TscScratch &ws = scratch[wave];
    const int nbx = (m.n[0] + TB_X - 1) / TB_X, nby = (m.n[1] + TB_Y - 1) / TB_Y;
    const int bi = (int)(blockIdx.x % (uint32_t)nbx);
    const int bj = (int)((blockIdx.x / (uint32_t)nbx) % (uint32_t)nby);
    const int bk = (int)(blockIdx.x / ((uint32_t)nbx * (uint32_t)nby));
    const int org[3] = {bi * TB_X, bj * TB_Y, bk * TB_Z};
    const int cnt[3] = {min(TB_X, m.n[0] - org[0]), min(TB_Y, m.n[1] - org[1]),
                        min(TB_Z, m.n[2] - org[2])};
    const int ngb = cnt[0] * cnt[1] * cnt[2];
    for (int i = threadIdx.x; i < TP_NODES * TSC_OFFS; i += blockDim.x)
        patch[i] = 0;
    // the brick's local group j: base org + (j % cnt0, (j / cnt0) % cnt1, j / (cnt0 cnt1))
    auto local = [&](int j, int *lg) {
        lg[0] = j % cnt[0];
        lg[1] = (j / cnt[0]) % cnt[1];
        lg[2] = j / (cnt[0] * cnt[1]);
    };
    auto slice = [&](const int *lg, int64_t &lo, int64_t &hi) {
        const uint32_t g = (uint32_t)(org[0] + lg[0]) +
                           (uint32_t)m.n[0] * ((uint32_t)(org[1] + lg[1]) +
                                               (uint32_t)m.n[1] * (uint32_t)(org[2] + lg[2]));
        lo = std::min<int64_t>(m.offsets[g], m.n_part);
        hi = std::max<int64_t>(lo, std::min<int64_t>(m.offsets[g + 1], m.n_part));
    };
    // the first two batches of each group (most groups hold 50 to 80
    // particles) are loaded while the wave's previous group is computed
    int64_t nlo = 0, nhi = 0;
    TscRaw nxt[2] = {};
    auto prefetch = [&](int j) {
        int lg[3];
        local(j, lg);
        slice(lg, nlo, nhi);
        if (nhi > nlo)
            nxt[0] = tsc_load(m, nlo, nhi, lane);
        if (nhi > nlo + 64)
            nxt[1] = tsc_load(m, nlo + 64, nhi, lane);
    };
    if (wave < ngb)
        prefetch(wave);  // in flight during the sum below
    // sum |q w| over the brick's particles (every wave its groups)
    float sum = 0.0f;
    for (int j = wave; j < ngb; j += TSC_BRICK_WAVES) {
        int lg[3];
        local(j, lg);
        int64_t lo, hi;
        slice(lg, lo, hi);
        for (int64_t p = lo + lane; p < hi; p += WAVE)
            sum += fabsf(ld(m.q, p) * ld(m.w, p));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        sum += __shfl_xor(sum, off);
    if (lane == 0)
        red[wave] = sum;
    __syncthreads();
    float total = 0.0f;
#pragma unroll
    for (int w = 0; w < TSC_BRICK_WAVES; ++w)
        total += red[w];
    if (total == 0.0f)
        return;  // no particle adds anything (every wave sees the same total)
    // 2^k (9/16) total < 2^30: half the int32 range, which covers the fp32
    // rounding of the sum and the half unit each rounded product may add
    int e = 0;
    frexpf(0.5625f * total, &e);  // value < 2^e
    const int k_scale = max(-126, min(126, 30 - e));
    const float scale = ldexpf(1.0f, k_scale), inv_scale = ldexpf(1.0f, -k_scale);

    // The lane's accumulator entries: slot 4 t + i is entry (a, b) of tile t
    // (0: (0,0), 1: (0,1), 2: (1,1)), a = 16 (t == 2) + 4 (lane / 16) + i,
    // b = 16 (t >= 1) + lane % 16; slot 12 + i is the transposed entry (b, a)
    // of tile (0,1), which stands for tile (1,0).  Each goes to the patch
    // straight from the registers, at a fixed offset from the group's row.
    const int r = lane & 15, kk = lane >> 4;
    auto patch_node = [](int a) { return a % 3 + TP_X * ((a / 3) % 3 + TP_Y * (a / 9)); };
    int cst[16];
    uint32_t live = 0;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int a = (t == 2 ? 16 : 0) + 4 * kk + i, b = (t >= 1 ? 16 : 0) + r;
            const bool ok = a < TSC_NODES && b < TSC_NODES;
            live |= ok ? 1u << (4 * t + i) : 0u;
            cst[4 * t + i] = ok ? patch_node(a) * TSC_OFFS + tsc_offset(a, b) : 0;
            if (t == 1) {
                live |= ok ? 1u << (12 + i) : 0u;
                cst[12 + i] = ok ? patch_node(b) * TSC_OFFS + tsc_offset(b, a) : 0;
            }
        }
    for (int j = wave; j < ngb; j += TSC_BRICK_WAVES) {
        int lg[3];
        local(j, lg);
        const int64_t lo = nlo, hi = nhi;
        const TscRaw cur[2] = {nxt[0], nxt[1]};
        if (j + TSC_BRICK_WAVES < ngb)
            prefetch(j + TSC_BRICK_WAVES);
        if (hi <= lo)
            continue;
        int gb[3];
#pragma unroll
        for (int k = 0; k < 3; ++k)
            gb[k] = org[k] + lg[k];
        float tv[TSC_PAIRS];
        floatx4 acc[3];
        tsc_group_block<true>(m, ws, lane, gb, lo, hi, tv, acc[0], acc[1], acc[2], cur);
        int *row = patch + (lg[0] + TP_X * (lg[1] + TP_Y * lg[2])) * TSC_OFFS;
#pragma unroll
        for (int sl = 0; sl < 16; ++sl)
            if (live & (1u << sl))
                atomicAdd(&row[cst[sl]],
                          __float2int_rn((sl < 12 ? acc[sl / 4][sl % 4] : acc[1][sl - 12]) * scale));
    }
    __syncthreads();
    // the patch to M: the reachable entries, consecutive threads on consecutive
    // floats of M; four entries at a time, their table words and patch values
    // read first; entries no group touched stay zero and are skipped
    constexpr int FL_UNROLL = 4;
    for (int f0 = threadIdx.x; f0 < TS_FULL; f0 += FL_UNROLL * blockDim.x) {
        uint32_t e[FL_UNROLL];
        int v[FL_UNROLL];
#pragma unroll
        for (int u = 0; u < FL_UNROLL; ++u) {
            const int f = f0 + u * (int)blockDim.x;
            e[u] = f < TS_FULL ? TS.e[f] : 0u;
        }
#pragma unroll
        for (int u = 0; u < FL_UNROLL; ++u)
            v[u] = f0 + u * (int)blockDim.x < TS_FULL ? patch[e[u] & 0x7fffu] : 0;
#pragma unroll
        for (int u = 0; u < FL_UNROLL; ++u) {
            if (v[u] == 0)
                continue;
            const int gx = wrap_add(org[0], (int)((e[u] >> 15) & 7u), m.n[0]);
            const int gy = wrap_add(org[1], (int)((e[u] >> 18) & 7u), m.n[1]);
            const int gz = wrap_add(org[2], (int)((e[u] >> 21) & 3u), m.n[2]);
            const size_t node =
                (size_t)gx + (size_t)m.n[0] * ((size_t)gy + (size_t)m.n[1] * gz);
            atomic_add_f32(&m.M[node * TSC_OFFS + (e[u] >> 23)], (float)v[u] * inv_scale);
        }
    }
}

// ---------------------------------------------------------------- tensor matrix

// omega = beta B, u = (1, omega), c = q w / (1 + |omega|^2).
__device__ inline void tsc_alpha(const TscArgs &m, int64_t p, float q, float w, float *u,
                                 float &c)
{
    const float bt = ld(m.beta, p);
    const float o0 = bt * ld(m.B[0], p), o1 = bt * ld(m.B[1], p), o2 = bt * ld(m.B[2], p);
    u[0] = 1.0f;
    u[1] = o0;
    u[2] = o1;
    u[3] = o2;
    c = q * w / (1.0f + (o0 * o0 + o1 * o1 + o2 * o2));
}

// Adds moment t of pair (k, l) into the nine components of a block ([MM]
// Eq.(5) written out: +eps_ijk omega_k for the rotation, omega_i omega_j).
__device__ inline void add_moment(int k, int l, float t, float *blk)
{
    if (k == 0 && l == 0) {
        blk[0] += t;
        blk[4] += t;
        blk[8] += t;
    } else if (k == 0) {  // T_0(l): omega_{l-1} in the rotation
        if (l == 1) {
            blk[5] += t;  // yz
            blk[7] -= t;  // zy
        } else if (l == 2) {
            blk[2] -= t;  // xz
            blk[6] += t;  // zx
        } else {
            blk[1] += t;  // xy
            blk[3] -= t;  // yx
        }
    } else {  // T_(i+1)(j+1) = omega_i omega_j, into (i, j) and (j, i)
        const int i = k - 1, j = l - 1;
        blk[3 * i + j] += t;
        if (i != j)
            blk[3 * j + i] += t;
    }
}

// The particle's whole 27 x 27 x 9 contribution with global atomics.
__device__ inline void tsc_tensor_global(const TscArgs &m, const TscParticle &P, const float *u,
                                         float c)
{
    for (int a = 0; a < TSC_NODES; ++a) {
        float *row = m.M + (size_t)tsc_node(m, P.base, a) * TSC_OFFS * 9;
        for (int b = 0; b < TSC_NODES; ++b) {
            const float wab = c * P.W[a] * P.W[b];
            float blk[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
            for (int k = 0; k < 4; ++k)
                for (int l = k; l < 4; ++l)
                    add_moment(k, l, wab * u[k] * u[l], blk);
            float *dst = row + tsc_offset(a, b) * 9;
            for (int ij = 0; ij < 9; ++ij)
                atomic_add_f32(&dst[ij], blk[ij]);
        }
    }
}

__global__ __launch_bounds__(256) void k_mass_tsc_tensor_flat(TscArgs m, int64_t begin,
                                                              int64_t end)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < end;
         p += stride) {
        const float q = ld(m.q, p), w = ld(m.w, p);
        const TscParticle P = tsc_particle(m, ld(m.x[0], p), ld(m.x[1], p), ld(m.x[2], p), q, w);
        float u[4], c;
        tsc_alpha(m, p, q, w, u, c);
        tsc_tensor_global(m, P, u, c);
    }
}

// The VALU variant: one wave per group, each lane summing the nine components
// of its node pairs (lane + 64 k) over the staged particles; the block goes to
// M with 6561 device atomics, staged in LDS so that consecutive lanes add
// consecutive floats of M (a lane per pair would put 36 bytes between
// neighbouring lanes' addresses).
struct TscTensorStage {
    float W[64][32];
    float u[64][4];
    float c[64];
};
// pairs per lane (729 over 64 lanes: TSC_PAIRS), flushed in two halves
constexpr int TSC_HALF = (TSC_PAIRS + 1) / 2;
union TscTensorScratch {
    TscTensorStage s;
    float F[WAVE * TSC_HALF * 9];  // one half's blocks, pair-major
};

// the ten moments (k <= l) in a fixed order
__device__ constexpr int MOM_K[10] = {0, 0, 0, 0, 1, 1, 1, 2, 2, 3};
__device__ constexpr int MOM_L[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};

__global__ __launch_bounds__(TSC_WAVES * WAVE) void k_mass_tsc_tensor_valu(TscArgs m)
{
    __shared__ TscTensorScratch scratch[TSC_WAVES];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    TscTensorScratch &ws = scratch[wave];
    const uint32_t nblocks = (m.ngroups + TSC_WAVES - 1) / TSC_WAVES;
    const uint32_t per = (nblocks + 7) / 8;
    const uint32_t blk_id = (blockIdx.x % 8) * per + blockIdx.x / 8;
    const uint32_t g = blk_id * TSC_WAVES + wave;
    if (blk_id >= nblocks || g >= m.ngroups)
        return;
    const int64_t lo = std::min<int64_t>(m.offsets[g], m.n_part);
    const int64_t hi = std::min<int64_t>(m.offsets[g + 1], m.n_part);
    if (hi <= lo)
        return;
    int gb[3];
    group_coords(m, g, gb);

    // lane owns node pairs lane + 64 k (k < 12) and their 9 components
    float tv[TSC_PAIRS][9];
#pragma unroll
    for (int k = 0; k < TSC_PAIRS; ++k)
#pragma unroll
        for (int ij = 0; ij < 9; ++ij)
            tv[k][ij] = 0.0f;

    for (int64_t base = lo; base < hi; base += 64) {
        const int64_t p = std::min<int64_t>(base + lane, hi - 1);  // clamped
        const bool valid = base + lane < hi;
        const float q = ld(m.q, p), w = ld(m.w, p);
        const TscParticle P = tsc_particle(m, ld(m.x[0], p), ld(m.x[1], p), ld(m.x[2], p), q, w);
        float u[4], c;
        tsc_alpha(m, p, q, w, u, c);
        const bool home = P.base[0] == gb[0] && P.base[1] == gb[1] && P.base[2] == gb[2];
        const bool take = valid && home;
        if (valid && !home)
            tsc_tensor_global(m, P, u, c);  // stale layout: this lane deposits it alone
        wave_sync();
#pragma unroll
        for (int a = 0; a < 32; a += 4) {
            float4 v4;
            v4.x = a + 0 < TSC_NODES ? P.W[a + 0] : 0.0f;
            v4.y = a + 1 < TSC_NODES ? P.W[a + 1] : 0.0f;
            v4.z = a + 2 < TSC_NODES ? P.W[a + 2] : 0.0f;
            v4.w = a + 3 < TSC_NODES ? P.W[a + 3] : 0.0f;
            *reinterpret_cast<float4 *>(&ws.s.W[lane][a]) = v4;
        }
        *reinterpret_cast<float4 *>(ws.s.u[lane]) = make_float4(u[0], u[1], u[2], u[3]);
        ws.s.c[lane] = take ? c : 0.0f;  // the factor of every product
        wave_sync();
        const int nb = (int)std::min<int64_t>(64, hi - base);
        for (int qq = 0; qq < nb; ++qq) {
            const float cq = ws.s.c[qq];
            const float4 uq = *reinterpret_cast<const float4 *>(ws.s.u[qq]);
            const float uk[4] = {uq.x, uq.y, uq.z, uq.w};
#pragma unroll
            for (int k2 = 0; k2 < TSC_PAIRS; ++k2) {
                const int pr = lane + WAVE * k2;
                if (pr < TSC_NODES * TSC_NODES) {
                    const float wab = cq * ws.s.W[qq][pr / TSC_NODES] * ws.s.W[qq][pr % TSC_NODES];
#pragma unroll
                    for (int mo = 0; mo < 10; ++mo)
                        add_moment(MOM_K[mo], MOM_L[mo], wab * uk[MOM_K[mo]] * uk[MOM_L[mo]],
                                   tv[k2]);
                }
            }
        }
    }
    wave_sync();
    // per half of the lane's pairs (lane + 64 (h TSC_HALF + k2)): the half's
    // 64 TSC_HALF x 9 floats flushed with consecutive lanes on consecutive
    // values v: pair 64 h TSC_HALF + v / 9, component v % 9
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k2 = 0; k2 < TSC_HALF; ++k2)
#pragma unroll
            for (int ij = 0; ij < 9; ++ij)
                ws.F[(k2 * WAVE + lane) * 9 + ij] = tv[h * TSC_HALF + k2][ij];
        wave_sync();
        for (int v = lane; v < WAVE * TSC_HALF * 9; v += WAVE) {
            const int pl = v / 9, ij = v - 9 * pl;
            const int pr = WAVE * TSC_HALF * h + pl;
            if (pr < TSC_NODES * TSC_NODES) {
                const int a = pr / TSC_NODES, b = pr % TSC_NODES;
                atomic_add_f32(
                    &m.M[((size_t)tsc_node(m, gb, a) * TSC_OFFS + tsc_offset(a, b)) * 9 + ij],
                    ws.F[v]);
            }
        }
        wave_sync();
    }
}

// ------------------------------------------------- tensor matrix in bricks
//
// Each component of the tensor matrix is itself a scalar-type matrix,
// M^ij_{g g'} = sum_p c_p alpha'^ij_p W_g(p) W_g'(p) with c = q w / (1 + |omega|^2)
// and alpha' = I + omega omega^T plus the rotation (+omega_z at (x,y), -omega_y
// at (x,z), ... as in add_moment): nine symmetric 27 x 27 blocks per group,
// three 16x16x4 tiles each (A = W_a, B = c alpha'^ij W_b), 27 matrix
// instructions per 4 particles and no moments to combine afterwards.  A
// work-group takes a brick of 2 x 2 x 2 groups and sums their blocks in an LDS
// patch of 32-bit fixed-point values, scaled as in k_mass_tsc_brick (|alpha^ij|
// <= 1: alpha is the inverse of I - [omega]x, whose singular values are >= 1).
// The brick's groups reach nodes 0..3 (local) per axis and a node pair
// (la, lb) of an axis occurs iff |la - lb| <= 2: 14 pairs per axis, 2744 node
// pairs.  As every component block is symmetric in its two nodes, the patch
// keeps one of (A, B) and (B, A), the one whose offset B - A is >= 0 in
// (z, y, x) order ("canonical"): 1404 pairs x 9 components, 50.5 KB, so two
// work-groups share a CU.  A group adds only its blocks' upper triangles (node
// b >= a in support order, which is exactly the canonical half), and the
// flush writes every pair of the brick, reading the canonical entry:
// 3087 device atomics per group instead of 6561, in runs of consecutive M
// floats.
constexpr int TT_B = 2;                  // groups per brick edge
constexpr int TT_N = TT_B + 2;           // patch nodes per axis
constexpr int TT_ALL = 5 * TT_B + 4;     // per axis: node pairs with |la - lb| <= 2
constexpr int TT_POS = 2 * TT_B + 1;     //   ... with lb > la
constexpr int TT_NN = 3 * TT_B + 3;      //   ... with lb >= la
constexpr int TT_FULL = TT_ALL * TT_ALL * TT_ALL;
constexpr int TT_ZBLK = TT_POS * TT_ALL + TT_N * TT_NN;
constexpr int TT_HALF = TT_POS * TT_ALL * TT_ALL + TT_N * TT_ZBLK;
constexpr int TT_UPPER = TSC_NODES * (TSC_NODES + 1) / 2;  // pairs a <= b of a support
constexpr int TT_WAVES = 4;
// a patch entry: the nine components as five 64-bit words, components 2 w and
// 2 w + 1 packed in word w (the last word holds component 8 alone)
constexpr int TT_WORDS = 5;
constexpr size_t TT_PATCH_BYTES = (size_t)TT_HALF * TT_WORDS * sizeof(unsigned long long);
constexpr uint32_t TT_XCD_RUN = 64;
static_assert(TT_B == 2, "the per-axis closed forms below are for bricks of edge 2");

// Per-axis pair indices (la, lb in 0..3): every pair, ordered by la then lb;
// the pairs with lb > la; the pairs with lb >= la.
__host__ __device__ constexpr int tt_all(int la, int lb)
{
    return 4 * la - (la > 0) - (la == 3) + lb;
}
__host__ __device__ constexpr int tt_pos(int la, int lb) { return la + lb - 1; }
__host__ __device__ constexpr int tt_nn(int la, int lb) { return la == 3 ? 8 : 2 * la + lb; }

// Patch index of the canonical pair (A, B): offset in z > 0; else in y > 0;
// else in x >= 0.
__host__ __device__ constexpr int tt_half(int ax, int ay, int az, int bx, int by, int bz)
{
    return bz > az ? (tt_pos(az, bz) * TT_ALL + tt_all(ay, by)) * TT_ALL + tt_all(ax, bx)
                   : TT_POS * TT_ALL * TT_ALL + az * TT_ZBLK +
                         (by > ay ? tt_pos(ay, by) * TT_ALL + tt_all(ax, bx)
                                  : TT_POS * TT_ALL + ay * TT_NN + tt_nn(ax, bx));
}

// Every canonical pair of the 4^3 patch nodes (offsets -2..2) has its own
// index below TT_HALF, and none is left over.
constexpr bool tt_half_is_a_bijection()
{
    bool seen[TT_HALF] = {};
    int count = 0;
    for (int A = 0; A < TT_N * TT_N * TT_N; ++A)
        for (int o = 0; o < TSC_OFFS; ++o) {
            const int ax = A % TT_N, ay = (A / TT_N) % TT_N, az = A / (TT_N * TT_N);
            const int dx = o % 5 - 2, dy = (o / 5) % 5 - 2, dz = o / 25 - 2;
            const int bx = ax + dx, by = ay + dy, bz = az + dz;
            if (bx < 0 || bx >= TT_N || by < 0 || by >= TT_N || bz < 0 || bz >= TT_N)
                continue;
            if (!(dz > 0 || (dz == 0 && (dy > 0 || (dy == 0 && dx >= 0)))))
                continue;
            const int h = tt_half(ax, ay, az, bx, by, bz);
            if (h < 0 || h >= TT_HALF || seen[h])
                return false;
            seen[h] = true;
            ++count;
        }
    return count == TT_HALF;
}
static_assert(tt_half_is_a_bijection(), "patch index of the canonical pairs");

struct TtTables {
    // node pair f of the brick (x pair fastest, pairs by tt_all per axis):
    // canonical patch index | local node A (ax + 4 ay + 16 az) << 11 | offset o << 17
    uint32_t dec[TT_FULL];
    // group cell c = cx + 2 cy + 4 cz of the brick, support pair u (a <= b,
    // row-major: u = 27 a - a (a - 1) / 2 + b - a): patch index
    uint16_t h[8][TT_UPPER];
};

constexpr TtTables tt_tables()
{
    TtTables t{};
    int la[TT_ALL] = {}, lb[TT_ALL] = {};
    for (int a = 0; a < TT_N; ++a)
        for (int b = 0; b < TT_N; ++b)
            if (a - b <= 2 && b - a <= 2) {
                la[tt_all(a, b)] = a;
                lb[tt_all(a, b)] = b;
            }
    for (int f = 0; f < TT_FULL; ++f) {
        const int p[3] = {f % TT_ALL, (f / TT_ALL) % TT_ALL, f / (TT_ALL * TT_ALL)};
        const int A[3] = {la[p[0]], la[p[1]], la[p[2]]}, B[3] = {lb[p[0]], lb[p[1]], lb[p[2]]};
        const int d[3] = {B[0] - A[0], B[1] - A[1], B[2] - A[2]};
        const bool canon = d[2] > 0 || (d[2] == 0 && (d[1] > 0 || (d[1] == 0 && d[0] >= 0)));
        const int h = canon ? tt_half(A[0], A[1], A[2], B[0], B[1], B[2])
                            : tt_half(B[0], B[1], B[2], A[0], A[1], A[2]);
        const int o = (d[0] + 2) + 5 * (d[1] + 2) + 25 * (d[2] + 2);
        t.dec[f] = (uint32_t)h | (uint32_t)(A[0] + TT_N * A[1] + TT_N * TT_N * A[2]) << 11 |
                   (uint32_t)o << 17;
    }
    int u = 0;
    for (int a = 0; a < TSC_NODES; ++a)
        for (int b = a; b < TSC_NODES; ++b, ++u) {
            for (int c = 0; c < 8; ++c) {
                const int cx = c & 1, cy = (c >> 1) & 1, cz = c >> 2;
                t.h[c][u] = (uint16_t)tt_half(cx + a % 3, cy + (a / 3) % 3, cz + a / 9,
                                              cx + b % 3, cy + (b / 3) % 3, cz + b / 9);
            }
        }
    return t;
}
__device__ constexpr TtTables TT = tt_tables();

// Per-wave LDS: one staged batch of 64 particles, each c alpha'^ij (at 0..8)
// and the nine axis weights (x0..2 y0..2 z0..2 at 9..17); rows of 20 floats, so
// that the lanes' 16-byte writes of a row cover all banks.
constexpr int TT_ROW = 20, TT_AXW = 9;
struct __attribute__((aligned(16))) TtScratch {
    float v[64][TT_ROW];
};

// One of the two sums of a patch word: the low one (signed 32-bit), or the
// high one, the word less the low sum shifted down.
__device__ inline int tt_split(unsigned long long word, int high)
{
    const int lo = (int)(uint32_t)word;
    return high ? (int)((long long)(word - (unsigned long long)(long long)lo) >> 32) : lo;
}

// A particle's nine inputs, as loaded (slot base + lane of a slice, clamped).
struct TtRaw {
    float x[3], q, w, B[3], beta;
};

__device__ inline TtRaw tt_load(const TscArgs &m, int64_t base, int64_t hi, int lane)
{
    const int64_t p = std::min<int64_t>(base + lane, hi - 1);  // clamped
    TtRaw r;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        r.x[k] = ld(m.x[k], p);
        r.B[k] = ld(m.B[k], p);
    }
    r.q = ld(m.q, p);
    r.w = ld(m.w, p);
    r.beta = ld(m.beta, p);
    return r;
}

__global__ __launch_bounds__(TT_WAVES * WAVE, 2) void k_mass_tsc_tensor_brick(TscArgs m)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // [TT_HALF][TT_WORDS]: two 32-bit fixed-point sums per word, added as one
    // 64-bit integer (the low sum signed: the high one gets its borrow back
    // when the word is split, as every partial sum stays below 2^30)
    unsigned long long *patch = reinterpret_cast<unsigned long long *>(smem);
    __shared__ TtScratch scratch[TT_WAVES];
    __shared__ float red[TT_WAVES];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    TtScratch &ws = scratch[wave];
    // runs of neighbouring bricks (which add to the same rows of M) on one XCD
    const uint32_t brick = xcd_item(blockIdx.x, m.xcd_run);
    if (brick >= m.nbricks)
        return;
    const int nbx = (m.n[0] + TT_B - 1) / TT_B, nby = (m.n[1] + TT_B - 1) / TT_B;
    const int bi = (int)(brick % (uint32_t)nbx);
    const int bj = (int)((brick / (uint32_t)nbx) % (uint32_t)nby);
    const int bk = (int)(brick / ((uint32_t)nbx * (uint32_t)nby));
    const int org[3] = {bi * TT_B, bj * TT_B, bk * TT_B};
    const int cnt[3] = {min(TT_B, m.n[0] - org[0]), min(TT_B, m.n[1] - org[1]),
                        min(TT_B, m.n[2] - org[2])};
    const int ngb = cnt[0] * cnt[1] * cnt[2];
    {
        int4 *p4 = reinterpret_cast<int4 *>(patch);
        for (int i = threadIdx.x; i < TT_HALF * TT_WORDS / 2; i += blockDim.x)
            p4[i] = int4{0, 0, 0, 0};
    }
    static_assert(TT_HALF * TT_WORDS % 2 == 0, "patch cleared as int4");
    auto local = [&](int j, int *lg) {
        lg[0] = j % cnt[0];
        lg[1] = (j / cnt[0]) % cnt[1];
        lg[2] = j / (cnt[0] * cnt[1]);
    };
    auto slice = [&](const int *lg, int64_t &lo, int64_t &hi) {
        const uint32_t g = (uint32_t)(org[0] + lg[0]) +
                           (uint32_t)m.n[0] * ((uint32_t)(org[1] + lg[1]) +
                                               (uint32_t)m.n[1] * (uint32_t)(org[2] + lg[2]));
        lo = std::min<int64_t>(m.offsets[g], m.n_part);
        hi = std::max<int64_t>(lo, std::min<int64_t>(m.offsets[g + 1], m.n_part));
    };
    // a wave's groups are j = wave and wave + TT_WAVES; their first batches are
    // loaded up front and serve the sum of |q w| as well
    static_assert(TT_B * TT_B * TT_B <= 2 * TT_WAVES, "two groups per wave at most");
    int64_t glo[2] = {0, 0}, ghi[2] = {0, 0};
    TtRaw first[2] = {};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int j = wave + TT_WAVES * t;
        if (j < ngb) {
            int lg[3];
            local(j, lg);
            slice(lg, glo[t], ghi[t]);
            if (ghi[t] > glo[t])
                first[t] = tt_load(m, glo[t], ghi[t], lane);
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (glo[t] + lane < ghi[t])
            sum += fabsf(first[t].q * first[t].w);
        for (int64_t p = glo[t] + WAVE + lane; p < ghi[t]; p += WAVE)
            sum += fabsf(ld(m.q, p) * ld(m.w, p));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        sum += __shfl_xor(sum, off);
    if (lane == 0)
        red[wave] = sum;
    __syncthreads();
    float total = 0.0f;
#pragma unroll
    for (int w = 0; w < TT_WAVES; ++w)
        total += red[w];
    if (total == 0.0f)
        return;  // nothing to add (every wave sees the same total)
    // a particle adds at most (9/16) |q w| to an entry: 2^k (9/16) total < 2^30
    int e = 0;
    frexpf(0.5625f * total, &e);
    const int k_scale = max(-126, min(126, 30 - e));
    const float scale = ldexpf(1.0f, k_scale), inv_scale = ldexpf(1.0f, -k_scale);

    const int r = lane & 15, kk = lane >> 4;
    // the lane's rows of the MFMA operands: node r and node 16 + r (< 27 for r < 11)
    const int ra[3] = {TT_AXW + r % 3, TT_AXW + 3 + (r / 3) % 3, TT_AXW + 6 + r / 9};
    const int s16 = r < 11 ? 16 + r : 0;
    const int sa[3] = {TT_AXW + s16 % 3, TT_AXW + 3 + (s16 / 3) % 3, TT_AXW + 6 + s16 / 9};
    // The lane's twelve accumulator values per component: slot 4 t + i holds
    // entry (a, b) of tile t (0: (0,0), 1: (0,1), 2: (1,1)), a = 16 (t == 2) +
    // 4 (lane / 16) + i, b = 16 (t >= 1) + lane % 16.  The slots on or above
    // the diagonal of the 27 x 27 block go to the patch straight from the
    // registers; their support pair index u (upper triangle, row-major) is
    // fixed per lane.
    int up[12];
    uint32_t live = 0;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int a = (t == 2 ? 16 : 0) + 4 * kk + i, b = (t >= 1 ? 16 : 0) + r;
            const bool ok = a <= b && b < TSC_NODES;
            live |= ok ? 1u << (4 * t + i) : 0u;
            up[4 * t + i] = ok ? a * TSC_NODES - a * (a - 1) / 2 + (b - a) : 0;
        }

    for (int t = 0; t < 2; ++t) {
        const int j = wave + TT_WAVES * t;
        const int64_t lo = glo[t], hi = ghi[t];
        if (j >= ngb || hi <= lo)
            continue;
        int lg[3];
        local(j, lg);
        const TtRaw cur = t == 0 ? first[0] : first[1];
        const int gb[3] = {org[0] + lg[0], org[1] + lg[1], org[2] + lg[2]};
        floatx4 acc[27];
#pragma unroll
        for (int i = 0; i < 27; ++i)
            acc[i] = floatx4{0, 0, 0, 0};
        for (int64_t base = lo; base < hi; base += 64) {
            const bool valid = base + lane < hi;
            const TtRaw in = base == lo ? cur : tt_load(m, base, hi, lane);
            const float x0 = in.x[0], x1 = in.x[1], x2 = in.x[2], q = in.q, w = in.w;
            const float o0 = in.beta * in.B[0], o1 = in.beta * in.B[1], o2 = in.beta * in.B[2];
            float wk[3][3];
            const int b0 = tsc_axis(m, x0, 0, wk[0]), b1 = tsc_axis(m, x1, 1, wk[1]),
                      b2 = tsc_axis(m, x2, 2, wk[2]);
            const bool home = b0 == gb[0] && b1 == gb[1] && b2 == gb[2];
            const float c = q * w / (1.0f + (o0 * o0 + o1 * o1 + o2 * o2));
            if (valid && !home) {  // stale layout: this lane deposits it alone
                const float u[4] = {1.0f, o0, o1, o2};
                tsc_tensor_global(m, tsc_particle(m, x0, x1, x2, q, w), u, c);
            }
            // c alpha'^ij, or 0 for a slot outside the group (the weights of a
            // loaded particle are finite, so its products vanish)
            const float cc = valid && home ? c : 0.0f;
            wave_sync();
            float4 *row = reinterpret_cast<float4 *>(ws.v[lane]);
            row[0] = make_float4(cc * (1.0f + o0 * o0), cc * (o2 + o0 * o1),
                                 cc * (o0 * o2 - o1), cc * (o1 * o0 - o2));
            row[1] = make_float4(cc * (1.0f + o1 * o1), cc * (o0 + o1 * o2),
                                 cc * (o1 + o2 * o0), cc * (o2 * o1 - o0));
            row[2] = make_float4(cc * (1.0f + o2 * o2), wk[0][0], wk[0][1], wk[0][2]);
            row[3] = make_float4(wk[1][0], wk[1][1], wk[1][2], wk[2][0]);
            row[4] = make_float4(wk[2][1], wk[2][2], 0.0f, 0.0f);
            wave_sync();
            const int nb = (int)std::min<int64_t>(64, hi - base);
            const int steps = (nb + 3) >> 2;
            for (int i = 0; i < steps; ++i) {
                const float *sv = ws.v[4 * i + kk];
                const float wr = sv[ra[0]] * sv[ra[1]] * sv[ra[2]];
                const float wsv = r < 11 ? sv[sa[0]] * sv[sa[1]] * sv[sa[2]] : 0.0f;
                const float4 c0 = *reinterpret_cast<const float4 *>(sv);
                const float4 c1 = *reinterpret_cast<const float4 *>(sv + 4);
                const float ca[9] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w, sv[8]};
                float bb0[9], bb1[9];
#pragma unroll
                for (int ij = 0; ij < 9; ++ij) {
                    bb0[ij] = ca[ij] * wr;
                    bb1[ij] = ca[ij] * wsv;
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ij = 0; ij < 9; ++ij) {
                    acc[3 * ij + 0] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(wr, bb0[ij], acc[3 * ij + 0], 0, 0, 0);
                    acc[3 * ij + 1] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(wr, bb1[ij], acc[3 * ij + 1], 0, 0, 0);
                    acc[3 * ij + 2] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(wsv, bb1[ij], acc[3 * ij + 2], 0, 0, 0);
                }
            }
        }
        // the group's upper triangles into the patch, from the accumulators
        const int cell = lg[0] + 2 * lg[1] + 4 * lg[2];
        int hs[12];
#pragma unroll
        for (int sl = 0; sl < 12; ++sl)
            hs[sl] = TT.h[cell][up[sl]] * TT_WORDS;
        auto fix = [&](int ij, int sl) {
            return (long long)__float2int_rn(acc[3 * ij + sl / 4][sl % 4] * scale);
        };
#pragma unroll
        for (int w = 0; w < TT_WORDS; ++w)
#pragma unroll
            for (int sl = 0; sl < 12; ++sl)
                if (live & (1u << sl)) {
                    const long long hi = 2 * w + 1 < 9 ? fix(2 * w + 1, sl) : 0;
                    atomicAdd(&patch[hs[sl] + w],
                              (unsigned long long)(hi * 4294967296LL + fix(2 * w, sl)));
                }
    }
    __syncthreads();
    // every node pair of the brick, read from its canonical entry: thread t <
    // 252 takes component t % 9 of the pairs f = t / 9 + 28 k, so consecutive
    // threads add consecutive floats of M (components, then offsets of a row);
    // seven pairs at a time, their table entries and patch values read first
    constexpr int FL_PAIRS = 28, FL_UNROLL = 7;
    static_assert(TT_FULL % (FL_PAIRS * FL_UNROLL) == 0, "flush rounds");
    static_assert(TT_WAVES * WAVE >= 9 * FL_PAIRS, "flush threads");
    if (threadIdx.x < 9 * FL_PAIRS) {
        const int ij = threadIdx.x % 9, f0 = threadIdx.x / 9;
        for (int f1 = f0; f1 < TT_FULL; f1 += FL_PAIRS * FL_UNROLL) {
            uint32_t d[FL_UNROLL];
            int v[FL_UNROLL];
#pragma unroll
            for (int u = 0; u < FL_UNROLL; ++u)
                d[u] = TT.dec[f1 + FL_PAIRS * u];
#pragma unroll
            for (int u = 0; u < FL_UNROLL; ++u)
                v[u] = tt_split(patch[(int)(d[u] & 2047u) * TT_WORDS + ij / 2], ij & 1);
#pragma unroll
            for (int u = 0; u < FL_UNROLL; ++u) {
                if (v[u] == 0)
                    continue;
                const int A = (int)((d[u] >> 11) & 63u), o = (int)(d[u] >> 17);
                const int gx = wrap_add(org[0], A % TT_N, m.n[0]);
                const int gy = wrap_add(org[1], (A / TT_N) % TT_N, m.n[1]);
                const int gz = wrap_add(org[2], A / (TT_N * TT_N), m.n[2]);
                const size_t node =
                    (size_t)gx + (size_t)m.n[0] * ((size_t)gy + (size_t)m.n[1] * gz);
                atomic_add_f32(&m.M[(node * TSC_OFFS + o) * 9 + ij], (float)v[u] * inv_scale);
            }
        }
    }
}

// M = 0 ahead of the additions (PCG_MASS_OVERWRITE).
__global__ __launch_bounds__(256) void k_mass_tsc_zero(float *__restrict__ M, int64_t len)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len; i += stride)
        M[i] = 0.0f;
}

}  // namespace
}  // namespace pcg

using namespace pcg;

namespace {

// Both entry points: the scalar matrix or (TENSOR, B and beta given) the ECSIM
// one, with TSC weights.
template <bool TENSOR>
pcg_status assemble_tsc(const char *who, const pcg_grid *grid, const pcg_particles *particles,
                        const float *const B[3], const float *beta, const pcg_tile *groups,
                        int32_t variant, float *M, void *stream)
{
    clear_error();
    PCG_TRY(check_grid(grid, who));
    if (grid->dim != 3)
        return fail(PCG_EUNSUPPORTED, "%s: only 3-D grids (dim = %d)", who, grid->dim);
    for (int k = 0; k < 3; ++k)
        if (grid->n[k] < 5)
            return fail(PCG_EINVAL, "%s: n[%d] = %d < 5 (the 125 offsets must be distinct nodes)",
                        who, k, grid->n[k]);
    if (!particles || !M)
        return fail(PCG_EINVAL, "%s: particles or M is NULL", who);
    const bool overwrite = (variant & PCG_MASS_OVERWRITE) != 0;
    variant &= ~PCG_MASS_OVERWRITE;
    if (variant < PCG_MASS_AUTO || variant > PCG_MASS_FLAT)
        return fail(PCG_EINVAL, "%s: unknown variant %d", who, variant);
    const int64_t count = particles->count;
    if (count < 0 || count >= (int64_t(1) << 30))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^30)", who, (long long)count);
    if (count > 0 && (!particles->x[0] || !particles->x[1] || !particles->x[2] ||
                      !particles->q || !particles->w))
        return fail(PCG_EINVAL, "%s: x, q or w is NULL", who);
    if (TENSOR && count > 0 && (!B || !B[0] || !B[1] || !B[2] || !beta))
        return fail(PCG_EINVAL, "%s: B or beta is NULL", who);
    const bool grouped = variant != PCG_MASS_FLAT && groups;
    if (!groups && (variant == PCG_MASS_MFMA || variant == PCG_MASS_VALU))
        return fail(PCG_EINVAL, "%s: the %s variant needs a support-group layout", who,
                    variant == PCG_MASS_VALU ? "VALU" : "MFMA");
    if (grouped) {
        if (groups->T != 1 || groups->order != 2)
            return fail(PCG_EINVAL,
                        "%s: groups must be a T = 1, order = 2 layout (T = %d, order = %d)", who,
                        groups->T, groups->order);
        if (!groups->tile_offsets)
            return fail(PCG_EINVAL, "%s: group offsets are NULL", who);
        if (groups->n_partitioned < 0 || groups->n_partitioned > count)
            return fail(PCG_EINVAL, "%s: n_partitioned outside [0, count]", who);
    }
    TscArgs m{};
    for (int k = 0; k < 3; ++k) {
        m.n[k] = grid->n[k];
        m.nf[k] = (float)grid->n[k];
        m.x[k] = particles->x[k];
        m.B[k] = TENSOR && B ? B[k] : nullptr;
    }
    m.q = particles->q;
    m.w = particles->w;
    m.beta = TENSOR ? beta : nullptr;
    m.M = M;
    m.ngroups = (uint32_t)((int64_t)grid->n[0] * grid->n[1] * grid->n[2]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (overwrite) {
        // every path here adds to M: clear it first (the arguments have
        // passed every check)
        const int64_t len = (int64_t)m.ngroups * TSC_OFFS * (TENSOR ? 9 : 1);
        const int64_t blocks = std::min<int64_t>((len + 255) / 256, (int64_t)device_cus() * 16);
        PCG_TRY(launch("mass_tsc_zero", k_mass_tsc_zero, dim3((unsigned)blocks), dim3(256), 0, st,
                       M, len));
    }
    if (count == 0)
        return PCG_OK;
    auto flat = [&](int64_t begin, int64_t end) -> pcg_status {
        if (end <= begin)
            return PCG_OK;
        const int64_t blocks =
            std::min<int64_t>((end - begin + 255) / 256, (int64_t)device_cus() * 32);
        if (TENSOR)
            return launch("mass_tsc_tensor_flat", k_mass_tsc_tensor_flat, dim3((unsigned)blocks),
                          dim3(256), 0, st, m, begin, end);
        return launch("mass_tsc_flat", k_mass_tsc_flat, dim3((unsigned)blocks), dim3(256), 0, st,
                      m, begin, end);
    };
    if (!grouped)
        return flat(0, count);
    m.offsets = groups->tile_offsets;
    m.n_part = groups->n_partitioned;
    if (m.n_part > 0) {
        const uint32_t nblocks = (m.ngroups + TSC_WAVES - 1) / TSC_WAVES;
        const uint32_t blocks = (nblocks + 7) / 8 * 8;
        const bool valu = variant == PCG_MASS_VALU;
        if (TENSOR && valu)
            PCG_TRY(launch("mass_tsc_tensor_valu", k_mass_tsc_tensor_valu, dim3(blocks),
                           dim3(TSC_WAVES * WAVE), 0, st, m));
        else if (TENSOR) {
            static const bool lds_ok =
                hipFuncSetAttribute((const void *)k_mass_tsc_tensor_brick,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)TT_PATCH_BYTES) == hipSuccess;
            if (!lds_ok)
                return fail(PCG_EHIP, "%s: cannot raise dynamic LDS to %zu bytes", who,
                            TT_PATCH_BYTES);
            m.nbricks = (uint32_t)(((grid->n[0] + TT_B - 1) / TT_B) *
                                   ((grid->n[1] + TT_B - 1) / TT_B) *
                                   ((grid->n[2] + TT_B - 1) / TT_B));
            m.xcd_run = TT_XCD_RUN;
            PCG_TRY(launch("mass_tsc_tensor_mfma", k_mass_tsc_tensor_brick,
                           dim3(xcd_grid(m.nbricks, m.xcd_run)), dim3(TT_WAVES * WAVE),
                           TT_PATCH_BYTES, st, m));
        } else if (valu)
            PCG_TRY(launch("mass_tsc_valu", k_mass_tsc_valu, dim3(blocks),
                           dim3(TSC_WAVES * WAVE), 0, st, m));
        else {
            static const bool lds_ok =
                hipFuncSetAttribute((const void *)k_mass_tsc_brick,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)TSC_PATCH_BYTES) == hipSuccess;
            if (!lds_ok)
                return fail(PCG_EHIP, "%s: cannot raise dynamic LDS to %zu bytes", who,
                            TSC_PATCH_BYTES);
            const uint32_t bricks = (uint32_t)(((grid->n[0] + TB_X - 1) / TB_X) *
                                               ((grid->n[1] + TB_Y - 1) / TB_Y) *
                                               ((grid->n[2] + TB_Z - 1) / TB_Z));
            PCG_TRY(launch("mass_tsc_mfma", k_mass_tsc_brick, dim3(bricks),
                           dim3(TSC_BRICK_WAVES * WAVE), TSC_PATCH_BYTES, st, m));
        }
    }
    return flat(groups->n_partitioned, count);
}

}  // namespace

extern "C" pcg_status assemble_mass_matrix_scalar_tsc(const pcg_grid *grid,
                                                      const pcg_particles *particles,
                                                      const pcg_tile *groups, int32_t variant,
                                                      float *M, void *stream)
{
    return assemble_tsc<false>("assemble_mass_matrix_scalar_tsc", grid, particles, nullptr,
                               nullptr, groups, variant, M, stream);
}

extern "C" pcg_status assemble_mass_matrix_tsc(const pcg_grid *grid,
                                               const pcg_particles *particles,
                                               const float *const B[3], const float *beta,
                                               const pcg_tile *groups, int32_t variant, float *M,
                                               void *stream)
{
    return assemble_tsc<true>("assemble_mass_matrix_tsc", grid, particles, B, beta, groups,
                              variant, M, stream);
}
