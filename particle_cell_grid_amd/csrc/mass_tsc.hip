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
// The tensor (ECSIM) matrix with TSC weights ([MM] Eq.(4)-(5); §4.1 Fig. 9)
// uses the moments of the CIC kernels: with u = (1, omega) and
// c = q w / (1 + |omega|^2), T_kl[a][b] = sum_p c u_k u_l W_a W_b (k <= l) and
//   M^ij = delta_ij T_00 + eps_ijk T_0(k+1) + T_(i+1)(j+1).
// Each T_kl is a symmetric 27 x 27 matrix: tiles (0,0), (0,1), (1,1), i.e.
// 30 products of 16x16x4 per 4 particles, accumulators in place (120 AGPRs).
// The block (729 node pairs x 9 components) is added to M with 6561 atomics,
// staged in LDS so that consecutive lanes add consecutive floats of M (a lane
// per pair would put 36 bytes between neighbouring lanes' addresses).
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

__device__ inline TscParticle tsc_particle(const TscArgs &m, float x0, float x1, float x2,
                                           float q, float w)
{
    TscParticle P;
    const float xs[3] = {x0, x1, x2};
    float wk[3][3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float x = clamp_coord(xs[k], m.nf[k]);
        const float fl = floorf(x);
        const bool low = x - fl < 0.5f;
        const float b = low ? fl - 1.0f : fl;
        const float t = x - (b + 1.0f);
        const int bi = (int)b;  // in [-1, n]
        P.base[k] = bi < 0 ? bi + m.n[k] : (bi >= m.n[k] ? bi - m.n[k] : bi);
        wk[k][0] = 0.5f * (0.5f - t) * (0.5f - t);
        wk[k][1] = 0.75f - t * t;
        wk[k][2] = 0.5f * (0.5f + t) * (0.5f + t);
    }
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
// zero), reused for the 32 x 32 block once the batches are done.
struct TscStage {
    float W[64][32];
    float c[64];
};
union TscScratch {
    TscStage s;
    float Tm[32][33];
};

__device__ inline void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The 27 x 27 block of one group (support base gb, wrapped; slice [lo, hi))
// into ws.Tm (rows and columns 0..26), one wave.  MFMA: the three 16x16 tiles
// on the matrix cores; VALU: each lane sums its node pairs pr = lane + 64 k
// into tv.  A particle of the slice that does not belong to the group (a stale
// layout) is deposited by its own lane with global atomics.
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
                                       int64_t lo, int64_t hi, float *tv,
                                       const TscRaw *ahead = nullptr)
{
    const int r = lane & 15, kk = lane >> 4;
    floatx4 acc00 = {0, 0, 0, 0}, acc01 = {0, 0, 0, 0}, acc11 = {0, 0, 0, 0};
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
    wave_sync();
    if (MFMA) {
        // register i of this lane holds D[4 (lane / 16) + i][lane % 16]; tile
        // (1,0) is filled as tile (0,1) transposed
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * kk + i, col = r;
            ws.Tm[row][col] = acc00[i];
            ws.Tm[row][16 + col] = acc01[i];
            ws.Tm[16 + col][row] = acc01[i];
            ws.Tm[16 + row][16 + col] = acc11[i];
        }
        wave_sync();
    }
}

// Group coordinates of linear group index g (gx + n_x (gy + n_y gz)).
__device__ inline void group_coords(const TscArgs &m, uint32_t g, int *gb)
{
    gb[0] = (int)(g % (uint32_t)m.n[0]);
    gb[1] = (int)((g / (uint32_t)m.n[0]) % (uint32_t)m.n[1]);
    gb[2] = (int)(g / ((uint32_t)m.n[0] * (uint32_t)m.n[1]));
}

// One wave per group: group = the wave's global index (groups are the support
// base nodes, linear index gx + n_x (gy + n_y gz)); its 729 node pairs go to M
// with device atomics.
template <bool MFMA>
__global__ __launch_bounds__(TSC_WAVES * WAVE) void k_mass_tsc_group(TscArgs m)
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
    tsc_group_block<MFMA>(m, ws, lane, gb, lo, hi, tv);
#pragma unroll
    for (int k = 0; k < TSC_PAIRS; ++k) {
        const int pr = lane + WAVE * k;
        if (pr < TSC_NODES * TSC_NODES) {
            const int a = pr / TSC_NODES, b = pr % TSC_NODES;
            const float v = MFMA ? ws.Tm[a][b] : tv[k];
            atomic_add_f32(&m.M[(size_t)tsc_node(m, gb, a) * TSC_OFFS + tsc_offset(a, b)], v);
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
        prefetch(wave);
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
        tsc_group_block<true>(m, ws, lane, gb, lo, hi, tv, cur);
#pragma unroll
        for (int k = 0; k < TSC_PAIRS; ++k) {
            const int pr = lane + WAVE * k;
            if (pr < TSC_NODES * TSC_NODES) {
                const int a = pr / TSC_NODES, b = pr % TSC_NODES;
                const int ln = (lg[0] + a % 3) + TP_X * ((lg[1] + (a / 3) % 3) + TP_Y * (lg[2] + a / 9));
                atomicAdd(&patch[ln * TSC_OFFS + tsc_offset(a, b)],
                          __float2int_rn(ws.Tm[a][b] * scale));
            }
        }
        wave_sync();  // Tm is the next group's staging area
    }
    __syncthreads();
    // the patch to M: node rows of 125 floats, consecutive threads on
    // consecutive offsets; entries no group touched stay zero and are skipped
    for (int i = threadIdx.x; i < TP_NODES * TSC_OFFS; i += blockDim.x) {
        const int v = patch[i];
        if (v == 0)
            continue;
        const int ln = i / TSC_OFFS, o = i - ln * TSC_OFFS;
        const int lx = ln % TP_X, ly = (ln / TP_X) % TP_Y, lz = ln / (TP_X * TP_Y);
        const int gx = wrap_add(org[0], lx, m.n[0]);
        const int gy = wrap_add(org[1], ly, m.n[1]);
        const int gz = wrap_add(org[2], lz, m.n[2]);
        const size_t node = (size_t)gx + (size_t)m.n[0] * ((size_t)gy + (size_t)m.n[1] * gz);
        atomic_add_f32(&m.M[node * TSC_OFFS + o], (float)v * inv_scale);
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

struct TscTensorStage {
    float W[64][32];
    float u[64][4];
    float c[64];
};
// pairs per lane (729 over 64 lanes: TSC_PAIRS), flushed in two halves
constexpr int TSC_HALF = (TSC_PAIRS + 1) / 2;
union TscTensorScratch {
    TscTensorStage s;
    float Tm[32][33];
    float F[WAVE * TSC_HALF * 9];  // one half's blocks, pair-major
};

// the ten moments (k <= l) in a fixed order
__device__ constexpr int MOM_K[10] = {0, 0, 0, 0, 1, 1, 1, 2, 2, 3};
__device__ constexpr int MOM_L[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};

template <bool MFMA>
__global__ __launch_bounds__(TSC_WAVES * WAVE) void k_mass_tsc_tensor_group(TscArgs m)
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
    gb[0] = (int)(g % (uint32_t)m.n[0]);
    gb[1] = (int)((g / (uint32_t)m.n[0]) % (uint32_t)m.n[1]);
    gb[2] = (int)(g / ((uint32_t)m.n[0] * (uint32_t)m.n[1]));

    const int r = lane & 15, kk = lane >> 4;
    // MFMA: acc[3 mom + t], tiles t = (0,0), (0,1), (1,1) of moment mom
    floatx4 acc[30];
#pragma unroll
    for (int i = 0; i < 30; ++i)
        acc[i] = floatx4{0, 0, 0, 0};
    // VALU: lane owns node pairs lane + 64 k (k < 12) and their 9 components
    constexpr int PAIRS = TSC_PAIRS;
    constexpr int VPAIRS = MFMA ? 1 : PAIRS;
    float tv[VPAIRS][9];
#pragma unroll
    for (int k = 0; k < VPAIRS; ++k)
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
        ws.s.c[lane] = take ? c : 0.0f;  // the factor of every product (see above)
        wave_sync();
        const int nb = (int)std::min<int64_t>(64, hi - base);
        if (MFMA) {
            const int steps = (nb + 3) >> 2;
            for (int i = 0; i < steps; ++i) {
                const int qq = 4 * i + kk;
                const float w0 = ws.s.W[qq][r], w1 = ws.s.W[qq][16 + r];
                const float4 uq = *reinterpret_cast<const float4 *>(ws.s.u[qq]);
                const float cq = ws.s.c[qq];
                const float uk[4] = {uq.x, uq.y, uq.z, uq.w};
                float a0[4], a1[4], b0[4], b1[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    a0[k] = uk[k] * w0;
                    a1[k] = uk[k] * w1;
                    b0[k] = cq * a0[k];
                    b1[k] = cq * a1[k];
                }
#pragma unroll
                for (int mo = 0; mo < 10; ++mo) {
                    const int k = MOM_K[mo], l = MOM_L[mo];
                    acc[3 * mo + 0] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(a0[k], b0[l], acc[3 * mo + 0], 0, 0, 0);
                    acc[3 * mo + 1] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(a0[k], b1[l], acc[3 * mo + 1], 0, 0, 0);
                    acc[3 * mo + 2] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(a1[k], b1[l], acc[3 * mo + 2], 0, 0, 0);
                }
            }
        } else {
            for (int qq = 0; qq < nb; ++qq) {
                const float cq = ws.s.c[qq];
                const float4 uq = *reinterpret_cast<const float4 *>(ws.s.u[qq]);
                const float uk[4] = {uq.x, uq.y, uq.z, uq.w};
#pragma unroll
                for (int k2 = 0; k2 < VPAIRS; ++k2) {
                    const int pr = lane + WAVE * k2;
                    if (pr < TSC_NODES * TSC_NODES) {
                        const float wab =
                            cq * ws.s.W[qq][pr / TSC_NODES] * ws.s.W[qq][pr % TSC_NODES];
#pragma unroll
                        for (int mo = 0; mo < 10; ++mo)
                            add_moment(MOM_K[mo], MOM_L[mo], wab * uk[MOM_K[mo]] * uk[MOM_L[mo]],
                                       tv[k2]);
                    }
                }
            }
        }
    }
    wave_sync();
    // per half of the lane's pairs (lane + 64 (h TSC_HALF + k2)): the blocks,
    // from the moments through LDS (MFMA) or from the lane's sums (VALU), then
    // the half's 64 TSC_HALF x 9 floats flushed with consecutive lanes on
    // consecutive values v: pair 64 h TSC_HALF + v / 9, component v % 9
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float blk[TSC_HALF][9];
#pragma unroll
        for (int k2 = 0; k2 < TSC_HALF; ++k2)
#pragma unroll
            for (int ij = 0; ij < 9; ++ij)
                blk[k2][ij] = MFMA ? 0.0f : tv[(h * TSC_HALF + k2) % VPAIRS][ij];
        if (MFMA) {
            // register i of this lane holds D[4 (lane / 16) + i][lane % 16];
            // tile (1,0) is tile (0,1) transposed
#pragma unroll
            for (int mo = 0; mo < 10; ++mo) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * kk + i, col = r;
                    ws.Tm[row][col] = acc[3 * mo + 0][i];
                    ws.Tm[row][16 + col] = acc[3 * mo + 1][i];
                    ws.Tm[16 + col][row] = acc[3 * mo + 1][i];
                    ws.Tm[16 + row][16 + col] = acc[3 * mo + 2][i];
                }
                wave_sync();
#pragma unroll
                for (int k2 = 0; k2 < TSC_HALF; ++k2) {
                    const int pr = lane + WAVE * (h * TSC_HALF + k2);
                    if (h * TSC_HALF + k2 < PAIRS && pr < TSC_NODES * TSC_NODES)
                        add_moment(MOM_K[mo], MOM_L[mo], ws.Tm[pr / TSC_NODES][pr % TSC_NODES],
                                   blk[k2]);
                }
                wave_sync();
            }
        }
#pragma unroll
        for (int k2 = 0; k2 < TSC_HALF; ++k2)
#pragma unroll
            for (int ij = 0; ij < 9; ++ij)
                ws.F[(k2 * WAVE + lane) * 9 + ij] = blk[k2][ij];
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
        if (TENSOR)
            PCG_TRY(launch(valu ? "mass_tsc_tensor_valu" : "mass_tsc_tensor_mfma",
                           valu ? k_mass_tsc_tensor_group<false> : k_mass_tsc_tensor_group<true>,
                           dim3(blocks), dim3(TSC_WAVES * WAVE), 0, st, m));
        else if (valu)
            PCG_TRY(launch("mass_tsc_valu", k_mass_tsc_group<false>, dim3(blocks),
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
