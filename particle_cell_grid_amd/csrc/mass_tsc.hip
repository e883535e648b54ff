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
// brick of groups in an LDS patch first and adds the patch to M once (see
// "MFMA variant: bricks" below).
//
// The tensor (ECSIM) matrix with TSC weights ([MM] Eq.(4)-(5); §4.1 Fig. 9):
// M^ij = sum_p c_p alpha'^ij_p W_a W_b with c = q w / (1 + |omega|^2) and
// alpha' = I + omega omega^T + the rotation terms.  Each of the nine
// components is a symmetric 27 x 27 block per group, so the MFMA variant runs
// three 16x16x4 tiles per component (27 matrix instructions per 4 particles)
// with the same bricks.
//
// Variants: MFMA (bricks), VALU (one wave per group, each lane summing its
// node pairs over the staged particles -- for the tensor matrix the ten moments
// u_k u_l, u = (1, omega) -- and adding the group's block to M with device
// atomics) and FLAT (one thread per particle; also the unsorted tail).  A
// particle found in a slice whose group it does not belong to (a stale layout)
// is deposited by its own lane with the flat path's atomics.
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

// Per-wave LDS of the VALU variant: one staged 64-particle batch (rows padded
// to 32 nodes, the pads zero).
struct TscStage {
    float W[64][32];
    float c[64];
};

__device__ inline void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int TSC_PAIRS = (TSC_NODES * TSC_NODES + WAVE - 1) / WAVE;  // pairs per lane

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
    __shared__ TscStage scratch[TSC_WAVES];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    TscStage &ws = scratch[wave];
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
    // lane sums its node pairs pr = lane + 64 k over the staged particles; a
    // particle of the slice that does not belong to the group (a stale layout)
    // is deposited by its own lane with global atomics
    float tv[TSC_PAIRS];
#pragma unroll
    for (int k = 0; k < TSC_PAIRS; ++k)
        tv[k] = 0.0f;
    for (int64_t base = lo; base < hi; base += 64) {
        const int64_t p = std::min<int64_t>(base + lane, hi - 1);  // clamped
        const bool valid = base + lane < hi;
        const TscParticle P = tsc_particle(m, ld(m.x[0], p), ld(m.x[1], p), ld(m.x[2], p),
                                           ld(m.q, p), ld(m.w, p));
        const bool home = P.base[0] == gb[0] && P.base[1] == gb[1] && P.base[2] == gb[2];
        if (valid && !home)
            tsc_deposit_global(m, P);
        wave_sync();
#pragma unroll
        for (int a = 0; a < 32; a += 4) {
            float4 v4;
            v4.x = a + 0 < TSC_NODES ? P.W[a + 0] : 0.0f;
            v4.y = a + 1 < TSC_NODES ? P.W[a + 1] : 0.0f;
            v4.z = a + 2 < TSC_NODES ? P.W[a + 2] : 0.0f;
            v4.w = a + 3 < TSC_NODES ? P.W[a + 3] : 0.0f;
            *reinterpret_cast<float4 *>(&ws.W[lane][a]) = v4;
        }
        // only c is zeroed for a slot outside the group: every product takes
        // c once, and the weights of a loaded particle are finite
        ws.c[lane] = valid && home ? P.c : 0.0f;
        wave_sync();
        const int nb = (int)std::min<int64_t>(64, hi - base);
        for (int q = 0; q < nb; ++q) {
            const float cq = ws.c[q];
#pragma unroll
            for (int k = 0; k < TSC_PAIRS; ++k) {
                const int pr = lane + WAVE * k;
                if (pr < TSC_NODES * TSC_NODES)
                    tv[k] += cq * ws.W[q][pr / TSC_NODES] * ws.W[q][pr % TSC_NODES];
            }
        }
    }
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

// ------------------------------------------------------ MFMA variant: bricks
//
// A work-group takes a brick of groups (4 x 4 x 2 for the scalar matrix,
// 2 x 2 x 2 for the tensor one) and sums their blocks in an LDS patch of
// 32-bit fixed-point values before adding the patch to M once.
//
// Blocks.  Every component of either matrix is a symmetric 27 x 27 block per
// group, sum_p k_p W_a(p) W_b(p): k = q w for the scalar matrix, and for
// component ij of the tensor one k = c alpha'^ij with c = q w / (1 + |omega|^2)
// and alpha' = I + omega omega^T plus the rotation (+omega_z at (x,y), -omega_y
// at (x,z), ... as in add_moment).  Rows padded to 32, a block is three
// 16x16x4 tiles, (0,0), (0,1), (1,1) (A = W_a, B = k W_b): 3 matrix
// instructions per 4 particles and component.
//
// Patch.  The brick's groups reach nodes 0..b+1 (local) on an axis of b groups,
// and a node pair (la, lb) of an axis occurs iff |la - lb| <= 2: 5 b + 4 pairs.
// As each component block is symmetric in its two nodes, the patch keeps one of
// (A, B) and (B, A), the one whose offset B - A is >= 0 in (z, y, x) order
// ("canonical"): 4104 pairs for the scalar brick (16 KB), 1404 x 9 components
// for the tensor one (55 KB as packed words), so two work-groups share a CU.
// A group adds only its blocks' entries on or above the diagonal (node b >= a
// in support order, which is exactly the canonical half), each lane straight
// from its accumulator registers; the flush writes every node pair of the
// brick (8064, or 2744 x 9), reading the canonical entry, in runs of
// consecutive floats of M: 252 device atomics per group for the scalar matrix
// (729 without the patch) and 3087 for the tensor one (6561).
//
// Scale.  2^k keeps every partial sum of a patch entry below 2^30: a particle
// adds at most (9/16) |q w| to an entry (|alpha^ij| <= 1: alpha is the inverse
// of I - [omega]x, whose singular values are >= 1), so 2^k (9/16) sum |q w|
// over the brick's particles < 2^30 bounds them all.  Products are rounded to
// the nearest unit, 2^-k, once per group and entry.
template <bool TENSOR>
struct Brick {
    static constexpr int BX = TENSOR ? 2 : 4, BY = TENSOR ? 2 : 4, BZ = 2;  // groups
    static constexpr int NX = BX + 2, NY = BY + 2, NZ = BZ + 2;  // patch nodes per axis
    static constexpr int NC = TENSOR ? 9 : 1;                    // components
    static constexpr int WAVES = TENSOR ? 4 : 8;
    static constexpr int GROUPS = BX * BY * BZ;
    static constexpr int GPW = GROUPS / WAVES;  // groups per wave
    // patch words per entry: the tensor's nine components as five 64-bit
    // words, components 2 w and 2 w + 1 packed in word w (the last one alone)
    static constexpr int WORDS = TENSOR ? 5 : 1;
    static constexpr int MIN_WAVES_PER_SIMD = TENSOR ? 2 : 4;
    // bricks per XCD run (xcd_item): neighbouring bricks add to the same rows
    static constexpr uint32_t XCD_RUN = TENSOR ? 64 : 0;
    // staged row per particle: k (NC floats) from 0, the nine axis weights
    // (x0..2 y0..2 z0..2) from AXW; ROW floats apart, so that the lanes'
    // 16-byte writes of their rows cover all banks
    static constexpr int AXW = TENSOR ? 9 : 1, ROW = TENSOR ? 20 : 12;
    static constexpr int FL_UNROLL = TENSOR ? 7 : 4;  // flush entries in flight per thread
};

constexpr int TSC_UPPER = TSC_NODES * (TSC_NODES + 1) / 2;  // pairs a <= b of a support

// Node pairs (la, lb) of one axis with n patch nodes and |la - lb| <= 2: every
// pair (ordered by la, then lb), those with lb > la, those with lb >= la.
struct AxisPairs {
    int all[6][6], pos[6][6], nn[6][6];  // index, or -1
    int la[24], lb[24];                  // pair of an `all` index
    int n_all, n_pos, n_nn;
};

constexpr AxisPairs axis_pairs(int n)
{
    AxisPairs t{};
    for (int a = 0; a < 6; ++a)
        for (int b = 0; b < 6; ++b)
            t.all[a][b] = t.pos[a][b] = t.nn[a][b] = -1;
    for (int a = 0; a < n; ++a)
        for (int b = 0; b < n; ++b)
            if (a - b <= 2 && b - a <= 2) {
                t.la[t.n_all] = a;
                t.lb[t.n_all] = b;
                t.all[a][b] = t.n_all++;
                if (b > a)
                    t.pos[a][b] = t.n_pos++;
                if (b >= a)
                    t.nn[a][b] = t.n_nn++;
            }
    return t;
}

template <bool TENSOR>
struct BrickPairs {
    using K = Brick<TENSOR>;
    static constexpr AxisPairs X = axis_pairs(K::NX), Y = axis_pairs(K::NY), Z = axis_pairs(K::NZ);
    static constexpr int FULL = X.n_all * Y.n_all * Z.n_all;  // node pairs of a brick
    static constexpr int ZBLK = Y.n_pos * X.n_all + K::NY * X.n_nn;
    static constexpr int HALF = Z.n_pos * Y.n_all * X.n_all + K::NZ * ZBLK;  // canonical
    // patch index of the canonical pair (A, B): offset in z > 0; else in
    // y > 0; else in x >= 0
    static constexpr int half(int ax, int ay, int az, int bx, int by, int bz)
    {
        return bz > az ? (Z.pos[az][bz] * Y.n_all + Y.all[ay][by]) * X.n_all + X.all[ax][bx]
                       : Z.n_pos * Y.n_all * X.n_all + az * ZBLK +
                             (by > ay ? Y.pos[ay][by] * X.n_all + X.all[ax][bx]
                                      : Y.n_pos * X.n_all + ay * X.n_nn + X.nn[ax][bx]);
    }
};

// Every canonical pair of the patch nodes (offsets -2..2) has its own index
// below HALF, and none is left over.
template <bool TENSOR>
constexpr bool half_is_a_bijection()
{
    using K = Brick<TENSOR>;
    using P = BrickPairs<TENSOR>;
    bool seen[P::HALF] = {};
    int count = 0;
    for (int A = 0; A < K::NX * K::NY * K::NZ; ++A)
        for (int o = 0; o < TSC_OFFS; ++o) {
            const int ax = A % K::NX, ay = (A / K::NX) % K::NY, az = A / (K::NX * K::NY);
            const int dx = o % 5 - 2, dy = (o / 5) % 5 - 2, dz = o / 25 - 2;
            const int bx = ax + dx, by = ay + dy, bz = az + dz;
            if (bx < 0 || bx >= K::NX || by < 0 || by >= K::NY || bz < 0 || bz >= K::NZ)
                continue;
            if (!(dz > 0 || (dz == 0 && (dy > 0 || (dy == 0 && dx >= 0)))))
                continue;
            const int h = P::half(ax, ay, az, bx, by, bz);
            if (h < 0 || h >= P::HALF || seen[h])
                return false;
            seen[h] = true;
            ++count;
        }
    return count == P::HALF;
}
static_assert(half_is_a_bijection<false>() && half_is_a_bijection<true>(),
              "patch index of the canonical pairs");
static_assert(BrickPairs<false>::HALF < (1 << 13) && BrickPairs<true>::HALF < (1 << 13) &&
                  9 * TSC_OFFS <= (1 << 11),
              "fields of a flush table entry");

template <bool TENSOR>
struct BrickTables {
    // node pair f of the brick (x pair fastest, then y, then z): canonical patch
    // index | ax << 13 | ay << 16 | az << 19 | NC o << 21 (local node A of the
    // row; o the offset of B from A, so NC o is its block in the row)
    uint32_t dec[BrickPairs<TENSOR>::FULL];
    // group cell c (c = lx + BX (ly + BY lz)) and support pair u (a <= b,
    // row-major: u = 27 a - a (a - 1) / 2 + b - a): patch index
    uint16_t h[Brick<TENSOR>::GROUPS][TSC_UPPER];
};

template <bool TENSOR>
constexpr BrickTables<TENSOR> brick_tables()
{
    using K = Brick<TENSOR>;
    using P = BrickPairs<TENSOR>;
    BrickTables<TENSOR> t{};
    for (int f = 0; f < P::FULL; ++f) {
        const int px = f % P::X.n_all, py = (f / P::X.n_all) % P::Y.n_all,
                  pz = f / (P::X.n_all * P::Y.n_all);
        const int A[3] = {P::X.la[px], P::Y.la[py], P::Z.la[pz]};
        const int B[3] = {P::X.lb[px], P::Y.lb[py], P::Z.lb[pz]};
        const int d[3] = {B[0] - A[0], B[1] - A[1], B[2] - A[2]};
        const bool canon = d[2] > 0 || (d[2] == 0 && (d[1] > 0 || (d[1] == 0 && d[0] >= 0)));
        const int h = canon ? P::half(A[0], A[1], A[2], B[0], B[1], B[2])
                            : P::half(B[0], B[1], B[2], A[0], A[1], A[2]);
        const int o = (d[0] + 2) + 5 * (d[1] + 2) + 25 * (d[2] + 2);
        t.dec[f] = (uint32_t)h | (uint32_t)A[0] << 13 | (uint32_t)A[1] << 16 |
                   (uint32_t)A[2] << 19 | (uint32_t)(K::NC * o) << 21;
    }
    int u = 0;
    for (int a = 0; a < TSC_NODES; ++a)
        for (int b = a; b < TSC_NODES; ++b, ++u)
            for (int c = 0; c < K::GROUPS; ++c) {
                const int cx = c % K::BX, cy = (c / K::BX) % K::BY, cz = c / (K::BX * K::BY);
                t.h[c][u] = (uint16_t)P::half(cx + a % 3, cy + (a / 3) % 3, cz + a / 9,
                                              cx + b % 3, cy + (b / 3) % 3, cz + b / 9);
            }
    return t;
}
__device__ constexpr BrickTables<false> BRICK_SCALAR = brick_tables<false>();
__device__ constexpr BrickTables<true> BRICK_TENSOR = brick_tables<true>();

template <bool TENSOR>
__device__ inline const BrickTables<TENSOR> &brick_table()
{
    if constexpr (TENSOR)
        return BRICK_TENSOR;
    else
        return BRICK_SCALAR;
}

template <bool TENSOR>
struct __attribute__((aligned(16))) BrickStage {
    float v[64][Brick<TENSOR>::ROW];
};

// One of the two sums of a packed patch word: the low one (signed 32-bit), or
// the high one, the word less the low sum shifted down.
__device__ inline int split_word(unsigned long long word, int high)
{
    const int lo = (int)(uint32_t)word;
    return high ? (int)((long long)(word - (unsigned long long)(long long)lo) >> 32) : lo;
}
__device__ inline int split_word(int word, int) { return word; }

// A particle's inputs, as loaded (slot base + lane of a slice, clamped); B and
// beta for the tensor matrix only.
struct BrickRaw {
    float x[3], q, w, B[3], beta;
};

template <bool TENSOR>
__device__ inline BrickRaw brick_load(const TscArgs &m, int64_t base, int64_t hi, int lane)
{
    const int64_t p = std::min<int64_t>(base + lane, hi - 1);  // clamped
    BrickRaw r{};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        r.x[k] = ld(m.x[k], p);
        if (TENSOR)
            r.B[k] = ld(m.B[k], p);
    }
    r.q = ld(m.q, p);
    r.w = ld(m.w, p);
    if (TENSOR)
        r.beta = ld(m.beta, p);
    return r;
}

template <bool TENSOR>
__global__ __launch_bounds__(Brick<TENSOR>::WAVES *WAVE, Brick<TENSOR>::MIN_WAVES_PER_SIMD) void
k_mass_tsc_brick(TscArgs m)
{
    using K = Brick<TENSOR>;
    using P = BrickPairs<TENSOR>;
    using Word = typename std::conditional<TENSOR, unsigned long long, int>::type;
    constexpr int NC = K::NC;
    const BrickTables<TENSOR> &tab = brick_table<TENSOR>();
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // [HALF][WORDS]; packed words are added as one 64-bit integer (the low sum
    // signed: the high one gets its borrow back when the word is split, as
    // every partial sum stays below 2^30)
    Word *patch = reinterpret_cast<Word *>(smem);
    __shared__ BrickStage<TENSOR> scratch[K::WAVES];
    __shared__ float red[K::WAVES];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    BrickStage<TENSOR> &ws = scratch[wave];
    const uint32_t brick = xcd_item(blockIdx.x, m.xcd_run);
    if (brick >= m.nbricks)
        return;
    const int nbx = (m.n[0] + K::BX - 1) / K::BX, nby = (m.n[1] + K::BY - 1) / K::BY;
    const int bi = (int)(brick % (uint32_t)nbx);
    const int bj = (int)((brick / (uint32_t)nbx) % (uint32_t)nby);
    const int bk = (int)(brick / ((uint32_t)nbx * (uint32_t)nby));
    const int org[3] = {bi * K::BX, bj * K::BY, bk * K::BZ};
    const int cnt[3] = {min(K::BX, m.n[0] - org[0]), min(K::BY, m.n[1] - org[1]),
                        min(K::BZ, m.n[2] - org[2])};
    const int ngb = cnt[0] * cnt[1] * cnt[2];
    {
        constexpr int n16 = P::HALF * K::WORDS * (int)sizeof(Word) / 16;
        static_assert(P::HALF * K::WORDS * sizeof(Word) % 16 == 0, "patch cleared as int4");
        int4 *p4 = reinterpret_cast<int4 *>(patch);
        for (int i = threadIdx.x; i < n16; i += blockDim.x)
            p4[i] = int4{0, 0, 0, 0};
    }
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
    // a wave's groups are j = wave + WAVES t; their first batches are loaded up
    // front and serve the sum of |q w| as well
    // (slice bounds kept in 32 bits: particle counts are below 2^30)
    int glo[K::GPW], ghi[K::GPW];
    BrickRaw first[K::GPW];
#pragma unroll
    for (int t = 0; t < K::GPW; ++t) {
        const int j = wave + K::WAVES * t;
        glo[t] = ghi[t] = 0;
        first[t] = BrickRaw{};
        if (j < ngb) {
            int lg[3];
            local(j, lg);
            int64_t lo, hi;
            slice(lg, lo, hi);
            glo[t] = (int)lo;
            ghi[t] = (int)hi;
            if (hi > lo)
                first[t] = brick_load<TENSOR>(m, lo, hi, lane);
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int t = 0; t < K::GPW; ++t) {
        if (glo[t] + lane < ghi[t])
            sum += fabsf(first[t].q * first[t].w);
        for (int p = glo[t] + WAVE + lane; p < ghi[t]; p += WAVE)
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
    for (int w = 0; w < K::WAVES; ++w)
        total += red[w];
    if (total == 0.0f)
        return;  // nothing to add (every wave sees the same total)
    int e = 0;
    frexpf(0.5625f * total, &e);  // (9/16) total < 2^e
    const int k_scale = max(-126, min(126, 30 - e));
    const float scale = ldexpf(1.0f, k_scale), inv_scale = ldexpf(1.0f, -k_scale);

    const int r = lane & 15, kk = lane >> 4;
    // the lane's rows of the MFMA operands: node r and node 16 + r (< 27 for r < 11)
    const int ra[3] = {K::AXW + r % 3, K::AXW + 3 + (r / 3) % 3, K::AXW + 6 + r / 9};
    const int s16 = r < 11 ? 16 + r : 0;
    const int sa[3] = {K::AXW + s16 % 3, K::AXW + 3 + (s16 / 3) % 3, K::AXW + 6 + s16 / 9};
    // The lane's twelve accumulator values per component: slot 4 t + i holds
    // entry (a, b) of tile t (0: (0,0), 1: (0,1), 2: (1,1)), a = 16 (t == 2) +
    // 4 (lane / 16) + i, b = 16 (t >= 1) + lane % 16.  The slots on or above
    // the diagonal of the 27 x 27 block go to the patch; their support pair
    // index u (upper triangle, row-major) is fixed per lane.
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

    for (int t = 0; t < K::GPW; ++t) {
        const int j = wave + K::WAVES * t;
        int lo = glo[0], hi = ghi[0];
        BrickRaw cur = first[0];
#pragma unroll
        for (int u = 1; u < K::GPW; ++u)
            if (t == u) {
                lo = glo[u];
                hi = ghi[u];
                cur = first[u];
            }
        if (j >= ngb || hi <= lo)
            continue;
        int lg[3];
        local(j, lg);
        const int gb[3] = {org[0] + lg[0], org[1] + lg[1], org[2] + lg[2]};
        floatx4 acc[3 * NC];
#pragma unroll
        for (int i = 0; i < 3 * NC; ++i)
            acc[i] = floatx4{0, 0, 0, 0};
        for (int base = lo; base < hi; base += 64) {
            const bool valid = base + lane < hi;
            const BrickRaw in = base == lo ? cur : brick_load<TENSOR>(m, base, hi, lane);
            float wk[3][3];
            const int b0 = tsc_axis(m, in.x[0], 0, wk[0]), b1 = tsc_axis(m, in.x[1], 1, wk[1]),
                      b2 = tsc_axis(m, in.x[2], 2, wk[2]);
            const bool home = b0 == gb[0] && b1 == gb[1] && b2 == gb[2];
            // k of the particle's products, or 0 for a slot outside the group
            // (the weights of a loaded particle are finite, so its products vanish)
            const bool take = valid && home;
            wave_sync();
            float4 *row = reinterpret_cast<float4 *>(ws.v[lane]);
            if constexpr (TENSOR) {
                const float o0 = in.beta * in.B[0], o1 = in.beta * in.B[1],
                            o2 = in.beta * in.B[2];
                const float c = in.q * in.w / (1.0f + (o0 * o0 + o1 * o1 + o2 * o2));
                if (valid && !home) {  // stale layout: this lane deposits it alone
                    const float u4[4] = {1.0f, o0, o1, o2};
                    tsc_tensor_global(m, tsc_particle(m, in.x[0], in.x[1], in.x[2], in.q, in.w),
                                      u4, c);
                }
                const float cc = take ? c : 0.0f;
                row[0] = make_float4(cc * (1.0f + o0 * o0), cc * (o2 + o0 * o1),
                                     cc * (o0 * o2 - o1), cc * (o1 * o0 - o2));
                row[1] = make_float4(cc * (1.0f + o1 * o1), cc * (o0 + o1 * o2),
                                     cc * (o1 + o2 * o0), cc * (o2 * o1 - o0));
                row[2] = make_float4(cc * (1.0f + o2 * o2), wk[0][0], wk[0][1], wk[0][2]);
                row[3] = make_float4(wk[1][0], wk[1][1], wk[1][2], wk[2][0]);
                row[4] = make_float4(wk[2][1], wk[2][2], 0.0f, 0.0f);
            } else {
                if (valid && !home)  // stale layout: this lane deposits it alone
                    tsc_deposit_global(m, tsc_particle(m, in.x[0], in.x[1], in.x[2], in.q, in.w));
                row[0] = make_float4(take ? in.q * in.w : 0.0f, wk[0][0], wk[0][1], wk[0][2]);
                row[1] = make_float4(wk[1][0], wk[1][1], wk[1][2], wk[2][0]);
                row[2] = make_float4(wk[2][1], wk[2][2], 0.0f, 0.0f);
            }
            wave_sync();
            const int nb = min(64, hi - base);
            const int steps = (nb + 3) >> 2;
            for (int i = 0; i < steps; ++i) {
                const float *sv = ws.v[4 * i + kk];
                const float wr = sv[ra[0]] * sv[ra[1]] * sv[ra[2]];
                const float wsv = r < 11 ? sv[sa[0]] * sv[sa[1]] * sv[sa[2]] : 0.0f;
                float ca[NC];
                if constexpr (TENSOR) {
                    const float4 c0 = *reinterpret_cast<const float4 *>(sv);
                    const float4 c1 = *reinterpret_cast<const float4 *>(sv + 4);
                    const float cs[9] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w, sv[8]};
#pragma unroll
                    for (int ij = 0; ij < NC; ++ij)
                        ca[ij] = cs[ij];
                } else {
                    ca[0] = sv[0];
                }
                float bb0[NC], bb1[NC];
#pragma unroll
                for (int ij = 0; ij < NC; ++ij) {
                    bb0[ij] = ca[ij] * wr;
                    bb1[ij] = ca[ij] * wsv;
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ij = 0; ij < NC; ++ij) {
                    acc[3 * ij + 0] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(wr, bb0[ij], acc[3 * ij + 0], 0, 0, 0);
                    acc[3 * ij + 1] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(wr, bb1[ij], acc[3 * ij + 1], 0, 0, 0);
                    acc[3 * ij + 2] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(wsv, bb1[ij], acc[3 * ij + 2], 0, 0, 0);
                }
            }
        }
        // the group's entries on or above the diagonal into the patch
        const int cell = lg[0] + K::BX * (lg[1] + K::BY * lg[2]);
        int hs[12];
#pragma unroll
        for (int sl = 0; sl < 12; ++sl)
            hs[sl] = tab.h[cell][up[sl]] * K::WORDS;
        auto fix = [&](int ij, int sl) {
            return __float2int_rn(acc[3 * ij + sl / 4][sl % 4] * scale);
        };
#pragma unroll
        for (int w = 0; w < K::WORDS; ++w)
#pragma unroll
            for (int sl = 0; sl < 12; ++sl)
                if (live & (1u << sl)) {
                    if constexpr (TENSOR) {
                        const long long hw = 2 * w + 1 < NC ? fix(2 * w + 1, sl) : 0;
                        atomicAdd(&patch[hs[sl] + w],
                                  (unsigned long long)(hw * 4294967296LL + fix(2 * w, sl)));
                    } else {
                        atomicAdd(&patch[hs[sl]], fix(0, sl));
                    }
                }
    }
    __syncthreads();
    // every node pair of the brick, read from its canonical entry: thread t <
    // NC FL_PAIRS takes component t % NC of the pairs f = t / NC + FL_PAIRS k, so
    // consecutive threads add consecutive floats of M (components, then offsets
    // of a row); FL_UNROLL pairs at a time, table entries and patch values first
    constexpr int FL_PAIRS = K::WAVES * WAVE / NC, U = K::FL_UNROLL;
    constexpr bool EXACT = P::FULL % (FL_PAIRS * U) == 0;  // no pair past the end
    if (threadIdx.x < NC * FL_PAIRS) {
        const int ij = threadIdx.x % NC, f0 = threadIdx.x / NC;
        for (int f1 = f0; f1 < P::FULL; f1 += FL_PAIRS * U) {
            uint32_t d[U];
            int v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int f = f1 + FL_PAIRS * u;
                d[u] = EXACT || f < P::FULL ? tab.dec[f] : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = EXACT || f1 + FL_PAIRS * u < P::FULL
                           ? split_word(patch[(int)(d[u] & 8191u) * K::WORDS + ij / 2], ij & 1)
                           : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (v[u] == 0)
                    continue;
                const int gx = wrap_add(org[0], (int)((d[u] >> 13) & 7u), m.n[0]);
                const int gy = wrap_add(org[1], (int)((d[u] >> 16) & 7u), m.n[1]);
                const int gz = wrap_add(org[2], (int)((d[u] >> 19) & 3u), m.n[2]);
                const size_t node =
                    (size_t)gx + (size_t)m.n[0] * ((size_t)gy + (size_t)m.n[1] * gz);
                atomic_add_f32(m.M + node * (TSC_OFFS * NC) + (d[u] >> 21) + ij,
                               (float)v[u] * inv_scale);
            }
        }
    }
}

template <bool TENSOR>
constexpr size_t brick_patch_bytes()
{
    return (size_t)BrickPairs<TENSOR>::HALF * Brick<TENSOR>::WORDS *
           (TENSOR ? sizeof(unsigned long long) : sizeof(int));
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

// The MFMA variant: one work-group per brick of groups.
template <bool TENSOR>
pcg_status launch_brick(const char *who, const pcg_grid *grid, TscArgs m, hipStream_t st)
{
    using K = Brick<TENSOR>;
    constexpr size_t bytes = brick_patch_bytes<TENSOR>();
    static const bool lds_ok =
        hipFuncSetAttribute((const void *)k_mass_tsc_brick<TENSOR>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
    if (!lds_ok)
        return fail(PCG_EHIP, "%s: cannot raise dynamic LDS to %zu bytes", who, bytes);
    m.nbricks = (uint32_t)(((grid->n[0] + K::BX - 1) / K::BX) * ((grid->n[1] + K::BY - 1) / K::BY) *
                           ((grid->n[2] + K::BZ - 1) / K::BZ));
    m.xcd_run = K::XCD_RUN;
    return launch(TENSOR ? "mass_tsc_tensor_mfma" : "mass_tsc_mfma", k_mass_tsc_brick<TENSOR>,
                  dim3(xcd_grid(m.nbricks, m.xcd_run)), dim3(K::WAVES * WAVE), bytes, st, m);
}

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
        else if (valu)
            PCG_TRY(launch("mass_tsc_valu", k_mass_tsc_valu, dim3(blocks),
                           dim3(TSC_WAVES * WAVE), 0, st, m));
        else
            PCG_TRY(launch_brick<TENSOR>(who, grid, m, st));
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
