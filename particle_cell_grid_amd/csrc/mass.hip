// mass.hip -- ECSIM mass-matrix assembly ([MM] Pennati & Markidis, "Mass Matrix
// Assembly on Tensor Cores for Implicit PIC": §2.1 Eq.(4)-(6), §2.2 Eq.(9)-(11),
// §3.1-§3.5), 3-D, CIC.
//
// Per particle: omega = beta B, a = 1 / (1 + |omega|^2) and
//   alpha_ij = a (delta_ij + eps_ijk omega_k + omega_i omega_j)
// (Eq.(5) written out with C(omega)_ij = -eps_ijk omega_k).  With
// u = (1, omega_x, omega_y, omega_z) and c_p = q w a, every component of the
// cell-local block M^{ij}_{ab} = sum_p s_p^{ij} W_ap W_bp (Eq.(15)) is a
// combination of ten "moment" matrices
//   T_kl[a][b] = sum_p c_p u_k u_l W_ap W_bp      (k <= l in 0..3):
//   M^ij = delta_ij T_00 + eps_ijk T_0(k+1) + T_(i+1)(j+1).
// Stacking rows r = 8k + a, the ten moments are the upper triangle of one
// 32x32 product  T = A B^T  with  A[r][p] = u_k W_a,  B[r][p] = c_p u_k W_a,
// a contraction over the cell's particles -- exactly the batched MMA form of
// §3.2 (Eq.(16)-(20)), here on v_mfma_f32_16x16x4_f32 tiles with K = 4
// particles per instruction and the accumulators kept in place across batches.
// Tiles (0,0), (0,1), (1,1) of the 2x2 tile grid hold all ten moments; tile
// (1,0) is skipped (symmetry, as in the paper's Table 1 for TSC).
//
// Assembly of M: instead of [MM] §3.4's per-cell flush with global atomics, a
// work-group owns a column of nodes, computes every cell that touches it (the
// cells on its low faces are computed by both neighbouring columns), adds each
// cell's block into LDS copies of two node planes and adds each finished plane
// to M once with plain loads and stores (see k_mass_column).  M is then
// written once per assembly, not once per cell-node pair.
//
// Variants: MFMA and VALU (the same column kernel; the moments of a cell come
// from the matrix cores or from per-lane FMAs) and FLAT (one thread per
// particle, alpha computed directly, 576 global atomics -- also used for the
// unsorted tail and for particles found in a cell slice they do not lie in).
//
// Scalar mass matrix ([MM] §2.1, the scalar case of Eq.(6): s_p = q_p w_p, one
// value per node pair, as for a mass matrix in MPM): the same kernels with
// SC = true.  B and beta are not read, u = (1, 0, 0, 0), only T_00 is formed
// and a node row of M holds 27 floats.  On the matrix cores one 16x16x4 product
// then takes eight particles: rows 0-7 of both operands carry the nodes of
// particles 8i + k and rows 8-15 those of particles 8i + 4 + k (k = 0..3), so
// the two diagonal 8x8 blocks of the result are T_00 of the two groups (the
// off-diagonal blocks mix particles and are dropped).
#include <algorithm>

#include "common.hpp"

namespace pcg {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// R, the arithmetic type of a variant: float, or double (M in fp64, every
// product and sum in fp64, the contractions on v_mfma_f64_16x16x4f64).  Both
// 16x16x4 products take A[i][k] and B[k][j] from lane i + 16 k (resp.
// j + 16 k); accumulator register r of lane l holds D[row][l % 16] with
// row = 4 (l / 16) + r in fp32 and row = l / 16 + 4 r in fp64 (measured).
template <typename R>
struct Real;
template <>
struct Real<float> {
    typedef floatx4 acc;
    typedef float2 pair;
};
template <>
struct Real<double> {
    typedef doublex4 acc;
    typedef double2 pair;
};

__device__ inline floatx4 mfma16x4(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ inline doublex4 mfma16x4(double a, double b, doublex4 c)
{
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <typename R>
__device__ inline int acc_row(int kk, int r)
{
    return sizeof(R) == 4 ? 4 * kk + r : kk + 4 * r;
}

__device__ inline void atomic_add_r(float *p, float v) { atomic_add_f32(p, v); }
__device__ inline void atomic_add_r(double *p, double v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct MassArgs {
    int n[3];
    float nf[3];
    const float *x[3];
    const float *B[3];
    const float *q;
    const float *w;
    const float *beta;
    void *M;  // R [n_z][n_y][n_x][27] (scalar) or [..][27][3][3]
    const uint32_t *cell_offsets;
    int64_t n_part;
    uint32_t ncells;
    int overwrite;  // the column kernel stores its rows of M without reading them
};

template <typename R>
__device__ inline R *mat(const MassArgs &m)
{
    return static_cast<R *>(m.M);
}

template <typename R>
struct Particle {
    R W[8];       // CIC node weights, a = ax + 2 ay + 4 az
    R u[4];       // (1, omega)
    R c;          // q w / (1 + |omega|^2)
    int base[3];  // cell (= first support node) per axis
};

// The nine per-particle input values, as loaded.
struct RawParticle {
    float x[3], B[3], q, w, beta;
};

// Floats per node row of M: 27 offsets x 9 tensor components, or 27 (scalar).
template <bool SC>
constexpr int row_floats()
{
    return SC ? 27 : 27 * 9;
}

// The scalar matrix reads no field: B and beta are zero constants, so omega,
// u = (1, 0, 0, 0) and c = q w fold at compile time.
template <bool SC>
__device__ inline RawParticle load_raw(const MassArgs &m, int64_t p)
{
    // particle counts are below 2^30, so a 32-bit byte offset from each array's
    // base addresses every element (one scalar base + one vector offset)
    const uint32_t off = (uint32_t)p * 4u;
    auto at = [off](const float *base) {
        return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + off);
    };
    RawParticle r;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        r.x[k] = at(m.x[k]);
        r.B[k] = SC ? 0.0f : at(m.B[k]);
    }
    r.q = at(m.q);
    r.w = at(m.w);
    r.beta = SC ? 0.0f : at(m.beta);
    return r;
}

// An empty use of every value of a particle: the compiler waits for its
// loads here.
template <bool SC>
__device__ __attribute__((always_inline)) inline void consume(const RawParticle &r)
{
    if constexpr (SC)
        asm volatile("" ::"v"(r.x[0]), "v"(r.x[1]), "v"(r.x[2]), "v"(r.q), "v"(r.w));
    else
        asm volatile("" ::"v"(r.x[0]), "v"(r.x[1]), "v"(r.x[2]), "v"(r.B[0]), "v"(r.B[1]),
                     "v"(r.B[2]), "v"(r.q), "v"(r.w), "v"(r.beta));
}

// i in [0, 2n) taken into [0, n): the node indices here are at most n (a
// coordinate clamped to [0, n], or the cell's upper neighbour), so one select
// replaces the general periodic wrap.
__device__ inline int wrap_once(int i, int n) { return i >= n ? i - n : i; }

// i in [-1, n] (a cell next to a column, whose nodes lie in [0, n)) wrapped.
__device__ inline int wrap_near(int i, int n) { return i < 0 ? i + n : wrap_once(i, n); }

template <typename R>
__device__ inline Particle<R> make_particle(const MassArgs &m, const RawParticle &r)
{
    Particle<R> P;
    R wx[3][2];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float x = clamp_coord(r.x[k], m.nf[k]);
        const float fl = floorf(x);
        const R xi = (R)(x - fl);  // exact in fp32
        P.base[k] = wrap_once((int)fl, m.n[k]);
        wx[k][0] = (R)1 - xi;
        wx[k][1] = xi;
    }
#pragma unroll
    for (int a = 0; a < 8; ++a)
        P.W[a] = wx[0][a & 1] * wx[1][(a >> 1) & 1] * wx[2][a >> 2];
    const R bt = r.beta;
    const R o0 = bt * (R)r.B[0], o1 = bt * (R)r.B[1], o2 = bt * (R)r.B[2];
    P.u[0] = (R)1;
    P.u[1] = o0;
    P.u[2] = o1;
    P.u[3] = o2;
    // fp32: the reciprocal instruction (within 1 ulp) instead of a correctly
    // rounded division, whose scaling and fix-up steps cost some ten more
    // instructions per particle
    if constexpr (sizeof(R) == 4)
        P.c = (r.q * r.w) * __builtin_amdgcn_rcpf(1.0f + (o0 * o0 + o1 * o1 + o2 * o2));
    else
        P.c = (R)r.q * (R)r.w / ((R)1 + (o0 * o0 + o1 * o1 + o2 * o2));
    return P;
}

template <bool SC, typename R>
__device__ inline Particle<R> load_particle(const MassArgs &m, int64_t p)
{
    return make_particle<R>(m, load_raw<SC>(m, p));
}

__device__ inline int64_t node_index(const MassArgs &m, const int *base, int a)
{
    const int gx = wrap_once(base[0] + (a & 1), m.n[0]);
    const int gy = wrap_once(base[1] + ((a >> 1) & 1), m.n[1]);
    const int gz = wrap_once(base[2] + (a >> 2), m.n[2]);
    return gx + (int64_t)m.n[0] * (gy + (int64_t)m.n[1] * gz);
}

__device__ inline int offset_index(int a, int b)
{
    return ((b & 1) - (a & 1) + 1) + 3 * (((b >> 1) & 1) - ((a >> 1) & 1) + 1) +
           9 * ((b >> 2) - (a >> 2) + 1);
}

// Nine components of M^{ij}_{ab} from the ten moments t[k][l] (k <= l).
template <typename R>
__device__ inline void moments_to_block(const R t[4][4], R *out)
{
    out[0] = t[0][0] + t[1][1];   // xx
    out[1] = t[0][3] + t[1][2];   // xy: +eps_xyz omega_z + omega_x omega_y
    out[2] = -t[0][2] + t[1][3];  // xz: -omega_y          + omega_x omega_z
    out[3] = -t[0][3] + t[1][2];  // yx
    out[4] = t[0][0] + t[2][2];   // yy
    out[5] = t[0][1] + t[2][3];   // yz: +omega_x          + omega_y omega_z
    out[6] = t[0][2] + t[1][3];   // zx
    out[7] = -t[0][1] + t[2][3];  // zy
    out[8] = t[0][0] + t[3][3];   // zz
}

// The particle's whole 8x8x9 (scalar: 8x8) contribution with global atomics.
template <bool SC, typename R>
__device__ inline void deposit_particle_global(const MassArgs &m, const Particle<R> &P)
{
    R t[4][4];
    int64_t g[8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
        g[a] = node_index(m, P.base, a);
    if constexpr (SC) {
        for (int a = 0; a < 8; ++a) {
            const R ca = P.c * P.W[a];
            R *row = mat<R>(m) + (size_t)g[a] * 27;
#pragma unroll
            for (int b = 0; b < 8; ++b)
                atomic_add_r(&row[offset_index(a, b)], ca * P.W[b]);
        }
        return;
    }
    for (int a = 0; a < 8; ++a) {
        for (int b = 0; b < 8; ++b) {
            const R wab = P.c * P.W[a] * P.W[b];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int l = k; l < 4; ++l)
                    t[k][l] = wab * P.u[k] * P.u[l];
            R blk[9];
            moments_to_block(t, blk);
            R *row = mat<R>(m) + ((size_t)g[a] * 27 + offset_index(a, b)) * 9;
#pragma unroll
            for (int ij = 0; ij < 9; ++ij)
                atomic_add_r(&row[ij], blk[ij]);
        }
    }
}

template <bool SC, typename R>
__global__ __launch_bounds__(256) void k_mass_flat(MassArgs m, int64_t begin, int64_t end)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < end; p += stride)
        deposit_particle_global<SC, R>(m, load_particle<SC, R>(m, p));
}

__device__ inline void cell_coords(const MassArgs &m, uint32_t cell, int *cc)
{
    cc[0] = (int)(cell % (uint32_t)m.n[0]);
    cc[1] = (int)((cell / (uint32_t)m.n[0]) % (uint32_t)m.n[1]);
    cc[2] = (int)(cell / ((uint32_t)m.n[0] * (uint32_t)m.n[1]));
}

// ---------------------------------------------------------------- column kernel
//
// Owner-computes assembly ([MM] §3.4 flushes per-cell blocks with atomics; here
// every row of M is written exactly once, by plain loads and stores):
// a work-group owns a column of COL_X x COL_Y x COL_Z nodes and walks the cell
// layers below and through it (z from the column's first node - 1 upwards).
// Node g receives from the eight cells g - {0,1}^3, so the work-group processes
// the (COL_X+1) x (COL_Y+1) x (COL_Z+1) cells that touch its nodes -- the cells
// on the low faces are also processed by the neighbouring column, each keeping
// only the entries of its own nodes.  Two node planes of the column live in
// LDS (27 x 9 fp32 per node): cell layer iz adds to node planes iz-1 and iz
// (local numbering), so node plane iz-1 is complete after layer iz and is added
// to M and its buffer cleared for plane iz+1.
// Within a layer, the cells are taken in four colour classes by (x, y) parity:
// two cells of one class share no node, so the waves that process them add to
// the planes without atomics; a barrier separates the classes.
#ifndef PCG_COL_X
#define PCG_COL_X 8
#define PCG_COL_Y 4
#define PCG_COL_Z 16
#endif
#ifndef PCG_COL_Z_SCALAR
#define PCG_COL_Z_SCALAR 8
#endif
constexpr int COL_X = PCG_COL_X, COL_Y = PCG_COL_Y, COL_Z = PCG_COL_Z;
constexpr int COL_WAVES = 4;
constexpr int COL_NODES = COL_X * COL_Y;

// Column height: the scalar matrix does little work per cell, so its
// work-groups wait on loads at every phase; a lower column takes fewer
// phases per work-group and spreads the grid over more of them.
template <bool SC>
constexpr int col_z()
{
    return SC ? PCG_COL_Z_SCALAR : COL_Z;
}

// LDS staging of one 64-particle batch of a cell, per wave; reused for the
// 32 x 32 moment tile once the batches are done.
template <typename R>
struct Stage {
    R W[64][8];
    R u[64][4];  // stored as (u0, u2, u1, u3) so (u_k, u_{k+2}) are adjacent
    R c[64];
};
template <typename R>
union WaveScratch {
    Stage<R> s;
    R Tm[32][33];
};

// The work-group's LDS: two node planes and one scratch per wave (fp64
// tensor: 158,208 bytes, within the 160 KiB of a CU).
template <bool SC, typename R>
constexpr size_t column_lds_bytes()
{
    return sizeof(R) * 2 * COL_NODES * row_floats<SC>() + sizeof(WaveScratch<R>) * COL_WAVES;
}
static_assert(column_lds_bytes<false, double>() <= 160 * 1024, "fp64 planes exceed the LDS");

// Orders this wave's earlier LDS accesses before its later ones (lanes exchange
// data through LDS within one wave only).
__device__ inline void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stages one particle (raw values, valid = the slot is inside the cell's slice)
// into the lane's row.  A particle that lies in another cell (a stale layout)
// is staged with c = 0 and reported through *stray: the follow-up pass
// deposits it.
template <bool SC, typename R>
__device__ inline void stage_raw(const MassArgs &m, Stage<R> &s, int lane, const RawParticle &r,
                                 bool valid, const int *cell, bool *stray)
{
    // computed for every lane (an empty slot holds zeros), then selected:
    // no divergent branches.  Only c is zeroed for a slot that is not the
    // cell's: every product of the moments takes c once, and the weights and
    // u of a loaded particle are finite
    const Particle<R> P = make_particle<R>(m, r);
    const bool home = P.base[0] == cell[0] && P.base[1] == cell[1] && P.base[2] == cell[2];
    const bool take = valid && home;
    *stray = *stray || (valid && !home);
    R W[8], u[4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
        W[a] = P.W[a];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        u[k] = P.u[k];
    const R c = take ? P.c : (R)0;
    if constexpr (sizeof(R) == 4) {
        float4 *w4 = reinterpret_cast<float4 *>(s.W[lane]);
        w4[0] = make_float4(W[0], W[1], W[2], W[3]);
        w4[1] = make_float4(W[4], W[5], W[6], W[7]);
        if constexpr (!SC)
            *reinterpret_cast<float4 *>(s.u[lane]) = make_float4(u[0], u[2], u[1], u[3]);
    } else {
        double2 *w2 = reinterpret_cast<double2 *>(s.W[lane]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w2[i] = make_double2(W[2 * i], W[2 * i + 1]);
        if constexpr (!SC) {
            double2 *u2 = reinterpret_cast<double2 *>(s.u[lane]);
            u2[0] = make_double2(u[0], u[2]);
            u2[1] = make_double2(u[1], u[3]);
        }
    }
    s.c[lane] = c;
}

// One wave: the ten moments of cell `cell` (wrapped coordinates), whose slice
// is [lo, hi), for this lane's node pair (a, b) = (lane / 8, lane % 8):
// t[k][l] for k <= l (scalar: t[0][0] only).  `first` holds the lane's
// particle of the first batch (slot lo + lane), loaded ahead by the caller;
// later batches (cells of more than 64 particles) are loaded here.
template <bool MFMA, bool SC, typename R>
__device__ inline void cell_moments(const MassArgs &m, WaveScratch<R> &ws, int lane,
                                    const int *cell, int64_t lo, int64_t hi,
                                    const RawParticle &first, bool *stray, R t[4][4])
{
    typedef typename Real<R>::acc Acc;
    typedef typename Real<R>::pair Pair;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int l = 0; l < 4; ++l)
            t[k][l] = (R)0;
    if (hi <= lo)
        return;
    const int pa = lane >> 3, pb = lane & 7;
    // operand coordinates (MFMA): row/col index r = lane % 16 of a 16-row
    // block, particle kk = lane / 16 of the 4-particle batch
    const int r = lane & 15, kk = lane >> 4;
    const int a = r & 7, khalf = r >> 3;  // node a, moment index k = khalf (+2)
    Acc acc00 = {0, 0, 0, 0}, acc01 = {0, 0, 0, 0}, acc11 = {0, 0, 0, 0};
    auto batch = [&](const RawParticle &rp, int64_t base) {
        wave_sync();
        stage_raw<SC, R>(m, ws.s, lane, rp, base + lane < hi, cell, stray);
        wave_sync();
        const int nb = (int)std::min<int64_t>(64, hi - base);
        if constexpr (MFMA && SC) {
            // eight particles per product: row half khalf takes particle
            // 8 i + 4 khalf + kk (staged rows past the slice are zero)
            auto slot = [&](int i) { return 8 * i + 4 * khalf + kk; };
            if (nb == 64) {
                R wa[8], cp[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    wa[i] = ws.s.W[slot(i)][a];
                    cp[i] = ws.s.c[slot(i)];
                }
                __builtin_amdgcn_sched_barrier(0);
                R cw[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    cw[i] = cp[i] * wa[i];
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc00 = mfma16x4(wa[i], cw[i], acc00);
            } else {
                const int batches = (nb + 7) >> 3;
                for (int bt = 0; bt < batches; ++bt) {
                    const R wa = ws.s.W[slot(bt)][a];
                    acc00 = mfma16x4(wa, ws.s.c[slot(bt)] * wa, acc00);
                }
            }
        } else if constexpr (SC) {
            for (int q = 0; q < nb; ++q)
                t[0][0] += ws.s.c[q] * ws.s.W[q][pa] * ws.s.W[q][pb];
        } else if constexpr (MFMA) {
            // one 4-particle batch: operands from the staged rows, three MFMAs
            auto mfma_batch = [&](R wa, Pair uu, R cp) {
                const R a0 = uu.x * wa;  // u_k W_a      (k = khalf)
                const R a1 = uu.y * wa;  // u_{k+2} W_a
                const R b0 = cp * a0;
                const R b1 = cp * a1;
                acc00 = mfma16x4(a0, b0, acc00);
                acc01 = mfma16x4(a0, b1, acc01);
                acc11 = mfma16x4(a1, b1, acc11);
            };
            if (nb == 64) {
                // a full batch: the operands of G 4-particle steps are read
                // first (one LDS round trip), then their 3 G products issue
                // back to back (G = 16 in fp32, 8 in fp64 for registers)
                constexpr int G = sizeof(R) == 4 ? 16 : 8;
#pragma unroll
                for (int g0 = 0; g0 < 16; g0 += G) {
                    R wa[G], cp[G];
                    Pair uu[G];
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        const int q = 4 * (g0 + i) + kk;
                        wa[i] = ws.s.W[q][a];
                        uu[i] = *reinterpret_cast<const Pair *>(&ws.s.u[q][2 * khalf]);
                        cp[i] = ws.s.c[q];
                    }
                    // keep the reads ahead of the products (the scheduler would
                    // otherwise interleave them and wait once per step), and
                    // the operand products ahead of the matrix instructions:
                    // a product issued just before the instruction that reads
                    // it costs wait states, and on this chip matrix and vector
                    // instructions of a SIMD do not overlap
                    __builtin_amdgcn_sched_barrier(0);
                    R A0[G], A1[G], B0[G], B1[G];
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        A0[i] = uu[i].x * wa[i];
                        A1[i] = uu[i].y * wa[i];
                        B0[i] = cp[i] * A0[i];
                        B1[i] = cp[i] * A1[i];
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        acc00 = mfma16x4(A0[i], B0[i], acc00);
                        acc01 = mfma16x4(A0[i], B1[i], acc01);
                        acc11 = mfma16x4(A1[i], B1[i], acc11);
                    }
                }
            } else {
                const int batches = (nb + 3) >> 2;
                for (int bt = 0; bt < batches; ++bt) {
                    const int q = 4 * bt + kk;
                    mfma_batch(ws.s.W[q][a], *reinterpret_cast<const Pair *>(&ws.s.u[q][2 * khalf]),
                               ws.s.c[q]);
                }
            }
        } else {
            for (int q = 0; q < nb; ++q) {
                const R wab = ws.s.c[q] * ws.s.W[q][pa] * ws.s.W[q][pb];
                const R u[4] = {ws.s.u[q][0], ws.s.u[q][2], ws.s.u[q][1], ws.s.u[q][3]};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const R wk = wab * u[k];
#pragma unroll
                    for (int l = k; l < 4; ++l)
                        t[k][l] += wk * u[l];
                }
            }
        }
    };
    batch(first, lo);
    // cells of more than 64 particles: the later batches load here
    for (int64_t base = lo + 64; base < hi; base += 64) {
        // clamped load, waited for at once: the wait stays on this rare path
        const RawParticle rp = load_raw<SC>(m, std::min<int64_t>(base + lane, hi - 1));
        consume<SC>(rp);
        batch(rp, base);
    }
    wave_sync();
    if constexpr (MFMA && SC) {
        // the two diagonal 8x8 blocks of the accumulator, summed
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ws.Tm[acc_row<R>(kk, i)][r] = acc00[i];
        wave_sync();
        t[0][0] = ws.Tm[pa][pb] + ws.Tm[8 + pa][8 + pb];
        wave_sync();
    } else if constexpr (MFMA) {
        // accumulator register i of this lane holds D[acc_row(kk, i)][lane % 16]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = acc_row<R>(kk, i), col = r;
            ws.Tm[row][col] = acc00[i];
            ws.Tm[row][16 + col] = acc01[i];
            ws.Tm[16 + row][16 + col] = acc11[i];
        }
        wave_sync();
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int l = k; l < 4; ++l)
                t[k][l] = ws.Tm[8 * k + pa][8 * l + pb];
        wave_sync();
    }
}

// Values of one y row of a column plane (COL_X nodes, contiguous in M) each
// thread adds to M after a layer.
template <bool SC>
constexpr int col_row_per_thread()
{
    return (COL_X * row_floats<SC>() + COL_WAVES * WAVE - 1) / (COL_WAVES * WAVE);
}

struct ColumnGeom {
    int ncol[3];  // columns per axis
    uint32_t nwork;
    uint32_t *stray_flag;
};

// The column one work-group owns: first node and node count per axis; the
// cells touching it have local index i <-> cell first - 1 + i, i < count + 1.
struct ColumnShape {
    int first[3], count[3];
};

// Cells of one colour class (x, y parity) in a layer; nx of them per row.
__device__ inline int colour_cells(const ColumnShape &c, int colour, int &nx)
{
    const int px = colour & 1, py = colour >> 1;
    nx = (c.count[0] + 1 - px + 1) / 2;
    return nx * ((c.count[1] + 1 - py + 1) / 2);
}

// Cells per wave and phase: the largest colour class of a full column,
// ceil((COL_X+2)/2) * ceil((COL_Y+2)/2), shared by the work-group's waves.
constexpr int COL_SLOTS =
    ((COL_X + 2) / 2 * ((COL_Y + 2) / 2) + COL_WAVES - 1) / COL_WAVES;

// The wave's cells of every colour class, tabled once per work-group (the
// class sizes are the same in every layer): lane colour * COL_SLOTS + k holds
// the local (x, y) index of the wave's k-th cell of that class as
// x | y << 8 with bit 31 set, or 0 if the wave has no such cell.
__device__ inline uint32_t colour_table(const ColumnShape &c, int wave)
{
    const int lane = lane_id();
    uint32_t e = 0;
    if (lane < 4 * COL_SLOTS) {
        const int colour = lane / COL_SLOTS, k = lane % COL_SLOTS;
        int nx;
        const int cnt = colour_cells(c, colour, nx);
        const int j = wave + COL_WAVES * k;
        if (j < cnt)
            e = 0x80000000u | (uint32_t)((colour & 1) + 2 * (j % nx)) |
                ((uint32_t)((colour >> 1) + 2 * (j / nx)) << 8);
    }
    return e;
}

// Local and wrapped coordinates of table entry e in layer iz; false if the
// entry is empty or the layer is past the column.
__device__ inline bool entry_cell(const MassArgs &m, const ColumnShape &c, uint32_t e, int iz,
                                  int *li, int *cell)
{
    if (!(e >> 31) || iz > c.count[2])
        return false;
    li[0] = (int)(e & 0xffu);
    li[1] = (int)((e >> 8) & 0xffu);
    li[2] = iz;
#pragma unroll
    for (int a = 0; a < 3; ++a)
        cell[a] = wrap_near(c.first[a] - 1 + li[a], m.n[a]);
    return true;
}

// A wave's k-th cell of phase ph (layer ph / 4, colour ph % 4): local and
// wrapped coordinates; false if the wave has no such cell.  ph and k are
// uniform: one lane read of the table.
__device__ inline bool phase_cell(const MassArgs &m, const ColumnShape &c, uint32_t table, int ph,
                                  int k, int *li, int *cell)
{
    const uint32_t e = __builtin_amdgcn_readlane(table, (ph & 3) * COL_SLOTS + k);
    return entry_cell(m, c, e, ph >> 2, li, cell);
}

__device__ inline uint32_t cell_id(const MassArgs &m, const int *cell)
{
    return (uint32_t)cell[0] + (uint32_t)m.n[0] * ((uint32_t)cell[1] + (uint32_t)m.n[1] * cell[2]);
}

// Slice bounds of this wave's cells of phase ph, one vector read: lane 2k
// gets the low bound of cell k, lane 2k+1 the high one (0 for no cell).
__device__ inline uint32_t phase_offsets(const MassArgs &m, const ColumnShape &c, uint32_t table,
                                        int ph)
{
    const int lane = lane_id();
    // every lane takes part in the shuffle; lanes past 2 COL_SLOTS drop it
    const uint32_t e = (uint32_t)__shfl((int)table, (ph & 3) * COL_SLOTS + ((lane >> 1) & 3), WAVE);
    uint32_t v = 0;
    int li[3], cell[3];
    if (lane < 2 * COL_SLOTS && entry_cell(m, c, e, ph >> 2, li, cell))
        v = m.cell_offsets[cell_id(m, cell) + (lane & 1)];
    return v;
}

// Bounds of cell k from a phase_offsets() vector, clipped to the partitioned
// prefix.
__device__ inline void slot_bounds(const MassArgs &m, uint32_t offv, int k, int64_t &lo,
                                   int64_t &hi)
{
    lo = std::min<int64_t>(__builtin_amdgcn_readlane(offv, 2 * k), m.n_part);
    hi = std::min<int64_t>(__builtin_amdgcn_readlane(offv, 2 * k + 1), m.n_part);
}

// The first batch of every cell of one phase, one particle per lane and cell
// (COL_SLOTS = 4 named slots, so that they stay in registers).
static_assert(COL_SLOTS >= 1 && COL_SLOTS <= 4, "PhaseRaw holds at most four slots");
struct PhaseRaw {
    RawParticle r0, r1, r2, r3;
};

template <bool SC>
__device__ inline RawParticle load_slot(const MassArgs &m, uint32_t offv, int k)
{
    int64_t lo, hi;
    slot_bounds(m, offv, k, lo, hi);
    RawParticle r{};
    if (lo + lane_id() < hi)
        r = load_raw<SC>(m, lo + lane_id());
    return r;
}

template <bool SC>
__device__ inline void load_phase(const MassArgs &m, uint32_t offv, PhaseRaw &pr)
{
    pr.r0 = load_slot<SC>(m, offv, 0);
    pr.r1 = COL_SLOTS > 1 ? load_slot<SC>(m, offv, 1) : RawParticle{};
    pr.r2 = COL_SLOTS > 2 ? load_slot<SC>(m, offv, 2) : RawParticle{};
    pr.r3 = COL_SLOTS > 3 ? load_slot<SC>(m, offv, 3) : RawParticle{};
}

template <bool SC>
__device__ __attribute__((always_inline)) inline void consume(const PhaseRaw &p)
{
    consume<SC>(p.r0);
    if (COL_SLOTS > 1)
        consume<SC>(p.r1);
    if (COL_SLOTS > 2)
        consume<SC>(p.r2);
    if (COL_SLOTS > 3)
        consume<SC>(p.r3);
}

// Slot k (uniform) of a phase, selected field by field.
__device__ inline float pick1(int k, float a, float b, float c, float d)
{
    return k == 0 ? a : (k == 1 ? b : (k == 2 ? c : d));
}

__device__ inline RawParticle pick(const PhaseRaw &p, int k)
{
    RawParticle r;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        r.x[i] = pick1(k, p.r0.x[i], p.r1.x[i], p.r2.x[i], p.r3.x[i]);
        r.B[i] = pick1(k, p.r0.B[i], p.r1.B[i], p.r2.B[i], p.r3.B[i]);
    }
    r.q = pick1(k, p.r0.q, p.r1.q, p.r2.q, p.r3.q);
    r.w = pick1(k, p.r0.w, p.r1.w, p.r2.w, p.r3.w);
    r.beta = pick1(k, p.r0.beta, p.r1.beta, p.r2.beta, p.r3.beta);
    return r;
}

template <bool MFMA, bool SC, typename R>
__global__ __launch_bounds__(COL_WAVES * WAVE) void k_mass_column(MassArgs m, ColumnGeom cg)
{
    constexpr int ROW = row_floats<SC>();
    constexpr int COL_ROW_PER_THREAD = col_row_per_thread<SC>();
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    R *planes = reinterpret_cast<R *>(smem);  // [2][COL_NODES][ROW]
    WaveScratch<R> *scratch =
        reinterpret_cast<WaveScratch<R> *>(smem + sizeof(R) * 2 * COL_NODES * ROW);
    // the wave index is uniform across the wave: keep the walk over the cells
    // (and everything derived from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = lane_id();
    WaveScratch<R> &ws = scratch[wave];

    // spread spatially adjacent columns over consecutive blocks of one XCD
    // (blocks are dealt to the 8 XCDs round-robin), so the cells two columns
    // share are read through the same L2
    const uint32_t nw = cg.nwork;
    const uint32_t per = (nw + 7) / 8;
    const uint32_t b = blockIdx.x;
    const uint32_t work = (b % 8) * per + b / 8;
    if (work >= nw)
        return;
    ColumnShape cs;
    {
        const int idx[3] = {(int)(work % (uint32_t)cg.ncol[0]),
                            (int)((work / (uint32_t)cg.ncol[0]) % (uint32_t)cg.ncol[1]),
                            (int)(work / ((uint32_t)cg.ncol[0] * (uint32_t)cg.ncol[1]))};
        const int edge[3] = {COL_X, COL_Y, col_z<SC>()};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            cs.first[k] = idx[k] * edge[k];
            cs.count[k] = min(edge[k], m.n[k] - cs.first[k]);
        }
    }
    const int BX = cs.count[0], BY = cs.count[1], BZ = cs.count[2];
    const int nphase = 4 * (BZ + 1);

    for (int i = threadIdx.x; i < 2 * COL_NODES * ROW; i += blockDim.x)
        planes[i] = (R)0;

    // Reads run one phase ahead of their use: during phase ph the first
    // batches of the wave's cells of phase ph + 1 and the slice bounds of
    // phase ph + 2 are in flight.
    const uint32_t table = colour_table(cs, wave);
    uint32_t off_next = phase_offsets(m, cs, table, 1);
    PhaseRaw cur, nxt;
    uint32_t off_cur = phase_offsets(m, cs, table, 0);
    load_phase<SC>(m, off_cur, cur);
    __syncthreads();

    consume<SC>(cur);
    asm volatile("" ::"v"(off_cur), "v"(off_next));
    bool stray = false;
    const int pa = lane >> 3, pb = lane & 7;
    const int ax = pa & 1, ay = (pa >> 1) & 1, az = pa >> 2;
    const int o = offset_index(pa, pb);
    for (int ph = 0; ph < nphase; ++ph) {
        const int iz = ph >> 2;
        load_phase<SC>(m, off_next, nxt);
        const uint32_t off_after = phase_offsets(m, cs, table, ph + 2);
        // the compiler must not sink these reads to their use
        asm volatile("" ::: "memory");

        const int lz = iz - 1 + az;  // local node plane of this lane's row
        // unrolled: each slot's particle registers are then named statically
        // (a runtime slot index costs a chain of uniform branches per field)
#pragma unroll
        for (int k = 0; k < COL_SLOTS; ++k) {
            int li[3], cell[3];
            if (!phase_cell(m, cs, table, ph, k, li, cell))
                break;
            int64_t lo, hi;
            slot_bounds(m, off_cur, k, lo, hi);
            bool st = false;
            R t[4][4];
            cell_moments<MFMA, SC, R>(m, ws, lane, cell, lo, hi, pick(cur, k), &st, t);
            // a cell's stray particles are reported by the column holding its
            // first node (each cell has exactly one such column)
            if (li[0] >= 1 && li[1] >= 1 && li[2] >= 1)
                stray |= st;
            const int lx = li[0] - 1 + ax, ly = li[1] - 1 + ay;
            if (lx >= 0 && lx < BX && ly >= 0 && ly < BY && lz >= 0 && lz < BZ) {
                // the product is kept out of the address add: fused, it becomes
                // a 64-bit multiply-add whose unused high addend can share a
                // register with an in-flight load, and then waits for every
                // outstanding load
                uint32_t e = ((lz & 1) * COL_NODES + ly * COL_X + lx) * ROW;
                asm("" : "+v"(e));
                R *node = planes + e;
                if constexpr (SC) {
                    node[o] += t[0][0];
                } else {
                    R blk[9];
                    moments_to_block(t, blk);
#pragma unroll
                    for (int ij = 0; ij < 9; ++ij)
                        node[o * 9 + ij] += blk[ij];
                }
            }
        }
        // the next phase's operands (loaded during this one) are taken over and
        // waited for here, before the write-out's stores: later uses then need
        // no waits, which would also drain those stores or the next loads
        cur = nxt;
        off_cur = off_next;
        off_next = off_after;
        consume<SC>(cur);
        asm volatile("" ::"v"(off_cur), "v"(off_next));
        __syncthreads();

        // after the layer's last colour node plane iz - 1 is complete: add it
        // to M (rows of the column are contiguous in M along x) and clear it
        const int done = iz - 1;
        if ((ph & 3) == 3 && done >= 0) {
            const int gz = cs.first[2] + done;
            R *pl = planes + (size_t)(done & 1) * COL_NODES * ROW;
            // every row's M values are read first (one round trip), then each
            // row is added and stored
            R v[COL_Y][COL_ROW_PER_THREAD];
#pragma unroll
            for (int ly = 0; ly < COL_Y; ++ly) {
                const R *dst = mat<R>(m) + (cs.first[0] + (int64_t)m.n[0] *
                                            ((cs.first[1] + ly) + (int64_t)m.n[1] * gz)) * ROW;
#pragma unroll
                for (int q = 0; q < COL_ROW_PER_THREAD; ++q) {
                    const int r = threadIdx.x + q * COL_WAVES * WAVE;
                    v[ly][q] = ly < BY && r < BX * ROW && !m.overwrite ? dst[r] : (R)0;
                }
            }
            // one wait for all of them, so that the stores below need none
#pragma unroll
            for (int ly = 0; ly < COL_Y; ++ly)
#pragma unroll
                for (int q = 0; q < COL_ROW_PER_THREAD; ++q)
                    asm volatile("" ::"v"(v[ly][q]));
#pragma unroll
            for (int ly = 0; ly < COL_Y; ++ly) {
                if (ly >= BY)
                    break;
                R *dst = mat<R>(m) + (cs.first[0] + (int64_t)m.n[0] *
                                      ((cs.first[1] + ly) + (int64_t)m.n[1] * gz)) * ROW;
                R *src = pl + ly * COL_X * ROW;
#pragma unroll
                for (int q = 0; q < COL_ROW_PER_THREAD; ++q) {
                    const int r = threadIdx.x + q * COL_WAVES * WAVE;
                    if (r < BX * ROW) {
                        dst[r] = v[ly][q] + src[r];
                        src[r] = (R)0;  // only this thread read this value
                    }
                }
            }
            __syncthreads();
        }
    }
    if (stray && cg.stray_flag)
        atomicOr(cg.stray_flag, 1u);
}

// Follow-up of the column kernel, run only when it found stray particles: each
// thread walks one cell's slice and deposits the particles that lie elsewhere
// with global atomics.
template <bool SC, typename R>
__global__ __launch_bounds__(256) void k_mass_strays(MassArgs m, const uint32_t *flag)
{
    if (*flag == 0u)
        return;
    for (uint32_t cid = blockIdx.x * blockDim.x + threadIdx.x; cid < m.ncells;
         cid += gridDim.x * blockDim.x) {
        int cc[3];
        cell_coords(m, cid, cc);
        const int64_t lo = std::min<int64_t>(m.cell_offsets[cid], m.n_part);
        const int64_t hi = std::min<int64_t>(m.cell_offsets[cid + 1], m.n_part);
        for (int64_t p = lo; p < hi; ++p) {
            const Particle<R> P = load_particle<SC, R>(m, p);
            if (P.base[0] != cc[0] || P.base[1] != cc[1] || P.base[2] != cc[2])
                deposit_particle_global<SC, R>(m, P);
        }
    }
}

__global__ void k_mass_clear_flag(uint32_t *flag) { *flag = 0u; }

// M = 0 ahead of a path that only adds (the overwrite flag without the column
// kernel).
template <typename R>
__global__ __launch_bounds__(256) void k_mass_zero(R *__restrict__ M, int64_t len)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len; i += stride)
        M[i] = (R)0;
}

}  // namespace
}  // namespace pcg

using namespace pcg;

namespace {

// Workspace: one device flag (the column kernel raises it when it meets stray
// particles), padded to 256 bytes.
constexpr size_t MASS_WORKSPACE = 256;

// Launch names: mass_[scalar_]{mfma,valu,flat,strays}[_f64].
template <bool SC, typename R>
const char *kernel_name(int which)
{
    static const char *const names[2][2][4] = {
        {{"mass_mfma", "mass_valu", "mass_flat", "mass_strays"},
         {"mass_mfma_f64", "mass_valu_f64", "mass_flat_f64", "mass_strays_f64"}},
        {{"mass_scalar_mfma", "mass_scalar_valu", "mass_scalar_flat", "mass_scalar_strays"},
         {"mass_scalar_mfma_f64", "mass_scalar_valu_f64", "mass_scalar_flat_f64",
          "mass_scalar_strays_f64"}}};
    return names[SC ? 1 : 0][sizeof(R) == 8 ? 1 : 0][which];
}

template <bool MFMA, bool SC, typename R>
pcg_status launch_column(const MassArgs &m, const ColumnGeom &cg, hipStream_t st)
{
    auto kern = k_mass_column<MFMA, SC, R>;
    const size_t lds = column_lds_bytes<SC, R>();
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
        return fail(PCG_EHIP, "mass matrix: cannot raise dynamic LDS to %zu bytes", lds);
    const uint32_t blocks = (cg.nwork + 7) / 8 * 8;
    return launch(kernel_name<SC, R>(MFMA ? 0 : 1), kern, dim3(blocks), dim3(COL_WAVES * WAVE),
                  lds, st, m, cg);
}

// Every entry point: the tensor matrix (B and beta given) or the scalar one,
// with M in R.
template <bool SC, typename R>
pcg_status assemble(const char *who, const pcg_grid *grid, const pcg_particles *particles,
                    const float *const B[3], const float *beta, const pcg_tile *cells,
                    int32_t variant, R *M, void *workspace, size_t workspace_bytes,
                    void *stream)
{
    clear_error();
    PCG_TRY(check_grid(grid, who));
    if (grid->dim != 3)
        return fail(PCG_EUNSUPPORTED, "%s: only 3-D grids (dim = %d)", who, grid->dim);
    for (int k = 0; k < 3; ++k)
        if (grid->n[k] < 3)
            return fail(PCG_EINVAL, "%s: n[%d] = %d < 3 (the 27 offsets must be distinct nodes)",
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
    if (count > 0) {
        for (int k = 0; k < 3; ++k)
            if (!particles->x[k] || (!SC && (!B || !B[k])))
                return fail(PCG_EINVAL, SC ? "%s: x[%d] is NULL" : "%s: x[%d] or B[%d] is NULL",
                            who, k, k);
        if (!particles->q || !particles->w || (!SC && !beta))
            return fail(PCG_EINVAL, SC ? "%s: q or w is NULL" : "%s: q, w or beta is NULL", who);
    }
    MassArgs m{};
    for (int k = 0; k < 3; ++k) {
        m.n[k] = grid->n[k];
        m.nf[k] = (float)grid->n[k];
        m.x[k] = particles->x[k];
        m.B[k] = !SC && B ? B[k] : nullptr;
    }
    m.q = particles->q;
    m.w = particles->w;
    m.beta = SC ? nullptr : beta;
    m.M = M;
    m.ncells = (uint32_t)((int64_t)grid->n[0] * grid->n[1] * grid->n[2]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // M = 0 (overwrite) where the column kernel will not set every row; run
    // only once the arguments have passed every check
    auto zero = [&]() -> pcg_status {
        if (!overwrite)
            return PCG_OK;
        const int64_t len = (int64_t)m.ncells * row_floats<SC>();
        const int64_t blocks = std::min<int64_t>((len + 255) / 256, (int64_t)device_cus() * 16);
        return launch("mass_zero", k_mass_zero<R>, dim3((unsigned)blocks), dim3(256), 0, st,
                      M, len);
    };
    if (count == 0)
        return zero();
    auto flat = [&](int64_t begin, int64_t end) -> pcg_status {
        if (end <= begin)
            return PCG_OK;
        const int64_t blocks =
            std::min<int64_t>((end - begin + 255) / 256, (int64_t)device_cus() * 32);
        return launch(kernel_name<SC, R>(2), k_mass_flat<SC, R>, dim3((unsigned)blocks),
                      dim3(256), 0, st, m, begin, end);
    };
    if (variant == PCG_MASS_FLAT || (!cells && variant == PCG_MASS_AUTO)) {
        PCG_TRY(zero());
        return flat(0, count);
    }
    if (!cells)
        return fail(PCG_EINVAL, "%s: the %s variant needs a cell layout", who,
                    variant == PCG_MASS_VALU ? "VALU" : "MFMA");
    if (cells->T != 1 || cells->order != 1)
        return fail(PCG_EINVAL, "%s: cells must be a T = 1, order = 1 layout (T = %d, order = %d)",
                    who, cells->T, cells->order);
    if (!cells->tile_offsets)
        return fail(PCG_EINVAL, "%s: cell offsets are NULL", who);
    if (cells->n_partitioned < 0 || cells->n_partitioned > count)
        return fail(PCG_EINVAL, "%s: n_partitioned outside [0, count]", who);
    if (!workspace || workspace_bytes < MASS_WORKSPACE)
        return fail(PCG_EWORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who,
                    workspace_bytes, MASS_WORKSPACE);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(PCG_EWORKSPACE, "%s: workspace is not 256-byte aligned", who);
    m.cell_offsets = cells->tile_offsets;
    m.n_part = cells->n_partitioned;
    ColumnGeom cg{};
    cg.ncol[0] = (grid->n[0] + COL_X - 1) / COL_X;
    cg.ncol[1] = (grid->n[1] + COL_Y - 1) / COL_Y;
    cg.ncol[2] = (grid->n[2] + col_z<SC>() - 1) / col_z<SC>();
    cg.nwork = (uint32_t)cg.ncol[0] * cg.ncol[1] * cg.ncol[2];
    cg.stray_flag = static_cast<uint32_t *>(workspace);
    if (m.n_part == 0)
        PCG_TRY(zero());
    m.overwrite = overwrite ? 1 : 0;  // the column kernel sets every row
    if (m.n_part > 0) {
        PCG_TRY(launch("mass_clear_flag", k_mass_clear_flag, dim3(1), dim3(1), 0, st,
                       cg.stray_flag));
        if (variant == PCG_MASS_VALU)
            PCG_TRY((launch_column<false, SC, R>(m, cg, st)));
        else
            PCG_TRY((launch_column<true, SC, R>(m, cg, st)));
        const int64_t sblocks =
            std::min<int64_t>((m.ncells + 255) / 256, (int64_t)device_cus() * 8);
        PCG_TRY(launch(kernel_name<SC, R>(3), k_mass_strays<SC, R>, dim3((unsigned)sblocks),
                       dim3(256), 0, st, m, (const uint32_t *)cg.stray_flag));
    }
    return flat(cells->n_partitioned, count);
}

}  // namespace

extern "C" size_t pcg_mass_workspace_bytes(const pcg_grid *grid)
{
    (void)grid;
    return MASS_WORKSPACE;
}

extern "C" pcg_status assemble_mass_matrix(const pcg_grid *grid, const pcg_particles *particles,
                                           const float *const B[3], const float *beta,
                                           const pcg_tile *cells, int32_t variant, float *M,
                                           void *workspace, size_t workspace_bytes, void *stream)
{
    return assemble<false, float>("assemble_mass_matrix", grid, particles, B, beta, cells,
                                  variant, M, workspace, workspace_bytes, stream);
}

extern "C" pcg_status assemble_mass_matrix_scalar(const pcg_grid *grid,
                                                  const pcg_particles *particles,
                                                  const pcg_tile *cells, int32_t variant, float *M,
                                                  void *workspace, size_t workspace_bytes,
                                                  void *stream)
{
    return assemble<true, float>("assemble_mass_matrix_scalar", grid, particles, nullptr, nullptr,
                                 cells, variant, M, workspace, workspace_bytes, stream);
}

extern "C" pcg_status assemble_mass_matrix_f64(const pcg_grid *grid,
                                               const pcg_particles *particles,
                                               const float *const B[3], const float *beta,
                                               const pcg_tile *cells, int32_t variant, double *M,
                                               void *workspace, size_t workspace_bytes,
                                               void *stream)
{
    return assemble<false, double>("assemble_mass_matrix_f64", grid, particles, B, beta, cells,
                                   variant, M, workspace, workspace_bytes, stream);
}

extern "C" pcg_status assemble_mass_matrix_scalar_f64(const pcg_grid *grid,
                                                      const pcg_particles *particles,
                                                      const pcg_tile *cells, int32_t variant,
                                                      double *M, void *workspace,
                                                      size_t workspace_bytes, void *stream)
{
    return assemble<true, double>("assemble_mass_matrix_scalar_f64", grid, particles, nullptr,
                                  nullptr, cells, variant, M, workspace, workspace_bytes, stream);
}
