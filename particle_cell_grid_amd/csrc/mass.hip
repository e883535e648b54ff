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
// Flush ([MM] §3.4): lane (a,b) forms the nine M^{ij}_{ab} and adds them to the
// 27-offset store at row g_a, offset o(b - a) with global atomics.
//
// Variants: MFMA (one wave per cell), VALU (same staging, each lane
// accumulating its (a,b) moments with FMAs) and FLAT (one thread per particle,
// alpha computed directly, 576 global atomics -- also used for the tail and for
// particles found in a cell slice they do not belong to).
#include <algorithm>

#include "common.hpp"

namespace pcg {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

struct MassArgs {
    int n[3];
    float nf[3];
    const float *x[3];
    const float *B[3];
    const float *q;
    const float *w;
    const float *beta;
    float *M;
    const uint32_t *cell_offsets;
    int64_t n_part;
    uint32_t ncells;
};

struct Particle {
    float W[8];     // CIC node weights, a = ax + 2 ay + 4 az
    float u[4];     // (1, omega)
    float c;        // q w / (1 + |omega|^2)
    int base[3];    // cell (= first support node) per axis
};

__device__ inline Particle load_particle(const MassArgs &m, int64_t p)
{
    Particle P;
    float wx[3][2];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float x = clamp_coord(m.x[k][p], m.nf[k]);
        const float fl = floorf(x);
        const float xi = x - fl;
        P.base[k] = wrap_index((int)fl, m.n[k]);
        wx[k][0] = 1.0f - xi;
        wx[k][1] = xi;
    }
#pragma unroll
    for (int a = 0; a < 8; ++a)
        P.W[a] = wx[0][a & 1] * wx[1][(a >> 1) & 1] * wx[2][a >> 2];
    const float bt = m.beta[p];
    const float o0 = bt * m.B[0][p], o1 = bt * m.B[1][p], o2 = bt * m.B[2][p];
    P.u[0] = 1.0f;
    P.u[1] = o0;
    P.u[2] = o1;
    P.u[3] = o2;
    P.c = m.q[p] * m.w[p] / (1.0f + (o0 * o0 + o1 * o1 + o2 * o2));
    return P;
}

__device__ inline int64_t node_index(const MassArgs &m, const int *base, int a)
{
    const int gx = wrap_index(base[0] + (a & 1), m.n[0]);
    const int gy = wrap_index(base[1] + ((a >> 1) & 1), m.n[1]);
    const int gz = wrap_index(base[2] + (a >> 2), m.n[2]);
    return gx + (int64_t)m.n[0] * (gy + (int64_t)m.n[1] * gz);
}

__device__ inline int offset_index(int a, int b)
{
    return ((b & 1) - (a & 1) + 1) + 3 * (((b >> 1) & 1) - ((a >> 1) & 1) + 1) +
           9 * ((b >> 2) - (a >> 2) + 1);
}

// Nine components of M^{ij}_{ab} from the ten moments t[k][l] (k <= l).
__device__ inline void moments_to_block(const float t[4][4], float *out)
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

// The particle's whole 8x8x9 contribution with global atomics.
__device__ inline void deposit_particle_global(const MassArgs &m, const Particle &P)
{
    float t[4][4];
    int64_t g[8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
        g[a] = node_index(m, P.base, a);
    for (int a = 0; a < 8; ++a) {
        for (int b = 0; b < 8; ++b) {
            const float wab = P.c * P.W[a] * P.W[b];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int l = k; l < 4; ++l)
                    t[k][l] = wab * P.u[k] * P.u[l];
            float blk[9];
            moments_to_block(t, blk);
            float *row = m.M + ((size_t)g[a] * 27 + offset_index(a, b)) * 9;
#pragma unroll
            for (int ij = 0; ij < 9; ++ij)
                atomic_add_f32(&row[ij], blk[ij]);
        }
    }
}

__global__ __launch_bounds__(256) void k_mass_flat(MassArgs m, int64_t begin, int64_t end)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < end; p += stride)
        deposit_particle_global(m, load_particle(m, p));
}

// LDS staging of one 64-particle batch of a cell (one wave per work-group).
struct Stage {
    float W[64][8];
    float u[64][4];  // stored as (u0, u2, u1, u3) so (u_k, u_{k+2}) are adjacent
    float c[64];
};

// Loads particle slot `p` (if it belongs to `cell`) into lane's staging row;
// particles that are not in `cell` are deposited directly and staged as zero.
__device__ inline void stage_particle(const MassArgs &m, Stage &s, int lane, int64_t p,
                                      int64_t end, const int *cell)
{
    float W[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float u[4] = {0, 0, 0, 0};
    float c = 0.0f;
    if (p < end) {
        Particle P = load_particle(m, p);
        if (P.base[0] == cell[0] && P.base[1] == cell[1] && P.base[2] == cell[2]) {
#pragma unroll
            for (int a = 0; a < 8; ++a)
                W[a] = P.W[a];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                u[k] = P.u[k];
            c = P.c;
        } else {
            deposit_particle_global(m, P);
        }
    }
#pragma unroll
    for (int a = 0; a < 8; ++a)
        s.W[lane][a] = W[a];
    s.u[lane][0] = u[0];
    s.u[lane][1] = u[2];
    s.u[lane][2] = u[1];
    s.u[lane][3] = u[3];
    s.c[lane] = c;
}

__device__ inline void cell_coords(const MassArgs &m, uint32_t cell, int *cc)
{
    cc[0] = (int)(cell % (uint32_t)m.n[0]);
    cc[1] = (int)((cell / (uint32_t)m.n[0]) % (uint32_t)m.n[1]);
    cc[2] = (int)(cell / ((uint32_t)m.n[0] * (uint32_t)m.n[1]));
}

// Adds lane (a,b)'s nine values, from moments t, to the global store.
__device__ inline void flush_pair(const MassArgs &m, const int *cc, int a, int b,
                                  const float t[4][4])
{
    float blk[9];
    moments_to_block(t, blk);
    const int64_t g = node_index(m, cc, a);
    float *row = m.M + ((size_t)g * 27 + offset_index(a, b)) * 9;
#pragma unroll
    for (int ij = 0; ij < 9; ++ij)
        atomic_add_f32(&row[ij], blk[ij]);
}

__global__ __launch_bounds__(64) void k_mass_mfma(MassArgs m)
{
    __shared__ Stage s;
    __shared__ float Tm[32][33];
    const uint32_t cell = blockIdx.x;
    const int64_t lo = std::min<int64_t>(m.cell_offsets[cell], m.n_part);
    const int64_t hi = std::min<int64_t>(m.cell_offsets[cell + 1], m.n_part);
    if (hi <= lo)
        return;
    const int lane = threadIdx.x;
    int cc[3];
    cell_coords(m, cell, cc);

    // operand coordinates of this lane: row/col index r = l % 16 of a 16-row
    // block, particle k = l / 16 of the 4-particle batch
    const int r = lane & 15, kk = lane >> 4;
    const int a = r & 7, khalf = r >> 3;  // node a, moment index k = khalf (+2)
    floatx4 acc00 = {0, 0, 0, 0}, acc01 = {0, 0, 0, 0}, acc11 = {0, 0, 0, 0};

    for (int64_t base = lo; base < hi; base += 64) {
        stage_particle(m, s, lane, base + lane, hi, cc);
        __syncthreads();
        const int nb = (int)std::min<int64_t>(64, hi - base);
        const int batches = (nb + 3) >> 2;
        for (int bt = 0; bt < batches; ++bt) {
            const int p = 4 * bt + kk;
            const float wa = s.W[p][a];
            const float2 uu = *reinterpret_cast<const float2 *>(&s.u[p][2 * khalf]);
            const float cp = s.c[p];
            const float a0 = uu.x * wa;  // u_k W_a      (k = khalf)
            const float a1 = uu.y * wa;  // u_{k+2} W_a
            const float b0 = cp * a0;
            const float b1 = cp * a1;
            acc00 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc00, 0, 0, 0);
            acc01 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc01, 0, 0, 0);
            acc11 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc11, 0, 0, 0);
        }
        __syncthreads();
    }
    // accumulator layout: lane holds D[4*(lane/16) + i][lane % 16], i = 0..3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * kk + i, col = r;
        Tm[row][col] = acc00[i];
        Tm[row][16 + col] = acc01[i];
        Tm[16 + row][16 + col] = acc11[i];
    }
    __syncthreads();
    {
        const int pa = lane >> 3, pb = lane & 7;
        float t[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int l = k; l < 4; ++l)
                t[k][l] = Tm[8 * k + pa][8 * l + pb];
        flush_pair(m, cc, pa, pb, t);
    }
}

__global__ __launch_bounds__(64) void k_mass_valu(MassArgs m)
{
    __shared__ Stage s;
    const uint32_t cell = blockIdx.x;
    const int64_t lo = std::min<int64_t>(m.cell_offsets[cell], m.n_part);
    const int64_t hi = std::min<int64_t>(m.cell_offsets[cell + 1], m.n_part);
    if (hi <= lo)
        return;
    const int lane = threadIdx.x;
    int cc[3];
    cell_coords(m, cell, cc);
    const int pa = lane >> 3, pb = lane & 7;
    float t[4][4] = {};
    for (int64_t base = lo; base < hi; base += 64) {
        stage_particle(m, s, lane, base + lane, hi, cc);
        __syncthreads();
        const int nb = (int)std::min<int64_t>(64, hi - base);
        for (int p = 0; p < nb; ++p) {
            const float wab = s.c[p] * s.W[p][pa] * s.W[p][pb];
            const float u[4] = {s.u[p][0], s.u[p][2], s.u[p][1], s.u[p][3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float wk = wab * u[k];
#pragma unroll
                for (int l = k; l < 4; ++l)
                    t[k][l] += wk * u[l];
            }
        }
        __syncthreads();
    }
    flush_pair(m, cc, pa, pb, t);
}

}  // namespace
}  // namespace pcg

using namespace pcg;

extern "C" pcg_status assemble_mass_matrix(const pcg_grid *grid, const pcg_particles *particles,
                                           const float *const B[3], const float *beta,
                                           const pcg_tile *cells, int32_t variant, float *M,
                                           void *stream)
{
    const char *who = "assemble_mass_matrix";
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
    if (variant < PCG_MASS_AUTO || variant > PCG_MASS_FLAT)
        return fail(PCG_EINVAL, "%s: unknown variant %d", who, variant);
    const int64_t count = particles->count;
    if (count < 0 || count >= (int64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^31)", who, (long long)count);
    if (count > 0) {
        for (int k = 0; k < 3; ++k)
            if (!particles->x[k] || !B || !B[k])
                return fail(PCG_EINVAL, "%s: x[%d] or B[%d] is NULL", who, k, k);
        if (!particles->q || !particles->w || !beta)
            return fail(PCG_EINVAL, "%s: q, w or beta is NULL", who);
    }
    MassArgs m{};
    for (int k = 0; k < 3; ++k) {
        m.n[k] = grid->n[k];
        m.nf[k] = (float)grid->n[k];
        m.x[k] = particles->x[k];
        m.B[k] = B ? B[k] : nullptr;
    }
    m.q = particles->q;
    m.w = particles->w;
    m.beta = beta;
    m.M = M;
    m.ncells = (uint32_t)((int64_t)grid->n[0] * grid->n[1] * grid->n[2]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (count == 0)
        return PCG_OK;
    auto flat = [&](int64_t begin, int64_t end) -> pcg_status {
        if (end <= begin)
            return PCG_OK;
        const int64_t blocks =
            std::min<int64_t>((end - begin + 255) / 256, (int64_t)device_cus() * 32);
        return launch("mass_flat", k_mass_flat, dim3((unsigned)blocks), dim3(256), 0, st, m, begin,
                      end);
    };
    if (variant == PCG_MASS_FLAT || (!cells && variant == PCG_MASS_AUTO))
        return flat(0, count);
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
    m.cell_offsets = cells->tile_offsets;
    m.n_part = cells->n_partitioned;
    if (variant == PCG_MASS_VALU)
        PCG_TRY(launch("mass_valu", k_mass_valu, dim3(m.ncells), dim3(64), 0, st, m));
    else
        PCG_TRY(launch("mass_mfma", k_mass_mfma, dim3(m.ncells), dim3(64), 0, st, m));
    return flat(cells->n_partitioned, count);
}
