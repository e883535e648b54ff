/*
 * oracle.c -- plain, slow, fp64 CPU reference for particle-to-grid scatter
 * deposition.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Its only users are the tests, the smoke check of the
 * graft entry module, and the cpu_baseline leg of bench.py.  It shares no code,
 * header, table or constant with the HIP library; both sides see only the same
 * seeded input arrays.
 *
 * Every routine is the plain definition of what the method computes, written
 * out as single-threaded loops in particle-index order, in double precision.
 * Particle inputs are the same fp32 arrays the GPU reads, widened exactly to
 * double, so integer decisions (cells, support bases, tiles, escapes) are made
 * on identical values.
 *
 * Sources (cited by page title and section/equation):
 *   [MM]  Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for
 *         Implicit Particle-In-Cell Methods" (arXiv:2604.19286).
 *   [TD]  Entity wiki, "Tiled current deposit".
 *   [CS]  WEANJ examples, "03. Compaction and scatter-add".
 *
 * Conventions (readings of the pages, stated once):
 *   - 2D/3D grids are periodic and node-centred with unit spacing: node g sits
 *     at integer coordinate g, cell g spans [g, g+1); positions are in cell
 *     units with 0 <= x_k < n_k.
 *   - Arrays are x-fastest: J[c][z][y][x], M[z][y][x][27][3][3].
 *   - The current deposit is direct: J_c(g) += q*w*v_c*W_g(x), all three
 *     components collocated on the nodes.
 *   - Status: 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* B-spline shape functions                                                  */
/* ------------------------------------------------------------------------ */

/* [MM] §2.3 Eq.(12): phi^(n) is the order-n B-spline, compactly supported on
 * [-(n+1)/2, (n+1)/2].  n = 1 is the cloud-in-cell hat, n = 2 the
 * triangular-shaped-cloud quadratic spline.  The argument s is the signed
 * particle-to-node distance in units of the grid spacing. */
static double phi(int order, double s)
{
    double a = fabs(s);
    if (order == 1)
        return a < 1.0 ? 1.0 - a : 0.0;
    /* order 2 */
    if (a <= 0.5)
        return 0.75 - a * a;
    if (a < 1.5)
        return 0.5 * (1.5 - a) * (1.5 - a);
    return 0.0;
}

/* [MM] §2.3: the lowest support node along one axis, before periodic wrap.
 * CIC: the lower corner j of the cell holding the particle.  TSC: the stencil
 * is centred on the nearest node, so a fractional coordinate below 1/2 uses
 * {j-1, j, j+1} and one at or above 1/2 uses {j, j+1, j+2}. */
static int64_t support_base(int order, double x)
{
    double j = floor(x);
    if (order == 2 && (x - j) < 0.5)
        return (int64_t)j - 1;
    return (int64_t)j;
}

static int64_t wrap(int64_t i, int64_t n)
{
    int64_t r = i % n;
    return r < 0 ? r + n : r;
}

/* One axis of the shape function: the (unwrapped) first support node and the
 * order+1 weights phi(x - node).  Returns the number of support nodes. */
int oracle_shape_1d(int order, double x, int64_t *base, double *weights)
{
    if (order != 1 && order != 2)
        return -1;
    int64_t b = support_base(order, x);
    for (int a = 0; a <= order; ++a)
        weights[a] = phi(order, x - (double)(b + a));
    *base = b;
    return order + 1;
}

static int check_grid(int dim, const int32_t n[3])
{
    if (dim < 1 || dim > 3)
        return -1;
    for (int k = 0; k < 3; ++k) {
        if (n[k] < 1)
            return -1;
        if (k >= dim && n[k] != 1)
            return -1;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Current deposit                                                           */
/* ------------------------------------------------------------------------ */

/* J_c(g) += q_p * w_p * v_{p,c} * W(x_p - x_g) for every particle p, every
 * node g of its support and every component c, with W the tensor product of
 * the 1-D splines ([MM] §2.3 Eq.(12)); node indices wrap periodically.  The
 * tiled and flat deposits of [TD] ("One deposit body, two launchers") both
 * reduce to this sum.  J is fp64 [3][n_z][n_y][n_x] and is accumulated. */
int oracle_deposit(int dim, const int32_t n[3], int order, int64_t np,
                   const float *const x[3], const float *const v[3],
                   const float *q, const float *w, double *J)
{
    if (check_grid(dim, n) || (order != 1 && order != 2) || np < 0)
        return -1;
    const int64_t ng = (int64_t)n[0] * n[1] * n[2];
    for (int64_t p = 0; p < np; ++p) {
        int64_t base[3] = {0, 0, 0};
        double W[3][3] = {{1.0, 0, 0}, {1.0, 0, 0}, {1.0, 0, 0}};
        int m[3] = {1, 1, 1};
        for (int k = 0; k < dim; ++k) {
            m[k] = oracle_shape_1d(order, (double)x[k][p], &base[k], W[k]);
        }
        double qw = (double)q[p] * (double)w[p];
        for (int az = 0; az < m[2]; ++az)
            for (int ay = 0; ay < m[1]; ++ay)
                for (int ax = 0; ax < m[0]; ++ax) {
                    int64_t gx = wrap(base[0] + ax, n[0]);
                    int64_t gy = wrap(base[1] + ay, n[1]);
                    int64_t gz = wrap(base[2] + az, n[2]);
                    int64_t g = gx + (int64_t)n[0] * (gy + (int64_t)n[1] * gz);
                    double wt = W[0][ax] * W[1][ay] * W[2][az];
                    for (int c = 0; c < 3; ++c)
                        J[c * ng + g] += qw * (double)v[c][p] * wt;
                }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Tile keys, stable sort, tile offsets                                      */
/* ------------------------------------------------------------------------ */

/* [TD] "The tile-based spatial sort": the domain is cut into tiles of T nodes
 * per used axis and a particle is keyed by the tile holding the first node its
 * deposit touches -- here the (wrapped) support base node.  The key is the
 * tile's linear index t_x + nt_x*(t_y + nt_y*t_z), nt_k = n_k / T. */
int oracle_tile_keys(int dim, const int32_t n[3], int order, int T, int64_t np,
                     const float *const x[3], uint32_t *key)
{
    if (check_grid(dim, n) || (order != 1 && order != 2) || T < 1 || np < 0)
        return -1;
    int64_t nt[3] = {1, 1, 1};
    for (int k = 0; k < dim; ++k) {
        if (n[k] % T)
            return -1;
        nt[k] = n[k] / T;
    }
    for (int64_t p = 0; p < np; ++p) {
        int64_t t[3] = {0, 0, 0};
        for (int k = 0; k < dim; ++k)
            t[k] = wrap(support_base(order, (double)x[k][p]), n[k]) / T;
        key[p] = (uint32_t)(t[0] + nt[0] * (t[1] + nt[1] * t[2]));
    }
    return 0;
}

/* Stable counting sort ([TD] "Sort" and "Offsets"): perm lists particle
 * indices in ascending key order, equal keys in ascending index order, and
 * offsets[t] = number of particles whose key is below t, for t = 0..nkeys, so
 * tile t owns the slice [offsets[t], offsets[t+1]). */
int oracle_stable_sort(int64_t np, const uint32_t *key, uint32_t nkeys,
                       uint32_t *perm, uint32_t *offsets)
{
    if (np < 0 || nkeys < 1)
        return -1;
    int64_t *count = (int64_t *)calloc((size_t)nkeys + 1, sizeof(int64_t));
    if (!count)
        return -1;
    for (int64_t p = 0; p < np; ++p) {
        if (key[p] >= nkeys) {
            free(count);
            return -1;
        }
        count[key[p] + 1] += 1;
    }
    for (uint32_t t = 0; t < nkeys; ++t)
        count[t + 1] += count[t];
    for (uint32_t t = 0; t <= nkeys; ++t)
        offsets[t] = (uint32_t)count[t];
    for (int64_t p = 0; p < np; ++p)
        perm[count[key[p]]++] = (uint32_t)p;
    free(count);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Escape valve classification                                               */
/* ------------------------------------------------------------------------ */

/* [TD] "How a tile deposit runs", "Halo sizing" and "Correctness is
 * independent of the halo": the team of tile t holds a scratch window of
 * TE = T + order + 2*D nodes per used axis, starting D nodes below the tile
 * origin (periodically wrapped).  A particle in tile t's slice deposits into
 * scratch only if, on every used axis, its whole run of order+1 support nodes
 * lies inside that window; otherwise it escapes and deposits straight to the
 * global array.  This routine decides "fits" by enumerating the window
 * placements, and writes escaped[j] for each layout slot j < n_part (slots of
 * the unpartitioned tail are marked 0: they are not tiled).  Returns the
 * escape count, or -1 on bad arguments. */
int64_t oracle_escape(int dim, const int32_t n[3], int order, int T, int D,
                      int64_t np, const float *const x[3],
                      const uint32_t *tile_offsets, int64_t n_part,
                      uint8_t *escaped)
{
    if (check_grid(dim, n) || (order != 1 && order != 2) || T < 1 || D < 0 ||
        np < 0 || n_part < 0 || n_part > np)
        return -1;
    int64_t nt[3] = {1, 1, 1};
    for (int k = 0; k < dim; ++k) {
        if (n[k] % T)
            return -1;
        nt[k] = n[k] / T;
    }
    const int64_t ntiles = nt[0] * nt[1] * nt[2];
    const int64_t TE = T + order + 2 * D;
    memset(escaped, 0, (size_t)np);
    int64_t count = 0;
    for (int64_t t = 0; t < ntiles; ++t) {
        int64_t tc[3] = {t % nt[0], (t / nt[0]) % nt[1], t / (nt[0] * nt[1])};
        int64_t lo = tile_offsets[t], hi = tile_offsets[t + 1];
        if (hi > n_part)
            hi = n_part;
        for (int64_t j = lo; j < hi; ++j) {
            int fits = 1;
            for (int k = 0; k < dim && fits; ++k) {
                int64_t origin = tc[k] * T;
                int64_t b = support_base(order, (double)x[k][j]);
                int found = 0;
                /* the first support node may sit at window position s0 only
                 * if the whole run s0..s0+order is inside [0, TE) */
                for (int64_t s0 = 0; s0 + order < TE && !found; ++s0)
                    if (wrap(origin - D + s0 - b, n[k]) == 0)
                        found = 1;
                fits = found;
            }
            if (!fits) {
                escaped[j] = 1;
                ++count;
            }
        }
    }
    return count;
}

/* ------------------------------------------------------------------------ */
/* ECSIM rotation-response tensor and mass matrix                            */
/* ------------------------------------------------------------------------ */

/* [MM] §2.1 Eq.(5): alpha = (I - C(omega) + omega omega^T) / (1 + |omega|^2),
 * where C(omega) u = omega x u.  C is built column by column from the cross
 * product with the unit vectors.  alpha is row-major [i][j]. */
void oracle_alpha(const double omega[3], double alpha[9])
{
    double C[3][3];
    for (int j = 0; j < 3; ++j) {
        double e[3] = {0.0, 0.0, 0.0};
        e[j] = 1.0;
        double c[3] = {omega[1] * e[2] - omega[2] * e[1],
                       omega[2] * e[0] - omega[0] * e[2],
                       omega[0] * e[1] - omega[1] * e[0]};
        for (int i = 0; i < 3; ++i)
            C[i][j] = c[i];
    }
    double den = 1.0 + omega[0] * omega[0] + omega[1] * omega[1] +
                 omega[2] * omega[2];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            alpha[i * 3 + j] =
                ((i == j ? 1.0 : 0.0) - C[i][j] + omega[i] * omega[j]) / den;
}

/* [MM] §2.1 Eq.(4)/(6) with the prefactor sigma = 1 (c = 1, V_g = 1), and
 * omega_p = beta_p * B_p ([MM] Eq.(5), B already at the particle):
 *   M^{ij}_{g g'} += q_p w_p alpha_p^{ij} W_{pg} W_{pg'}
 * over every ordered pair (g, g') of the particle's 8 CIC support nodes.  The
 * sparse store follows [MM] §3.4: row g, column g' = g + o with the stencil
 * offset o = (dx, dy, dz) in {-1,0,1}^3 taken between the two support nodes
 * (before wrapping), stored at index (dx+1) + 3(dy+1) + 9(dz+1).
 * M is fp64 [n_z][n_y][n_x][27][3][3] and is accumulated.  3D, CIC only;
 * every n_k must be >= 3 so the 27 offsets name distinct nodes. */
int oracle_mass_matrix(const int32_t n[3], int64_t np, const float *const x[3],
                       const float *const B[3], const float *q, const float *w,
                       const float *beta, double *M)
{
    if (n[0] < 3 || n[1] < 3 || n[2] < 3 || np < 0)
        return -1;
    for (int64_t p = 0; p < np; ++p) {
        double omega[3], alpha[9], s[9];
        for (int k = 0; k < 3; ++k)
            omega[k] = (double)beta[p] * (double)B[k][p];
        oracle_alpha(omega, alpha);
        double qw = (double)q[p] * (double)w[p];
        for (int ij = 0; ij < 9; ++ij)
            s[ij] = qw * alpha[ij];
        int64_t base[3];
        double W[3][2];
        for (int k = 0; k < 3; ++k)
            oracle_shape_1d(1, (double)x[k][p], &base[k], W[k]);
        for (int a = 0; a < 8; ++a) {
            int ax = a & 1, ay = (a >> 1) & 1, az = a >> 2;
            int64_t ga = wrap(base[0] + ax, n[0]) +
                         (int64_t)n[0] * (wrap(base[1] + ay, n[1]) +
                                          (int64_t)n[1] * wrap(base[2] + az, n[2]));
            double wa = W[0][ax] * W[1][ay] * W[2][az];
            for (int b = 0; b < 8; ++b) {
                int bx = b & 1, by = (b >> 1) & 1, bz = b >> 2;
                double wb = W[0][bx] * W[1][by] * W[2][bz];
                int o = (bx - ax + 1) + 3 * (by - ay + 1) + 9 * (bz - az + 1);
                double wab = wa * wb;
                double *row = M + (ga * 27 + o) * 9;
                for (int ij = 0; ij < 9; ++ij)
                    row[ij] += s[ij] * wab;
            }
        }
    }
    return 0;
}

/* [MM] §2.1, the scalar case of Eq.(6): the per-particle coefficient is
 * q_p w_p times the identity, so a node pair carries one component
 * (the mass matrix of MPM), with sigma = 1:
 *   M_{g g'} += q_p w_p W_{pg} W_{pg'}
 * over every ordered pair (g, g') of the particle's 8 CIC support nodes, in
 * the same 27-offset store as oracle_mass_matrix: M is fp64
 * [n_z][n_y][n_x][27] and is accumulated.  3D, CIC only; n_k >= 3. */
int oracle_mass_matrix_scalar(const int32_t n[3], int64_t np, const float *const x[3],
                              const float *q, const float *w, double *M)
{
    if (n[0] < 3 || n[1] < 3 || n[2] < 3 || np < 0)
        return -1;
    for (int64_t p = 0; p < np; ++p) {
        const double s = (double)q[p] * (double)w[p];
        int64_t base[3];
        double W[3][2];
        for (int k = 0; k < 3; ++k)
            oracle_shape_1d(1, (double)x[k][p], &base[k], W[k]);
        for (int az = 0; az < 2; ++az)
            for (int ay = 0; ay < 2; ++ay)
                for (int ax = 0; ax < 2; ++ax) {
                    const int64_t g = wrap(base[0] + ax, n[0]) +
                                      (int64_t)n[0] * (wrap(base[1] + ay, n[1]) +
                                                       (int64_t)n[1] * wrap(base[2] + az, n[2]));
                    const double wg = W[0][ax] * W[1][ay] * W[2][az];
                    for (int bz = 0; bz < 2; ++bz)
                        for (int by = 0; by < 2; ++by)
                            for (int bx = 0; bx < 2; ++bx) {
                                const double wh = W[0][bx] * W[1][by] * W[2][bz];
                                const int o = (bx - ax + 1) + 3 * (by - ay + 1) + 9 * (bz - az + 1);
                                M[g * 27 + o] += s * wg * wh;
                            }
                }
    }
    return 0;
}

/* [MM] §2.1 Eq.(6), scalar case, with TSC shape functions ([MM] §2.3 Eq.(12),
 * order 2; the paper's TSC experiments, §4.1 Fig. 8): every ordered pair of
 * the 27 support nodes of every particle,
 *   M_{g, g+o} += q_p w_p W_{pg} W_{p,g+o},
 * into a 125-offset store: M is fp64 [n_z][n_y][n_x][125] with
 * o = (dx+2) + 5 (dy+2) + 25 (dz+2) for the node g + (dx,dy,dz), and is
 * accumulated.  3D; n_k >= 5 (the 125 offsets are then distinct nodes). */
int oracle_mass_matrix_scalar_tsc(const int32_t n[3], int64_t np, const float *const x[3],
                                  const float *q, const float *w, double *M)
{
    if (n[0] < 5 || n[1] < 5 || n[2] < 5 || np < 0)
        return -1;
    for (int64_t p = 0; p < np; ++p) {
        const double s = (double)q[p] * (double)w[p];
        int64_t base[3];
        double W[3][3];
        for (int k = 0; k < 3; ++k)
            oracle_shape_1d(2, (double)x[k][p], &base[k], W[k]);
        for (int az = 0; az < 3; ++az)
            for (int ay = 0; ay < 3; ++ay)
                for (int ax = 0; ax < 3; ++ax) {
                    const int64_t g = wrap(base[0] + ax, n[0]) +
                                      (int64_t)n[0] * (wrap(base[1] + ay, n[1]) +
                                                       (int64_t)n[1] * wrap(base[2] + az, n[2]));
                    const double wg = W[0][ax] * W[1][ay] * W[2][az];
                    for (int bz = 0; bz < 3; ++bz)
                        for (int by = 0; by < 3; ++by)
                            for (int bx = 0; bx < 3; ++bx) {
                                const double wh = W[0][bx] * W[1][by] * W[2][bz];
                                const int o = (bx - ax + 2) + 5 * (by - ay + 2) + 25 * (bz - az + 2);
                                M[g * 125 + o] += s * wg * wh;
                            }
                }
    }
    return 0;
}

/* [MM] §2.1 Eq.(4)-(6) with TSC shape functions (§2.3 Eq.(12) at order 2; the
 * paper's tensorial TSC runs, §4.1 Fig. 9): every ordered pair of the 27
 * support nodes of every particle,
 *   M^{ij}_{g, g+o} += q_p w_p alpha_p^{ij} W_{pg} W_{p,g+o},
 * alpha_p from oracle_alpha.  M is fp64 [n_z][n_y][n_x][125][3][3] with the
 * 125 offsets numbered as in oracle_mass_matrix_scalar_tsc, and is
 * accumulated.  3D; n_k >= 5. */
int oracle_mass_matrix_tsc(const int32_t n[3], int64_t np, const float *const x[3],
                           const float *const B[3], const float *q, const float *w,
                           const float *beta, double *M)
{
    if (n[0] < 5 || n[1] < 5 || n[2] < 5 || np < 0)
        return -1;
    for (int64_t p = 0; p < np; ++p) {
        double omega[3], alpha[9], s[9];
        for (int k = 0; k < 3; ++k)
            omega[k] = (double)beta[p] * (double)B[k][p];
        oracle_alpha(omega, alpha);
        double qw = (double)q[p] * (double)w[p];
        for (int ij = 0; ij < 9; ++ij)
            s[ij] = qw * alpha[ij];
        int64_t base[3];
        double W[3][3];
        for (int k = 0; k < 3; ++k)
            oracle_shape_1d(2, (double)x[k][p], &base[k], W[k]);
        for (int a = 0; a < 27; ++a) {
            int ax = a % 3, ay = (a / 3) % 3, az = a / 9;
            int64_t ga = wrap(base[0] + ax, n[0]) +
                         (int64_t)n[0] * (wrap(base[1] + ay, n[1]) +
                                          (int64_t)n[1] * wrap(base[2] + az, n[2]));
            double wa = W[0][ax] * W[1][ay] * W[2][az];
            for (int b = 0; b < 27; ++b) {
                int bx = b % 3, by = (b / 3) % 3, bz = b / 9;
                double wb = W[0][bx] * W[1][by] * W[2][bz];
                int o = (bx - ax + 2) + 5 * (by - ay + 2) + 25 * (bz - az + 2);
                double *row = M + (ga * 125 + o) * 9;
                for (int ij = 0; ij < 9; ++ij)
                    row[ij] += s[ij] * (wa * wb);
            }
        }
    }
    return 0;
}

/* [TD] "Halo sizing": the charge-conserving zigzag deposit (shape order 0 in
 * Entity's numbering), which writes up to two cells above min(i, i_prev).  The
 * page names the scheme without its formulas; the reading taken: a move from
 * xp to x (less than one cell per axis) is split at the relay point
 *   xr_k = min(min(i1_k, i2_k) + 1, max(max(i1_k, i2_k), (xp_k + x_k) / 2))
 * (i1 = floor(xp), i2 = floor(x)) into two segments that each stay in one
 * cell, and each segment deposits the exact current of a straight path inside
 * its cell: with F = q w (end - start) and W = midpoint - cell per axis,
 *   J_c(cell + d1 e_k1 + d2 e_k2) += F_c [w(d1, W_k1) w(d2, W_k2) +/- F'_k1 F'_k2 / 12]
 * (k1, k2 the other two axes, w(0, W) = 1 - W, w(1, W) = W, + when d1 = d2,
 * F' = end - start).  J_c[g] sits at g + e_c / 2 (staggered), so that
 *   rho(x) - rho(xp) + sum_c (J_c[g] - J_c[g - e_c]) = 0
 * with rho the CIC charge density at the nodes.  J is fp64 [3][n_z][n_y][n_x]
 * and is accumulated; xp is the unwrapped previous position. */
int oracle_deposit_zigzag(const int32_t n[3], int64_t np, const float *const x[3],
                          const float *const xp[3], const float *q, const float *w, double *J)
{
    if (n[0] < 1 || n[1] < 1 || n[2] < 1 || np < 0)
        return -1;
    const int64_t ng = (int64_t)n[0] * n[1] * n[2];
    for (int64_t p = 0; p < np; ++p) {
        const double qw = (double)q[p] * (double)w[p];
        double a[3], b[3], xr[3];
        int64_t i1[3], i2[3];
        for (int k = 0; k < 3; ++k) {
            a[k] = (double)xp[k][p];
            b[k] = (double)x[k][p];
            i1[k] = (int64_t)floor(a[k]);
            i2[k] = (int64_t)floor(b[k]);
            double lo = (double)(i1[k] < i2[k] ? i1[k] : i2[k]) + 1.0;
            double hi = (double)(i1[k] > i2[k] ? i1[k] : i2[k]);
            xr[k] = fmin(lo, fmax(hi, 0.5 * (a[k] + b[k])));
        }
        for (int s = 0; s < 2; ++s) {
            const double *st = s == 0 ? a : xr, *en = s == 0 ? xr : b;
            const int64_t *cell = s == 0 ? i1 : i2;
            double F[3], W[3];
            for (int k = 0; k < 3; ++k) {
                F[k] = en[k] - st[k];
                W[k] = 0.5 * (st[k] + en[k]) - (double)cell[k];
            }
            for (int c = 0; c < 3; ++c) {
                const int k1 = c == 0 ? 1 : 0, k2 = c == 2 ? 1 : 2;
                for (int d2 = 0; d2 < 2; ++d2)
                    for (int d1 = 0; d1 < 2; ++d1) {
                        const double w1 = d1 ? W[k1] : 1.0 - W[k1];
                        const double w2 = d2 ? W[k2] : 1.0 - W[k2];
                        const double cross = F[k1] * F[k2] / 12.0;
                        const double wt = w1 * w2 + (d1 == d2 ? cross : -cross);
                        int64_t g[3] = {cell[0], cell[1], cell[2]};
                        g[k1] += d1;
                        g[k2] += d2;
                        const int64_t idx = wrap(g[0], n[0]) +
                                            (int64_t)n[0] * (wrap(g[1], n[1]) +
                                                             (int64_t)n[1] * wrap(g[2], n[2]));
                        J[c * ng + idx] += qw * F[c] * wt;
                    }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 1-D windowed sweep deposit                                                */
/* ------------------------------------------------------------------------ */

/* [CS] "The problem" and "Code" (deposit_loss, deposit_step!, deposit!):
 * H is zeroed, then for t = 1..T with window centre c = t/T:
 *   x  = x0 + v*(t*dt), wrapped into [0,1) as x - floor(x);
 *   d  = (x - c) - rint(x - c)           (minimum-image distance);
 *   if |d| < hw:  weight = (1 - |d|/hw)^2,
 *                 g = x*nb - 1/2, j = floor(g), f = g - j,
 *                 H[j mod nb] += weight*(1-f), H[(j+1) mod nb] += weight*f.
 * The distance is measured from the wrapped position, as the GPU kernel on the
 * page does.  All arithmetic is fp64; H is fp64 [nb] and is overwritten. */
int oracle_sweep1d(int nb, int64_t np, const double *x0, const double *v,
                   int T, double dt, double hw, double *H)
{
    if (nb < 1 || np < 0 || T < 0 || !(hw > 0.0))
        return -1;
    for (int b = 0; b < nb; ++b)
        H[b] = 0.0;
    for (int t = 1; t <= T; ++t) {
        double c = (double)t / (double)T;
        double shift = (double)t * dt;
        for (int64_t p = 0; p < np; ++p) {
            double x = x0[p] + v[p] * shift;
            x = x - floor(x);
            double r = x - c;
            double d = r - rint(r);
            if (fabs(d) < hw) {
                double u = 1.0 - fabs(d) / hw;
                double weight = u * u;
                double g = x * (double)nb - 0.5;
                double jf = floor(g);
                double f = g - jf;
                int64_t j = (int64_t)jf;
                H[wrap(j, nb)] += weight * (1.0 - f);
                H[wrap(j + 1, nb)] += weight * f;
            }
        }
    }
    return 0;
}

/* [CS] "Code": the reverse of the sweep above, as the page's autodiff call
 * computes it: x0 active, v and the set-up constant.  dH holds dL/dH (the page
 * seeds it with 2 (H - target)); dx0[p] is overwritten with dL/dx0[p].  For a
 * selected particle at step t (same x, d, u, w, g, j, f as the forward pass):
 *   dx/dx0 = 1 and dd/dx = 1 (the wrap and the minimum image are locally
 *   shifts); dw/dx = -2 u sign(d) / hw; df/dx = nb;
 *   the deposits w (1 - f) into j and w f into j + 1 give
 *   dx0 += dw/dx ((1 - f) dH[j] + f dH[j+1]) + w nb (dH[j+1] - dH[j]).
 * sign(0) is taken as 0 (the derivative of |d| at 0). */
int oracle_sweep1d_grad(int nb, int64_t np, const double *x0, const double *v,
                        int T, double dt, double hw, const double *dH, double *dx0)
{
    if (nb < 1 || np < 0 || T < 0 || !(hw > 0.0))
        return -1;
    for (int64_t p = 0; p < np; ++p)
        dx0[p] = 0.0;
    for (int t = 1; t <= T; ++t) {
        double c = (double)t / (double)T;
        double shift = (double)t * dt;
        for (int64_t p = 0; p < np; ++p) {
            double x = x0[p] + v[p] * shift;
            x = x - floor(x);
            double r = x - c;
            double d = r - rint(r);
            if (fabs(d) < hw) {
                double u = 1.0 - fabs(d) / hw;
                double weight = u * u;
                double sgn = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
                double dw = -2.0 * u * sgn / hw;
                double g = x * (double)nb - 0.5;
                double jf = floor(g);
                double f = g - jf;
                int64_t j = (int64_t)jf;
                double h0 = dH[wrap(j, nb)], h1 = dH[wrap(j + 1, nb)];
                dx0[p] += dw * ((1.0 - f) * h0 + f * h1) + weight * (double)nb * (h1 - h0);
            }
        }
    }
    return 0;
}
