/*
 * pcg.h -- C ABI of the particle-to-grid scatter-deposition library for AMD
 * Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array pointer is a DEVICE pointer owned by the caller; the
 *   library never allocates, frees or retains device memory.  Struct arguments
 *   and the small pointer arrays that carry device pointers are host memory,
 *   read during the call only.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Every call only enqueues work on that stream and returns; results
 *   are ready once the stream is synchronised.  Calls on different streams that
 *   write the same output race.
 * Layouts.  Particles are structure-of-arrays fp32.  Grids are periodic and
 *   node-centred with unit spacing: node g sits at integer coordinate g and
 *   cell g spans [g, g+1), so positions are in cell units with
 *   0 <= x_k < n_k.  Grid arrays are x-fastest (linear node
 *   g = gx + n_x*(gy + n_y*gz)).  Unused axes of a 1-D or 2-D grid have n_k = 1.
 * Accumulation.  deposit_currents(_zigzag) and assemble_mass_matrix ADD into their
 *   output (the caller zeroes it); the 1-D sweep entry points OVERWRITE their
 *   outputs.
 * Errors.  Every entry point returns a pcg_status.  Arguments are validated on
 *   the host before anything is enqueued; on failure nothing is launched and
 *   pcg_last_error() gives a message (per host thread).  A launch failure
 *   reported by the HIP runtime returns PCG_EHIP.  Positions outside [0, n_k)
 *   or non-finite break the precondition: the kernels clamp and wrap every
 *   index so such input cannot make them access memory out of bounds, but the
 *   values they deposit are then unspecified.
 *
 * Sources cited below:
 *   [TD] Entity wiki, "Tiled current deposit".
 *   [MM] Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
 *        Particle-In-Cell Methods" (arXiv:2604.19286).
 *   [CS] WEANJ examples, "03. Compaction and scatter-add".
 */
#ifndef PCG_H
#define PCG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pcg_status;
#define PCG_OK 0
#define PCG_EINVAL (-1)        /* bad argument (null pointer, size, range)      */
#define PCG_EUNSUPPORTED (-2)  /* valid but not built (dim/order/variant combo) */
#define PCG_ELDS (-3)          /* scratch tile does not fit the 160 KiB LDS     */
#define PCG_EWORKSPACE (-4)    /* workspace missing or too small                */
#define PCG_EHIP (-6)          /* the HIP runtime reported a launch error       */

/* Periodic grid: dim in {1,2,3}; n[k] nodes (= cells) per axis, n[k] = 1 for
 * k >= dim. */
typedef struct pcg_grid {
    int32_t dim;
    int32_t n[3];
} pcg_grid;

/* Particles, SoA fp32 device arrays of `count` entries: count < 2^31 for
 * pcg_tile_sort, count < 2^30 for deposit_currents, deposit_currents_regroup and
 * assemble_mass_matrix (they address the arrays with 32-bit byte offsets).
 * x[k] is used for k < dim (others may be NULL); v[0..2] are always the three
 * velocity components (unused by assemble_mass_matrix, may be NULL there). */
typedef struct pcg_particles {
    int64_t count;
    const float *x[3];
    const float *v[3];
    const float *q;
    const float *w;
} pcg_particles;

/* A tile layout ([TD] "How a tile deposit runs", "The tile-based spatial
 * sort"), as written by pcg_tile_sort.  Tile t owns the particle slice
 * [tile_offsets[t], tile_offsets[t+1]); particles [n_partitioned, count) are an
 * unsorted tail handled by the flat kernel ([TD] "Coverage: the tail pass").
 *   T          tile edge in nodes on every used axis (1 = a cell layout).
 *   order      shape order the layout was keyed with (1 CIC, 2 TSC).
 *   drift      halo budget D >= 0 in cells ([TD] "Halo sizing"): the scratch
 *              tile spans TE = T + order + 2*D nodes per used axis.
 *   block      work-group size; 0 = automatic (512), otherwise clamped to
 *              [64, 512] and rounded down to a multiple of 64 ([TD] team size
 *              knob).
 *   tile_offsets  device uint32 [ntiles + 1], ntiles = prod_k (n_k / T). */
typedef struct pcg_tile {
    int32_t T;
    int32_t order;
    int32_t drift;
    int32_t block;
    int64_t n_partitioned;
    const uint32_t *tile_offsets;
} pcg_tile;

/* ------------------------------------------------------------------------ */
/* Tile sort  ([TD] "The tile-based spatial sort")                           */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace pcg_tile_sort needs for `count` particles.  Returns
 * 0 if the arguments are invalid. */
size_t pcg_sort_workspace_bytes(const pcg_grid *grid, int64_t count, int32_t T);

/* Stable tile sort.
 * Key: the tile (edge T nodes per used axis, n_k % T == 0) holding each
 *   particle's first support node -- the cell's lower node for order 1, and for
 *   order 2 the node below it when the fractional coordinate is < 1/2 ([MM]
 *   §2.3) -- wrapped periodically; key = t_x + nt_x*(t_y + nt_y*t_z).  With
 *   T = 1 the key is the cell index (a cell sort, [MM] §3.1).
 * Output: perm[j] (device uint32 [count], or NULL when not wanted) is the
 *   input index of the particle
 *   placed in slot j: ascending key, ties in ascending input index (stable, so
 *   the result is unique).  sorted_keys (device uint32 [count], or NULL) gets
 *   the keys in slot order.  tile_offsets (device uint32 [ntiles+1]) gets
 *   tile_offsets[t] = number of particles with key < t.
 *   out_arrays[i][j] = in_arrays[i][perm[j]] for i < n_arrays (0..16 fp32
 *   device arrays of `count` entries; out-of-place, out != in).  The keys are
 *   computed from key_x[k], k < dim.
 * prev: optional; the layout the input is currently grouped by (the previous
 *   sort's output, T and order equal to this call's, device offsets distinct
 *   from tile_offsets).  When it covers all particles, the sort runs as a
 *   single-pass counting sort over the 27 neighbouring tiles of each particle's
 *   previous tile -- the every-step case of [TD] "Halo sizing", where particles
 *   move at most one cell between sorts.  If the offsets are not a partition of
 *   [0, count) or any particle moved further, the general radix path runs
 *   instead, decided on the device (the call stays asynchronous).  The output
 *   is identical either way.
 * workspace: device memory of at least pcg_sort_workspace_bytes(), 256-byte
 *   aligned, contents undefined on entry and exit. */
pcg_status pcg_tile_sort(const pcg_grid *grid, int32_t order, int32_t T, int64_t count,
                         const float *const key_x[3], int32_t n_arrays,
                         const float *const in_arrays[], float *const out_arrays[],
                         uint32_t *perm, uint32_t *sorted_keys, uint32_t *tile_offsets,
                         const pcg_tile *prev, void *workspace, size_t workspace_bytes,
                         void *stream);

/* ------------------------------------------------------------------------ */
/* Current deposit  ([TD]; [MM] §2.3 Eq.(12) shape functions)                */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace deposit_currents needs for this layout (tile may
 * be NULL: then 0). */
size_t pcg_deposit_workspace_bytes(const pcg_grid *grid, const pcg_tile *tile);

/* J_c(g) += q_p w_p v_{p,c} W(x_p - x_g) for every particle p, every node g of
 * its order-`order` B-spline support (CIC = 1: 2^dim nodes, TSC = 2: 3^dim
 * nodes) and c = x, y, z; node indices wrap periodically.
 * J: device fp32 [3][n_z][n_y][n_x], accumulated.
 * tile: the layout from pcg_tile_sort keyed with the same order (tile->order
 *   must equal order), or NULL.  With a layout, one work-group per tile (heavy
 *   tiles split into chunks) accumulates into an LDS scratch tile of
 *   TE = T + order + 2*drift nodes per used axis and flushes it once with
 *   global atomics; a particle whose stencil does not fit the window takes the
 *   escape valve to global atomics ([TD] "Correctness is independent of the
 *   halo").  The scratch holds int64 fixed-point sums scaled per work-group
 *   (exact, order-independent in-tile accumulation of the fp32 products); a
 *   particle whose |q w v| lies far outside its work-group's scale also takes
 *   the valve but is not counted in n_escaped.  When the int64 scratch
 *   (3*TE^dim*8 bytes) exceeds the LDS, fp32 scratch is used instead.  The tail [n_partitioned, count) and the tile == NULL case use the
 *   flat one-thread-per-particle global-atomic kernel ([TD] "Coverage").
 *   Requires n_k % T == 0 and drift + order < n_k on used axes, and
 *   3*TE^dim*4 bytes <= 160 KiB (else PCG_ELDS).
 * n_escaped: optional device uint64 counter; the number of escaped particles
 *   is ADDED to it.  workspace: pcg_deposit_workspace_bytes() bytes (may be
 *   NULL when that is 0). */
pcg_status deposit_currents(const pcg_grid *grid, const pcg_particles *particles, int32_t order,
                            const pcg_tile *tile, float *J, unsigned long long *n_escaped,
                            void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and results as deposit_currents, with no workspace
 * argument.  The work-item map deposit_currents keeps in its workspace lives
 * in a static device array of PCG_NOALLOC_SCRATCH_BYTES bytes instead (each
 * GPU the library runs on holds one until the process ends; looked up once
 * per device).  A layout whose map needs more (pcg_deposit_workspace_bytes()
 * above the maximum; it takes about 20 bytes per tile and 16 per 2048
 * partitioned particles, so 4096 tiles and 67M particles need 0.6 MB) returns
 * PCG_EWORKSPACE before anything is enqueued.  Every call on one GPU shares
 * that GPU's array, so calls that overlap on one GPU (different streams or
 * host threads) race; calls in one stream order are safe.  The array holds no
 * state from one call to the next that a call relies on. */
#define PCG_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
pcg_status deposit_currents_noalloc(const pcg_grid *grid, const pcg_particles *particles,
                                    int32_t order, const pcg_tile *tile, float *J,
                                    unsigned long long *n_escaped, void *stream);

/* Bytes of device workspace deposit_currents_regroup needs (0 if invalid). */
size_t pcg_deposit_regroup_workspace_bytes(const pcg_grid *grid, const pcg_tile *tile,
                                           int64_t count);

/* One pass of a step over the particle data ([TD] "How a tile deposit runs"
 * followed by "The tile-based spatial sort", the sort at the end of a step):
 * the same results as
 *     deposit_currents(grid, particles, order, tile, J, n_escaped, ...);
 *     pcg_tile_sort(grid, order, tile->T, particles->count, particles->x,
 *                   n_arrays, in_arrays, out_arrays, NULL, NULL,
 *                   tile_offsets, tile, ...);
 * (J and n_escaped accumulated as there; out_arrays and tile_offsets equal to
 * the sort's, bit for bit), but when `tile` covers every particle
 * (n_partitioned == count) and in_arrays are exactly x[0..dim), v[0..3), q, w
 * of `particles`, in that order, the sort's move is made by the deposit
 * kernel from the values it has loaded, so the particle arrays are read once
 * instead of twice.  `tile` is the layout the particles are grouped by
 * (required); the sort uses it as `prev`, so particles that moved further
 * than one tile, or a layout that is not a partition, send the regrouping to
 * the general sort path (decided on the device; the deposit is unaffected).
 * With a tail, or with any other list of arrays, the two calls run one after
 * the other.  in_arrays / out_arrays as in pcg_tile_sort (out of place).  The
 * sort's argument checks run before anything is enqueued.  tile_offsets: device uint32 [ntiles + 1], the new
 * layout, distinct from tile->tile_offsets.  workspace: at least
 * pcg_deposit_regroup_workspace_bytes(), 256-byte aligned. */
pcg_status deposit_currents_regroup(const pcg_grid *grid, const pcg_particles *particles,
                                    int32_t order, const pcg_tile *tile, float *J,
                                    unsigned long long *n_escaped, int32_t n_arrays,
                                    const float *const in_arrays[], float *const out_arrays[],
                                    uint32_t *tile_offsets, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* The charge-conserving zigzag current deposit ([TD] "Halo sizing", which
 * names it as writing up to two cells above min(i, i_prev)).  Each particle p
 * moves from x_prev to x, less than one cell per axis (x_prev unwrapped:
 * x_prev_k - x_k in (-1, 1); x in [0, n_k)).  The move is split at the relay
 * point xr_k = min(min(i1_k, i2_k) + 1, max(max(i1_k, i2_k), (x_prev_k + x_k)/2))
 * (i1 = floor(x_prev), i2 = floor(x)) into two segments that each stay in one
 * cell; each segment deposits the exact current of a straight path inside its
 * cell: with F = q w (end - start), F' = end - start and W = midpoint - cell,
 *   J_c(cell + d1 e_k1 + d2 e_k2) += F_c [w(d1, W_k1) w(d2, W_k2) +/- F'_k1 F'_k2 / 12]
 * (k1 < k2 the other axes, w(0, W) = 1 - W, w(1, W) = W, + when d1 = d2),
 * 24 contributions per particle.  J_c[g] is the current through the face at
 * g + e_c/2, so that rho(x) - rho(x_prev) + sum_c (J_c[g] - J_c[g - e_c]) = 0
 * at every node, rho the CIC charge density.  3-D grids only.
 * J: device fp32 [3][n_z][n_y][n_x], accumulated.  x_prev: host array of 3
 *   device fp32 pointers [count].
 * tile: a layout from pcg_tile_sort with order 1 keyed on x (the new
 *   positions) or on the previous ones, or NULL.  With a layout, one
 *   work-group per tile accumulates into an LDS window of TE = T + 2*drift + 3
 *   nodes per axis starting drift + 1 nodes below the tile origin ([TD] "How a
 *   tile deposit runs") and adds it to J with one atomic per non-zero node.
 *   The window holds exact int64 fixed-point sums, scaled per tile from its
 *   largest |q w| so that every add fits an int32 and no sum can overflow (a
 *   tile is deposited a second time if its first estimate proves low), or
 *   fp32 sums when 3*TE^3*8 bytes exceed the LDS.  A particle whose stencil does
 *   not fit (its layout is more than `drift` cells stale, or it crossed more
 *   than one cell boundary on an axis) takes the escape valve to global
 *   atomics and is counted.  The tail [n_partitioned, count) and tile == NULL
 *   use the flat one-thread-per-particle kernel.  Requires n_k % T == 0 and
 *   3*TE^3*4 bytes <= 160 KiB (else PCG_ELDS).
 * n_escaped: optional device uint64 counter, ADDED to.
 * Errors: PCG_EUNSUPPORTED for dim != 3; PCG_EINVAL for a NULL array with
 *   count > 0, a count outside [0, 2^31) or a bad layout. */
pcg_status deposit_currents_zigzag(const pcg_grid *grid, const pcg_particles *particles,
                                   const float *const x_prev[3], const pcg_tile *tile, float *J,
                                   unsigned long long *n_escaped, void *stream);

/* The zigzag deposit and the next sort in one pass over the particle data
 * ([TD] "How a tile deposit runs" followed by "The tile-based spatial sort",
 * the sort at the end of a step): the same results as
 *     deposit_currents_zigzag(grid, particles, x_prev, tile, J, n_escaped, ...);
 *     pcg_tile_sort(grid, 1, tile->T, particles->count, particles->x,
 *                   n_arrays, in_arrays, out_arrays, NULL, NULL,
 *                   tile_offsets, tile, ...);
 * (J and n_escaped accumulated as there; out_arrays and tile_offsets equal to
 * the sort's, bit for bit).  When `tile` covers every particle, in_arrays are
 * exactly x[0..3), x_prev[0..3), q, w of the deposit, in that order, and the
 * window holds int64 sums, the deposit kernel makes the sort's move from the
 * values it has loaded (one work-group per tile, its waves walking the sort's
 * chunks in order), so the particle arrays are read once instead of twice.
 * `tile` is the layout the particles are grouped by (required); the sort uses
 * it as `prev`, and a particle that moved further than one tile, or a layout
 * that is not a partition, sends the regrouping to the general sort path
 * (decided on the device; the deposit is unaffected).  Otherwise the two
 * calls run one after the other.  in_arrays / out_arrays as in pcg_tile_sort
 * (out of place); tile_offsets: device uint32 [ntiles + 1], the new layout,
 * distinct from tile->tile_offsets.  workspace: at least
 * pcg_sort_workspace_bytes(grid, count, tile->T) bytes, 256-byte aligned.
 * Errors: as for the two calls; every check runs before anything is
 * enqueued. */
pcg_status deposit_currents_zigzag_regroup(const pcg_grid *grid, const pcg_particles *particles,
                                           const float *const x_prev[3], const pcg_tile *tile,
                                           float *J, unsigned long long *n_escaped,
                                           int32_t n_arrays, const float *const in_arrays[],
                                           float *const out_arrays[], uint32_t *tile_offsets,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream);

/* ------------------------------------------------------------------------ */
/* ECSIM mass matrix  ([MM] §2.1 Eq.(4)-(6), §2.2 Eq.(9)-(11), §3)           */
/* ------------------------------------------------------------------------ */

#define PCG_MASS_AUTO 0   /* the matrix-core path                                  */
#define PCG_MASS_MFMA 1   /* per-cell contraction on fp32 MFMA (16x16x4)           */
#define PCG_MASS_VALU 2   /* the same per-cell contraction with vector FMAs         */
#define PCG_MASS_FLAT 3   /* one thread per particle, 576 global atomics each      */
/* OR'ed into a variant of any assemble_mass_matrix* call: M is set to the
 * matrix instead of added to.  With a layout (MFMA, VALU) the CIC column
 * kernels then store each row of M without reading it; the other paths clear
 * M first.  The tail and stray particles still add after the rows are set. */
#define PCG_MASS_OVERWRITE 16

/* Bytes of device workspace assemble_mass_matrix needs with a cell layout
 * (MFMA and VALU variants). */
size_t pcg_mass_workspace_bytes(const pcg_grid *grid);

/* M^{ij}_{g, g+o} += q_p w_p alpha_p^{ij} W_{pg} W_{p,g+o} over every ordered
 * pair of the 8 CIC support nodes of every particle, with
 * alpha_p = (I - C(omega) + omega omega^T) / (1 + |omega|^2), C(omega)u = omega x u,
 * omega = beta_p B_p ([MM] Eq.(5), c = 1; the prefactor of Eq.(4) is 1).
 * 3-D, CIC, every n_k >= 3.
 * M: device fp32 [n_z][n_y][n_x][27][3][3], accumulated; row g, stencil offset
 *   o = (dx+1) + 3(dy+1) + 9(dz+1) for the node g + (dx,dy,dz) (wrapped).
 * B[3], beta: device fp32 per-particle magnetic field and beta = q dt / (2m).
 * cells: a T = 1, order = 1 layout from pcg_tile_sort (cell c owns its slice;
 *   [MM] §3.1 assumes particles sorted by cell), or NULL (flat path).  With a
 *   layout, the per-cell contractions ([MM] §3.2, Eq.(14)-(20)) are summed
 *   into each row of M by the work-group that owns the row, and every row is
 *   read and written once (no atomics).  A particle found in the slice of a
 *   cell it is not in is deposited by the flat path after that; the tail
 *   [n_partitioned, count) likewise.  Calls that write the same M on
 *   different streams race.
 * variant: PCG_MASS_*, optionally OR'ed with PCG_MASS_OVERWRITE; VALU and
 *   MFMA need `cells`.
 * workspace: device memory of at least pcg_mass_workspace_bytes() bytes,
 *   256-byte aligned, needed when `cells` is given (may be NULL otherwise);
 *   contents undefined on entry and exit. */
pcg_status assemble_mass_matrix(const pcg_grid *grid, const pcg_particles *particles,
                                const float *const B[3], const float *beta,
                                const pcg_tile *cells, int32_t variant, float *M,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Scalar mass matrix ([MM] §2.1: Eq.(6) with the scalar coefficient
 * s_p = q_p w_p in place of the tensor q_p w_p alpha_p, one value per node pair,
 * the form a mass matrix takes in MPM):
 *   M_{g, g+o} += q_p w_p W_{pg} W_{p,g+o}
 * over every ordered pair of the 8 CIC support nodes of every particle.
 * 3-D, CIC, every n_k >= 3; no field is read.
 * M: device fp32 [n_z][n_y][n_x][27], accumulated; offsets numbered as for
 *   assemble_mass_matrix.
 * cells, variant, workspace, stream: as for assemble_mass_matrix, with the same
 *   column assembly (each row of M read and written once), stray and tail
 *   handling, and the same workspace size (pcg_mass_workspace_bytes()).
 *   PCG_MASS_MFMA takes eight particles per 16x16x4 fp32 product.
 * Errors: as for assemble_mass_matrix (B and beta are not taken). */
pcg_status assemble_mass_matrix_scalar(const pcg_grid *grid, const pcg_particles *particles,
                                       const pcg_tile *cells, int32_t variant, float *M,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Scalar mass matrix with TSC weights ([MM] §2.1 Eq.(6) scalar case, §2.3
 * Eq.(12) at order 2; the paper's TSC runs, §4.1 Fig. 8):
 *   M_{g, g+o} += q_p w_p W_{pg} W_{p,g+o}
 * over every ordered pair of the 27 TSC support nodes of every particle.
 * 3-D, every n_k >= 5.
 * M: device fp32 [n_z][n_y][n_x][125], accumulated; o = (dx+2) + 5(dy+2) +
 *   25(dz+2) for the node g + (dx,dy,dz) (wrapped).
 * groups: a T = 1, order = 2 layout from pcg_tile_sort (group = the particles
 *   sharing one TSC support base, [MM] §3.3), or NULL (flat path).  With it,
 *   each group's 27 x 27 block is one product over its particles on the matrix
 *   cores (PCG_MASS_MFMA) or vector FMAs (PCG_MASS_VALU).  MFMA sums the blocks
 *   of 4 x 4 x 2 groups in LDS (32-bit fixed point, its unit set by the
 *   brick's sum of |q w|: q w must be finite) and adds the brick's node pairs
 *   to M once with device atomics; VALU adds every block with device atomics
 *   ([MM] §3.4).  A particle in a slice whose group it is not in, and the tail
 *   [n_partitioned, count), take the flat path (729 atomics each).
 * No workspace.  Calls that write the same M on different streams race.
 * Errors: PCG_EINVAL for n_k < 5, a NULL array, a count outside [0, 2^30), a
 *   layout that is not T = 1, order = 2, or MFMA/VALU without a layout;
 *   PCG_EUNSUPPORTED for dim != 3. */
pcg_status assemble_mass_matrix_scalar_tsc(const pcg_grid *grid, const pcg_particles *particles,
                                           const pcg_tile *groups, int32_t variant, float *M,
                                           void *stream);

/* The ECSIM (tensor) mass matrix with TSC weights ([MM] Eq.(4)-(6) with §2.3
 * Eq.(12) at order 2; the paper's tensorial TSC runs, §4.1 Fig. 9):
 *   M^{ij}_{g, g+o} += q_p w_p alpha_p^{ij} W_{pg} W_{p,g+o},
 * alpha_p as for assemble_mass_matrix, over every ordered pair of the 27 TSC
 * support nodes.  3-D, every n_k >= 5.
 * M: device fp32 [n_z][n_y][n_x][125][3][3], accumulated; offsets as for
 *   assemble_mass_matrix_scalar_tsc.
 * B[3], beta: as for assemble_mass_matrix.  groups, variant, strays, tail and
 *   errors: as for assemble_mass_matrix_scalar_tsc.  MFMA forms the nine
 *   component blocks (27 x 27 each) per group and sums those of 2 x 2 x 2
 *   groups in LDS (32-bit fixed point as above: q w, B and beta must be
 *   finite) before adding them to M; VALU forms the ten moment matrices of the
 *   CIC kernels per group and adds the 9-component block with 6561 device
 *   atomics ([MM] §3.4).  No workspace. */
pcg_status assemble_mass_matrix_tsc(const pcg_grid *grid, const pcg_particles *particles,
                                    const float *const B[3], const float *beta,
                                    const pcg_tile *groups, int32_t variant, float *M,
                                    void *stream);

/* fp64 variants of the two matrices ([MM] §4 and §4.1, Figs. 6-7: the CIC
 * scalar and tensor assemblies are measured with every operand in FP64; §5
 * "Tile-support matching and portability" names AMD's FP64 16x16x4 product):
 * the same operation and arguments as
 * assemble_mass_matrix and assemble_mass_matrix_scalar, with M in fp64 and
 * every product and sum formed in fp64 (the inputs stay fp32).
 * PCG_MASS_MFMA contracts on v_mfma_f64_16x16x4f64.
 * M: device fp64, layout as for the fp32 entry points, accumulated.
 * Errors: as for the fp32 entry points. */
pcg_status assemble_mass_matrix_f64(const pcg_grid *grid, const pcg_particles *particles,
                                    const float *const B[3], const float *beta,
                                    const pcg_tile *cells, int32_t variant, double *M,
                                    void *workspace, size_t workspace_bytes, void *stream);
pcg_status assemble_mass_matrix_scalar_f64(const pcg_grid *grid, const pcg_particles *particles,
                                           const pcg_tile *cells, int32_t variant, double *M,
                                           void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* 1-D windowed sweep  ([CS] "The problem", "Code")                          */
/* ------------------------------------------------------------------------ */

/* H is overwritten with the fused result of `steps` windowed CIC deposits on
 * the periodic interval [0,1) split into nb bins (1 <= nb <= 16384): for
 * t = 1..steps, x = x0 + v (t dt) wrapped as x - floor(x), window centre
 * c = t/steps, minimum-image d = (x-c) - rint(x-c); if |d| < half_width the
 * particle deposits weight (1 - |d|/half_width)^2 split linearly between bins
 * floor(x nb - 1/2) and the next one (mod nb).  Positions and weights are
 * computed in fp64 without fused multiply-adds; H is fp32 [nb].
 * x0, v: device fp64 [count]. */
pcg_status deposit_sweep1d(int32_t nb, int64_t count, const double *x0, const double *v,
                           int32_t steps, double dt, double half_width, float *H, void *stream);

/* The reverse of deposit_sweep1d ([CS] "Code": the gradient the page takes of
 * its loss sum (H - target)^2 with respect to x0, with v and the set-up held
 * constant).  Given dH = dL/dH (fp64 [nb]; the page's loss gives
 * 2 (H - target)), dx0[p] is OVERWRITTEN with dL/dx0[p]: for every step at
 * which the particle is selected (the same fp64 decisions as the forward call),
 *   dx0 += dw/dx ((1 - f) dH[j] + f dH[j+1]) + w nb (dH[j+1] - dH[j])
 * with w = (1 - |d|/half_width)^2, dw/dx = -2 (1 - |d|/half_width) sign(d) /
 * half_width (sign(0) = 0), f and j the forward split and bin (mod nb).
 * x0, v, dx0: device fp64 [count]; dH: device fp64 [nb].
 * Errors: PCG_EINVAL as for deposit_sweep1d, or a NULL array with count > 0. */
pcg_status deposit_sweep1d_grad(int32_t nb, int64_t count, const double *x0, const double *v,
                                int32_t steps, double dt, double half_width, const double *dH,
                                double *dx0, void *stream);

/* The page's whole gradient call ([CS] "Code", deposit_gradient): the forward
 * sweep into H, the seed dL/dH = 2 (H - target) of its loss sum (H - target)^2,
 * and the reverse above, enqueued as one call.  H: device fp32 [nb], OVERWRITTEN
 * with the forward histogram (the seed is formed from these fp32 values);
 * target: device fp64 [nb]; dx0: device fp64 [count], OVERWRITTEN.
 * Errors: as for deposit_sweep1d_grad; H and target may not be NULL. */
pcg_status deposit_sweep1d_loss_grad(int32_t nb, int64_t count, const double *x0,
                                     const double *v, int32_t steps, double dt,
                                     double half_width, const double *target, float *H,
                                     double *dx0, void *stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics and measurement                                               */
/* ------------------------------------------------------------------------ */

const char *pcg_status_string(pcg_status status);
/* Message of the last failed call on this host thread ("" if none). */
const char *pcg_last_error(void);
/* Library version string. */
const char *pcg_version(void);

/* Kernel timing tap, for measurement.  While enabled, every kernel launch is
 * bracketed by a pair of HIP events recorded on its launch stream.
 * pcg_timing_read synchronises the recorded events of the named kernel (e.g.
 * "deposit_tiled") and returns their summed elapsed time in ms and the number
 * of launches since the last reset.  pcg_timing_names writes a comma-separated
 * list of the kernel names seen into buf (truncated to len). */
pcg_status pcg_timing_enable(int32_t enable);
pcg_status pcg_timing_reset(void);
pcg_status pcg_timing_read(const char *kernel, double *total_ms, int64_t *launches);
pcg_status pcg_timing_names(char *buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* PCG_H */
