// sweep.hip -- fused 1-D windowed cloud-in-cell sweep ([CS] WEANJ "03.
// Compaction and scatter-add", sections "The problem" and "Code").
//
// The page launches one kernel per step with one thread per particle.  Here all
// steps run in one launch: each thread loads its particle once and walks the
// steps, every work-group accumulates into an LDS copy of the histogram, and
// the copies are added into H with one global atomic per non-zero bin.  The
// window test and the bin index are decided in fp64 with contraction off so
// they round exactly as written.
//
// The reverse (the gradient the page takes with its autodiff call, x0 active,
// v and the set-up constant) is a gather: each thread walks its particle's
// steps as the forward kernel does, with the same fp64 decisions, and at each
// selected step reads dL/dH at the two bins the step deposited into:
//   dx0 += dw/dx ((1 - f) dH[j] + f dH[j+1]) + w nb (dH[j+1] - dH[j]),
//   dw/dx = -2 u sign(d) / hw   (the wrap and minimum image are local shifts).
// dH is copied to LDS once per work-group; there are no atomics and dx0 is
// written once per particle.
#include <algorithm>

#include "common.hpp"

namespace pcg {
namespace {

// Per-step window centre c = t / steps and shift t dt, the same for every
// particle: tabled once per work-group in LDS after the histogram (when the
// host finds room: up to STEP_TABLE_MAX steps within the CU's LDS), by the
// same fp64 operations as inline, so the same bits.  The inline division cost
// as much as the rest of a step's test.
constexpr int STEP_TABLE_MAX = 4096;
constexpr size_t SWEEP_LDS_MAX = 160 * 1024;

__device__ inline size_t align16(size_t b) { return (b + 15) & ~size_t(15); }

__device__ inline void fill_steps(double2 *tab, int steps, double dt)
{
#pragma clang fp contract(off)
    for (int t = 1 + (int)threadIdx.x; t <= steps; t += blockDim.x)
        tab[t - 1] = make_double2((double)t / (double)steps, (double)t * dt);
}

__device__ inline double2 step_consts(const double2 *tab, bool tabled, int t, int steps, double dt)
{
#pragma clang fp contract(off)
    return tabled ? tab[t - 1] : make_double2((double)t / (double)steps, (double)t * dt);
}

__global__ __launch_bounds__(256) void k_fill(float *__restrict__ H, int nb, float value)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nb; i += gridDim.x * blockDim.x)
        H[i] = value;
}

__global__ __launch_bounds__(256) void k_sweep1d(int nb, int64_t count,
                                                 const double *__restrict__ x0,
                                                 const double *__restrict__ v, int steps,
                                                 double dt, double hw, float *__restrict__ H,
                                                 int tabled)
{
#pragma clang fp contract(off)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float *hist = reinterpret_cast<float *>(smem);
    double2 *tab = reinterpret_cast<double2 *>(smem + align16((size_t)nb * sizeof(float)));
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
        hist[i] = 0.0f;
    if (tabled)
        fill_steps(tab, steps, dt);
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < count; p += stride) {
        const double xp = x0[p], vp = v[p];
        for (int t = 1; t <= steps; ++t) {
            const double2 cs = step_consts(tab, tabled, t, steps, dt);
            const double c = cs.x, shift = cs.y;
            double x = xp + vp * shift;
            x = x - floor(x);
            const double r = x - c;
            const double d = r - rint(r);
            if (fabs(d) < hw) {
                const double u = 1.0 - fabs(d) / hw;
                const double weight = u * u;
                const double g = x * (double)nb - 0.5;
                const double jf = floor(g);
                const double f = g - jf;
                const int j = (int)jf;  // in [-1, nb-1]: x is in [0, 1]
                const int j0 = wrap_index(j, nb), j1 = wrap_index(j + 1, nb);
                __hip_atomic_fetch_add(&hist[j0], (float)(weight * (1.0 - f)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(&hist[j1], (float)(weight * f), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += blockDim.x) {
        const float h = hist[i];
        if (h != 0.0f)
            atomic_add_f32(&H[i], h);
    }
}

// SEED: dL/dH is formed here from the forward histogram H and the target as
// the page's loss gives it, 2 (H - target), instead of being read from dH.
template <bool SEED>
__global__ __launch_bounds__(256) void k_sweep1d_grad(int nb, int64_t count,
                                                      const double *__restrict__ x0,
                                                      const double *__restrict__ v, int steps,
                                                      double dt, double hw,
                                                      const double *__restrict__ dH,
                                                      const float *__restrict__ H,
                                                      const double *__restrict__ target,
                                                      double *__restrict__ dx0, int tabled)
{
#pragma clang fp contract(off)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    double *dh = reinterpret_cast<double *>(smem);
    double2 *tab = reinterpret_cast<double2 *>(smem + align16((size_t)nb * sizeof(double)));
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
        dh[i] = SEED ? 2.0 * ((double)H[i] - target[i]) : dH[i];
    if (tabled)
        fill_steps(tab, steps, dt);
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < count; p += stride) {
        const double xp = x0[p], vp = v[p];
        double acc = 0.0;
        for (int t = 1; t <= steps; ++t) {
            const double2 cs = step_consts(tab, tabled, t, steps, dt);
            const double c = cs.x, shift = cs.y;
            double x = xp + vp * shift;
            x = x - floor(x);
            const double r = x - c;
            const double d = r - rint(r);
            if (fabs(d) < hw) {
                const double u = 1.0 - fabs(d) / hw;
                const double weight = u * u;
                const double sgn = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
                const double dw = -2.0 * u * sgn / hw;
                const double g = x * (double)nb - 0.5;
                const double jf = floor(g);
                const double f = g - jf;
                const int j = (int)jf;  // in [-1, nb-1]
                const double h0 = dh[wrap_index(j, nb)], h1 = dh[wrap_index(j + 1, nb)];
                acc += dw * ((1.0 - f) * h0 + f * h1) + weight * (double)nb * (h1 - h0);
            }
        }
        dx0[p] = acc;
    }
}

}  // namespace
}  // namespace pcg

using namespace pcg;

namespace {

// Dynamic LDS of a sweep kernel: the histogram (hist_bytes, at most 128 KiB)
// and, if it fits beside it, the per-step table (16 B a step); *tabled says
// whether the table is used.
size_t sweep_lds(size_t hist_bytes, int32_t steps, int *tabled)
{
    const size_t h = (hist_bytes + 15) & ~size_t(15);
    const size_t with = h + (size_t)steps * sizeof(double2);
    *tabled = steps <= STEP_TABLE_MAX && with <= SWEEP_LDS_MAX;
    return *tabled ? with : h;
}

}  // namespace

extern "C" pcg_status deposit_sweep1d(int32_t nb, int64_t count, const double *x0,
                                      const double *v, int32_t steps, double dt,
                                      double half_width, float *H, void *stream)
{
    const char *who = "deposit_sweep1d";
    clear_error();
    if (nb < 1 || nb > 16384)
        return fail(PCG_EINVAL, "%s: nb = %d outside [1, 16384]", who, nb);
    if (count < 0 || count >= (int64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^31)", who, (long long)count);
    if (steps < 0)
        return fail(PCG_EINVAL, "%s: steps %d < 0", who, steps);
    if (!(half_width > 0.0) || !(dt == dt))
        return fail(PCG_EINVAL, "%s: half_width must be > 0 and dt finite", who);
    if (!H || (count > 0 && (!x0 || !v)))
        return fail(PCG_EINVAL, "%s: NULL array", who);
    hipStream_t st = static_cast<hipStream_t>(stream);
    PCG_TRY(launch("sweep_fill", k_fill, dim3((nb + 255) / 256), dim3(256), 0, st, H, (int)nb,
                   0.0f));
    if (count == 0 || steps == 0)
        return PCG_OK;
    int tabled = 0;
    const size_t lds = sweep_lds((size_t)nb * sizeof(float), steps, &tabled);
    if (hipFuncSetAttribute((const void *)k_sweep1d, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
        return fail(PCG_EHIP, "%s: cannot raise dynamic LDS to %zu bytes", who, lds);
    const int64_t blocks = std::min<int64_t>((count + 255) / 256, (int64_t)device_cus() * 8);
    return launch("sweep1d", k_sweep1d, dim3((unsigned)blocks), dim3(256), lds, st, (int)nb,
                  count, x0, v, (int)steps, dt, half_width, H, tabled);
}

namespace {

// Argument checks shared by the sweep entry points.
pcg_status check_sweep(const char *who, int32_t nb, int64_t count, int32_t steps, double dt,
                       double half_width)
{
    if (nb < 1 || nb > 16384)
        return fail(PCG_EINVAL, "%s: nb = %d outside [1, 16384]", who, nb);
    if (count < 0 || count >= (int64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^31)", who, (long long)count);
    if (steps < 0)
        return fail(PCG_EINVAL, "%s: steps %d < 0", who, steps);
    if (!(half_width > 0.0) || !(dt == dt))
        return fail(PCG_EINVAL, "%s: half_width must be > 0 and dt finite", who);
    return PCG_OK;
}

template <bool SEED>
pcg_status launch_grad(const char *who, int32_t nb, int64_t count, const double *x0,
                       const double *v, int32_t steps, double dt, double half_width,
                       const double *dH, const float *H, const double *target, double *dx0,
                       hipStream_t st)
{
    int tabled = 0;
    const size_t lds = sweep_lds((size_t)nb * sizeof(double), steps, &tabled);
    if (hipFuncSetAttribute((const void *)k_sweep1d_grad<SEED>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return fail(PCG_EHIP, "%s: cannot raise dynamic LDS to %zu bytes", who, lds);
    const int64_t blocks = std::min<int64_t>((count + 255) / 256, (int64_t)device_cus() * 8);
    return launch("sweep1d_grad", k_sweep1d_grad<SEED>, dim3((unsigned)blocks), dim3(256), lds,
                  st, (int)nb, count, x0, v, (int)steps, dt, half_width, dH, H, target, dx0,
                  tabled);
}

}  // namespace

extern "C" pcg_status deposit_sweep1d_grad(int32_t nb, int64_t count, const double *x0,
                                           const double *v, int32_t steps, double dt,
                                           double half_width, const double *dH, double *dx0,
                                           void *stream)
{
    const char *who = "deposit_sweep1d_grad";
    clear_error();
    PCG_TRY(check_sweep(who, nb, count, steps, dt, half_width));
    if (count > 0 && (!x0 || !v || !dH || !dx0))
        return fail(PCG_EINVAL, "%s: NULL array", who);
    if (count == 0)
        return PCG_OK;
    return launch_grad<false>(who, nb, count, x0, v, steps, dt, half_width, dH, nullptr, nullptr,
                              dx0, static_cast<hipStream_t>(stream));
}

extern "C" pcg_status deposit_sweep1d_loss_grad(int32_t nb, int64_t count, const double *x0,
                                                const double *v, int32_t steps, double dt,
                                                double half_width, const double *target,
                                                float *H, double *dx0, void *stream)
{
    const char *who = "deposit_sweep1d_loss_grad";
    clear_error();
    PCG_TRY(check_sweep(who, nb, count, steps, dt, half_width));
    if (!H || !target || (count > 0 && (!x0 || !v || !dx0)))
        return fail(PCG_EINVAL, "%s: NULL array", who);
    PCG_TRY(deposit_sweep1d(nb, count, x0, v, steps, dt, half_width, H, stream));
    if (count == 0)
        return PCG_OK;
    return launch_grad<true>(who, nb, count, x0, v, steps, dt, half_width, nullptr, H, target,
                             dx0, static_cast<hipStream_t>(stream));
}
