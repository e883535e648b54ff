// sweep.hip -- fused 1-D windowed cloud-in-cell sweep ([CS] WEANJ "03.
// Compaction and scatter-add", sections "The problem" and "Code").
//
// The page launches one kernel per step with one thread per particle.  Here all
// steps run in one launch: each thread loads its particle once and walks the
// steps, every work-group accumulates into an LDS copy of the histogram, and
// the copies are added into H with one global atomic per non-zero bin.  The
// window test and the bin index are decided in fp64 with contraction off so
// they round exactly as written.
#include <algorithm>

#include "common.hpp"

namespace pcg {
namespace {

__global__ __launch_bounds__(256) void k_fill(float *__restrict__ H, int nb, float value)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nb; i += gridDim.x * blockDim.x)
        H[i] = value;
}

__global__ __launch_bounds__(256) void k_sweep1d(int nb, int64_t count,
                                                 const double *__restrict__ x0,
                                                 const double *__restrict__ v, int steps,
                                                 double dt, double hw, float *__restrict__ H)
{
#pragma clang fp contract(off)
    extern __shared__ float hist[];
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
        hist[i] = 0.0f;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < count; p += stride) {
        const double xp = x0[p], vp = v[p];
        for (int t = 1; t <= steps; ++t) {
            const double c = (double)t / (double)steps;
            const double shift = (double)t * dt;
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

}  // namespace
}  // namespace pcg

using namespace pcg;

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
    const int64_t blocks = std::min<int64_t>((count + 255) / 256, (int64_t)device_cus() * 8);
    return launch("sweep1d", k_sweep1d, dim3((unsigned)blocks), dim3(256),
                  (size_t)nb * sizeof(float), st, (int)nb, count, x0, v, (int)steps, dt,
                  half_width, H);
}
