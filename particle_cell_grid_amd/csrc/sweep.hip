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
// Compaction inside the wave (what the page lists as not done on its GPU
// side): about 1% of particle-steps fall in the window, yet with one lane per
// particle about half of all wave-steps hold at least one such lane, and the
// whole wave would run the deposit for it.  Instead each step only tests; the
// lanes in the window append (x, d, lane) to the wave's LDS queue (ballot and
// rank), and the queue is deposited 64 items at a time, one per lane.
//
// The reverse (the gradient the page takes with its autodiff call, x0 active,
// v and the set-up constant) walks the same steps with the same fp64
// decisions and queue, and for each queued item reads dL/dH at the two bins
// the step deposited into:
//   dx0 += dw/dx ((1 - f) dH[j] + f dH[j+1]) + w nb (dH[j+1] - dH[j]),
//   dw/dx = -2 u sign(d) / hw   (the wrap and minimum image are local shifts).
// dH is copied to LDS once per work-group.  An item's term is added (LDS fp64
// add) to its particle's slot, and each particle's dx0 is written once.
#include <algorithm>

#include "common.hpp"

namespace pcg {
namespace {

// Per-step window centre c = t / steps and shift t dt, the same for every
// particle: tabled once per work-group in LDS after the histogram (when the
// host finds room: up to STEP_TABLE_MAX steps within the CU's LDS beside the
// static queues), by the same fp64 operations as inline, so the same bits.  The
// inline division cost as much as the rest of a step's test.
constexpr int STEP_TABLE_MAX = 4096;
constexpr size_t SWEEP_LDS_MAX = 152 * 1024;
constexpr int SWEEP_WAVES = 256 / WAVE;

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

// One wave's queue of selected (particle, step) items, and (reverse) the
// per-lane sums of the current particles.
struct SweepQueue {
    double x[WAVE];   // wrapped position
    double d[WAVE];   // minimum-image distance to the window centre
    int owner[WAVE];  // lane whose particle it is
    double acc[WAVE];
};

// Orders this wave's earlier LDS accesses before its later ones.
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The step's window test for one particle (fp64, no contraction): wrapped x
// and minimum-image d; true if |d| < hw.
__device__ inline bool window_test(double xp, double vp, double2 cs, double hw, double &x,
                                   double &d)
{
#pragma clang fp contract(off)
    x = xp + vp * cs.y;
    x = x - floor(x);
    const double r = x - cs.x;
    d = r - rint(r);
    return fabs(d) < hw;
}

// Bins of an item: j = floor(x nb - 1/2) in [-1, nb - 1] (x in [0, 1]) and the
// next one, wrapped; f the share of the second.
__device__ inline void item_bins(double x, int nb, int &j0, int &j1, double &f)
{
#pragma clang fp contract(off)
    const double g = x * (double)nb - 0.5;
    const double jf = floor(g);
    f = g - jf;
    const int j = (int)jf;
    j0 = j < 0 ? j + nb : j;
    j1 = j + 1 >= nb ? j + 1 - nb : j + 1;
}

// Appends the wave's selected lanes (mask) to the queue at qn (uniform), after
// handling what is queued if the new items would not fit.
template <typename Handle>
__device__ inline void enqueue(SweepQueue &q, int &qn, uint64_t mask, bool sel, double x,
                               double d, int lane, Handle &&handle)
{
    const int n = __popcll(mask);
    if (qn + n > WAVE) {
        handle(qn);
        qn = 0;
    }
    if (sel) {
        const int k = qn + (int)__builtin_amdgcn_mbcnt_hi(
                               (uint32_t)(mask >> 32),
                               __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        q.x[k] = x;
        q.d[k] = d;
        q.owner[k] = lane;
    }
    qn += n;
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
    __shared__ SweepQueue queues[SWEEP_WAVES];
    float *hist = reinterpret_cast<float *>(smem);
    double2 *tab = reinterpret_cast<double2 *>(smem + align16((size_t)nb * sizeof(float)));
    const int lane = lane_id(), wave = (int)(threadIdx.x / WAVE);
    SweepQueue &q = queues[wave];
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
        hist[i] = 0.0f;
    if (tabled)
        fill_steps(tab, steps, dt);
    __syncthreads();
    // deposits the first n queued items, one per lane
    auto handle = [&](int n) {
        wave_lds_sync();
        if (lane < n) {
            const double x = q.x[lane], d = q.d[lane];
            const double u = 1.0 - fabs(d) / hw;
            const double weight = u * u;
            int j0, j1;
            double f;
            item_bins(x, nb, j0, j1, f);
            __hip_atomic_fetch_add(&hist[j0], (float)(weight * (1.0 - f)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(&hist[j1], (float)(weight * f), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        wave_lds_sync();
    };
    int qn = 0;
    // the wave walks its particles together (the queue needs every lane):
    // lanes past the end test a clamped particle and never select it
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x + wave * WAVE; base < count;
         base += stride) {
        const int64_t p = base + lane;
        const bool live = p < count;
        const int64_t pc = live ? p : count - 1;
        const double xp = x0[pc], vp = v[pc];
        for (int t = 1; t <= steps; ++t) {
            double x, d;
            const bool sel = window_test(xp, vp, step_consts(tab, tabled, t, steps, dt), hw, x,
                                         d) && live;
            const uint64_t mask = __ballot(sel);
            if (mask)
                enqueue(q, qn, mask, sel, x, d, lane, handle);
        }
    }
    if (qn)
        handle(qn);
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
    __shared__ SweepQueue queues[SWEEP_WAVES];
    double *dh = reinterpret_cast<double *>(smem);
    double2 *tab = reinterpret_cast<double2 *>(smem + align16((size_t)nb * sizeof(double)));
    const int lane = lane_id(), wave = (int)(threadIdx.x / WAVE);
    SweepQueue &q = queues[wave];
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
        dh[i] = SEED ? 2.0 * ((double)H[i] - target[i]) : dH[i];
    if (tabled)
        fill_steps(tab, steps, dt);
    __syncthreads();
    // adds the terms of the first n queued items to their particles' sums
    auto handle = [&](int n) {
        wave_lds_sync();
        if (lane < n) {
            const double x = q.x[lane], d = q.d[lane];
            const double u = 1.0 - fabs(d) / hw;
            const double weight = u * u;
            const double sgn = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
            const double dw = -2.0 * u * sgn / hw;
            int j0, j1;
            double f;
            item_bins(x, nb, j0, j1, f);
            const double h0 = dh[j0], h1 = dh[j1];
            __hip_atomic_fetch_add(&q.acc[q.owner[lane]],
                                   dw * ((1.0 - f) * h0 + f * h1) + weight * (double)nb * (h1 - h0),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        wave_lds_sync();
    };
    int qn = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x + wave * WAVE; base < count;
         base += stride) {
        const int64_t p = base + lane;
        const bool live = p < count;
        const int64_t pc = live ? p : count - 1;
        const double xp = x0[pc], vp = v[pc];
        q.acc[lane] = 0.0;
        for (int t = 1; t <= steps; ++t) {
            double x, d;
            const bool sel = window_test(xp, vp, step_consts(tab, tabled, t, steps, dt), hw, x,
                                         d) && live;
            const uint64_t mask = __ballot(sel);
            if (mask)
                enqueue(q, qn, mask, sel, x, d, lane, handle);
        }
        // the queue refers to these particles: drain it before moving on
        if (qn) {
            handle(qn);
            qn = 0;
        }
        wave_lds_sync();
        if (live)
            dx0[p] = q.acc[lane];
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
