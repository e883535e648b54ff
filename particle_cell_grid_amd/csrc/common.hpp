// common.hpp -- internal helpers shared by the library's HIP sources: status
// handling, the launch wrapper (with the optional event-timing tap), and small
// device utilities for wave64 and periodic indexing.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "pcg.h"

namespace pcg {

// ---------------------------------------------------------------- host side

// Records a formatted message as this thread's last error and returns status.
pcg_status fail(pcg_status status, const char *fmt, ...);
void clear_error();

// Timing tap: when enabled, brackets launches with events on their stream.
bool timing_on();
void timing_before(const char *name, hipStream_t stream);
void timing_after(const char *name, hipStream_t stream);

// Launch `kernel` and check the runtime's launch status.
template <typename Kernel, typename... Args>
pcg_status launch(const char *name, Kernel kernel, dim3 grid, dim3 block, size_t lds,
                  hipStream_t stream, Args... args)
{
    if (grid.x == 0 || grid.y == 0 || grid.z == 0)
        return PCG_OK;
    const bool tap = timing_on();
    if (tap)
        timing_before(name, stream);
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
    hipError_t e = hipGetLastError();
    if (tap)
        timing_after(name, stream);
    if (e != hipSuccess)
        return fail(PCG_EHIP, "%s: launch failed: %s", name, hipGetErrorString(e));
    return PCG_OK;
}

#define PCG_TRY(expr)                    \
    do {                                 \
        pcg_status _s = (expr);          \
        if (_s != PCG_OK)                \
            return _s;                   \
    } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Carves 256-byte aligned sub-buffers out of a caller workspace.
struct Carver {
    char *base;
    size_t used = 0;
    explicit Carver(void *p) : base(static_cast<char *>(p)) {}
    template <typename T>
    T *take(size_t n)
    {
        T *p = reinterpret_cast<T *>(base ? base + used : nullptr);
        used = align_up(used + n * sizeof(T), 256);
        return p;
    }
};

// Validates a grid; used axes n_k >= 1, unused axes exactly 1.
pcg_status check_grid(const pcg_grid *grid, const char *who);

// Number of compute units of the current device (cached).
int device_cus();

// ---------------------------------------------------------------- device side

constexpr int WAVE = 64;

__device__ inline int lane_id() { return __lane_id(); }

// Mask of lanes below this one.
__device__ inline uint64_t lanemask_lt() { return (uint64_t(1) << lane_id()) - 1; }

// x mod n for any int (n > 0), cheap when x is already within one period.
__device__ inline int wrap_index(int x, int n)
{
    if (x >= 0 && x < n)
        return x;
    if (x < 0 && x >= -n)
        return x + n;
    if (x >= n && x < 2 * n)
        return x - n;
    int r = x % n;
    return r < 0 ? r + n : r;
}

// a * b + c for a, b, c >= 0 and a, b < 2^24 (an index within a tile's
// window): a 24-bit multiply issues at the full rate, a 32-bit one (or the
// 64-bit multiply-add the compiler may pick) at a quarter of it.
__device__ inline int mad24(int a, int b, int c)
{
    return (int)(__umul24((unsigned)a, (unsigned)b) + (unsigned)c);
}

// Clamp a coordinate into [0, n] (NaN -> 0) so a broken precondition can never
// produce an out-of-range index; exact for valid input.
__device__ inline float clamp_coord(float x, float n) { return fminf(fmaxf(x, 0.0f), n); }

// Relaxed device-scope float add with no return value (global_atomic_add_f32).
__device__ inline void atomic_add_f32(float *p, float v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The chip's work-groups are dealt to its 8 XCDs (each with its own L2) in
// turn: block b runs on XCD b % 8.  xcd_item(b, run) gives each XCD runs of
// `run` consecutive work items instead of every 8th one, so that items next to
// each other in a layout (neighbouring tiles, whose windows overlap in J) run
// on one XCD at about the same time.  A bijection of the naturals: a grid
// rounded up by xcd_grid covers every item below it exactly once.  run = 0:
// the plain order.
constexpr uint32_t NXCD = 8;

__device__ inline uint32_t xcd_item(uint32_t b, uint32_t run)
{
    if (run == 0)
        return b;
    const uint32_t j = b % NXCD, k = b / NXCD;
    return (k / run) * (NXCD * run) + j * run + k % run;
}

inline uint32_t xcd_grid(uint32_t items, uint32_t run)
{
    return run ? (uint32_t)align_up(items, (size_t)NXCD * run) : items;
}

// One entry of a chunk map (a work item of a tile layout): the chunk's tile
// and particle range [lo, hi).
struct alignas(16) ChunkEntry {
    uint32_t tile, lo, hi, pad;
};

}  // namespace pcg
