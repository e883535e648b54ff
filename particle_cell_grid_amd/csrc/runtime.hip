// runtime.hip -- status strings, per-thread last error, grid validation and the
// kernel timing tap (HIP events around launches, for measurement).
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace pcg {

static thread_local char g_last_error[512] = "";

pcg_status fail(pcg_status status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = '\0'; }

pcg_status check_grid(const pcg_grid *grid, const char *who)
{
    if (!grid)
        return fail(PCG_EINVAL, "%s: grid is NULL", who);
    if (grid->dim < 1 || grid->dim > 3)
        return fail(PCG_EINVAL, "%s: dim %d not in {1,2,3}", who, grid->dim);
    int64_t ng = 1;
    for (int k = 0; k < 3; ++k) {
        if (grid->n[k] < 1)
            return fail(PCG_EINVAL, "%s: n[%d] = %d < 1", who, k, grid->n[k]);
        if (k >= grid->dim && grid->n[k] != 1)
            return fail(PCG_EINVAL, "%s: unused axis %d must have n = 1 (got %d)", who, k,
                        grid->n[k]);
        ng *= grid->n[k];
    }
    if (ng > (int64_t(1) << 31) / 27)
        return fail(PCG_EINVAL, "%s: grid of %lld nodes is too large", who, (long long)ng);
    return PCG_OK;
}

int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// ------------------------------------------------------------ timing tap

namespace {
struct Pending {
    hipEvent_t start, stop;
};
struct KernelTimes {
    std::vector<Pending> pending;
    double ms = 0.0;
    int64_t launches = 0;
};
std::mutex g_tmu;
bool g_timing = false;
std::map<std::string, KernelTimes> g_times;
std::vector<hipEvent_t> g_free_events;
thread_local hipEvent_t g_open_start = nullptr;

hipEvent_t take_event()
{
    if (!g_free_events.empty()) {
        hipEvent_t e = g_free_events.back();
        g_free_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}
}  // namespace

bool timing_on()
{
    std::lock_guard<std::mutex> lk(g_tmu);
    return g_timing;
}

void timing_before(const char *, hipStream_t stream)
{
    std::lock_guard<std::mutex> lk(g_tmu);
    g_open_start = take_event();
    if (g_open_start)
        (void)hipEventRecord(g_open_start, stream);
}

void timing_after(const char *name, hipStream_t stream)
{
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_open_start)
        return;
    hipEvent_t stop = take_event();
    if (!stop) {
        g_free_events.push_back(g_open_start);
        g_open_start = nullptr;
        return;
    }
    (void)hipEventRecord(stop, stream);
    g_times[name].pending.push_back({g_open_start, stop});
    g_open_start = nullptr;
}

}  // namespace pcg

using namespace pcg;

extern "C" {

const char *pcg_status_string(pcg_status s)
{
    switch (s) {
    case PCG_OK: return "PCG_OK";
    case PCG_EINVAL: return "PCG_EINVAL: invalid argument";
    case PCG_EUNSUPPORTED: return "PCG_EUNSUPPORTED: combination not supported";
    case PCG_ELDS: return "PCG_ELDS: scratch tile exceeds the LDS limit";
    case PCG_EWORKSPACE: return "PCG_EWORKSPACE: workspace missing or too small";
    case PCG_EHIP: return "PCG_EHIP: HIP runtime error";
    default: return "unknown pcg_status";
    }
}

const char *pcg_last_error(void) { return g_last_error; }

const char *pcg_version(void) { return "pcg 0.1 (gfx950)"; }

pcg_status pcg_timing_enable(int32_t enable)
{
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = enable != 0;
    return PCG_OK;
}

pcg_status pcg_timing_reset(void)
{
    std::lock_guard<std::mutex> lk(g_tmu);
    for (auto &kv : g_times) {
        for (auto &p : kv.second.pending) {
            (void)hipEventSynchronize(p.stop);
            g_free_events.push_back(p.start);
            g_free_events.push_back(p.stop);
        }
    }
    g_times.clear();
    return PCG_OK;
}

pcg_status pcg_timing_read(const char *kernel, double *total_ms, int64_t *launches)
{
    if (!kernel || !total_ms || !launches)
        return fail(PCG_EINVAL, "pcg_timing_read: NULL argument");
    std::lock_guard<std::mutex> lk(g_tmu);
    auto it = g_times.find(kernel);
    if (it == g_times.end()) {
        *total_ms = 0.0;
        *launches = 0;
        return PCG_OK;
    }
    KernelTimes &kt = it->second;
    for (auto &p : kt.pending) {
        if (hipEventSynchronize(p.stop) != hipSuccess)
            return fail(PCG_EHIP, "pcg_timing_read: event synchronisation failed");
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
            kt.ms += ms;
            kt.launches += 1;
        }
        g_free_events.push_back(p.start);
        g_free_events.push_back(p.stop);
    }
    kt.pending.clear();
    *total_ms = kt.ms;
    *launches = kt.launches;
    return PCG_OK;
}

pcg_status pcg_timing_names(char *buf, size_t len)
{
    if (!buf || len == 0)
        return fail(PCG_EINVAL, "pcg_timing_names: NULL buffer");
    std::lock_guard<std::mutex> lk(g_tmu);
    std::string s;
    for (auto &kv : g_times) {
        if (!s.empty())
            s += ",";
        s += kv.first;
    }
    std::strncpy(buf, s.c_str(), len - 1);
    buf[len - 1] = '\0';
    return PCG_OK;
}

}  // extern "C"
