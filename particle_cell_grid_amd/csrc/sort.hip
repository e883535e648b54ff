// sort.hip -- stable tile sort of particles ([TD] Entity wiki "Tiled current
// deposit", section "The tile-based spatial sort"; with T = 1 the cell sort the
// mass-matrix paper's §3.1 assumes).
//
// Pipeline on the caller's stream:
//   1. k_tile_keys      key = tile of the first support node (uint32).
//   2. LSD radix sort of (key, index) pairs, ceil(bits/8) passes of <= 8 bits:
//        k_radix_hist     per-block digit histograms, digit-major [R][nblocks];
//        scan             exclusive prefix over that array (3 kernels);
//        k_radix_scatter  stable scatter: every wave ranks its 64 keys with
//                         ballot-based peer masks, the block orders its waves
//                         and items with per-(slot, digit) counts in LDS.
//      Each pass is stable, so the composition sorts by key with ties in input
//      order, i.e. the unique stable permutation.
//   3. k_tile_offsets   offsets[t] = #keys < t, from key transitions.
//   4. k_permute        out_a[j] = in_a[perm[j]] for each SoA array.
#include "common.hpp"

namespace pcg {
namespace {

constexpr int SORT_BLOCK = 256;
constexpr int SORT_IPT = 16;
constexpr int SORT_TILE = SORT_BLOCK * SORT_IPT;            // items per block
constexpr int SORT_SLOTS = SORT_IPT * (SORT_BLOCK / WAVE);  // wave-slots per block
constexpr int SCAN_BLOCK = 256;
constexpr int SCAN_IPT = 16;
constexpr int SCAN_TILE = SCAN_BLOCK * SCAN_IPT;
constexpr int MAX_ARRAYS = 16;

struct KeyGeom {
    int n[3];
    int nt[3];
    int T;
    int T_shift;  // log2(T) if T is a power of two, else -1
};

// ----------------------------------------------------------------- keys

template <int DIM, int ORDER>
__global__ __launch_bounds__(256) void k_tile_keys(int64_t count, const float *__restrict__ x0,
                                                   const float *__restrict__ x1,
                                                   const float *__restrict__ x2, KeyGeom g,
                                                   uint32_t *__restrict__ keys)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const float *xs[3] = {x0, x1, x2};
        uint32_t key = 0, mul = 1;
#pragma unroll
        for (int k = 0; k < DIM; ++k) {
            float xf = clamp_coord(xs[k][i], (float)g.n[k]);
            float fl = floorf(xf);
            int b = (int)fl;
            if (ORDER == 2 && (xf - fl) < 0.5f)
                b -= 1;
            b = wrap_index(b, g.n[k]);
            int t = g.T_shift >= 0 ? (b >> g.T_shift) : (b / g.T);
            key += mul * (uint32_t)t;
            mul *= (uint32_t)g.nt[k];
        }
        keys[i] = key;
    }
}

// ----------------------------------------------------------------- radix

// Lanes of this wave whose `bits`-bit digit equals mine (among valid lanes).
template <int BITS>
__device__ inline uint64_t peer_mask(uint32_t digit, bool valid)
{
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
        const bool bit = (digit >> b) & 1u;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

template <int BITS>
__global__ __launch_bounds__(SORT_BLOCK) void k_radix_hist(const uint32_t *__restrict__ keys,
                                                           int64_t count, int shift,
                                                           uint32_t *__restrict__ counts,
                                                           uint32_t nblocks)
{
    constexpr uint32_t R = 1u << BITS;
    __shared__ uint32_t hist[R];
    for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK)
        hist[d] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
#pragma unroll 4
    for (int j = 0; j < SORT_IPT; ++j) {
        const int64_t idx = base + (int64_t)j * SORT_BLOCK + threadIdx.x;
        const bool valid = idx < count;
        const uint32_t digit = valid ? (keys[idx] >> shift) & (R - 1) : 0u;
        const uint64_t peers = peer_mask<BITS>(digit, valid);
        // the lowest lane of each peer group adds the group's size
        if (valid && (peers & lanemask_lt()) == 0)
            atomicAdd(&hist[digit], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK)
        counts[(size_t)d * nblocks + blockIdx.x] = hist[d];
}

template <int BITS>
__global__ __launch_bounds__(SORT_BLOCK) void k_radix_scatter(
    const uint32_t *__restrict__ keys_in, const uint32_t *__restrict__ vals_in,
    uint32_t *__restrict__ keys_out, uint32_t *__restrict__ vals_out, int64_t count, int shift,
    const uint32_t *__restrict__ offsets, uint32_t nblocks)
{
    constexpr uint32_t R = 1u << BITS;
    __shared__ uint16_t cnt[SORT_SLOTS][R];  // items of digit d in wave-slot s, then prefix
    __shared__ uint32_t gbase[R];
    {
        uint32_t *c32 = reinterpret_cast<uint32_t *>(&cnt[0][0]);
        constexpr int words = SORT_SLOTS * R / 2;
        for (int i = threadIdx.x; i < words; i += SORT_BLOCK)
            c32[i] = 0;
    }
    for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK)
        gbase[d] = offsets[(size_t)d * nblocks + blockIdx.x];
    __syncthreads();

    const int wave = threadIdx.x / WAVE;
    const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
    uint32_t key[SORT_IPT], val[SORT_IPT];
    uint16_t rank[SORT_IPT];
#pragma unroll
    for (int j = 0; j < SORT_IPT; ++j) {
        const int64_t idx = base + (int64_t)j * SORT_BLOCK + threadIdx.x;
        const bool valid = idx < count;
        key[j] = valid ? keys_in[idx] : 0u;
        val[j] = valid ? (vals_in ? vals_in[idx] : (uint32_t)idx) : 0u;
        const uint32_t digit = (key[j] >> shift) & (R - 1);
        const uint64_t peers = peer_mask<BITS>(digit, valid);
        rank[j] = (uint16_t)__popcll(peers & lanemask_lt());
        if (valid && rank[j] == 0)
            cnt[j * (SORT_BLOCK / WAVE) + wave][digit] = (uint16_t)__popcll(peers);
    }
    __syncthreads();
    // exclusive prefix over wave-slots, per digit (slot order = item order)
    for (uint32_t d = threadIdx.x; d < R; d += SORT_BLOCK) {
        uint32_t run = 0;
        for (int s = 0; s < SORT_SLOTS; ++s) {
            const uint32_t c = cnt[s][d];
            cnt[s][d] = (uint16_t)run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SORT_IPT; ++j) {
        const int64_t idx = base + (int64_t)j * SORT_BLOCK + threadIdx.x;
        if (idx < count) {
            const uint32_t digit = (key[j] >> shift) & (R - 1);
            const uint32_t dst =
                gbase[digit] + cnt[j * (SORT_BLOCK / WAVE) + wave][digit] + rank[j];
            if (dst < (uint64_t)count) {  // always true for a consistent histogram
                keys_out[dst] = key[j];
                vals_out[dst] = val[j];
            }
        }
    }
}

// ----------------------------------------------------------------- scan

__device__ inline uint32_t wave_inclusive_scan(uint32_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t o = __shfl_up(v, off, WAVE);
        if (lane >= off)
            v += o;
    }
    return v;
}

// Exclusive scan of one value per thread across the block; returns the
// exclusive prefix and writes the block total to *total.
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t *total)
{
    __shared__ uint32_t wsum[NT / WAVE];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == WAVE - 1)
        wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / WAVE; ++w) {
        const uint32_t s = wsum[w];
        before += (w < wave) ? s : 0u;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_reduce(const uint32_t *__restrict__ in,
                                                            size_t len,
                                                            uint32_t *__restrict__ partial)
{
    const size_t base = (size_t)blockIdx.x * SCAN_TILE;
    uint32_t s = 0;
    for (int j = 0; j < SCAN_IPT; ++j) {
        const size_t idx = base + (size_t)j * SCAN_BLOCK + threadIdx.x;
        if (idx < len)
            s += in[idx];
    }
    uint32_t total;
    block_exclusive_scan<SCAN_BLOCK>(s, &total);
    if (threadIdx.x == 0)
        partial[blockIdx.x] = total;
}

// Single work-group exclusive scan of the partial sums (in place).
__global__ __launch_bounds__(1024) void k_scan_partials(uint32_t *__restrict__ partial,
                                                        uint32_t nparts)
{
    const uint32_t per = (nparts + 1023) / 1024;
    const uint32_t lo = threadIdx.x * per;
    const uint32_t hi = min(lo + per, nparts);
    uint32_t s = 0;
    for (uint32_t i = lo; i < hi; ++i)
        s += partial[i];
    uint32_t total;
    uint32_t run = block_exclusive_scan<1024>(s, &total);
    for (uint32_t i = lo; i < hi; ++i) {
        const uint32_t v = partial[i];
        partial[i] = run;
        run += v;
    }
}

__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_down(uint32_t *__restrict__ data, size_t len,
                                                          const uint32_t *__restrict__ partial)
{
    // thread t owns SCAN_IPT consecutive elements of the block's tile
    const size_t base = (size_t)blockIdx.x * SCAN_TILE + (size_t)threadIdx.x * SCAN_IPT;
    uint32_t v[SCAN_IPT];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < SCAN_IPT; ++j) {
        v[j] = (base + j < len) ? data[base + j] : 0u;
        s += v[j];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<SCAN_BLOCK>(s, &total) + partial[blockIdx.x];
#pragma unroll
    for (int j = 0; j < SCAN_IPT; ++j) {
        if (base + j < len)
            data[base + j] = run;
        run += v[j];
    }
}

pcg_status exclusive_scan(uint32_t *data, size_t len, uint32_t *partial, hipStream_t st)
{
    const uint32_t nparts = (uint32_t)((len + SCAN_TILE - 1) / SCAN_TILE);
    PCG_TRY(launch("sort_scan_reduce", k_scan_reduce, dim3(nparts), dim3(SCAN_BLOCK), 0, st,
                   (const uint32_t *)data, len, partial));
    PCG_TRY(launch("sort_scan_partials", k_scan_partials, dim3(1), dim3(1024), 0, st, partial,
                   nparts));
    PCG_TRY(launch("sort_scan_down", k_scan_down, dim3(nparts), dim3(SCAN_BLOCK), 0, st, data,
                   len, (const uint32_t *)partial));
    return PCG_OK;
}

// ----------------------------------------------------------------- offsets, permute

__global__ __launch_bounds__(256) void k_tile_offsets(const uint32_t *__restrict__ sk,
                                                      int64_t count, uint32_t ntiles,
                                                      uint32_t *__restrict__ off)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i <= count; i += stride) {
        // tiles t in (sk[i-1], sk[i]] start at slot i (with sk[-1] = -1, sk[count] = ntiles)
        const uint32_t lo = (i == 0) ? 0u : sk[i - 1] + 1u;
        const uint32_t hi = (i == count) ? ntiles : sk[i];
        for (uint32_t t = lo; t <= hi && t <= ntiles; ++t)
            off[t] = (uint32_t)i;
    }
}

struct PermArgs {
    const float *in[MAX_ARRAYS];
    float *out[MAX_ARRAYS];
    int n;
};

__global__ __launch_bounds__(256) void k_permute(PermArgs a, const uint32_t *__restrict__ perm,
                                                 int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint32_t p = min(perm[i], (uint32_t)(count - 1));  // perm is a permutation
        float v[MAX_ARRAYS];
#pragma unroll
        for (int k = 0; k < MAX_ARRAYS; ++k)
            if (k < a.n)
                v[k] = a.in[k][p];
#pragma unroll
        for (int k = 0; k < MAX_ARRAYS; ++k)
            if (k < a.n)
                a.out[k][i] = v[k];
    }
}

// ----------------------------------------------------------------- host

struct SortPlan {
    int64_t count = 0;
    uint32_t ntiles = 1;
    int key_bits = 0;
    int passes = 1;
    int bits = 1;
    uint32_t nblocks = 0;
    size_t counts_len = 0;
};

SortPlan make_plan(const pcg_grid *grid, int64_t count, int T)
{
    SortPlan p;
    p.count = count;
    uint64_t nt = 1;
    for (int k = 0; k < grid->dim; ++k)
        nt *= (uint64_t)(grid->n[k] / T);
    p.ntiles = (uint32_t)nt;
    int kb = 0;
    while ((uint64_t(1) << kb) < nt)
        ++kb;
    p.key_bits = kb;
    p.passes = kb == 0 ? 1 : (kb + 7) / 8;
    p.bits = kb == 0 ? 1 : (kb + p.passes - 1) / p.passes;
    p.nblocks = (uint32_t)((count + SORT_TILE - 1) / SORT_TILE);
    p.counts_len = (size_t)(1u << p.bits) * p.nblocks;
    return p;
}

struct SortBuffers {
    uint32_t *k0, *ak, *av, *bv, *fk, *counts, *partial;
};

size_t carve(const SortPlan &p, void *ws, SortBuffers *b)
{
    Carver c(ws);
    const size_t n = (size_t)p.count;
    b->k0 = c.take<uint32_t>(n);
    b->ak = c.take<uint32_t>(n);
    b->av = c.take<uint32_t>(n);
    b->bv = c.take<uint32_t>(n);
    b->fk = c.take<uint32_t>(n);
    b->counts = c.take<uint32_t>(p.counts_len);
    b->partial = c.take<uint32_t>((p.counts_len + SCAN_TILE - 1) / SCAN_TILE + 1);
    return c.used;
}

pcg_status check_sort_args(const pcg_grid *grid, int64_t count, int T, const char *who)
{
    PCG_TRY(check_grid(grid, who));
    if (T < 1)
        return fail(PCG_EINVAL, "%s: T = %d < 1", who, T);
    for (int k = 0; k < grid->dim; ++k)
        if (grid->n[k] % T)
            return fail(PCG_EINVAL, "%s: n[%d] = %d is not a multiple of T = %d", who, k,
                        grid->n[k], T);
    if (count < 0 || count >= (int64_t(1) << 31))
        return fail(PCG_EINVAL, "%s: count %lld outside [0, 2^31)", who, (long long)count);
    return PCG_OK;
}

template <int BITS>
pcg_status radix_pass(const SortPlan &p, int shift, const uint32_t *kin, const uint32_t *vin,
                      uint32_t *kout, uint32_t *vout, const SortBuffers &b, hipStream_t st)
{
    PCG_TRY(launch("sort_hist", k_radix_hist<BITS>, dim3(p.nblocks), dim3(SORT_BLOCK), 0, st,
                   kin, p.count, shift, b.counts, p.nblocks));
    PCG_TRY(exclusive_scan(b.counts, p.counts_len, b.partial, st));
    PCG_TRY(launch("sort_scatter", k_radix_scatter<BITS>, dim3(p.nblocks), dim3(SORT_BLOCK), 0,
                   st, kin, vin, kout, vout, p.count, shift, (const uint32_t *)b.counts,
                   p.nblocks));
    return PCG_OK;
}

pcg_status radix_pass_dispatch(int bits, const SortPlan &p, int shift, const uint32_t *kin,
                               const uint32_t *vin, uint32_t *kout, uint32_t *vout,
                               const SortBuffers &b, hipStream_t st)
{
    switch (bits) {
    case 1: return radix_pass<1>(p, shift, kin, vin, kout, vout, b, st);
    case 2: return radix_pass<2>(p, shift, kin, vin, kout, vout, b, st);
    case 3: return radix_pass<3>(p, shift, kin, vin, kout, vout, b, st);
    case 4: return radix_pass<4>(p, shift, kin, vin, kout, vout, b, st);
    case 5: return radix_pass<5>(p, shift, kin, vin, kout, vout, b, st);
    case 6: return radix_pass<6>(p, shift, kin, vin, kout, vout, b, st);
    case 7: return radix_pass<7>(p, shift, kin, vin, kout, vout, b, st);
    case 8: return radix_pass<8>(p, shift, kin, vin, kout, vout, b, st);
    default: return fail(PCG_EUNSUPPORTED, "radix pass of %d bits", bits);
    }
}

template <int DIM, int ORDER>
pcg_status launch_keys(int64_t count, const float *const x[3], const KeyGeom &g, uint32_t *keys,
                       hipStream_t st)
{
    const int64_t blocks = std::min<int64_t>((count + 255) / 256, (int64_t)device_cus() * 32);
    return launch("sort_keys", k_tile_keys<DIM, ORDER>, dim3((unsigned)std::max<int64_t>(blocks, 1)),
                  dim3(256), 0, st, count, x[0], DIM > 1 ? x[1] : nullptr,
                  DIM > 2 ? x[2] : nullptr, g, keys);
}

}  // namespace
}  // namespace pcg

using namespace pcg;

extern "C" {

size_t pcg_sort_workspace_bytes(const pcg_grid *grid, int64_t count, int32_t T)
{
    if (check_sort_args(grid, count, T, "pcg_sort_workspace_bytes") != PCG_OK)
        return 0;
    SortPlan p = make_plan(grid, count, T);
    SortBuffers b;
    return std::max<size_t>(carve(p, nullptr, &b), 256);
}

pcg_status pcg_tile_sort(const pcg_grid *grid, int32_t order, int32_t T, int64_t count,
                         const float *const key_x[3], int32_t n_arrays,
                         const float *const in_arrays[], float *const out_arrays[],
                         uint32_t *perm, uint32_t *sorted_keys, uint32_t *tile_offsets,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    const char *who = "pcg_tile_sort";
    clear_error();
    PCG_TRY(check_sort_args(grid, count, T, who));
    if (order != 1 && order != 2)
        return fail(PCG_EUNSUPPORTED, "%s: order %d not in {1,2}", who, order);
    if (count > 0 && !key_x)
        return fail(PCG_EINVAL, "%s: key_x is NULL", who);
    for (int k = 0; k < grid->dim && count > 0; ++k)
        if (!key_x[k])
            return fail(PCG_EINVAL, "%s: key_x[%d] is NULL", who, k);
    if (n_arrays < 0 || n_arrays > MAX_ARRAYS)
        return fail(PCG_EINVAL, "%s: n_arrays = %d not in [0, %d]", who, n_arrays, MAX_ARRAYS);
    if (n_arrays > 0 && (!in_arrays || !out_arrays))
        return fail(PCG_EINVAL, "%s: array lists are NULL", who);
    for (int i = 0; i < n_arrays && count > 0; ++i) {
        if (!in_arrays[i] || !out_arrays[i])
            return fail(PCG_EINVAL, "%s: array %d is NULL", who, i);
        if ((const void *)in_arrays[i] == (const void *)out_arrays[i])
            return fail(PCG_EINVAL, "%s: array %d is permuted in place (out == in)", who, i);
    }
    if ((!perm && count > 0) || !tile_offsets)
        return fail(PCG_EINVAL, "%s: perm or tile_offsets is NULL", who);
    SortPlan p = make_plan(grid, count, T);
    SortBuffers b;
    const size_t need = carve(p, nullptr, &b);
    if (!workspace || workspace_bytes < need)
        return fail(PCG_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(PCG_EWORKSPACE, "%s: workspace must be 256-byte aligned", who);
    carve(p, workspace, &b);
    hipStream_t st = static_cast<hipStream_t>(stream);

    if (count == 0) {
        return launch("sort_offsets", k_tile_offsets, dim3(1), dim3(256), 0, st,
                      (const uint32_t *)nullptr, count, p.ntiles, tile_offsets);
    }

    KeyGeom g;
    for (int k = 0; k < 3; ++k) {
        g.n[k] = grid->n[k];
        g.nt[k] = k < grid->dim ? grid->n[k] / T : 1;
    }
    g.T = T;
    g.T_shift = -1;
    for (int s = 0; s < 31; ++s)
        if ((1 << s) == T)
            g.T_shift = s;
    const int key = grid->dim * 10 + order;
    pcg_status s = PCG_OK;
    switch (key) {
    case 11: s = launch_keys<1, 1>(count, key_x, g, b.k0, st); break;
    case 12: s = launch_keys<1, 2>(count, key_x, g, b.k0, st); break;
    case 21: s = launch_keys<2, 1>(count, key_x, g, b.k0, st); break;
    case 22: s = launch_keys<2, 2>(count, key_x, g, b.k0, st); break;
    case 31: s = launch_keys<3, 1>(count, key_x, g, b.k0, st); break;
    case 32: s = launch_keys<3, 2>(count, key_x, g, b.k0, st); break;
    }
    PCG_TRY(s);

    uint32_t *final_keys = sorted_keys ? sorted_keys : b.fk;
    const uint32_t *kin = b.k0;
    const uint32_t *vin = nullptr;  // pass 0 ranks input indices
    for (int pass = 0; pass < p.passes; ++pass) {
        const bool last = pass == p.passes - 1;
        uint32_t *kout = last ? final_keys : (pass % 2 == 0 ? b.ak : b.k0);
        uint32_t *vout = last ? perm : (pass % 2 == 0 ? b.av : b.bv);
        PCG_TRY(radix_pass_dispatch(p.bits, p, pass * p.bits, kin, vin, kout, vout, b, st));
        kin = kout;
        vin = vout;
    }
    {
        const int64_t blocks = std::min<int64_t>((count + 1 + 255) / 256, (int64_t)device_cus() * 32);
        PCG_TRY(launch("sort_offsets", k_tile_offsets, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint32_t *)final_keys, count, p.ntiles, tile_offsets));
    }
    if (n_arrays > 0) {
        PermArgs a{};
        for (int i = 0; i < n_arrays; ++i) {
            a.in[i] = in_arrays[i];
            a.out[i] = out_arrays[i];
        }
        a.n = n_arrays;
        const int64_t blocks = std::min<int64_t>((count + 255) / 256, (int64_t)device_cus() * 64);
        PCG_TRY(launch("sort_permute", k_permute, dim3((unsigned)blocks), dim3(256), 0, st, a,
                       (const uint32_t *)perm, count));
    }
    return PCG_OK;
}

}  // extern "C"
