// tb_check.hip -- the TB_CHECK debug mode: device-side checks of a call's
// inputs, enqueued before its kernels when the mode is on (gfx950).
//
// The hot-path kernels clamp what could take them out of bounds (context
// lengths, list counts, list entries) and compute garbage, not faults, from
// non-finite inputs; in debug mode these kernels say which of those
// happened.  Each check ORs a bit into one word per device (TB_CHECK_* in
// tokenbutler.h); the host reads and clears it with tb_check_flags().
#include "tb_internal.h"

#include <atomic>
#include <cstdlib>

namespace tb {

__device__ uint32_t check_word;

namespace {

constexpr int kCheckThreads = 256;

template <typename T> __device__ __forceinline__ bool finite_elt(T x);
template <> __device__ __forceinline__ bool finite_elt<float>(float x)
{
    return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u;
}
template <> __device__ __forceinline__ bool finite_elt<bf16_t>(bf16_t x)
{
    return (x & 0x7f80u) != 0x7f80u;
}

// Every element of a dense array of n elements.
template <typename T>
__global__ __launch_bounds__(kCheckThreads) void finite_kernel(const T *__restrict__ p, size_t n,
                                                               uint32_t bit, uint32_t *flags)
{
    bool bad = false;
    for (size_t e = (size_t)blockIdx.x * kCheckThreads + threadIdx.x; e < n;
         e += (size_t)gridDim.x * kCheckThreads)
        bad |= !finite_elt<T>(p[e]);
    if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0)
        atomicOr(flags, bit);
}

// Rows [0, min(len[b] - minus, cap)) of a cache [b][heads][cap][row] (the
// rows a call reads); len NULL: every row.
template <typename T>
__global__ __launch_bounds__(kCheckThreads) void cache_kernel(const T *__restrict__ c,
                                                              const int32_t *__restrict__ len,
                                                              int minus, int heads, int cap,
                                                              int row, uint32_t bit,
                                                              uint32_t *flags)
{
    const int bh = blockIdx.y, b = bh / heads;
    const int n = len == nullptr ? cap : clamp_len(len[b] - minus, cap);
    const size_t base = (size_t)bh * cap * row, m = (size_t)n * row;
    bool bad = false;
    for (size_t e = (size_t)blockIdx.x * kCheckThreads + threadIdx.x; e < m;
         e += (size_t)gridDim.x * kCheckThreads)
        bad |= !finite_elt<T>(c[base + e]);
    if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0)
        atomicOr(flags, bit);
}

// Context lengths and keep_from in [0, cap]; with lists, counts in
// [0, stride] and the first count entries ascending in [0, cap).  One
// work-group per (b, importance head) row of the lists (one per b without).
__global__ __launch_bounds__(kCheckThreads) void index_kernel(
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ keep_from, int Himp, int cap,
    const int32_t *__restrict__ sel_idx, int stride, const int32_t *__restrict__ sel_count,
    uint32_t *flags)
{
    const int row = blockIdx.x, b = sel_idx != nullptr ? row / Himp : row;
    if (threadIdx.x == 0) {
        const int n = ctx_len[b];
        if (n < 0 || n > cap)
            atomicOr(flags, (uint32_t)TB_CHECK_CTX_RANGE);
        if (keep_from != nullptr && (keep_from[b] < 0 || keep_from[b] > cap))
            atomicOr(flags, (uint32_t)TB_CHECK_KEEP_RANGE);
    }
    if (sel_idx == nullptr)
        return;
    const int cnt = sel_count[row];
    bool bad = threadIdx.x == 0 && (cnt < 0 || cnt > stride);
    const int m = cnt < 0 ? 0 : (cnt > stride ? stride : cnt);
    const int32_t *L = sel_idx + (size_t)row * stride;
    for (int e = threadIdx.x; e < m; e += kCheckThreads) {
        const int t = L[e];
        bad |= t < 0 || t >= cap || (e > 0 && L[e - 1] >= t);
    }
    if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0)
        atomicOr(flags, (uint32_t)TB_CHECK_SEL_RANGE);
}

std::atomic<int> g_mode{-1}; // -1: not yet read from the environment

uint32_t *flags_of_current_device(hipError_t &e)
{
    static std::atomic<uint32_t *> known[64];
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess || dev >= 64)
        return nullptr;
    uint32_t *p = known[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress((void **)&p, HIP_SYMBOL(check_word));
        if (e != hipSuccess)
            return nullptr;
        known[dev].store(p, std::memory_order_release);
    }
    return p;
}

int grid_for(size_t n)
{
    const size_t g = (n + kCheckThreads - 1) / kCheckThreads;
    return (int)(g < 1 ? 1 : (g > 2048 ? 2048 : g));
}

} // namespace

bool check_enabled()
{
    int m = g_mode.load(std::memory_order_relaxed);
    if (m < 0) {
        const char *v = std::getenv("TB_CHECK");
        m = v != nullptr && v[0] != '\0' && v[0] != '0' ? 1 : 0;
        int expect = -1;
        g_mode.compare_exchange_strong(expect, m, std::memory_order_relaxed);
        m = g_mode.load(std::memory_order_relaxed);
    }
    return m == 1;
}

void set_check(bool on) { g_mode.store(on ? 1 : 0, std::memory_order_relaxed); }

hipError_t check_dense(const void *p, size_t n, int dtype, uint32_t bit, hipStream_t st)
{
    if (p == nullptr || n == 0)
        return hipSuccess;
    hipError_t e;
    uint32_t *flags = flags_of_current_device(e);
    if (flags == nullptr)
        return e;
    if (dtype == TB_BF16)
        hipLaunchKernelGGL(finite_kernel<bf16_t>, dim3(grid_for(n)), dim3(kCheckThreads), 0, st,
                           (const bf16_t *)p, n, bit, flags);
    else
        hipLaunchKernelGGL(finite_kernel<float>, dim3(grid_for(n)), dim3(kCheckThreads), 0, st,
                           (const float *)p, n, bit, flags);
    return hipGetLastError();
}

hipError_t check_cache(const void *c, const int32_t *len, int minus, int batch, int heads,
                       int cap, int row, int dtype, uint32_t bit, hipStream_t st)
{
    if (c == nullptr)
        return hipSuccess;
    hipError_t e;
    uint32_t *flags = flags_of_current_device(e);
    if (flags == nullptr)
        return e;
    const dim3 grid(grid_for((size_t)cap * row / 4), batch * heads);
    if (dtype == TB_BF16)
        hipLaunchKernelGGL(cache_kernel<bf16_t>, grid, dim3(kCheckThreads), 0, st,
                           (const bf16_t *)c, len, minus, heads, cap, row, bit, flags);
    else
        hipLaunchKernelGGL(cache_kernel<float>, grid, dim3(kCheckThreads), 0, st,
                           (const float *)c, len, minus, heads, cap, row, bit, flags);
    return hipGetLastError();
}

hipError_t check_indices(const int32_t *ctx_len, const int32_t *keep_from, int batch, int Himp,
                         int cap, const int32_t *sel_idx, int stride, const int32_t *sel_count,
                         hipStream_t st)
{
    hipError_t e;
    uint32_t *flags = flags_of_current_device(e);
    if (flags == nullptr)
        return e;
    const bool lists = sel_idx != nullptr && sel_count != nullptr;
    hipLaunchKernelGGL(index_kernel, dim3(lists ? batch * Himp : batch), dim3(kCheckThreads), 0,
                       st, ctx_len, keep_from, Himp, cap, lists ? sel_idx : nullptr, stride,
                       lists ? sel_count : nullptr, flags);
    return hipGetLastError();
}

hipError_t read_check_flags(uint32_t *out, bool clear)
{
    hipError_t e;
    uint32_t *flags = flags_of_current_device(e);
    if (flags == nullptr)
        return e;
    e = hipDeviceSynchronize();
    if (e != hipSuccess)
        return e;
    e = hipMemcpy(out, flags, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess || !clear)
        return e;
    const uint32_t zero = 0u;
    return hipMemcpy(flags, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
}

} // namespace tb
