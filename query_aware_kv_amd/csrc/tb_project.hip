// tb_project.hip -- key projection into the projected-key cache, and the
// append of new K/V rows (gfx950).
//
// TokenButler (gist.science technical summary, Methodology > Core
// Architecture): at each consumer layer the cached keys are mapped into the
// low-dimensional importance space by one learned matrix W [D][d].  Inference
// Strategy > Optimizations: this projection is done for a batch of new tokens
// at a time.
//
// Precision contract: kp = round_to_dtype( sum_{i ascending} k[i] * W[i][j] )
// with the sum in fp64.  Every product of two bf16 (or two fp32) values is
// exact in fp64, so a fused multiply-add in ascending i yields the same bits
// as the plain fp64 sum; the result is rounded once.  MI355X runs fp64 FMA at
// the same vector rate as non-packed fp32, and fp64 MFMA has the same peak,
// so the dense contraction stays on the vector ALU where its summation order
// is fixed.
#include "tb_internal.h"

namespace tb {
namespace {

// W [D][DI] into LDS as fp64, read in 16-byte pieces that are all requested
// before any is used (256 threads).
template <typename T, int D, int DI>
__device__ __forceinline__ void stage_w_f64(const T *__restrict__ w, double *sW)
{
    constexpr int EPC = 16 / sizeof(T);
    constexpr int WP = D * DI / EPC;
    constexpr int WPT = (WP + 255) / 256;
    uint4 wp[WPT];
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
        const int pi = threadIdx.x + q * 256;
        wp[q] = reinterpret_cast<const uint4 *>(w)[pi < WP ? pi : 0];
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
        const int pi = threadIdx.x + q * 256;
        if (pi < WP) {
            T v[EPC];
            __builtin_memcpy(v, &wp[q], 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                sW[pi * EPC + e] = to_f64(v[e]);
        }
    }
}

// ---------------------------------------------------------------------------
// Few rows (the per-step append): one thread per (row, output column).  The
// W matrix and the work-group's K rows are staged in LDS as fp64.
// ---------------------------------------------------------------------------
template <typename T, int D, int DI, bool APPEND>
__global__ __launch_bounds__(256) void project_rows_kernel(
    const T *__restrict__ src, const T *__restrict__ vsrc, const T *__restrict__ w,
    const int32_t *__restrict__ pos_or_len, int n_tokens, int Hkv, int cap, int rows_total,
    T *__restrict__ k_cache, T *__restrict__ v_cache, T *__restrict__ kp)
{
    constexpr int ROWS = 256 / DI;
    __shared__ double sW[D * DI];
    __shared__ double sK[ROWS][D + 1];

    stage_w_f64<T, D, DI>(w, sW);

    const int rl = threadIdx.x / DI;
    const int j = threadIdx.x % DI;
    const int row = blockIdx.x * ROWS + rl;
    bool valid = row < rows_total;
    int bg = 0, t = 0, jj = 0;
    if (valid) {
        bg = row / n_tokens;
        jj = row - bg * n_tokens;
        const int b = bg / Hkv;
        if (APPEND)
            t = clamp_len(pos_or_len[b], cap) - n_tokens + jj;
        else
            t = pos_or_len[b] + jj;
        valid = t >= 0 && t < cap;
    }
    const size_t crow = ((size_t)bg * cap + t) * D;
    const size_t srow = APPEND ? ((size_t)bg * n_tokens + jj) * D : crow;
    if (valid) {
        for (int i = j; i < D; i += DI) {
            const T kv = src[srow + i];
            sK[rl][i] = to_f64(kv);
            if (APPEND) {
                k_cache[crow + i] = kv;
                v_cache[crow + i] = vsrc[srow + i];
            }
        }
    }
    __syncthreads();
    if (valid) {
        double acc = 0.0;
#pragma unroll 8
        for (int i = 0; i < D; ++i)
            acc = fma(sK[rl][i], sW[i * DI + j], acc);
        kp[((size_t)bg * cap + t) * DI + j] = from_f64<T>(acc);
    }
}

// ---------------------------------------------------------------------------
// Many rows (prefill-sized batches): each thread owns RPT rows x OPT output
// columns, so every W value read from LDS feeds RPT fma and every K value
// feeds OPT fma.  K rows stream from HBM in 16-byte pieces.
// ---------------------------------------------------------------------------
template <typename T, int D, int DI>
__global__ __launch_bounds__(256) void project_wide_kernel(
    const T *__restrict__ k_cache, const T *__restrict__ w, const int32_t *__restrict__ pos0,
    int n_tokens, int Hkv, int cap, int rows_total, T *__restrict__ kp)
{
    constexpr int OPT = 8;
    constexpr int RPT = 4;
    constexpr int JS = DI / OPT;
    constexpr int RG = 256 / JS;
    constexpr int ROWS = RG * RPT;
    constexpr int EPC = 16 / sizeof(T); // elements per 16-byte piece
    __shared__ double sW[D * DI];

    stage_w_f64<T, D, DI>(w, sW);
    __syncthreads();

    const int js = threadIdx.x % JS;
    const int rg = threadIdx.x / JS;
    size_t rowoff[RPT];
    bool valid[RPT];
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
        const int row = blockIdx.x * ROWS + rg + RG * rr;
        valid[rr] = false;
        rowoff[rr] = 0;
        if (row < rows_total) {
            const int bg = row / n_tokens;
            const int jj = row - bg * n_tokens;
            const int t = pos0[bg / Hkv] + jj;
            if (t >= 0 && t < cap) {
                valid[rr] = true;
                rowoff[rr] = (size_t)bg * cap + t;
            }
        }
    }

    double acc[RPT][OPT];
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
        for (int o = 0; o < OPT; ++o)
            acc[rr][o] = 0.0;

    for (int i0 = 0; i0 < D; i0 += EPC) {
        T kv[RPT][EPC];
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) {
            // unconditional (an invalid row reads row 0 and is not stored), so
            // the loads issue back to back
            const uint4 piece = *reinterpret_cast<const uint4 *>(k_cache + rowoff[rr] * D + i0);
            __builtin_memcpy(kv[rr], &piece, 16);
        }
#pragma unroll
        for (int ii = 0; ii < EPC; ++ii) {
            const double2 *wp = reinterpret_cast<const double2 *>(&sW[(i0 + ii) * DI + js * OPT]);
            double wv[OPT];
#pragma unroll
            for (int o2 = 0; o2 < OPT / 2; ++o2) {
                const double2 p = wp[o2];
                wv[2 * o2] = p.x;
                wv[2 * o2 + 1] = p.y;
            }
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr) {
                const double k = to_f64(kv[rr][ii]);
#pragma unroll
                for (int o = 0; o < OPT; ++o)
                    acc[rr][o] = fma(k, wv[o], acc[rr][o]);
            }
        }
    }

#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
        if (!valid[rr])
            continue;
        T res[OPT];
#pragma unroll
        for (int o = 0; o < OPT; ++o)
            res[o] = from_f64<T>(acc[rr][o]);
        T *dst = kp + rowoff[rr] * DI + js * OPT;
#pragma unroll
        for (int p = 0; p < OPT * (int)sizeof(T) / 16; ++p)
            reinterpret_cast<uint4 *>(dst)[p] = reinterpret_cast<const uint4 *>(res)[p];
    }
}

template <typename T, int D, int DI>
hipError_t project_dispatch_t(const tb_shape &s, const void *k_cache, const void *w,
                              const int32_t *pos0, int n, void *kp, hipStream_t st)
{
    const long rows = (long)s.batch * s.n_kv_heads * n;
    if (rows >= 16384) {
        constexpr int ROWS = (256 / (DI / 8)) * 4;
        const int grid = (int)((rows + ROWS - 1) / ROWS);
        hipLaunchKernelGGL((project_wide_kernel<T, D, DI>), dim3(grid), dim3(256), 0, st,
                           (const T *)k_cache, (const T *)w, pos0, n, s.n_kv_heads, s.ctx_cap,
                           (int)rows, (T *)kp);
    } else {
        constexpr int ROWS = 256 / DI;
        const int grid = (int)((rows + ROWS - 1) / ROWS);
        hipLaunchKernelGGL((project_rows_kernel<T, D, DI, false>), dim3(grid), dim3(256), 0, st,
                           (const T *)k_cache, (const T *)nullptr, (const T *)w, pos0, n,
                           s.n_kv_heads, s.ctx_cap, (int)rows, (T *)nullptr, (T *)nullptr,
                           (T *)kp);
    }
    return hipGetLastError();
}

template <typename T, int D, int DI>
hipError_t append_dispatch_t(const tb_shape &s, const void *k_new, const void *v_new, int n,
                             const void *w, void *k_cache, void *v_cache, void *kp,
                             const int32_t *ctx_len, hipStream_t st)
{
    const long rows = (long)s.batch * s.n_kv_heads * n;
    constexpr int ROWS = 256 / DI;
    const int grid = (int)((rows + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((project_rows_kernel<T, D, DI, true>), dim3(grid), dim3(256), 0, st,
                       (const T *)k_new, (const T *)v_new, (const T *)w, ctx_len, n,
                       s.n_kv_heads, s.ctx_cap, (int)rows, (T *)k_cache, (T *)v_cache, (T *)kp);
    return hipGetLastError();
}

#define TB_DISPATCH_D_DI(FN, T, ...)                                                         \
    do {                                                                                      \
        if (s.head_dim == 64 && s.d_imp == 16) return FN<T, 64, 16>(__VA_ARGS__);            \
        if (s.head_dim == 64 && s.d_imp == 32) return FN<T, 64, 32>(__VA_ARGS__);            \
        if (s.head_dim == 128 && s.d_imp == 16) return FN<T, 128, 16>(__VA_ARGS__);          \
        if (s.head_dim == 128 && s.d_imp == 32) return FN<T, 128, 32>(__VA_ARGS__);          \
    } while (0)

} // namespace

hipError_t launch_project(const tb_shape &s, const void *k_cache, const void *w,
                          const int32_t *pos0, int n_tokens, void *kp_cache, hipStream_t st)
{
    if (s.dtype == TB_BF16)
        TB_DISPATCH_D_DI(project_dispatch_t, bf16_t, s, k_cache, w, pos0, n_tokens, kp_cache, st);
    else
        TB_DISPATCH_D_DI(project_dispatch_t, float, s, k_cache, w, pos0, n_tokens, kp_cache, st);
    return hipErrorInvalidValue;
}

hipError_t launch_append_project(const tb_shape &s, const void *k_new, const void *v_new,
                                 int n_new, const void *w, void *k_cache, void *v_cache,
                                 void *kp_cache, const int32_t *ctx_len, hipStream_t st)
{
    if (s.dtype == TB_BF16)
        TB_DISPATCH_D_DI(append_dispatch_t, bf16_t, s, k_new, v_new, n_new, w, k_cache, v_cache,
                         kp_cache, ctx_len, st);
    else
        TB_DISPATCH_D_DI(append_dispatch_t, float, s, k_new, v_new, n_new, w, k_cache, v_cache,
                         kp_cache, ctx_len, st);
    return hipErrorInvalidValue;
}

} // namespace tb
