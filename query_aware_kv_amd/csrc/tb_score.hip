// tb_score.hip -- importance scores (gfx950).
//
// TokenButler (gist.science technical summary, Methodology > Core
// Architecture): each predicted low-dimensional importance query is dotted
// with the projected keys of its KV head to score every cached token.
//
// One streaming pass over the projected-key cache: a lane owns one token of
// one KV head, reads its d projected-key values (d*elt bytes, contiguous) in
// 16-byte loads, widens them to fp64 once, and produces the scores of all
// importance heads that read this KV head.  The importance queries of the
// work-group are wave-uniform: they are read as fp64 through the scalar cache
// (scalar loads into SGPRs), so each lane-token costs d fp64 fma per head.
//
// Precision contract: score = fp32( sum_{j ascending} q[j] * kp[j] ) with the
// sum in fp64.  Products of two bf16/fp32 values are exact in fp64, so the
// fma chain equals the plain fp64 sum bit for bit; the one rounding to fp32
// gives the selection key.
#include "tb_internal.h"

namespace tb {
namespace {

constexpr int kScoreThreads = 256;

template <typename T, int DI, int GI>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const double *__restrict__ q64, const T *__restrict__ kp, const int32_t *__restrict__ ctx_len,
    int Himp, int Hkv, int cap, float *__restrict__ scores)
{
    const int b = blockIdx.z;
    const int g = blockIdx.y;
    const int n = clamp_len(ctx_len[b], cap);
    const int t0 = blockIdx.x * kScoreThreads;
    if (t0 >= n)
        return;
    const int t = t0 + threadIdx.x;
    const bool valid = t < n;

    constexpr int EPC = 16 / sizeof(T);
    double k[DI];
    {
        const T *row = kp + (((size_t)b * Hkv + g) * cap + (valid ? t : t0)) * DI;
#pragma unroll
        for (int p = 0; p < DI / EPC; ++p) {
            const uint4 piece = reinterpret_cast<const uint4 *>(row)[p];
            T v[EPC];
            __builtin_memcpy(v, &piece, 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                k[p * EPC + e] = to_f64(v[e]);
        }
    }

    const double *qb = q64 + ((size_t)b * Himp + (size_t)g * GI) * DI;
    float *sb = scores + ((size_t)b * Himp + (size_t)g * GI) * cap;
#pragma unroll
    for (int hh = 0; hh < GI; ++hh) {
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < DI; ++j)
            acc = fma(qb[hh * DI + j], k[j], acc);
        if (valid)
            sb[(size_t)hh * cap + t] = (float)acc;
    }
}

template <typename T, int DI, int GI>
hipError_t score_t(const tb_shape &s, const double *q64, const void *kp, const int32_t *ctx_len,
                   float *scores, hipStream_t st)
{
    dim3 grid((s.ctx_cap + kScoreThreads - 1) / kScoreThreads, s.n_kv_heads, s.batch);
    hipLaunchKernelGGL((score_kernel<T, DI, GI>), grid, dim3(kScoreThreads), 0, st, q64,
                       (const T *)kp, ctx_len, s.n_imp_heads, s.n_kv_heads, s.ctx_cap, scores);
    return hipGetLastError();
}

template <typename T, int DI>
hipError_t score_gi(const tb_shape &s, const double *q64, const void *kp, const int32_t *ctx_len,
                    float *scores, hipStream_t st)
{
    switch (s.n_imp_heads / s.n_kv_heads) {
    case 1: return score_t<T, DI, 1>(s, q64, kp, ctx_len, scores, st);
    case 2: return score_t<T, DI, 2>(s, q64, kp, ctx_len, scores, st);
    case 4: return score_t<T, DI, 4>(s, q64, kp, ctx_len, scores, st);
    case 8: return score_t<T, DI, 8>(s, q64, kp, ctx_len, scores, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_score(const tb_shape &s, const double *q64, const void *kp_cache,
                        const int32_t *ctx_len, float *scores, hipStream_t st)
{
    if (s.dtype == TB_BF16) {
        if (s.d_imp == 16) return score_gi<bf16_t, 16>(s, q64, kp_cache, ctx_len, scores, st);
        if (s.d_imp == 32) return score_gi<bf16_t, 32>(s, q64, kp_cache, ctx_len, scores, st);
    } else {
        if (s.d_imp == 16) return score_gi<float, 16>(s, q64, kp_cache, ctx_len, scores, st);
        if (s.d_imp == 32) return score_gi<float, 32>(s, q64, kp_cache, ctx_len, scores, st);
    }
    return hipErrorInvalidValue;
}

} // namespace tb
