// tb_mlp.hip -- the importance-query producer: a two-layer MLP on the
// producer layer's hidden states, on the matrix cores (gfx950).
//
// TokenButler, gist.science technical summary, Methodology > Core
// Architecture > Query Prediction: a lightweight MLP maps the hidden state
// of a producer layer to G slot-specific low-dimensional query vectors per
// attention head (one slot per consumer layer that the producer serves).
//
//   u = round( act( h W1^T ) )     h [M][E], W1 [F][E]
//   q = round( u W2^T )            W2 [N][F], N = G * Himp * d
// written slot-major: q_imp[g][m][i][j] = q[m][(g * Himp + i) * d + j], so
// slot g is the [M][Himp][d] importance query that tb_score takes.
//
// Each layer is one launch of a split-K GEMM (k-slices are multiples of
// kMlpKGrain values, so a wave's loop covers whole groups of kMlpUnroll
// pieces).  Grid: (64-column block of the
// output, k-slice); 256 threads, wave w owns 16 output columns.  A wave
// multiplies its k-slice with MFMA 16x16 tiles, one accumulator tile per 16
// tokens: lane l supplies token / column l % 16 and the l / 16-th quarter of
// each k group from one 16-byte piece (bf16: one 16x16x32 step per piece;
// fp32: four 16x16x4 steps per piece).  Token rows past M read as zero.
// With one k-slice the tile is finished in registers; otherwise the
// k-slices' fp32 partials go to the workspace (agent-scope stores, which
// reach the device coherence point) and the last work-group of a column
// block to arrive sums them in k-slice order -- the result does not depend
// on arrival order -- applies the activation, rounds to the dtype, writes
// the output and resets the block's counter to zero.
#include "tb_internal.h"

namespace tb {
namespace {

constexpr int kMlpThreads = 256;
constexpr int kMlpCols = 64;  // output columns per work-group (16 per wave)
constexpr int kMlpUnroll = 8; // 16-byte pieces per lane requested together
constexpr int kMlpSumBatch = 8; // k-slice partials loaded together by the finisher

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct LayerArgs {
    const void *x;      // [M][K]
    const void *w;      // [N][K]
    void *y;            // [M][N], or slot-major [N / slot][M][slot]
    float *part;        // [KS][M][N] fp32 partials
    uint32_t *counters; // [N / kMlpCols], zero between calls
    int M, K, N, KS;
    int slot;           // columns per slot of a slot-major output (0: row-major)
    int act;            // TB_ACT_RELU / TB_ACT_SILU, or -1 for none
};

__device__ __forceinline__ float activate(float x, int act)
{
    if (act == TB_ACT_RELU)
        return x > 0.f ? x : 0.f;
    if (act == TB_ACT_SILU)
        return x / (1.f + __expf(-x));
    return x;
}

template <typename T>
__device__ __forceinline__ void store_out(const LayerArgs &a, int m, int n, float v)
{
    const float r = activate(v, a.act);
    size_t o;
    if (a.slot > 0)
        o = ((size_t)(n / a.slot) * a.M + m) * a.slot + n % a.slot;
    else
        o = (size_t)m * a.N + n;
    reinterpret_cast<T *>(a.y)[o] = from_f32<T>(r);
}

template <typename T, int MT>
__global__ __launch_bounds__(kMlpThreads) void mlp_layer_kernel(LayerArgs a)
{
    constexpr int EPL = 16 / (int)sizeof(T); // k values per lane piece
    constexpr int GK = 4 * EPL;              // k values per piece group (4 lane quarters)
    static_assert(kMlpKGrain % (GK * kMlpUnroll) == 0, "whole unrolled groups per k-slice");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = blockIdx.x, ks = blockIdx.y;
    const int n0 = nb * kMlpCols + wave * 16;
    const int kslice = a.K / a.KS, kbeg = ks * kslice;
    const int r = lane & 15, q4 = lane >> 4;

    const T *wrow = (const T *)a.w + (size_t)(n0 + r) * a.K + kbeg + EPL * q4;
    const T *xrow[MT];
    bool xin[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        xin[t] = 16 * t + r < a.M;
        xrow[t] = (const T *)a.x + (size_t)(xin[t] ? 16 * t + r : 0) * a.K + kbeg + EPL * q4;
    }
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < kslice; k += GK * kMlpUnroll) {
        uint4 bp[kMlpUnroll], ap[MT][kMlpUnroll];
#pragma unroll
        for (int u = 0; u < kMlpUnroll; ++u)
            bp[u] = *reinterpret_cast<const uint4 *>(wrow + k + u * GK);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int u = 0; u < kMlpUnroll; ++u)
                ap[t][u] = *reinterpret_cast<const uint4 *>(xrow[t] + k + u * GK);
#pragma unroll
        for (int u = 0; u < kMlpUnroll; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const uint4 av = xin[t] ? ap[t][u] : make_uint4(0u, 0u, 0u, 0u);
                if constexpr (sizeof(T) == 2) {
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bp[u]), acc[t],
                        0, 0, 0);
                } else {
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        __uint_as_float(av.x), __uint_as_float(bp[u].x), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        __uint_as_float(av.y), __uint_as_float(bp[u].y), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        __uint_as_float(av.z), __uint_as_float(bp[u].z), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        __uint_as_float(av.w), __uint_as_float(bp[u].w), acc[t], 0, 0, 0);
                }
            }
    }

    // acc[t][i] is the tile element (token 16t + 4*q4 + i, column n0 + r)
    const int n = n0 + r;
    if (a.KS == 1) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * t + 4 * q4 + i;
                if (m < a.M)
                    store_out<T>(a, m, n, acc[t][i]);
            }
        return;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * q4 + i;
            if (m < a.M)
                __hip_atomic_store(&a.part[((size_t)ks * a.M + m) * a.N + n], acc[t][i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    // The partial stores complete (vmcnt 0) before the counter moves; the
    // signal fence keeps the compiler from sinking them below it.
    __shared__ uint32_t last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&a.counters[nb], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last = old == (uint32_t)(a.KS - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (last == 0u)
        return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    float sum[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sum[t][i] = 0.f;
    // every partial of a batch of k-slices is requested before any is added
    constexpr int SB = MT == 1 ? kMlpSumBatch : kMlpSumBatch / 2;
    for (int k0 = 0; k0 < a.KS; k0 += SB) {
        float v[SB][MT][4];
#pragma unroll
        for (int b2 = 0; b2 < SB; ++b2)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 16 * t + 4 * q4 + i, k2 = k0 + b2;
                    v[b2][t][i] =
                        m < a.M && k2 < a.KS
                            ? __hip_atomic_load(&a.part[((size_t)k2 * a.M + m) * a.N + n],
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0.f;
                }
#pragma unroll
        for (int b2 = 0; b2 < SB; ++b2)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sum[t][i] += v[b2][t][i]; // k-slice order
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * q4 + i;
            if (m < a.M)
                store_out<T>(a, m, n, sum[t][i]);
        }
    if (tid == 0)
        __hip_atomic_store(&a.counters[nb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
hipError_t layer_t(const LayerArgs &a, hipStream_t st)
{
    const dim3 grid(a.N / kMlpCols, a.KS);
    switch ((a.M + 15) / 16) {
    case 1: hipLaunchKernelGGL((mlp_layer_kernel<T, 1>), grid, dim3(kMlpThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((mlp_layer_kernel<T, 2>), grid, dim3(kMlpThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((mlp_layer_kernel<T, 3>), grid, dim3(kMlpThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((mlp_layer_kernel<T, 4>), grid, dim3(kMlpThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t layer(const tb_mlp_shape &s, const LayerArgs &a, hipStream_t st)
{
    return s.dtype == TB_BF16 ? layer_t<bf16_t>(a, st) : layer_t<float>(a, st);
}

} // namespace

int mlp_k_slices(int K, int N)
{
    // enough work-groups to cover the chip twice, each k-slice a whole number
    // of kMlpKGrain values
    int ks = 1;
    while ((N / kMlpCols) * ks < 512 && K % (2 * ks * kMlpKGrain) == 0)
        ks *= 2;
    return ks;
}

MlpLayout mlp_layout(const tb_mlp_shape &s)
{
    MlpLayout L;
    const int N = s.n_slots * s.n_imp_heads * s.d_imp;
    const size_t elt = s.dtype == TB_BF16 ? 2 : 4;
    const int ks1 = mlp_k_slices(s.hidden, s.inner), ks2 = mlp_k_slices(s.inner, N);
    const size_t wide = (size_t)(s.inner > N ? s.inner : N);
    const size_t kmax = (size_t)(ks1 > ks2 ? ks1 : ks2);
    size_t off = 0;
    L.hidden = off;
    off += align_up((size_t)s.tokens * s.inner * elt);
    L.part = off;
    off += align_up(kmax * s.tokens * wide * sizeof(float));
    L.counters = off;
    off += align_up(wide / kMlpCols * sizeof(uint32_t));
    L.total = off;
    return L;
}

hipError_t launch_mlp(const tb_mlp_shape &s, const void *h, const void *w1, const void *w2,
                      void *q_imp, void *ws, hipStream_t st)
{
    const MlpLayout L = mlp_layout(s);
    char *base = (char *)ws;
    const int N = s.n_slots * s.n_imp_heads * s.d_imp;
    LayerArgs a;
    a.x = h;
    a.w = w1;
    a.y = base + L.hidden;
    a.part = (float *)(base + L.part);
    a.counters = (uint32_t *)(base + L.counters);
    a.M = s.tokens;
    a.K = s.hidden;
    a.N = s.inner;
    a.KS = mlp_k_slices(s.hidden, s.inner);
    a.slot = 0;
    a.act = s.act;
    hipError_t e = layer(s, a, st);
    if (e != hipSuccess)
        return e;
    a.x = base + L.hidden;
    a.w = w2;
    a.y = q_imp;
    a.K = s.inner;
    a.N = N;
    a.KS = mlp_k_slices(s.inner, N);
    a.slot = s.n_imp_heads * s.d_imp;
    a.act = -1;
    return layer(s, a, st);
}

} // namespace tb
