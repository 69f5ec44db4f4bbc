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
// Each layer is one launch: one work-group per 16 output columns, one wave
// per k-slice (K / 256 slices, at most 16 waves; a wave takes the 256-value
// chunks w, w + waves, ...).  A wave multiplies its slice with MFMA 16x16
// tiles, one accumulator tile per 16 tokens: lane l supplies token / column
// l % 16 and the l / 16-th quarter of each k group from one 16-byte piece
// (bf16: one 16x16x32 step per piece; fp32: four 16x16x4 steps per piece).
// Token rows past M read as zero.  The waves' fp32 tiles meet in LDS and
// are summed in slice order -- no partials leave the work-group, and the
// result does not depend on timing -- then activated, rounded to the dtype
// and written.  One token (a decode step) is a matrix-vector product: there
// each wave takes R weight rows and reads them in whole 1 KB pieces (one
// 16-byte piece per lane, every load coalesced), the token's matching pieces
// in registers, an fp32 fma chain per lane in piece order and a wave sum per
// row.
#include "tb_internal.h"

namespace tb {
namespace {

constexpr int kMlpCols = 16;     // output columns per work-group (one MFMA tile)
constexpr int kMlpMaxWaves = 16; // k-slices per work-group
// 16-byte pieces per lane requested together (fewer with more token tiles,
// whose pieces take more registers)
template <int MT> constexpr int mlp_unroll() { return MT >= 4 ? 2 : MT >= 3 ? 4 : 8; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct LayerArgs {
    const void *x;      // [M][K]
    const void *w;      // [N][K]
    void *y;            // [M][N], or slot-major [N / slot][M][slot]
    int M, K, N;
    int slot;           // columns per slot of a slot-major output (0: row-major)
    int act;            // TB_ACT_RELU / TB_ACT_SILU, or -1 for none
    int splits;         // work-groups per column tile, each K / splits of the sum
    f32x4 *part;        // their partial tiles (splits > 1)
    uint32_t *counters; // one arrival counter per column tile, kept zero
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
__global__ __launch_bounds__(64 * kMlpMaxWaves) void mlp_layer_kernel(LayerArgs a)
{
    constexpr int EPL = 16 / (int)sizeof(T); // k values per lane piece
    constexpr int GK = 4 * EPL;              // k values per piece group (4 lane quarters)
    constexpr int UNR = mlp_unroll<MT>();
    constexpr int CHUNK = GK * UNR;          // k values per wave iteration
    static_assert(kMlpKGrain % CHUNK == 0, "whole iterations per 256-value chunk");
    extern __shared__ f32x4 tiles[];         // [waves][MT][64]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = (int)blockDim.x / 64;
    const int tile = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
    const int n0 = tile * kMlpCols;
    const int kbeg = split * (a.K / a.splits), kend = kbeg + a.K / a.splits;
    const int r = lane & 15, q4 = lane >> 4;

    const T *wrow = (const T *)a.w + (size_t)(n0 + r) * a.K + EPL * q4;
    const T *xrow[MT];
    bool xin[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        xin[t] = 16 * t + r < a.M;
        xrow[t] = (const T *)a.x + (size_t)(xin[t] ? 16 * t + r : 0) * a.K + EPL * q4;
    }
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this wave's slice of the work-group's k range: 256-value chunks wave,
    // wave + nwaves, ...
    for (int k0 = kbeg + wave * kMlpKGrain; k0 < kend; k0 += nwaves * kMlpKGrain) {
        for (int k = k0; k < k0 + kMlpKGrain; k += CHUNK) {
            uint4 bp[UNR], ap[MT][UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u)
                bp[u] = *reinterpret_cast<const uint4 *>(wrow + k + u * GK);
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int u = 0; u < UNR; ++u)
                    ap[t][u] = *reinterpret_cast<const uint4 *>(xrow[t] + k + u * GK);
#pragma unroll
            for (int u = 0; u < UNR; ++u)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const uint4 av = xin[t] ? ap[t][u] : make_uint4(0u, 0u, 0u, 0u);
                    if constexpr (sizeof(T) == 2) {
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bp[u]),
                            acc[t], 0, 0, 0);
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
    }

    // acc[t][i] is the slice's tile element (token 16t + 4*q4 + i, column
    // n0 + r); the slices are summed in order by wave 0
#pragma unroll
    for (int t = 0; t < MT; ++t)
        tiles[(wave * MT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wave != 0)
        return;
    const int n = n0 + r;
    f32x4 sum[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        sum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nwaves; ++w)
            sum[t] += tiles[(w * MT + t) * 64 + lane];
    }
    if (a.splits > 1) {
        // Split over k: the work-group publishes its partial tiles with
        // device-coherent stores and, once they are complete, counts its
        // arrival; the last of the tile's work-groups adds the partials in
        // split order (the sum does not depend on arrival order) and
        // finishes the tile.  Same ordering argument as the attention's
        // cross-chunk merge; the last arriver resets the counter.
        f32x4 *mine = a.part + ((size_t)(tile * a.splits + split) * MT) * 64;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; i += 2)
                store2_agent(reinterpret_cast<float *>(&mine[t * 64 + lane]) + i, sum[t][i],
                             sum[t][i + 1]);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        uint32_t old = 0u;
        if (lane == 0)
            old = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old != (uint32_t)(a.splits - 1))
            return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0)
            __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        const f32x4 *parts = a.part + ((size_t)tile * a.splits * MT) * 64;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            f32x4 acc4 = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int sp = 0; sp < a.splits; ++sp) {
                const float4 v = load4_agent(
                    reinterpret_cast<const float *>(&parts[(sp * MT + t) * 64 + lane]));
                acc4 += f32x4{v.x, v.y, v.z, v.w};
            }
            sum[t] = acc4;
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * q4 + i;
            if (m < a.M)
                store_out<T>(a, m, n, sum[t][i]);
        }
}

// One token: wave v of the work-group owns weight rows R * (4 * blockIdx.x
// + v) .. + R - 1; NCH = K / (64 * 16 / sizeof(T)) pieces per row.
constexpr int kGemvWaves = 4;
template <typename T, int NCH, int R>
__global__ __launch_bounds__(64 * kGemvWaves) void gemv_kernel(LayerArgs a)
{
    constexpr int EPL = 16 / (int)sizeof(T);
    constexpr int KC = 64 * EPL; // k values per piece (a whole wave)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row0 = R * (kGemvWaves * blockIdx.x + wave);
    const T *xb = (const T *)a.x + EPL * lane;
    const T *wb = (const T *)a.w + (size_t)row0 * a.K + EPL * lane;
    uint4 xp[NCH], wp[R][NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        xp[c] = *reinterpret_cast<const uint4 *>(xb + c * KC);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            wp[r][c] = *reinterpret_cast<const uint4 *>(wb + (size_t)r * a.K + c * KC);
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            T xv[EPL], wv[EPL];
            __builtin_memcpy(xv, &xp[c], 16);
            __builtin_memcpy(wv, &wp[r][c], 16);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[r] = fmaf(to_f32(xv[e]), to_f32(wv[e]), acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float v = wave_sum(acc[r]);
        if (lane == r)
            store_out<T>(a, 0, row0 + r, v);
    }
}

template <typename T, int NCH>
hipError_t gemv_r(const LayerArgs &a, hipStream_t st)
{
    // about 256 work-groups: R rows per wave
    const int R = a.N >= 4 * 1024 ? 4 : a.N >= 2 * 1024 ? 2 : 1;
    const dim3 grid(a.N / (kGemvWaves * R)), block(64 * kGemvWaves);
    if (R == 4)
        hipLaunchKernelGGL((gemv_kernel<T, NCH, 4>), grid, block, 0, st, a);
    else if (R == 2)
        hipLaunchKernelGGL((gemv_kernel<T, NCH, 2>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((gemv_kernel<T, NCH, 1>), grid, block, 0, st, a);
    return hipGetLastError();
}

// The one-token path, when K is a power-of-two number of whole pieces (at
// most 16); otherwise hipErrorNotSupported and the MFMA path runs.
template <typename T>
hipError_t gemv_t(const LayerArgs &a, hipStream_t st)
{
    constexpr int KC = 64 * 16 / (int)sizeof(T);
    if (a.M != 1 || a.K % KC != 0 || a.N % (kGemvWaves * 4) != 0)
        return hipErrorNotSupported;
    switch (a.K / KC) {
    case 1: return gemv_r<T, 1>(a, st);
    case 2: return gemv_r<T, 2>(a, st);
    case 4: return gemv_r<T, 4>(a, st);
    case 8: return gemv_r<T, 8>(a, st);
    case 16: return gemv_r<T, 16>(a, st);
    }
    return hipErrorNotSupported;
}

template <typename T>
hipError_t layer_t(const LayerArgs &a, hipStream_t st)
{
    const hipError_t g = gemv_t<T>(a, st);
    if (g != hipErrorNotSupported)
        return g;
    const int chunks = a.K / kMlpKGrain / a.splits;
    const int waves = chunks < kMlpMaxWaves ? chunks : kMlpMaxWaves;
    const dim3 grid(a.N / kMlpCols * a.splits);
    const int mt = (a.M + 15) / 16;
    const size_t lds = (size_t)waves * mt * 64 * sizeof(f32x4);
    switch (mt) {
    case 1: hipLaunchKernelGGL((mlp_layer_kernel<T, 1>), grid, dim3(64 * waves), lds, st, a); break;
    case 2: hipLaunchKernelGGL((mlp_layer_kernel<T, 2>), grid, dim3(64 * waves), lds, st, a); break;
    case 3: hipLaunchKernelGGL((mlp_layer_kernel<T, 3>), grid, dim3(64 * waves), lds, st, a); break;
    case 4: hipLaunchKernelGGL((mlp_layer_kernel<T, 4>), grid, dim3(64 * waves), lds, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t layer(const tb_mlp_shape &s, const LayerArgs &a, hipStream_t st)
{
    return s.dtype == TB_BF16 ? layer_t<bf16_t>(a, st) : layer_t<float>(a, st);
}

} // namespace

MlpLayout mlp_layout(const tb_mlp_shape &s)
{
    MlpLayout L;
    const size_t elt = s.dtype == TB_BF16 ? 2 : 4;
    const int N = s.n_slots * s.n_imp_heads * s.d_imp;
    const int mt = (s.tokens + 15) / 16;
    // partial tiles and counters for whichever layer is split the most
    size_t part = 0, tiles = 0;
    const int dims[2][2] = {{s.inner, s.hidden}, {N, s.inner}};
    for (const auto &nk : dims) {
        const int sp = mlp_splits(nk[0], nk[1]);
        const size_t t = (size_t)(nk[0] / 16);
        if (sp > 1) {
            part = part > t * sp ? part : t * sp;
            tiles = tiles > t ? tiles : t;
        }
    }
    L.hidden = 0;
    size_t off = align_up((size_t)s.tokens * s.inner * elt);
    L.part = off;
    off += align_up(part * mt * 64 * sizeof(f32x4));
    L.counters = off;
    off += align_up(tiles * sizeof(uint32_t));
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
    a.M = s.tokens;
    a.K = s.hidden;
    a.N = s.inner;
    a.slot = 0;
    a.act = s.act;
    a.part = (f32x4 *)(base + L.part);
    a.counters = (uint32_t *)(base + L.counters);
    a.splits = s.tokens > 1 ? mlp_splits(a.N, a.K) : 1;
    hipError_t e = layer(s, a, st);
    if (e != hipSuccess)
        return e;
    a.x = base + L.hidden;
    a.w = w2;
    a.y = q_imp;
    a.K = s.inner;
    a.N = N;
    a.slot = s.n_imp_heads * s.d_imp;
    a.act = -1;
    a.splits = s.tokens > 1 ? mlp_splits(a.N, a.K) : 1;
    return layer(s, a, st);
}

} // namespace tb
