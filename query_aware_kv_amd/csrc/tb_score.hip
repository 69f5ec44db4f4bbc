// tb_score.hip -- importance scores, with the append of new tokens folded in
// (gfx950).
//
// TokenButler (gist.science technical summary, Methodology > Core
// Architecture): each predicted low-dimensional importance query is dotted
// with the projected keys of its KV head to score every cached token.
// Inference Strategy > Optimizations: the projected-key cache is extended as
// tokens arrive.
//
// One streaming pass over the projected-key cache: a lane owns one token of
// one KV head, reads its d projected-key values (d*elt bytes, contiguous) in
// 16-byte loads, and produces the scores of all importance heads that read
// this KV head.  The importance queries are wave-uniform and come through the
// scalar cache.
//
// Precision contract: a score is the fp32 fused multiply-add chain over the
// d coordinates in ascending order, starting from +0; this fp32 value is the
// selection key.  The fused step stores the two 16-bit halves of its
// order-preserving key in two arrays instead of the fp32 value (and the top
// half again, compactly, for positions 8m): the selection classifies
// positions from the top halves alone and completes only its candidates'
// keys.
//
// Where the grid runs in several rounds of work-groups per compute unit, each
// wave of the fused step stages its positions' split keys in LDS and writes
// them as 16-byte pieces, one store instruction per wave instead of two
// 2-byte ones per importance head and lane.
//
// When the call also appends tokens, one extra work-group per (sequence, KV
// head) -- the first one dispatched -- writes the new K/V rows into the
// caches, projects their keys (fp64 sum in ascending head_dim order, rounded
// once to the dtype) and scores them; the streaming work-groups skip those
// positions, so no work-group waits for another.
#include "tb_internal.h"

namespace tb {
namespace {

constexpr int kScoreThreads = 512;
constexpr int kMaxFusedNew = 8; // appended rows handled inside the score launch
static_assert(kMaxFusedNew * 32 <= kScoreThreads, "one 16-byte piece of a new row per thread");

struct ScoreArgs {
    const void *q_imp;  // [b][Himp][d]
    void *kp;           // [b][Hkv][cap][d]
    const int32_t *ctx_len;
    float *scores;      // [b][Himp][cap]
    int Himp, Hkv, cap, batch, ntiles;
    // append (n_new == 0: none)
    int n_new;
    const void *k_new, *v_new; // [b][Hkv][n_new][D]
    const void *w;             // [D][d]
    void *k_cache, *v_cache;
    uint16_t *keys16;   // [b][Himp][k16s] top 16 key bits of every score (pair order), or NULL
    uint16_t *keys16lo; // [b][Himp][k16s] the low 16 key bits, the same order
    uint16_t *sample16; // [b][Himp][s16] the same for positions 8m
    int s16, k16s;
    int wide;           // score_kernel<..., true>: split keys of whole waves through LDS
};

// Stores the score of (row, t): the fp32 value, or the two 16-bit halves of
// its order-preserving key (and the top half again for positions 8m).
__device__ __forceinline__ void put_score(const ScoreArgs &a, size_t row, int t, float v)
{
    if (a.keys16 != nullptr) {
        const uint32_t key = score_key(v);
        const size_t e = row * a.k16s + keys16_entry(t);
        a.keys16[e] = (uint16_t)(key >> 16);
        a.keys16lo[e] = (uint16_t)(key & 0xFFFFu);
        if ((t & 7) == 0)
            a.sample16[row * a.s16 + (t >> 3)] = (uint16_t)(key >> 16);
    } else {
        a.scores[row * a.cap + t] = v;
    }
}

// The group's importance queries, requested in 16-byte pieces before any
// score is stored (the stores could alias them for all the compiler knows,
// which would otherwise serialise one load round trip per piece).
template <typename T, int DI, int GI>
__device__ __forceinline__ void load_queries(const ScoreArgs &a, int b, int g,
                                             uint4 (&qv)[GI][DI * sizeof(T) / 16])
{
    const uint4 *qb = reinterpret_cast<const uint4 *>(
        (const T *)a.q_imp + ((size_t)b * a.Himp + (size_t)g * GI) * DI);
#pragma unroll
    for (int hh = 0; hh < GI; ++hh)
#pragma unroll
        for (int p = 0; p < DI * (int)sizeof(T) / 16; ++p)
            qv[hh][p] = qb[hh * (DI * sizeof(T) / 16) + p];
}

template <typename T, int DI, int GI>
__device__ __forceinline__ void score_acc(const float (&k)[DI],
                                          const uint4 (&qv)[GI][DI * sizeof(T) / 16],
                                          float (&acc)[GI])
{
    constexpr int EPC = 16 / sizeof(T);
#pragma unroll
    for (int hh = 0; hh < GI; ++hh) {
        acc[hh] = 0.f;
#pragma unroll
        for (int p = 0; p < DI / EPC; ++p) {
            T q[EPC];
            __builtin_memcpy(q, &qv[hh][p], 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                acc[hh] = fmaf(to_f32(q[e]), k[p * EPC + e], acc[hh]);
        }
    }
}

// The split keys of a wave's 64 positions t0w .. t0w + 63, all of them below
// the appended rows: staged in LDS in pair order, then stored as 16-byte
// pieces -- one store instruction for the 2 * GI lines of 64 entries (128
// bytes each) instead of 2 * GI two-byte ones per lane -- and the sample's
// 8 entries per head as one more.  Same values and addresses as put_score.
template <int GI>
__device__ __forceinline__ void put_keys_wave(const ScoreArgs &a, size_t row0, int t0w, int lane,
                                              const float (&acc)[GI],
                                              uint16_t (&stg)[2 * GI][64])
{
    const int e = keys16_entry(lane); // the entry of position t0w + lane
#pragma unroll
    for (int hh = 0; hh < GI; ++hh) {
        const uint32_t key = score_key(acc[hh]);
        stg[2 * hh][e] = (uint16_t)(key >> 16);
        stg[2 * hh + 1][e] = (uint16_t)(key & 0xFFFFu);
    }
    wave_lds_sync();
#pragma unroll
    for (int idx = lane; idx < 16 * GI; idx += 64) {
        const int line = idx >> 3, q = idx & 7;
        const uint4 v = *reinterpret_cast<const uint4 *>(&stg[line][8 * q]);
        uint16_t *arr = (line & 1) ? a.keys16lo : a.keys16;
        *reinterpret_cast<uint4 *>(arr + (row0 + (line >> 1)) * a.k16s + t0w + 8 * q) = v;
    }
    if (lane < GI) {
        uint32_t s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[i] = (uint32_t)stg[2 * lane][keys16_entry(16 * i)] |
                   ((uint32_t)stg[2 * lane][keys16_entry(16 * i + 8)] << 16);
        *reinterpret_cast<uint4 *>(a.sample16 + (row0 + lane) * a.s16 + (t0w >> 3)) =
            make_uint4(s[0], s[1], s[2], s[3]);
    }
}

template <typename T, int D, int DI, int GI, bool WIDE>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a)
{
    // 1-D grid.  With appended rows the first batch*Hkv work-groups (the
    // first dispatched, so their serial chains start early) are the append
    // work-groups of each (b, g); the streaming tiles follow, tile-fastest.
    const int napp = a.n_new > 0 ? a.batch * a.Hkv : 0;
    const int id = blockIdx.x;
    const bool is_append = id < napp;
    const int sid = is_append ? id : id - napp;
    const int bg = is_append ? sid : sid / a.ntiles;
    const int tile = is_append ? 0 : sid % a.ntiles;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int n = clamp_len(a.ctx_len[b], a.cap);
    const int nfresh = a.n_new < n ? a.n_new : n; // appended rows present in [0, n)
    const int t_new = n - nfresh;                  // first appended position

    if (is_append) {
        // ---- append work-group: copy, project and score the new rows ----
        __shared__ float sW[D * DI];
        __shared__ float sK[kMaxFusedNew][D];
        if (nfresh == 0)
            return;
        // W and the new K rows arrive in 16-byte pieces, all loads issued
        // before any is used
        constexpr int EPC = 16 / sizeof(T);
        constexpr int WP = D * DI / EPC; // pieces of W
        constexpr int WPT = (WP + kScoreThreads - 1) / kScoreThreads;
        uint4 wp[WPT];
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            const int pi = threadIdx.x + q * kScoreThreads;
            wp[q] = reinterpret_cast<const uint4 *>(a.w)[pi < WP ? pi : 0];
        }
        const size_t src0 = ((size_t)b * a.Hkv + g) * a.n_new + (a.n_new - nfresh);
        const size_t dst0 = ((size_t)b * a.Hkv + g) * a.cap + t_new;
        constexpr int RP = D / EPC; // pieces per row
        const int npc = nfresh * RP;
        uint4 kpc = make_uint4(0, 0, 0, 0), vpc = make_uint4(0, 0, 0, 0);
        const int e0 = threadIdx.x < npc ? (int)threadIdx.x : 0;
        kpc = reinterpret_cast<const uint4 *>((const T *)a.k_new + src0 * D)[e0];
        vpc = reinterpret_cast<const uint4 *>((const T *)a.v_new + src0 * D)[e0];
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            const int pi = threadIdx.x + q * kScoreThreads;
            if (pi < WP) {
                T v[EPC];
                __builtin_memcpy(v, &wp[q], 16);
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    sW[pi * EPC + e] = to_f32(v[e]);
            }
        }
        if ((int)threadIdx.x < npc) {
            const int r = threadIdx.x / RP, i0 = (threadIdx.x % RP) * EPC;
            reinterpret_cast<uint4 *>((T *)a.k_cache + (dst0 + r) * D)[threadIdx.x % RP] = kpc;
            reinterpret_cast<uint4 *>((T *)a.v_cache + (dst0 + r) * D)[threadIdx.x % RP] = vpc;
            T v[EPC];
            __builtin_memcpy(v, &kpc, 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                sK[r][i0 + e] = to_f32(v[e]);
        }
        __syncthreads();
        __shared__ float sKp[kMaxFusedNew][DI];
        for (int e = threadIdx.x; e < nfresh * DI; e += kScoreThreads) {
            const int r = e / DI, j = e % DI;
            double acc = 0.0;
#pragma unroll 8
            for (int i = 0; i < D; ++i)
                acc = fma((double)sK[r][i], (double)sW[i * DI + j], acc);
            const T kp = from_f64<T>(acc);
            ((T *)a.kp)[(dst0 + r) * DI + j] = kp;
            sKp[r][j] = to_f32(kp);
        }
        __syncthreads();
        if ((int)threadIdx.x < nfresh * GI) {
            // one thread per (new row, importance head)
            const int r = threadIdx.x / GI, hh = threadIdx.x % GI;
            const T *qh = (const T *)a.q_imp + ((size_t)b * a.Himp + (size_t)g * GI + hh) * DI;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < DI; ++j)
                acc = fmaf(to_f32(qh[j]), sKp[r][j], acc);
            put_score(a, (size_t)b * a.Himp + (size_t)g * GI + hh, t_new + r, acc);
        }
        return;
    }

    // ---- streaming work-group: positions [t0, t0 + kScoreThreads) below t_new ----
    const int t0 = tile * kScoreThreads;
    if (t0 >= t_new)
        return;
    const int t = t0 + threadIdx.x;
    const bool valid = t < t_new;

    constexpr int EPC = 16 / sizeof(T);
    uint4 qv[GI][DI * sizeof(T) / 16];
    load_queries<T, DI, GI>(a, b, g, qv);
    float k[DI];
    {
        const T *row = (const T *)a.kp + (((size_t)b * a.Hkv + g) * a.cap + (valid ? t : t0)) * DI;
#pragma unroll
        for (int p = 0; p < DI / EPC; ++p) {
            const uint4 piece = reinterpret_cast<const uint4 *>(row)[p];
            T v[EPC];
            __builtin_memcpy(v, &piece, 16);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                k[p * EPC + e] = to_f32(v[e]);
        }
    }
    float acc[GI];
    score_acc<T, DI, GI>(k, qv, acc);
    const size_t row0 = (size_t)b * a.Himp + (size_t)g * GI;
    if constexpr (WIDE) {
        const int lane = threadIdx.x & 63;
        const int t0w = t - lane; // the wave's first position
        __shared__ __align__(16) uint16_t stg[kScoreThreads / 64][2 * GI][64];
        if (t0w + 64 <= t_new) {
            put_keys_wave<GI>(a, row0, t0w, lane, acc, stg[threadIdx.x >> 6]);
            return;
        }
    }
    if (valid) {
#pragma unroll
        for (int hh = 0; hh < GI; ++hh)
            put_score(a, row0 + hh, t, acc[hh]);
    }
}

template <typename T, int D, int DI, int GI>
hipError_t score_t(const tb_shape &s, const ScoreArgs &a, hipStream_t st)
{
    const int bg = s.batch * s.n_kv_heads;
    dim3 grid((a.n_new > 0 ? bg : 0) + a.ntiles * bg);
    if (a.wide)
        hipLaunchKernelGGL((score_kernel<T, D, DI, GI, true>), grid, dim3(kScoreThreads), 0, st, a);
    else
        hipLaunchKernelGGL((score_kernel<T, D, DI, GI, false>), grid, dim3(kScoreThreads), 0, st, a);
    return hipGetLastError();
}

template <typename T, int D, int DI>
hipError_t score_gi(const tb_shape &s, const ScoreArgs &a, hipStream_t st)
{
    switch (s.n_imp_heads / s.n_kv_heads) {
    case 1: return score_t<T, D, DI, 1>(s, a, st);
    case 2: return score_t<T, D, DI, 2>(s, a, st);
    case 4: return score_t<T, D, DI, 4>(s, a, st);
    case 8: return score_t<T, D, DI, 8>(s, a, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t score_dtype(const tb_shape &s, const ScoreArgs &a, hipStream_t st)
{
    if (s.head_dim == 64 && s.d_imp == 16) return score_gi<T, 64, 16>(s, a, st);
    if (s.head_dim == 64 && s.d_imp == 32) return score_gi<T, 64, 32>(s, a, st);
    if (s.head_dim == 128 && s.d_imp == 16) return score_gi<T, 128, 16>(s, a, st);
    if (s.head_dim == 128 && s.d_imp == 32) return score_gi<T, 128, 32>(s, a, st);
    return hipErrorInvalidValue;
}

} // namespace

int score_max_fused_new() { return kMaxFusedNew; }

hipError_t launch_score(const tb_shape &s, const void *q_imp, void *kp_cache,
                        const int32_t *ctx_len, float *scores, int n_new, const void *k_new,
                        const void *v_new, const void *w, void *k_cache, void *v_cache,
                        uint16_t *keys16, uint16_t *keys16lo, uint16_t *sample16,
                        hipStream_t st)
{
    ScoreArgs a;
    a.q_imp = q_imp;
    a.kp = kp_cache;
    a.ctx_len = ctx_len;
    a.scores = scores;
    a.Himp = s.n_imp_heads;
    a.Hkv = s.n_kv_heads;
    a.cap = s.ctx_cap;
    a.batch = s.batch;
    a.ntiles = (s.ctx_cap + kScoreThreads - 1) / kScoreThreads;
    a.n_new = n_new;
    a.k_new = k_new;
    a.v_new = v_new;
    a.w = w;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.keys16 = keys16;
    a.keys16lo = keys16lo;
    a.sample16 = sample16;
    a.s16 = sample16_stride(s.ctx_cap);
    a.k16s = keys16_stride(s.ctx_cap);
    // The 16-byte key stores pay where the grid runs in several rounds of
    // work-groups per compute unit (a round's writes then overlap the next
    // round's loads: 128K context 74.3 -> 72.4 us per step); a grid of one
    // round (32K context, 512 tiles) drains its writes at the end either
    // way, and the staging only adds to it (32.2 -> 32.4 us).
    int cus = 0;
    const hipError_t ce = device_cus(cus);
    if (ce != hipSuccess)
        return ce;
    a.wide = keys16 != nullptr && (long)a.ntiles * s.batch * s.n_kv_heads > 2L * cus;
    if (s.dtype == TB_BF16)
        return score_dtype<bf16_t>(s, a, st);
    return score_dtype<float>(s, a, st);
}

} // namespace tb
