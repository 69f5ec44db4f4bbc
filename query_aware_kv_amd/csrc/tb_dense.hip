// tb_dense.hip -- dense decode attention over the whole context (gfx950).
//
// The comparator of the sparse step: TokenButler's speedups are stated
// against dense attention (gist.science technical summary, Key
// Contributions > Efficiency Gains and Experimental Results > Latency).
// For query head h of sequence b with n = ctx_len[b] tokens,
//   out[b][h] = sum_{t < n} softmax_t(scale * q[b][h] . K[b][g(h)][t]) V[b][g(h)][t].
//
// Grid: (chunk of kDenseChunk positions, KV head, sequence); 512 threads.
// Every K/V row is read once and serves all GQ query heads of its KV head:
//   1. Wave w streams positions [c0 + w*P, c0 + (w+1)*P) of the chunk,
//      D*elt/16 lanes per row (16-byte pieces), 64/(lanes per row) rows side
//      by side; two batches of row steps alternate so that one is in flight
//      while the other is used.  Each row slot keeps one online softmax per
//      query head in base 2, updated once per batch: all the batch's logits
//      (v_dot2 on bf16 pairs, DPP row reductions), then one max update and
//      rescale per head, then the weights -- no branches, so the query
//      heads' dependency chains interleave.
//   2. The row slots of a wave merge by lane exchanges (DPP and the
//      permlane swaps, no LDS), the waves through LDS, into one partial
//      (max, sum, acc[D]) per query head and chunk.
//   3. The partials are merged across chunks by the last work-group of the
//      (sequence, KV head) to arrive, as in the sparse kernel.
#include "tb_attn_common.h"

namespace tb {
namespace {

constexpr int kDenseThreads = 512;
constexpr int kDenseWaves = kDenseThreads / 64;
constexpr int kMaxDenseChunks = kMaxCtxCap / kDenseChunk;

struct DenseArgs {
    const void *q, *k, *v;
    const int32_t *ctx_len;
    int Hq, Hkv, cap;
    float qscale;      // softmax scale * log2(e)
    float *part_o;     // [b*Hq][nchunk][D]
    float *part_ml;    // [b*Hq][nchunk][2]
    uint32_t *counters;
    void *out;
};

template <typename T, int D, int GQ>
__global__ __launch_bounds__(kDenseThreads) void dense_kernel(DenseArgs a)
{
    constexpr int EPL = 16 / (int)sizeof(T); // elements per lane piece
    constexpr int LPR = D / EPL;             // lanes per row
    constexpr int RPW = 64 / LPR;            // row slots per wave
    // row steps per batch (two batches in flight); fewer for wide groups,
    // whose accumulators take more registers
    constexpr int kDenseRows = GQ >= 8 ? 2 : 4;
    constexpr int PW = kDenseChunk / kDenseWaves;
    constexpr int STEP = kDenseRows * RPW;   // positions per wave iteration
    static_assert(PW % STEP == 0, "whole iterations per wave");
    static_assert((GQ * D) % 64 == 0, "whole waves in the partial loop (lane pairs)");

    __shared__ float wm[GQ][kDenseWaves];
    __shared__ float wl[GQ][kDenseWaves];
    __shared__ float wacc[GQ][kDenseWaves][D];
    __shared__ CombineLds<GQ, kDenseThreads, kMaxDenseChunks> cmb;

    const T *__restrict__ q = (const T *)a.q;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int nchunk = gridDim.x;
    const int c0 = c * kDenseChunk;
    const size_t head0 = (size_t)b * a.Hq + (size_t)g * GQ;
    const int slot = lane / LPR, sub = lane % LPR;

    const int p0 = c0 + wave * PW;
    const size_t kvbase = ((size_t)b * a.Hkv + g) * a.cap;
    const T *kb = (const T *)a.k + kvbase * D + sub * EPL;
    const T *vb = (const T *)a.v + kvbase * D + sub * EPL;
    auto load_rows = [&](int base, int p1, uint4 (&kk)[kDenseRows], uint4 (&vv)[kDenseRows],
                         bool (&ok)[kDenseRows]) {
#pragma unroll
        for (int r = 0; r < kDenseRows; ++r) {
            const int pos = base + r * RPW + slot;
            ok[r] = pos < p1;
            const size_t pr = (size_t)(ok[r] ? pos : c0) * D;
            kk[r] = *reinterpret_cast<const uint4 *>(kb + pr);
            vv[r] = *reinterpret_cast<const uint4 *>(vb + pr);
        }
    };
    // Requested before the context length is known: this lane's q pieces of
    // every query head of the group (storage type) and the wave's first rows
    // (positions below the capacity; the ones at or past n get no weight).
    uint4 qh[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
        qh[h] = *reinterpret_cast<const uint4 *>(q + (head0 + h) * D + sub * EPL);
    uint4 ka[kDenseRows], va[kDenseRows], kb2[kDenseRows], vb2[kDenseRows];
    bool oa[kDenseRows], ob[kDenseRows];
    load_rows(p0, min(p0 + PW, a.cap), ka, va, oa);
    const int n = clamp_len(a.ctx_len[b], a.cap);
    const bool active = c0 < n;

    if (active) {
        // ---- 1. stream this wave's rows ----
        const int p1 = min(p0 + PW, n);
#pragma unroll
        for (int r = 0; r < kDenseRows; ++r)
            oa[r] = oa[r] && p0 + r * RPW + slot < p1;
        float m[GQ], l[GQ], acc[GQ][EPL];
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[h][e] = 0.f;
        }
        // The loop is uniform over the wave.  Loads are unconditional: a
        // position past the end reads the chunk's first row (which exists)
        // and gets no weight.  Two batches of rows alternate, so one batch
        // is in flight while the other is used.
        // One batch at a time: every logit first (the query heads' chains
        // interleave), then one max update and rescale per head, then the
        // weights and the V accumulation, all without branches.
        auto use_rows = [&](const uint4 (&kk)[kDenseRows], const uint4 (&vv)[kDenseRows],
                            const bool (&ok)[kDenseRows]) {
            float z[kDenseRows][GQ];
#pragma unroll
            for (int r = 0; r < kDenseRows; ++r)
#pragma unroll
                for (int h = 0; h < GQ; ++h)
                    z[r][h] = lane_dot<T>(qh[h], kk[r]);
#pragma unroll
            for (int r = 0; r < kDenseRows; ++r)
#pragma unroll
                for (int h = 0; h < GQ; ++h)
                    z[r][h] = group_sum<LPR>(z[r][h]) * a.qscale;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float mb = m[h];
#pragma unroll
                for (int r = 0; r < kDenseRows; ++r)
                    mb = ok[r] ? fmaxf(mb, z[r][h]) : mb;
                // unchanged max (also -inf before any row): no rescale
                const float corr = mb == m[h] ? 1.f : __builtin_amdgcn_exp2f(m[h] - mb);
                l[h] *= corr;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[h][e] *= corr;
                m[h] = mb;
            }
#pragma unroll
            for (int r = 0; r < kDenseRows; ++r) {
                T vt[EPL];
                __builtin_memcpy(vt, &vv[r], 16);
                float vf[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    vf[e] = to_f32(vt[e]);
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    const float pr = ok[r] ? __builtin_amdgcn_exp2f(z[r][h] - m[h]) : 0.f;
                    l[h] += pr;
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
                }
            }
        };
        // The prefetch past the end is unconditional (it reads the chunk's
        // first row again): a conditional load would make the compiler wait
        // for every load in flight at the loop head.
        for (int base = p0; base < p1; base += 2 * STEP) {
            load_rows(base + STEP, p1, kb2, vb2, ob);
            use_rows(ka, va, oa);
            load_rows(base + 2 * STEP, p1, ka, va, oa);
            use_rows(kb2, vb2, ob);
        }

        // ---- 2a. merge the wave's row slots (lanes sub, sub+LPR, ...) ----
        auto fmax2 = [](float x, float y) { return fmaxf(x, y); };
        auto add2 = [](float x, float y) { return x + y; };
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float M = across_slots<LPR>(m[h], fmax2);
            const float f = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - M);
            const float L = across_slots<LPR>(l[h] * f, add2);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[h][e] = across_slots<LPR>(acc[h][e] * f, add2);
            if (slot == 0) {
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    wacc[h][wave][sub * EPL + e] = acc[h][e];
                if (sub == 0) {
                    wm[h][wave] = M;
                    wl[h][wave] = L;
                }
            }
        }
    }
    __syncthreads();
    if (active) {
        // ---- 2b. merge the waves: one thread per (query head, dimension) ----
        for (int pi = tid; pi < GQ * D; pi += kDenseThreads) {
            const int h = pi / D, dim = pi % D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kDenseWaves; ++w)
                M = fmaxf(M, wm[h][w]);
            float O = 0.f, L = 0.f;
#pragma unroll
            for (int w = 0; w < kDenseWaves; ++w) {
                const float mw = wm[h][w];
                const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
                O = fmaf(wacc[h][w][dim], f, O);
                L = fmaf(wl[h][w], f, L);
            }
            publish_partial<D>(a.part_o, a.part_ml, (head0 + h) * nchunk + c, dim, O, M, L);
        }
    }

    // ---- 3. arrival; the last work-group of this (b, g) merges the chunks ----
    arrive_and_combine<T, D, GQ, kDenseThreads, kMaxDenseChunks>(
        cmb, &a.counters[(size_t)b * a.Hkv + g], a.part_o, a.part_ml, nchunk,
        (n + kDenseChunk - 1) / kDenseChunk, head0, (T *)a.out);
}

template <typename T, int D, int GQ>
hipError_t dense_t(const tb_shape &s, const DenseArgs &a, hipStream_t st)
{
    dim3 grid(dense_chunks(s.ctx_cap), s.n_kv_heads, s.batch);
    hipLaunchKernelGGL((dense_kernel<T, D, GQ>), grid, dim3(kDenseThreads), 0, st, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t dense_gq(const tb_shape &s, const DenseArgs &a, hipStream_t st)
{
    switch (s.n_q_heads / s.n_kv_heads) {
    case 1: return dense_t<T, D, 1>(s, a, st);
    case 2: return dense_t<T, D, 2>(s, a, st);
    case 4: return dense_t<T, D, 4>(s, a, st);
    case 8: return dense_t<T, D, 8>(s, a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_dense(const tb_shape &s, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *ctx_len, float softmax_scale,
                        void *out, float *part_o, float *part_ml, uint32_t *counters,
                        hipStream_t st)
{
    DenseArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.ctx_len = ctx_len;
    a.Hq = s.n_q_heads;
    a.Hkv = s.n_kv_heads;
    a.cap = s.ctx_cap;
    a.qscale = softmax_scale * 1.4426950408889634f; // logits in base 2
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.counters = counters;
    a.out = out;
    if (s.dtype == TB_BF16) {
        if (s.head_dim == 64) return dense_gq<bf16_t, 64>(s, a, st);
        if (s.head_dim == 128) return dense_gq<bf16_t, 128>(s, a, st);
    } else {
        if (s.head_dim == 64) return dense_gq<float, 64>(s, a, st);
        if (s.head_dim == 128) return dense_gq<float, 128>(s, a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace tb
