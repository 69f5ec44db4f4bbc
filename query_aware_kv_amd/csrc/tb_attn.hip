// tb_attn.hip -- exact softmax attention over the selected K/V rows (gfx950).
//
// TokenButler abstract (2026) and gist.science technical summary,
// Significance: the full KV cache stays resident and each decode step reads
// only the selected tokens; attention over them is ordinary softmax attention.
//
// Grid: (position chunk of kAttnChunk tokens, KV head, sequence).  A
// work-group handles one KV head and one chunk for all the query heads that
// share it (GQA):
//   1. For each query head, the part of its ascending selection list that
//      falls in the chunk is found by a wave-parallel search (64 samples per
//      round) and marked in an LDS bitmap; the always-kept range
//      [keep_from, n) is added to every head.
//   2. The union over the heads is compacted into a list of (row, head mask),
//      so each selected K/V row is read from HBM once for the whole group.
//   3. Rows stream through the lanes in 16-byte pieces (D*elt/16 lanes per
//      row, several rows per wave); each row slot keeps an online softmax
//      (running max, sum and fp32 accumulator) per query head in base 2.
//   4. Row slots are merged by cross-lane shuffles, waves through LDS, into
//      one partial (max, sum, acc[D]) per query head and chunk.
//   5. The last work-group of a (sequence, KV head) to arrive (device-scope
//      counter) merges the chunk partials and writes the output rows, then
//      resets the counter to zero for the next call.
#include "tb_internal.h"

namespace tb {
namespace {

constexpr int kAttnThreads = 256;

// First index e in [0, cnt] with L[e] >= v for an ascending list, found by
// one wave; every lane returns the answer.
__device__ int wave_lower_bound(const int32_t *__restrict__ L, int cnt, int v)
{
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = cnt;
    while (hi - lo > 64) {
        const int step = (hi - lo + 63) / 64;
        const int e = lo + lane * step;
        const bool less = e < hi && L[e] < v;
        const int c = __popcll(__ballot(less));
        const int nlo = c == 0 ? lo : lo + (c - 1) * step + 1;
        const int nhi = min(hi, lo + c * step);
        lo = nlo;
        hi = nhi;
    }
    const int e = lo + lane;
    const bool less = e < hi && L[e] < v;
    return lo + __popcll(__ballot(less));
}

template <typename T, int D, int GQ>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    const int32_t *__restrict__ sel_idx, int sel_stride, const int32_t *__restrict__ sel_count,
    const int32_t *__restrict__ keep_from, const int32_t *__restrict__ ctx_len, int Hq, int Hkv,
    int Himp, int cap, float qscale, float *__restrict__ part, uint32_t *__restrict__ counters,
    T *__restrict__ out)
{
    constexpr int EPL = 16 / (int)sizeof(T); // elements per lane piece
    constexpr int LPR = D / EPL;             // lanes per row
    constexpr int RPW = 64 / LPR;            // rows per wave step
    constexpr int NSLOT = 4 * RPW;           // row slots per work-group
    constexpr int NWD = kAttnChunk / 32;     // bitmap words per head
    static_assert(NWD <= 64, "one wave compacts the union");

    __shared__ uint32_t bm[GQ][NWD];
    __shared__ uint32_t ulist[kAttnChunk];
    __shared__ uint32_t s_misc[4];
    __shared__ float mrg_m[4][GQ];
    __shared__ float mrg_l[4][GQ];
    __shared__ float mrg_acc[4][GQ][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int nchunk = gridDim.x;
    const int n = clamp_len(ctx_len[b], cap);
    const int c0 = c * kAttnChunk;
    const int c1 = min(c0 + kAttnChunk, n);
    const bool active = c0 < n;
    const size_t head0 = (size_t)b * Hq + (size_t)g * GQ; // first query head of the group

    if (active) {
        // ---- 1. per-head membership bitmaps of this chunk ----
        for (int e = tid; e < GQ * NWD; e += kAttnThreads)
            (&bm[0][0])[e] = 0u;
        __syncthreads();
        for (int hl = wave; hl < GQ; hl += 4) {
            const int h = g * GQ + hl;
            const int i = (int)((long)h * Himp / Hq);
            const size_t li = (size_t)b * Himp + i;
            const int32_t *L = sel_idx + li * sel_stride;
            int cnt = sel_count[li];
            cnt = cnt < 0 ? 0 : (cnt > sel_stride ? sel_stride : cnt);
            const int lo = wave_lower_bound(L, cnt, c0);
            const int hi = wave_lower_bound(L, cnt, c1);
            for (int e = lo + lane; e < hi; e += 64) {
                const int t = L[e];
                if (t >= c0 && t < c1)
                    atomicOr(&bm[hl][(t - c0) >> 5], 1u << ((t - c0) & 31));
            }
        }
        if (keep_from != nullptr) {
            const int kf = clamp_len(keep_from[b], n);
            for (int t = max(kf, c0) + tid; t < c1; t += kAttnThreads)
#pragma unroll
                for (int hl = 0; hl < GQ; ++hl)
                    atomicOr(&bm[hl][(t - c0) >> 5], 1u << ((t - c0) & 31));
        }
        __syncthreads();

        // ---- 2. union over the heads, compacted with head masks ----
        if (wave == 0) {
            uint32_t words[GQ];
            uint32_t u = 0u;
#pragma unroll
            for (int hl = 0; hl < GQ; ++hl) {
                words[hl] = lane < NWD ? bm[hl][lane] : 0u;
                u |= words[hl];
            }
            const uint32_t cnt = __popc(u);
            uint32_t inc = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_up(inc, off);
                if (lane >= off)
                    inc += v;
            }
            uint32_t pos = inc - cnt;
            while (u) {
                const int bit = __ffs(u) - 1;
                uint32_t mask = 0u;
#pragma unroll
                for (int hl = 0; hl < GQ; ++hl)
                    mask |= ((words[hl] >> bit) & 1u) << hl;
                ulist[pos++] = (uint32_t)(lane * 32 + bit) | (mask << 16);
                u &= u - 1u;
            }
            if (lane == 63)
                s_misc[0] = inc;
        }
        __syncthreads();

        // ---- 3. stream the rows ----
        const int nu = (int)s_misc[0];
        const int slot = lane / LPR, sub = lane % LPR;
        float qf[GQ][EPL];
#pragma unroll
        for (int hl = 0; hl < GQ; ++hl) {
            const uint4 piece =
                *reinterpret_cast<const uint4 *>(q + (head0 + hl) * D + sub * EPL);
            T v[EPL];
            __builtin_memcpy(v, &piece, 16);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                qf[hl][e] = to_f32(v[e]) * qscale;
        }
        float m[GQ], l[GQ], acc[GQ][EPL];
#pragma unroll
        for (int hl = 0; hl < GQ; ++hl) {
            m[hl] = -INFINITY;
            l[hl] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[hl][e] = 0.f;
        }
        const size_t kvbase = ((size_t)b * Hkv + g) * cap;
        const T *kb = kc + kvbase * D + sub * EPL;
        const T *vb = vc + kvbase * D + sub * EPL;

        auto consume = [&](uint32_t ent, const uint4 &kp, const uint4 &vp) {
            T kv[EPL], vv[EPL];
            __builtin_memcpy(kv, &kp, 16);
            __builtin_memcpy(vv, &vp, 16);
            const uint32_t mask = ent >> 16;
            float z[GQ];
#pragma unroll
            for (int hl = 0; hl < GQ; ++hl) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    d = fmaf(qf[hl][e], to_f32(kv[e]), d);
                z[hl] = d;
            }
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1)
#pragma unroll
                for (int hl = 0; hl < GQ; ++hl)
                    z[hl] += __shfl_xor(z[hl], off);
#pragma unroll
            for (int hl = 0; hl < GQ; ++hl) {
                if ((mask >> hl) & 1u) {
                    const float mn = fmaxf(m[hl], z[hl]);
                    const float corr = exp2f(m[hl] - mn);
                    const float p = exp2f(z[hl] - mn);
                    l[hl] = l[hl] * corr + p;
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[hl][e] = fmaf(acc[hl][e], corr, p * to_f32(vv[e]));
                    m[hl] = mn;
                }
            }
        };

        int u = wave * RPW + slot;
        for (; u + NSLOT < nu; u += 2 * NSLOT) {
            const uint32_t e0 = ulist[u], e1 = ulist[u + NSLOT];
            const size_t t0 = (size_t)(c0 + (int)(e0 & 0xffffu)) * D;
            const size_t t1 = (size_t)(c0 + (int)(e1 & 0xffffu)) * D;
            const uint4 k0 = *reinterpret_cast<const uint4 *>(kb + t0);
            const uint4 v0 = *reinterpret_cast<const uint4 *>(vb + t0);
            const uint4 k1 = *reinterpret_cast<const uint4 *>(kb + t1);
            const uint4 v1 = *reinterpret_cast<const uint4 *>(vb + t1);
            consume(e0, k0, v0);
            consume(e1, k1, v1);
        }
        if (u < nu) {
            const uint32_t e0 = ulist[u];
            const size_t t0 = (size_t)(c0 + (int)(e0 & 0xffffu)) * D;
            const uint4 k0 = *reinterpret_cast<const uint4 *>(kb + t0);
            const uint4 v0 = *reinterpret_cast<const uint4 *>(vb + t0);
            consume(e0, k0, v0);
        }

        // ---- 4. merge row slots (shuffles) and waves (LDS) into the chunk partial ----
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int hl = 0; hl < GQ; ++hl) {
                const float mo = __shfl_xor(m[hl], off);
                const float lo_ = __shfl_xor(l[hl], off);
                const float mn = fmaxf(m[hl], mo);
                const float fa = m[hl] == -INFINITY ? 0.f : exp2f(m[hl] - mn);
                const float fb = mo == -INFINITY ? 0.f : exp2f(mo - mn);
                l[hl] = l[hl] * fa + lo_ * fb;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const float ao = __shfl_xor(acc[hl][e], off);
                    acc[hl][e] = acc[hl][e] * fa + ao * fb;
                }
                m[hl] = mn;
            }
        }
        if (slot == 0) {
#pragma unroll
            for (int hl = 0; hl < GQ; ++hl) {
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    mrg_acc[wave][hl][sub * EPL + e] = acc[hl][e];
                if (sub == 0) {
                    mrg_m[wave][hl] = m[hl];
                    mrg_l[wave][hl] = l[hl];
                }
            }
        }
        __syncthreads();
        for (int pi = tid; pi < GQ * D; pi += kAttnThreads) {
            const int hl = pi / D, dim = pi % D;
            float M = -INFINITY;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                M = fmaxf(M, mrg_m[s][hl]);
            float Ls = 0.f, O = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float ms = mrg_m[s][hl];
                    if (ms != -INFINITY) {
                        const float f = exp2f(ms - M);
                        Ls = fmaf(mrg_l[s][hl], f, Ls);
                        O = fmaf(mrg_acc[s][hl][dim], f, O);
                    }
                }
            }
            float *pp = part + ((head0 + hl) * nchunk + c) * (D + 2);
            pp[2 + dim] = O;
            if (dim == 0) {
                pp[0] = M;
                pp[1] = Ls;
            }
        }
    }

    // ---- 5. arrival; the last work-group of this (b, g) merges the chunks ----
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = atomicAdd(&counters[(size_t)b * Hkv + g], 1u);
        s_misc[1] = old == (uint32_t)(nchunk - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (s_misc[1] == 0u)
        return;
    __threadfence();
    const int nact = (n + kAttnChunk - 1) / kAttnChunk;
    for (int pi = tid; pi < GQ * D; pi += kAttnThreads) {
        const int hl = pi / D, dim = pi % D;
        const float *base = part + (head0 + hl) * nchunk * (D + 2);
        float M = -INFINITY;
        for (int cc = 0; cc < nact; ++cc)
            M = fmaxf(M, base[(size_t)cc * (D + 2)]);
        float Ls = 0.f, O = 0.f;
        if (M != -INFINITY) {
            for (int cc = 0; cc < nact; ++cc) {
                const float *pp = base + (size_t)cc * (D + 2);
                const float ms = pp[0];
                if (ms != -INFINITY) {
                    const float f = exp2f(ms - M);
                    Ls = fmaf(pp[1], f, Ls);
                    O = fmaf(pp[2 + dim], f, O);
                }
            }
        }
        out[(head0 + hl) * D + dim] = from_f32<T>(Ls > 0.f ? O / Ls : 0.f);
    }
    if (tid == 0)
        counters[(size_t)b * Hkv + g] = 0u;
}

template <typename T, int D, int GQ>
hipError_t attn_t(const tb_shape &s, const void *q, const void *k, const void *v,
                  const int32_t *sel_idx, int sel_stride, const int32_t *sel_count,
                  const int32_t *keep_from, const int32_t *ctx_len, float scale, void *out,
                  float *part, uint32_t *counters, hipStream_t st)
{
    dim3 grid(attn_chunks(s.ctx_cap), s.n_kv_heads, s.batch);
    const float qscale = scale * 1.4426950408889634f; // logits in base 2
    hipLaunchKernelGGL((attn_kernel<T, D, GQ>), grid, dim3(kAttnThreads), 0, st, (const T *)q,
                       (const T *)k, (const T *)v, sel_idx, sel_stride, sel_count, keep_from,
                       ctx_len, s.n_q_heads, s.n_kv_heads, s.n_imp_heads, s.ctx_cap, qscale, part,
                       counters, (T *)out);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t attn_gq(const tb_shape &s, const void *q, const void *k, const void *v,
                   const int32_t *sel_idx, int sel_stride, const int32_t *sel_count,
                   const int32_t *keep_from, const int32_t *ctx_len, float scale, void *out,
                   float *part, uint32_t *counters, hipStream_t st)
{
    switch (s.n_q_heads / s.n_kv_heads) {
    case 1: return attn_t<T, D, 1>(s, q, k, v, sel_idx, sel_stride, sel_count, keep_from, ctx_len, scale, out, part, counters, st);
    case 2: return attn_t<T, D, 2>(s, q, k, v, sel_idx, sel_stride, sel_count, keep_from, ctx_len, scale, out, part, counters, st);
    case 4: return attn_t<T, D, 4>(s, q, k, v, sel_idx, sel_stride, sel_count, keep_from, ctx_len, scale, out, part, counters, st);
    case 8: return attn_t<T, D, 8>(s, q, k, v, sel_idx, sel_stride, sel_count, keep_from, ctx_len, scale, out, part, counters, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_attn(const tb_shape &s, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *sel_idx, int sel_stride,
                       const int32_t *sel_count, const int32_t *keep_from,
                       const int32_t *ctx_len, float softmax_scale, void *out, float *part,
                       uint32_t *counters, hipStream_t st)
{
#define TB_ATTN_ARGS s, q, k_cache, v_cache, sel_idx, sel_stride, sel_count, keep_from, ctx_len, \
                     softmax_scale, out, part, counters, st
    if (s.dtype == TB_BF16) {
        if (s.head_dim == 64) return attn_gq<bf16_t, 64>(TB_ATTN_ARGS);
        if (s.head_dim == 128) return attn_gq<bf16_t, 128>(TB_ATTN_ARGS);
    } else {
        if (s.head_dim == 64) return attn_gq<float, 64>(TB_ATTN_ARGS);
        if (s.head_dim == 128) return attn_gq<float, 128>(TB_ATTN_ARGS);
    }
#undef TB_ATTN_ARGS
    return hipErrorInvalidValue;
}

} // namespace tb
