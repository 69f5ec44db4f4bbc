// tb_attn.hip -- exact softmax attention over the selected K/V rows (gfx950).
//
// TokenButler abstract (2026) and gist.science technical summary,
// Significance: the full KV cache stays resident and each decode step reads
// only the selected tokens; attention over them is ordinary softmax attention.
//
// Grid: (position chunk of kAttnChunk tokens, KV head, sequence).  A
// work-group handles one KV head and one chunk for all the query heads that
// share it (GQA):
//   1. Each query head's membership in the chunk comes either from its
//      selection bitmap (one 32-bit word per 32 positions, read directly) or
//      from its ascending selection list (the chunk's segment is located by a
//      wave-parallel search, 64 samples per round); the always-kept range
//      [keep_from, n) is added to every head.
//   2. The union over the heads is compacted in LDS into (row, head mask)
//      entries, so each selected K/V row is read from HBM once per group.
//   3. Rows stream through the lanes in 16-byte pieces (D*elt/16 lanes per
//      row, several rows per wave, four rows in flight per row slot); each row
//      slot keeps an online softmax (running max, sum, fp32 accumulator) per
//      query head in base 2.  Dot products are reduced across the row's lanes
//      with DPP row permutations.
//   4. Row slots are merged by cross-lane shuffles, waves through LDS, into
//      one partial (max, sum, acc[D]) per query head and chunk.
//   5. The last work-group of a (sequence, KV head) to arrive (device-scope
//      counter) merges the chunk partials -- max and weights first, then the
//      weighted sums with all of its threads -- writes the output rows, and
//      resets the counter to zero for the next call.
#include "tb_internal.h"

namespace tb {
namespace {

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kMaxChunks = kMaxCtxCap / kAttnChunk;
constexpr int kRowsInFlight = 8; // rows per row slot loaded before use

// Chunk partials cross work-groups (and XCDs, whose L2 caches are not
// coherent with each other).  They are written and read with agent-scope
// atomic accesses, which go through to the device coherence point, so no
// full L2 write-back fence is needed to publish them.
__device__ __forceinline__ void store_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 load4_agent(const float *p)
{
    return make_float4(load_agent(p), load_agent(p + 1), load_agent(p + 2), load_agent(p + 3));
}

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

// Sum of x over aligned groups of N lanes (N in {1, 2, 4, 8, 16, 32}); every
// lane of the group receives the sum.  Within a 16-lane DPP row the partners
// come from quad permutations and the half/full row mirrors.
template <int N> __device__ __forceinline__ float group_sum(float x)
{
    if constexpr (N >= 2)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    if constexpr (N >= 4)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    if constexpr (N >= 8)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    if constexpr (N >= 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    if constexpr (N >= 32)
        x += __shfl_xor(x, 16);
    return x;
}

struct AttnArgs {
    const void *q, *k, *v;
    const int32_t *sel_idx;  // list mode
    int sel_stride;
    const int32_t *sel_count;
    const uint32_t *sel_bits; // bitmap mode
    int bits_stride;          // words per head
    const int32_t *keep_from;
    const int32_t *ctx_len;
    int Hq, Hkv, Himp, cap;
    float qscale;
    float *part_o;     // [b*Hq][nchunk][D]
    float *part_ml;    // [b*Hq][nchunk][2]
    uint32_t *counters;
    void *out;
};

template <typename T, int D, int GQ, bool BITMAP>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnArgs a)
{
    constexpr int EPL = 16 / (int)sizeof(T); // elements per lane piece
    constexpr int LPR = D / EPL;             // lanes per row
    constexpr int RPW = 64 / LPR;            // rows per wave step
    constexpr int NSLOT = kAttnWaves * RPW;  // row slots per work-group
    constexpr int NWD = kAttnChunk / 32;     // bitmap words per head
    static_assert(NWD <= 64, "one wave compacts the union");

    __shared__ uint32_t bm[GQ][NWD];
    __shared__ uint32_t ulist[kAttnChunk];
    __shared__ uint32_t s_misc[4];
    __shared__ float mrg_m[kAttnWaves][GQ];
    __shared__ float mrg_l[kAttnWaves][GQ];
    __shared__ float mrg_acc[kAttnWaves][GQ][D];
    __shared__ float cmb_f[GQ][kMaxChunks];
    __shared__ float cmb_ml[GQ][2];
    __shared__ float4 red[kAttnThreads];

    const T *__restrict__ q = (const T *)a.q;
    const T *__restrict__ kc = (const T *)a.k;
    const T *__restrict__ vc = (const T *)a.v;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int nchunk = gridDim.x;
    const int n = clamp_len(a.ctx_len[b], a.cap);
    const int c0 = c * kAttnChunk;
    const int c1 = min(c0 + kAttnChunk, n);
    const bool active = c0 < n;
    const size_t head0 = (size_t)b * a.Hq + (size_t)g * GQ; // first query head of the group

    if (active) {
        // ---- 1. per-head membership of this chunk ----
        const int kf = a.keep_from != nullptr ? clamp_len(a.keep_from[b], n) : n;
        if constexpr (BITMAP) {
            for (int e = tid; e < GQ * NWD; e += kAttnThreads) {
                const int hl = e / NWD, w = e % NWD;
                const int i = (int)((long)(g * GQ + hl) * a.Himp / a.Hq);
                const int p0 = c0 + 32 * w; // first position of this word
                uint32_t word = 0u;
                if (p0 < c1)
                    word = a.sel_bits[((size_t)b * a.Himp + i) * a.bits_stride + (p0 >> 5)];
                // clip to [c0, c1) and add the always-kept range
                const int lo = max(kf, p0), hi = min(c1, p0 + 32);
                if (hi - p0 < 32)
                    word &= hi <= p0 ? 0u : ((1u << (hi - p0)) - 1u);
                if (lo < hi) {
                    const uint32_t upto = hi - p0 == 32 ? 0xffffffffu : ((1u << (hi - p0)) - 1u);
                    word |= upto & ~((1u << (lo - p0)) - 1u);
                }
                bm[hl][w] = word;
            }
        } else {
            for (int e = tid; e < GQ * NWD; e += kAttnThreads)
                (&bm[0][0])[e] = 0u;
            __syncthreads();
            for (int hl = wave; hl < GQ; hl += kAttnWaves) {
                const int h = g * GQ + hl;
                const int i = (int)((long)h * a.Himp / a.Hq);
                const size_t li = (size_t)b * a.Himp + i;
                const int32_t *L = a.sel_idx + li * a.sel_stride;
                int cnt = a.sel_count[li];
                cnt = cnt < 0 ? 0 : (cnt > a.sel_stride ? a.sel_stride : cnt);
                const int lo = wave_lower_bound(L, cnt, c0);
                const int hi = wave_lower_bound(L, cnt, c1);
                for (int e = lo + lane; e < hi; e += 64) {
                    const int t = L[e];
                    if (t >= c0 && t < c1)
                        atomicOr(&bm[hl][(t - c0) >> 5], 1u << ((t - c0) & 31));
                }
            }
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
                qf[hl][e] = to_f32(v[e]) * a.qscale;
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
        const size_t kvbase = ((size_t)b * a.Hkv + g) * a.cap;
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
                z[hl] = group_sum<LPR>(d);
            }
#pragma unroll
            for (int hl = 0; hl < GQ; ++hl) {
                if ((mask >> hl) & 1u) {
                    const float mn = fmaxf(m[hl], z[hl]);
                    const float corr = exp2f(m[hl] - mn);
                    const float p = exp2f(z[hl] - mn);
                    l[hl] = fmaf(l[hl], corr, p);
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[hl][e] = fmaf(acc[hl][e], corr, p * to_f32(vv[e]));
                    m[hl] = mn;
                }
            }
        };
        auto rowptr = [&](uint32_t ent) -> size_t {
            return (size_t)(c0 + (int)(ent & 0xffffu)) * D;
        };

        // all of a slot's rows (up to kRowsInFlight) are requested before any is used
        for (int base = wave * RPW + slot; base < nu; base += kRowsInFlight * NSLOT) {
            uint32_t e[kRowsInFlight];
            uint4 kk[kRowsInFlight], vv[kRowsInFlight];
#pragma unroll
            for (int r = 0; r < kRowsInFlight; ++r) {
                const int u = base + r * NSLOT;
                e[r] = u < nu ? ulist[u] : 0xffffffffu;
            }
#pragma unroll
            for (int r = 0; r < kRowsInFlight; ++r) {
                if (e[r] != 0xffffffffu) {
                    kk[r] = *reinterpret_cast<const uint4 *>(kb + rowptr(e[r]));
                    vv[r] = *reinterpret_cast<const uint4 *>(vb + rowptr(e[r]));
                }
            }
#pragma unroll
            for (int r = 0; r < kRowsInFlight; ++r)
                if (e[r] != 0xffffffffu)
                    consume(e[r], kk[r], vv[r]);
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
            for (int s = 0; s < kAttnWaves; ++s)
                M = fmaxf(M, mrg_m[s][hl]);
            float Ls = 0.f, O = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int s = 0; s < kAttnWaves; ++s) {
                    const float ms = mrg_m[s][hl];
                    if (ms != -INFINITY) {
                        const float f = exp2f(ms - M);
                        Ls = fmaf(mrg_l[s][hl], f, Ls);
                        O = fmaf(mrg_acc[s][hl][dim], f, O);
                    }
                }
            }
            const size_t pc = (head0 + hl) * nchunk + c;
            store_agent(&a.part_o[pc * D + dim], O);
            if (dim == 0) {
                store_agent(&a.part_ml[pc * 2], M);
                store_agent(&a.part_ml[pc * 2 + 1], Ls);
            }
        }
    }

    // ---- 5. arrival; the last work-group of this (b, g) merges the chunks ----
    // The partial stores complete (vmcnt 0) before the counter moves; the
    // signal fence keeps the compiler from sinking them below it.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&a.counters[(size_t)b * a.Hkv + g], 1u,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_misc[1] = old == (uint32_t)(nchunk - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (s_misc[1] == 0u)
        return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int nact = (n + kAttnChunk - 1) / kAttnChunk;
    // (a) chunk maxima and sums into LDS
    for (int e = tid; e < GQ * nact; e += kAttnThreads) {
        const int hl = e / nact, cc = e % nact;
        const size_t pc = (head0 + hl) * nchunk + cc;
        cmb_f[hl][cc] = load_agent(&a.part_ml[pc * 2]);
    }
    __syncthreads();
    // (b) per head: global max, chunk weights, total sum (one wave per head)
    for (int hl = wave; hl < GQ; hl += kAttnWaves) {
        float M = -INFINITY;
        for (int cc = lane; cc < nact; cc += 64)
            M = fmaxf(M, cmb_f[hl][cc]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            M = fmaxf(M, __shfl_xor(M, off));
        float Ls = 0.f;
        for (int cc = lane; cc < nact; cc += 64) {
            const float mc = cmb_f[hl][cc];
            const float f = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
            cmb_f[hl][cc] = f;
            Ls = fmaf(load_agent(&a.part_ml[((head0 + hl) * nchunk + cc) * 2 + 1]), f, Ls);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            Ls += __shfl_xor(Ls, off);
        if (lane == 0)
            cmb_ml[hl][0] = Ls;
    }
    __syncthreads();
    // (c) weighted sums: thread = (float4 column, chunk residue class)
    constexpr int NCOL = GQ * D / 4;
    constexpr int NPART = kAttnThreads / NCOL;
    static_assert(NPART >= 1 && NPART * NCOL == kAttnThreads, "column split");
    {
        const int col = tid % NCOL, p = tid / NCOL;
        const int hl = col / (D / 4), d4 = col % (D / 4);
        const float *po = a.part_o + (head0 + hl) * nchunk * D + d4 * 4;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        int cc = p;
        for (; cc + 3 * NPART < nact; cc += 4 * NPART) {
            float4 v[4];
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = load4_agent(po + (size_t)(cc + r * NPART) * D);
                f[r] = cmb_f[hl][cc + r * NPART];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s.x = fmaf(v[r].x, f[r], s.x);
                s.y = fmaf(v[r].y, f[r], s.y);
                s.z = fmaf(v[r].z, f[r], s.z);
                s.w = fmaf(v[r].w, f[r], s.w);
            }
        }
        for (; cc < nact; cc += NPART) {
            const float4 v = load4_agent(po + (size_t)cc * D);
            const float f = cmb_f[hl][cc];
            s.x = fmaf(v.x, f, s.x);
            s.y = fmaf(v.y, f, s.y);
            s.z = fmaf(v.z, f, s.z);
            s.w = fmaf(v.w, f, s.w);
        }
        red[p * NCOL + col] = s;
    }
    __syncthreads();
    T *out = (T *)a.out;
    for (int col = tid; col < NCOL; col += kAttnThreads) {
        const int hl = col / (D / 4), d4 = col % (D / 4);
        float4 s = red[col];
        for (int p = 1; p < NPART; ++p) {
            const float4 t = red[p * NCOL + col];
            s.x += t.x;
            s.y += t.y;
            s.z += t.z;
            s.w += t.w;
        }
        const float Ls = cmb_ml[hl][0];
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        T *o = out + (head0 + hl) * D + d4 * 4;
        o[0] = from_f32<T>(s.x * inv);
        o[1] = from_f32<T>(s.y * inv);
        o[2] = from_f32<T>(s.z * inv);
        o[3] = from_f32<T>(s.w * inv);
    }
    if (tid == 0)
        __hip_atomic_store(&a.counters[(size_t)b * a.Hkv + g], 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int D, int GQ>
hipError_t attn_t(const tb_shape &s, const AttnArgs &a, hipStream_t st)
{
    dim3 grid(attn_chunks(s.ctx_cap), s.n_kv_heads, s.batch);
    if (a.sel_bits != nullptr)
        hipLaunchKernelGGL((attn_kernel<T, D, GQ, true>), grid, dim3(kAttnThreads), 0, st, a);
    else
        hipLaunchKernelGGL((attn_kernel<T, D, GQ, false>), grid, dim3(kAttnThreads), 0, st, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t attn_gq(const tb_shape &s, const AttnArgs &a, hipStream_t st)
{
    switch (s.n_q_heads / s.n_kv_heads) {
    case 1: return attn_t<T, D, 1>(s, a, st);
    case 2: return attn_t<T, D, 2>(s, a, st);
    case 4: return attn_t<T, D, 4>(s, a, st);
    case 8: return attn_t<T, D, 8>(s, a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_attn(const tb_shape &s, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *sel_idx, int sel_stride,
                       const int32_t *sel_count, const uint32_t *sel_bits,
                       const int32_t *keep_from, const int32_t *ctx_len, float softmax_scale,
                       void *out, float *part_o, float *part_ml, uint32_t *counters,
                       hipStream_t st)
{
    AttnArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.sel_idx = sel_idx;
    a.sel_stride = sel_stride;
    a.sel_count = sel_count;
    a.sel_bits = sel_bits;
    a.bits_stride = bitmap_words(s.ctx_cap);
    a.keep_from = keep_from;
    a.ctx_len = ctx_len;
    a.Hq = s.n_q_heads;
    a.Hkv = s.n_kv_heads;
    a.Himp = s.n_imp_heads;
    a.cap = s.ctx_cap;
    a.qscale = softmax_scale * 1.4426950408889634f; // logits in base 2
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.counters = counters;
    a.out = out;
    if (s.dtype == TB_BF16) {
        if (s.head_dim == 64) return attn_gq<bf16_t, 64>(s, a, st);
        if (s.head_dim == 128) return attn_gq<bf16_t, 128>(s, a, st);
    } else {
        if (s.head_dim == 64) return attn_gq<float, 64>(s, a, st);
        if (s.head_dim == 128) return attn_gq<float, 128>(s, a, st);
    }
    return hipErrorInvalidValue;
}

} // namespace tb
