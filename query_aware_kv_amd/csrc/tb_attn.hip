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
//   2. Each query head is served by 8/GQ of the eight waves, each wave taking
//      a part of the chunk and compacting that head's positions in it with
//      ballots; the head's waves then split the concatenated list evenly.
//      Rows that several query heads of the group select are requested by
//      sibling waves of the same work-group at about the same time, so the
//      repeats are served from cache and HBM sees each row about once.
//   3. Rows stream through the lanes in 16-byte pieces (D*elt/16 lanes per
//      row, several rows per wave, four rows in flight per row slot); each row
//      slot keeps an online softmax (running max, sum, fp32 accumulator) for
//      its wave's head in base 2, rescaling only when the running max grows.
//      Lane dot products use v_dot2 on bf16 pairs and are reduced across the
//      row's lanes with DPP row permutations.
//   4. The row slots of a head are merged through LDS into one partial
//      (max, sum, acc[D]) per query head and chunk.
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
constexpr int kRowsInFlight = 4; // rows per row slot loaded before use

// Chunk partials cross work-groups (and XCDs, whose L2 caches are not
// coherent with each other).  They are written and read with agent-scope
// atomic accesses, which go through to the device coherence point, so no
// full L2 write-back fence is needed to publish them.
// Two 64-bit accesses per four floats: every agent-scope access is its own
// memory transaction, so wider ones matter.
__device__ __forceinline__ float4 load4_agent(const float *p)
{
    const double x = __hip_atomic_load(reinterpret_cast<const double *>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    const double y = __hip_atomic_load(reinterpret_cast<const double *>(p) + 1,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float2 lo = __builtin_bit_cast(float2, x), hi = __builtin_bit_cast(float2, y);
    return make_float4(lo.x, lo.y, hi.x, hi.y);
}
__device__ __forceinline__ void store2_agent(float *p, float x, float y)
{
    __hip_atomic_store(reinterpret_cast<double *>(p), __builtin_bit_cast(double, make_float2(x, y)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Dot product of the 16-byte q and k pieces held by one lane.
__device__ __forceinline__ float lane_dot_bf16(const uint4 &q, const uint4 &k)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float d = 0.f;
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x),
                                        __builtin_bit_cast(bf16x2, k.x), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y),
                                        __builtin_bit_cast(bf16x2, k.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z),
                                        __builtin_bit_cast(bf16x2, k.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w),
                                        __builtin_bit_cast(bf16x2, k.w), d, false);
    return d;
}
__device__ __forceinline__ float lane_dot_f32(const uint4 &q, const uint4 &k)
{
    float d = __uint_as_float(q.x) * __uint_as_float(k.x);
    d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
    d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
    d = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
    return d;
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
    auto lane_dot = [](const uint4 &qp, const uint4 &kp) -> float {
        if constexpr (sizeof(T) == 2)
            return lane_dot_bf16(qp, kp);
        else
            return lane_dot_f32(qp, kp);
    };
    constexpr int EPL = 16 / (int)sizeof(T); // elements per lane piece
    constexpr int LPR = D / EPL;             // lanes per row
    constexpr int RPW = 64 / LPR;            // rows per wave step
    constexpr int NWD = kAttnChunk / 32;     // bitmap words per head
    static_assert(GQ <= kAttnWaves && kAttnWaves % GQ == 0, "whole waves per query head");
    constexpr int WPH = kAttnWaves / GQ;     // waves per query head
    constexpr int PW = kAttnChunk / WPH;     // positions of one wave's part of the chunk
    constexpr int NS = WPH * RPW;            // row slots per query head
    static_assert(PW % 64 == 0 && NS <= 64, "parts of whole ballots; one lane per slot");

    __shared__ uint32_t bm[GQ][NWD];
    __shared__ uint16_t hlist[kAttnWaves][PW]; // positions of each wave's part
    __shared__ uint32_t wcnt[kAttnWaves];
    __shared__ uint32_t s_misc[4];
    __shared__ float mrg_m[GQ][NS];
    __shared__ float mrg_l[GQ][NS];
    __shared__ float mrg_f[GQ][NS];
    __shared__ float mrg_acc[GQ][NS][D];
    __shared__ float mrg_M[GQ], mrg_L[GQ];
    __shared__ float cmb_f[GQ][kMaxChunks];
    __shared__ float cmb_l[GQ][kMaxChunks];
    __shared__ float cmb_ml[GQ][2];
    __shared__ float4 red[kAttnThreads];

    const T *__restrict__ q = (const T *)a.q;
    const T *__restrict__ kc = (const T *)a.k;
    const T *__restrict__ vc = (const T *)a.v;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int nchunk = gridDim.x;
    const int c0 = c * kAttnChunk;
    const size_t head0 = (size_t)b * a.Hq + (size_t)g * GQ; // first query head of the group
    const int slot = lane / LPR, sub = lane % LPR;
    static_assert(GQ * NWD <= kAttnThreads, "one bitmap word per thread");

    // Wave w serves query head hw = w / WPH on part w % WPH of the chunk.
    const int hw = wave / WPH, wpart = wave % WPH;
    // Everything that does not depend on the lengths is requested first: the
    // q slice of this lane for the wave's head (kept in the storage type;
    // bf16 pairs feed v_dot2) and, in bitmap mode, this thread's membership
    // word.
    const uint4 qh = *reinterpret_cast<const uint4 *>(q + (head0 + hw) * D + sub * EPL);
    uint32_t word0 = 0u;
    if constexpr (BITMAP) {
        if (tid < GQ * NWD) {
            const int hl = tid / NWD, w = tid % NWD;
            const int i = (int)((long)(g * GQ + hl) * a.Himp / a.Hq);
            const int p0 = c0 + 32 * w; // first position of this word
            if (p0 < a.cap)
                word0 = a.sel_bits[((size_t)b * a.Himp + i) * a.bits_stride + (p0 >> 5)];
        }
    }
    const int kf_raw = a.keep_from != nullptr ? a.keep_from[b] : a.cap;
    const int n = clamp_len(a.ctx_len[b], a.cap);
    const int c1 = min(c0 + kAttnChunk, n);
    const bool active = c0 < n;

    if (active) {
        // ---- 1. per-head membership of this chunk ----
        const int kf = clamp_len(kf_raw, n);
        if constexpr (BITMAP) {
            if (tid < GQ * NWD) {
                const int hl = tid / NWD, w = tid % NWD;
                const int p0 = c0 + 32 * w;
                uint32_t word = p0 < c1 ? word0 : 0u;
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

        // ---- 2. this wave's positions, compacted by ballots ----
        {
            uint32_t run = 0u;
#pragma unroll
            for (int k = 0; k < PW / 64; ++k) {
                const int pos = wpart * PW + 64 * k + lane;
                const bool in = (bm[hw][pos >> 5] >> (pos & 31)) & 1u;
                const unsigned long long m = __ballot(in);
                if (in)
                    hlist[wave][run + __builtin_amdgcn_mbcnt_hi(
                                          (uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] =
                        (uint16_t)pos;
                run += __popcll(m);
            }
            if (lane == 0)
                wcnt[wave] = run;
        }
        __syncthreads();

        // ---- 3. stream the head's rows ----
        // The head's positions are the concatenation of its WPH parts; each
        // of its waves takes an equal share, and each row slot of a wave an
        // interleaved share of that.
        uint32_t pre[WPH], nh = 0u;
#pragma unroll
        for (int pp = 0; pp < WPH; ++pp) {
            pre[pp] = nh;
            nh += wcnt[hw * WPH + pp];
        }
        const uint32_t e0 = nh * wpart / WPH, e1 = nh * (wpart + 1) / WPH;
        auto position = [&](uint32_t u) -> uint32_t { // u < nh
            int src = hw * WPH;
            uint32_t off = u;
#pragma unroll
            for (int pp = 1; pp < WPH; ++pp) {
                const bool at = u >= pre[pp];
                src = at ? hw * WPH + pp : src;
                off = at ? u - pre[pp] : off;
            }
            return hlist[src][off];
        };
        float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[e] = 0.f;
        const size_t kvbase = ((size_t)b * a.Hkv + g) * a.cap + c0;
        const T *kb = kc + kvbase * D + sub * EPL;
        const T *vb = vc + kvbase * D + sub * EPL;

        // All of a slot's rows (up to kRowsInFlight) are requested before any
        // is used.  The loads are unconditional -- a missing row reads the
        // chunk's first row, which always exists, and is given weight 0 -- so
        // they issue back to back.
        for (uint32_t base = e0 + slot; base < e1; base += kRowsInFlight * RPW) {
            uint32_t pos[kRowsInFlight];
            bool ok[kRowsInFlight];
            uint4 kk[kRowsInFlight], vv[kRowsInFlight];
#pragma unroll
            for (int r = 0; r < kRowsInFlight; ++r) {
                const uint32_t u = base + r * RPW;
                ok[r] = u < e1;
                pos[r] = ok[r] ? position(u) : 0u;
            }
#pragma unroll
            for (int r = 0; r < kRowsInFlight; ++r) {
                kk[r] = *reinterpret_cast<const uint4 *>(kb + (size_t)pos[r] * D);
                vv[r] = *reinterpret_cast<const uint4 *>(vb + (size_t)pos[r] * D);
            }
#pragma unroll
            for (int r = 0; r < kRowsInFlight; ++r) {
                // logit in base 2, reduced over the row's lanes
                const float z = group_sum<LPR>(lane_dot(qh, kk[r])) * a.qscale;
                if (ok[r]) {
                    if (z > m) {
                        const float corr = __builtin_amdgcn_exp2f(m - z);
                        l *= corr;
#pragma unroll
                        for (int e = 0; e < EPL; ++e)
                            acc[e] *= corr;
                        m = z;
                    }
                    const float pr = __builtin_amdgcn_exp2f(z - m);
                    l += pr;
                    T vt[EPL];
                    __builtin_memcpy(vt, &vv[r], 16);
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[e] = fmaf(pr, to_f32(vt[e]), acc[e]);
                }
            }
        }

        // ---- 4. merge each head's row slots into the chunk partial ----
        // Every slot's (max, sum, acc) goes to LDS; one wave per head finds
        // the head's max and each slot's weight, then one thread per (head,
        // dim) sums the weighted accumulators.
        {
            const int ms = wpart * RPW + slot;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                mrg_acc[hw][ms][sub * EPL + e] = acc[e];
            if (sub == 0) {
                mrg_m[hw][ms] = m;
                mrg_l[hw][ms] = l;
            }
        }
        __syncthreads();
        for (int h2 = wave; h2 < GQ; h2 += kAttnWaves) {
            const float mv = lane < NS ? mrg_m[h2][lane] : -INFINITY;
            const float M = wave_max(mv);
            const float f = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
            const float Ls = wave_sum(lane < NS ? mrg_l[h2][lane] * f : 0.f);
            if (lane < NS)
                mrg_f[h2][lane] = f;
            if (lane == 0) {
                mrg_M[h2] = M;
                mrg_L[h2] = Ls;
            }
        }
        __syncthreads();
        static_assert((GQ * D) % 64 == 0, "whole waves in the partial loop (lane pairs)");
        for (int pi = tid; pi < GQ * D; pi += kAttnThreads) {
            const int h2 = pi / D, dim = pi % D;
            float O = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2)
                O = fmaf(mrg_acc[h2][s2][dim], mrg_f[h2][s2], O);
            const float M = mrg_M[h2], Ls = mrg_L[h2];
            const size_t pc = (head0 + h2) * nchunk + c;
            // even lanes store their own and the next lane's value (the
            // next dimension of the same head) as one 64-bit access
            const float On = __uint_as_float(dpp<0xB1>(__float_as_uint(O)));
            if ((dim & 1) == 0)
                store2_agent(&a.part_o[pc * D + dim], O, On);
            if (dim == 0)
                __hip_atomic_store(reinterpret_cast<double *>(a.part_ml) + pc,
                                   __builtin_bit_cast(double, make_float2(M, Ls)),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    // Every load of the merge is issued up front: the chunk (max, sum) pairs
    // into LDS, and each thread's weighted-sum inputs into registers.
    constexpr int NCOL = GQ * D / 4;
    constexpr int NPART = kAttnThreads / NCOL;
    static_assert(NPART >= 1 && NPART * NCOL == kAttnThreads, "column split");
    constexpr int PER = kMaxChunks / NPART; // chunks per thread at most
    const int col = tid % NCOL, part = tid / NCOL;
    const int chl = col / (D / 4), d4 = col % (D / 4);
    for (int e = tid; e < GQ * nact; e += kAttnThreads) {
        const int hl = e / nact, cc = e % nact;
        const size_t pc = (head0 + hl) * nchunk + cc;
        const double ml = __hip_atomic_load(reinterpret_cast<const double *>(a.part_ml) + pc,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float2 v = __builtin_bit_cast(float2, ml);
        cmb_f[hl][cc] = v.x;
        cmb_l[hl][cc] = v.y;
    }
    const float *po = a.part_o + (head0 + chl) * nchunk * D + d4 * 4;
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    // chunk weights need the maxima; the first batch of partial sums is
    // loaded meanwhile
    constexpr int BATCH = 8;
    float4 v0[BATCH];
#pragma unroll
    for (int r = 0; r < BATCH; ++r) {
        const int cc = part + r * NPART;
        v0[r] = load4_agent(po + (size_t)(cc < nact ? cc : 0) * D);
    }
    __syncthreads();
    for (int hl = wave; hl < GQ; hl += kAttnWaves) {
        float M = -INFINITY;
        for (int cc = lane; cc < nact; cc += 64)
            M = fmaxf(M, cmb_f[hl][cc]);
        M = wave_max(M);
        float Ls = 0.f;
        for (int cc = lane; cc < nact; cc += 64) {
            const float mc = cmb_f[hl][cc];
            const float f = (mc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mc - M);
            cmb_f[hl][cc] = f;
            Ls = fmaf(cmb_l[hl][cc], f, Ls);
        }
        Ls = wave_sum(Ls);
        if (lane == 0)
            cmb_ml[hl][0] = Ls;
    }
    __syncthreads();
    for (int c0b = part; c0b < nact; c0b += BATCH * NPART) {
        float4 v[BATCH];
#pragma unroll
        for (int r = 0; r < BATCH; ++r) {
            const int cc = c0b + r * NPART;
            v[r] = c0b == part ? v0[r] : load4_agent(po + (size_t)(cc < nact ? cc : 0) * D);
        }
#pragma unroll
        for (int r = 0; r < BATCH; ++r) {
            const int cc = c0b + r * NPART;
            const float f = cc < nact ? cmb_f[chl][cc] : 0.f;
            s4.x = fmaf(v[r].x, f, s4.x);
            s4.y = fmaf(v[r].y, f, s4.y);
            s4.z = fmaf(v[r].z, f, s4.z);
            s4.w = fmaf(v[r].w, f, s4.w);
        }
    }
    red[part * NCOL + col] = s4;
    (void)PER;
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
