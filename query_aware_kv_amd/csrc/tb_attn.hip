// tb_attn.hip -- exact softmax attention over the selected K/V rows (gfx950).
//
// TokenButler abstract (2026) and gist.science technical summary,
// Significance: the full KV cache stays resident and each decode step reads
// only the selected tokens; attention over them is ordinary softmax attention.
//
// Grid: (chunk, KV head, sequence); a chunk is kAttnChunk positions, or two
// or four times that past 64K positions (attn_chunk_len).  A work-group
// handles one KV head and one chunk for all the query heads that share it
// (GQA).  With bitmaps a chunk is every nchunk-th 32-position word of the
// row, so each work-group takes an equal share of any dense region (an
// always-kept window, the sink, new tokens); with lists it is a contiguous
// range, located in the lists by binary search.
//   1. Each query head is served by 8/GQ of the eight waves, each wave taking
//      a part of the chunk.  A wave's membership words come, one per lane,
//      either straight from the head's selection bitmap (one 32-bit word per
//      32 positions) or from its ascending selection list (the chunk's
//      segment is located by a wave-parallel search, 64 samples per round,
//      and scattered into an LDS bitmap); the always-kept range
//      [keep_from, n) is added to every head.
//   2. Two consecutive words are the 64-bit mask of 64 positions, so the
//      wave compacts its positions from scalar masks with no ballot and no
//      work-group barrier.  Rows that several query heads of the group
//      select are requested by sibling waves of the same work-group, and the
//      repeats are served from L2 as long as the siblings stay close.  With
//      one work-group per compute unit they do.  With several per unit each
//      head's waves run at their own pace and drift apart, so there (16-bit
//      rows of 128) the waves walk their parts in steps of 128
//      positions with a work-group barrier after each step.
//   3. Rows stream through the lanes in 16-byte pieces (D*elt/16 lanes per
//      row, several rows per wave, four rows in flight per row slot); each row
//      slot keeps an online softmax (running max, sum, fp32 accumulator) for
//      its wave's head in base 2, rescaling only when the running max grows.
//      Lane dot products use v_dot2 on bf16 pairs and are reduced across the
//      row's lanes with DPP row permutations.
//   4. The row slots of a wave are merged in registers (DPP and the
//      permlane swaps), the waves of a head through LDS, into one partial
//      (max, sum, acc[D]) per query head and chunk.
//   5. The last work-group of a (sequence, KV head) to arrive (device-scope
//      counter) merges the chunk partials -- max and weights first, then the
//      weighted sums with all of its threads -- writes the output rows, and
//      resets the counter to zero for the next call.  A row of one chunk
//      writes its output directly.
// Reuse steps of the fused step append their few new rows inside this
// launch: one more work-group per (sequence, KV head), dispatched after all
// attention work-groups, stores them in the caches and projects their keys,
// while the attention work-groups read those positions from k_new / v_new.
#include "tb_attn_common.h"

#include <atomic>

namespace tb {
namespace {

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
// rows per row slot loaded before use: 4 where the windowed walk keeps eight
// waves per SIMD (64 registers), 8 where a work-group has its unit alone
template <int WIN> constexpr int rows_in_flight() { return WIN > 0 ? 4 : 8; }

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
    int q_per_imp_log2; // log2(Hq / Himp)
    float qscale;
    float *part_o;     // [b*Hq][nchunk][D]
    float *part_ml;    // [b*Hq][nchunk][2]
    uint32_t *counters;
    void *out;
    // rows appended by this launch (reuse steps): copied and projected by
    // one extra work-group per (sequence, KV head), read from k_new / v_new
    const void *k_new, *v_new, *w;
    void *k_store, *v_store, *kp;
    int n_new, d_imp;
    int nchunk, batch; // chunks per row and sequences (the 1-D grid of an appending launch)
};

constexpr int kAttnMaxAppend = 8; // rows an attention launch appends
constexpr int kAttnMaxDImp = 32;

// LDS of the append work-group: W and the new key rows, in the storage type.
template <typename T, int D> struct AppendLds {
    T w[D * kAttnMaxDImp];
    T k[kAttnMaxAppend][D];
};

// The extra work-group of a (sequence b, KV head g): stores the new rows in
// the caches and their projected keys (fp64 fma over head_dim in ascending
// order, rounded once to the storage type, as every projection path does).
// W and the key rows are staged in LDS first, so each output's serial fma
// chain reads its operands there.  The attention work-groups of the same
// launch read these rows from k_new / v_new, never from the cache rows being
// written.
template <typename T, int D>
__device__ void append_rows(const AttnArgs &a, int b, int g, AppendLds<T, D> &S)
{
    const int n = clamp_len(a.ctx_len[b], a.cap);
    const int nfresh = a.n_new < n ? a.n_new : n; // appended rows present in [0, n)
    const size_t src0 = ((size_t)b * a.Hkv + g) * a.n_new + (a.n_new - nfresh);
    const size_t dst0 = ((size_t)b * a.Hkv + g) * a.cap + (n - nfresh);
    constexpr int RP = D * (int)sizeof(T) / 16; // 16-byte pieces per row
    const int wp = D * a.d_imp * (int)sizeof(T) / 16;
    for (int e = threadIdx.x; e < wp; e += kAttnThreads)
        reinterpret_cast<uint4 *>(S.w)[e] = reinterpret_cast<const uint4 *>(a.w)[e];
    for (int e = threadIdx.x; e < nfresh * RP; e += kAttnThreads) {
        const int r = e / RP, p = e % RP;
        const uint4 kv = reinterpret_cast<const uint4 *>((const T *)a.k_new + (src0 + r) * D)[p];
        const uint4 vv = reinterpret_cast<const uint4 *>((const T *)a.v_new + (src0 + r) * D)[p];
        reinterpret_cast<uint4 *>((T *)a.k_store + (dst0 + r) * D)[p] = kv;
        reinterpret_cast<uint4 *>((T *)a.v_store + (dst0 + r) * D)[p] = vv;
        reinterpret_cast<uint4 *>(S.k[r])[p] = kv;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nfresh * a.d_imp; e += kAttnThreads) {
        const int r = e / a.d_imp, j = e % a.d_imp;
        double acc = 0.0;
#pragma unroll 16
        for (int i = 0; i < D; ++i)
            acc = fma(to_f64(S.k[r][i]), to_f64(S.w[i * a.d_imp + j]), acc);
        ((T *)a.kp)[(dst0 + r) * a.d_imp + j] = from_f64<T>(acc);
    }
}

// The windowed walk is built where it keeps eight waves per SIMD (four
// work-groups per compute unit) without spills: 16-bit storage, head_dim 128
// and at least two query heads per KV head (a lone head shares no rows).
template <typename T, int D, int GQ> constexpr bool attn_windowed_ok()
{
    return sizeof(T) == 2 && D == 128 && GQ >= 2;
}

template <typename T, int D, int GQ, bool BITMAP, int WIN, bool APPEND, int CH>
__global__ __launch_bounds__(kAttnThreads)
__attribute__((amdgpu_waves_per_eu(WIN > 0 && !APPEND ? 8 : 1))) void attn_kernel(AttnArgs a)
{
    constexpr int EPL = 16 / (int)sizeof(T); // elements per lane piece
    constexpr int LPR = D / EPL;             // lanes per row
    constexpr int RPW = 64 / LPR;            // rows per wave step
    constexpr int NWD = CH / 32;             // bitmap words per head
    constexpr int RIF = rows_in_flight<WIN>();
    static_assert(GQ <= kAttnWaves && kAttnWaves % GQ == 0, "whole waves per query head");
    constexpr int WPH = kAttnWaves / GQ;     // waves per query head
    constexpr int PW = CH / WPH;             // positions of one wave's part of the chunk
    static_assert(PW % 64 == 0, "parts of whole 64-position masks");

    __shared__ uint32_t bm[GQ][NWD];
    __shared__ uint16_t hlist[kAttnWaves][PW]; // positions of each wave's part
    __shared__ float mrg_m[GQ][WPH];
    __shared__ float mrg_l[GQ][WPH];
    __shared__ float mrg_acc[GQ][WPH][D];
    // the append work-group uses the merge's LDS, which it never reaches
    // chunks of a row: at most 64 of 1024 positions (rows up to 64K), else
    // at most kMaxCtxCap / CH
    constexpr int NCH = (CH == kAttnChunk ? 65536 : kMaxCtxCap) / CH;
    __shared__ union {
        CombineLds<GQ, kAttnThreads, NCH> c;
        AppendLds<T, D> app;
    } shu;
    CombineLds<GQ, kAttnThreads, NCH> &cmb = shu.c;

    const T *__restrict__ q = (const T *)a.q;
    const T *__restrict__ kc = (const T *)a.k;
    const T *__restrict__ vc = (const T *)a.v;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    static_assert(!APPEND || BITMAP, "appending launches read bitmaps");
    // An appending launch has a 1-D grid: the attention work-groups in
    // (chunk, KV head, sequence) order, then one append work-group per
    // (sequence, KV head), dispatched last so that they land beside the
    // attention work-groups instead of displacing them.
    int c, g, b, nchunk;
    if constexpr (APPEND) {
        nchunk = a.nchunk;
        const int id = blockIdx.x, nattn = nchunk * a.Hkv * a.batch;
        if (id >= nattn) {
            append_rows<T, D>(a, (id - nattn) / a.Hkv, (id - nattn) % a.Hkv, shu.app);
            return;
        }
        c = id % nchunk;
        g = (id / nchunk) % a.Hkv;
        b = id / (nchunk * a.Hkv);
    } else {
        c = blockIdx.x;
        g = blockIdx.y;
        b = blockIdx.z;
        nchunk = gridDim.x;
    }
    const int c0 = c * CH;
    // The work-group's 32 bitmap words: in bitmap mode the words c,
    // c + nchunk, c + 2 nchunk, ... of the row (so every work-group takes an
    // equal share of any dense region: an always-kept window, the sink, new
    // tokens); in list mode the contiguous words of positions
    // [c0, c0 + CH).  A chunk-local position 32 k + j (word k, bit j)
    // is row position 32 gword(k) + j.
    auto gword = [&](int k) { return BITMAP ? c + nchunk * k : c * NWD + k; };
    auto gpos = [&](uint32_t local) {
        return 32u * (uint32_t)gword((int)(local >> 5)) + (local & 31u);
    };
    const size_t head0 = (size_t)b * a.Hq + (size_t)g * GQ; // first query head of the group
    const int slot = lane / LPR, sub = lane % LPR;

    // Wave w serves query head hw = w / WPH on part wpart = w % WPH of the
    // chunk: chunk-local positions [wpart * PW, (wpart + 1) * PW), which are
    // the chunk's words wpart * WPW .. + WPW - 1, one per lane.
    const int hw = wave / WPH, wpart = wave % WPH;
    constexpr int WPW = PW / 32;
    static_assert(WPW <= 64 && WPW % 2 == 0, "a part's words fit one wave, in pairs");
    // Windowed walk (WIN > 0): the waves cover their parts in
    // steps of WIN word pairs and meet at a barrier after each step, so all
    // query heads of the group read a shared row within a short time of
    // each other and the later reads find it in L2.  wend holds the end of
    // each step in the wave's position list.
    static_assert(WIN == 0 || (WPW / 2) % WIN == 0, "whole steps per part");
    constexpr int NWIN = WIN > 0 ? WPW / 2 / WIN : 1;
    __shared__ uint16_t wend[kAttnWaves][NWIN];
    // Everything that does not depend on the lengths is requested first: the
    // q slice of this lane for the wave's head (kept in the storage type;
    // bf16 pairs feed v_dot2) and, in bitmap mode, this lane's word.
    const uint4 qh = *reinterpret_cast<const uint4 *>(q + (head0 + hw) * D + sub * EPL);
    const int p0w = 32 * gword(wpart * WPW + lane); // first position of this lane's word
    uint32_t word = 0u;
    if constexpr (BITMAP) {
        // query head h follows importance head h / (Hq / Himp), a power-of-two
        // ratio; the load is unconditional (a word past the row reads the
        // row's first) and masked afterwards
        const int i = (g * GQ + hw) >> a.q_per_imp_log2;
        const uint32_t wv = a.sel_bits[((size_t)b * a.Himp + i) * a.bits_stride +
                                       (p0w < a.cap ? p0w >> 5 : 0)];
        word = wv & (0u - (uint32_t)(lane < WPW && p0w < a.cap));
    }
    const int kf_raw = a.keep_from != nullptr ? a.keep_from[b] : a.cap;
    const int n = clamp_len(a.ctx_len[b], a.cap);
    // positions of the chunk are below c1 (and those of a word below n)
    const int c1 = BITMAP ? n : min(c0 + CH, n);
    const bool active = BITMAP ? 32 * c < n : c0 < n;
    const int nact = BITMAP ? min(nchunk, (n + 31) / 32) : (n + CH - 1) / CH;

    if (active) {
        // ---- 1. the wave's membership words ----
        const int kf = clamp_len(kf_raw, n);
        if constexpr (!BITMAP) {
            // list mode: the group's lists are scattered into an LDS bitmap first
            for (int e = tid; e < GQ * NWD; e += kAttnThreads)
                (&bm[0][0])[e] = 0u;
            __syncthreads();
            for (int hl = wave; hl < GQ; hl += kAttnWaves) {
                const int h = g * GQ + hl;
                const int i = h >> a.q_per_imp_log2;
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
            __syncthreads();
            if (lane < WPW)
                word = bm[hw][wpart * WPW + lane];
        }
        if (lane < WPW) {
            // clip to the chunk's positions below c1 and add the always-kept
            // range [kf, n)
            const int lo = max(kf, p0w), hi = min(c1, p0w + 32);
            if (hi - p0w < 32)
                word &= hi <= p0w ? 0u : ((1u << (hi - p0w)) - 1u);
            if (lo < hi) {
                const uint32_t upto = hi - p0w == 32 ? 0xffffffffu : ((1u << (hi - p0w)) - 1u);
                word |= upto & ~((1u << (lo - p0w)) - 1u);
            }
        }

        // ---- 2. the wave's positions, in order ----
        // Two consecutive words are the 64-bit membership mask of 64
        // positions; a lane's slot is the count of set bits below it.
        uint32_t nh = 0u;
#pragma unroll
        for (int k = 0; k < WPW / 2; ++k) {
            const uint32_t m_lo = __builtin_amdgcn_readlane(word, 2 * k);
            const uint32_t m_hi = __builtin_amdgcn_readlane(word, 2 * k + 1);
            const uint64_t msk = (uint64_t)m_lo | ((uint64_t)m_hi << 32);
            if ((msk >> lane) & 1ull)
                hlist[wave][nh + __builtin_amdgcn_mbcnt_hi(m_hi, __builtin_amdgcn_mbcnt_lo(m_lo, 0u))] =
                    (uint16_t)(wpart * PW + 64 * k + lane);
            nh += (uint32_t)__popcll(msk);
            if constexpr (WIN > 0)
                if (k % WIN == WIN - 1 && lane == 0)
                    wend[wave][k / WIN] = (uint16_t)nh;
        }
        // the list is written and read by this wave only
        __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();

        // ---- 3. stream the wave's rows ----
        float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[e] = 0.f;
        const size_t kvbase = ((size_t)b * a.Hkv + g) * a.cap;
        const T *kb = kc + kvbase * D + sub * EPL;
        const T *vb = vc + kvbase * D + sub * EPL;
        // appending launch: rows from t_new on come from k_new / v_new
        int t_new = 0;
        const T *knb = nullptr, *vnb = nullptr;
        if constexpr (APPEND) {
            const int nfresh = a.n_new < n ? a.n_new : n;
            t_new = n - nfresh;
            const size_t src0 = ((size_t)b * a.Hkv + g) * a.n_new + (a.n_new - nfresh);
            knb = (const T *)a.k_new + src0 * D + sub * EPL;
            vnb = (const T *)a.v_new + src0 * D + sub * EPL;
        }

        // All of a slot's rows (up to RIF) are requested before any
        // is used.  The loads are unconditional -- a missing row reads the
        // chunk's first position, which always exists, and is given weight
        // 0 -- so they issue back to back.
        uint32_t lo = 0u;
#pragma unroll 1
        for (int wi = 0; wi < NWIN; ++wi) {
            const uint32_t hi =
                WIN > 0 ? __builtin_amdgcn_readfirstlane((uint32_t)wend[wave][wi]) : nh;
            for (uint32_t base = lo + slot; base < hi; base += RIF * RPW) {
                uint32_t pos[RIF];
                bool ok[RIF];
                uint4 kk[RIF], vv[RIF];
#pragma unroll
                for (int r = 0; r < RIF; ++r) {
                    const uint32_t u = base + r * RPW;
                    ok[r] = u < hi;
                    pos[r] = gpos(ok[r] ? hlist[wave][u] : 0u);
                }
#pragma unroll
                for (int r = 0; r < RIF; ++r) {
                    const T *kr = kb + (size_t)pos[r] * D, *vr = vb + (size_t)pos[r] * D;
                    if constexpr (APPEND)
                        if (pos[r] >= (uint32_t)t_new) {
                            kr = knb + (size_t)(pos[r] - t_new) * D;
                            vr = vnb + (size_t)(pos[r] - t_new) * D;
                        }
                    kk[r] = *reinterpret_cast<const uint4 *>(kr);
                    vv[r] = *reinterpret_cast<const uint4 *>(vr);
                }
#pragma unroll
                for (int r = 0; r < RIF; ++r) {
                    // logit in base 2, reduced over the row's lanes
                    const float z = group_sum<LPR>(lane_dot<T>(qh, kk[r])) * a.qscale;
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
            if constexpr (WIN > 0)
                __syncthreads();
            lo = hi;
        }

        // ---- 4. merge each head's row slots into the chunk partial ----
        // A wave's row slots merge in registers (DPP and the permlane
        // swaps); the head's waves then meet in LDS, one thread per (head,
        // dim) weighting each wave's accumulator by its max.
        {
            auto fmax2 = [](float x, float y) { return fmaxf(x, y); };
            auto add2 = [](float x, float y) { return x + y; };
            const float M = across_slots<LPR>(m, fmax2);
            const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
            const float L = across_slots<LPR>(l * f, add2);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[e] = across_slots<LPR>(acc[e] * f, add2);
            if (slot == 0) {
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    mrg_acc[hw][wpart][sub * EPL + e] = acc[e];
                if (sub == 0) {
                    mrg_m[hw][wpart] = M;
                    mrg_l[hw][wpart] = L;
                }
            }
        }
        __syncthreads();
        static_assert((GQ * D) % 64 == 0, "whole waves in the partial loop (lane pairs)");
        for (int pi = tid; pi < GQ * D; pi += kAttnThreads) {
            const int h2 = pi / D, dim = pi % D;
            float M = -INFINITY;
#pragma unroll
            for (int pp = 0; pp < WPH; ++pp)
                M = fmaxf(M, mrg_m[h2][pp]);
            float O = 0.f, Ls = 0.f;
#pragma unroll
            for (int pp = 0; pp < WPH; ++pp) {
                const float mp = mrg_m[h2][pp];
                const float f = mp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp - M);
                O = fmaf(mrg_acc[h2][pp][dim], f, O);
                Ls = fmaf(mrg_l[h2][pp], f, Ls);
            }
            if (nchunk == 1) {
                // the only chunk: its partial is the result (what the merge
                // of one partial computes, bit for bit)
                const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
                reinterpret_cast<T *>(a.out)[(head0 + h2) * D + dim] = from_f32<T>(O * inv);
            } else {
                publish_partial<D>(a.part_o, a.part_ml, (head0 + h2) * nchunk + c, dim, O, M,
                                   Ls);
            }
        }
    } else if (nchunk == 1) {
        // an empty row: zero outputs, as the merge of no partials gives
        for (int pi = tid; pi < GQ * D; pi += kAttnThreads)
            reinterpret_cast<T *>(a.out)[head0 * D + pi] = from_f32<T>(0.f);
    }

    // ---- 5. arrival; the last work-group of this (b, g) merges the chunks ----
    if (nchunk > 1)
        arrive_and_combine<T, D, GQ, kAttnThreads, NCH>(
            cmb, &a.counters[(size_t)b * a.Hkv + g], a.part_o, a.part_ml, nchunk,
            nact, head0, (T *)a.out);
}

// Word pairs per step of the windowed walk.
constexpr int kAttnWindowPairs = 2;



template <typename T, int D, int GQ, bool BITMAP, bool APPEND, int CH>
hipError_t attn_launch_ch(const tb_shape &s, const AttnArgs &a, hipStream_t st)
{
    const int nchunk = attn_chunks(s);
    const dim3 grid = APPEND ? dim3((nchunk + 1) * s.n_kv_heads * s.batch)
                             : dim3(nchunk, s.n_kv_heads, s.batch);
    // With two or more work-groups per compute unit the others fill the
    // SIMDs while one waits at a window barrier, and the group's query heads
    // then share their rows through L2 instead of re-reading them from HBM.
    // With one work-group per unit the waits would idle it.
    int cus = 0;
    const hipError_t e = device_cus(cus);
    if (e != hipSuccess)
        return e;
    const long wgs = (long)nchunk * s.n_kv_heads * s.batch;
    bool windowed = false;
    if constexpr (attn_windowed_ok<T, D, GQ>())
        windowed = wgs >= 2L * cus;
    if constexpr (attn_windowed_ok<T, D, GQ>())
        if (windowed)
            hipLaunchKernelGGL((attn_kernel<T, D, GQ, BITMAP, kAttnWindowPairs, APPEND, CH>), grid,
                               dim3(kAttnThreads), 0, st, a);
    if (!windowed)
        hipLaunchKernelGGL((attn_kernel<T, D, GQ, BITMAP, 0, APPEND, CH>), grid,
                           dim3(kAttnThreads), 0, st, a);
    return hipGetLastError();
}

template <typename T, int D, int GQ, bool BITMAP, bool APPEND>
hipError_t attn_launch_t(const tb_shape &s, const AttnArgs &a, hipStream_t st)
{
    // (four times kAttnChunk needs at least two waves per query head)
    if constexpr (GQ <= 4)
        if (attn_chunk_len(s) == 4 * kAttnChunk)
            return attn_launch_ch<T, D, GQ, BITMAP, APPEND, 4 * kAttnChunk>(s, a, st);
    if (attn_chunk_len(s) == 2 * kAttnChunk)
        return attn_launch_ch<T, D, GQ, BITMAP, APPEND, 2 * kAttnChunk>(s, a, st);
    return attn_launch_ch<T, D, GQ, BITMAP, APPEND, kAttnChunk>(s, a, st);
}

template <typename T, int D, int GQ>
hipError_t attn_t(const tb_shape &s, const AttnArgs &a, hipStream_t st)
{
    if (a.sel_bits != nullptr)
        return a.n_new > 0 ? attn_launch_t<T, D, GQ, true, true>(s, a, st)
                           : attn_launch_t<T, D, GQ, true, false>(s, a, st);
    return attn_launch_t<T, D, GQ, false, false>(s, a, st);
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

// Compute units of the current device, queried once per device.
hipError_t device_cus(int &cus)
{
    static std::atomic<int> known[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    cus = dev < 64 ? known[dev].load(std::memory_order_relaxed) : 0;
    if (cus > 0)
        return hipSuccess;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    if (dev < 64)
        known[dev].store(cus, std::memory_order_relaxed);
    return hipSuccess;
}

hipError_t launch_attn(const tb_shape &s, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *sel_idx, int sel_stride,
                       const int32_t *sel_count, const uint32_t *sel_bits,
                       const int32_t *keep_from, const int32_t *ctx_len, float softmax_scale,
                       void *out, float *part_o, float *part_ml, uint32_t *counters,
                       hipStream_t st, const AttnAppend &app)
{
    if (app.n_new > kAttnMaxAppend || s.d_imp > kAttnMaxDImp)
        return hipErrorInvalidValue;
    if (app.n_new > 0 && (sel_bits == nullptr || app.k_new == nullptr || app.v_new == nullptr ||
                          app.w == nullptr || app.k_cache == nullptr ||
                          app.v_cache == nullptr || app.kp_cache == nullptr))
        return hipErrorInvalidValue;
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
    a.q_per_imp_log2 = 0;
    while ((s.n_imp_heads << a.q_per_imp_log2) < s.n_q_heads)
        ++a.q_per_imp_log2;
    a.qscale = softmax_scale * 1.4426950408889634f; // logits in base 2
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.counters = counters;
    a.out = out;
    a.k_new = app.k_new;
    a.v_new = app.v_new;
    a.w = app.w;
    a.k_store = app.k_cache;
    a.v_store = app.v_cache;
    a.kp = app.kp_cache;
    a.n_new = app.n_new > 0 ? app.n_new : 0;
    a.d_imp = s.d_imp;
    a.nchunk = attn_chunks(s);
    a.batch = s.batch;
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
