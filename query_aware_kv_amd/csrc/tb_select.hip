// tb_select.hip -- per-head top-B selection and neighbor fetching (gfx950).
//
// TokenButler abstract (2026) and gist.science technical summary,
// Methodology > Core Architecture: per-token selection of the highest-scoring
// tokens under a fixed budget B.  Inference Strategy > Optimizations: neighbor
// fetching widens each kept token t to [t-r, t+r].
//
// One 1024-thread work-group per (sequence, importance head):
//   1. Scores become order-preserving u32 keys (-0 folded onto +0).  Each
//      thread owns whole 32-position words of the bitmap (word w = tid +
//      j * 1024); up to two words (64 keys) per thread stay in registers, so
//      the scores are read once, with 16-byte loads.
//   2. Radix select from the top, 8 bits per pass, over the keys that match
//      the prefix found so far.  Histograms live in LDS as 16 copies (lane
//      mod 16), padded so that equal digits in different copies fall in
//      different banks: at most four lanes of a wave hit one address.  A
//      wave-wide suffix scan picks the digit holding the B-th largest key.
//      When every key of that digit is needed the search stops early.
//      Result: the threshold tau and how many keys equal to it are kept (the
//      lowest positions first).
//   3. Every thread builds its own words of the kept set T from its keys; a
//      block scan of per-word tie counts settles ties at tau by position.
//   4. Dilation by r is word-wise shifts of the bitmap, clipped to [0, n).
//   5. A block scan of per-word popcounts compacts the bitmap into the
//      ascending index list; the bitmap itself can be written out too.
#include "tb_internal.h"

namespace tb {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kCopies = 16;
constexpr int kCopyStride = 257; // words; the odd stride spreads copies over banks

__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u)
        u = 0u; // -0.0 ties with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of popcount(words[w]) over w < nw into out[w]; returns the
// total to every thread.  wsum: kSelWaves + 1 words of LDS scratch.
__device__ uint32_t block_popc_exscan(const uint32_t *words, uint32_t *out, int nw,
                                      uint32_t *wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (nw + kSelThreads - 1) / kSelThreads;
    const int w0 = tid * per;
    uint32_t local = 0;
    for (int w = w0; w < w0 + per && w < nw; ++w)
        local += __popc(words[w]);
    uint32_t inc = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(inc, off);
        if (lane >= off)
            inc += v;
    }
    if (lane == 63)
        wsum[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const uint32_t v = lane < kSelWaves ? wsum[lane] : 0u;
        uint32_t x = v;
#pragma unroll
        for (int off = 1; off < kSelWaves; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off)
                x += y;
        }
        if (lane < kSelWaves)
            wsum[lane] = x - v; // exclusive prefix of waves
        if (lane == kSelWaves - 1)
            wsum[kSelWaves] = x; // total
    }
    __syncthreads();
    uint32_t run = wsum[wave] + inc - local;
    for (int w = w0; w < w0 + per && w < nw; ++w) {
        out[w] = run;
        run += __popc(words[w]);
    }
    const uint32_t total = wsum[kSelWaves];
    __syncthreads();
    return total;
}

// Writes the positions of the set bits of words[0..nw) in ascending order.
__device__ void compact_bits(const uint32_t *words, const uint32_t *offs, int nw, int32_t *dst)
{
    for (int w = threadIdx.x; w < nw; w += kSelThreads) {
        uint32_t bits = words[w];
        int pos = (int)offs[w];
        while (bits) {
            const int bi = __ffs(bits) - 1;
            dst[pos++] = w * 32 + bi;
            bits &= bits - 1u;
        }
    }
}

// Loads the 32 keys of bitmap word w (positions >= n become key 0, which is
// below every real key and never counted).  Whole words of 16-byte aligned
// rows use four-float loads; a partial last word, or a row whose start is
// not 16-byte aligned, is read one float at a time without touching
// positions >= n.
__device__ __forceinline__ void load_word_keys(const float *row, int w, int n, bool vec,
                                               uint32_t (&k)[32])
{
    const int p0 = w * 32;
    if (vec && p0 + 32 <= n) {
        const float4 *src = reinterpret_cast<const float4 *>(row + p0);
        float4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = src[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            k[4 * i + 0] = score_key(v[i].x);
            k[4 * i + 1] = score_key(v[i].y);
            k[4 * i + 2] = score_key(v[i].z);
            k[4 * i + 3] = score_key(v[i].w);
        }
    } else {
        float f[32];
#pragma unroll
        for (int e = 0; e < 32; ++e)
            f[e] = row[p0 + e < n ? p0 + e : 0];
#pragma unroll
        for (int e = 0; e < 32; ++e)
            k[e] = p0 + e < n ? score_key(f[e]) : 0u;
    }
}

template <int WPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx_len, int Himp, int cap,
    int nwc, int B, int r, int32_t *__restrict__ sel_idx, int sel_stride,
    int32_t *__restrict__ sel_count, int32_t *__restrict__ topb_idx,
    uint32_t *__restrict__ sel_bits, int bits_stride, int32_t *__restrict__ keep_from, int n_new)
{
    extern __shared__ uint32_t lds[];
    uint32_t *hist = lds;                         // [kCopies][kCopyStride]
    uint32_t *tot = hist + kCopies * kCopyStride; // [256]
    uint32_t *misc = tot + 256;                   // 64 words
    uint32_t *Tb = misc + 64;                     // [nwc] kept set
    uint32_t *Sb = Tb + nwc;                      // [nwc] widened set / tie bits
    uint32_t *Xb = Sb + nwc;                      // [nwc] dilation ping-pong
    uint32_t *scan = Xb + nwc;                    // [nwc] scan output

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y, i = blockIdx.x;
    const size_t rowid = (size_t)b * Himp + i;
    const float *row = scores + rowid * cap;
    const int n = clamp_len(ctx_len[b], cap);
    int32_t *out_sel = sel_idx + rowid * sel_stride;
    if (keep_from != nullptr && i == 0 && tid == 0)
        keep_from[b] = n - n_new > 0 ? n - n_new : 0;
    if (n == 0) {
        if (tid == 0)
            sel_count[rowid] = 0;
        if (sel_bits != nullptr)
            for (int w = tid; w < bits_stride; w += kSelThreads)
                sel_bits[rowid * bits_stride + w] = 0u;
        return;
    }
    const int nw = (n + 31) >> 5;
    const int nwt = (nw + kSelThreads - 1) / kSelThreads; // words per thread (global mode)
    const bool vec = (cap & 3) == 0; // every row starts 16-byte aligned

    // Keys of this thread: keys[j][bit] is position (tid + j * kSelThreads) * 32 + bit.
    constexpr int WR = WPT > 0 ? WPT : 1;
    uint32_t keys[WR][32];
    if constexpr (WPT > 0) {
#pragma unroll
        for (int j = 0; j < WR; ++j)
            load_word_keys(row, tid + j * kSelThreads, n, vec, keys[j]);
    }

    const bool take_all = B >= n;
    uint32_t tau = 0u, fmask = 0u, need = 0u, cnt_eq = 0u;
    if (!take_all) {
        for (int e = tid; e < kCopies * kCopyStride; e += kSelThreads)
            hist[e] = 0u;
        __syncthreads();
        uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)B;
        uint32_t *h = hist + (lane & (kCopies - 1)) * kCopyStride;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            // key 0 marks a position >= n; real keys are never 0
            auto count = [&](const uint32_t (&k)[32]) {
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    if (k[e] != 0u && (k[e] & pmask) == prefix)
                        atomicAdd(&h[(k[e] >> shift) & 255u], 1u);
            };
            if constexpr (WPT > 0) {
#pragma unroll
                for (int j = 0; j < WR; ++j)
                    count(keys[j]);
            } else {
                for (int j = 0; j < nwt; ++j) {
                    uint32_t k[32];
                    load_word_keys(row, tid + j * kSelThreads, n, vec, k);
                    count(k);
                }
            }
            __syncthreads();
            if (tid < 256) {
                uint32_t cnt = 0u;
#pragma unroll
                for (int cp = 0; cp < kCopies; ++cp) {
                    cnt += hist[cp * kCopyStride + tid];
                    hist[cp * kCopyStride + tid] = 0u; // ready for the next pass
                }
                tot[tid] = cnt;
            }
            __syncthreads();
            if (wave == 0) {
                const uint32_t c0 = tot[4 * lane], c1 = tot[4 * lane + 1];
                const uint32_t c2 = tot[4 * lane + 2], c3 = tot[4 * lane + 3];
                const uint32_t sl = c0 + c1 + c2 + c3;
                uint32_t suf = sl; // inclusive suffix sum over lanes
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t v = __shfl_down(suf, off);
                    if (lane + off < 64)
                        suf += v;
                }
                const unsigned long long m = __ballot(suf >= krem);
                const int L = 63 - __clzll(m);
                if (lane == L) {
                    uint32_t above = suf - sl;
                    uint32_t dg, cd;
                    if (above + c3 >= krem) {
                        dg = 4u * L + 3u;
                        cd = c3;
                    } else if (above + c3 + c2 >= krem) {
                        above += c3;
                        dg = 4u * L + 2u;
                        cd = c2;
                    } else if (above + c3 + c2 + c1 >= krem) {
                        above += c3 + c2;
                        dg = 4u * L + 1u;
                        cd = c1;
                    } else {
                        above += c3 + c2 + c1;
                        dg = 4u * L;
                        cd = c0;
                    }
                    misc[0] = prefix | (dg << shift);
                    misc[1] = krem - above;
                    misc[2] = cd;
                }
            }
            __syncthreads();
            prefix = misc[0];
            krem = misc[1];
            cnt_eq = misc[2];
            pmask |= 255u << shift;
            if (krem == cnt_eq)
                break; // every key with this prefix is kept
        }
        tau = prefix;
        fmask = pmask;
        need = krem; // keys equal to tau (under fmask) kept, lowest positions first
    }
    const bool partial_ties = !take_all && need < cnt_eq;

    // ---- kept-set bitmap (and tie bitmap when ties are split) ----
    auto emit = [&](int w, const uint32_t (&k)[32]) {
        if (w >= nw)
            return;
        uint32_t gt = 0u, eq = 0u;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const uint32_t km = k[e] & fmask;
            const bool valid = k[e] != 0u;
            const bool in = valid && (take_all || km > tau || (!partial_ties && km == tau));
            const bool tie = valid && partial_ties && km == tau;
            gt |= (uint32_t)in << e;
            eq |= (uint32_t)tie << e;
        }
        Tb[w] = gt;
        Sb[w] = eq;
    };
    if constexpr (WPT > 0) {
#pragma unroll
        for (int j = 0; j < WR; ++j)
            emit(tid + j * kSelThreads, keys[j]);
    } else {
        for (int j = 0; j < nwt; ++j) {
            uint32_t k[32];
            load_word_keys(row, tid + j * kSelThreads, n, vec, k);
            emit(tid + j * kSelThreads, k);
        }
    }
    __syncthreads();
    if (partial_ties) {
        block_popc_exscan(Sb, scan, nw, misc + 8);
        for (int w = tid; w < nw; w += kSelThreads) {
            uint32_t e = Sb[w];
            const uint32_t pre = scan[w];
            if (pre >= need) {
                e = 0u;
            } else if (pre + __popc(e) > need) {
                uint32_t m = e;
                for (uint32_t c = need - pre; c > 0u; --c)
                    m &= m - 1u;
                e ^= m; // the lowest (need - pre) tie bits
            }
            Tb[w] |= e;
        }
        __syncthreads();
    }

    // ---- optional pre-widening output ----
    if (topb_idx != nullptr) {
        block_popc_exscan(Tb, scan, nw, misc + 8);
        compact_bits(Tb, scan, nw, topb_idx + rowid * (size_t)B);
        __syncthreads();
    }

    // ---- neighbor fetching: dilate T by r within [0, n) ----
    const uint32_t *fin = Tb;
    if (r > 0) {
        const uint32_t *src = Tb;
        uint32_t *dst = Sb;
        int left = r;
        while (left > 0) {
            const int step = left < 31 ? left : 31;
            for (int w = tid; w < nw; w += kSelThreads) {
                const uint32_t x = src[w];
                const uint32_t prv = w > 0 ? src[w - 1] : 0u;
                const uint32_t nxt = w + 1 < nw ? src[w + 1] : 0u;
                uint32_t res = x;
                for (int s2 = 1; s2 <= step; ++s2)
                    res |= (x << s2) | (prv >> (32 - s2)) | (x >> s2) | (nxt << (32 - s2));
                if (w == nw - 1 && (n & 31))
                    res &= (1u << (n & 31)) - 1u;
                dst[w] = res;
            }
            __syncthreads();
            left -= step;
            fin = dst;
            src = dst;
            dst = (dst == Sb) ? Xb : Sb;
        }
    }

    // ---- compaction into the ascending list (and the bitmap, if asked) ----
    const uint32_t total = block_popc_exscan(fin, scan, nw, misc + 8);
    compact_bits(fin, scan, nw, out_sel);
    if (sel_bits != nullptr)
        for (int w = tid; w < bits_stride; w += kSelThreads)
            sel_bits[rowid * bits_stride + w] = w < nw ? fin[w] : 0u;
    if (tid == 0)
        sel_count[rowid] = (int32_t)total;
}

template <int WPT>
hipError_t select_t(const tb_shape &s, const tb_select_params &p, const float *scores,
                    const int32_t *ctx_len, int32_t *sel_idx, int sel_stride,
                    int32_t *sel_count, int32_t *topb_idx, uint32_t *sel_bits,
                    int32_t *keep_from, int n_new, hipStream_t st)
{
    const int nwc = (s.ctx_cap + 31) / 32 + 1;
    const size_t lds =
        ((size_t)kCopies * kCopyStride + 256 + 64 + 4 * (size_t)nwc) * sizeof(uint32_t);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)select_kernel<WPT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    dim3 grid(s.n_imp_heads, s.batch);
    hipLaunchKernelGGL(select_kernel<WPT>, grid, dim3(kSelThreads), lds, st, scores, ctx_len,
                       s.n_imp_heads, s.ctx_cap, nwc, p.budget, p.radius, sel_idx, sel_stride,
                       sel_count, topb_idx, sel_bits, bitmap_words(s.ctx_cap), keep_from,
                       n_new);
    return hipGetLastError();
}

} // namespace

hipError_t launch_select(const tb_shape &s, const tb_select_params &p, const float *scores,
                         const int32_t *ctx_len, int32_t *sel_idx, int sel_stride,
                         int32_t *sel_count, int32_t *topb_idx, uint32_t *sel_bits,
                         int32_t *keep_from, int n_new, hipStream_t st)
{
#define TB_SEL_ARGS                                                                          \
    s, p, scores, ctx_len, sel_idx, sel_stride, sel_count, topb_idx, sel_bits, keep_from, n_new, st
    const int words = (s.ctx_cap + 31) / 32;
    if (words <= kSelThreads) return select_t<1>(TB_SEL_ARGS);
    if (words <= 2 * kSelThreads) return select_t<2>(TB_SEL_ARGS);
    return select_t<0>(TB_SEL_ARGS);
#undef TB_SEL_ARGS
}

} // namespace tb
