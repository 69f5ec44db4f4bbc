// tb_select.hip -- per-head top-B selection and neighbor fetching (gfx950).
//
// TokenButler abstract (2026) and gist.science technical summary,
// Methodology > Core Architecture: per-token selection of the highest-scoring
// tokens under a fixed budget B.  Inference Strategy > Optimizations: neighbor
// fetching widens each kept token t to [t-r, t+r].
//
// One work-group per (sequence, importance head): 1024 threads, or 512 for
// rows of up to 512 words on the 16-bit-key path (two such work-groups fit a
// compute unit).  Thread t owns bitmap words w = t + THREADS j, i.e. the 32
// positions 32w .. 32w+31.
//   1. Scores become order-preserving u32 keys (-0 folded onto +0; positions
//      >= n get key 0, below every real key).  Rows of up to 1024 words keep
//      their keys in registers (read once, in 16-byte loads); longer rows
//      re-read them (from L2) at each pass.  In the fused step the score
//      launch has also stored the top 16 bits of every key, within each
//      32-position word in pair order (positions j and j + 16 side by side),
//      and compactly for positions 8m; rows of up to 1024 words then take
//      step 2's sample and first pass from those (half the bytes, the sample
//      requested first), classify two keys per packed 16-bit op, and read
//      full keys only for the candidates and the fallback.
//   2. The B-th largest key tau is bracketed from a sample of one position in
//      eight (positions 8m): the sample goes into a 4096-bin histogram of the
//      keys' top 12 bits, and two bins a safe margin either side of the
//      sample quantile B/m (m: positions competing) bound a candidate range.
//      One compare-only pass marks the keys above it (kept) and in it; each
//      wave lists its candidates' positions in LDS, re-reads their keys with
//      its lanes sharing the reads evenly, and counts them by their top 20
//      bits.  When tau provably lies in the range and the candidates fit,
//      that histogram gives tau's top 20 bits; candidates above them are
//      kept, and the few sharing them are ranked by one wave (a histogram
//      of their low 12 bits when more than 64 share them).  Otherwise a
//      radix select runs over every key: from the top, 8 bits per pass, over
//      the keys that match the prefix found so far, with the histogram in
//      LDS as 16 copies (lane mod 16) padded so that equal digits in
//      different copies fall in different banks; a wave-wide suffix sum picks
//      the digit holding the wanted key, and the search stops early when
//      every key of that digit is needed.  Result: the threshold tau and how
//      many keys equal to it are kept (the lowest positions first).  Either
//      route gives the same tau.
//   3. Every thread builds its own words of the kept set T from its keys; a
//      block scan of per-word tie counts settles ties at tau by position.
//   4. Dilation by r is word-wise shifts of the bitmap, clipped to [0, n).
//      Inference Strategy (the three buffers): the sink [0, n_sink) and the
//      local window (the last n_local positions) are always kept; only the
//      positions between them compete for the budget (their keys are the
//      only non-zero ones), and both ranges are ORed in after the dilation.
//   5. A block count of set bits gives |S|; when the list is asked for, a
//      block scan of per-word popcounts compacts the bitmap into the
//      ascending index list.  The bitmap itself can be written out too.
#include "tb_internal.h"

#include <atomic>

namespace tb {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kCopies = 16;
constexpr int kCopyStride = 257; // words; the odd stride spreads copies over banks
constexpr int kSampleBins = 4096;
constexpr int kWaveCap = 512;       // candidates held per wave
constexpr int kBinShift = 20;       // sample bins: the top 12 bits of a key
constexpr int kMinSampleWords = 64; // shorter rows go straight to the full radix
static_assert(kSampleBins == 64 * 64 && (1u << (32 - kBinShift)) == kSampleBins,
              "64 sample bins per lane of one wave");
static_assert(kSampleBins <= kCopies * kCopyStride, "sample histogram reuses the radix one");
// misc words
constexpr int kMiscScan = 8;   // kSelWaves + 1 words of block-scan scratch
constexpr int kMiscList = 40;  // length of the list of keys sharing tau's 20-bit prefix

// Exclusive scan of popcount(words[w]) over w < nw into out[w] (skipped when
// out is NULL); returns the total to every thread.  wsum: kSelWaves words of
// LDS scratch.
template <int THREADS>
__device__ uint32_t block_popc_exscan(const uint32_t *words, uint32_t *out, int nw,
                                      uint32_t *wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (nw + THREADS - 1) / THREADS;
    const int w0 = tid * per;
    uint32_t local = 0;
    for (int w = w0; w < w0 + per && w < nw; ++w)
        local += __popc(words[w]);
    const uint32_t inc = wave_incl_scan(local, lane);
    if (lane == 63)
        wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0u, total = 0u;
#pragma unroll
    for (int v = 0; v < (THREADS / 64); ++v) {
        const uint32_t x = wsum[v];
        before += v < wave ? x : 0u;
        total += x;
    }
    if (out != nullptr) {
        uint32_t run = before + inc - local;
        for (int w = w0; w < w0 + per && w < nw; ++w) {
            out[w] = run;
            run += __popc(words[w]);
        }
    }
    __syncthreads();
    return total;
}

// Writes the positions of the set bits of words[0..nw) in ascending order.
// Set bits over nw words, the whole work-group (one barrier; wsum:
// kSelWaves words, not reused afterwards).
template <int THREADS>
__device__ uint32_t block_popc_total(const uint32_t *words, int nw, uint32_t *wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t local = 0u;
    for (int w = tid; w < nw; w += THREADS)
        local += __popc(words[w]);
    const uint32_t t = wave_reduce(local, [](uint32_t x, uint32_t y) { return x + y; });
    if (lane == 0)
        wsum[wave] = t;
    __syncthreads();
    uint32_t total = 0u;
#pragma unroll
    for (int v = 0; v < (THREADS / 64); ++v)
        total += wsum[v];
    return total;
}

template <int THREADS>
__device__ void compact_bits(const uint32_t *words, const uint32_t *offs, int nw, int32_t *dst)
{
    for (int w = threadIdx.x; w < nw; w += THREADS) {
        uint32_t bits = words[w];
        int pos = (int)offs[w];
        while (bits) {
            const int bi = __ffs(bits) - 1;
            dst[pos++] = w * 32 + bi;
            bits &= bits - 1u;
        }
    }
}

// Wave-wide digit choice: lane l holds the counts c of digits 4l .. 4l+3 of
// the keys that match the prefix.  Finds the digit holding the krem-th
// largest of them; afterwards, in every lane, prefix includes that digit
// (at shift), krem is the rank left inside it and cnt is its count.
__device__ __forceinline__ void pick_digit(uint4 c, int lane, int shift, uint32_t &prefix,
                                           uint32_t &krem, uint32_t &cnt)
{
    const uint32_t sl = c.x + c.y + c.z + c.w;
    const uint32_t inc = wave_incl_scan(sl, lane);
    const uint32_t all = __builtin_amdgcn_readlane(inc, 63);
    const uint32_t suf = all - inc + sl; // keys in digits >= 4 * lane
    const unsigned long long m = __ballot(suf >= krem);
    const int L = 63 - __clzll(m);
    uint32_t above = suf - sl, dg, cd;
    if (above + c.w >= krem) {
        dg = 4u * lane + 3u;
        cd = c.w;
    } else if (above + c.w + c.z >= krem) {
        above += c.w;
        dg = 4u * lane + 2u;
        cd = c.z;
    } else if (above + c.w + c.z + c.y >= krem) {
        above += c.w + c.z;
        dg = 4u * lane + 1u;
        cd = c.y;
    } else {
        above += c.w + c.z + c.y;
        dg = 4u * lane;
        cd = c.x;
    }
    prefix |= __builtin_amdgcn_readlane(dg, L) << shift;
    krem -= __builtin_amdgcn_readlane(above, L);
    cnt = __builtin_amdgcn_readlane(cd, L);
}

struct BinHit {
    uint32_t bin;   // the bin holding the wanted rank
    uint32_t above; // keys in the bins above it
    uint32_t count; // keys in it
};

// One wave over a 4096-bin LDS histogram, read from the top: lane l sums
// bins 64l .. 64l+63.  find(r) returns the bin holding the key of rank r
// (0 = largest), r < total; every lane gets the same answer.
struct BinScan {
    uint32_t ls, above_l, total;
    const uint32_t *h;
    int lane;
    __device__ BinScan(const uint32_t *hist, int lane_) : h(hist), lane(lane_)
    {
        // (each lane starts its 16 reads at its own rotation, so that the
        // lanes of one read, 256 bytes apart, fall into different banks)
        uint32_t s = 0u;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const uint4 v = reinterpret_cast<const uint4 *>(hist)[lane * 16 + ((c + lane) & 15)];
            s += v.x + v.y + v.z + v.w;
        }
        ls = s;
        const uint32_t inc = wave_incl_scan(s, lane);
        total = __builtin_amdgcn_readlane(inc, 63);
        above_l = total - inc; // keys in bins above this lane's
    }
    __device__ BinHit find(uint32_t r) const
    {
        const unsigned long long m1 = __ballot(above_l <= r && r < above_l + ls);
        const int L = __ffsll(m1) - 1;
        const uint32_t aL = __builtin_amdgcn_readlane(above_l, L);
        const uint32_t c = h[64 * L + lane];
        const uint32_t inc = wave_incl_scan(c, lane);
        const uint32_t up = aL + __builtin_amdgcn_readlane(inc, 63) - inc; // bins above 64L+lane
        const unsigned long long m2 = __ballot(up <= r && r < up + c);
        const int x = __ffsll(m2) - 1;
        return BinHit{64u * L + (uint32_t)x, (uint32_t)__builtin_amdgcn_readlane(up, x),
                      (uint32_t)__builtin_amdgcn_readlane(c, x)};
    }
};

// Packed unsigned 16-bit saturating subtract and minimum (two keys per op).
__device__ __forceinline__ uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b)
{
    uint32_t d;
    asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b)
{
    uint32_t d;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// Loads the 32 keys of bitmap word w.  Only positions in [lo, hi) (the
// middle region between the sink and the local window, hi <= n) compete for
// the budget; every other position gets key 0.  Whole words of 16-byte
// aligned rows use four-float loads; a partial last word, or a row whose
// start is not 16-byte aligned, is read one float at a time without touching
// positions >= n.
__device__ __forceinline__ void load_word_keys(const float *row, int w, int lo, int hi, int n,
                                               bool vec, uint32_t (&k)[32])
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
        if (p0 < lo || p0 + 32 > hi) {
#pragma unroll
            for (int e = 0; e < 32; ++e)
                k[e] = p0 + e >= lo && p0 + e < hi ? k[e] : 0u;
        }
    } else {
        float f[32];
#pragma unroll
        for (int e = 0; e < 32; ++e)
            f[e] = row[p0 + e < n ? p0 + e : 0];
#pragma unroll
        for (int e = 0; e < 32; ++e)
            k[e] = p0 + e >= lo && p0 + e < hi ? score_key(f[e]) : 0u;
    }
}

// Bits of word w for the positions p < x.
__device__ __forceinline__ uint32_t mask_below(int w, int x)
{
    const int c = x - 32 * w;
    return c <= 0 ? 0u : (c >= 32 ? 0xFFFFFFFFu : (1u << c) - 1u);
}

template <int WPT, bool K16, int THREADS>
__global__ __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(4))) void select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx_len, int Himp, int cap,
    int nwc, int B, int r, int32_t *__restrict__ sel_idx, int sel_stride,
    int32_t *__restrict__ sel_count, int32_t *__restrict__ topb_idx,
    uint32_t *__restrict__ sel_bits, int bits_stride, int32_t *__restrict__ keep_from, int n_new,
    int n_sink, int n_local, const uint16_t *__restrict__ keys16,
    const uint16_t *__restrict__ keys16lo, const uint16_t *__restrict__ sample16, int s16)
{
    static_assert(!K16 || WPT <= 1, "16-bit first pass: one word per thread, or words re-read");
    static_assert(THREADS == 1024 || (THREADS == 512 && K16), "1024 threads, or 512 on rows of <= 512 words");
    constexpr int NWAVES = THREADS / 64;
    extern __shared__ __align__(16) uint32_t lds[];
    uint32_t *hist = lds;                         // [kCopies][kCopyStride]
    uint32_t *tot = hist + kCopies * kCopyStride; // [256]
    uint32_t *misc = tot + 256;                   // 64 words
    uint32_t *Tb = misc + 64;                     // [nwc] kept set
    uint32_t *Sb = Tb + nwc;                      // [nwc] widened set / tie bits
    uint32_t *Xb = Sb + nwc;                      // [nwc] dilation ping-pong
    uint32_t *scan = Xb + nwc;                    // [nwc] scan output
    // candidates (key, position), kWaveCap per wave; shares Xb / scan,
    // which are used only after the candidates are consumed
    uint2 *cpair = reinterpret_cast<uint2 *>(Xb);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y, i = blockIdx.x;
    const size_t rowid = (size_t)b * Himp + i;
    // fp32 scores (without 16-bit keys), or the keys' two 16-bit halves
    const float *row = K16 ? nullptr : scores + rowid * cap;
    // With 16-bit keys, this thread's four sample keys (positions 8m,
    // m = 4 tid .. 4 tid + 3) and its word's 32 keys are requested before
    // the context length is known, the sample first so that its histogram
    // can be built while the keys arrive (masked by position afterwards).
    // The keys come in whole words of 64 bytes (rows of keys16_stride(cap)
    // entries, pair order), so every load is a 16-byte one.  The loads are
    // unconditional, at clamped addresses (so that the compiler can wait for
    // the sample alone): a thread past the row reads the row's last word
    // again.
    uint2 s16v = make_uint2(0u, 0u);
    uint4 k16v[4] = {};
    // 16-bit keys of whole word w (64 bytes, pair order), and its sample pair
    const int wlast = (cap + 31) / 32 - 1; // the row's last word
    auto k16_word = [&](int w, uint4 (&kv)[4]) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            keys16 + rowid * (size_t)(32 * (wlast + 1)) + 32 * (w < wlast ? w : wlast));
#pragma unroll
        for (int q = 0; q < 4; ++q)
            kv[q] = src[q];
    };
    // the full keys of word w from their two halves (pair j of a word holds
    // positions j and 16 + j); positions outside [lo, hi) get key 0
    auto k32_word = [&](int w, int lo_, int hi_, uint32_t (&k)[32]) {
        const size_t base = rowid * (size_t)(32 * (wlast + 1)) + 32 * (w < wlast ? w : wlast);
        const uint4 *ph = reinterpret_cast<const uint4 *>(keys16 + base);
        const uint4 *pl = reinterpret_cast<const uint4 *>(keys16lo + base);
        uint4 hv[4], lv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hv[q] = ph[q];
            lv[q] = pl[q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t hp[4] = {hv[q].x, hv[q].y, hv[q].z, hv[q].w};
            const uint32_t lp[4] = {lv[q].x, lv[q].y, lv[q].z, lv[q].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = 4 * q + c;
                k[j] = (hp[c] << 16) | (lp[c] & 0xFFFFu);
                k[16 + j] = (hp[c] & 0xFFFF0000u) | (lp[c] >> 16);
            }
        }
#pragma unroll
        for (int e = 0; e < 32; ++e)
            k[e] = 32 * w + e >= lo_ && 32 * w + e < hi_ ? k[e] : 0u;
    };
    auto s16_word = [&](int w) {
        const int ms = 4 * w < s16 ? 4 * w : s16 - 4;
        return *reinterpret_cast<const uint2 *>(sample16 + rowid * s16 + ms);
    };
    if constexpr (K16 && WPT == 1) {
        s16v = s16_word(tid);
        k16_word(tid, k16v);
        // Nothing is scheduled across this point: the requests stay ahead of
        // the early exit instead of being moved below it, after the context
        // length arrives.
        __builtin_amdgcn_sched_barrier(0);
    }
    // LDS that starts at zero (radix and sample histograms, misc words),
    // cleared before anything depends on the context length
    for (int e = tid; e < kCopies * kCopyStride; e += THREADS)
        hist[e] = 0u;
    for (int e = tid; e < kSampleBins; e += THREADS)
        reinterpret_cast<uint32_t *>(cpair)[e] = 0u;
    if (tid < 64)
        misc[tid] = 0u;
    const int n = clamp_len(ctx_len[b], cap);
    if (n == 0) {
        if (keep_from != nullptr && i == 0 && tid == 0)
            keep_from[b] = 0;
        if (tid == 0)
            sel_count[rowid] = 0;
        if (sel_bits != nullptr)
            for (int w = tid; w < bits_stride; w += THREADS)
                sel_bits[rowid * bits_stride + w] = 0u;
        return;
    }
    const int nw = (n + 31) >> 5;
    const int nwt = (nw + THREADS - 1) / THREADS; // words per thread
    const bool vec = (cap & 3) == 0; // every row starts 16-byte aligned
    // the sink [0, lo) and the local window [hi, n) are kept outright; the
    // budget goes to the middle region [lo, hi)
    const int lo = n_sink < n ? n_sink : n;
    const int hi = n_local < n - lo ? n - n_local : lo;

    // full keys live in registers with one word per thread (not needed when
    // the first pass reads the 16-bit keys)
    constexpr bool REG = WPT > 0 && !K16;
    uint32_t keys[32];
    if constexpr (REG)
        load_word_keys(row, tid, lo, hi, n, vec, keys);
    // With split keys and one word per thread, the word's full keys are
    // assembled once before the radix passes, which then read them from
    // registers, and once more for the kept words (SPLIT1: for_words reads
    // them there).
    constexpr bool SPLIT1 = K16 && WPT > 0;
    // Rows of at most THREADS / 32 words (SPLIT1): the passes over every
    // key give each thread one key (position tid) instead of leaving a
    // word's 32 keys to each of nw threads, whose serial LDS atomics would
    // set the pace; the keys are staged through the candidate area, which
    // these passes do not use otherwise.
    const bool small = SPLIT1 && nw * 32 <= THREADS;
    uint32_t mykey = 0u;
    auto stage_keys = [&]() {
        uint32_t *kst = reinterpret_cast<uint32_t *>(cpair);
        k32_word(tid, lo, hi, keys);
        if (tid < nw) {
#pragma unroll
            for (int e = 0; e < 32; ++e)
                kst[32 * tid + e] = keys[e];
        }
        __syncthreads();
        mykey = tid < 32 * nw ? kst[tid] : 0u;
    };
    // fn(w, k) over this thread's words, k[e] the key of position 32w + e
    auto for_words = [&](auto &&fn) {
        if constexpr (SPLIT1) {
            fn(tid, keys);
        } else if constexpr (K16) {
            for (int j = 0; j < nwt; ++j) {
                uint32_t k[32];
                k32_word(tid + j * THREADS, lo, hi, k);
                fn(tid + j * THREADS, k);
            }
        } else if constexpr (REG) {
            fn(tid, keys);
        } else if constexpr (WPT > 0) {
            uint32_t k[32];
            load_word_keys(row, tid, lo, hi, n, vec, k);
            fn(tid, k);
        } else {
            for (int j = 0; j < nwt; ++j) {
                uint32_t k[32];
                load_word_keys(row, tid + j * THREADS, lo, hi, n, vec, k);
                fn(tid + j * THREADS, k);
            }
        }
    };

    // One radix pass.  count() adds the digit (bits shift..shift+7) of every
    // key it visits that matches the prefix to the histogram (copy h16 when
    // many, else copy 0).  Then misc[0] = the prefix extended by the digit
    // that holds the krem-th largest of those keys, misc[1] = the rank left
    // inside that digit and misc[2] = the digit's count.  The histogram is
    // left zeroed.
    uint32_t *h16 = hist + (lane & (kCopies - 1)) * kCopyStride;
    auto radix_pass = [&](int shift, uint32_t prefix, uint32_t krem, bool many, auto &&count) {
        count();
        __syncthreads();
        const uint32_t *src = hist;
        if (many) {
            if (tid < 256) {
                uint32_t cnt = 0u;
#pragma unroll
                for (int cp = 0; cp < kCopies; ++cp) {
                    cnt += hist[cp * kCopyStride + tid];
                    hist[cp * kCopyStride + tid] = 0u;
                }
                tot[tid] = cnt;
            }
            __syncthreads();
            src = tot;
        }
        if (wave == 0) {
            const uint4 c = reinterpret_cast<const uint4 *>(src)[lane];
            if (!many)
                reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
            uint32_t pf = prefix, kr = krem, cd = 0u;
            pick_digit(c, lane, shift, pf, kr, cd);
            if (lane == 0) {
                misc[0] = pf;
                misc[1] = kr;
                misc[2] = cd;
            }
        }
        __syncthreads();
    };

    const bool take_all = B >= hi - lo;
    uint32_t tau = 0u, fmask = 0xFFFFFFFFu, need = 0u, cnt_eq = 0u;
    bool emitted = false; // Tb / Sb already hold the kept and tie bits
    if (!take_all) {
        // The sample histogram lives in the candidate area, which is not
        // written before the histogram has been read.
        uint32_t *shist = reinterpret_cast<uint32_t *>(cpair);
        const bool sampled = nw >= kMinSampleWords;
        // (the 16-bit keys may still be arriving: only LDS is synchronised
        // until the classification pass)
        lds_barrier();
        bool found = false;
        if (sampled) {
            // ---- bracket tau from the keys at positions 8m ----
            // (keys 0, 8, 16, 24 of every word), binned by their top 12 bits
            auto sample_word = [&](int j, uint32_t (&s4)[4]) {
                if constexpr (K16) {
                    // the 16-bit keys of positions 8(4 w + q) of this
                    // thread's word w, as the top half of a key (enough for
                    // the 12-bit sample bins)
                    const int w = tid + j * THREADS;
                    const uint2 sv = WPT == 1 ? s16v : s16_word(w);
                    const uint32_t pair[2] = {sv.x, sv.y};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int p = 8 * (4 * w + q);
                        const uint32_t k16 = (pair[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
                        s4[q] = p < n && p >= lo && p < hi ? k16 << 16 : 0u;
                    }
                } else if constexpr (REG) {
                    (void)j;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        s4[q] = keys[8 * q];
                } else {
                    const int p0 = (tid + j * THREADS) * 32;
                    float f[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int p = p0 + 8 * q;
                        f[q] = row[p < n ? p : 0];
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int p = p0 + 8 * q;
                        s4[q] = p >= lo && p < hi ? score_key(f[q]) : 0u;
                    }
                }
            };
            const int nsw = WPT > 0 ? 1 : nwt; // words sampled per thread
            for (int j = 0; j < nsw; ++j) {
                uint32_t s4[4];
                sample_word(j, s4);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (s4[q] != 0u)
                        atomicAdd(&shist[s4[q] >> kBinShift], 1u);
            }
            lds_barrier();
            if (wave == 0) {
                // sample ranks a margin either side of the expected rank of tau
                const BinScan sc(shist, lane);
                const float pb = (float)B / (float)(hi - lo);
                const float tr = pb * (float)sc.total;
                const float mg = 4.5f * sqrtf((float)sc.total * pb * (1.f - pb)) + 3.f;
                const int hi_rank = (int)floorf(tr - mg);
                const int lo_rank = (int)ceilf(tr + mg);
                uint32_t b_hi = kSampleBins - 1, b_lo = 0u;
                if (hi_rank >= 0)
                    b_hi = sc.find((uint32_t)hi_rank).bin;
                if (lo_rank >= 1 && lo_rank <= (int)sc.total)
                    b_lo = sc.find((uint32_t)lo_rank - 1u).bin;
                if (lane == 0) {
                    misc[4] = b_lo;
                    misc[5] = b_hi;
                }
            }
            lds_barrier();
            // candidate range [plo, phim1]: bins b_lo .. b_hi; keys above are
            // kept.  Candidates are also counted by their top 20 bits (bin and
            // the next 8 bits) when their bins are few enough for that.
            const uint32_t b_lo = misc[4], b_hi = misc[5];
            const uint32_t plo = b_lo ? b_lo << kBinShift : 1u;
            const uint32_t phim1 = (uint32_t)(((uint64_t)b_hi + 1u) << kBinShift) - 1u;
            const uint32_t span = phim1 - plo;
            const bool lvl = b_hi - b_lo < (uint32_t)(kSampleBins >> 8);
            const uint32_t d0 = b_lo << 8; // first 20-bit prefix of the range
            // ---- one pass: kept words of the keys above the range and
            // candidate words; then the candidates (key, position), per wave ----
            uint2 *cwave = cpair + wave * kWaveCap;
            uint32_t run = 0u, na = 0u;
            auto pass_word = [&](int w, uint32_t wt, uint32_t wc) {
                if (w < nw) {
                    Tb[w] = wt;
                    Sb[w] = 0u;
                }
                na += __popc(wt);
                // this lane's slots, after those of the lower lanes
                const uint32_t c = __popc(wc);
                const uint32_t inc = wave_incl_scan(c, lane);
                uint32_t slot = run + inc - c;
                run += __builtin_amdgcn_readlane(inc, 63);
                // this lane's candidate positions, in slot order (their keys
                // are read below, the wave's lanes sharing the reads evenly)
                // (past the wave's capacity the last slot is overwritten:
                // the selection then takes the full radix path, which does
                // not read the candidates)
                while (wc) {
                    cwave[slot < (uint32_t)kWaveCap ? slot : (uint32_t)kWaveCap - 1u].y =
                        (uint32_t)(w * 32 + __ffs(wc) - 1);
                    ++slot;
                    wc &= wc - 1u;
                }
            };
            if constexpr (K16) {
                // a word from its 16 key pairs (pair j: the 16-bit keys of
                // positions 32 w + j and 32 w + 16 + j), two keys per packed
                // op: a key's 12-bit bin is key16 >> 4, so bin > b_hi is
                // key16 >= kt and bin < b_lo is key16 < kl.  sat(kt - key16)
                // is nonzero iff the key is not above the range,
                // sat(kl - key16) iff it is below; min(., 1) turns each into
                // the word's bit j (low half) or 16 + j (high half).
                const uint32_t kt = b_hi + 1u < 4096u ? (b_hi + 1u) << 4 : 0xFFFFu;
                const uint32_t ktv = kt * 0x10001u, klv = (b_lo << 4) * 0x10001u;
                auto classify = [&](int w, const uint4 (&kv)[4]) {
                    const uint32_t kw[16] = {kv[0].x, kv[0].y, kv[0].z, kv[0].w,
                                             kv[1].x, kv[1].y, kv[1].z, kv[1].w,
                                             kv[2].x, kv[2].y, kv[2].z, kv[2].w,
                                             kv[3].x, kv[3].y, kv[3].z, kv[3].w};
                    uint32_t not_above = 0u, below = 0u;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        not_above |= pk_min_u16(pk_sub_sat_u16(ktv, kw[j]), 0x10001u) << j;
                        below |= pk_min_u16(pk_sub_sat_u16(klv, kw[j]), 0x10001u) << j;
                    }
                    // valid: positions of the middle region [lo, hi)
                    const uint32_t vm = mask_below(w, hi) & ~mask_below(w, lo);
                    // (with b_hi the top bin no key is above the range)
                    const uint32_t wt = b_hi + 1u < 4096u ? ~not_above & vm : 0u;
                    const uint32_t wc = not_above & ~below & vm;
                    pass_word(w, wt, wc);
                };
                if constexpr (WPT == 1) {
                    classify(tid, k16v);
                } else {
                    // longer rows: the words' keys are read here, two words
                    // in flight at a time
                    for (int j = 0; j < nwt; j += 2) {
                        uint4 ka[4], kb[4];
                        k16_word(tid + j * THREADS, ka);
                        k16_word(tid + (j + 1) * THREADS, kb);
                        classify(tid + j * THREADS, ka);
                        if (j + 1 < nwt)
                            classify(tid + (j + 1) * THREADS, kb);
                    }
                }
            } else {
                for_words([&](int w, const auto &k) {
                    uint32_t wt = 0u, wc = 0u;
#pragma unroll
                    for (int e = 0; e < 32; ++e) {
                        wt |= (uint32_t)(k[e] > phim1) << e;
                        wc |= (uint32_t)(k[e] - plo <= span) << e;
                    }
                    pass_word(w, wt, wc);
                });
            }
            {
                // the wave's candidate keys, re-read (from cache) with every
                // lane taking an equal share and all requests in flight
                // together; the positions were written by this wave only
                __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0)
                __builtin_amdgcn_wave_barrier();
                const uint32_t nc = run < (uint32_t)kWaveCap ? run : (uint32_t)kWaveCap;
                const size_t kbase = rowid * (size_t)(32 * (wlast + 1));
                for (uint32_t e0 = 0; e0 < nc; e0 += 4 * 64) {
                    uint32_t pos[4];
                    uint32_t f[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        // (every lane reads a slot, masked after: no branch
                        // between the reads)
                        const uint32_t e = e0 + 64 * t + lane;
                        const uint32_t pv = cwave[e < nc ? e : 0u].y;
                        pos[t] = pv & (0u - (uint32_t)(e < nc));
                    }
                    uint32_t flo[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if constexpr (K16) {
                            // the key's two halves
                            const size_t en = kbase + keys16_entry((int)pos[t]);
                            f[t] = keys16[en];
                            flo[t] = keys16lo[en];
                        } else {
                            f[t] = __float_as_uint(row[pos[t]]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        // the key is stored by every lane (past the list
                        // into a word of its own in the prefix-list area,
                        // written only later), so no branch holds the loads
                        const uint32_t e = e0 + 64 * t + lane;
                        const uint32_t kc =
                            K16 ? (f[t] << 16) | flo[t] : score_key(__uint_as_float(f[t]));
                        *(e < nc ? &cwave[e < nc ? e : 0u].x : &tot[64 + lane]) = kc;
                        if (lvl && e < nc)
                            atomicAdd(&hist[(kc >> 12) - d0], 1u);
                    }
                }
            }
            na = wave_reduce(na, [](uint32_t x, uint32_t y) { return x + y; });
            if (lane == 0) {
                tot[wave] = run;
                tot[NWAVES + wave] = na;
            }
            __syncthreads();
            uint32_t A = 0u, C = 0u;
            bool over = false;
#pragma unroll
            for (int v = 0; v < NWAVES; ++v) {
                C += tot[v];
                A += tot[NWAVES + v];
                over |= tot[v] > (uint32_t)kWaveCap;
            }
            found = lvl && !over && A < (uint32_t)B && (uint32_t)B <= A + C;
            if (found) {
                // ---- tau among the candidates: top 20 bits, then the rest ----
                if (wave == 0) {
                    const BinScan sc(hist, lane);
                    const BinHit h = sc.find((uint32_t)B - A - 1u);
                    if (lane == 0) {
                        misc[0] = d0 + h.bin;          // 20-bit prefix of tau
                        misc[1] = (uint32_t)B - A - h.above; // rank inside it
                        misc[2] = h.count;             // candidates with that prefix
                    }
                }
                __syncthreads();
                const uint32_t p20 = misc[0], krem = misc[1], m20 = misc[2];
                if (m20 <= 64u) {
                    // Few keys share the prefix (the usual case): candidates
                    // above it are kept now, each wave taking its own, and
                    // those with it gather in a list that one wave ranks.
                    uint2 *tl = reinterpret_cast<uint2 *>(tot + 64);
                    const uint32_t tw = tot[wave];
                    for (uint32_t e = lane; e < tw; e += 64) {
                        const uint2 c = cwave[e];
                        const uint32_t pf = c.x >> 12;
                        if (pf > p20)
                            atomicOr(&Tb[c.y >> 5], 1u << (c.y & 31u));
                        else if (pf == p20)
                            tl[atomicAdd(&misc[kMiscList], 1u)] = c;
                    }
                    __syncthreads();
                    if (wave == 0) {
                        // tau is the key with (keys above) < krem <= (keys
                        // above or equal) among the m20 listed keys
                        const uint2 c = tl[lane < (int)m20 ? lane : 0];
                        uint32_t above = 0u, eq = 0u;
                        for (uint32_t j = 0; j < m20; ++j) {
                            const uint32_t kj = __builtin_amdgcn_readlane(c.x, j);
                            above += kj > c.x ? 1u : 0u;
                            eq += kj == c.x ? 1u : 0u;
                        }
                        const bool hit = lane < (int)m20 && above < krem && krem <= above + eq;
                        const int x = __ffsll(__ballot(hit)) - 1;
                        const uint32_t t = __builtin_amdgcn_readlane(c.x, x);
                        const uint32_t nd = krem - __builtin_amdgcn_readlane(above, x);
                        const uint32_t ce = __builtin_amdgcn_readlane(eq, x);
                        // the listed keys at or above tau join the kept
                        // words; those equal to it are ties when ties split
                        if (lane < (int)m20) {
                            const uint32_t bit = 1u << (c.y & 31u);
                            if (c.x > t || (c.x == t && nd >= ce))
                                atomicOr(&Tb[c.y >> 5], bit);
                            else if (c.x == t)
                                atomicOr(&Sb[c.y >> 5], bit);
                        }
                        if (lane == 0) {
                            misc[3] = t;  // tau
                            misc[6] = nd; // ties at tau kept
                            misc[7] = ce; // keys equal to tau
                        }
                    }
                    __syncthreads();
                    tau = misc[3];
                    need = misc[6];
                    cnt_eq = misc[7];
                } else {
                    // many keys share the prefix: a histogram of their low
                    // 12 bits finds tau, then every candidate is placed
                    for (int e = tid; e < kSampleBins; e += THREADS)
                        hist[e] = 0u;
                    __syncthreads();
                    for (int i = tid; i < NWAVES * kWaveCap; i += THREADS) {
                        if ((uint32_t)(i % kWaveCap) < tot[i / kWaveCap]) {
                            const uint32_t kc = cpair[i].x;
                            if ((kc >> 12) == p20)
                                atomicAdd(&hist[kc & 4095u], 1u);
                        }
                    }
                    __syncthreads();
                    if (wave == 0) {
                        const BinScan sc(hist, lane);
                        const BinHit h = sc.find(krem - 1u);
                        if (lane == 0) {
                            misc[3] = (p20 << 12) | h.bin; // tau
                            misc[6] = krem - h.above;      // ties at tau kept
                            misc[7] = h.count;             // keys equal to tau
                        }
                    }
                    __syncthreads();
                    tau = misc[3];
                    need = misc[6];
                    cnt_eq = misc[7];
                    // candidates at or above tau join the kept words; those
                    // equal to tau are ties when ties are split
                    const bool split = need < cnt_eq;
                    for (int i = tid; i < NWAVES * kWaveCap; i += THREADS) {
                        if ((uint32_t)(i % kWaveCap) < tot[i / kWaveCap]) {
                            const uint2 c = cpair[i];
                            const uint32_t bit = 1u << (c.y & 31u);
                            if (c.x > tau || (c.x == tau && !split))
                                atomicOr(&Tb[c.y >> 5], bit);
                            else if (c.x == tau)
                                atomicOr(&Sb[c.y >> 5], bit);
                        }
                    }
                    __syncthreads();
                }
                emitted = true;
            } else {
                for (int e = tid; e < kCopies * kCopyStride; e += THREADS)
                    hist[e] = 0u;
                __syncthreads();
            }
        }
        if (!found) {
            // ---- radix select over every key ----
            if constexpr (SPLIT1) {
                if (small)
                    stage_keys();
                else
                    k32_word(tid, lo, hi, keys);
            }
            uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)B;
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                radix_pass(shift, prefix, krem, true, [&]() {
                    if (small) {
                        if (mykey != 0u && (mykey & pmask) == prefix)
                            atomicAdd(&h16[(mykey >> shift) & 255u], 1u);
                        return;
                    }
                    for_words([&](int w, const auto &k) {
                        (void)w;
#pragma unroll
                        for (int e = 0; e < 32; ++e)
                            if (k[e] != 0u && (k[e] & pmask) == prefix)
                                atomicAdd(&h16[(k[e] >> shift) & 255u], 1u);
                    });
                });
                prefix = misc[0];
                krem = misc[1];
                cnt_eq = misc[2];
                pmask |= 255u << shift;
                if (krem == cnt_eq)
                    break; // every key with this prefix is kept
            }
            tau = prefix;
            fmask = pmask;
            need = krem;
        }
    }
    // (stored late: an early store would make the first loads' waits
    // conservative)
    if (keep_from != nullptr && i == 0 && tid == 0)
        keep_from[b] = n - n_new > 0 ? n - n_new : 0;
    // Kept: every valid key with (key & fmask) >= thr (every valid key when
    // thr is 0, none when none_kept).  With split ties the keys with
    // (key & fmask) == tau are ties, need of them kept, lowest positions first.
    const bool partial_ties = !take_all && need < cnt_eq;
    uint32_t thr = 0u;
    bool none_kept = false;
    if (!take_all) {
        if (!partial_ties)
            thr = tau;
        else if (tau == 0xFFFFFFFFu)
            none_kept = true;
        else
            thr = tau + 1u;
    }

    // ---- kept-set bitmap (and tie bitmap when ties are split) ----
    if (!emitted && small) {
        // one key per thread: a word's bits are a ballot of its 32 lanes
        if (take_all)
            stage_keys();
        const bool kept = !none_kept && (thr == 0u ? mykey != 0u : (mykey & fmask) >= thr);
        const bool tie = partial_ties && mykey != 0u && (mykey & fmask) == tau;
        const uint64_t bk = __ballot(kept), bq = __ballot(tie);
        if (lane == 0) {
            const int w0 = 2 * wave;
            if (w0 < nw) {
                Tb[w0] = (uint32_t)bk;
                Sb[w0] = (uint32_t)bq;
            }
            if (w0 + 1 < nw) {
                Tb[w0 + 1] = (uint32_t)(bk >> 32);
                Sb[w0 + 1] = (uint32_t)(bq >> 32);
            }
        }
        __syncthreads();
    } else if (!emitted) {
        if constexpr (SPLIT1)
            k32_word(tid, lo, hi, keys);
        for_words([&](int w, const auto &k) {
            if (w >= nw)
                return;
            uint32_t wt = 0u, wq = 0u;
            if (none_kept) {
            } else if (thr == 0u) {
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    wt |= (uint32_t)(k[e] != 0u) << e;
            } else {
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    wt |= (uint32_t)((k[e] & fmask) >= thr) << e;
            }
            if (partial_ties) {
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    wq |= (uint32_t)(k[e] != 0u && (k[e] & fmask) == tau) << e;
            }
            Tb[w] = wt;
            Sb[w] = wq;
        });
        __syncthreads();
    }
    if (partial_ties) {
        block_popc_exscan<THREADS>(Sb, scan, nw, misc + kMiscScan);
        for (int w = tid; w < nw; w += THREADS) {
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
        block_popc_exscan<THREADS>(Tb, scan, nw, misc + kMiscScan);
        compact_bits<THREADS>(Tb, scan, nw, topb_idx + rowid * (size_t)B);
        __syncthreads();
    }

    // ---- neighbor fetching: dilate T by r within [0, n) ----
    uint32_t *fin = Tb;
    if (r > 0) {
        const uint32_t *src = Tb;
        uint32_t *dst = Sb;
        int left = r;
        while (left > 0) {
            const int step = left < 31 ? left : 31;
            for (int w = tid; w < nw; w += THREADS) {
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

    // ---- the sink and the local window join the set ----
    if (lo > 0 || hi < n) {
        for (int w = tid; w < nw; w += THREADS)
            fin[w] |= mask_below(w, lo) | (mask_below(w, n) & ~mask_below(w, hi));
        __syncthreads();
    }

    // ---- |S|, the ascending list (when asked) and the bitmap (when asked) ----
    const uint32_t total = sel_idx != nullptr
                               ? block_popc_exscan<THREADS>(fin, scan, nw, misc + kMiscScan)
                               : block_popc_total<THREADS>(fin, nw, misc + kMiscScan);
    if (sel_idx != nullptr)
        compact_bits<THREADS>(fin, scan, nw, sel_idx + rowid * sel_stride);
    if (sel_bits != nullptr)
        for (int w = tid; w < bits_stride; w += THREADS)
            sel_bits[rowid * bits_stride + w] = w < nw ? fin[w] : 0u;
    if (tid == 0)
        sel_count[rowid] = (int32_t)total;
}

// words per bitmap array, even so that the candidate pairs stay 8-byte aligned
inline int sel_words(int cap) { return ((cap + 31) / 32 + 2) & ~1; }
// dynamic LDS of one selection work-group
inline size_t sel_lds_bytes(int cap, int waves)
{
    const size_t nwc = (size_t)sel_words(cap);
    const size_t u = 2 * nwc > 2 * (size_t)waves * kWaveCap ? 2 * nwc
                                                             : 2 * (size_t)waves * kWaveCap;
    return ((size_t)kCopies * kCopyStride + 256 + 64 + 2 * nwc + u) * sizeof(uint32_t);
}

// Rows of up to 512 words (16K positions, a sample of at most 2048 keys)
// take the 16-bit-key selection in 512-thread work-groups, two of which fit
// a compute unit; longer rows take 1024 threads, one word per thread.
constexpr int kSelShortCap = 16384;

template <int WPT, bool K16, int THREADS>
hipError_t select_t(const tb_shape &s, const tb_select_params &p, const float *scores,
                    const int32_t *ctx_len, int32_t *sel_idx, int sel_stride,
                    int32_t *sel_count, int32_t *topb_idx, uint32_t *sel_bits,
                    int32_t *keep_from, int n_new, const uint16_t *keys16,
                    const uint16_t *keys16lo, const uint16_t *sample16, hipStream_t st)
{
    const int nwc = sel_words(s.ctx_cap);
    const size_t lds = sel_lds_bytes(s.ctx_cap, THREADS / 64);
    if (lds > 64 * 1024) {
        // the launch limit is raised once per device, to what the largest
        // capacity needs
        static std::atomic<uint64_t> raised{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        const uint64_t bit = dev < 64 ? 1ull << dev : 0ull;
        if (bit == 0ull || (raised.load(std::memory_order_relaxed) & bit) == 0ull) {
            e = hipFuncSetAttribute((const void *)select_kernel<WPT, K16, THREADS>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)sel_lds_bytes(kMaxCtxCap, THREADS / 64));
            if (e != hipSuccess)
                return e;
            raised.fetch_or(bit, std::memory_order_relaxed);
        }
    }
    dim3 grid(s.n_imp_heads, s.batch);
    hipLaunchKernelGGL((select_kernel<WPT, K16, THREADS>), grid, dim3(THREADS), lds, st, scores,
                       ctx_len, s.n_imp_heads, s.ctx_cap, nwc, p.budget, p.radius, sel_idx,
                       sel_stride, sel_count, topb_idx, sel_bits, bitmap_words(s.ctx_cap),
                       keep_from, n_new, p.n_sink, p.n_local, keys16, keys16lo, sample16,
                       sample16_stride(s.ctx_cap));
    return hipGetLastError();
}

} // namespace

hipError_t launch_select(const tb_shape &s, const tb_select_params &p, const float *scores,
                         const int32_t *ctx_len, int32_t *sel_idx, int sel_stride,
                         int32_t *sel_count, int32_t *topb_idx, uint32_t *sel_bits,
                         int32_t *keep_from, int n_new, const uint16_t *keys16,
                         const uint16_t *keys16lo, const uint16_t *sample16, hipStream_t st)
{
#define TB_SEL_ARGS                                                                          \
    s, p, scores, ctx_len, sel_idx, sel_stride, sel_count, topb_idx, sel_bits, keep_from,       \
        n_new, keys16, keys16lo, sample16, st
    static_assert(kSelThreads == 1024, "select_key16: one word per thread up to 1024 words");
    static_assert(kSelShortCap / 32 <= 512 && kSelShortCap / 8 <= 4 * 512,
                  "short rows: one word and four sample keys per thread of 512");
    const bool k16 = keys16 != nullptr && keys16lo != nullptr && sample16 != nullptr;
    if (select_key16(s.ctx_cap)) {
        if (k16) {
            if (s.ctx_cap <= kSelShortCap)
                return select_t<1, true, 512>(TB_SEL_ARGS);
            return select_t<1, true, 1024>(TB_SEL_ARGS);
        }
        return select_t<1, false, 1024>(TB_SEL_ARGS);
    }
    return k16 ? select_t<0, true, 1024>(TB_SEL_ARGS) : select_t<0, false, 1024>(TB_SEL_ARGS);
#undef TB_SEL_ARGS
}

} // namespace tb
