// tb_internal.h -- shared device helpers and launcher declarations of
// libtokenbutler (gfx950 only).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tokenbutler.h"

namespace tb {

// ---------------------------------------------------------------- dtypes
// Storage element types: fp32 (`float`) and bf16 (raw bits in `uint16_t`).
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ double to_f64(float x) { return (double)x; }
__device__ __forceinline__ double to_f64(bf16_t x) { return (double)to_f32(x); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// fp64 -> bf16, correctly rounded (to nearest even).  x is first rounded to
// fp32 with round-to-odd (toward zero, last bit set when inexact), then to
// bf16 to nearest even: fp32 has 16 more significand bits than bf16 over the
// same exponent range (subnormals included), so the odd bit carries all a
// second rounding needs and the two steps round once (Boldo and Melquiond,
// "When double rounding is odd", 2005).  Needs fp32 subnormals preserved,
// the default mode of these kernels.
__device__ __forceinline__ bf16_t f64_to_bf16(double x)
{
    if (x != x)
        return (bf16_t)(((uint32_t)((uint64_t)__double_as_longlong(x) >> 48) & 0x8000u) | 0x7fc0u);
    const float f = (float)x; // to nearest even
    const double back = (double)f;
    uint32_t u = __float_as_uint(f);
    if (back != x) {
        if (fabs(back) > fabs(x))
            u -= 1u; // one step toward zero (infinity becomes the largest finite)
        u |= 1u;
    }
    return f32_to_bf16(__uint_as_float(u));
}

template <typename T> __device__ __forceinline__ T from_f64(double x);
template <> __device__ __forceinline__ float from_f64<float>(double x) { return (float)x; }
template <> __device__ __forceinline__ bf16_t from_f64<bf16_t>(double x) { return f64_to_bf16(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

__device__ __forceinline__ int clamp_len(int v, int cap) { return v < 0 ? 0 : (v > cap ? cap : v); }

// Order-preserving u32 key of an fp32 score: larger scores get larger keys,
// -0.0 and +0.0 share one key, and every finite score's key is >= 2^23 (so
// key 0 can mark "no score").
__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u)
        u = 0u; // -0.0 ties with +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Work-group barrier for LDS traffic only: each wave's LDS operations have
// completed when it arrives and the compiler moves no memory access across
// it, but global loads still in flight are not waited for.  (__syncthreads
// would wait for them: its fences must cover global stores, and on this
// architecture one counter tracks global loads and stores together.)  Only
// for phases that communicate through LDS alone.
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Partial results that cross work-groups (and XCDs, whose L2 caches are
// not coherent with each other): attention chunk partials, split-k MLP tiles.  They are written and read with agent-scope
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

// Bulk reads of such partials: 16-byte buffer loads carrying the same
// cache-policy bit (sc1) that an agent-scope atomic load is given, so they
// too are served from the device coherence point, at a quarter of the
// instructions of 32-bit atomics (a 64 KB read by one work-group: 0.9 us
// against 1.2 us with coalesced 64-bit atomic loads).  The resource covers
// [base, base + bytes); a load past it reads zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, uint32_t bytes)
{
    // stride 0, so the record count is in bytes; 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ float4 load4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    constexpr int kSc1 = 16; // cache policy: device-coherent access
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSc1));
}

// The same for the lanes of one wave: the wave's LDS operations have
// completed, so other lanes of the wave read what it wrote.
__device__ __forceinline__ void wave_lds_sync()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- wave ops
// Cross-lane steps through DPP row permutations (no LDS round trip); out of
// row sources read 0.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes: shifts within rows of 16, then the
// row totals are added across rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane)
{
    x += dpp<0x111>(x); // row_shr:1
    x += dpp<0x112>(x); // row_shr:2
    x += dpp<0x114>(x); // row_shr:4
    x += dpp<0x118>(x); // row_shr:8
    const uint32_t r0 = __builtin_amdgcn_readlane(x, 15);
    const uint32_t r1 = __builtin_amdgcn_readlane(x, 31);
    const uint32_t r2 = __builtin_amdgcn_readlane(x, 47);
    x += (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
    return x;
}

// Wave-wide reduction of a 32-bit value (op on its bits: min / max / sum of
// u32, or of floats through bit casts); every lane gets the result.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op)
{
    x = op(x, dpp<0xB1>(x));  // quad_perm [1,0,3,2]
    x = op(x, dpp<0x4E>(x));  // quad_perm [2,3,0,1]
    x = op(x, dpp<0x141>(x)); // row_half_mirror
    x = op(x, dpp<0x140>(x)); // row_mirror
    return op(op(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
              op(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

__device__ __forceinline__ float wave_max(float x)
{
    return __uint_as_float(wave_reduce(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}

__device__ __forceinline__ float wave_sum(float x)
{
    return __uint_as_float(wave_reduce(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}

// ---------------------------------------------------------------- sizes
constexpr int kAttnChunk = 1024;    // positions per sparse attention work-group
constexpr int kDenseChunk = 1024;   // positions per dense attention work-group
constexpr int kMaxCtxCap = 262144;  // bounded by the selection kernel's LDS bitmaps
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace layout (offsets in bytes from the workspace base).
struct WsLayout {
    size_t part_o;   // attention partial sums [b][Hq][nchunk][D] fp32
    size_t part_ml;  // attention partial (max, sum) [b][Hq][nchunk][2] fp32
    size_t counters; // attention arrival counters [b][Hkv] u32 (kept zero)
    size_t keys16;   // top 16 bits of each score's key [b][Himp][keys16_stride] u16,
                     // in pair order (fused step)
    size_t keys16lo; // the low 16 bits, the same layout
    size_t sample16; // the same for positions 8m, compact [b][Himp][sample16_stride] u16
    size_t zeroed;       // the words that must be zero when a call starts (the
    int zeroed_words;    //  arrival counters), kept zero by every completed call
    size_t total;
};

// Positions per sparse attention work-group: past 64K positions four times
// kAttnChunk (twice with eight query heads per KV head, whose single wave
// per head lists at most 64 words), so that the work-groups are about one
// per compute unit and the last one of a KV head merges fewer partials.
inline int attn_chunk_len(const tb_shape &s)
{
    if (s.ctx_cap <= 65536)
        return kAttnChunk;
    return s.n_q_heads / s.n_kv_heads <= 4 ? 4 * kAttnChunk : 2 * kAttnChunk;
}
inline int attn_chunks(const tb_shape &s)
{
    return (s.ctx_cap + attn_chunk_len(s) - 1) / attn_chunk_len(s);
}
inline int bitmap_words(int cap) { return (cap + 31) / 32; }

inline int dense_chunks(int cap) { return (cap + kDenseChunk - 1) / kDenseChunk; }
// u16 entries per row of the compact sample (positions 8m), a multiple of 8
inline int sample16_stride(int cap) { return ((cap + 7) / 8 + 7) & ~7; }
// u16 entries per row of the 16-bit keys: whole 32-position words.  Within
// word w the key of position 32w + j (j < 16) is entry 32w + 2j and that of
// position 32w + 16 + j is entry 32w + 2j + 1, so that the 32-bit pair j
// holds bits j and 16 + j of the word's membership masks.
inline int keys16_stride(int cap) { return (cap + 31) & ~31; }
// The selection's first pass reads the 16-bit keys when a row is at most one
// 32-position word per selection thread (1024 words).
inline bool select_key16(int cap) { return (cap + 31) / 32 <= 1024; }
__host__ __device__ inline int keys16_entry(int t)
{
    return (t & ~31) | ((t & 15) << 1) | ((t >> 4) & 1);
}
// Chunk partials are laid out per kernel's own chunk count; the region fits
// the larger of the two.
inline int max_chunks(const tb_shape &s)
{
    return attn_chunks(s) > dense_chunks(s.ctx_cap) ? attn_chunks(s) : dense_chunks(s.ctx_cap);
}

inline WsLayout ws_layout(const tb_shape &s)
{
    WsLayout L;
    size_t off = 0;
    L.part_o = off;
    off += align_up((size_t)s.batch * s.n_q_heads * max_chunks(s) * s.head_dim *
                    sizeof(float));
    L.part_ml = off;
    off += align_up((size_t)s.batch * s.n_q_heads * max_chunks(s) * 2 * sizeof(float));
    L.counters = off;
    L.zeroed = off;
    L.zeroed_words = s.batch * s.n_kv_heads;
    off += align_up((size_t)s.batch * s.n_kv_heads * sizeof(uint32_t));
    L.keys16 = off;
    off += align_up((size_t)s.batch * s.n_imp_heads * keys16_stride(s.ctx_cap) *
                    sizeof(uint16_t));
    L.keys16lo = off;
    off += align_up((size_t)s.batch * s.n_imp_heads * keys16_stride(s.ctx_cap) *
                    sizeof(uint16_t));
    L.sample16 = off;
    off += align_up((size_t)s.batch * s.n_imp_heads * sample16_stride(s.ctx_cap) *
                    sizeof(uint16_t));
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- launchers
// Compute units of the current device, queried once per device.
hipError_t device_cus(int &cus);

// Debug mode (TB_CHECK): check kernels that OR TB_CHECK_* bits into the
// device's check word; the caller enqueues them only when check_enabled().
bool check_enabled();
void set_check(bool on);
// every element of a dense array of n elements (dtype TB_F32 / TB_BF16)
hipError_t check_dense(const void *p, size_t n, int dtype, uint32_t bit, hipStream_t st);
// rows [0, len[b] - minus) of a cache [b][heads][cap][row] (len NULL: all)
hipError_t check_cache(const void *c, const int32_t *len, int minus, int batch, int heads,
                       int cap, int row, int dtype, uint32_t bit, hipStream_t st);
// ctx_len / keep_from ranges, and with sel_idx the lists' counts and entries
hipError_t check_indices(const int32_t *ctx_len, const int32_t *keep_from, int batch, int Himp,
                         int cap, const int32_t *sel_idx, int stride, const int32_t *sel_count,
                         hipStream_t st);
hipError_t read_check_flags(uint32_t *out, bool clear);

// Each returns hipSuccess or the launch error.  Shapes are already validated.
hipError_t launch_project(const tb_shape &s, const void *k_cache, const void *w,
                          const int32_t *pos0, int n_tokens, void *kp_cache, hipStream_t st);
hipError_t launch_append_project(const tb_shape &s, const void *k_new, const void *v_new,
                                 int n_new, const void *w, void *k_cache, void *v_cache,
                                 void *kp_cache, const int32_t *ctx_len, hipStream_t st);
// Scores; when n_new > 0 (at most score_max_fused_new()) the same launch
// appends the n_new rows of k_new / v_new at [ctx - n_new, ctx), projects
// and scores them.
int score_max_fused_new();
// When keys16 is not NULL the launch stores, instead of the fp32 scores,
// the top and low 16 bits of every score's order-preserving key into
// keys16 / keys16lo[row][keys16_entry(t)] (row stride keys16_stride(cap))
// and, for positions t = 8m, the top half into sample16[row][m] (row stride
// sample16_stride(cap)); scores is then not written.
hipError_t launch_score(const tb_shape &s, const void *q_imp, void *kp_cache,
                        const int32_t *ctx_len, float *scores, int n_new, const void *k_new,
                        const void *v_new, const void *w, void *k_cache, void *v_cache,
                        uint16_t *keys16, uint16_t *keys16lo, uint16_t *sample16,
                        hipStream_t st);
// Selection; when keep_from is not NULL it also records
// keep_from[b] = max(0, ctx_len[b] - n_new).  keys16 / keys16lo / sample16
// (or NULL): the score launch's split keys, read in place of the fp32
// scores (which may then be NULL); the first pass reads the top halves only.
hipError_t launch_select(const tb_shape &s, const tb_select_params &p, const float *scores,
                         const int32_t *ctx_len, int32_t *sel_idx, int sel_stride,
                         int32_t *sel_count, int32_t *topb_idx, uint32_t *sel_bits,
                         int32_t *keep_from, int n_new, const uint16_t *keys16,
                         const uint16_t *keys16lo, const uint16_t *sample16, hipStream_t st);
// Rows a reuse step appends inside the attention launch (bitmap mode, at
// most score_max_fused_new() of them): the launch copies them into the
// caches and projects their keys, and reads them from k_new / v_new.
struct AttnAppend {
    const void *k_new = nullptr, *v_new = nullptr, *w = nullptr;
    void *k_cache = nullptr, *v_cache = nullptr, *kp_cache = nullptr;
    int n_new = 0;
};
hipError_t launch_attn(const tb_shape &s, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *sel_idx, int sel_stride,
                       const int32_t *sel_count, const uint32_t *sel_bits,
                       const int32_t *keep_from, const int32_t *ctx_len, float softmax_scale,
                       void *out, float *part_o, float *part_ml, uint32_t *counters,
                       hipStream_t st, const AttnAppend &app = AttnAppend());

// Importance-query producer (tb_mlp.hip).  Workspace layout in bytes.
constexpr int kMlpKGrain = 256; // K of both layers is a multiple of this
struct MlpLayout {
    size_t hidden; // [M][F] hidden layer in the dtype
    size_t part;   // k-split partial tiles fp32 [tiles][splits][M/16][64][4]
    size_t counters; // k-split arrival counters u32 [tiles] (kept zero)
    size_t total;
};
// k-splits of an MLP layer with N outputs and K inputs: layers with fewer
// than 128 column tiles of 16 are split four ways over K (when K is a whole
// number of 256-value chunks per split), so that the launch spreads over
// the chip.
inline int mlp_splits(int N, int K)
{
    return N / 16 < 128 && K % (4 * 256) == 0 ? 4 : 1;
}
MlpLayout mlp_layout(const tb_mlp_shape &s);
hipError_t launch_mlp(const tb_mlp_shape &s, const void *h, const void *w1, const void *w2,
                      void *q_imp, void *ws, hipStream_t st);

hipError_t launch_dense(const tb_shape &s, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *ctx_len, float softmax_scale,
                        void *out, float *part_o, float *part_ml, uint32_t *counters,
                        hipStream_t st);

} // namespace tb
