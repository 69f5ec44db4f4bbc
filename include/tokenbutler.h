/*
 * tokenbutler.h -- C ABI of libtokenbutler.so, the MI355X (gfx950) sparse-decode
 * hot path of TokenButler ("TokenButler: Token Importance is Predictable").
 *
 * At each decode step a low-dimensional importance query per head is scored
 * against a learned low-dimensional projection of the cached keys; each head
 * keeps its top-B tokens, optionally widened by neighbor fetching and reused
 * across a prediction interval; exact softmax attention then runs over the
 * gathered K/V rows only while the full cache stays resident.
 *
 * Citations name the page and section of the method description:
 *   [ABS]  TokenButler abstract, 2026 version (author page, searcharxiv.com)
 *   [ARCH] gist.science technical summary, Methodology > Core Architecture
 *   [INF]  gist.science technical summary, Inference Strategy > Optimizations
 *   [RES]  gist.science technical summary, Key Contributions and Experimental
 *          Results (the speedups against dense attention, on the GPU and with
 *          the cache offloaded to CPU memory)
 *   [SIG]  gist.science technical summary, Significance
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers on the current HIP device, except
 *   the tb_shape / tb_select_params / tb_step_args structs themselves, which
 *   are read on the host during the call.  The caller owns every buffer; the
 *   library never allocates device memory, frees, or keeps a pointer after a
 *   call returns.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   the call returns without waiting for it.  Calls on one stream run in
 *   order; calls that share a workspace must not overlap.
 * - Element dtype: every K/V/Kp/W/q/q_imp/out tensor has the dtype of
 *   tb_shape.dtype (TB_F32 or TB_BF16).  Scores are fp32.  Index tensors are
 *   int32.
 * - Layouts (row-major, innermost last):
 *     K, V cache   [batch][n_kv_heads][ctx_cap][head_dim]
 *     Kp cache     [batch][n_kv_heads][ctx_cap][d_imp]      (projected keys)
 *     W            [head_dim][d_imp]  one matrix shared by all KV heads
 *     q            [batch][n_q_heads][head_dim]
 *     q_imp        [batch][n_imp_heads][d_imp]
 *     scores       [batch][n_imp_heads][ctx_cap]
 *     sel_idx      [batch][n_imp_heads][sel_stride]  ascending positions
 *     sel_count    [batch][n_imp_heads]
 *     sel_bits     [batch][n_imp_heads][tb_bitmap_words()]  bit t%32 of word
 *                  t/32 set iff position t is selected
 *     ctx_len, keep_from, pos0   [batch]
 *     out          [batch][n_q_heads][head_dim]
 * - Head maps: query head h reads KV head h*Hkv/Hq and importance head
 *   h*Himp/Hq; importance head i scores KV head i*Hkv/Himp (integer division).
 * - ctx_len[b] is the number of valid cache rows of sequence b; values are
 *   clamped to [0, ctx_cap] on the device.
 * - Arithmetic: projected keys are fp64 sums in ascending head_dim order,
 *   rounded once (to nearest even) to the dtype; scores are fp32 fused
 *   multiply-add chains in ascending d_imp order starting from +0; attention
 *   accumulates in fp32.  Inputs must be finite.
 * - Offloading ([ABS], [RES]: decoding with the cache in CPU memory): the K
 *   and V caches may live in device memory or in pinned host memory that is
 *   mapped for the device (hipHostMalloc; pass the device-side address from
 *   hipHostGetDevicePointer).  The kernels then read only the rows they use
 *   over the host link and write appended rows there; the projected-key
 *   cache, queries, scores, selection state and workspace stay in device
 *   memory.  Results do not depend on where the caches live.
 * - Alignment: tensors read or written in 16-byte pieces (K/V/Kp caches, q,
 *   W, k_new, v_new, the scores given to tb_select) must be 16-byte aligned,
 *   else TB_EINVAL.
 * - Return value: TB_OK, or a negative TB_E* code.  Every argument check runs
 *   on the host before anything is enqueued, so an error return means nothing
 *   was launched -- except TB_EHIP, which reports a failed launch.
 * - Workspace: calls that take `ws` need at least tb_workspace_bytes() bytes
 *   of device memory, 256-byte aligned, ZERO-FILLED before its first use.
 *   Every call leaves it in a state the next call with the same shape
 *   accepts, so one allocation can be reused; zero-fill it again after a
 *   TB_EHIP error or before using it with another shape.  Calls that share
 *   a workspace must not overlap.
 */
#ifndef TOKENBUTLER_H
#define TOKENBUTLER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TB_OK 0
#define TB_EINVAL (-1)       /* null pointer, bad size or inconsistent heads */
#define TB_EUNSUPPORTED (-2) /* dtype / head_dim / d_imp / group size / ctx_cap outside the built set */
#define TB_EWORKSPACE (-3)   /* workspace smaller than tb_workspace_bytes() */
#define TB_EHIP (-4)         /* a kernel launch failed */

#define TB_F32 0
#define TB_BF16 1

typedef struct tb_shape {
    int32_t batch;       /* sequences, >= 1 */
    int32_t n_q_heads;   /* Hq, a multiple of n_imp_heads */
    int32_t n_kv_heads;  /* Hkv; Hq/Hkv in {1,2,4,8} */
    int32_t n_imp_heads; /* Himp, a multiple of Hkv; Himp/Hkv in {1,2,4,8} */
    int32_t head_dim;    /* D in {64, 128} */
    int32_t d_imp;       /* d in {16, 32} */
    int32_t ctx_cap;     /* cache capacity in tokens, 1 .. 262144 */
    int32_t dtype;       /* TB_F32 or TB_BF16 */
} tb_shape;

typedef struct tb_select_params {
    int32_t budget;  /* B >= 1: tokens kept per importance head before widening */
    int32_t radius;  /* r in [0, 1024]: neighbor-fetch radius */
    int32_t n_sink;  /* >= 0: the first n_sink tokens are always kept ([INF] sink) */
    int32_t n_local; /* >= 0: the last n_local tokens are always kept ([INF] local window) */
} tb_select_params;

/* Library version (major*10000 + minor*100 + patch).  Host only. */
int tb_version(void);

/* Static description of a return code.  Host only. */
const char *tb_strerror(int code);

/* Bytes of workspace needed by tb_score / tb_select / tb_sparse_attn /
 * tb_decode_step for this shape, or 0 if the shape or params are invalid.
 * Host only. */
size_t tb_workspace_bytes(const tb_shape *shape, const tb_select_params *params);

/* Capacity of one head's selected-index list:
 * min(ctx_cap, (2r+1)*B + n_sink + n_local).  The sel_idx stride written by
 * tb_select and tb_decode_step.  0 if invalid. */
int32_t tb_selection_capacity(const tb_shape *shape, const tb_select_params *params);

/* 32-bit words of one head's selection bitmap: ceil(ctx_cap / 32).  0 if the
 * shape is invalid. */
int32_t tb_bitmap_words(const tb_shape *shape);

/*
 * tb_project_keys -- append-time key projection into the projected-key cache.
 * [ARCH]: the real cache keys are mapped into the low-dimensional importance
 * space by one learned matrix per consumer layer; [INF]: this is done for a
 * batch of new tokens at a time rather than token by token.
 *
 * For every sequence b, KV head g and j in [0, n_tokens) with
 * t = pos0[b] + j in [0, ctx_cap):
 *     kp_cache[b][g][t][:] = round( k_cache[b][g][t][:] . W )   (fp64 sum)
 * Rows with t outside [0, ctx_cap) are skipped.  pos0 is a device array.
 * n_tokens == 0 is a no-op.  Errors: TB_EINVAL (null pointer, n_tokens < 0),
 * TB_EUNSUPPORTED.
 */
int tb_project_keys(const tb_shape *shape, const void *k_cache, const void *w,
                    const int32_t *pos0, int32_t n_tokens, void *kp_cache, void *stream);

/*
 * tb_score -- importance scores.  [ARCH]: each predicted importance query is
 * dotted with the projected keys of its KV head.
 *
 * scores[b][i][t] = acc_d, acc_0 = +0, acc_{j+1} = fmaf(q_imp[b][i][j],
 * kp_cache[b][g(i)][t][j], acc_j) in fp32, for t < ctx_len[b]; entries
 * t >= ctx_len[b] are left untouched.  The workspace is not used by this
 * call but must still be given (it is checked like the others).
 * Errors: TB_EINVAL, TB_EUNSUPPORTED, TB_EWORKSPACE.
 */
int tb_score(const tb_shape *shape, const void *q_imp, const void *kp_cache,
             const int32_t *ctx_len, float *scores, void *ws, size_t ws_bytes, void *stream);

/*
 * tb_select -- per-head top-B under a fixed budget, then neighbor fetching.
 * [ABS], [ARCH]: per-token selection of the highest-scoring tokens under a
 * fixed budget; [INF]: each kept token is widened to its spatial neighbors,
 * and the cache is split into a sink, a local window and the important
 * buffer that the scores fill.
 *
 * For each (b, i) with n = ctx_len[b], lo = min(n_sink, n) and
 * hi = max(lo, n - n_local) (the middle region is [lo, hi)):
 *   T = the first min(B, hi - lo) tokens of [lo, hi) ordered by (score
 *       descending, position ascending); -0.0 and +0.0 compare equal;
 *   S = union over t in T of [max(0, t-r), min(n-1, t+r)], united with the
 *       sink [0, lo) and the local window [hi, n).
 * With n_sink = n_local = 0 this is plain top-B over [0, n) then widening.
 * sel_count[b][i] = |S|.  If sel_idx is not NULL, sel_idx[b][i][0 .. |S|)
 * receives S ascending (stride tb_selection_capacity() =
 * min(ctx_cap, (2r+1) B + n_sink + n_local)).  If topb_idx is not NULL it
 * receives T ascending with stride B (its count is min(B, hi - lo)).  If
 * sel_bits is not NULL it receives S as a bitmap (all tb_bitmap_words()
 * words of the head are written; bits at positions >= n are zero).  At
 * least one of sel_idx and sel_bits must be given.
 * Errors: TB_EINVAL, TB_EUNSUPPORTED, TB_EWORKSPACE.
 */
int tb_select(const tb_shape *shape, const tb_select_params *params, const float *scores,
              const int32_t *ctx_len, int32_t *sel_idx, int32_t *sel_count, int32_t *topb_idx,
              uint32_t *sel_bits, void *ws, size_t ws_bytes, void *stream);

/*
 * tb_sparse_attn -- exact softmax attention over the selected rows only.
 * [ABS], [SIG]: the full cache stays resident and each step reads only the
 * selected tokens.
 *
 * For query head h (KV head g, importance head i) of sequence b with
 * n = ctx_len[b], the attended set is
 *   A = { sel_idx[b][i][k] : k < sel_count[b][i], value in [0, n) }
 *       united with [keep_from[b], n) when keep_from is not NULL,
 * and out[b][h] = sum_{t in A} softmax_t(scale * q[b][h] . K[b][g][t]) V[b][g][t],
 * accumulated in fp32 and rounded to the dtype.  An empty A gives a zero row.
 * sel_idx lists must be ascending and duplicate-free; sel_count is clamped to
 * sel_stride.  When sel_bits is not NULL the selected set is read from that
 * bitmap instead and sel_idx / sel_count are ignored (they may be NULL);
 * the two routes accumulate the rows in different orders and agree to
 * rounding.  Rows that several query heads of one KV head select are
 * requested at about the same time, so HBM serves each about once.
 * Errors: TB_EINVAL, TB_EUNSUPPORTED, TB_EWORKSPACE.
 */
int tb_sparse_attn(const tb_shape *shape, const void *q, const void *k_cache,
                   const void *v_cache, const int32_t *sel_idx, int32_t sel_stride,
                   const int32_t *sel_count, const uint32_t *sel_bits, const int32_t *keep_from,
                   const int32_t *ctx_len, float softmax_scale, void *out, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * tb_dense_attn -- dense decode attention over the whole context, the
 * baseline that TokenButler's speedups are measured against ([RES]: the
 * on-GPU and CPU-offloading latency comparisons with dense attention).
 *
 * For query head h (KV head g = h*Hkv/Hq) of sequence b with n = ctx_len[b],
 *   out[b][h] = sum_{t < n} softmax_t(scale * q[b][h] . K[b][g][t]) V[b][g][t],
 * accumulated in fp32 and rounded to the dtype; n = 0 gives a zero row.
 * Layouts as for tb_sparse_attn.  Every K/V row is read once and serves all
 * query heads of its KV head.  The workspace holds the per-chunk partials.
 * Errors: TB_EINVAL, TB_EUNSUPPORTED, TB_EWORKSPACE.
 */
int tb_dense_attn(const tb_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *ctx_len, float softmax_scale, void *out, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * The importance-query producer ([ARCH] Query Prediction): a lightweight MLP
 * maps the hidden states of a producer layer to G slot-specific importance
 * queries per importance head, one slot per consumer layer it serves.
 */
#define TB_ACT_RELU 0
#define TB_ACT_SILU 1

typedef struct tb_mlp_shape {
    int32_t tokens;      /* M: hidden-state rows (sequences in a decode step), 1 .. 64 */
    int32_t hidden;      /* E: producer hidden size, a multiple of 256 */
    int32_t inner;       /* F: MLP inner width, a multiple of 256 */
    int32_t n_slots;     /* G: query slots (consumer layers served), >= 1 */
    int32_t n_imp_heads; /* Himp: importance heads of each consumer layer */
    int32_t d_imp;       /* d: importance dimension; G*Himp*d a multiple of 64 */
    int32_t dtype;       /* TB_F32 or TB_BF16 (inputs, weights, hidden layer, output) */
    int32_t act;         /* TB_ACT_RELU or TB_ACT_SILU */
} tb_mlp_shape;

/* Workspace bytes of tb_predict_queries (0 if the shape is invalid). */
size_t tb_mlp_workspace_bytes(const tb_mlp_shape *shape);

/*
 * tb_predict_queries -- importance queries from hidden states.
 *   u[m][f] = round( act( sum_e h[m][e] * w1[f][e] ) )
 *   q_imp[g][m][i][j] = round( sum_f u[m][f] * w2[(g*Himp + i)*d + j][f] )
 * h [M][E], w1 [F][E], w2 [G*Himp*d][F] (output-major, like a linear
 * layer's weight), q_imp [G][M][Himp][d]: slot g is the q_imp argument of
 * tb_score / tb_decode_step for its consumer layer (batch = M).  No biases.
 * Products are accumulated in fp32 on the matrix cores; round() is to the
 * dtype, nearest even.  h, w1, w2 16-byte aligned.  The workspace (at least
 * tb_mlp_workspace_bytes(), 256-byte aligned) holds the hidden layer and,
 * for layers with few output columns, partial sums over parts of k and
 * their arrival counters: it must be zero-filled before its first use, and
 * every completed call leaves the counters zero again.  Calls sharing a
 * workspace must not overlap.
 * Errors: TB_EINVAL, TB_EUNSUPPORTED, TB_EWORKSPACE, TB_EHIP.
 */
int tb_predict_queries(const tb_mlp_shape *shape, const void *h, const void *w1, const void *w2,
                       void *q_imp, void *ws, size_t ws_bytes, void *stream);

/* Arguments of one fused decode step (all pointers device pointers). */
typedef struct tb_step_args {
    const void *q;        /* [b][Hq][D] */
    const void *q_imp;    /* [b][Himp][d]; read on refresh steps only */
    const void *k_new;    /* [b][Hkv][n_new][D]; NULL iff n_new == 0 */
    const void *v_new;    /* [b][Hkv][n_new][D]; NULL iff n_new == 0 */
    int32_t n_new;        /* tokens appended by this step, >= 0 */
    int32_t refresh;      /* non-zero: recompute the selection this step */
    const void *w;        /* [D][d] key-projection matrix */
    void *k_cache;        /* [b][Hkv][ctx_cap][D] */
    void *v_cache;        /* [b][Hkv][ctx_cap][D] */
    void *kp_cache;       /* [b][Hkv][ctx_cap][d] */
    const int32_t *ctx_len; /* [b]: context length AFTER the append */
    float softmax_scale;
    int32_t *sel_idx;     /* [b][Himp][tb_selection_capacity()] or NULL */
    int32_t *sel_count;   /* state [b][Himp] */
    uint32_t *sel_bits;   /* state [b][Himp][tb_bitmap_words()] */
    int32_t *keep_from;   /* state [b] */
    void *out;            /* [b][Hq][D] */
} tb_step_args;

/*
 * tb_decode_step -- one fused decode step of one consumer layer.
 * [INF]: projected keys are extended as tokens arrive; the predictor runs
 * only every P steps (the caller sets `refresh` when step % P == 0) and its
 * selection, widened by neighbor fetching, is reused in between; [ABS],
 * [SIG]: attention reads only the selected rows.
 *
 * 1. The n_new rows of k_new / v_new are written to positions
 *    [ctx_len[b] - n_new, ctx_len[b]) of the caches and their keys projected
 *    (as tb_project_keys).
 * 2. If refresh: scores over [0, ctx_len[b]) (as tb_score), T and S (as
 *    tb_select) are stored in sel_count / sel_bits (and as the ascending
 *    list in sel_idx when it is not NULL), and keep_from[b] = ctx_len[b] -
 *    n_new.
 * 3. out = attention over S united with [keep_from[b], ctx_len[b]) (as
 *    tb_sparse_attn), so tokens appended since the last refresh are always
 *    attended.
 * On a non-refresh step the state (sel_bits and keep_from) is read, not
 * written.  ctx_len[b] - n_new
 * must be >= 0.  Errors: TB_EINVAL, TB_EUNSUPPORTED, TB_EWORKSPACE.
 * Launches on `stream`: a refresh step is three (scores, selection,
 * attention) and a non-refresh step one (attention); up to 8 new rows are
 * appended inside the first of them, more in a launch of their own before.
 */
int tb_decode_step(const tb_shape *shape, const tb_select_params *params,
                   const tb_step_args *args, void *ws, size_t ws_bytes, void *stream);

/*
 * tb_decode_step_noalloc -- tb_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a fixed device array
 * inside the library (TB_NOALLOC_SCRATCH_BYTES per GPU, held from the
 * library's load until the process ends), so the caller passes only the
 * step's arguments.  Same computation, kernels and results as
 * tb_decode_step; no hipMalloc, hipFree or allocating library call is made.
 * Each call first clears the scratch words that must start at zero with a
 * small kernel on `stream`.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on
 * one GPU (other streams, other threads) race and give undefined results.
 * Errors: as tb_decode_step; TB_EWORKSPACE when tb_workspace_bytes() of the
 * shape exceeds TB_NOALLOC_SCRATCH_BYTES (nothing is launched);
 * TB_EHIP if the scratch's device address cannot be obtained.
 */
#define TB_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int tb_decode_step_noalloc(const tb_shape *shape, const tb_select_params *params,
                           const tb_step_args *args, void *stream);

/*
 * Debug mode (TB_CHECK).  Off by default; the environment variable TB_CHECK
 * set to anything but "" or "0" turns it on when the library is first used,
 * and tb_set_check() overrides that.  While it is on, every call enqueues
 * small check kernels on its stream before its own kernels; each failed
 * check ORs its bit into a word kept on the device (one per GPU).  The hot
 * path itself never faults on the conditions checked here -- it clamps
 * context lengths, list counts and list entries, and produces garbage from
 * non-finite inputs -- so the bits say why a result may be wrong.
 *   TB_CHECK_NONFINITE_INPUT  a NaN or infinity in q, q_imp, k_new, v_new,
 *                             w (tb_predict_queries: h, w1, w2)
 *   TB_CHECK_NONFINITE_CACHE  ... in the rows [0, ctx_len) of the K, V or
 *                             projected-key cache that the call reads (in
 *                             tb_decode_step the rows before the appended
 *                             ones; in tb_project_keys the whole key cache)
 *   TB_CHECK_CTX_RANGE        ctx_len[b] outside [0, ctx_cap]
 *   TB_CHECK_KEEP_RANGE       keep_from[b] outside [0, ctx_cap] (attention)
 *   TB_CHECK_SEL_RANGE        a list count outside [0, sel_stride], or a list
 *                             entry outside [0, ctx_cap) or not ascending
 *                             (tb_sparse_attn with lists)
 *   TB_CHECK_NONFINITE_SCORES a NaN or infinity among the scores of
 *                             [0, ctx_len) (tb_select)
 * tb_check_flags waits for the device (hipDeviceSynchronize), stores the
 * current device's word in *flags and, if clear is non-zero, resets it to
 * 0.  Returns TB_OK, TB_EINVAL (flags NULL) or TB_EHIP.
 */
#define TB_CHECK_NONFINITE_INPUT 1u
#define TB_CHECK_NONFINITE_CACHE 2u
#define TB_CHECK_CTX_RANGE 4u
#define TB_CHECK_KEEP_RANGE 8u
#define TB_CHECK_SEL_RANGE 16u
#define TB_CHECK_NONFINITE_SCORES 32u
void tb_set_check(int on);
int tb_check_enabled(void);
int tb_check_flags(uint32_t *flags, int clear);

#ifdef __cplusplus
}
#endif

#endif /* TOKENBUTLER_H */
