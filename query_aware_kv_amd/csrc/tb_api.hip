// tb_api.hip -- the C ABI of libtokenbutler: argument checks on the host,
// workspace layout, and the launch sequence of each entry point.
#include <string.h>

#include <atomic>
#include <mutex>

#include "tb_internal.h"

using namespace tb;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool pow2_group(int a, int b) // a / b in {1, 2, 4, 8}
{
    if (b <= 0 || a % b != 0)
        return false;
    const int g = a / b;
    return g == 1 || g == 2 || g == 4 || g == 8;
}

int check_shape(const tb_shape *s)
{
    if (s == nullptr)
        return TB_EINVAL;
    if (s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->n_imp_heads <= 0 ||
        s->head_dim <= 0 || s->d_imp <= 0 || s->ctx_cap <= 0)
        return TB_EINVAL;
    if (s->n_q_heads % s->n_kv_heads != 0 || s->n_imp_heads % s->n_kv_heads != 0 ||
        s->n_q_heads % s->n_imp_heads != 0)
        return TB_EINVAL;
    if (s->dtype != TB_F32 && s->dtype != TB_BF16)
        return TB_EUNSUPPORTED;
    if (s->head_dim != 64 && s->head_dim != 128)
        return TB_EUNSUPPORTED;
    if (s->d_imp != 16 && s->d_imp != 32)
        return TB_EUNSUPPORTED;
    if (!pow2_group(s->n_q_heads, s->n_kv_heads) || !pow2_group(s->n_imp_heads, s->n_kv_heads))
        return TB_EUNSUPPORTED;
    if (s->ctx_cap > kMaxCtxCap)
        return TB_EUNSUPPORTED;
    return TB_OK;
}

int check_params(const tb_select_params *p)
{
    if (p == nullptr)
        return TB_EINVAL;
    if (p->budget <= 0 || p->radius < 0 || p->radius > 1024 || p->n_sink < 0 || p->n_local < 0)
        return TB_EINVAL;
    return TB_OK;
}

int32_t sel_capacity(const tb_shape &s, const tb_select_params &p)
{
    const long long widened =
        (2LL * p.radius + 1) * (long long)p.budget + (long long)p.n_sink + (long long)p.n_local;
    return (int32_t)(widened < s.ctx_cap ? widened : s.ctx_cap);
}

int hip_rc(hipError_t e) { return e == hipSuccess ? TB_OK : TB_EHIP; }

// Debug mode: the checks of a fused step's inputs (the caches' rows before
// the appended ones, and keep_from only where it is read: on reuse steps).
int check_step_inputs(const tb_shape &s, const tb_step_args &a, hipStream_t st)
{
    const int dt = s.dtype;
    const size_t kv_new = (size_t)s.batch * s.n_kv_heads * a.n_new * s.head_dim;
    const hipError_t es[] = {
        check_dense(a.q, (size_t)s.batch * s.n_q_heads * s.head_dim, dt, TB_CHECK_NONFINITE_INPUT, st),
        a.refresh ? check_dense(a.q_imp, (size_t)s.batch * s.n_imp_heads * s.d_imp, dt,
                                TB_CHECK_NONFINITE_INPUT, st)
                  : hipSuccess,
        check_dense(a.k_new, kv_new, dt, TB_CHECK_NONFINITE_INPUT, st),
        check_dense(a.v_new, kv_new, dt, TB_CHECK_NONFINITE_INPUT, st),
        check_dense(a.w, (size_t)s.head_dim * s.d_imp, dt, TB_CHECK_NONFINITE_INPUT, st),
        check_cache(a.k_cache, a.ctx_len, a.n_new, s.batch, s.n_kv_heads, s.ctx_cap, s.head_dim,
                    dt, TB_CHECK_NONFINITE_CACHE, st),
        check_cache(a.v_cache, a.ctx_len, a.n_new, s.batch, s.n_kv_heads, s.ctx_cap, s.head_dim,
                    dt, TB_CHECK_NONFINITE_CACHE, st),
        check_cache(a.kp_cache, a.ctx_len, a.n_new, s.batch, s.n_kv_heads, s.ctx_cap, s.d_imp, dt,
                    TB_CHECK_NONFINITE_CACHE, st),
        check_indices(a.ctx_len, a.refresh ? nullptr : a.keep_from, s.batch, s.n_imp_heads,
                      s.ctx_cap, nullptr, 0, nullptr, st)};
    for (hipError_t e : es)
        if (e != hipSuccess)
            return TB_EHIP;
    return TB_OK;
}

struct Ws {
    float *part_o;
    float *part_ml;
    uint32_t *counters;
    uint16_t *keys16;
    uint16_t *keys16lo;
    uint16_t *sample16;
};

Ws carve(void *ws, const WsLayout &L)
{
    char *base = (char *)ws;
    return Ws{(float *)(base + L.part_o), (float *)(base + L.part_ml),
              (uint32_t *)(base + L.counters), (uint16_t *)(base + L.keys16),
              (uint16_t *)(base + L.keys16lo), (uint16_t *)(base + L.sample16)};
}

int check_ws(const tb_shape &s, void *ws, size_t ws_bytes, WsLayout *L)
{
    *L = ws_layout(s);
    if (ws == nullptr || ((uintptr_t)ws & (kAlign - 1)) != 0)
        return TB_EINVAL;
    if (ws_bytes < L->total)
        return TB_EWORKSPACE;
    return TB_OK;
}

int check_mlp(const tb_mlp_shape *s)
{
    if (s == nullptr)
        return TB_EINVAL;
    if (s->tokens <= 0 || s->hidden <= 0 || s->inner <= 0 || s->n_slots <= 0 ||
        s->n_imp_heads <= 0 || s->d_imp <= 0)
        return TB_EINVAL;
    if (s->dtype != TB_F32 && s->dtype != TB_BF16)
        return TB_EUNSUPPORTED;
    if (s->act != TB_ACT_RELU && s->act != TB_ACT_SILU)
        return TB_EUNSUPPORTED;
    const long long N = (long long)s->n_slots * s->n_imp_heads * s->d_imp;
    if (s->tokens > 64 || s->hidden % kMlpKGrain != 0 || s->inner % kMlpKGrain != 0 ||
        N % 64 != 0 || N > (1LL << 20) || s->hidden > (1 << 20) || s->inner > (1 << 20))
        return TB_EUNSUPPORTED;
    return TB_OK;
}

#define TB_TRY(x)                                                                                  \
    do {                                                                                           \
        const int rc_ = (x);                                                                       \
        if (rc_ != TB_OK)                                                                          \
            return rc_;                                                                            \
    } while (0)

// Clears n words (a kernel rather than a memset, so that graph capture
// records no memset node).
__global__ void zero_words_kernel(uint32_t *p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t *p, int n, hipStream_t st)
{
    if (n <= 0)
        return hipSuccess;
    const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

int check_step(const tb_shape *shape, const tb_select_params *params, const tb_step_args *a)
{
    TB_TRY(check_shape(shape));
    TB_TRY(check_params(params));
    if (a == nullptr)
        return TB_EINVAL;
    if (a->q == nullptr || a->w == nullptr || a->k_cache == nullptr || a->v_cache == nullptr ||
        a->kp_cache == nullptr || a->ctx_len == nullptr || a->sel_count == nullptr ||
        a->sel_bits == nullptr || a->keep_from == nullptr || a->out == nullptr)
        return TB_EINVAL;
    if (a->n_new < 0 || (a->n_new > 0 && (a->k_new == nullptr || a->v_new == nullptr)))
        return TB_EINVAL;
    if (a->refresh && a->q_imp == nullptr)
        return TB_EINVAL;
    if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) ||
        !aligned16(a->kp_cache) || !aligned16(a->w) || !aligned16(a->k_new) ||
        !aligned16(a->v_new))
        return TB_EINVAL;
    if (!(a->softmax_scale == a->softmax_scale))
        return TB_EINVAL;
    return TB_OK;
}

// The launch sequence of one fused step on a checked workspace.
int decode_step_run(const tb_shape &shape, const tb_select_params &params, const tb_step_args &args,
                    void *ws, const WsLayout &L, hipStream_t st)
{
    const tb_step_args *a = &args;
    Ws W = carve(ws, L);
    const int32_t stride = sel_capacity(shape, params);

    // A few new rows are appended inside the score launch (refresh steps) or
    // the attention launch (reuse steps); more take a launch of their own.
    const bool fused_append = a->n_new > 0 && a->n_new <= score_max_fused_new();
    if (a->n_new > 0 && !fused_append)
        TB_TRY(hip_rc(launch_append_project(shape, a->k_new, a->v_new, a->n_new, a->w,
                                            a->k_cache, a->v_cache, a->kp_cache, a->ctx_len,
                                            st)));
    if (a->refresh) {
        // the score launch stores each score's key as two 16-bit halves and
        // a sample of the top halves; the selection classifies positions
        // from the top halves and completes only its candidates' keys
        TB_TRY(hip_rc(launch_score(shape, a->q_imp, a->kp_cache, a->ctx_len, nullptr,
                                   fused_append ? a->n_new : 0, a->k_new, a->v_new, a->w,
                                   a->k_cache, a->v_cache, W.keys16, W.keys16lo, W.sample16,
                                   st)));
        TB_TRY(hip_rc(launch_select(shape, params, nullptr, a->ctx_len, a->sel_idx, stride,
                                    a->sel_count, nullptr, a->sel_bits, a->keep_from, a->n_new,
                                    W.keys16, W.keys16lo, W.sample16, st)));
    }
    AttnAppend app;
    if (!a->refresh && fused_append) {
        app.k_new = a->k_new;
        app.v_new = a->v_new;
        app.w = a->w;
        app.k_cache = a->k_cache;
        app.v_cache = a->v_cache;
        app.kp_cache = a->kp_cache;
        app.n_new = a->n_new;
    }
    return hip_rc(launch_attn(shape, a->q, a->k_cache, a->v_cache, a->sel_idx, stride,
                              a->sel_count, a->sel_bits, a->keep_from, a->ctx_len,
                              a->softmax_scale, a->out, W.part_o, W.part_ml, W.counters, st,
                              app));
}

// ---------------------------------------------------------------- scratch
// The device memory of tb_decode_step_noalloc: a file-scope array that every
// device holds from the library's load until the process ends.  In host code
// the array's name only stands for the symbol; its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// that address is what the kernels receive.
__device__ __align__(256) unsigned char scratch[TB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return TB_EHIP;
    if (dev < 0 || dev >= kMaxDevices)
        return TB_EUNSUPPORTED;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return TB_EHIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return TB_OK;
}

} // namespace

extern "C" {

int tb_version(void) { return 10000; }

const char *tb_strerror(int code)
{
    switch (code) {
    case TB_OK: return "ok";
    case TB_EINVAL: return "invalid argument (null pointer, bad size, misaligned pointer or inconsistent head counts)";
    case TB_EUNSUPPORTED: return "unsupported dtype, head_dim, d_imp, group size, ctx_cap, activation or MLP size";
    case TB_EWORKSPACE:
        return "workspace smaller than tb_workspace_bytes() (for tb_decode_step_noalloc: the "
               "shape needs more than the library's fixed device scratch, "
               "TB_NOALLOC_SCRATCH_BYTES)";
    case TB_EHIP: return "HIP kernel launch failed";
    }
    return "unknown tokenbutler error code";
}

size_t tb_workspace_bytes(const tb_shape *shape, const tb_select_params *params)
{
    if (check_shape(shape) != TB_OK)
        return 0;
    if (params != nullptr && check_params(params) != TB_OK)
        return 0;
    return ws_layout(*shape).total;
}

int32_t tb_selection_capacity(const tb_shape *shape, const tb_select_params *params)
{
    if (check_shape(shape) != TB_OK || check_params(params) != TB_OK)
        return 0;
    return sel_capacity(*shape, *params);
}

int32_t tb_bitmap_words(const tb_shape *shape)
{
    if (check_shape(shape) != TB_OK)
        return 0;
    return bitmap_words(shape->ctx_cap);
}

int tb_project_keys(const tb_shape *shape, const void *k_cache, const void *w,
                    const int32_t *pos0, int32_t n_tokens, void *kp_cache, void *stream)
{
    TB_TRY(check_shape(shape));
    if (k_cache == nullptr || w == nullptr || pos0 == nullptr || kp_cache == nullptr ||
        n_tokens < 0)
        return TB_EINVAL;
    if (!aligned16(k_cache) || !aligned16(kp_cache) || !aligned16(w))
        return TB_EINVAL;
    if (n_tokens == 0)
        return TB_OK;
    if ((long long)shape->batch * shape->n_kv_heads * n_tokens > 0x7fffffffLL)
        return TB_EINVAL;
    if (check_enabled()) {
        const hipStream_t st = (hipStream_t)stream;
        TB_TRY(hip_rc(check_dense(w, (size_t)shape->head_dim * shape->d_imp, shape->dtype,
                                  TB_CHECK_NONFINITE_INPUT, st)));
        TB_TRY(hip_rc(check_cache(k_cache, nullptr, 0, shape->batch, shape->n_kv_heads,
                                  shape->ctx_cap, shape->head_dim, shape->dtype,
                                  TB_CHECK_NONFINITE_CACHE, st)));
    }
    return hip_rc(launch_project(*shape, k_cache, w, pos0, n_tokens, kp_cache,
                                 (hipStream_t)stream));
}

int tb_score(const tb_shape *shape, const void *q_imp, const void *kp_cache,
             const int32_t *ctx_len, float *scores, void *ws, size_t ws_bytes, void *stream)
{
    TB_TRY(check_shape(shape));
    if (q_imp == nullptr || kp_cache == nullptr || ctx_len == nullptr || scores == nullptr)
        return TB_EINVAL;
    if (!aligned16(kp_cache))
        return TB_EINVAL;
    WsLayout L;
    TB_TRY(check_ws(*shape, ws, ws_bytes, &L));
    if (check_enabled()) {
        const hipStream_t st = (hipStream_t)stream;
        TB_TRY(hip_rc(check_dense(q_imp, (size_t)shape->batch * shape->n_imp_heads * shape->d_imp,
                                  shape->dtype, TB_CHECK_NONFINITE_INPUT, st)));
        TB_TRY(hip_rc(check_cache(kp_cache, ctx_len, 0, shape->batch, shape->n_kv_heads,
                                  shape->ctx_cap, shape->d_imp, shape->dtype,
                                  TB_CHECK_NONFINITE_CACHE, st)));
        TB_TRY(hip_rc(check_indices(ctx_len, nullptr, shape->batch, shape->n_imp_heads,
                                    shape->ctx_cap, nullptr, 0, nullptr, st)));
    }
    return hip_rc(launch_score(*shape, q_imp, const_cast<void *>(kp_cache), ctx_len, scores, 0,
                               nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, (hipStream_t)stream));
}

int tb_select(const tb_shape *shape, const tb_select_params *params, const float *scores,
              const int32_t *ctx_len, int32_t *sel_idx, int32_t *sel_count, int32_t *topb_idx,
              uint32_t *sel_bits, void *ws, size_t ws_bytes, void *stream)
{
    TB_TRY(check_shape(shape));
    TB_TRY(check_params(params));
    if (scores == nullptr || ctx_len == nullptr || sel_count == nullptr ||
        (sel_idx == nullptr && sel_bits == nullptr))
        return TB_EINVAL;
    if (!aligned16(scores))
        return TB_EINVAL;
    WsLayout L;
    TB_TRY(check_ws(*shape, ws, ws_bytes, &L));
    if (check_enabled()) {
        const hipStream_t st = (hipStream_t)stream;
        TB_TRY(hip_rc(check_cache(scores, ctx_len, 0, shape->batch, shape->n_imp_heads,
                                  shape->ctx_cap, 1, TB_F32, TB_CHECK_NONFINITE_SCORES, st)));
        TB_TRY(hip_rc(check_indices(ctx_len, nullptr, shape->batch, shape->n_imp_heads,
                                    shape->ctx_cap, nullptr, 0, nullptr, st)));
    }
    return hip_rc(launch_select(*shape, *params, scores, ctx_len, sel_idx,
                                sel_capacity(*shape, *params), sel_count, topb_idx, sel_bits,
                                nullptr, 0, nullptr, nullptr, nullptr, (hipStream_t)stream));
}

int tb_sparse_attn(const tb_shape *shape, const void *q, const void *k_cache,
                   const void *v_cache, const int32_t *sel_idx, int32_t sel_stride,
                   const int32_t *sel_count, const uint32_t *sel_bits, const int32_t *keep_from,
                   const int32_t *ctx_len, float softmax_scale, void *out, void *ws,
                   size_t ws_bytes, void *stream)
{
    TB_TRY(check_shape(shape));
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || ctx_len == nullptr ||
        out == nullptr)
        return TB_EINVAL;
    if (sel_bits == nullptr && (sel_idx == nullptr || sel_count == nullptr || sel_stride <= 0))
        return TB_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return TB_EINVAL;
    if (!(softmax_scale == softmax_scale))
        return TB_EINVAL;
    WsLayout L;
    TB_TRY(check_ws(*shape, ws, ws_bytes, &L));
    if (check_enabled()) {
        const hipStream_t st = (hipStream_t)stream;
        const tb_shape &s = *shape;
        TB_TRY(hip_rc(check_dense(q, (size_t)s.batch * s.n_q_heads * s.head_dim, s.dtype,
                                  TB_CHECK_NONFINITE_INPUT, st)));
        TB_TRY(hip_rc(check_cache(k_cache, ctx_len, 0, s.batch, s.n_kv_heads, s.ctx_cap,
                                  s.head_dim, s.dtype, TB_CHECK_NONFINITE_CACHE, st)));
        TB_TRY(hip_rc(check_cache(v_cache, ctx_len, 0, s.batch, s.n_kv_heads, s.ctx_cap,
                                  s.head_dim, s.dtype, TB_CHECK_NONFINITE_CACHE, st)));
        TB_TRY(hip_rc(check_indices(ctx_len, keep_from, s.batch, s.n_imp_heads, s.ctx_cap,
                                    sel_bits == nullptr ? sel_idx : nullptr, sel_stride,
                                    sel_count, st)));
    }
    Ws W = carve(ws, L);
    return hip_rc(launch_attn(*shape, q, k_cache, v_cache, sel_idx, sel_stride, sel_count,
                              sel_bits, keep_from, ctx_len, softmax_scale, out, W.part_o,
                              W.part_ml, W.counters, (hipStream_t)stream));
}

int tb_dense_attn(const tb_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *ctx_len, float softmax_scale, void *out, void *ws,
                  size_t ws_bytes, void *stream)
{
    TB_TRY(check_shape(shape));
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || ctx_len == nullptr ||
        out == nullptr)
        return TB_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return TB_EINVAL;
    if (!(softmax_scale == softmax_scale))
        return TB_EINVAL;
    WsLayout L;
    TB_TRY(check_ws(*shape, ws, ws_bytes, &L));
    if (check_enabled()) {
        const hipStream_t st = (hipStream_t)stream;
        const tb_shape &s = *shape;
        TB_TRY(hip_rc(check_dense(q, (size_t)s.batch * s.n_q_heads * s.head_dim, s.dtype,
                                  TB_CHECK_NONFINITE_INPUT, st)));
        TB_TRY(hip_rc(check_cache(k_cache, ctx_len, 0, s.batch, s.n_kv_heads, s.ctx_cap,
                                  s.head_dim, s.dtype, TB_CHECK_NONFINITE_CACHE, st)));
        TB_TRY(hip_rc(check_cache(v_cache, ctx_len, 0, s.batch, s.n_kv_heads, s.ctx_cap,
                                  s.head_dim, s.dtype, TB_CHECK_NONFINITE_CACHE, st)));
        TB_TRY(hip_rc(check_indices(ctx_len, nullptr, s.batch, s.n_imp_heads, s.ctx_cap, nullptr,
                                    0, nullptr, st)));
    }
    Ws W = carve(ws, L);
    return hip_rc(launch_dense(*shape, q, k_cache, v_cache, ctx_len, softmax_scale, out, W.part_o,
                               W.part_ml, W.counters, (hipStream_t)stream));
}

size_t tb_mlp_workspace_bytes(const tb_mlp_shape *shape)
{
    if (check_mlp(shape) != TB_OK)
        return 0;
    return mlp_layout(*shape).total;
}

int tb_predict_queries(const tb_mlp_shape *shape, const void *h, const void *w1, const void *w2,
                       void *q_imp, void *ws, size_t ws_bytes, void *stream)
{
    TB_TRY(check_mlp(shape));
    if (h == nullptr || w1 == nullptr || w2 == nullptr || q_imp == nullptr)
        return TB_EINVAL;
    if (!aligned16(h) || !aligned16(w1) || !aligned16(w2))
        return TB_EINVAL;
    if (ws == nullptr || ((uintptr_t)ws & (kAlign - 1)) != 0)
        return TB_EINVAL;
    if (ws_bytes < mlp_layout(*shape).total)
        return TB_EWORKSPACE;
    if (check_enabled()) {
        const hipStream_t st = (hipStream_t)stream;
        const tb_mlp_shape &s = *shape;
        const size_t N = (size_t)s.n_slots * s.n_imp_heads * s.d_imp;
        TB_TRY(hip_rc(check_dense(h, (size_t)s.tokens * s.hidden, s.dtype,
                                  TB_CHECK_NONFINITE_INPUT, st)));
        TB_TRY(hip_rc(check_dense(w1, (size_t)s.inner * s.hidden, s.dtype,
                                  TB_CHECK_NONFINITE_INPUT, st)));
        TB_TRY(hip_rc(check_dense(w2, N * s.inner, s.dtype, TB_CHECK_NONFINITE_INPUT, st)));
    }
    return hip_rc(launch_mlp(*shape, h, w1, w2, q_imp, ws, (hipStream_t)stream));
}

int tb_decode_step(const tb_shape *shape, const tb_select_params *params,
                   const tb_step_args *a, void *ws, size_t ws_bytes, void *stream)
{
    TB_TRY(check_step(shape, params, a));
    WsLayout L;
    TB_TRY(check_ws(*shape, ws, ws_bytes, &L));
    if (check_enabled())
        TB_TRY(check_step_inputs(*shape, *a, (hipStream_t)stream));
    return decode_step_run(*shape, *params, *a, ws, L, (hipStream_t)stream);
}

int tb_decode_step_noalloc(const tb_shape *shape, const tb_select_params *params,
                           const tb_step_args *a, void *stream)
{
    TB_TRY(check_step(shape, params, a));
    const WsLayout L = ws_layout(*shape);
    if (L.total > (size_t)TB_NOALLOC_SCRATCH_BYTES)
        return TB_EWORKSPACE;
    void *ws = nullptr;
    TB_TRY(scratch_of_current_device(&ws));
    hipStream_t st = (hipStream_t)stream;
    // the scratch keeps whatever the last call on this device left: the
    // words that must start at zero are cleared by a kernel (not a memset
    // node, so that the call can be captured in a graph)
    TB_TRY(hip_rc(launch_zero_words((uint32_t *)((char *)ws + L.zeroed), L.zeroed_words, st)));
    if (check_enabled())
        TB_TRY(check_step_inputs(*shape, *a, st));
    return decode_step_run(*shape, *params, *a, ws, L, st);
}

void tb_set_check(int on) { set_check(on != 0); }

int tb_check_enabled(void) { return check_enabled() ? 1 : 0; }

int tb_check_flags(uint32_t *flags, int clear)
{
    if (flags == nullptr)
        return TB_EINVAL;
    return hip_rc(read_check_flags(flags, clear != 0));
}

} // extern "C"
