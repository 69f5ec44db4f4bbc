// abi_driver.cpp -- drives the C ABI's host-side code under host
// AddressSanitizer / UndefinedBehaviorSanitizer: size queries over many
// shapes, and every call with arguments that the host checks reject before
// any HIP call (so no GPU is needed).  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cmath>
#include <cstring>

#include "tokenbutler.h"

static tb_shape shape(int b, int hq, int hkv, int himp, int D, int d, int cap, int dt)
{
    tb_shape s;
    s.batch = b;
    s.n_q_heads = hq;
    s.n_kv_heads = hkv;
    s.n_imp_heads = himp;
    s.head_dim = D;
    s.d_imp = d;
    s.ctx_cap = cap;
    s.dtype = dt;
    return s;
}

static int fails = 0;
static void expect(bool ok, const char *what)
{
    if (!ok) {
        std::fprintf(stderr, "unexpected result: %s\n", what);
        ++fails;
    }
}

int main()
{
    expect(tb_version() > 0, "version");
    for (int c = -6; c <= 1; ++c)
        expect(tb_strerror(c) != nullptr && std::strlen(tb_strerror(c)) > 0, "strerror");
    // size queries over shapes, valid and not
    const int caps[] = {-1, 0, 1, 31, 32, 33, 512, 1997, 16384, 16385, 32768, 32769, 65537,
                        131072, 262144, 262145};
    const int Ds[] = {64, 96, 128};
    const int ds[] = {8, 16, 32};
    for (int cap : caps)
        for (int D : Ds)
            for (int d : ds)
                for (int dt = -1; dt <= 2; ++dt) {
                    tb_shape s = shape(3, 8, 2, 8, D, d, cap, dt);
                    tb_select_params p = {50, 1, 2, 7};
                    (void)tb_workspace_bytes(&s, &p);
                    (void)tb_workspace_bytes(&s, nullptr);
                    (void)tb_selection_capacity(&s, &p);
                    (void)tb_bitmap_words(&s);
                }
    tb_shape bad = shape(1, 6, 4, 6, 128, 32, 1024, TB_BF16); // Hq % Hkv != 0
    tb_select_params p = {10, 0, 0, 0};
    expect(tb_workspace_bytes(&bad, &p) == 0, "bad heads: no workspace");
    expect(tb_workspace_bytes(nullptr, &p) == 0, "null shape");
    // every call rejects null pointers and bad shapes on the host
    tb_shape s = shape(2, 8, 2, 8, 128, 32, 4096, TB_BF16);
    char dummy[256] __attribute__((aligned(256)));
    void *f = dummy;
    expect(tb_project_keys(&s, nullptr, f, (const int32_t *)f, 4, f, nullptr) == TB_EINVAL,
           "project null");
    expect(tb_project_keys(&bad, f, f, (const int32_t *)f, 4, f, nullptr) != TB_OK,
           "project bad shape");
    expect(tb_project_keys(&s, f, f, (const int32_t *)f, -1, f, nullptr) == TB_EINVAL,
           "project negative n");
    expect(tb_score(&s, nullptr, f, (const int32_t *)f, (float *)f, f, 1, nullptr) == TB_EINVAL,
           "score null");
    expect(tb_score(&s, f, f, (const int32_t *)f, (float *)f, f, 1, nullptr) == TB_EWORKSPACE,
           "score small workspace");
    tb_select_params badp = {0, 0, 0, 0};
    expect(tb_select(&s, &badp, (const float *)f, (const int32_t *)f, (int32_t *)f,
                     (int32_t *)f, nullptr, nullptr, f, 1 << 30, nullptr) == TB_EINVAL,
           "select bad budget");
    expect(tb_sparse_attn(&s, f, f, f, nullptr, 0, nullptr, nullptr, nullptr,
                          (const int32_t *)f, 0.1f, f, f, 1 << 30, nullptr) == TB_EINVAL,
           "attention without a selection");
    expect(tb_dense_attn(&s, f, f, f, (const int32_t *)f, std::nanf(""), f, f, 1 << 30,
                         nullptr) == TB_EINVAL,
           "dense NaN scale");
    tb_mlp_shape m = {2, 256, 256, 1, 4, 16, TB_BF16, TB_ACT_RELU};
    (void)tb_mlp_workspace_bytes(&m);
    tb_mlp_shape mbad = {0, 100, 256, 1, 4, 16, TB_BF16, TB_ACT_RELU};
    expect(tb_mlp_workspace_bytes(&mbad) == 0, "mlp bad shape");
    expect(tb_predict_queries(&m, nullptr, f, f, f, f, 1 << 20, nullptr) == TB_EINVAL,
           "mlp null");
    tb_step_args a;
    std::memset(&a, 0, sizeof a);
    expect(tb_decode_step(&s, &p, &a, f, 1 << 30, nullptr) == TB_EINVAL, "step null args");
    a.q = a.q_imp = a.w = f;
    a.k_cache = a.v_cache = a.kp_cache = a.out = f;
    a.ctx_len = (const int32_t *)f;
    a.sel_count = (int32_t *)f;
    a.sel_bits = (uint32_t *)f;
    a.keep_from = (int32_t *)f;
    a.refresh = 1;
    a.softmax_scale = 0.1f;
    a.n_new = 9;                    // rows without k_new / v_new
    expect(tb_decode_step(&s, &p, &a, f, 1 << 30, nullptr) == TB_EINVAL, "step missing rows");
    a.n_new = 0;
    expect(tb_decode_step(&s, &p, &a, f, 1, nullptr) == TB_EWORKSPACE, "step small workspace");
    tb_shape big = shape(64, 32, 8, 32, 128, 32, 32768, TB_BF16);
    tb_select_params pb = {3277, 0, 0, 0};
    expect(tb_decode_step_noalloc(&big, &pb, &a, nullptr) == TB_EWORKSPACE, "noalloc too big");
    // the debug-mode switch is host state
    tb_set_check(1);
    expect(tb_check_enabled() == 1, "check on");
    tb_set_check(0);
    expect(tb_check_enabled() == 0, "check off");
    expect(tb_check_flags(nullptr, 1) == TB_EINVAL, "check flags null");
    if (fails == 0)
        std::puts("abi driver done");
    return fails == 0 ? 0 : 1;
}
