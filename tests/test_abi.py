"""The C ABI: exported symbols and host-side argument checks (no GPU).

Every call below fails validation on the host, before any HIP call, so it is
safe on a machine without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

from query_aware_kv_amd import tokenbutler as tbl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokenbutler.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tb_[a-z_]+)\s*\(", text)))


def _exported_symbols():
    out = subprocess.check_output(["nm", "-D", "--defined-only", tbl.LIB_PATH]).decode()
    return {ln.split()[-1] for ln in out.splitlines() if " T " in ln}


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert {"tb_project_keys", "tb_score", "tb_select", "tb_sparse_attn", "tb_dense_attn",
            "tb_decode_step", "tb_predict_queries", "tb_mlp_workspace_bytes"} <= set(declared)
    exported = _exported_symbols()
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    L = tbl.lib()
    for f in declared:
        assert hasattr(L, f)


def _shape(**kw):
    d = dict(batch=1, n_q_heads=32, n_kv_heads=8, n_imp_heads=32, head_dim=128, d_imp=32,
             ctx_cap=32768, dtype=tbl.TB_BF16)
    d.update(kw)
    return tbl.Shape(**d)


def test_version_and_strerror():
    assert tbl.version() >= 10000
    for code in (0, -1, -2, -3, -4):
        assert tbl.strerror(code)
    assert "unknown" in tbl.strerror(7)


def test_workspace_and_capacity():
    s = _shape()
    p = tbl.make_params(3277, 0)
    ws = tbl.workspace_bytes(s, p)
    # scores alone need b * Himp * cap * 4 bytes
    assert ws >= 32 * 32768 * 4 and ws % 256 == 0
    assert tbl.selection_capacity(s, p) == 3277
    assert tbl.selection_capacity(s, tbl.make_params(3277, 1)) == 3 * 3277
    assert tbl.selection_capacity(_shape(ctx_cap=1000), tbl.make_params(600, 2)) == 1000
    # the sink and the local window add their sizes
    assert tbl.selection_capacity(s, tbl.make_params(3277, 1, n_sink=4, n_local=64)) == \
        3 * 3277 + 68
    assert tbl.bitmap_words(_shape(ctx_cap=1000)) == 32
    assert tbl.bitmap_words(_shape(ctx_cap=1024)) == 32
    assert tbl.workspace_bytes(_shape(head_dim=96), p) == 0
    assert tbl.workspace_bytes(_shape(n_q_heads=12), p) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), tbl.TB_EINVAL),
    (dict(n_kv_heads=5), tbl.TB_EINVAL),
    (dict(n_imp_heads=12), tbl.TB_EINVAL),
    (dict(dtype=7), tbl.TB_EUNSUPPORTED),
    (dict(head_dim=96), tbl.TB_EUNSUPPORTED),
    (dict(d_imp=24), tbl.TB_EUNSUPPORTED),
    (dict(n_q_heads=48, n_kv_heads=3, n_imp_heads=48), tbl.TB_EUNSUPPORTED),
    (dict(ctx_cap=1 << 20), tbl.TB_EUNSUPPORTED),
])
def test_bad_shapes_rejected_before_launch(kw, code):
    L = tbl.lib()
    s = _shape(**kw)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    rc = L.tb_score(ctypes.byref(s), fake, fake, fake, fake, fake, 1 << 30, None)
    assert rc == code


def test_null_pointers_and_params_rejected():
    L = tbl.lib()
    s = _shape()
    p = tbl.make_params(100, 1)
    fake = ctypes.c_void_p(1 << 20)
    assert L.tb_score(ctypes.byref(s), None, fake, fake, fake, fake, 1 << 30, None) == tbl.TB_EINVAL
    assert L.tb_select(ctypes.byref(s), ctypes.byref(tbl.make_params(0, 0)), fake, fake, fake,
                       fake, None, None, fake, 1 << 30, None) == tbl.TB_EINVAL
    assert L.tb_select(ctypes.byref(s), ctypes.byref(tbl.make_params(5, -1)), fake, fake, fake,
                       fake, None, None, fake, 1 << 30, None) == tbl.TB_EINVAL
    assert L.tb_select(ctypes.byref(s), ctypes.byref(tbl.make_params(5, 1, n_sink=-1)), fake,
                       fake, fake, fake, None, None, fake, 1 << 30, None) == tbl.TB_EINVAL
    assert L.tb_select(ctypes.byref(s), ctypes.byref(tbl.make_params(5, 1, n_local=-3)), fake,
                       fake, fake, fake, None, None, fake, 1 << 30, None) == tbl.TB_EINVAL
    assert L.tb_project_keys(ctypes.byref(s), fake, fake, fake, -1, fake, None) == tbl.TB_EINVAL
    assert L.tb_project_keys(ctypes.byref(s), fake, fake, None, 4, fake, None) == tbl.TB_EINVAL
    # n_tokens == 0 is a no-op that launches nothing
    assert L.tb_project_keys(ctypes.byref(s), fake, fake, fake, 0, fake, None) == tbl.TB_OK
    # lists without a stride, and neither lists nor a bitmap
    assert L.tb_sparse_attn(ctypes.byref(s), fake, fake, fake, fake, 0, fake, None, None, fake,
                            ctypes.c_float(0.1), fake, fake, 1 << 30, None) == tbl.TB_EINVAL
    assert L.tb_sparse_attn(ctypes.byref(s), fake, fake, fake, None, 0, None, None, None, fake,
                            ctypes.c_float(0.1), fake, fake, 1 << 30, None) == tbl.TB_EINVAL
    assert L.tb_decode_step(ctypes.byref(s), ctypes.byref(p), None, fake, 1 << 30,
                            None) == tbl.TB_EINVAL


def test_workspace_checks():
    L = tbl.lib()
    s = _shape()
    p = tbl.make_params(100, 1)
    need = tbl.workspace_bytes(s, p)
    fake = ctypes.c_void_p(1 << 20)
    assert L.tb_select(ctypes.byref(s), ctypes.byref(p), fake, fake, fake, fake, None, None, fake,
                       need - 1, None) == tbl.TB_EWORKSPACE
    misaligned = ctypes.c_void_p((1 << 20) + 8)
    assert L.tb_select(ctypes.byref(s), ctypes.byref(p), fake, fake, fake, fake, None, None,
                       misaligned, need, None) == tbl.TB_EINVAL
    # the selection must go somewhere: a list, a bitmap or both
    assert L.tb_select(ctypes.byref(s), ctypes.byref(p), fake, fake, None, fake, None, None,
                       fake, need, None) == tbl.TB_EINVAL
    # scores are read in 16-byte pieces
    assert L.tb_select(ctypes.byref(s), ctypes.byref(p), ctypes.c_void_p((1 << 20) + 4), fake,
                       fake, fake, None, None, fake, need, None) == tbl.TB_EINVAL


def test_dense_attn_argument_checks():
    L = tbl.lib()
    s = _shape()
    need = tbl.workspace_bytes(s, tbl.make_params(100, 1))
    fake = ctypes.c_void_p(1 << 20)
    misaligned = ctypes.c_void_p((1 << 20) + 2)
    scale = ctypes.c_float(0.1)
    assert L.tb_dense_attn(ctypes.byref(s), None, fake, fake, fake, scale, fake, fake, need,
                           None) == tbl.TB_EINVAL
    assert L.tb_dense_attn(ctypes.byref(s), fake, fake, fake, None, scale, fake, fake, need,
                           None) == tbl.TB_EINVAL
    assert L.tb_dense_attn(ctypes.byref(s), fake, misaligned, fake, fake, scale, fake, fake,
                           need, None) == tbl.TB_EINVAL
    assert L.tb_dense_attn(ctypes.byref(s), fake, fake, fake, fake, ctypes.c_float(float("nan")),
                           fake, fake, need, None) == tbl.TB_EINVAL
    assert L.tb_dense_attn(ctypes.byref(s), fake, fake, fake, fake, scale, fake, fake, need - 1,
                           None) == tbl.TB_EWORKSPACE
    bad = _shape(head_dim=96)
    assert L.tb_dense_attn(ctypes.byref(bad), fake, fake, fake, fake, scale, fake, fake, need,
                           None) == tbl.TB_EUNSUPPORTED


def test_predict_queries_argument_checks():
    L = tbl.lib()
    mk = tbl.make_mlp_shape
    good = mk(16, 4096, 1024, 4, 32, 32, tbl.TB_BF16, tbl.TB_ACT_SILU)
    need = tbl.mlp_workspace_bytes(good)
    assert need > 0
    fake = ctypes.c_void_p(1 << 20)
    call = lambda sh, h=fake, w1=fake, w2=fake, q=fake, ws=fake, nb=need: L.tb_predict_queries(  # noqa: E731
        ctypes.byref(sh), h, w1, w2, q, ws, nb, None)
    assert call(good, h=None) == tbl.TB_EINVAL
    assert call(good, w2=ctypes.c_void_p((1 << 20) + 8)) == tbl.TB_EINVAL
    assert call(good, nb=need - 1) == tbl.TB_EWORKSPACE
    assert call(good, ws=ctypes.c_void_p((1 << 20) + 64)) == tbl.TB_EINVAL
    assert call(mk(0, 4096, 1024, 4, 32, 32, tbl.TB_BF16)) == tbl.TB_EINVAL
    assert call(mk(65, 4096, 1024, 4, 32, 32, tbl.TB_BF16)) == tbl.TB_EUNSUPPORTED
    assert call(mk(16, 4000, 1024, 4, 32, 32, tbl.TB_BF16)) == tbl.TB_EUNSUPPORTED
    assert call(mk(16, 4096, 1000, 4, 32, 32, tbl.TB_BF16)) == tbl.TB_EUNSUPPORTED
    assert call(mk(16, 4096, 1024, 1, 3, 5, tbl.TB_BF16)) == tbl.TB_EUNSUPPORTED
    assert call(mk(16, 4096, 1024, 4, 32, 32, tbl.TB_BF16, 7)) == tbl.TB_EUNSUPPORTED
    assert call(mk(16, 4096, 1024, 4, 32, 32, 9)) == tbl.TB_EUNSUPPORTED
    assert tbl.mlp_workspace_bytes(mk(65, 4096, 1024, 4, 32, 32, tbl.TB_BF16)) == 0


def test_decode_step_argument_checks():
    L = tbl.lib()
    s = _shape()
    p = tbl.make_params(100, 1)
    need = tbl.workspace_bytes(s, p)
    fake = 1 << 20
    a = tbl.StepArgs()
    for f in ("q", "w", "k_cache", "v_cache", "kp_cache", "ctx_len", "sel_idx", "sel_count",
              "sel_bits", "keep_from", "out", "q_imp"):
        setattr(a, f, fake)
    a.n_new = 1          # new rows announced but not given
    a.refresh = 1
    a.softmax_scale = 0.1
    assert L.tb_decode_step(ctypes.byref(s), ctypes.byref(p), ctypes.byref(a),
                            ctypes.c_void_p(fake), need, None) == tbl.TB_EINVAL
    a.n_new = 0
    a.q_imp = None       # a refresh step needs importance queries
    assert L.tb_decode_step(ctypes.byref(s), ctypes.byref(p), ctypes.byref(a),
                            ctypes.c_void_p(fake), need, None) == tbl.TB_EINVAL
    a.q_imp = fake
    a.sel_bits = None    # the fused step keeps its selection as a bitmap
    assert L.tb_decode_step(ctypes.byref(s), ctypes.byref(p), ctypes.byref(a),
                            ctypes.c_void_p(fake), need, None) == tbl.TB_EINVAL
    a.sel_bits = fake
    a.softmax_scale = float("nan")
    assert L.tb_decode_step(ctypes.byref(s), ctypes.byref(p), ctypes.byref(a),
                            ctypes.c_void_p(fake), need, None) == tbl.TB_EINVAL


def test_noalloc_step_rejects_a_shape_beyond_its_scratch_on_the_host():
    # the size check precedes every HIP call: no GPU needed
    shape = _shape(batch=64)
    params = tbl.make_params(3277, 0)
    assert tbl.workspace_bytes(shape, params) > tbl.NOALLOC_SCRATCH_BYTES
    args = tbl.StepArgs()
    for f in ("q", "q_imp", "w", "k_cache", "v_cache", "kp_cache", "out", "ctx_len",
              "sel_count", "sel_bits", "keep_from"):
        setattr(args, f, 256)
    args.softmax_scale = 0.1
    args.refresh = 1
    rc = tbl.lib().tb_decode_step_noalloc(ctypes.byref(shape), ctypes.byref(params),
                                          ctypes.byref(args), None)
    assert rc == tbl.TB_EWORKSPACE
    # and the shape checks come first
    bad = _shape(head_dim=96)
    assert tbl.lib().tb_decode_step_noalloc(ctypes.byref(bad), ctypes.byref(params),
                                            ctypes.byref(args), None) == tbl.TB_EUNSUPPORTED


def test_check_mode_switch_and_flag_argument():
    # the switch is host state; a NULL destination is rejected before any HIP call
    was = tbl.check_enabled()
    try:
        tbl.set_check(True)
        assert tbl.check_enabled()
        tbl.set_check(False)
        assert not tbl.check_enabled()
    finally:
        tbl.set_check(was)
    assert tbl.lib().tb_check_flags(None, 0) == tbl.TB_EINVAL


@pytest.mark.parametrize("value,on", [("1", True), ("yes", True), ("0", False), ("", False)])
def test_check_mode_from_the_environment(value, on):
    code = ("from query_aware_kv_amd import tokenbutler as t; "
            "print(int(t.check_enabled()))")
    env = dict(os.environ, TB_CHECK=value)
    out = subprocess.check_output(["python3", "-c", code], cwd=ROOT, env=env).decode().strip()
    assert out == str(int(on))
