"""Thin Python binding of libtokenbutler.so (ctypes).

Argument marshalling only: every function checks that tensors are contiguous
device tensors, passes raw pointers and sizes to the C ABI declared in
``include/tokenbutler.h`` together with torch's current HIP stream, and turns
a negative return code into :class:`TokenButlerError`.  All work runs in the
library's HIP kernels; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtokenbutler.so")

TB_OK, TB_EINVAL, TB_EUNSUPPORTED, TB_EWORKSPACE, TB_EHIP = 0, -1, -2, -3, -4
TB_F32, TB_BF16 = 0, 1

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class Shape(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
                ("n_imp_heads", _i32), ("head_dim", _i32), ("d_imp", _i32),
                ("ctx_cap", _i32), ("dtype", _i32)]


class MlpShape(ctypes.Structure):
    _fields_ = [("tokens", _i32), ("hidden", _i32), ("inner", _i32), ("n_slots", _i32),
                ("n_imp_heads", _i32), ("d_imp", _i32), ("dtype", _i32), ("act", _i32)]


TB_ACT_RELU, TB_ACT_SILU = 0, 1


class SelectParams(ctypes.Structure):
    _fields_ = [("budget", _i32), ("radius", _i32), ("n_sink", _i32), ("n_local", _i32)]


class StepArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("q_imp", _vp), ("k_new", _vp), ("v_new", _vp),
                ("n_new", _i32), ("refresh", _i32), ("w", _vp), ("k_cache", _vp),
                ("v_cache", _vp), ("kp_cache", _vp), ("ctx_len", _vp),
                ("softmax_scale", ctypes.c_float), ("sel_idx", _vp), ("sel_count", _vp),
                ("sel_bits", _vp), ("keep_from", _vp), ("out", _vp)]


class TokenButlerError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m query_aware_kv_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.tb_version.restype = ctypes.c_int
        L.tb_strerror.restype = ctypes.c_char_p
        L.tb_strerror.argtypes = [ctypes.c_int]
        L.tb_workspace_bytes.restype = ctypes.c_size_t
        L.tb_workspace_bytes.argtypes = [P(Shape), P(SelectParams)]
        L.tb_selection_capacity.restype = _i32
        L.tb_selection_capacity.argtypes = [P(Shape), P(SelectParams)]
        L.tb_bitmap_words.restype = _i32
        L.tb_bitmap_words.argtypes = [P(Shape)]
        L.tb_project_keys.argtypes = [P(Shape), _vp, _vp, _vp, _i32, _vp, _vp]
        L.tb_score.argtypes = [P(Shape), _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.tb_select.argtypes = [P(Shape), P(SelectParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                ctypes.c_size_t, _vp]
        L.tb_sparse_attn.argtypes = [P(Shape), _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                     ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]
        L.tb_dense_attn.argtypes = [P(Shape), _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp,
                                    ctypes.c_size_t, _vp]
        L.tb_decode_step.argtypes = [P(Shape), P(SelectParams), P(StepArgs), _vp,
                                     ctypes.c_size_t, _vp]
        L.tb_decode_step_noalloc.argtypes = [P(Shape), P(SelectParams), P(StepArgs), _vp]
        L.tb_mlp_workspace_bytes.argtypes = [P(MlpShape)]
        L.tb_mlp_workspace_bytes.restype = ctypes.c_size_t
        L.tb_predict_queries.argtypes = [P(MlpShape), _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                         _vp]
        L.tb_set_check.argtypes = [ctypes.c_int]
        L.tb_set_check.restype = None
        L.tb_check_enabled.restype = ctypes.c_int
        L.tb_check_flags.argtypes = [P(ctypes.c_uint32), ctypes.c_int]
        L.tb_check_flags.restype = ctypes.c_int
        for fn in ("tb_project_keys", "tb_score", "tb_select", "tb_sparse_attn",
                   "tb_dense_attn", "tb_decode_step", "tb_decode_step_noalloc",
                   "tb_predict_queries"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().tb_strerror(code).decode()


def _check(fn: str, rc: int) -> None:
    if rc != TB_OK:
        raise TokenButlerError(fn, rc, strerror(rc))


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtokenbutler must be contiguous")
    return _vp(t.data_ptr())


_hip = None


def _cache_ptr(t: torch.Tensor | None):
    """Pointer of a K or V cache for the kernels.  A cache may live in device
    memory or, offloaded, in pinned host memory that the GPU reads over the
    host link; for the latter the device-side address is taken from
    hipHostGetDevicePointer, which also proves that the GPU can reach it."""
    global _hip
    if t is None or t.is_cuda:
        return _ptr(t)
    if not t.is_pinned():
        raise ValueError("an offloaded cache must be pinned host memory (pin_memory=True)")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtokenbutler must be contiguous")
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
    dev = _vp()
    rc = _hip.hipHostGetDevicePointer(ctypes.byref(dev), _vp(t.data_ptr()), 0)
    if rc != 0 or not dev.value:
        raise RuntimeError(f"pinned cache is not mapped for the GPU (hip error {rc})")
    return dev


def _expect(name: str, t: torch.Tensor | None, numel: int, dtype=None,
            host_ok: bool = False) -> None:
    """Host-side size check of a tensor against the shape it must have
    (host_ok: a pinned host tensor is accepted too, for offloaded caches)."""
    if t is None:
        return
    if not t.is_cuda and not (host_ok and t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor"
                         + (" or pinned host memory" if host_ok else ""))
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")


def _elt(shape: Shape):
    return torch.float32 if shape.dtype == TB_F32 else torch.bfloat16


def _cache_numel(s: Shape, width: int) -> int:
    return s.batch * s.n_kv_heads * s.ctx_cap * width


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return _vp(s.cuda_stream)


def make_shape(batch, n_q_heads, n_kv_heads, n_imp_heads, head_dim, d_imp, ctx_cap,
               dtype) -> Shape:
    code = {torch.float32: TB_F32, torch.bfloat16: TB_BF16}.get(dtype, dtype)
    return Shape(batch, n_q_heads, n_kv_heads, n_imp_heads, head_dim, d_imp, ctx_cap, code)


def make_params(budget: int, radius: int, n_sink: int = 0, n_local: int = 0) -> SelectParams:
    return SelectParams(budget, radius, n_sink, n_local)


def version() -> int:
    return lib().tb_version()


def workspace_bytes(shape: Shape, params: SelectParams | None = None) -> int:
    return int(lib().tb_workspace_bytes(ctypes.byref(shape),
                                        ctypes.byref(params) if params is not None else None))


def selection_capacity(shape: Shape, params: SelectParams) -> int:
    return int(lib().tb_selection_capacity(ctypes.byref(shape), ctypes.byref(params)))


def bitmap_words(shape: Shape) -> int:
    return int(lib().tb_bitmap_words(ctypes.byref(shape)))


def alloc_workspace(shape: Shape, params: SelectParams | None = None, device="cuda"):
    """A zero-filled workspace of the size the library asks for."""
    n = workspace_bytes(shape, params)
    if n == 0:
        raise ValueError("invalid shape or params")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def project_keys(shape, k_cache, w, pos0, n_tokens, kp_cache, stream=None):
    e = _elt(shape)
    _expect("k_cache", k_cache, _cache_numel(shape, shape.head_dim), e, host_ok=True)
    _expect("kp_cache", kp_cache, _cache_numel(shape, shape.d_imp), e)
    _expect("w", w, shape.head_dim * shape.d_imp, e)
    _expect("pos0", pos0, shape.batch, torch.int32)
    _check("tb_project_keys", lib().tb_project_keys(
        ctypes.byref(shape), _cache_ptr(k_cache), _ptr(w), _ptr(pos0), int(n_tokens),
        _ptr(kp_cache), _stream(stream)))


def score(shape, q_imp, kp_cache, ctx_len, scores, ws, stream=None):
    e = _elt(shape)
    _expect("q_imp", q_imp, shape.batch * shape.n_imp_heads * shape.d_imp, e)
    _expect("kp_cache", kp_cache, _cache_numel(shape, shape.d_imp), e)
    _expect("ctx_len", ctx_len, shape.batch, torch.int32)
    _expect("scores", scores, shape.batch * shape.n_imp_heads * shape.ctx_cap, torch.float32)
    _check("tb_score", lib().tb_score(
        ctypes.byref(shape), _ptr(q_imp), _ptr(kp_cache), _ptr(ctx_len), _ptr(scores),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def select(shape, params, scores, ctx_len, sel_idx, sel_count, ws, topb_idx=None,
           sel_bits=None, stream=None):
    rows = shape.batch * shape.n_imp_heads
    _expect("scores", scores, rows * shape.ctx_cap, torch.float32)
    _expect("ctx_len", ctx_len, shape.batch, torch.int32)
    _expect("sel_idx", sel_idx, rows * selection_capacity(shape, params), torch.int32)
    _expect("sel_count", sel_count, rows, torch.int32)
    _expect("topb_idx", topb_idx, rows * params.budget, torch.int32)
    _expect("sel_bits", sel_bits, rows * bitmap_words(shape), torch.int32)
    _check("tb_select", lib().tb_select(
        ctypes.byref(shape), ctypes.byref(params), _ptr(scores), _ptr(ctx_len), _ptr(sel_idx),
        _ptr(sel_count), _ptr(topb_idx), _ptr(sel_bits), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


def sparse_attn(shape, q, k_cache, v_cache, sel_idx, sel_stride, sel_count, keep_from, ctx_len,
                softmax_scale, out, ws, sel_bits=None, stream=None):
    """Attention over the selected rows; membership from sel_bits when given,
    else from the sel_idx / sel_count lists."""
    e = _elt(shape)
    rows = shape.batch * shape.n_imp_heads
    qn = shape.batch * shape.n_q_heads * shape.head_dim
    _expect("q", q, qn, e)
    _expect("out", out, qn, e)
    _expect("k_cache", k_cache, _cache_numel(shape, shape.head_dim), e, host_ok=True)
    _expect("v_cache", v_cache, _cache_numel(shape, shape.head_dim), e, host_ok=True)
    if sel_idx is not None:
        _expect("sel_idx", sel_idx, rows * int(sel_stride), torch.int32)
    _expect("sel_count", sel_count, rows, torch.int32)
    _expect("sel_bits", sel_bits, rows * bitmap_words(shape), torch.int32)
    _expect("keep_from", keep_from, shape.batch, torch.int32)
    _expect("ctx_len", ctx_len, shape.batch, torch.int32)
    _check("tb_sparse_attn", lib().tb_sparse_attn(
        ctypes.byref(shape), _ptr(q), _cache_ptr(k_cache), _cache_ptr(v_cache), _ptr(sel_idx),
        int(sel_stride), _ptr(sel_count), _ptr(sel_bits), _ptr(keep_from), _ptr(ctx_len),
        float(softmax_scale), _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(stream)))


def dense_attn(shape, q, k_cache, v_cache, ctx_len, softmax_scale, out, ws, stream=None):
    """Dense attention over every cached token [0, ctx_len)."""
    e = _elt(shape)
    qn = shape.batch * shape.n_q_heads * shape.head_dim
    _expect("q", q, qn, e)
    _expect("out", out, qn, e)
    _expect("k_cache", k_cache, _cache_numel(shape, shape.head_dim), e, host_ok=True)
    _expect("v_cache", v_cache, _cache_numel(shape, shape.head_dim), e, host_ok=True)
    _expect("ctx_len", ctx_len, shape.batch, torch.int32)
    _check("tb_dense_attn", lib().tb_dense_attn(
        ctypes.byref(shape), _ptr(q), _cache_ptr(k_cache), _cache_ptr(v_cache), _ptr(ctx_len),
        float(softmax_scale), _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(stream)))


def make_mlp_shape(tokens, hidden, inner, n_slots, n_imp_heads, d_imp, dtype,
                   act=TB_ACT_RELU) -> MlpShape:
    code = {torch.float32: TB_F32, torch.bfloat16: TB_BF16}.get(dtype, dtype)
    return MlpShape(tokens, hidden, inner, n_slots, n_imp_heads, d_imp, code, act)


def mlp_workspace_bytes(shape: MlpShape) -> int:
    return int(lib().tb_mlp_workspace_bytes(ctypes.byref(shape)))


def alloc_mlp_workspace(shape: MlpShape, device="cuda"):
    """A zero-filled workspace for tb_predict_queries."""
    n = mlp_workspace_bytes(shape)
    if n == 0:
        raise ValueError("invalid MLP shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def predict_queries(shape: MlpShape, h, w1, w2, q_imp, ws, stream=None):
    """Importance queries q_imp [G][M][Himp][d] from hidden states h [M][E]
    through the two-layer MLP w1 [F][E], w2 [G*Himp*d][F]."""
    e = torch.float32 if shape.dtype == TB_F32 else torch.bfloat16
    N = shape.n_slots * shape.n_imp_heads * shape.d_imp
    _expect("h", h, shape.tokens * shape.hidden, e)
    _expect("w1", w1, shape.inner * shape.hidden, e)
    _expect("w2", w2, N * shape.inner, e)
    _expect("q_imp", q_imp, shape.n_slots * shape.tokens * shape.n_imp_heads * shape.d_imp, e)
    _check("tb_predict_queries", lib().tb_predict_queries(
        ctypes.byref(shape), _ptr(h), _ptr(w1), _ptr(w2), _ptr(q_imp), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


def step_args(shape, params, *, q, q_imp, k_new, v_new, refresh, w, k_cache, v_cache, kp_cache,
              ctx_len, softmax_scale, sel_idx, sel_count, sel_bits, keep_from, out) -> StepArgs:
    """Pointers of one fused step, after checking every tensor's size.  The
    tensors must stay alive until the step has run."""
    n_new = 0 if k_new is None else int(k_new.shape[2])
    e = _elt(shape)
    rows = shape.batch * shape.n_imp_heads
    qn = shape.batch * shape.n_q_heads * shape.head_dim
    _expect("q", q, qn, e)
    _expect("out", out, qn, e)
    _expect("q_imp", q_imp, rows * shape.d_imp, e)
    _expect("k_new", k_new, shape.batch * shape.n_kv_heads * n_new * shape.head_dim, e)
    _expect("v_new", v_new, shape.batch * shape.n_kv_heads * n_new * shape.head_dim, e)
    _expect("w", w, shape.head_dim * shape.d_imp, e)
    _expect("k_cache", k_cache, _cache_numel(shape, shape.head_dim), e, host_ok=True)
    _expect("v_cache", v_cache, _cache_numel(shape, shape.head_dim), e, host_ok=True)
    _expect("kp_cache", kp_cache, _cache_numel(shape, shape.d_imp), e)
    _expect("ctx_len", ctx_len, shape.batch, torch.int32)
    _expect("sel_idx", sel_idx, rows * selection_capacity(shape, params), torch.int32)
    _expect("sel_count", sel_count, rows, torch.int32)
    _expect("sel_bits", sel_bits, rows * bitmap_words(shape), torch.int32)
    _expect("keep_from", keep_from, shape.batch, torch.int32)
    a = StepArgs()
    a.q, a.q_imp, a.k_new, a.v_new = _ptr(q), _ptr(q_imp), _ptr(k_new), _ptr(v_new)
    a.n_new, a.refresh = n_new, int(bool(refresh))
    a.w, a.k_cache, a.v_cache = _ptr(w), _cache_ptr(k_cache), _cache_ptr(v_cache)
    a.kp_cache = _ptr(kp_cache)
    a.ctx_len, a.softmax_scale = _ptr(ctx_len), float(softmax_scale)
    a.sel_idx, a.sel_count, a.sel_bits = _ptr(sel_idx), _ptr(sel_count), _ptr(sel_bits)
    a.keep_from, a.out = _ptr(keep_from), _ptr(out)
    return a


def decode_step(shape, params, args: StepArgs, ws, stream=None):
    _check("tb_decode_step", lib().tb_decode_step(
        ctypes.byref(shape), ctypes.byref(params), ctypes.byref(args), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # TB_NOALLOC_SCRATCH_BYTES


def decode_step_noalloc(shape, params, args: StepArgs, stream=None):
    """tb_decode_step on the library's fixed device scratch (no workspace)."""
    _check("tb_decode_step_noalloc", lib().tb_decode_step_noalloc(
        ctypes.byref(shape), ctypes.byref(params), ctypes.byref(args), _stream(stream)))


# debug mode (TB_CHECK): bits of the device's check word
CHECK_NONFINITE_INPUT = 1
CHECK_NONFINITE_CACHE = 2
CHECK_CTX_RANGE = 4
CHECK_KEEP_RANGE = 8
CHECK_SEL_RANGE = 16
CHECK_NONFINITE_SCORES = 32


def set_check(on: bool) -> None:
    """Turn the debug-mode input checks on or off (overrides TB_CHECK)."""
    lib().tb_set_check(int(bool(on)))


def check_enabled() -> bool:
    return bool(lib().tb_check_enabled())


def check_flags(clear: bool = True) -> int:
    """Wait for the device and return its check word (cleared if asked)."""
    v = ctypes.c_uint32(0)
    _check("tb_check_flags", lib().tb_check_flags(ctypes.byref(v), int(bool(clear))))
    return int(v.value)
