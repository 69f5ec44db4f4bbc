"""Python access to the fp64 CPU oracle (``tb_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle is the plain, single-threaded reference
that the GPU library is checked against.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package; the GPU product path never does, and it shares no code with it.

Every function takes numpy arrays of float64 holding the exact values the GPU
reads (bf16/fp32 values upcast without rounding) and returns numpy arrays.
The arithmetic lives in ``tb_oracle.c``; this module only marshals arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tb_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile ``tb_oracle.c`` into ``liboracle.so`` with gcc (CPU only)."""
    stale = not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.orc_round.argtypes = [P, P, i64, ctypes.c_int]
        lib.orc_project.argtypes = [P, P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        lib.orc_score.argtypes = [P, P] + [ctypes.c_int] * 5 + [P, P]
        lib.orc_topb.argtypes = [P, i32, i32, P]
        lib.orc_topb.restype = i32
        lib.orc_topb64.argtypes = [P, i32, i32, P]
        lib.orc_topb64.restype = i32
        lib.orc_expand.argtypes = [P, i32, i32, i32, P]
        lib.orc_expand.restype = i32
        lib.orc_mlp.argtypes = [P, P, P] + [ctypes.c_int] * 8 + [P]
        lib.orc_mlp.restype = None
        lib.orc_buffers.argtypes = [i32, i32, i32, P, P]
        lib.orc_buffers.restype = None
        lib.orc_select.argtypes = [P, i32, i32, i32, i32, i32, P, P, P]
        lib.orc_select.restype = i32
        lib.orc_select64.argtypes = [P, i32, i32, i32, i32, i32, P, P, P]
        lib.orc_select64.restype = i32
        lib.orc_attend.argtypes = [P, P, P, ctypes.c_int, P, i32, dbl, P, P]
        lib.orc_decode_step.argtypes = (
            [ctypes.c_int] * 7 + [P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, P, P,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, dbl,
                                  P, P, P, ctypes.c_int, P])
        lib.orc_decode_step.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def round_to(x, dtype: int) -> np.ndarray:
    """Round every element to the storage dtype (F32 or BF16), ties to even."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().orc_round(_p(x), _p(y), x.size, dtype)
    return y


def project(K, W, dtype: int) -> np.ndarray:
    """Kp[..., j] = round(sum_i K[..., i] W[i, j]) for K [..., D], W [D, d]."""
    K = _f64(K)
    W = _f64(W)
    D, d = W.shape
    assert K.shape[-1] == D
    rows = K.size // D
    out = np.empty(K.shape[:-1] + (d,), dtype=np.float64)
    _load().orc_project(_p(K), _p(W), rows, D, d, dtype, _p(out))
    return out


def score(q_imp, Kp, n: int | None = None):
    """Scores of one sequence.  q_imp [Himp, d], Kp [Hkv, cap, d].

    Returns (s64 [Himp, n], s32 [Himp, n]) over tokens t < n (default: cap):
    the fp64 dot products, and the fp32 fused multiply-add chains (ascending
    coordinate order) that decide the selection."""
    q_imp = _f64(q_imp)
    Kp = _f64(Kp)
    Himp, d = q_imp.shape
    Hkv, cap, d2 = Kp.shape
    assert d == d2
    n = cap if n is None else int(n)
    s64 = np.empty((Himp, n), dtype=np.float64)
    s32 = np.empty((Himp, n), dtype=np.float32)
    _load().orc_score(_p(q_imp), _p(Kp), Himp, Hkv, cap, d, n, _p(s64), _p(s32))
    return s64, s32


def topb(s32, B: int) -> np.ndarray:
    """Ascending indices of the top-B entries of s32 (score desc, index asc)."""
    s = np.ascontiguousarray(s32, dtype=np.float32)
    n = s.size
    T = np.empty(max(n, 1), dtype=np.int32)
    c = _load().orc_topb(_p(s), n, int(B), _p(T))
    return T[:c].copy()


def topb64(s64, B: int) -> np.ndarray:
    """Ascending indices of the top-B entries of fp64 scores (score desc,
    index asc): the ranking of the exact dot products."""
    s = _f64(s64)
    n = s.size
    T = np.empty(max(n, 1), dtype=np.int32)
    c = _load().orc_topb64(_p(s), n, int(B), _p(T))
    return T[:c].copy()


def expand(T, n: int, r: int) -> np.ndarray:
    """Sorted union of [t-r, t+r] clipped to [0, n) over t in T."""
    T = _i32(T)
    S = np.empty(max(n, 1), dtype=np.int32)
    c = _load().orc_expand(_p(T), T.size, int(n), int(r), _p(S))
    return S[:c].copy()


def attend(q, K, V, S, scale: float, return_weights: bool = False):
    """Softmax attention of q [D] over rows S of K, V [*, D] (fp64)."""
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    S = _i32(S)
    D = q.size
    out = np.empty(D, dtype=np.float64)
    w = np.empty(max(S.size, 1), dtype=np.float64)
    _load().orc_attend(_p(q), _p(K), _p(V), D, _p(S), S.size, float(scale), _p(out), _p(w))
    if return_weights:
        return out, w[:S.size].copy()
    return out


ACT_RELU = 0
ACT_SILU = 1


def mlp(h, W1, W2, G: int, Himp: int, d: int, act: int, dtype: int) -> np.ndarray:
    """Importance queries from hidden states h [M, E] through the two-layer
    MLP (W1 [F, E], W2 [G*Himp*d, F], output-major, no biases); returns
    q_imp [G, M, Himp, d] rounded to the dtype."""
    h, W1, W2 = _f64(h), _f64(W1), _f64(W2)
    M, E = h.shape
    F = W1.shape[0]
    assert W1.shape == (F, E) and W2.shape == (G * Himp * d, F)
    out = np.empty((G, M, Himp, d), dtype=np.float64)
    _load().orc_mlp(_p(h), _p(W1), _p(W2), M, E, F, G, Himp, d, int(act), int(dtype), _p(out))
    return out


def buffers(n: int, n_sink: int, n_local: int):
    """(lo, hi): the sink is [0, lo), the local window [hi, n), the middle
    region between them."""
    lo = ctypes.c_int32()
    hi = ctypes.c_int32()
    _load().orc_buffers(int(n), int(n_sink), int(n_local), ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def select(s32, B: int, r: int, n_sink: int = 0, n_local: int = 0):
    """(T, S) of one head over a context of s32.size tokens: T the top-B of
    the middle region, S = widen(T, r) united with the sink and local window."""
    s = np.ascontiguousarray(s32, dtype=np.float32)
    n = s.size
    T = np.empty(max(n, 1), dtype=np.int32)
    S = np.empty(max(n, 1), dtype=np.int32)
    nT = ctypes.c_int32()
    c = _load().orc_select(_p(s), n, int(B), int(r), int(n_sink), int(n_local), _p(T),
                           ctypes.byref(nT), _p(S))
    return T[:nT.value].copy(), S[:c].copy()


def select64(s64, B: int, r: int, n_sink: int = 0, n_local: int = 0):
    """As :func:`select`, ranking fp64 scores (the exact dot products)."""
    s = _f64(s64)
    n = s.size
    T = np.empty(max(n, 1), dtype=np.int32)
    S = np.empty(max(n, 1), dtype=np.int32)
    nT = ctypes.c_int32()
    c = _load().orc_select64(_p(s), n, int(B), int(r), int(n_sink), int(n_local), _p(T),
                             ctypes.byref(nT), _p(S))
    return T[:nT.value].copy(), S[:c].copy()


def cap_s(cap: int, B: int, r: int, n_sink: int = 0, n_local: int = 0) -> int:
    """Capacity of one head's stored selection: min(cap, (2r+1) B + n_sink + n_local)."""
    return min(cap, (2 * r + 1) * B + n_sink + n_local)


class SequenceState:
    """Caches and selection state of one sequence for :func:`decode_step`.

    K, V [Hkv, cap, D], Kp [Hkv, cap, d] as float64; sel [Himp, cap_S] int32,
    cnt [Himp] int32, keep_from [1] int32."""

    def __init__(self, K, V, Kp, Himp: int, B: int, r: int, n_sink: int = 0, n_local: int = 0):
        self.K = _f64(K).copy()
        self.V = _f64(V).copy()
        self.Kp = _f64(Kp).copy()
        Hkv, cap, _ = self.K.shape
        self.cap = cap
        self.B = int(B)
        self.r = int(r)
        self.n_sink = int(n_sink)
        self.n_local = int(n_local)
        self.cap_S = cap_s(cap, B, r, n_sink, n_local)
        self.sel = np.zeros((Himp, self.cap_S), dtype=np.int32)
        self.cnt = np.zeros(Himp, dtype=np.int32)
        self.keep_from = np.zeros(1, dtype=np.int32)


def decode_step(st: SequenceState, W, q, q_imp, ctx: int, dtype: int, refresh: bool,
                scale: float, k_new=None, v_new=None) -> np.ndarray:
    """One decode step of one sequence; returns out [Hq, D] (fp64).

    k_new / v_new [Hkv, n_new, D] are appended at [ctx - n_new, ctx)."""
    W = _f64(W)
    q = _f64(q)
    Hq, D = q.shape
    Hkv, cap, _ = st.K.shape
    d = W.shape[1]
    Himp = st.sel.shape[0]
    if k_new is None:
        n_new = 0
        kn = np.zeros(1)
        vn = np.zeros(1)
    else:
        kn = _f64(k_new)
        vn = _f64(v_new)
        n_new = kn.shape[1]
    qi = _f64(q_imp) if q_imp is not None else np.zeros((Himp, d))
    out = np.empty((Hq, D), dtype=np.float64)
    rc = _load().orc_decode_step(
        Hq, Hkv, Himp, D, d, cap, dtype, _p(st.K), _p(st.V), _p(st.Kp), _p(W),
        _p(kn), _p(vn), n_new, int(ctx), _p(q), _p(qi), int(bool(refresh)), st.B, st.r,
        st.n_sink, st.n_local, float(scale), _p(st.sel), _p(st.cnt), _p(st.keep_from), st.cap_S, _p(out))
    if rc != 0:
        raise RuntimeError("oracle decode_step: selection exceeds its capacity")
    return out

