"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to something it could get wrong: a library
routine it must agree with on a special case, a brute-force count on tiny
inputs, a closed form, an invariant, or a case worked by hand from the
definitions on the TokenButler pages (stored under tests/golden/).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# rounding to the storage dtype
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_on_fp32_values():
    # torch's fp32 -> bf16 conversion is round-to-nearest-even (a library routine)
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-38).astype(np.float32),
                        (rng.standard_normal(20000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_to(x.astype(np.float64), orc.BF16)
    np.testing.assert_array_equal(got, ref)


def _bf16_nearest_exact(x: float) -> float:
    """Brute force: nearest bf16 value to x by exact rational arithmetic
    (8 significant bits, spacing 2^-133 below 2^-126, ties to the even
    multiple of the spacing)."""
    if x == 0:
        return x
    ax = Fraction(abs(x))
    _, E = math.frexp(abs(x))          # |x| in [2^(E-1), 2^E)
    e = E - 1
    step = Fraction(2) ** (e - 7) if e >= -126 else Fraction(2) ** -133
    k = ax / step
    m = math.floor(k)
    frac = k - m
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return math.copysign(float(m * step), x)


def test_bf16_rounding_of_doubles_brute_force():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(3000), rng.standard_normal(500) * 1e-39])
    got = orc.round_to(xs, orc.BF16)
    for x, g in zip(xs.tolist(), got.tolist()):
        assert g == _bf16_nearest_exact(x), x


def test_bf16_rounding_ties_to_even():
    cases = {
        1.0 + 2.0 ** -8: 1.0,                    # halfway 1 .. 1+2^-7 -> even (1)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,    # halfway -> even (1+2^-6)
        1.0 + 2.0 ** -8 + 2.0 ** -40: 1.0 + 2.0 ** -7,  # just above halfway
        -(1.0 + 2.0 ** -8): -1.0,
        2.0 ** -134: 0.0,                        # half the smallest subnormal
        3 * 2.0 ** -134: 2.0 ** -132,            # 1.5 ulp -> even (2 ulp)
        2.0 ** 128: math.inf,
        float.fromhex("0x1.FFp127"): math.inf,
    }
    got = orc.round_to(np.array(list(cases.keys())), orc.BF16)
    assert got.tolist() == list(cases.values())


def test_f32_rounding_is_ieee_cast():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10000)
    np.testing.assert_array_equal(orc.round_to(x, orc.F32), x.astype(np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# key projection
# --------------------------------------------------------------------------

def test_projection_of_basis_rows_picks_rows_of_w():
    # K = e_i must give row i of W: catches a transposed W or swapped loop bounds.
    D, d = 12, 5
    rng = np.random.default_rng(3)
    W = orc.round_to(rng.standard_normal((D, d)), orc.BF16)
    Kp = orc.project(np.eye(D), W, orc.BF16)
    np.testing.assert_array_equal(Kp, W)


def test_projection_exact_on_small_integers():
    # small integers: every sum is exact, so the result equals the integer product
    D, d = 16, 7
    rng = np.random.default_rng(4)
    K = rng.integers(-8, 9, size=(5, 3, D)).astype(np.float64)
    W = rng.integers(-8, 9, size=(D, d)).astype(np.float64)
    ref = np.einsum("abi,ij->abj", K.astype(np.int64), W.astype(np.int64)).astype(np.float64)
    np.testing.assert_array_equal(orc.project(K, W, orc.F32), ref)


def test_projection_rounds_once_to_dtype():
    # the projection is the fp64 sum rounded once: with D = 2 the sum is exact in fp64
    K = np.array([[1.0, 2.0 ** -9]])
    W = np.array([[1.0], [1.0]])
    assert orc.project(K, W, orc.BF16)[0, 0] == 1.0                 # 1 + 2^-9 -> 1
    K = np.array([[1.0, 2.0 ** -8 + 2.0 ** -30]])
    assert orc.project(K, W, orc.BF16)[0, 0] == 1.0 + 2.0 ** -7     # above half -> up
    assert orc.project(K, W, orc.F32)[0, 0] == np.float32(1.0 + 2.0 ** -8 + 2.0 ** -30)


def test_projection_associativity():
    # q . (K W) == (W q) . K in exact arithmetic; the only difference here is
    # the single fp32 rounding of each projected element
    rng = np.random.default_rng(5)
    D, d = 64, 16
    K = rng.standard_normal((40, D)).astype(np.float32).astype(np.float64)
    W = (rng.standard_normal((D, d)) * 2 ** 7).round() / 2 ** 10
    q = rng.standard_normal(d)
    lhs = orc.project(K, W, orc.F32) @ q
    rhs = K @ (W @ q)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-6 * np.abs(K).sum(1).max() * np.abs(q).sum())


# --------------------------------------------------------------------------
# importance scores
# --------------------------------------------------------------------------

def test_score_basis_query_reads_one_coordinate():
    rng = np.random.default_rng(6)
    Hkv, cap, d = 2, 9, 4
    Kp = rng.standard_normal((Hkv, cap, d))
    for j in range(d):
        q_imp = np.zeros((2, d))
        q_imp[:, j] = 1.0
        s64, _ = orc.score(q_imp, Kp)
        np.testing.assert_array_equal(s64[0], Kp[0, :, j])
        np.testing.assert_array_equal(s64[1], Kp[1, :, j])


def test_score_head_to_group_mapping_is_contiguous_blocks():
    # 8 importance heads over 2 KV heads: heads 0-3 read group 0, heads 4-7 group 1
    Hkv, cap, d = 2, 5, 3
    Kp = np.zeros((Hkv, cap, d))
    Kp[0, :, 0] = 1.0
    Kp[1, :, 0] = 2.0
    q_imp = np.zeros((8, d))
    q_imp[:, 0] = 1.0
    s64, _ = orc.score(q_imp, Kp)
    assert s64[:, 0].tolist() == [1, 1, 1, 1, 2, 2, 2, 2]


def test_score_against_integer_matmul():
    rng = np.random.default_rng(7)
    Hkv, cap, d = 4, 33, 8
    Kp = rng.integers(-50, 51, size=(Hkv, cap, d)).astype(np.float64)
    q_imp = rng.integers(-50, 51, size=(8, d)).astype(np.float64)
    s64, s32 = orc.score(q_imp, Kp, n=30)
    for i in range(8):
        g = i // 2
        ref = (Kp[g, :30].astype(np.int64) @ q_imp[i].astype(np.int64)).astype(np.float64)
        np.testing.assert_array_equal(s64[i], ref)
        np.testing.assert_array_equal(s32[i].astype(np.float64), ref)  # small integers: exact


def _fma_chain_exact(q, k):
    """Brute force of an fp32 fused multiply-add chain: each step rounds the
    exact rational q_j * k_j + acc to the nearest fp32 (ties to even) -- done
    here through Fraction arithmetic and a correctly rounded conversion."""
    acc = Fraction(0)
    for qj, kj in zip(q, k):
        exact = Fraction(float(qj)) * Fraction(float(kj)) + acc
        acc = Fraction(float(np.float32(_round_fraction_to_f32(exact))))
    return float(acc)


def _round_fraction_to_f32(x: Fraction) -> float:
    # nearest fp32 to a rational, ties to even, by exact comparison of neighbours
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    ax = abs(x)
    f = float(ax)                     # correctly rounded to double
    c = np.float32(f)                 # candidate near the answer
    cands = {float(c), float(np.nextafter(c, np.float32(0))), float(np.nextafter(c, np.float32(np.inf)))}
    best = min(cands, key=lambda v: (abs(Fraction(v) - ax),
                                     int(np.float32(v).view(np.uint32)) & 1))
    return sign * best


def test_score_fp32_fma_chain_brute_force():
    # the selection score is the fp32 fma chain; checked against exact
    # rational arithmetic rounded at every step, on fp32 inputs where a
    # separate multiply and add would differ
    rng = np.random.default_rng(8)
    d = 16
    for trial in range(200):
        q = rng.standard_normal(d).astype(np.float32)
        k = rng.standard_normal((1, 1, d)).astype(np.float32)
        _, s32 = orc.score(q[None, :].astype(np.float64), k.astype(np.float64))
        assert float(s32[0, 0]) == _fma_chain_exact(q, k[0, 0]), trial


def test_score_fp32_chain_is_ordered():
    # ascending order matters: a large cancellation early keeps a small term
    q = np.array([[1.0, 1.0, 1.0]])
    kp = np.array([[[2.0 ** 30, -(2.0 ** 30), 1.0]]])
    _, s32 = orc.score(q, kp)
    assert s32[0, 0] == 1.0
    kp = np.array([[[2.0 ** 30, 1.0, -(2.0 ** 30)]]])   # 2^30 + 1 rounds to 2^30 in fp32
    _, s32 = orc.score(q, kp)
    assert s32[0, 0] == 0.0


# --------------------------------------------------------------------------
# top-B
# --------------------------------------------------------------------------

def _rank_count_topb(s: np.ndarray, B: int) -> list:
    # t is kept iff fewer than B tokens beat it: a larger score, or an equal
    # score at a lower index (brute force, O(n^2))
    n = s.size
    keep = []
    for t in range(n):
        beat = sum(1 for u in range(n) if s[u] > s[t] or (s[u] == s[t] and u < t))
        if beat < B:
            keep.append(t)
    return keep


@pytest.mark.parametrize("seed", range(40))
def test_topb_brute_force_rank_count(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 65))
    if seed % 3 == 0:
        s = rng.standard_normal(n).astype(np.float32)
    elif seed % 3 == 1:     # tie-heavy, with signed zeros
        s = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32), size=n)
    else:
        s = rng.integers(-3, 4, size=n).astype(np.float32)
    for B in {1, 2, n // 2 + 1, n, n + 3}:
        assert orc.topb(s, B).tolist() == _rank_count_topb(s, B)


@pytest.mark.parametrize("seed", range(30))
def test_topb64_brute_force_rank_count(seed):
    # the fp64 ranking (the selection of the exact dot products): the same
    # rank-count definition on doubles, with pairs that differ only below
    # float precision, so a ranking that went through fp32 would tie them
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 65))
    if seed % 3 == 0:
        s = rng.standard_normal(n)
    elif seed % 3 == 1:     # tie-heavy, with signed zeros
        s = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0]), size=n)
    else:                   # values 2^-40 apart: distinct in fp64, equal in fp32
        s = 1.0 + rng.integers(0, 4, size=n) * 2.0 ** -40
        assert np.unique(s.astype(np.float32)).size == 1
    for B in {1, 2, n // 2 + 1, n, n + 3}:
        assert orc.topb64(s, B).tolist() == _rank_count_topb(s, B)


def test_select64_brute_force_with_buffers():
    # select64 = rank-count top-B of the fp64 middle region, widened, united
    # with the sink and the local window (each step written out by hand here)
    rng = np.random.default_rng(760)
    for _ in range(25):
        n = int(rng.integers(1, 70))
        s = 1.0 + rng.integers(0, 5, size=n) * 2.0 ** -45 + rng.standard_normal(n) * (
            rng.random() < 0.5)
        B, r = int(rng.integers(1, 12)), int(rng.integers(0, 3))
        ns, nl = int(rng.integers(0, 6)), int(rng.integers(0, 6))
        lo = min(ns, n)
        hi = max(lo, n - nl)
        T = [lo + t for t in _rank_count_topb(s[lo:hi], B)]
        S = set(range(lo)) | set(range(hi, n))
        for t in T:
            S |= set(range(max(0, t - r), min(n, t + r + 1)))
        T_o, S_o = orc.select64(s, B, r, ns, nl)
        assert T_o.tolist() == T and S_o.tolist() == sorted(S)


def test_topb_golden_hand_cases():
    for c in _golden("topb_cases.json")["cases"]:
        s = np.array([float(v) for v in c["scores"]], dtype=np.float32)
        assert orc.topb(s, c["budget"]).tolist() == c["expected"], c


def test_topb_budget_covers_context():
    s = np.random.default_rng(9).standard_normal(17).astype(np.float32)
    assert orc.topb(s, 17).tolist() == list(range(17))
    assert orc.topb(s, 1000).tolist() == list(range(17))


def test_topb_single_is_first_argmax():
    s = np.array([1, 3, 0, 3, 2], dtype=np.float32)
    assert orc.topb(s, 1).tolist() == [int(np.argmax(s))] == [1]


# --------------------------------------------------------------------------
# neighbor expansion
# --------------------------------------------------------------------------

def test_expand_golden_hand_cases():
    for c in _golden("expand_cases.json")["cases"]:
        assert orc.expand(c["T"], c["n"], c["r"]).tolist() == c["expected"], c


# --------------------------------------------------------------------------
# importance-query producer (two-layer MLP)
# --------------------------------------------------------------------------

def _rne_fraction(x: Fraction, bits: int) -> Fraction:
    """x rounded to `bits` significant bits, ties to even (no range limits)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 2 ** (bits - 1)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * Fraction(fl) / 2 ** (bits - 1) * Fraction(2) ** e


def _mlp_exact(h, W1, W2, G, Himp, d, bits):
    # independent formulation: exact rational arithmetic, ReLU, rounding to
    # `bits` significant bits after the activation and at the output
    M, E = h.shape
    F = W1.shape[0]
    N = G * Himp * d
    u = [[_rne_fraction(max(Fraction(0), sum(Fraction(int(h[m, e])) * int(W1[f, e])
                                             for e in range(E))), bits)
          for f in range(F)] for m in range(M)]
    out = np.zeros((G, M, Himp, d))
    for m in range(M):
        for n in range(N):
            y = _rne_fraction(sum(u[m][f] * int(W2[n, f]) for f in range(F)), bits)
            g, rest = divmod(n, Himp * d)
            i, j = divmod(rest, d)
            out[g, m, i, j] = float(y)
    return out


@pytest.mark.parametrize("dtype,bits,scale", [(orc.F32, 24, 3), (orc.BF16, 8, 3),
                                              (orc.BF16, 8, 100)])
def test_mlp_exact_integers(dtype, bits, scale):
    rng = np.random.default_rng(500 + scale)
    M, E, F, G, Himp, d = 3, 8, 6, 2, 2, 3
    h = rng.integers(-scale, scale + 1, size=(M, E)).astype(np.float64)
    W1 = rng.integers(-3, 4, size=(F, E)).astype(np.float64)
    W2 = rng.integers(-3, 4, size=(G * Himp * d, F)).astype(np.float64)
    got = orc.mlp(h, W1, W2, G, Himp, d, orc.ACT_RELU, dtype)
    np.testing.assert_array_equal(got, _mlp_exact(h, W1, W2, G, Himp, d, bits))
    if scale == 100:   # some hidden values need more than 8 bits: rounding matters
        pre = np.maximum(h @ W1.T, 0)
        assert any(_rne_fraction(Fraction(int(v)), 8) != int(v) for v in pre.ravel())


def test_mlp_activation_closed_forms():
    one = np.ones((1, 1))
    # SiLU(1) = 1 / (1 + e^-1), rounded once to fp32 (hidden), then times 1
    y = orc.mlp(one, one, one, 1, 1, 1, orc.ACT_SILU, orc.F32)
    assert y[0, 0, 0, 0] == float(np.float32(1.0 / (1.0 + math.exp(-1.0))))
    # SiLU(-2) = -2 / (1 + e^2)
    y = orc.mlp(one, -2 * one, one, 1, 1, 1, orc.ACT_SILU, orc.F32)
    assert y[0, 0, 0, 0] == float(np.float32(-2.0 / (1.0 + math.exp(2.0))))
    # ReLU clips a negative pre-activation to zero
    y = orc.mlp(one, -one, one, 1, 1, 1, orc.ACT_RELU, orc.F32)
    assert y[0, 0, 0, 0] == 0.0


def test_mlp_slot_major_layout():
    # W2 row n copies hidden unit n, so q_imp[g][m][i][j] must equal the
    # hidden unit n = (g * Himp + i) * d + j of token m
    M, G, Himp, d = 2, 3, 2, 2
    N = G * Himp * d
    h = np.arange(1, M * N + 1, dtype=np.float64).reshape(M, N)
    W1 = np.eye(N)
    W2 = np.eye(N)
    q = orc.mlp(h, W1, W2, G, Himp, d, orc.ACT_RELU, orc.F32)
    for g in range(G):
        for m in range(M):
            for i in range(Himp):
                for j in range(d):
                    assert q[g, m, i, j] == h[m, (g * Himp + i) * d + j]


# --------------------------------------------------------------------------
# sink, local window and important buffer
# --------------------------------------------------------------------------

def test_select_buffers_golden_hand_cases():
    for c in _golden("select_buffers_cases.json")["cases"]:
        s = np.array(c["scores"], dtype=np.float32)
        T, S = orc.select(s, c["budget"], c["radius"], c["n_sink"], c["n_local"])
        assert T.tolist() == c["T"], c
        assert S.tolist() == c["expected"], c


def _select_brute(s, B, r, n_sink, n_local):
    # independent formulation: membership tests position by position
    n = s.size
    lo = min(n_sink, n)
    hi = max(lo, n - n_local)
    T = [i for i in range(lo, hi)
         if sum(1 for j in range(lo, hi) if s[j] > s[i] or (s[j] == s[i] and j < i)) < B]
    S = [t for t in range(n)
         if t < lo or t >= hi or any(abs(t - i) <= r for i in T)]
    return T, S


@pytest.mark.parametrize("seed", range(24))
def test_select_buffers_brute_force(seed):
    rng = np.random.default_rng(900 + seed)
    n = int(rng.integers(1, 40))
    if seed % 3 == 0:
        s = rng.integers(-2, 3, size=n).astype(np.float32)     # heavy ties
    elif seed % 3 == 1:
        s = rng.choice(np.array([-0.0, 0.0, 1.0], np.float32), size=n)
    else:
        s = rng.standard_normal(n).astype(np.float32)
    for _ in range(4):
        B = int(rng.integers(1, n + 3))
        r = int(rng.integers(0, 4))
        ns, nl = int(rng.integers(0, n + 2)), int(rng.integers(0, n + 2))
        T, S = orc.select(s, B, r, ns, nl)
        Tb, Sb = _select_brute(s, B, r, ns, nl)
        assert T.tolist() == Tb and S.tolist() == Sb, (n, B, r, ns, nl)
        assert len(S) <= orc.cap_s(n, B, r, ns, nl)


def test_select_without_buffers_is_topb_then_expand():
    s = np.random.default_rng(3).standard_normal(50).astype(np.float32)
    for B, r in [(1, 0), (7, 2), (60, 1)]:
        T, S = orc.select(s, B, r)
        assert T.tolist() == orc.topb(s, B).tolist()
        assert S.tolist() == orc.expand(orc.topb(s, B), 50, r).tolist()


def test_buffers_bounds():
    assert orc.buffers(10, 2, 3) == (2, 7)
    assert orc.buffers(10, 0, 0) == (0, 10)
    assert orc.buffers(5, 7, 0) == (5, 5)
    assert orc.buffers(5, 3, 4) == (3, 3)
    assert orc.buffers(0, 3, 4) == (0, 0)


def _expand_by_convolution(T, n, r):
    # independent formulation: dilate the indicator with a box filter
    ind = np.zeros(n)
    ind[np.asarray(T, dtype=np.int64)] = 1
    dil = np.convolve(ind, np.ones(2 * r + 1), mode="full")[r:r + n] > 0
    return np.nonzero(dil)[0].tolist()


@pytest.mark.parametrize("seed", range(20))
def test_expand_properties(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 80))
    T = np.sort(rng.choice(n, size=int(rng.integers(0, n + 1)), replace=False))
    r1, r2 = int(rng.integers(0, 4)), int(rng.integers(0, 4))
    S = orc.expand(T, n, r1)
    assert S.tolist() == _expand_by_convolution(T, n, r1)
    assert orc.expand(T, n, 0).tolist() == T.tolist()
    assert len(S) <= min(n, (2 * r1 + 1) * len(T))
    assert orc.expand(S, n, r2).tolist() == orc.expand(T, n, r1 + r2).tolist()


# --------------------------------------------------------------------------
# attention over the selected rows
# --------------------------------------------------------------------------

def _dense_attention_scipy(q, K, V, scale):
    from scipy.special import softmax
    return softmax(scale * (K @ q)) @ V


@pytest.mark.parametrize("seed", range(5))
def test_attend_full_set_equals_dense_attention(seed):
    rng = np.random.default_rng(300 + seed)
    n, D = 50, 16
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    scale = 1 / math.sqrt(D)
    out = orc.attend(q, K, V, np.arange(n), scale)
    np.testing.assert_allclose(out, _dense_attention_scipy(q, K, V, scale), rtol=0, atol=1e-12)
    # and the selection path with budget >= context keeps every token
    s = rng.standard_normal(n).astype(np.float32)
    S = orc.expand(orc.topb(s, n), n, 0)
    np.testing.assert_array_equal(orc.attend(q, K, V, S, scale), out)


def test_attend_subset_equals_dense_on_subset():
    rng = np.random.default_rng(310)
    n, D = 40, 8
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    S = np.array([1, 5, 6, 20, 39])
    np.testing.assert_allclose(orc.attend(q, K, V, S, 0.3),
                               _dense_attention_scipy(q, K[S], V[S], 0.3), rtol=0, atol=1e-12)


def test_attend_closed_forms():
    rng = np.random.default_rng(320)
    n, D = 30, 8
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    # a single attended row gets weight exactly 1
    np.testing.assert_array_equal(orc.attend(q, K, V, [7], 0.5), V[7])
    # q = 0: uniform weights, the output is the mean of the attended rows
    S = np.array([0, 3, 4, 29])
    np.testing.assert_allclose(orc.attend(np.zeros(D), K, V, S, 0.5), V[S].mean(0), atol=1e-15)
    # weights sum to one
    _, w = orc.attend(q, K, V, np.arange(n), 0.5, return_weights=True)
    assert abs(w.sum() - 1) < 1e-12
    # empty attended set -> zero row
    np.testing.assert_array_equal(orc.attend(q, K, V, [], 0.5), np.zeros(D))


def test_attend_permutation_invariance():
    rng = np.random.default_rng(330)
    n, D = 25, 8
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    perm = rng.permutation(n)
    a = orc.attend(q, K, V, np.arange(n), 0.4)
    b = orc.attend(q, K[perm], V[perm], np.arange(n), 0.4)
    np.testing.assert_allclose(a, b, atol=1e-14)


def test_budget_one_selects_argmax_row():
    # B = 1, r = 0: the output is the V row of the first argmax, exactly
    rng = np.random.default_rng(340)
    n, D = 20, 4
    s = rng.standard_normal(n).astype(np.float32)
    V = rng.standard_normal((n, D))
    K = rng.standard_normal((n, D))
    S = orc.expand(orc.topb(s, 1), n, 0)
    np.testing.assert_array_equal(orc.attend(rng.standard_normal(D), K, V, S, 1.0),
                                  V[int(np.argmax(s))])


# --------------------------------------------------------------------------
# the decode step: prediction interval and always-kept new tokens
# --------------------------------------------------------------------------

def _one_hot_sequence(scores, D):
    """A 1-head sequence whose importance score at position t is scores[t]
    (K[t] = scores[t] e_0, W = e_0 e_0^T, q_imp = e_0) and whose V rows are
    one-hot, so that with q = 0 the output reveals the attended set."""
    n = len(scores)
    K = np.zeros((n, D))
    K[:, 0] = scores
    V = np.eye(n, D)
    W = np.zeros((D, 1))
    W[0, 0] = 1.0
    return K, V, W


@pytest.mark.parametrize("name", ["interval_case.json", "interval_buffers_case.json"])
def test_interval_golden_hand_case(name):
    g = _golden(name)
    scores = g["scores_by_position"]
    n_total = len(scores)
    D = 16
    K, V, W = _one_hot_sequence(scores, D)
    ctx0 = g["ctx0"]
    cap = n_total
    Kc = np.zeros((1, cap, D))
    Vc = np.zeros((1, cap, D))
    Kc[0, :ctx0] = K[:ctx0]
    Vc[0, :ctx0] = V[:ctx0]
    Kp = orc.project(Kc, W, orc.F32)
    st = orc.SequenceState(Kc, Vc, Kp, Himp=1, B=g["budget"], r=g["radius"],
                           n_sink=g.get("n_sink", 0), n_local=g.get("n_local", 0))
    for s, attended in enumerate(g["attended_by_step"]):
        ctx = ctx0 + s + 1
        refresh = s % g["interval"] == 0
        out = orc.decode_step(st, W, np.zeros((1, D)), np.ones((1, 1)), ctx, orc.F32,
                              refresh, 1.0, k_new=K[None, ctx - 1:ctx], v_new=V[None, ctx - 1:ctx])
        expect = np.zeros(D)
        expect[attended] = 1.0 / len(attended)
        np.testing.assert_allclose(out[0], expect, atol=1e-15)
        assert st.sel[0, :st.cnt[0]].tolist() == g["stored_by_step"][s]
        assert int(st.keep_from[0]) == g["keep_from_by_step"][s]


def test_refresh_with_several_new_rows_golden_hand_case():
    # steps that append three rows each: the refresh scores the new rows with
    # the rest, and keep_from = ctx - n_new keeps all three attended
    g = _golden("interval_multirow_case.json")
    scores = g["scores_by_position"]
    D = 16
    K, V, W = _one_hot_sequence(scores, D)
    ctx0, nn = g["ctx0"], g["n_new"]
    cap = len(scores)
    Kc = np.zeros((1, cap, D))
    Vc = np.zeros((1, cap, D))
    Kc[0, :ctx0] = K[:ctx0]
    Vc[0, :ctx0] = V[:ctx0]
    for r_key in ("radius_0", "radius_1"):
        case = g[r_key]
        st = orc.SequenceState(Kc, Vc, orc.project(Kc, W, orc.F32), Himp=1, B=g["budget"],
                               r=case["radius"])
        for s_, attended in enumerate(case["attended_by_step"]):
            ctx = ctx0 + (s_ + 1) * nn
            refresh = s_ % g["interval"] == 0
            out = orc.decode_step(st, W, np.zeros((1, D)), np.ones((1, 1)), ctx, orc.F32,
                                  refresh, 1.0, k_new=K[None, ctx - nn:ctx],
                                  v_new=V[None, ctx - nn:ctx])
            expect = np.zeros(D)
            expect[attended] = 1.0 / len(attended)
            np.testing.assert_allclose(out[0], expect, atol=1e-15)
            assert st.sel[0, :st.cnt[0]].tolist() == case["stored_by_step"][s_], (r_key, s_)
            assert int(st.keep_from[0]) == g["keep_from_by_step"][s_]
            # the appended rows and their projections are in the caches
            np.testing.assert_array_equal(st.K[0, ctx - nn:ctx], K[ctx - nn:ctx])
            np.testing.assert_array_equal(st.Kp[0, ctx - nn:ctx, 0], np.array(scores[ctx - nn:ctx]))


def test_interval_one_is_per_step_recompute():
    # P = 1: every step refreshes, the attended set is Expand(TopB) plus the new token
    rng = np.random.default_rng(400)
    D, ctx0, steps, B, r = 8, 20, 6, 3, 1
    n_total = ctx0 + steps
    scores = rng.standard_normal(n_total)
    K, V, W = _one_hot_sequence(scores, 32)
    Kc = np.zeros((1, n_total, 32))
    Vc = np.zeros((1, n_total, 32))
    Kc[0, :ctx0] = K[:ctx0]
    Vc[0, :ctx0] = V[:ctx0]
    st = orc.SequenceState(Kc, Vc, orc.project(Kc, W, orc.F32), Himp=1, B=B, r=r)
    for s in range(steps):
        ctx = ctx0 + s + 1
        out = orc.decode_step(st, W, np.zeros((1, 32)), np.ones((1, 1)), ctx, orc.F32, True,
                              1.0, k_new=K[None, ctx - 1:ctx], v_new=V[None, ctx - 1:ctx])
        sel = set(orc.expand(orc.topb(scores[:ctx].astype(np.float32), B), ctx, r).tolist())
        sel.add(ctx - 1)
        expect = np.zeros(32)
        expect[sorted(sel)] = 1.0 / len(sel)
        np.testing.assert_allclose(out[0], expect, atol=1e-15)


def test_gqa_query_heads_use_their_group_and_importance_head():
    # Hq = 4, Hkv = 2, Himp = 2: query heads 0,1 -> KV head 0 and importance head 0;
    # heads 2,3 -> KV head 1 and importance head 1
    D, n = 8, 6
    K = np.zeros((2, n, D))
    V = np.zeros((2, n, D))
    V[0, :, 0] = 1.0      # KV head 0 marks coordinate 0
    V[1, :, 1] = 1.0      # KV head 1 marks coordinate 1
    K[0, :, 2] = np.arange(n)          # importance head 0 prefers late tokens
    K[1, :, 2] = -np.arange(n)         # importance head 1 prefers early tokens
    V[0, :, 2 + 0] += np.arange(n)     # value reveals which token was attended
    V[1, :, 2 + 1] += np.arange(n)
    W = np.zeros((D, 1))
    W[2, 0] = 1.0
    Kc, Vc = K.copy(), V.copy()
    st = orc.SequenceState(Kc, Vc, orc.project(Kc, W, orc.F32), Himp=2, B=1, r=0)
    out = orc.decode_step(st, W, np.zeros((4, D)), np.ones((2, 1)), n, orc.F32, True, 1.0)
    # head 0/1: token n-1 of KV head 0; head 2/3: token 0 of KV head 1 (no append: keep_from = n)
    for h in (0, 1):
        assert out[h, 0] == 1.0 and out[h, 1] == 0.0 and out[h, 2] == n - 1
    for h in (2, 3):
        assert out[h, 1] == 1.0 and out[h, 0] == 0.0 and out[h, 3] == 0.0
