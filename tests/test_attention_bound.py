"""The derived bf16 attention bound has power: it accepts the exact output
rounded to bf16 and rejects outputs over a set that misses one percent of
the attended rows, at the shape of the 32K-context workload (CPU only)."""
import numpy as np
import torch

import oracle as orc
from tests.tolerances import TOL, bf16_bound


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def _case(seed, n_att=3600, ctx=32768, D=128, heads=8):
    rng = np.random.default_rng(seed)
    K = _bf16(rng.standard_normal((ctx, D)))
    V = _bf16(rng.standard_normal((ctx, D)))
    q = _bf16(rng.standard_normal((heads, D)))
    A = np.sort(rng.choice(ctx, size=n_att, replace=False))
    return rng, K, V, q, A


def test_bound_accepts_rounded_exact_output():
    _, K, V, q, A = _case(1)
    scale = 1 / np.sqrt(128)
    for h in range(q.shape[0]):
        o, w = orc.attend(q[h], K, V, A, scale, return_weights=True)
        bound = bf16_bound(o, w, V[A])
        assert np.all(np.abs(_bf16(o) - o) <= bound)


def test_bound_rejects_one_percent_of_rows_dropped():
    rng, K, V, q, A = _case(2)
    scale = 1 / np.sqrt(128)
    worst = []
    for h in range(q.shape[0]):
        o, w = orc.attend(q[h], K, V, A, scale, return_weights=True)
        bound = bf16_bound(o, w, V[A])
        kept = np.sort(rng.choice(A, size=A.size - A.size // 100, replace=False))
        o_drop = _bf16(orc.attend(q[h], K, V, kept, scale))
        ratio = float(np.max(np.abs(o_drop - o) / bound))
        worst.append(ratio)
        # the contract bar alone lets this through
        assert np.abs(o_drop - o).max() <= TOL["bf16"]
    # every head's wrong output breaks the derived bound somewhere
    assert min(worst) > 1.0, worst


def test_bound_rejects_rows_swapped_for_neighbors():
    # one percent of the attended rows replaced by their next position: the
    # sets have the same size, only membership is off
    rng, K, V, q, A = _case(3)
    scale = 1 / np.sqrt(128)
    for h in range(q.shape[0]):
        o, w = orc.attend(q[h], K, V, A, scale, return_weights=True)
        bound = bf16_bound(o, w, V[A])
        B = A.copy()
        idx = rng.choice(A.size, size=A.size // 100, replace=False)
        B[idx] = np.minimum(B[idx] + 1, K.shape[0] - 1)
        B = np.unique(B)
        o_bad = _bf16(orc.attend(q[h], K, V, B, scale))
        assert np.max(np.abs(o_bad - o) / bound) > 1.0
