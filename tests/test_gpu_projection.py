"""Key projection on crafted values, bit for bit against the oracle.

The keys are sparse rows of values whose fp64 sums land on bf16 rounding ties
and next to them, past the largest finite value, in the subnormal range and
below it, and on signed zeros; W holds powers of two.  Both launches are
covered: the small-batch one and the prefill-sized one (16384 rows or more),
for every head_dim / d / dtype the library instantiates, with rows before 0
and past the capacity skipped and the rest of the cache left untouched."""
import numpy as np
import pytest
import torch

import oracle as orc
from query_aware_kv_amd import tokenbutler as tbl
from tests.gpu_cases import need_gpu

pytestmark = pytest.mark.gpu

SENTINEL = -77.0  # exact in bf16 and fp32; never a projection of these keys


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def crafted_keys(rng, rows, D, dtype):
    """Rows with 3 nonzeros drawn from values chosen for their rounding."""
    vals = np.array([1.0, 2.0 ** -8, 3 * 2.0 ** -9, 2.0 ** -24, 2.0 ** -40, 1.0 + 2.0 ** -7,
                     255 / 128, 2.0 ** -126, 2.0 ** -130, 2.0 ** -133, 2.0 ** 127,
                     1.5 * 2.0 ** 127, 2.0 ** -70, 0.0])
    K = np.zeros((rows, D))
    pos = np.argsort(rng.random((rows, D)), axis=1)[:, :3]
    K[np.arange(rows)[:, None], pos] = rng.choice(vals, size=(rows, 3)) * \
        rng.choice([-1.0, 1.0], size=(rows, 3))
    if dtype == torch.float32:  # fp32 keys also carry bits bf16 would drop
        K[::7, 0] = 1.0 + 2.0 ** -20
    return K


def crafted_w(rng, D, d):
    powers = np.array([0.0, 1.0, 0.5, 2.0 ** -8, 2.0 ** -60, 4.0, 2.0 ** -3])
    return rng.choice(powers, size=(D, d)) * rng.choice([-1.0, 1.0], size=(D, d))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D,d", [(128, 32), (128, 16), (64, 32), (64, 16)])
@pytest.mark.parametrize("n", [1040, 37], ids=["prefill", "small"])
def test_projection_crafted_rounding(dtype, D, d, n):
    batch, Hkv, cap = 2, 8, 1100
    pos0 = np.array([-5, 70], dtype=np.int32)  # rows t < 0 and t >= cap are skipped
    rng = np.random.default_rng(1000 * D + 10 * d + n)
    K64 = crafted_keys(rng, batch * Hkv * cap, D, dtype).reshape(batch, Hkv, cap, D)
    W64 = crafted_w(rng, D, d)
    K = torch.from_numpy(K64).to(dtype)
    W = torch.from_numpy(W64).to(dtype)
    assert np.array_equal(K.double().numpy(), K64) and np.array_equal(W.double().numpy(), W64)
    shape = tbl.make_shape(batch, Hkv, Hkv, Hkv, D, d, cap, dtype)
    Kp = torch.full((batch, Hkv, cap, d), SENTINEL, dtype=dtype, device="cuda")
    tbl.project_keys(shape, K.cuda(), W.cuda(), torch.from_numpy(pos0).cuda(), n, Kp)
    torch.cuda.synchronize()
    got = Kp.cpu()
    code = orc.BF16 if dtype == torch.bfloat16 else orc.F32
    want = torch.full((batch, Hkv, cap, d), SENTINEL, dtype=torch.float64)
    for b in range(batch):
        t0, t1 = max(pos0[b], 0), min(pos0[b] + n, cap)
        want[b, :, t0:t1] = torch.from_numpy(orc.project(K64[b, :, t0:t1], W64, code))
    # compare the stored bits (NaN-free here; infinities and signed zeros included)
    want = want.to(dtype)
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    diff = (got.view(bits) != want.view(bits))
    assert not diff.any(), f"{int(diff.sum())} mismatches, first at {diff.nonzero()[0].tolist()}"
    # the crafted values really reach the edge cases
    w = want.double()
    assert torch.isinf(w).any() and (w == 0).any()
    assert ((w.abs() > 0) & (w.abs() < 2.0 ** -126)).any()  # bf16 / fp32 subnormal results
