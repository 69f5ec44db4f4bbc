"""The importance-query producer MLP (tb_predict_queries) against the oracle.

Tolerance, from the arithmetic: the GPU sums each layer's products in fp32
on the matrix cores (in an order of its own) and rounds the hidden layer and
the output to the dtype, as the oracle does from fp64 sums.  A hidden value
near a rounding midpoint may round the other way (one unit in the last place,
2^-7 relative in bf16, 2^-23 in fp32), the fp32 sums carry at most F * 2^-24
of the sum of magnitudes, and the output rounding can differ by one unit.  So
per output, with S = sum_f |u_f * W2[n][f]| over the oracle's hidden layer u:
  bf16: |gpu - ref| <= (2^-6 + F * 2^-24) * S
  fp32: |gpu - ref| <= (F + 16) * 2^-23 * S   (16 units cover SiLU's exp)
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as orc
from gpu_cases import f64, need_gpu
from query_aware_kv_amd import synth
from query_aware_kv_amd import tokenbutler as tbl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


ACTS = {tbl.TB_ACT_RELU: orc.ACT_RELU, tbl.TB_ACT_SILU: orc.ACT_SILU}


def _run(M, E, F, G, Himp, d, dtype, act, seed=3, ws=None):
    N = G * Himp * d
    inp = synth.mlp_inputs(M, E, F, N, dtype, seed)
    shape = tbl.make_mlp_shape(M, E, F, G, Himp, d, dtype, act)
    ws = ws if ws is not None else tbl.alloc_mlp_workspace(shape)
    q = torch.full((G, M, Himp, d), float("nan"), dtype=dtype, device="cuda")
    tbl.predict_queries(shape, inp.h.cuda(), inp.w1.cuda(), inp.w2.cuda(), q, ws)
    torch.cuda.synchronize()
    return inp, q, ws


def _check(inp, q, G, Himp, d, dtype, act):
    od = orc.F32 if dtype == torch.float32 else orc.BF16
    h, W1, W2 = f64(inp.h), f64(inp.w1), f64(inp.w2)
    F = W1.shape[0]
    ref = orc.mlp(h, W1, W2, G, Himp, d, ACTS[act], od)
    # the oracle's hidden layer: the same MLP with an identity second layer
    u = orc.mlp(h, W1, np.eye(F), 1, 1, F, ACTS[act], od)[0, :, 0, :]
    S = np.abs(u) @ np.abs(W2).T                                  # [M][N]
    S = S.reshape(h.shape[0], G, Himp, d).transpose(1, 0, 2, 3)  # slot-major
    if dtype == torch.bfloat16:
        tol = (2.0 ** -6 + F * 2.0 ** -24) * S
    else:
        tol = (F + 16) * 2.0 ** -23 * S
    got = f64(q)
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))
    return got, ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("act", [tbl.TB_ACT_RELU, tbl.TB_ACT_SILU], ids=["relu", "silu"])
@pytest.mark.parametrize("M", [1, 3, 16, 17, 64])
def test_mlp_small(dtype, act, M):
    G, Himp, d = 2, 4, 16
    inp, q, _ = _run(M, 512, 256, G, Himp, d, dtype, act)
    _check(inp, q, G, Himp, d, dtype, act)


@pytest.mark.parametrize("M", [1, 16])
def test_mlp_llama_producer(M):
    # Llama-3-8B hidden size, inner width 1024, four consumer slots of 32
    # heads x 32 dims (the decode-step shape the benchmark times)
    G, Himp, d = 4, 32, 32
    inp, q, ws = _run(M, 4096, 1024, G, Himp, d, torch.bfloat16, tbl.TB_ACT_SILU)
    got, ref = _check(inp, q, G, Himp, d, torch.bfloat16, tbl.TB_ACT_SILU)
    # most outputs round to the oracle's value exactly
    assert np.mean(got == ref) > 0.9
    # deterministic: the same call on the reused workspace gives the same bits
    q2 = torch.empty_like(q)
    shape = tbl.make_mlp_shape(M, 4096, 1024, G, Himp, d, torch.bfloat16, tbl.TB_ACT_SILU)
    tbl.predict_queries(shape, inp.h.cuda(), inp.w1.cuda(), inp.w2.cuda(), q2, ws)
    torch.cuda.synchronize()
    assert torch.equal(q, q2)


def test_mlp_slot_feeds_score():
    # slot g of the output is a [M][Himp][d] importance query: scoring with it
    # through tb_score equals scoring with the oracle's slot
    M, G, Himp, d = 2, 2, 8, 16
    inp, q, _ = _run(M, 256, 256, G, Himp, d, torch.float32, tbl.TB_ACT_RELU, seed=9)
    ref = orc.mlp(f64(inp.h), f64(inp.w1), f64(inp.w2), G, Himp, d, orc.ACT_RELU, orc.F32)
    np.testing.assert_allclose(f64(q), ref, rtol=0, atol=1e-5)
    assert q[1].is_contiguous() and tuple(q[1].shape) == (M, Himp, d)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("E,F", [(1024, 512), (512, 2048)], ids=["split_layer1", "split_layer2"])
@pytest.mark.parametrize("M", [3, 17, 64])
def test_mlp_split_over_k(dtype, E, F, M):
    # layers with few output columns split k over four work-groups whose
    # partial tiles the last one adds in split order: within the bound, the
    # same bits on every call, and the arrival counters left at zero (the
    # reused workspace gives the same result twice more)
    G, Himp, d = 2, 4, 16
    inp, q, ws = _run(M, E, F, G, Himp, d, dtype, tbl.TB_ACT_SILU)
    _check(inp, q, G, Himp, d, dtype, tbl.TB_ACT_SILU)
    shape = tbl.make_mlp_shape(M, E, F, G, Himp, d, dtype, tbl.TB_ACT_SILU)
    for _ in range(2):
        q2 = torch.empty_like(q)
        tbl.predict_queries(shape, inp.h.cuda(), inp.w1.cuda(), inp.w2.cuda(), q2, ws)
        torch.cuda.synchronize()
        assert torch.equal(q, q2)
