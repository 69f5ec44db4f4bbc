"""Dense decode attention (tb_dense_attn) against the oracle's softmax
attention over every cached token, plus its agreement with the sparse kernel
when the selection covers the whole context."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as orc
from gpu_cases import TOL, f64, need_gpu, shape_of
from query_aware_kv_amd import synth
from query_aware_kv_amd import tokenbutler as tbl
from query_aware_kv_amd.workloads import LLAMA_32K, LONG_128K, TINY_F32, Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _w(**kw) -> Workload:
    base = dict(name="dense_small", batch=3, layers=1, n_q_heads=8, n_kv_heads=2, n_imp_heads=8,
                head_dim=128, d_imp=32, dtype="bf16", ctx0=1999, steps=1, budget=50, radius=0,
                interval=1, plant_per_head=0, plant_runs=0, plant_run_len=0, plant_shift=0.0,
                seed=21)
    base.update(kw)
    return Workload(**base)


def _run_dense(w: Workload, lens, pre=None):
    pre = pre if pre is not None else synth.prefill(w)
    shape = shape_of(w)
    ws = tbl.alloc_workspace(shape, tbl.make_params(w.budget, w.radius))
    K, V = pre.K.cuda(), pre.V.cuda()
    q = synth.step_inputs(w, 0, pre).q.cuda()
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), dtype=K.dtype,
                     device="cuda")
    tbl.dense_attn(shape, q, K, V, ctx, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    return pre, q, K, V, ctx, ws, out


def _check(w: Workload, pre, q, out, lens, heads=None):
    worst = 0.0
    for b, n in enumerate(lens):
        q64 = f64(q[b])
        for g in range(w.n_kv_heads):
            hs = [h for h in range(w.n_q_heads) if h * w.n_kv_heads // w.n_q_heads == g]
            hs = [h for h in hs if heads is None or h in heads]
            if not hs:
                continue
            K64 = f64(pre.K[b, g])
            V64 = f64(pre.V[b, g])
            for h in hs:
                ref = orc.attend(q64[h], K64, V64, np.arange(n), w.softmax_scale)
                worst = max(worst, float(np.abs(f64(out[b, h]) - ref).max()))
    assert worst <= TOL[w.dtype], worst


@pytest.mark.parametrize("w,heads", [(TINY_F32, None), (LLAMA_32K, None),
                                     (LONG_128K, (0, 13, 31))],
                         ids=["tiny_f32", "llama32k", "long128k"])
def test_dense_full_size(w, heads):
    # the context ends inside a chunk (ctx0 = 2^k - 1)
    lens = [w.ctx0] * w.batch
    pre, q, _, _, _, _, out = _run_dense(w, lens)
    _check(w, pre, q, out, lens, heads)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(dtype="f32", head_dim=64, d_imp=16),
    dict(n_q_heads=16, n_kv_heads=2, n_imp_heads=16),          # group 8
    dict(n_q_heads=2, n_kv_heads=2, n_imp_heads=2, head_dim=64),
    dict(dtype="f32", head_dim=128, n_q_heads=4, n_kv_heads=2, n_imp_heads=4),
], ids=["bf16_g4", "f32_d64_g4", "bf16_g8", "mha_d64", "f32_d128_g2"])
def test_dense_ragged_batch(kw):
    # lengths 1, one chunk plus a tail, and the full capacity in one launch
    w = _w(**kw)
    lens = [1, 700, 2000]
    pre, q, _, _, _, _, out = _run_dense(w, lens)
    _check(w, pre, q, out, lens)


def test_dense_empty_context_and_repeat():
    w = _w()
    lens = [0, 513, 1999]
    pre, q, K, V, ctx, ws, out = _run_dense(w, lens)
    assert torch.count_nonzero(out[0]) == 0
    _check(w, pre, q, out, lens)
    # the arrival counters are left ready: a second call gives the same bits
    out2 = torch.empty_like(out)
    tbl.dense_attn(shape_of(w), q, K, V, ctx, w.softmax_scale, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_dense_agrees_with_sparse_over_everything():
    # the sparse kernel with every position selected attends the same set
    w = _w()
    lens = [1, 700, 2000]
    pre, q, K, V, ctx, ws, out = _run_dense(w, lens)
    shape = shape_of(w)
    bits = torch.full((w.batch, w.n_imp_heads, tbl.bitmap_words(shape)), -1, dtype=torch.int32,
                      device="cuda")
    out2 = torch.empty_like(out)
    tbl.sparse_attn(shape, q, K, V, None, 0, None, None, ctx, w.softmax_scale, out2, ws,
                    sel_bits=bits)
    torch.cuda.synchronize()
    assert float((out.float() - out2.float()).abs().max()) <= TOL[w.dtype]


@pytest.mark.parametrize("kw", [dict(), dict(dtype="f32", head_dim=64, d_imp=16, n_q_heads=4,
                                            n_kv_heads=4, n_imp_heads=4)],
                         ids=["bf16_g4", "f32_mha_d64"])
def test_sparse_one_chunk_rows(kw):
    # a capacity of at most one attention chunk: every work-group writes its
    # outputs directly (no partials, no arrival); an empty row gives zeros,
    # bitmaps and lists agree, and a repeated call gives the same bits
    w = _w(ctx0=1000, **kw)
    lens = [0, 1, 700, 1000]
    w = Workload(**{**w.__dict__, "batch": len(lens)})
    pre, q, K, V, ctx, ws, _ = _run_dense(w, lens)
    shape = shape_of(w)
    bits = torch.full((w.batch, w.n_imp_heads, tbl.bitmap_words(shape)), -1, dtype=torch.int32,
                      device="cuda")
    out = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), dtype=K.dtype,
                     device="cuda")
    tbl.sparse_attn(shape, q, K, V, None, 0, None, None, ctx, w.softmax_scale, out, ws,
                    sel_bits=bits)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0]) == 0
    _check(w, pre, q, out, lens)
    out2 = torch.empty_like(out)
    tbl.sparse_attn(shape, q, K, V, None, 0, None, None, ctx, w.softmax_scale, out2, ws,
                    sel_bits=bits)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    # the same sets as ascending lists
    cap_s = w.ctx_cap
    sel = torch.arange(cap_s, dtype=torch.int32, device="cuda").expand(
        w.batch, w.n_imp_heads, cap_s).contiguous()
    cnt = ctx[:, None].expand(w.batch, w.n_imp_heads).contiguous()
    out3 = torch.empty_like(out)
    tbl.sparse_attn(shape, q, K, V, sel, cap_s, cnt, None, ctx, w.softmax_scale, out3, ws)
    torch.cuda.synchronize()
    assert float((out.float() - out3.float()).abs().max()) <= TOL[w.dtype]
