"""The TB_CHECK debug mode on the GPU: each condition it reports is planted
from the host in otherwise valid calls (the kernels clamp or ignore every
one of them, so nothing faults), and clean calls report nothing."""
import pytest
import torch

from query_aware_kv_amd import synth
from query_aware_kv_amd import tokenbutler as tbl
from query_aware_kv_amd.workloads import Workload
from tests.gpu_cases import device_case, need_gpu

pytestmark = pytest.mark.gpu

W = Workload("check_bf16", batch=2, layers=1, n_q_heads=8, n_kv_heads=2, n_imp_heads=8,
             head_dim=128, d_imp=32, dtype="bf16", ctx0=999, steps=1, budget=50, radius=1,
             interval=1, plant_per_head=5, plant_runs=0, plant_run_len=0, plant_shift=3.0,
             seed=21)


@pytest.fixture(autouse=True)
def _check_mode():
    need_gpu()
    tbl.set_check(True)
    tbl.check_flags(clear=True)
    yield
    tbl.set_check(False)
    tbl.check_flags(clear=True)


@pytest.fixture(scope="module")
def case():
    need_gpu()
    return device_case(W), synth.step_inputs(W, 0, synth.prefill(W))


def _step(dc, inp, *, q=None, ctx=None, refresh=True):
    w = dc.w
    ctx_t = torch.full((w.batch,), w.ctx if ctx is None else ctx, dtype=torch.int32,
                       device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    args = tbl.step_args(dc.shape, dc.params, q=(inp.q if q is None else q).cuda(),
                         q_imp=inp.q_imp.cuda(), k_new=inp.k_new.cuda(), v_new=inp.v_new.cuda(),
                         refresh=refresh, w=dc.W, k_cache=dc.K, v_cache=dc.V, kp_cache=dc.Kp,
                         ctx_len=ctx_t, softmax_scale=w.softmax_scale, sel_idx=dc.sel,
                         sel_count=dc.cnt, sel_bits=dc.bits, keep_from=dc.keep, out=out)
    tbl.decode_step(dc.shape, dc.params, args, dc.ws)
    return tbl.check_flags(clear=True), ctx_t, out


def test_clean_calls_report_nothing(case):
    dc, inp = case
    assert tbl.check_enabled()
    flags, ctx, out = _step(dc, inp)
    assert flags == 0
    tbl.sparse_attn(dc.shape, inp.q.cuda(), dc.K, dc.V, dc.sel, dc.cap_s, dc.cnt, dc.keep, ctx,
                    W.softmax_scale, out, dc.ws)
    assert tbl.check_flags(clear=True) == 0
    _step(dc, inp, refresh=False)
    assert tbl.check_flags(clear=True) == 0


def test_nonfinite_query(case):
    dc, inp = case
    q = inp.q.clone()
    q[1, 3, 7] = float("nan")
    assert _step(dc, inp, q=q)[0] == tbl.CHECK_NONFINITE_INPUT


def test_nonfinite_cache_rows_read_by_the_step(case):
    dc, inp = case
    saved = dc.Kp[1, 0, 10].clone()
    dc.Kp[1, 0, 10, 3] = float("inf")
    try:
        assert _step(dc, inp)[0] == tbl.CHECK_NONFINITE_CACHE
    finally:
        dc.Kp[1, 0, 10] = saved
    # the appended row's position is written by the step, not read before it
    dc.V[0, 1, W.ctx - 1, 0] = float("nan")
    assert _step(dc, inp)[0] == 0


def test_context_length_beyond_capacity(case):
    dc, inp = case
    assert _step(dc, inp, ctx=W.ctx_cap + 3)[0] == tbl.CHECK_CTX_RANGE
    assert _step(dc, inp)[0] == 0


def test_lists_and_keep_from_out_of_range(case):
    dc, inp = case
    flags, ctx, out = _step(dc, inp)
    assert flags == 0
    sel, keep = dc.sel.clone(), dc.keep.clone()
    sel[0, 2, 0] = W.ctx_cap + 7       # past the capacity, and no longer ascending
    keep[1] = W.ctx_cap + 1
    tbl.sparse_attn(dc.shape, inp.q.cuda(), dc.K, dc.V, sel, dc.cap_s, dc.cnt, keep, ctx,
                    W.softmax_scale, out, dc.ws)
    assert tbl.check_flags(clear=True) == tbl.CHECK_SEL_RANGE | tbl.CHECK_KEEP_RANGE
    cnt = dc.cnt.clone()
    cnt[1, 5] = dc.cap_s + 1
    tbl.sparse_attn(dc.shape, inp.q.cuda(), dc.K, dc.V, dc.sel, dc.cap_s, cnt, dc.keep, ctx,
                    W.softmax_scale, out, dc.ws)
    assert tbl.check_flags(clear=True) == tbl.CHECK_SEL_RANGE


def test_nonfinite_scores_given_to_the_selection(case):
    dc, inp = case
    ctx = torch.full((W.batch,), W.ctx, dtype=torch.int32, device="cuda")
    scores = torch.empty((W.batch, W.n_imp_heads, W.ctx_cap), dtype=torch.float32, device="cuda")
    tbl.score(dc.shape, inp.q_imp.cuda(), dc.Kp, ctx, scores, dc.ws)
    assert tbl.check_flags(clear=True) == 0
    scores[1, 4, 17] = float("nan")
    tbl.select(dc.shape, dc.params, scores, ctx, dc.sel, dc.cnt, dc.ws)
    assert tbl.check_flags(clear=True) == tbl.CHECK_NONFINITE_SCORES


def test_mlp_weights():
    shape = tbl.make_mlp_shape(2, 256, 256, 1, 4, 16, torch.bfloat16, tbl.TB_ACT_RELU)
    m = synth.mlp_inputs(2, 256, 256, 64, torch.bfloat16, 5)
    h, w1, w2 = m.h.cuda(), m.w1.cuda(), m.w2.cuda()
    ws = tbl.alloc_mlp_workspace(shape)
    q = torch.empty((1, 2, 4, 16), dtype=torch.bfloat16, device="cuda")
    tbl.predict_queries(shape, h, w1, w2, q, ws)
    assert tbl.check_flags(clear=True) == 0
    w1[7, 100] = float("-inf")
    tbl.predict_queries(shape, h, w1, w2, q, ws)
    assert tbl.check_flags(clear=True) == tbl.CHECK_NONFINITE_INPUT


def test_mode_off_runs_no_check(case):
    dc, inp = case
    tbl.set_check(False)
    q = inp.q.clone()
    q[0, 0, 0] = float("nan")
    assert _step(dc, inp, q=q, ctx=W.ctx_cap + 2)[0] == 0
