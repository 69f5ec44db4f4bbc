"""GPU parity: every stage of the HIP path, called through the C ABI, against
the fp64 CPU oracle on the same seeded inputs.

Bars: projected keys and scores bit-exact (both sides round the same fp64
sums once); index sets bit-exact against the oracle's fp32-chain selection
and, independently, equal to the selection of the exact fp64 scores outside
the 1e-6 relative band around the B-th score; attention outputs within
max-abs 1e-4 (fp32) / 2e-2 (bf16), and bf16 outputs also within the derived
per-element bound (half a bf16 unit plus an fp32 accumulation allowance)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as orc
from query_aware_kv_amd import synth
from query_aware_kv_amd import tokenbutler as tbl
from query_aware_kv_amd.workloads import INTERVAL_16K, LLAMA_32K, LONG_128K, TINY_F32, Workload
from tests.gpu_cases import (TOL, assert_attention, assert_fp64_selection, attended_sets,
                             band_members, bitmap_positions, device_case, f64, lists_of,
                             need_gpu, odtype, oracle_attention, oracle_state, step_on_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _imp(w, h):
    return h * w.n_imp_heads // w.n_q_heads


def _kv(w, h):
    return h * w.n_kv_heads // w.n_q_heads


# --------------------------------------------------------------------------
# stage by stage: projection -> scores -> selection -> attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("w", [TINY_F32, LLAMA_32K], ids=lambda w: w.name)
def test_stage_parity(w):
    dc = device_case(w)
    pre = dc.pre
    b = 0
    ctx = w.ctx
    dt = odtype(w)
    W64 = f64(pre.W)
    # prefill projection: bit-exact
    K64 = f64(pre.K[b])
    Kp_ref = np.zeros((w.n_kv_heads, w.ctx_cap, w.d_imp))
    Kp_ref[:, :w.ctx0] = orc.project(K64[:, :w.ctx0], W64, dt)
    np.testing.assert_array_equal(f64(dc.Kp[b][:, :w.ctx0]), Kp_ref[:, :w.ctx0])
    # append the step's token (a plain copy) and project that one row
    dc.K[:, :, w.ctx0] = pre.k_next[:, :, 0].cuda()
    dc.V[:, :, w.ctx0] = pre.v_next[:, :, 0].cuda()
    pos0 = torch.full((w.batch,), w.ctx0, dtype=torch.int32, device="cuda")
    tbl.project_keys(dc.shape, dc.K, dc.W, pos0, 1, dc.Kp)
    K64[:, w.ctx0] = f64(pre.k_next[b][:, 0])
    V64 = f64(pre.V[b])
    V64[:, w.ctx0] = f64(pre.v_next[b][:, 0])
    Kp_ref[:, w.ctx0] = orc.project(K64[:, w.ctx0], W64, dt)
    np.testing.assert_array_equal(f64(dc.Kp[b][:, :ctx]), Kp_ref[:, :ctx])
    # scores: bit-exact fp32
    ctx_len = torch.full((w.batch,), ctx, dtype=torch.int32, device="cuda")
    scores = torch.zeros((w.batch, w.n_imp_heads, w.ctx_cap), dtype=torch.float32, device="cuda")
    qi = pre.q_imp0.cuda()
    tbl.score(dc.shape, qi, dc.Kp, ctx_len, scores, dc.ws)
    s64, s32 = orc.score(f64(pre.q_imp0[b]), Kp_ref, n=ctx)
    np.testing.assert_array_equal(scores[b, :, :ctx].cpu().numpy(), s32)
    # the fp32 fma chains stay within the a-priori bound d * 2^-24 * sum |q_j kp_j|
    # of the fp64 dot products
    qa = np.abs(f64(pre.q_imp0[b]))
    for i in range(w.n_imp_heads):
        g = i * w.n_kv_heads // w.n_imp_heads
        bound = w.d_imp * 2.0 ** -24 * (np.abs(Kp_ref[g, :ctx]) @ qa[i])
        assert np.all(np.abs(s32[i].astype(np.float64) - s64[i]) <= bound + 1e-30), i
    # top-B and neighbor expansion: exact index sets
    topb = torch.full((w.batch, w.n_imp_heads, w.budget), -1, dtype=torch.int32, device="cuda")
    tbl.select(dc.shape, dc.params, scores, ctx_len, dc.sel, dc.cnt, dc.ws, topb_idx=topb,
               sel_bits=dc.bits)
    torch.cuda.synchronize()
    got = lists_of(dc.sel, dc.cnt, b)
    got_bits = bitmap_positions(dc.bits, b, ctx)
    S_ref = []
    topb_h = topb[b].cpu().numpy()
    for i in range(w.n_imp_heads):
        T_ref = orc.topb(s32[i], w.budget)
        assert topb_h[i, :T_ref.size].tolist() == T_ref.tolist(), i
        S_ref.append(orc.expand(T_ref, ctx, w.radius))
        assert got[i] == S_ref[-1].tolist(), i
        assert got_bits[i] == S_ref[-1].tolist(), i
        # independently: the ranking of the exact fp64 scores
        assert_fp64_selection(got[i], s64[i], ctx, w.budget, w.radius,
                              T_gpu=topb_h[i, :min(w.budget, ctx)], what=("stage", i))
    # attention over S united with the appended token
    keep = torch.full((w.batch,), ctx - 1, dtype=torch.int32, device="cuda")
    q = synth.draw_q(w, 0)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=q.dtype, device="cuda")
    out2 = torch.empty_like(out)
    tbl.sparse_attn(dc.shape, q.cuda(), dc.K, dc.V, dc.sel, dc.cap_s, dc.cnt, keep, ctx_len,
                    w.softmax_scale, out, dc.ws)
    tbl.sparse_attn(dc.shape, q.cuda(), dc.K, dc.V, None, 0, None, keep, ctx_len,
                    w.softmax_scale, out2, dc.ws, sel_bits=dc.bits)
    torch.cuda.synchronize()
    q64 = f64(q[b])
    sets = [sorted(set(S_ref[_imp(w, h)].tolist()) | {ctx - 1}) for h in range(w.n_q_heads)]
    o_ref, bound = oracle_attention(w, K64, V64, q64, sets)
    assert_attention(f64(out[b]), o_ref, bound, w.dtype, what="list route")
    # list membership (contiguous chunks) and bitmap membership (interleaved
    # chunks) visit the rows in different chunk orders: the same values up
    # to rounding, each within the bars of the oracle, and within the sum of
    # both bounds of each other
    assert_attention(f64(out2[b]), o_ref, bound, w.dtype, what="bitmap route")
    assert_attention(f64(out2[b]), f64(out[b]), 2 * bound, w.dtype, what="list vs bitmap")


def _check_step(w, dc, st, inp, out, s, b, n, q_imp=None, refresh=None, k_new=None,
                v_new=None, use_bits=False):
    """One oracle step of sequence b (context n after the append) and the
    comparison of the GPU's stored selection and output with it: the stored
    sets bit for bit and against the fp64 ranking (on refresh steps), the
    output within the bars."""
    refresh = inp.refresh if refresh is None else refresh
    qi = (inp.q_imp[b] if inp.q_imp is not None else None) if q_imp is None else q_imp
    kn = inp.k_new[b] if k_new is None else k_new
    vn = inp.v_new[b] if v_new is None else v_new
    orc.decode_step(st, f64(dc.pre.W), f64(inp.q[b]), f64(qi) if qi is not None else None, n,
                    odtype(w), refresh, w.softmax_scale, k_new=f64(kn), v_new=f64(vn))
    if refresh:
        got = bitmap_positions(dc.bits, b, n) if use_bits else lists_of(dc.sel, dc.cnt, b)
        s64 = orc.score(f64(qi), st.Kp, n=n)[0]
        for i in range(w.n_imp_heads):
            assert got[i] == st.sel[i, :st.cnt[i]].tolist(), (s, b, i)
            assert_fp64_selection(got[i], s64[i], n, w.budget, w.radius, w.n_sink, w.n_local,
                                  what=(s, b, i))
    o_ref, bound = oracle_attention(w, st.K, st.V, f64(inp.q[b]), attended_sets(w, st, n))
    return assert_attention(f64(out[b]), o_ref, bound, w.dtype, what=(s, b))


# --------------------------------------------------------------------------
# the fused step at full size (the launch the benchmark times)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("w", [TINY_F32, LLAMA_32K, LONG_128K], ids=lambda w: w.name)
def test_fused_step_full_size(w):
    dc = device_case(w)
    inp = synth.step_inputs(w, 0, dc.pre)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    step_on_device(dc, 0, inp, out)
    for b in range(w.batch):
        st = oracle_state(w, dc.pre, b)
        _check_step(w, dc, st, inp, out, 0, b, w.ctx)
        assert int(dc.keep[b]) == int(st.keep_from[0]) == w.ctx0
        # the whole projected-key cache, the appended row included, bit for bit
        np.testing.assert_array_equal(f64(dc.Kp[b][:, :w.ctx]), st.Kp[:, :w.ctx])


@pytest.mark.parametrize("kw", [dict(ctx0=1996), dict(ctx0=1996, dtype="f32", head_dim=64, d_imp=16,
                                                  n_sink=3, n_local=10)],
                         ids=["bf16", "f32_sink_local"])
def test_fused_step_odd_capacity(kw):
    # a capacity that is not a multiple of 8 (1997): the selection's 16-bit
    # keys are read one at a time instead of in 16-byte pieces
    w = _small(**kw)
    assert w.ctx_cap % 8 != 0
    dc = device_case(w)
    inp = synth.step_inputs(w, 0, dc.pre)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    step_on_device(dc, 0, inp, out)
    for b in range(w.batch):
        _check_step(w, dc, oracle_state(w, dc.pre, b), inp, out, 0, b, w.ctx)


@pytest.mark.parametrize("ctx0", [16383, 16384], ids=["cap16384", "cap16385"])
def test_fused_step_selection_block_sizes(ctx0):
    # the fused step selects rows of up to 16384 positions with 512 threads
    # (every thread holding one 32-position word and four sample keys at
    # 16384) and longer rows with 1024
    w = _small(ctx0=ctx0, batch=2, budget=1600)
    dc = device_case(w)
    inp = synth.step_inputs(w, 0, dc.pre)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    step_on_device(dc, 0, inp, out)
    for b in range(w.batch):
        _check_step(w, dc, oracle_state(w, dc.pre, b), inp, out, 0, b, w.ctx)


@pytest.mark.parametrize("kw", [
    dict(ctx0=32768, batch=2, budget=2000, radius=1),                   # 1025 words
    dict(ctx0=70000, batch=1, budget=3500, radius=0, n_sink=5, n_local=64,
         plant_per_head=0, plant_runs=6, plant_run_len=32),             # 2188 words, odd cap
    dict(ctx0=40000, batch=1, budget=1, radius=2),                      # a budget of one
], ids=["cap32769", "cap70001_sink_local_runs", "cap40001_budget1"])
def test_fused_step_long_rows_16bit_keys(kw):
    # rows longer than 1024 words: the selection classifies each thread's
    # several words from the 16-bit keys the score launch stored, re-read
    # per word, and samples them from the compact sample
    w = _small(**kw)
    assert (w.ctx_cap + 31) // 32 > 1024
    dc = device_case(w)
    inp = synth.step_inputs(w, 0, dc.pre)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    step_on_device(dc, 0, inp, out)
    for b in range(w.batch):
        _check_step(w, dc, oracle_state(w, dc.pre, b), inp, out, 0, b, w.ctx)


def test_planted_tokens_are_found():
    # sanity of the synthetic workload, not a parity bar: with a shift of 4
    # score standard deviations nearly every planted token is selected
    w = TINY_F32
    dc = device_case(w)
    inp = synth.step_inputs(w, 0, dc.pre)
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    step_on_device(dc, 0, inp, out)
    got = lists_of(dc.sel, dc.cnt, 0)
    hit = sum(len(set(dc.pre.planted[(0, i)].tolist()) & set(got[i])) for i in range(4))
    assert hit >= 28, hit


def test_prediction_interval_with_sink_and_window():
    # the interval workload with a sink of 4 and a local window of 256 over
    # 20 steps, every sequence (the plain 64-step run is in
    # test_gpu_workloads.py)
    w = replace(INTERVAL_16K, name="interval_sink_local", steps=20, n_sink=4, n_local=256)
    dc = device_case(w)
    states = {b: oracle_state(w, dc.pre, b) for b in range(w.batch)}
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    for s in range(w.steps):
        inp = synth.step_inputs(w, s, dc.pre)
        step_on_device(dc, s, inp, out)
        for b in range(w.batch):
            _check_step(w, dc, states[b], inp, out, s, b, w.ctx0 + s + 1)
            assert int(dc.keep[b]) == w.ctx0 + (s // w.interval) * w.interval


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def _small(**kw) -> Workload:
    base = dict(name="small", batch=3, layers=1, n_q_heads=8, n_kv_heads=2, n_imp_heads=8,
                head_dim=128, d_imp=32, dtype="bf16", ctx0=1999, steps=1, budget=50, radius=1,
                interval=1, plant_per_head=5, plant_runs=0, plant_run_len=0, plant_shift=3.0,
                seed=11)
    base.update(kw)
    return Workload(**base)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(dtype="f32", head_dim=64, d_imp=16),
    dict(n_imp_heads=2),                              # one importance head per KV head
    dict(n_q_heads=16, n_kv_heads=2, n_imp_heads=4),  # group 8, importance heads shared by 4
    dict(budget=1, radius=0),
    dict(budget=3000),                                # budget >= context: dense
    dict(radius=40),                                  # dilation in several passes
    dict(n_q_heads=2, n_kv_heads=2, n_imp_heads=2, head_dim=64),
    dict(n_sink=4, n_local=64),                       # sink and local window
    dict(n_sink=800, n_local=1500, budget=20),        # the buffers cover every context
    dict(n_sink=3, n_local=5, radius=2, dtype="f32", head_dim=64, d_imp=16),
    # one importance head per KV head: a group's query heads share their
    # rows, which the attention streams once for all of them
    dict(n_q_heads=16, n_kv_heads=2, n_imp_heads=2),
    dict(dtype="f32", head_dim=64, d_imp=16, n_imp_heads=2),
    # rows of 513..1024 words (1024-thread selection), most of every row
    # past the sequences' lengths
    dict(ctx0=19999, budget=600),
    dict(ctx0=19999, budget=600, n_sink=4, n_local=64, dtype="f32", head_dim=64, d_imp=16),
], ids=["base", "f32", "imp_per_kv", "group8", "B1", "dense", "r40", "mha_d64", "sink_local",
        "buffers_cover", "sink_local_f32", "group8_shared", "f32_shared", "cap20000",
        "cap20000_f32_sink_local"])
def test_ragged_batch_fused(kw):
    # three sequences of different lengths (1, 700 and 2000 tokens) in one launch
    w = _small(**kw)
    dc = device_case(w)
    inp = synth.step_inputs(w, 0, dc.pre)
    lens = [1, 700, 2000]
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    args = tbl.step_args(dc.shape, dc.params, q=inp.q.cuda(), q_imp=inp.q_imp.cuda(), k_new=inp.k_new.cuda(),
                         v_new=inp.v_new.cuda(), refresh=True, w=dc.W, k_cache=dc.K,
                         v_cache=dc.V, kp_cache=dc.Kp, ctx_len=ctx,
                         softmax_scale=w.softmax_scale, sel_idx=dc.sel, sel_count=dc.cnt,
                         sel_bits=dc.bits, keep_from=dc.keep, out=out)
    tbl.decode_step(dc.shape, dc.params, args, dc.ws)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        st = oracle_state(w, dc.pre, b)
        _check_step(w, dc, st, inp, out, 0, b, n)
        if w.budget >= n:   # budget covering the context reproduces dense attention
            for h in range(w.n_q_heads):
                dense = orc.attend(f64(inp.q[b, h]), st.K[_kv(w, h)], st.V[_kv(w, h)],
                                   np.arange(n), w.softmax_scale)
                assert np.abs(f64(out[b, h]) - dense).max() <= TOL[w.dtype]


@pytest.mark.parametrize("kw", [
    # 8 query heads per KV head sharing 2 importance heads, sink and window
    dict(batch=40, n_q_heads=16, n_kv_heads=2, n_imp_heads=4, n_sink=4, n_local=64),
    # 2 query heads per KV head, one importance head each
    dict(batch=20, n_q_heads=8, n_kv_heads=4, n_imp_heads=8),
    # past 64K positions a work-group takes 4096 of them (2048 with eight
    # query heads per KV head)
    dict(ctx0=70000, budget=2000, batch=16, n_q_heads=8, n_kv_heads=2, n_imp_heads=8),
    dict(ctx0=70000, budget=2000, batch=16, n_q_heads=16, n_kv_heads=2, n_imp_heads=4),
], ids=["group8", "group2", "long_chunks", "long_chunks_group8"])
def test_windowed_attention_walk(kw):
    # a grid of at least two work-groups per compute unit: the bitmap
    # attention walks its rows in barrier-separated windows; ragged lengths
    # leave some chunks with no positions and others ending mid-word
    w = _small(**{"ctx0": 7000, "budget": 300, **kw})
    chunk = 1024 if w.ctx_cap <= 65536 else (4096 if w.group <= 4 else 2048)
    wgs = -(-w.ctx_cap // chunk) * w.n_kv_heads * w.batch
    assert wgs >= 2 * torch.cuda.get_device_properties(0).multi_processor_count
    dc = device_case(w)
    inp = synth.step_inputs(w, 0, dc.pre)
    lens = [w.ctx_cap] * w.batch
    lens[:4] = [1, 33, chunk + 1, w.ctx_cap - 2000]
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    args = tbl.step_args(dc.shape, dc.params, q=inp.q.cuda(), q_imp=inp.q_imp.cuda(),
                         k_new=inp.k_new.cuda(), v_new=inp.v_new.cuda(), refresh=True, w=dc.W,
                         k_cache=dc.K, v_cache=dc.V, kp_cache=dc.Kp, ctx_len=ctx,
                         softmax_scale=w.softmax_scale, sel_idx=dc.sel, sel_count=dc.cnt,
                         sel_bits=dc.bits, keep_from=dc.keep, out=out)
    tbl.decode_step(dc.shape, dc.params, args, dc.ws)
    # the same attention from the index lists (contiguous chunks)
    out_l = torch.empty_like(out)
    tbl.sparse_attn(dc.shape, inp.q.cuda(), dc.K, dc.V, dc.sel, dc.cap_s, dc.cnt, dc.keep, ctx,
                    w.softmax_scale, out_l, dc.ws)
    torch.cuda.synchronize()
    for b in (0, 1, 2, 3, w.batch - 1):
        n = lens[b]
        st = oracle_state(w, dc.pre, b)
        _check_step(w, dc, st, inp, out, 0, b, n, use_bits=True)
        o_ref, bound = oracle_attention(w, st.K, st.V, f64(inp.q[b]), attended_sets(w, st, n))
        assert_attention(f64(out_l[b]), o_ref, bound, w.dtype, what=("list route", b))


def _rows(rng, w, n_new):
    dt = synth.torch_dtype(w)
    return torch.from_numpy(rng.standard_normal((w.batch, w.n_kv_heads, n_new,
                                                 w.head_dim))).to(dt)


@pytest.mark.parametrize("n_new", [3, 8, 9, 40])
@pytest.mark.parametrize("kw", [dict(), dict(ctx0=1996), dict(ctx0=7000, budget=300, batch=40,
                                                            n_q_heads=16, n_kv_heads=2,
                                                            n_imp_heads=4, n_sink=2,
                                                            n_local=100),
                                dict(ctx0=20000, budget=700)],
                         ids=["small_grid", "odd_capacity", "windowed_grid", "cap20000"])
def test_multi_row_appends(kw, n_new):
    # steps that append several rows: up to 8 inside the first launch of the
    # step (the score launch on refresh steps, the attention launch on reuse
    # steps), more in a launch of their own.  A refresh that appends n_new
    # rows, then a reuse step, then another refresh, each appending n_new:
    # the cache rows, their projected keys (bit for bit), keep_from, the
    # stored selections (both comparators) and the outputs follow the oracle
    steps = 3
    w = _small(**kw)
    w = replace(w, ctx0=w.ctx0 - steps * n_new + 1, steps=steps * n_new)
    dc = device_case(w)
    rng = np.random.default_rng(77 + n_new)
    states = {b: oracle_state(w, dc.pre, b) for b in range(w.batch)}
    check = range(w.batch) if w.batch <= 4 else (0, 1, w.batch - 1)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    for s, refresh in enumerate((True, False, True)):
        kn, vn = _rows(rng, w, n_new), _rows(rng, w, n_new)
        dt = synth.torch_dtype(w)
        q = torch.from_numpy(rng.standard_normal((w.batch, w.n_q_heads, w.head_dim))).to(dt)
        qi = torch.from_numpy(rng.standard_normal((w.batch, w.n_imp_heads, w.d_imp))).to(dt)
        n = w.ctx0 + (s + 1) * n_new
        ctx = torch.full((w.batch,), n, dtype=torch.int32, device="cuda")
        args = tbl.step_args(dc.shape, dc.params, q=q.cuda(), q_imp=qi.cuda(), k_new=kn.cuda(),
                             v_new=vn.cuda(), refresh=refresh, w=dc.W, k_cache=dc.K,
                             v_cache=dc.V, kp_cache=dc.Kp, ctx_len=ctx,
                             softmax_scale=w.softmax_scale, sel_idx=dc.sel, sel_count=dc.cnt,
                             sel_bits=dc.bits, keep_from=dc.keep, out=out)
        tbl.decode_step(dc.shape, dc.params, args, dc.ws)
        torch.cuda.synchronize()
        inp = synth.StepInputs(k_new=kn, v_new=vn, q=q, q_imp=qi if refresh else None,
                               refresh=refresh)
        for b in check:
            st = states[b]
            _check_step(w, dc, st, inp, out, s, b, n, use_bits=True)
            rows = slice(n - n_new, n)
            assert torch.equal(dc.K[b][:, rows].cpu(), kn[b])
            assert torch.equal(dc.V[b][:, rows].cpu(), vn[b])
            np.testing.assert_array_equal(f64(dc.Kp[b][:, :n]), st.Kp[:, :n])
            assert int(dc.keep[b]) == int(st.keep_from[0])
            if refresh:
                assert int(dc.keep[b]) == n - n_new
        if refresh:
            # the stored list matches the bitmap
            for b in check:
                assert lists_of(dc.sel, dc.cnt, b) == bitmap_positions(dc.bits, b, n)


def _select_case(scores_rows, lens, B, r, n_sink=0, n_local=0):
    """tb_select on crafted fp32 scores [b][H][cap]."""
    bsz, H, cap = scores_rows.shape
    shape = tbl.make_shape(bsz, H, H, H, 64, 16, cap, torch.float32)
    params = tbl.make_params(B, r, n_sink, n_local)
    cap_s = tbl.selection_capacity(shape, params)
    ws = tbl.alloc_workspace(shape, params)
    sc = torch.from_numpy(np.ascontiguousarray(scores_rows, dtype=np.float32)).cuda()
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sel = torch.full((bsz, H, cap_s), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((bsz, H), -1, dtype=torch.int32, device="cuda")
    topb = torch.full((bsz, H, B), -1, dtype=torch.int32, device="cuda")
    bits = torch.full((bsz, H, tbl.bitmap_words(shape)), -1, dtype=torch.int32, device="cuda")
    tbl.select(shape, params, sc, ctx, sel, cnt, ws, topb_idx=topb, sel_bits=bits)
    # the bitmap alone (no list) carries the same selection
    cnt2 = torch.full_like(cnt, -1)
    bits2 = torch.full_like(bits, -1)
    tbl.select(shape, params, sc, ctx, None, cnt2, ws, sel_bits=bits2)
    torch.cuda.synchronize()
    assert torch.equal(cnt2, cnt) and torch.equal(bits2, bits)
    for b in range(bsz):
        n = lens[b]
        got = lists_of(sel, cnt, b)
        got_bits = bitmap_positions(bits, b, n)
        for i in range(H):
            T_ref, S_ref = orc.select(scores_rows[b, i, :n], B, r, n_sink, n_local)
            assert topb[b, i, :T_ref.size].cpu().tolist() == T_ref.tolist(), (b, i)
            assert got[i] == S_ref.tolist(), (b, i)
            assert got_bits[i] == got[i], (b, i)


@pytest.mark.parametrize("B,r", [(1, 0), (5, 0), (37, 1), (100, 2), (700, 0), (64, 33)])
def test_select_crafted_ties_and_signed_zeros(B, r):
    rng = np.random.default_rng(B * 100 + r)
    cap = 1500
    rows = np.empty((3, 4, cap), dtype=np.float32)
    rows[:, 0] = rng.standard_normal((3, cap))
    rows[:, 1] = rng.integers(-3, 4, size=(3, cap))                    # heavy ties
    rows[:, 2] = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), size=(3, cap))
    rows[:, 3] = 2.5                                                   # all equal
    _select_case(rows, [1, 777, 1500], B, r)


def _long_rows(kind, bsz, H, cap, seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((bsz, H, cap)).astype(np.float32)
    if kind == "gauss":
        return g * 5.0
    if kind == "levels":        # 4096 distinct values: ties at the threshold
        return np.floor(g * 512.0).astype(np.float32)
    if kind == "coarse":        # steps of 1/32: about 180 keys share the threshold's value
        return (np.floor(g * 32.0) / 32.0).astype(np.float32)
    if kind == "sample_low":    # every eighth position far below the rest
        g[..., ::8] -= 100.0
        return g
    if kind == "sample_high":   # every eighth position far above the rest
        g[..., ::8] += 100.0
        return g
    if kind == "narrow":        # all scores inside one binade
        return (1.0 + np.abs(g) * 1e-3).astype(np.float32)
    if kind == "equal":
        return np.full((bsz, H, cap), -3.25, np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["gauss", "levels", "coarse", "sample_low", "sample_high",
                                  "narrow", "equal"])
@pytest.mark.parametrize("cap,lens", [(32768, [32768, 20001, 2049]), (70000, [70000, 40000])])
def test_select_long_rows(kind, cap, lens):
    # long rows go through the sampled bracket of the threshold when it holds
    # and through the full radix select when it does not; the kept set is
    # the same either way
    rows = _long_rows(kind, len(lens), 2, cap, seed=cap + len(kind))
    for B, r in [(max(lens) // 10, 1), (1, 0), (lens[-1] - 1, 0), (4000, 2)]:
        _select_case(rows, lens, B, r)


@pytest.mark.parametrize("kind", ["gauss", "levels", "equal"])
@pytest.mark.parametrize("cap,lens", [(32768, [32768, 20001, 2049]), (70000, [70000, 40000])])
def test_select_long_rows_sink_and_window(kind, cap, lens):
    # the sink and the local window are kept outright and the budget goes to
    # the positions between them (ranges that end inside bitmap words)
    rows = _long_rows(kind, len(lens), 2, cap, seed=cap + 3 * len(kind))
    for B, r, ns, nl in [(max(lens) // 10, 1, 7, 1000), (1, 0, 4, 1), (2000, 2, 33, 4095),
                         (lens[-1], 0, 100, 100), (500, 0, 0, 64), (500, 1, 64, 0)]:
        _select_case(rows, lens, B, r, ns, nl)


@pytest.mark.parametrize("B,r", [(1, 0), (37, 1), (700, 0)])
def test_select_sink_and_window_crafted(B, r):
    rng = np.random.default_rng(B * 10 + r)
    cap = 1500
    rows = np.empty((3, 4, cap), dtype=np.float32)
    rows[:, 0] = rng.standard_normal((3, cap))
    rows[:, 1] = rng.integers(-3, 4, size=(3, cap))
    rows[:, 2] = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), size=(3, cap))
    rows[:, 3] = 2.5
    for ns, nl in [(4, 16), (0, 300), (900, 0), (800, 800), (1, 1499), (3000, 0)]:
        _select_case(rows, [1, 777, 1500], B, r, ns, nl)


def test_select_many_rows_reused_workspace():
    # more work-groups than the chip holds at once (4 x 32 rows of 32K
    # positions, several work-groups per row), and one workspace reused by
    # bitmap-only calls with different budgets: each call must match the
    # list route, which the oracle checks
    bsz, H, cap = 4, 32, 32768
    lens = [32768, 30001, 16385, 4096]
    rows = _long_rows("gauss", bsz, H, cap, seed=77)
    _select_case(rows, lens, 3277, 1)
    shape = tbl.make_shape(bsz, H, H, H, 64, 16, cap, torch.float32)
    sc = torch.from_numpy(rows).cuda()
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws = tbl.alloc_workspace(shape, tbl.make_params(4000, 2))
    for B, r in [(3277, 1), (1000, 0), (4000, 2), (3277, 1)]:
        params = tbl.make_params(B, r)
        sel = torch.full((bsz, H, tbl.selection_capacity(shape, params)), -1, dtype=torch.int32,
                         device="cuda")
        cnt = torch.full((bsz, H), -1, dtype=torch.int32, device="cuda")
        bits = torch.full((bsz, H, tbl.bitmap_words(shape)), -1, dtype=torch.int32, device="cuda")
        tbl.select(shape, params, sc, ctx, sel, cnt, ws, sel_bits=bits)
        cnt2 = torch.full_like(cnt, -1)
        bits2 = torch.full_like(bits, -1)
        tbl.select(shape, params, sc, ctx, None, cnt2, ws, sel_bits=bits2)
        torch.cuda.synchronize()
        assert torch.equal(cnt2, cnt) and torch.equal(bits2, bits), (B, r)
        b = 1
        got = lists_of(sel, cnt, b)
        for i in (0, 31):
            T_ref = orc.topb(rows[b, i, :lens[b]], B)
            assert got[i] == orc.expand(T_ref, lens[b], r).tolist(), (B, r, i)


def test_select_single_and_empty_contexts():
    rows = np.random.default_rng(5).standard_normal((2, 4, 64)).astype(np.float32)
    _select_case(rows, [0, 1], 3, 1)


@pytest.mark.parametrize("kw", [dict(dtype="f32", head_dim=64, d_imp=16),
                                dict(dtype="bf16", head_dim=128, d_imp=32, ctx0=5000, budget=400),
                                # rows of 513..1024 words (1024-thread selection)
                                dict(dtype="bf16", head_dim=128, d_imp=32, ctx0=20000, budget=1500),
                                # rows of at most 16 words: one key per thread in
                                # the radix passes, a ballot per word for the kept set
                                dict(dtype="bf16", head_dim=128, d_imp=32, ctx0=400),
                                dict(dtype="bf16", head_dim=128, d_imp=32, ctx0=300, n_sink=3,
                                     n_local=20, radius=2),
                                dict(dtype="f32", head_dim=64, d_imp=16, ctx0=500, budget=600)],
                         ids=["f32_radix", "bf16_sampled", "bf16_cap20001", "bf16_cap401",
                              "bf16_cap301_sink_local", "f32_cap501_budget_covers"])
def test_tie_heavy_scores_through_score_kernel(kw):
    # integer-valued projected keys and importance queries: many exact score
    # ties, decided by position on both sides (rows under 64 words take the
    # radix passes directly; longer ones first try the sample bracket)
    w = _small(**{"budget": 40, "radius": 1, "plant_per_head": 0, **kw})
    pre = synth.prefill(w)
    rng = np.random.default_rng(9)
    K = np.zeros((w.batch, w.n_kv_heads, w.ctx_cap, w.head_dim), dtype=np.float32)
    K[..., :w.d_imp] = rng.integers(-2, 3, size=K[..., :w.d_imp].shape)
    Wm = np.zeros((w.head_dim, w.d_imp), dtype=np.float32)
    Wm[np.arange(w.d_imp), np.arange(w.d_imp)] = 1.0
    qi = rng.integers(-1, 2, size=(w.batch, w.n_imp_heads, w.d_imp)).astype(np.float32)
    dt = synth.torch_dtype(w)
    pre = replace(pre, K=torch.from_numpy(K).to(dt), W=torch.from_numpy(Wm).to(dt),
                  q_imp0=torch.from_numpy(qi).to(dt),
                  k_next=torch.from_numpy(K[:, :, w.ctx0:w.ctx0 + 1].copy()).to(dt))
    dc = device_case(w, pre=pre)
    inp = synth.step_inputs(w, 0, pre)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dt, device="cuda")
    step_on_device(dc, 0, inp, out)
    for b in range(w.batch):
        st = oracle_state(w, pre, b)
        _, s32 = orc.score(qi[b].astype(np.float64), st.Kp, n=w.ctx0)
        if w.budget < w.ctx0:
            assert band_members(s32[0], w.budget).size > 1   # the case really has ties at tau
        _check_step(w, dc, st, inp, out, 0, b, w.ctx)


def test_empty_attended_set_gives_zero_rows():
    w = _small(batch=2)
    dc = device_case(w)
    q = synth.draw_q(w, 0).cuda()
    dc.cnt.zero_()
    ctx = torch.tensor([0, 1500], dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.n_q_heads, w.head_dim), 7.0, dtype=dc.K.dtype, device="cuda")
    tbl.sparse_attn(dc.shape, q, dc.K, dc.V, dc.sel, dc.cap_s, dc.cnt, None, ctx,
                    w.softmax_scale, out, dc.ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    dc.bits.zero_()
    out.fill_(7.0)
    tbl.sparse_attn(dc.shape, q, dc.K, dc.V, None, 0, None, None, ctx, w.softmax_scale, out,
                    dc.ws, sel_bits=dc.bits)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


def test_attention_ignores_list_entries_beyond_context():
    # a stored list may hold positions of a longer context; only [0, n) counts
    w = _small(batch=1, ctx0=999)
    dc = device_case(w)
    q = synth.draw_q(w, 0)
    lst = np.array([3, 10, 500, 998, 999], dtype=np.int32)
    dc.sel.fill_(0)
    dc.sel[0, :, :lst.size] = torch.from_numpy(lst).cuda()
    dc.cnt.fill_(lst.size)
    ctx = torch.tensor([600], dtype=torch.int32, device="cuda")
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    tbl.sparse_attn(dc.shape, q.cuda(), dc.K, dc.V, dc.sel, dc.cap_s, dc.cnt, None, ctx,
                    w.softmax_scale, out, dc.ws)
    torch.cuda.synchronize()
    K64, V64 = f64(dc.pre.K[0]), f64(dc.pre.V[0])
    o_ref, bound = oracle_attention(w, K64, V64, f64(q[0]), [[3, 10, 500]] * w.n_q_heads)
    assert_attention(f64(out[0]), o_ref, bound, w.dtype)


def test_fused_step_is_deterministic():
    # two runs give the same bits; the second keeps no list, only the bitmap
    w = LLAMA_32K
    outs = []
    for with_list in (True, False):
        dc = device_case(w)
        inp = synth.step_inputs(w, 0, dc.pre)
        out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
        step_on_device(dc, 0, inp, out, with_list=with_list)
        outs.append((out.clone(), dc.cnt.clone(), dc.bits.clone(), dc.Kp.clone(),
                     dc.keep.clone()))
        if with_list:
            assert lists_of(dc.sel, dc.cnt, 0) == bitmap_positions(dc.bits, 0, w.ctx)
    for a, b in zip(*outs):
        assert torch.equal(a, b)
