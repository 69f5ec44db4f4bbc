"""tb_decode_step_noalloc (the entry point for callers that cannot allocate)
against tb_decode_step on identical copies of the same state: the same
kernels, so every output, cache row and selection must agree bit for bit.
Two shapes in a row on the one device scratch, the second smaller, each with
a refresh step and a reuse step."""
from dataclasses import replace

import pytest
import torch

from query_aware_kv_amd import synth
from query_aware_kv_amd import tokenbutler as tbl
from query_aware_kv_amd.workloads import LLAMA_32K, Workload
from tests.gpu_cases import device_case, need_gpu

pytestmark = pytest.mark.gpu


def _pair(w: Workload):
    need_gpu()
    a = device_case(w)
    b = device_case(w, pre=a.pre)
    assert tbl.workspace_bytes(a.shape, a.params) <= tbl.NOALLOC_SCRATCH_BYTES
    outs = [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=a.K.dtype, device="cuda")
            for _ in range(2)]
    for s in range(w.steps):
        inp = synth.step_inputs(w, s, a.pre)
        ctx = torch.full((w.batch,), w.ctx0 + s + 1, dtype=torch.int32, device="cuda")
        args = []
        for dc, out in zip((a, b), outs):
            args.append(tbl.step_args(
                dc.shape, dc.params, q=inp.q.cuda(),
                q_imp=inp.q_imp.cuda() if inp.q_imp is not None else None,
                k_new=inp.k_new.cuda(), v_new=inp.v_new.cuda(), refresh=inp.refresh, w=dc.W,
                k_cache=dc.K, v_cache=dc.V, kp_cache=dc.Kp, ctx_len=ctx,
                softmax_scale=w.softmax_scale, sel_idx=dc.sel, sel_count=dc.cnt,
                sel_bits=dc.bits, keep_from=dc.keep, out=out))
        tbl.decode_step(a.shape, a.params, args[0], a.ws)
        tbl.decode_step_noalloc(b.shape, b.params, args[1])
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), (w.name, s)
        for x, y in ((a.cnt, b.cnt), (a.bits, b.bits), (a.keep, b.keep), (a.sel, b.sel),
                     (a.K, b.K), (a.V, b.V), (a.Kp, b.Kp)):
            assert torch.equal(x, y), (w.name, s)


def test_noalloc_matches_workspace_entry_point_twice():
    # the 32K-context step (refresh, then a reuse step), then a smaller shape
    # on the same scratch: three sequences of ragged capacity, radius 1, a
    # sink and a local window
    big = replace(LLAMA_32K, ctx0=32766, steps=2, interval=2)
    small = Workload("small", batch=3, layers=1, n_q_heads=8, n_kv_heads=2, n_imp_heads=8,
                     head_dim=128, d_imp=32, dtype="bf16", ctx0=1995, steps=2, budget=50,
                     radius=1, interval=2, plant_per_head=5, plant_runs=0, plant_run_len=0,
                     plant_shift=3.0, seed=11, n_sink=4, n_local=64)
    _pair(big)
    _pair(small)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    need_gpu()
    shape = tbl.make_shape(64, 32, 8, 32, 128, 32, 32768, torch.bfloat16)
    params = tbl.make_params(3277, 0)
    assert tbl.workspace_bytes(shape, params) > tbl.NOALLOC_SCRATCH_BYTES
    dev = "cuda"
    z = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    zi = torch.zeros(16, dtype=torch.int32, device=dev)
    args = tbl.StepArgs()
    for f in ("q", "q_imp", "w", "k_cache", "v_cache", "kp_cache", "out"):
        setattr(args, f, z.data_ptr())
    for f in ("ctx_len", "sel_count", "sel_bits", "keep_from"):
        setattr(args, f, zi.data_ptr())
    args.softmax_scale = 0.1
    args.refresh = 1
    with pytest.raises(tbl.TokenButlerError) as e:
        tbl.decode_step_noalloc(shape, params, args)
    assert e.value.code == tbl.TB_EWORKSPACE
