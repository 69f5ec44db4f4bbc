"""Fused decode steps captured in a HIP graph (torch.cuda.graph) and replayed.

A graph of one refresh step and one reuse step (each appending a token) is
replayed several times, with eager library calls on other buffers, a
PyTorch fill of the outputs and host synchronisations between the replays.
Every replay must reproduce, bit for bit, what the same two steps give when
launched eagerly on an identical copy of the state: the same kernels run in
the same order, so nothing may depend on what a previous replay left behind
(the attention's arrival counters, which every completed call leaves at
zero, and for tb_decode_step_noalloc the scratch words that each call clears
with a kernel of its own rather than a memset node)."""
from dataclasses import replace

import pytest
import torch

from query_aware_kv_amd import synth
from query_aware_kv_amd import tokenbutler as tbl
from query_aware_kv_amd.workloads import TINY_F32, Workload
from tests.gpu_cases import device_case, need_gpu

pytestmark = pytest.mark.gpu

SMALL_BF16 = Workload("graph_bf16", batch=3, layers=1, n_q_heads=8, n_kv_heads=2,
                      n_imp_heads=8, head_dim=128, d_imp=32, dtype="bf16", ctx0=3001, steps=2,
                      budget=150, radius=1, interval=2, plant_per_head=5, plant_runs=0,
                      plant_run_len=0, plant_shift=3.0, seed=21, n_sink=4, n_local=64)
WORKLOADS = {"tiny_f32": replace(TINY_F32, steps=2, interval=2), "bf16_sink_window": SMALL_BF16}


def _step_args(dc, w, s, out):
    inp = synth.step_inputs(w, s, dc.pre)
    ctx = torch.full((w.batch,), w.ctx0 + s + 1, dtype=torch.int32, device="cuda")
    qi = inp.q_imp.cuda() if inp.q_imp is not None else None
    tensors = (ctx, inp.q.cuda(), qi, inp.k_new.cuda(), inp.v_new.cuda())
    args = tbl.step_args(dc.shape, dc.params, q=tensors[1], q_imp=qi, k_new=tensors[3],
                         v_new=tensors[4], refresh=inp.refresh, w=dc.W, k_cache=dc.K,
                         v_cache=dc.V, kp_cache=dc.Kp, ctx_len=ctx,
                         softmax_scale=w.softmax_scale, sel_idx=dc.sel, sel_count=dc.cnt,
                         sel_bits=dc.bits, keep_from=dc.keep, out=out)
    return args, inp.refresh, tensors


def _state(dc):
    return [t.clone() for t in (dc.cnt, dc.bits, dc.keep, dc.sel, dc.K, dc.V, dc.Kp)]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_graph_replays_match_eager_steps(name, noalloc):
    need_gpu()
    w = WORKLOADS[name]
    ref = device_case(w)
    cap = device_case(w, pre=ref.pre)
    other = device_case(w, pre=ref.pre)

    def call(dc, args):
        if noalloc:
            tbl.decode_step_noalloc(dc.shape, dc.params, args)
        else:
            tbl.decode_step(dc.shape, dc.params, args, dc.ws)

    def outs():
        return [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=ref.K.dtype,
                            device="cuda") for _ in range(2)]

    # eager reference: refresh step, then reuse step
    ref_out = outs()
    keep_alive = []
    for s in range(2):
        args, refresh, t = _step_args(ref, w, s, ref_out[s])
        assert refresh == (s == 0)
        keep_alive.append(t)
        call(ref, args)
    torch.cuda.synchronize()
    ref_state = _state(ref)

    # the same two steps captured once (after one eager warm-up of their own)
    cap_out = outs()
    cap_args = []
    for s in range(2):
        args, _, t = _step_args(cap, w, s, cap_out[s])
        keep_alive.append(t)
        cap_args.append(args)
    for args in cap_args:
        call(cap, args)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for args in cap_args:
            call(cap, args)
    torch.cuda.synchronize()

    other_out = outs()
    other_args = []
    for s in range(2):
        args, _, t = _step_args(other, w, s, other_out[s])
        keep_alive.append(t)
        other_args.append(args)
    for rep in range(4):
        for o in cap_out:
            o.fill_(float("nan"))
        cap.bits.zero_()
        cap.cnt.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(cap_out, ref_out):
            assert torch.equal(got, want), (name, noalloc, rep)
        for got, want in zip(_state(cap), ref_state):
            assert torch.equal(got, want), (name, noalloc, rep)
        # eager work on other buffers (the same library calls) between replays
        for args in other_args:
            call(other, args)
        torch.cuda.synchronize()
        for got, want in zip(other_out, ref_out):
            assert torch.equal(got, want), (name, noalloc, rep)
    del g
