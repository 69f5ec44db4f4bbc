"""The batched and prediction-interval workloads in full, through the C ABI:
every sequence of every layer of the batch-16 / 32-layer / 8K workload, and
every sequence of every step of the 64-step interval workload.

The oracle runs in worker processes (one sequence per job, CPU only), which
also draw the sequences' inputs; the GPU side uploads those exact bits.
Selections are compared two ways: bit for bit with the oracle's fp32-chain
selection, and against the ranking of the exact (fp64) scores outside the
1e-6 relative band around the B-th score.  Outputs are held to the contract
bars and, in bf16, to the derived per-element bound."""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

from query_aware_kv_amd import synth
from query_aware_kv_amd.workloads import BATCHED_8K, INTERVAL_16K
from tests.gpu_cases import (assert_attention, assert_fp64_selection, device_case, f64,
                             lists_of, need_gpu, step_on_device)
from tests.oracle_jobs import from_bits, sequence_job

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(scope="module")
def pool():
    n = max(1, min(16, os.cpu_count() or 1))
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        yield ex


def _prefill_from_jobs(w, layer, res):
    K = torch.stack([from_bits(r["K"], w) for r in res])
    V = torch.stack([from_bits(r["V"], w) for r in res])
    k_next = v_next = None
    if "k_next" in res[0]:
        k_next = torch.stack([from_bits(r["k_next"], w) for r in res])
        v_next = torch.stack([from_bits(r["v_next"], w) for r in res])
    return synth.Prefill(K=K, V=V, W=synth.draw_w(w, layer), q_imp0=synth.draw_q_imp(w, 0, layer),
                         k_next=k_next, v_next=v_next)


def _check_refresh(w, dc, res, s, what):
    bands = 0
    for r in res:
        b = r["b"]
        st = r["steps"][s]
        got = lists_of(dc.sel, dc.cnt, b)
        for i in range(w.n_imp_heads):
            assert got[i] == st["sel"][i].tolist(), (what, s, b, i)
            bands += assert_fp64_selection(got[i], st["s64"][i], st["n"], w.budget, w.radius,
                                           w.n_sink, w.n_local, what=(what, s, b, i))
    return bands


def _check_outputs(w, out, res, s, what):
    worst = 0.0
    for r in res:
        st = r["steps"][s]
        got = f64(out[r["b"]])
        # (the oracle's step and the per-head recomputation over its stored
        # sets are the same sums)
        np.testing.assert_array_equal(st["out"], st["o"])
        worst = max(worst, assert_attention(got, st["o"], st["bound"], w.dtype,
                                            what=(what, s, r["b"])))
    return worst


@pytest.mark.parametrize("layer", range(BATCHED_8K.layers))
def test_batched_8k_every_sequence(layer, pool):
    # one layer of the batch-16 / 8K / radius-1 workload at full shape, all
    # 16 sequences against the oracle, the projected-key cache in full
    w = BATCHED_8K
    res = list(pool.map(sequence_job, [w] * w.batch, [layer] * w.batch, range(w.batch)))
    pre = _prefill_from_jobs(w, layer, res)
    dc = device_case(w, pre=pre)
    inp = synth.step_inputs(w, 0, pre, layer)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    step_on_device(dc, 0, inp, out)
    _check_refresh(w, dc, res, 0, ("layer", layer))
    _check_outputs(w, out, res, 0, ("layer", layer))
    keep = dc.keep.cpu().numpy()
    for r in res:
        assert int(keep[r["b"]]) == r["steps"][0]["keep"] == w.ctx0
        np.testing.assert_array_equal(dc.Kp[r["b"]][:, :w.ctx].float().cpu().numpy(),
                                      r["Kp"][:, :w.ctx])
    cnt = dc.cnt.cpu().numpy()
    assert cnt.max() <= 3 * w.budget and cnt.min() >= w.budget


def test_interval_every_sequence_every_step(pool):
    # 64 steps, selection recomputed every 8 steps and reused in between,
    # radius 2, new tokens always kept: all four sequences at every step
    w = INTERVAL_16K
    res = list(pool.map(sequence_job, [w] * w.batch, [0] * w.batch, range(w.batch)))
    pre = _prefill_from_jobs(w, 0, res)
    dc = device_case(w, pre=pre)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=dc.K.dtype, device="cuda")
    bands = 0
    worst = 0.0
    for s in range(w.steps):
        inp = synth.step_inputs(w, s, pre)
        step_on_device(dc, s, inp, out)
        if inp.refresh:
            bands += _check_refresh(w, dc, res, s, "interval")
        worst = max(worst, _check_outputs(w, out, res, s, "interval"))
        keep = dc.keep.cpu().numpy()
        for r in res:
            assert int(keep[r["b"]]) == r["steps"][s]["keep"] == (
                w.ctx0 + (s // w.interval) * w.interval), (s, r["b"])
    for r in res:
        # every projected key, the 64 appended rows included
        np.testing.assert_array_equal(dc.Kp[r["b"]].float().cpu().numpy(), r["Kp"])
    print(f"interval: band members {bands}, worst error/bound {worst:.3f}")
