"""Oracle work of the full-workload GPU tests, run in worker processes.

Each job draws one sequence of a workload from the seeded generator, runs the
fp64 oracle on it, and returns the sequence's inputs (as raw bf16/fp32 bits,
so the GPU side uploads exactly these values) with everything the comparison
needs: the oracle's stored selections and outputs, the fp64 scores of every
refresh, the derived bf16 bounds and the projected keys.  CPU only: the jobs
never touch the GPU."""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc
from query_aware_kv_amd import synth
from query_aware_kv_amd.workloads import Workload
from tests.gpu_cases import attended_sets, f64, odtype, oracle_attention, oracle_state


def _bits(t: torch.Tensor) -> np.ndarray:
    return (t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16
            else t.contiguous().view(torch.int32)).numpy().copy()


def from_bits(a: np.ndarray, w: Workload) -> torch.Tensor:
    t = torch.from_numpy(a)
    return t.view(torch.bfloat16) if w.dtype == "bf16" else t.view(torch.float32)


def sequence_job(w: Workload, layer: int, b: int) -> dict:
    """Every decode step of sequence b of one layer of workload w (prefill
    from the generator, step inputs per step, refresh every w.interval
    steps)."""
    pre = synth.prefill(w, layer, items=[b])
    st = oracle_state(w, pre, 0)
    res = {"b": b, "K": _bits(pre.K[0]), "V": _bits(pre.V[0]), "steps": []}
    if pre.k_next is not None:
        res["k_next"] = _bits(pre.k_next[0])
        res["v_next"] = _bits(pre.v_next[0])
    Wd = f64(pre.W)
    for s in range(w.steps):
        inp = synth.step_inputs(w, s, pre, layer, items=[b])
        n = w.ctx0 + s + 1
        out = orc.decode_step(st, Wd, f64(inp.q[0]),
                              f64(inp.q_imp[0]) if inp.q_imp is not None else None, n,
                              odtype(w), inp.refresh, w.softmax_scale,
                              k_new=f64(inp.k_new[0]), v_new=f64(inp.v_new[0]))
        o, bound = oracle_attention(w, st.K, st.V, f64(inp.q[0]), attended_sets(w, st, n))
        step = {"n": n, "out": out, "o": o, "bound": bound, "keep": int(st.keep_from[0])}
        if inp.refresh:
            step["sel"] = [st.sel[i, :st.cnt[i]].copy() for i in range(w.n_imp_heads)]
            step["s64"] = orc.score(f64(inp.q_imp[0]), st.Kp, n=n)[0]
        res["steps"].append(step)
    res["Kp"] = st.Kp[:, :w.ctx_last].astype(np.float32)
    return res
