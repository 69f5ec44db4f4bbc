"""Seeded synthetic inputs for the sparse-decode path.

This module draws input tensors only; it holds none of the method's
arithmetic and is shared, as data, by the GPU tests, the oracle checks and the
benchmark.  Every tensor comes from its own numpy PCG64 stream keyed by
``[seed, tensor_id, layer, batch_item, slot]``:

    tensor_id 0 K, 1 V, 2 q, 3 q_imp, 4 W, 5 planted positions,
              6 producer hidden states, 7 MLP W1, 8 MLP W2
    slot      0 for the prefill, s + 1 for decode step s (q, q_imp, new K/V),
              the importance-head index for planted positions

Values are N(0, 1) drawn in fp32 (W is scaled by 1/sqrt(head_dim)) and then
rounded to the workload dtype (round-to-nearest-even).  Tensors are returned
on the CPU in the workload dtype; tests and the benchmark move them to the GPU
and hand the same values, upcast to float64, to the oracle.

Heavy-token planting.  A planted token t of importance head i (KV head g)
gets its key row shifted in K space: K[g][t] += shift * u_i with
u_i = W q_imp_i / |W q_imp_i|.  Because the importance score of a key row k is
k . (W q_imp_i) up to rounding, this raises head i's score of t by ``shift``
standard deviations of its unplanted score (std = |W q_imp_i| for N(0, I) keys).
The shift is computed in float64 from the dtype-rounded W and q_imp and the
row is then rounded to the dtype.  Shifts of several heads on one row add.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from .workloads import Workload

K_ID, V_ID, Q_ID, QIMP_ID, W_ID, PLANT_ID = 0, 1, 2, 3, 4, 5
H_ID, W1_ID, W2_ID = 6, 7, 8


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _rng(w: Workload, tensor_id: int, layer: int, b: int, slot: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, tensor_id, layer, b, slot])


def _normal(w: Workload, shape, tensor_id, layer, b, slot) -> np.ndarray:
    return _rng(w, tensor_id, layer, b, slot).standard_normal(shape, dtype=np.float32)


def _to_dtype(a: np.ndarray, w: Workload) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(w))


def draw_w(w: Workload, layer: int = 0) -> torch.Tensor:
    """Key-projection matrix W [D][d], N(0, 1/D)."""
    z = _normal(w, (w.head_dim, w.d_imp), W_ID, layer, 0, 0)
    return _to_dtype(z.astype(np.float64) / np.sqrt(w.head_dim), w)


def _items(w: Workload, items) -> list[int]:
    return list(range(w.batch)) if items is None else [int(b) for b in items]


def draw_q_imp(w: Workload, step: int, layer: int = 0, items=None) -> torch.Tensor:
    """Importance queries of decode step ``step``: [b][H_imp][d] (the batch
    items ``items``, default all)."""
    z = np.stack([_normal(w, (w.n_imp_heads, w.d_imp), QIMP_ID, layer, b, step + 1)
                  for b in _items(w, items)])
    return _to_dtype(z, w)


def draw_q(w: Workload, step: int, layer: int = 0, items=None) -> torch.Tensor:
    """Attention queries of decode step ``step``: [b][Hq][D]."""
    z = np.stack([_normal(w, (w.n_q_heads, w.head_dim), Q_ID, layer, b, step + 1)
                  for b in _items(w, items)])
    return _to_dtype(z, w)


def planted_positions(w: Workload, b: int, i: int, n: int, layer: int = 0) -> np.ndarray:
    """Sorted planted token positions of importance head i in [0, n)."""
    rng = _rng(w, PLANT_ID, layer, b, i)
    if w.plant_runs > 0:
        L = w.plant_run_len
        starts: list[int] = []
        while len(starts) < w.plant_runs:
            s = int(rng.integers(0, n - L + 1))
            if all(s + L <= t or t + L <= s for t in starts):
                starts.append(s)
        return np.sort(np.concatenate([np.arange(s, s + L) for s in starts]))
    if w.plant_per_head > 0:
        return np.sort(rng.choice(n, size=w.plant_per_head, replace=False))
    return np.zeros(0, dtype=np.int64)


@dataclass
class Prefill:
    """Cache contents before the first decode step (CPU tensors, workload dtype).

    K, V [b][Hkv][cap][D]: rows [0, ctx0) hold the prefilled tokens, the rest
    are zero.  For single-step workloads the token that step 0 appends is
    returned separately in k_next / v_next [b][Hkv][1][D] (it belongs to the
    prefill draw, so planting can land on it)."""
    K: torch.Tensor
    V: torch.Tensor
    W: torch.Tensor
    q_imp0: torch.Tensor
    k_next: torch.Tensor | None
    v_next: torch.Tensor | None
    planted: dict = field(default_factory=dict)


def prefill(w: Workload, layer: int = 0, items=None) -> Prefill:
    Hkv, D, cap = w.n_kv_heads, w.head_dim, w.ctx_cap
    single = w.steps == 1
    rows = w.ctx0 + 1 if single else w.ctx0
    its = _items(w, items)
    W = draw_w(w, layer)
    q_imp0 = draw_q_imp(w, 0, layer, its)
    W64 = W.to(torch.float64).numpy()
    qi64 = q_imp0.to(torch.float64).numpy()
    K = torch.zeros((len(its), Hkv, cap, D), dtype=torch_dtype(w))
    V = torch.zeros_like(K)
    planted = {}
    for j, b in enumerate(its):
        k32 = _normal(w, (Hkv, rows, D), K_ID, layer, b, 0)
        v32 = _normal(w, (Hkv, rows, D), V_ID, layer, b, 0)
        shifts: dict[tuple[int, int], np.ndarray] = {}
        for i in range(w.n_imp_heads):
            pos = planted_positions(w, b, i, rows, layer)
            planted[(b, i)] = pos
            if pos.size == 0:
                continue
            g = i * Hkv // w.n_imp_heads
            u = W64 @ qi64[j, i]
            u = u / np.linalg.norm(u)
            for t in pos.tolist():
                key = (g, t)
                shifts[key] = shifts.get(key, 0.0) + w.plant_shift * u
        for (g, t), delta in shifts.items():
            k32[g, t] = (k32[g, t].astype(np.float64) + delta).astype(np.float32)
        K[j, :, :rows] = _to_dtype(k32, w)
        V[j, :, :rows] = _to_dtype(v32, w)
    k_next = v_next = None
    if single:
        k_next = K[:, :, w.ctx0:w.ctx0 + 1].clone()
        v_next = V[:, :, w.ctx0:w.ctx0 + 1].clone()
        K[:, :, w.ctx0:] = 0
        V[:, :, w.ctx0:] = 0
    return Prefill(K=K, V=V, W=W, q_imp0=q_imp0, k_next=k_next, v_next=v_next,
                   planted=planted)


@dataclass
class StepInputs:
    k_new: torch.Tensor          # [b][Hkv][1][D]
    v_new: torch.Tensor          # [b][Hkv][1][D]
    q: torch.Tensor              # [b][Hq][D]
    q_imp: torch.Tensor | None   # [b][H_imp][d] on refresh steps, else None
    refresh: bool


def step_inputs(w: Workload, s: int, pre: Prefill, layer: int = 0, items=None) -> StepInputs:
    """Inputs of decode step s (token appended at position ctx0 + s) for the
    batch items of ``pre`` (``items``, default all)."""
    refresh = s % w.interval == 0
    its = _items(w, items)
    if w.steps == 1:
        k_new, v_new = pre.k_next, pre.v_next
    else:
        k_new = torch.stack([_to_dtype(_normal(w, (w.n_kv_heads, 1, w.head_dim), K_ID, layer,
                                               b, s + 1), w) for b in its])
        v_new = torch.stack([_to_dtype(_normal(w, (w.n_kv_heads, 1, w.head_dim), V_ID, layer,
                                               b, s + 1), w) for b in its])
    q = draw_q(w, s, layer, its)
    q_imp = (pre.q_imp0 if s == 0 else draw_q_imp(w, s, layer, its)) if refresh else None
    return StepInputs(k_new=k_new, v_new=v_new, q=q, q_imp=q_imp, refresh=refresh)


@dataclass
class MlpInputs:
    h: torch.Tensor   # [M][E] producer hidden states, N(0, 1)
    w1: torch.Tensor  # [F][E], N(0, 1/E)
    w2: torch.Tensor  # [N][F], N(0, 1/F)


def mlp_inputs(M: int, E: int, F: int, N: int, dtype: torch.dtype, seed: int,
               step: int = 0) -> MlpInputs:
    """Random-init weights and hidden states of the importance-query MLP
    (no trained weights exist here), rounded to the dtype."""
    def draw(shape, tid, scale, slot=0):
        z = np.random.default_rng([seed, tid, 0, 0, slot]).standard_normal(shape, dtype=np.float32)
        a = z.astype(np.float64) * scale
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)
    return MlpInputs(h=draw((M, E), H_ID, 1.0, step + 1), w1=draw((F, E), W1_ID, 1 / np.sqrt(E)),
                     w2=draw((N, F), W2_ID, 1 / np.sqrt(F)))
