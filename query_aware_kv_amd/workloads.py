"""The five synthetic workloads of the sparse-decode path.

Each workload fixes the shapes, the budget, the neighbor radius, the
prediction interval and the heavy-token planting recipe.  Sizes follow the
shapes the TokenButler pages evaluate on (Llama-3-8B-class attention: 32 query
heads, 8 KV heads, head_dim 128) at several context lengths; the pages print no
speed workload of their own, so these synthetic shapes stand in for it.

Context convention: ``ctx`` is the context length *after* the decode step's
append.  A single-step workload prefills ``ctx - 1`` tokens and the step
appends the last one.  The interval workload prefills ``ctx0`` tokens and
appends one token per step, so step s runs at context ``ctx0 + s + 1``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    layers: int
    n_q_heads: int
    n_kv_heads: int
    n_imp_heads: int
    head_dim: int
    d_imp: int
    dtype: str            # "f32" or "bf16"
    ctx0: int             # tokens present before the first step
    steps: int            # decode steps (one token appended per step)
    budget: int           # B: tokens kept per importance head
    radius: int           # r: neighbor-fetch radius
    interval: int         # P: selection recomputed when step % P == 0
    plant_per_head: int   # planted heavy tokens per importance head (scattered)
    plant_runs: int       # or: contiguous runs per head ...
    plant_run_len: int    # ... of this length
    plant_shift: float    # score shift of a planted token, in score std units
    seed: int
    n_sink: int = 0       # first tokens always kept (sink buffer)
    n_local: int = 0      # last tokens always kept (local window)

    @property
    def ctx(self) -> int:
        """Context at the first step (after its append)."""
        return self.ctx0 + 1

    @property
    def ctx_last(self) -> int:
        return self.ctx0 + self.steps

    @property
    def ctx_cap(self) -> int:
        return self.ctx0 + self.steps

    @property
    def cap_s(self) -> int:
        return min(self.ctx_cap, (2 * self.radius + 1) * self.budget + self.n_sink + self.n_local)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def _budget(frac: float, ctx: int) -> int:
    return int(math.ceil(frac * ctx - 1e-9))


# 1: tiny fp32 single step.
TINY_F32 = Workload("tiny_f32_ctx512", batch=1, layers=1, n_q_heads=4, n_kv_heads=4,
                    n_imp_heads=4, head_dim=64, d_imp=16, dtype="f32", ctx0=511, steps=1,
                    budget=64, radius=0, interval=1, plant_per_head=8, plant_runs=0,
                    plant_run_len=0, plant_shift=4.0, seed=1)

# 2: Llama-3-8B-shaped one-layer step at 32K context, budget 10 %.
LLAMA_32K = Workload("llama3_8b_ctx32k", batch=1, layers=1, n_q_heads=32, n_kv_heads=8,
                     n_imp_heads=32, head_dim=128, d_imp=32, dtype="bf16", ctx0=32767,
                     steps=1, budget=_budget(0.10, 32768), radius=0, interval=1,
                     plant_per_head=round(0.01 * 32768), plant_runs=0, plant_run_len=0,
                     plant_shift=3.0, seed=2)

# 3: batch 16, 32 layers, 8K context, budget 12.5 %, radius 1, 2 % planted.
BATCHED_8K = Workload("batched_b16_l32_ctx8k", batch=16, layers=32, n_q_heads=32,
                      n_kv_heads=8, n_imp_heads=32, head_dim=128, d_imp=32, dtype="bf16",
                      ctx0=8191, steps=1, budget=_budget(0.125, 8192), radius=1, interval=1,
                      plant_per_head=round(0.02 * 8192), plant_runs=0, plant_run_len=0,
                      plant_shift=3.0, seed=3)

# 4: prediction interval 8 over 64 steps from 16K context, radius 2.  The
#    budget is not stated for this run; 10 % of the starting context is used.
INTERVAL_16K = Workload("interval_b4_ctx16k_p8", batch=4, layers=1, n_q_heads=32,
                        n_kv_heads=8, n_imp_heads=32, head_dim=128, d_imp=32, dtype="bf16",
                        ctx0=16384, steps=64, budget=_budget(0.10, 16384), radius=2,
                        interval=8, plant_per_head=0, plant_runs=0, plant_run_len=0,
                        plant_shift=0.0, seed=4)

# 5: 128K context, budget 4096, radius 1, planted tokens in 16 runs of 32.
LONG_128K = Workload("long_ctx128k", batch=1, layers=1, n_q_heads=32, n_kv_heads=8,
                     n_imp_heads=32, head_dim=128, d_imp=32, dtype="bf16", ctx0=131071,
                     steps=1, budget=4096, radius=1, interval=1, plant_per_head=0,
                     plant_runs=16, plant_run_len=32, plant_shift=3.0, seed=5)

# Offloading: 256K context with the K/V caches in pinned host memory (the
# pages report the offloaded regime at 256K+ tokens), budget 10 %, no planting.
OFFLOAD_256K = Workload("offload_ctx256k", batch=1, layers=1, n_q_heads=32, n_kv_heads=8,
                        n_imp_heads=32, head_dim=128, d_imp=32, dtype="bf16", ctx0=262143,
                        steps=1, budget=_budget(0.10, 262144), radius=0, interval=1,
                        plant_per_head=0, plant_runs=0, plant_run_len=0, plant_shift=0.0,
                        seed=6)

ALL = [TINY_F32, LLAMA_32K, BATCHED_8K, INTERVAL_16K, LONG_128K]
BY_NAME = {w.name: w for w in ALL}
