"""Host-side checks of the seeded input generator (no GPU)."""
import numpy as np
import torch

from query_aware_kv_amd import synth
from query_aware_kv_amd.workloads import ALL, INTERVAL_16K, LLAMA_32K, TINY_F32, Workload


def _small(w: Workload, **kw) -> Workload:
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


def test_workload_table():
    names = [w.name for w in ALL]
    assert len(set(names)) == 5
    assert LLAMA_32K.budget == 3277 and LLAMA_32K.ctx == 32768
    assert INTERVAL_16K.ctx_cap == 16448 and INTERVAL_16K.budget == 1639
    for w in ALL:
        assert w.n_q_heads % w.n_kv_heads == 0
        assert w.n_imp_heads % w.n_kv_heads == 0 and w.n_q_heads % w.n_imp_heads == 0


def test_generator_is_deterministic_and_keyed():
    w = TINY_F32
    a = synth.prefill(w)
    b = synth.prefill(w)
    assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V) and torch.equal(a.W, b.W)
    c = synth.prefill(w, layer=1)
    assert not torch.equal(a.K, c.K)
    s0 = synth.step_inputs(w, 0, a)
    assert torch.equal(s0.q_imp, a.q_imp0) and s0.refresh
    assert a.K.shape == (1, 4, 512, 64) and a.K.dtype == torch.float32
    assert a.k_next.shape == (1, 4, 1, 64)
    # the row the step appends is not in the prefilled cache
    assert torch.count_nonzero(a.K[:, :, 511]) == 0


def test_bf16_workload_dtype_and_interval_steps():
    w = _small(INTERVAL_16K, ctx0=64, steps=10, budget=6, batch=2)
    pre = synth.prefill(w)
    assert pre.K.dtype == torch.bfloat16 and pre.K.shape == (2, 8, 74, 128)
    assert torch.count_nonzero(pre.K[:, :, 64:]) == 0
    refresh = [synth.step_inputs(w, s, pre).refresh for s in range(10)]
    assert refresh == [s % 8 == 0 for s in range(10)]
    s1 = synth.step_inputs(w, 1, pre)
    assert s1.q_imp is None and s1.k_new.shape == (2, 8, 1, 128)


def test_planting_shifts_score_by_requested_std():
    w = TINY_F32
    pre = synth.prefill(w)
    W = pre.W.double().numpy()
    qi = pre.q_imp0.double().numpy()
    K = torch.cat([pre.K[:, :, :w.ctx0], pre.k_next], dim=2).double().numpy()
    # the unplanted draw, regenerated from the same stream
    k0 = synth._normal(w, (w.n_kv_heads, w.ctx, w.head_dim), synth.K_ID, 0, 0, 0).astype(np.float64)
    for i in range(w.n_imp_heads):
        g = i * w.n_kv_heads // w.n_imp_heads
        wi = W @ qi[0, i]
        pos = pre.planted[(0, i)]
        assert pos.size == 8
        shift = (K[0, g, pos] - k0[g, pos]) @ wi / np.linalg.norm(wi)
        # fp32 rounding of the shifted rows only; no other head plants in this group
        np.testing.assert_allclose(shift, w.plant_shift, rtol=1e-5)


def test_planted_runs_are_disjoint_runs():
    w = _small(LLAMA_32K, plant_per_head=0, plant_runs=16, plant_run_len=32)
    pos = synth.planted_positions(w, 0, 3, 4096)
    assert pos.size == 16 * 32 and np.unique(pos).size == pos.size
    starts = pos[np.r_[True, np.diff(pos) != 1]]
    assert starts.size <= 16 and pos.max() < 4096
