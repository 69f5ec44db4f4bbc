"""Decode-step throughput of the sparse-decode hot path on one MI355X.

Workload: the Llama-3-8B-shaped one-layer decode step at 32K context (batch 1,
32 query / 8 KV heads, head_dim 128, d_imp 32, bf16 caches, budget 3277,
radius 0, selection recomputed every step).  One step = tb_decode_step:
append + project the new key, score every cached token, top-B select, and
attend over the selected rows.  Inputs are seeded synthetic data already
resident in HBM.  The caches are replicated R times at distinct addresses and
the steps rotate over the replicas, so the 256 MB last-level cache cannot
serve one step's reads from the previous steps.

Prints one JSON line.  Extra legs:
  roofline      the attention kernel (the step's largest HBM consumer), timed
                with HIP events on its stream over K launches, against 8 TB/s;
  configs       every workload at its own timed unit, with its HBM fraction
                and the CPU oracle's rate: the tiny fp32 step, the 32K step
                (the headline), the batch-16 decode step over 32 layers at 8K,
                the batch-4 16K run of 64 growing steps with prediction
                interval 8 (refresh and reuse steps apart), the 128K step;
  projection    the prefill projection of the 32K context (fp64 on the
                matrix cores) against the fp64 peak;
  dense_attention  the dense decode-attention kernel over the whole context at
                the same shape (the baseline of the pages' speedup claims);
  predictor_mlp the importance-query producer MLP at 1 and 16 tokens;
  offload       a 256K-context step with K/V in pinned host memory against
                dense attention over the same offloaded caches;
  cpu_baseline  the fp64 C oracle's decode step on the host (1 thread): the
                median of three bounded samples per workload.
"""
from __future__ import annotations

import argparse
import json
from dataclasses import replace
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from query_aware_kv_amd import synth  # noqa: E402
from query_aware_kv_amd import tokenbutler as tbl  # noqa: E402
from query_aware_kv_amd.workloads import (BATCHED_8K, BY_NAME, INTERVAL_16K,  # noqa: E402
                                          LLAMA_32K, LONG_128K, OFFLOAD_256K, TINY_F32)

PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6  # MI355X dense fp64 (matrix and vector)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_llama3_8b_ctx32k_traffic.json")
METRIC = "sparse decode steps/sec at 32K ctx (Llama-3-8B shape); achieved HBM GB/s vs peak"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def unique_rows(bits, w, ctx: int) -> tuple[int, int]:
    """(unique K/V rows over the KV groups, logical rows over the query heads)
    of one sequence, counted from the library's own selection bitmap; the
    always kept appended token is included."""
    words = bits[0].cpu().numpy().astype(np.uint32)
    members = np.unpackbits(words.view(np.uint8), axis=-1, bitorder="little")[:, :ctx]
    members[:, ctx - 1] = 1
    G = w.n_q_heads // w.n_kv_heads
    uniq = 0
    logical = 0
    for g in range(w.n_kv_heads):
        heads = [h * w.n_imp_heads // w.n_q_heads for h in range(g * G, (g + 1) * G)]
        logical += int(members[heads].sum())
        uniq += int(members[sorted(set(heads))].any(axis=0).sum())
    return uniq, logical


def measured_traffic() -> float | None:
    """HBM bytes per attention launch from the committed rocprofv3 counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for
    a plain copy of known size), or None when the kernel sources changed
    after the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        h = hashlib.sha256()
        for rel in t["source_files"]:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != t["source_sha256"]:
            return None
        return (t["fetch_kib_per_dispatch"] * t["fetch_scale"]
                + t["write_kib_per_dispatch"] * t["write_scale"]) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def offload_leg(steps: int) -> dict:
    """The 256K-context step with K and V in pinned host memory (read over
    the host link) against dense attention over the same offloaded caches.
    Host-link bytes: the unique gathered rows (sparse) or every row (dense)."""
    w = OFFLOAD_256K
    dev = "cuda:0"
    log(f"bench: offload leg, generating {w.name}")
    pre = synth.prefill(w)
    inp = synth.step_inputs(w, 0, pre)
    shape = tbl.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.n_imp_heads, w.head_dim,
                           w.d_imp, w.ctx_cap, synth.torch_dtype(w))
    params = tbl.make_params(w.budget, w.radius, w.n_sink, w.n_local)
    Kh, Vh = pre.K.pin_memory(), pre.V.pin_memory()
    del pre
    W = synth.draw_w(w).to(dev)
    Kp = torch.zeros((w.batch, w.n_kv_heads, w.ctx_cap, w.d_imp), dtype=Kh.dtype, device=dev)
    tbl.project_keys(shape, Kh, W, torch.zeros(w.batch, dtype=torch.int32, device=dev), w.ctx0,
                     Kp)
    ws = tbl.alloc_workspace(shape, params, dev)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device=dev)
    q, qi = inp.q.to(dev), inp.q_imp.to(dev)
    kn, vn = inp.k_new.to(dev), inp.v_new.to(dev)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=q.dtype, device=dev)
    cnt = torch.zeros((w.batch, w.n_imp_heads), dtype=torch.int32, device=dev)
    bits = torch.zeros((w.batch, w.n_imp_heads, tbl.bitmap_words(shape)), dtype=torch.int32,
                       device=dev)
    keep = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    args = tbl.step_args(shape, params, q=q, q_imp=qi, k_new=kn, v_new=vn, refresh=True, w=W,
                         k_cache=Kh, v_cache=Vh, kp_cache=Kp, ctx_len=ctx,
                         softmax_scale=w.softmax_scale, sel_idx=None, sel_count=cnt,
                         sel_bits=bits, keep_from=keep, out=out)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, k):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    ms_step = timed(lambda: tbl.decode_step(shape, params, args, ws), steps)
    ms_reuse = timed(lambda: tbl.sparse_attn(shape, q, Kh, Vh, None, 0, None, keep, ctx,
                                             w.softmax_scale, out, ws, sel_bits=bits), steps)
    ms_dense = timed(lambda: tbl.dense_attn(shape, q, Kh, Vh, ctx, w.softmax_scale, out, ws),
                     max(2, steps // 4))
    uniq, _ = unique_rows(bits, w, w.ctx)
    row = w.head_dim * w.elt_bytes
    sparse_bytes, dense_bytes = uniq * 2 * row, w.ctx * w.n_kv_heads * 2 * row
    res = {"workload": w.name, "ctx": w.ctx, "budget": w.budget, "caches": "pinned host memory",
           "step_ms": ms_step, "reuse_step_ms": ms_reuse, "dense_ms": ms_dense,
           "speedup_vs_dense": ms_dense / ms_step,
           "reuse_speedup_vs_dense": ms_dense / ms_reuse,
           "step_host_link_GBs": sparse_bytes / (ms_step * 1e-3) / 1e9,
           "dense_host_link_GBs": dense_bytes / (ms_dense * 1e-3) / 1e9,
           "gathered_bytes": sparse_bytes, "dense_bytes": dense_bytes}
    log(f"bench: offload 256K: step {ms_step:.2f} ms (reuse {ms_reuse:.2f} ms), dense "
        f"{ms_dense:.2f} ms -> {ms_dense / ms_step:.2f}x; host link "
        f"{res['step_host_link_GBs']:.1f} / {res['dense_host_link_GBs']:.1f} GB/s")
    return res


def _seq_unique(bits, keep, w, ctx: int, b: int) -> int:
    """Unique K/V rows attended by sequence b over its KV groups: bitmap
    members plus the rows [keep_from, ctx) that are always kept."""
    words = bits[b].cpu().numpy().astype(np.uint32)
    members = np.unpackbits(words.view(np.uint8), axis=-1, bitorder="little")[:, :ctx]
    members[:, max(0, min(int(keep[b]), ctx)):ctx] = 1
    members[:, ctx - 1] = 1
    G = w.n_q_heads // w.n_kv_heads
    uniq = 0
    for g in range(w.n_kv_heads):
        heads = sorted({h * w.n_imp_heads // w.n_q_heads for h in range(g * G, (g + 1) * G)})
        uniq += int(members[heads].any(axis=0).sum())
    return uniq


class _Timer:
    """HIP-event timing on torch's current stream."""

    def __init__(self):
        self.stream = torch.cuda.current_stream()
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def ms(self, fn, n: int) -> float:
        torch.cuda.synchronize()
        self.e0.record(self.stream)
        for i in range(n):
            fn(i)
        self.e1.record(self.stream)
        torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1) / n

    def graph_ms(self, fn, n_calls: int, replays: int, check) -> float:
        """Capture fn(0..n_calls-1) once, check two replays, time `replays`
        replays; returns ms per call."""
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n_calls):
                fn(i)
        for _ in range(2):
            g.replay()
            torch.cuda.synchronize()
            check()
        ms = self.ms(lambda i: g.replay(), replays)
        del g
        return ms / n_calls


def _device_case(w, dev, n_layers: int = 1, rotate: int = 0, max_bytes: int = 1 << 30,
                 max_reps: int = 64):
    """Prefilled caches of workload w on the device.  With n_layers > 1 each
    layer's caches are the first draw rotated along the token axis by
    rotate * layer positions (the same statistics at other addresses);
    otherwise the caches are replicated so that the replicas together exceed
    max_bytes and the 256 MB MALL cannot carry rows from launch to launch."""
    pre = synth.prefill(w)
    shape = tbl.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.n_imp_heads, w.head_dim,
                           w.d_imp, w.ctx_cap, synth.torch_dtype(w))
    params = tbl.make_params(w.budget, w.radius, w.n_sink, w.n_local)
    K0, V0, W = pre.K.to(dev), pre.V.to(dev), pre.W.to(dev)
    Kp0 = torch.zeros((w.batch, w.n_kv_heads, w.ctx_cap, w.d_imp), dtype=K0.dtype, device=dev)
    tbl.project_keys(shape, K0, W, torch.zeros(w.batch, dtype=torch.int32, device=dev), w.ctx0,
                     Kp0)
    per = (K0.numel() + V0.numel() + Kp0.numel()) * K0.element_size()
    n = n_layers if n_layers > 1 else min(max_reps, max(2, -(-max_bytes // per)))
    sets = []
    for i in range(n):
        if n_layers > 1:
            sh = (rotate * i) % w.ctx0
            K, V, Kp = (torch.zeros_like(t) for t in (K0, V0, Kp0))
            for dst, src in ((K, K0), (V, V0), (Kp, Kp0)):
                dst[:, :, :w.ctx0] = torch.roll(src[:, :, :w.ctx0], sh, dims=2)
        else:
            K, V, Kp = K0.clone(), V0.clone(), Kp0.clone()
        sets.append(dict(
            K=K, V=V, Kp=Kp,
            cnt=torch.zeros((w.batch, w.n_imp_heads), dtype=torch.int32, device=dev),
            bits=torch.zeros((w.batch, w.n_imp_heads, tbl.bitmap_words(shape)),
                             dtype=torch.int32, device=dev),
            keep=torch.zeros(w.batch, dtype=torch.int32, device=dev)))
    del K0, V0, Kp0
    return pre, shape, params, W, sets


def _bytes_of(w, sets, ctx: int, with_kp: bool = True) -> int:
    """Algorithmic bytes of one fused step over every set: projected keys of
    the context (refresh steps) plus unique gathered K/V rows."""
    row = w.head_dim * w.elt_bytes
    total = 0
    for r in sets:
        keep = r["keep"].cpu().numpy()
        uniq = sum(_seq_unique(r["bits"], keep, w, ctx, b) for b in range(w.batch))
        total += uniq * 2 * row
        if with_kp:
            total += w.batch * w.n_kv_heads * ctx * w.d_imp * w.elt_bytes
    return total


def single_step_leg(w, launches: int) -> dict:
    """A single-step workload (one layer, one fused refresh step): eager
    launches rotating over cache replicas, and HIP-graph replays of one
    captured step per replica (the GPU time per step, without Python's
    issue time)."""
    dev = "cuda:0"
    pre, shape, params, W, sets = _device_case(w, dev)
    inp = synth.step_inputs(w, 0, pre)
    ws = tbl.alloc_workspace(shape, params, dev)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device=dev)
    q, qi = inp.q.to(dev), inp.q_imp.to(dev)
    kn, vn = inp.k_new.to(dev), inp.v_new.to(dev)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=q.dtype, device=dev)
    args = [tbl.step_args(shape, params, q=q, q_imp=qi, k_new=kn, v_new=vn, refresh=True, w=W,
                          k_cache=r["K"], v_cache=r["V"], kp_cache=r["Kp"], ctx_len=ctx,
                          softmax_scale=w.softmax_scale, sel_idx=None, sel_count=r["cnt"],
                          sel_bits=r["bits"], keep_from=r["keep"], out=out) for r in sets]
    R = len(sets)
    step = lambda i: tbl.decode_step(shape, params, args[i % R], ws)  # noqa: E731
    tm = _Timer()
    tm.ms(step, max(R, 10))
    eager = tm.ms(step, launches)
    step(R - 1)
    torch.cuda.synchronize()
    ref = out.clone()

    def check():
        if not torch.equal(out, ref):
            raise RuntimeError(f"{w.name}: graph replay differs from the eager step")
    graph = tm.graph_ms(step, R, max(2, launches // R), check)
    by = _bytes_of(w, sets[:1], w.ctx)
    res = {"workload": w.name, "timed_unit": "1 fused step", "unit": "steps/s",
           "value": 1e3 / graph, "us_per_unit": graph * 1e3, "eager_us_per_unit": eager * 1e3,
           "timing": "HIP-graph replay", "replicas": R, "algorithmic_bytes": by,
           "achieved": by / (graph * 1e-3) / 1e9, "frac": by / (graph * 1e-3) / 1e9 / PEAK_HBM_GBS}
    log(f"bench: {w.name}: {graph * 1e3:.1f} us/step (graph), {eager * 1e3:.1f} us eager, "
        f"{by / 1e6:.1f} MB, {res['achieved']:.0f} GB/s")
    del sets, ws
    torch.cuda.empty_cache()
    return res


def layers_leg(w, decode_steps: int) -> dict:
    """The batched workload: one decode step is w.layers serial per-layer
    fused steps over w.batch sequences, each layer with caches of its own."""
    dev = "cuda:0"
    pre, shape, params, W, sets = _device_case(w, dev, n_layers=w.layers, rotate=257)
    inp = synth.step_inputs(w, 0, pre)
    del pre
    ws = tbl.alloc_workspace(shape, params, dev)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device=dev)
    q, qi = inp.q.to(dev), inp.q_imp.to(dev)
    kn, vn = inp.k_new.to(dev), inp.v_new.to(dev)
    out = torch.empty((w.layers, w.batch, w.n_q_heads, w.head_dim), dtype=q.dtype, device=dev)
    args = [tbl.step_args(shape, params, q=q, q_imp=qi, k_new=kn, v_new=vn, refresh=True, w=W,
                          k_cache=r["K"], v_cache=r["V"], kp_cache=r["Kp"], ctx_len=ctx,
                          softmax_scale=w.softmax_scale, sel_idx=None, sel_count=r["cnt"],
                          sel_bits=r["bits"], keep_from=r["keep"], out=out[i])
            for i, r in enumerate(sets)]

    def decode(_):
        for a in args:
            tbl.decode_step(shape, params, a, ws)
    tm = _Timer()
    tm.ms(decode, 2)
    eager = tm.ms(decode, decode_steps)
    ref = out.clone()

    def check():
        if not torch.equal(out, ref):
            raise RuntimeError(f"{w.name}: graph replay differs from the eager decode step")
    graph = tm.graph_ms(decode, 1, decode_steps, check)
    by = _bytes_of(w, sets, w.ctx)
    res = {"workload": w.name, "timed_unit": f"1 decode step = {w.layers} serial per-layer "
                                             f"fused steps over {w.batch} sequences",
           "unit": "decode steps/s", "value": 1e3 / graph, "us_per_unit": graph * 1e3,
           "eager_us_per_unit": eager * 1e3, "timing": "HIP-graph replay",
           "tokens_per_s": w.batch * 1e3 / graph, "algorithmic_bytes": by,
           "achieved": by / (graph * 1e-3) / 1e9, "frac": by / (graph * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "layer_caches": "layer l holds the first draw rotated by 257*l tokens"}
    log(f"bench: {w.name}: {graph * 1e3:.0f} us/decode step (graph), {eager * 1e3:.0f} us eager,"
        f" {by / 1e6:.0f} MB, {res['achieved']:.0f} GB/s")
    del sets, ws, out
    torch.cuda.empty_cache()
    return res


def interval_leg(w) -> dict:
    """The prediction-interval run: w.steps steps from context w.ctx0, one new
    token per step, selection recomputed every w.interval steps and reused in
    between.  The whole run is captured once as a HIP graph; the refresh
    steps alone form a second graph, and reuse steps take the difference."""
    dev = "cuda:0"
    pre, shape, params, W, sets = _device_case(w, dev, max_reps=1, max_bytes=0)
    r = sets[0]
    ws = tbl.alloc_workspace(shape, params, dev)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=synth.torch_dtype(w), device=dev)
    keep_alive = []
    args = []
    qi = None
    for s in range(w.steps):
        si = synth.step_inputs(w, s, pre)
        if si.refresh:
            qi = si.q_imp.to(dev)
        t = dict(q=si.q.to(dev), qi=qi, kn=si.k_new.to(dev), vn=si.v_new.to(dev),
                 ctx=torch.full((w.batch,), w.ctx0 + s + 1, dtype=torch.int32, device=dev))
        keep_alive.append(t)
        args.append(tbl.step_args(shape, params, q=t["q"], q_imp=t["qi"], k_new=t["kn"],
                                  v_new=t["vn"], refresh=si.refresh, w=W, k_cache=r["K"],
                                  v_cache=r["V"], kp_cache=r["Kp"], ctx_len=t["ctx"],
                                  softmax_scale=w.softmax_scale, sel_idx=None,
                                  sel_count=r["cnt"], sel_bits=r["bits"], keep_from=r["keep"],
                                  out=out))
    del pre
    refresh_ids = [s for s in range(w.steps) if s % w.interval == 0]
    # one eager pass, recording each step's unique rows
    by_ref, by_reuse = 0, 0
    row = w.head_dim * w.elt_bytes
    for s in range(w.steps):
        tbl.decode_step(shape, params, args[s], ws)
        torch.cuda.synchronize()
        ctx = w.ctx0 + s + 1
        keep = r["keep"].cpu().numpy()
        uniq = sum(_seq_unique(r["bits"], keep, w, ctx, b) for b in range(w.batch))
        if s in refresh_ids:
            by_ref += uniq * 2 * row + w.batch * w.n_kv_heads * ctx * w.d_imp * w.elt_bytes
        else:
            by_reuse += uniq * 2 * row
    ref = out.clone()

    def check_all():
        if not torch.equal(out, ref):
            raise RuntimeError(f"{w.name}: graph replay of the run differs from the eager run")
    tm = _Timer()
    all_ms = tm.graph_ms(lambda i: tbl.decode_step(shape, params, args[i], ws), w.steps, 10,
                         check_all) * w.steps
    ref_ms = tm.graph_ms(lambda i: tbl.decode_step(shape, params, args[refresh_ids[i]], ws),
                         len(refresh_ids), 10, lambda: None) * len(refresh_ids)
    n_ref, n_reuse = len(refresh_ids), w.steps - len(refresh_ids)
    by = by_ref + by_reuse
    res = {"workload": w.name, "timed_unit": f"{w.steps} growing-context steps over "
                                             f"{w.batch} sequences",
           "unit": "steps/s", "value": w.steps * 1e3 / all_ms,
           "us_per_unit": all_ms * 1e3, "mean_step_us": all_ms * 1e3 / w.steps,
           "refresh_step_us": ref_ms * 1e3 / n_ref,
           "reuse_step_us": (all_ms - ref_ms) * 1e3 / n_reuse,
           "timing": "HIP-graph replay (reuse = whole run minus the refresh steps)",
           "algorithmic_bytes": by, "achieved": by / (all_ms * 1e-3) / 1e9,
           "frac": by / (all_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "refresh_bytes_per_step": by_ref / n_ref, "reuse_bytes_per_step": by_reuse / n_reuse}
    log(f"bench: {w.name}: {all_ms * 1e3:.0f} us per {w.steps} steps (graph); refresh "
        f"{res['refresh_step_us']:.1f} us, reuse {res['reuse_step_us']:.1f} us; "
        f"{res['achieved']:.0f} GB/s")
    del sets, ws, keep_alive, args
    torch.cuda.empty_cache()
    return res


def projection_leg(w, launches: int) -> dict:
    """The prefill projection of w's whole context (tb_project_keys), HBM
    resident: fp64 multiply-adds on the matrix cores; bytes = keys read +
    projected keys written."""
    dev = "cuda:0"
    pre = synth.prefill(w)
    shape = tbl.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.n_imp_heads, w.head_dim,
                           w.d_imp, w.ctx_cap, synth.torch_dtype(w))
    K, W = pre.K.to(dev), pre.W.to(dev)
    del pre
    Kp = torch.zeros((w.batch, w.n_kv_heads, w.ctx_cap, w.d_imp), dtype=K.dtype, device=dev)
    pos0 = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    tm = _Timer()
    call = lambda i: tbl.project_keys(shape, K, W, pos0, w.ctx0, Kp)  # noqa: E731
    tm.ms(call, 3)
    ms = tm.ms(call, launches)
    rows = w.batch * w.n_kv_heads * w.ctx0
    by = rows * (w.head_dim + w.d_imp) * w.elt_bytes
    flops = 2.0 * rows * w.head_dim * w.d_imp
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": w.name, "kernel": "project_wide_kernel (tb_project_keys)",
           "rows": rows, "us_per_launch": ms * 1e3, "bound": "mfma",
           "achieved": tf, "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
           "frac": tf / PEAK_FP64_TFLOPS, "algorithmic_bytes": by,
           "hbm_GBs": by / (ms * 1e-3) / 1e9}
    log(f"bench: projection of {rows} rows: {ms * 1e3:.1f} us, fp64 {tf:.1f} TFLOP/s, "
        f"{res['hbm_GBs']:.0f} GB/s")
    del K, Kp
    torch.cuda.empty_cache()
    return res


def mlp_leg(w, tokens: int, R: int, warmup: int, steps: int) -> dict:
    """The importance-query producer MLP (tb_predict_queries) for `tokens`
    tokens: Llama-3-8B hidden size 4096, inner width 1024, four consumer slots
    of w's importance heads.  Two short launches per call take less GPU time
    than the host needs to issue them, so R calls (one per weight replica)
    are captured in a HIP graph and replayed; a replay must reproduce the
    eager call's output."""
    dev = "cuda:0"
    dt = synth.torch_dtype(w)
    mshape = tbl.make_mlp_shape(tokens, 4096, 1024, 4, w.n_imp_heads, w.d_imp, dt,
                                tbl.TB_ACT_SILU)
    n_out = 4 * w.n_imp_heads * w.d_imp
    mdev = []
    for r in range(R):
        m = synth.mlp_inputs(tokens, 4096, 1024, n_out, dt, 40 + r)
        mdev.append((m.h.to(dev), m.w1.to(dev), m.w2.to(dev)))
    mws = tbl.alloc_mlp_workspace(mshape, dev)
    q_pred = torch.empty((4, tokens, w.n_imp_heads, w.d_imp), dtype=dt, device=dev)
    call = lambda i: tbl.predict_queries(mshape, *mdev[i % R], q_pred, mws)  # noqa: E731
    tm = _Timer()
    tm.ms(call, warmup)
    call(R - 1)
    torch.cuda.synchronize()
    q_eager = q_pred.clone()

    def check():
        if not torch.equal(q_pred, q_eager):
            raise RuntimeError("graph replay of tb_predict_queries differs from the eager call")
    ms = tm.graph_ms(call, R, max(1, steps // R), check)
    by = (4096 * 1024 + 1024 * n_out + tokens * 4096) * w.elt_bytes
    gbs = by / (ms * 1e-3) / 1e9
    flops = 2.0 * tokens * (4096 * 1024 + 1024 * n_out)
    log(f"bench: importance-query MLP, {tokens} tokens: {ms * 1e3:.2f} us, {gbs:.0f} GB/s")
    return {"kernel": "two layer launches (tb_predict_queries), HIP-graph replay",
            "shape": {"tokens": tokens, "hidden": 4096, "inner": 1024, "slots": 4,
                      "imp_heads": w.n_imp_heads, "d_imp": w.d_imp},
            "us_per_call": ms * 1e3, "algorithmic_bytes": by, "achieved": gbs,
            "frac": gbs / PEAK_HBM_GBS, "tflops": flops / (ms * 1e-3) / 1e12}


def cpu_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def _median_rate(sample, repeats: int = 3) -> tuple[float, list]:
    rates = []
    for _ in range(repeats):
        units, dt = sample()
        rates.append(units / dt)
    return float(np.median(rates)), rates


def cpu_baseline(w, seconds: float) -> dict:
    """The fp64 C oracle (single thread) on a bounded sample of workload w:
    whole decode steps of one sequence (one layer) for about `seconds`,
    repeated three times; the median rate is scaled to w's timed unit.  Cache
    set-up, including the oracle's projection of the context, is not timed."""
    import oracle as orc
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    pre = synth.prefill(w, items=[0])
    code = orc.F32 if w.dtype == "f32" else orc.BF16
    K = f64(pre.K[0])
    Kp = np.zeros((w.n_kv_heads, w.ctx_cap, w.d_imp))
    Kp[:, :w.ctx0] = orc.project(K[:, :w.ctx0], f64(pre.W), code)
    st = orc.SequenceState(K, f64(pre.V[0]), Kp, w.n_imp_heads, w.budget, w.radius,
                           w.n_sink, w.n_local)
    Wf = f64(pre.W)
    steps = [synth.step_inputs(w, s, pre, items=[0]) for s in range(min(w.steps, w.interval))]
    ins = [(f64(si.q[0]), None if si.q_imp is None else f64(si.q_imp[0]), f64(si.k_new[0]),
            f64(si.v_new[0]), si.refresh) for si in steps]
    del pre
    qi_last = [None]

    def sample():
        n = 0
        t0 = time.perf_counter()
        while True:
            for s, (q, qi, kn, vn, refresh) in enumerate(ins):
                if qi is not None:
                    qi_last[0] = qi
                orc.decode_step(st, Wf, q, qi_last[0], w.ctx0 + s + 1, code, refresh,
                                w.softmax_scale, k_new=kn, v_new=vn)
                n += 1
            if time.perf_counter() - t0 >= seconds:
                return n, time.perf_counter() - t0
    rate, rates = _median_rate(sample)
    per_unit = {"steps/s": w.batch, "decode steps/s": w.batch * w.layers}
    unit = "decode steps/s" if w.layers > 1 else "steps/s"
    scale = per_unit[unit]
    info = cpu_info()
    kind = (f"{len(ins)}-step interval (1 refresh, {len(ins) - 1} reuse)" if len(ins) > 1
            else "refresh step")
    return {"value": rate / scale, "unit": unit, "cores": 1, "kind": "oracle",
            "nproc": info["nproc"], "cpu_model": info["cpu_model"],
            "repeats": [r / scale for r in rates],
            "sample": f"median of 3 samples of ~{seconds:g} s, each whole {kind}s of one "
                      f"sequence of one layer (fp64 C oracle, single thread), scaled by "
                      f"{scale} sequence-layer steps per {unit.split('/')[0][:-1]}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="seconds per CPU-oracle sample (three samples per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--n-sink", type=int, default=0,
                    help="tokens always kept at the start of the context (sink buffer)")
    ap.add_argument("--n-local", type=int, default=0,
                    help="most recent tokens always kept (local window)")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the 256K CPU-offloaded K/V leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other four workloads (tiny fp32, batch-16 32-layer 8K, "
                         "batch-4 16K interval, 128K)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (for HBM counter scaling)")
    ap.add_argument("--workload", choices=[TINY_F32.name, BATCHED_8K.name, INTERVAL_16K.name,
                                           LONG_128K.name],
                    help="time only this workload's leg and print its JSON object (for "
                         "per-workload kernel traces)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {a.gpus}); "
              "sharding is described in the design notes but not built", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    torch.cuda.set_device(0)
    if a.workload:
        wl = BY_NAME[a.workload]
        leg = {BATCHED_8K.name: lambda: layers_leg(wl, max(3, a.steps // 20)),
               INTERVAL_16K.name: lambda: interval_leg(wl)}.get(wl.name,
                                                              lambda: single_step_leg(wl, a.steps))
        res = leg()
        if not a.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline(wl, a.cpu_seconds)
        print(json.dumps(res), flush=True)
        return 0

    w = replace(LLAMA_32K, n_sink=a.n_sink, n_local=a.n_local)
    dev = "cuda:0"
    log(f"bench: generating {w.name}")
    pre = synth.prefill(w)
    inp = synth.step_inputs(w, 0, pre)
    shape = tbl.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.n_imp_heads, w.head_dim,
                           w.d_imp, w.ctx_cap, synth.torch_dtype(w))
    params = tbl.make_params(w.budget, w.radius, w.n_sink, w.n_local)

    K0, V0, W = pre.K.to(dev), pre.V.to(dev), pre.W.to(dev)
    Kp0 = torch.zeros((w.batch, w.n_kv_heads, w.ctx_cap, w.d_imp), dtype=K0.dtype, device=dev)
    tbl.project_keys(shape, K0, W, torch.zeros(w.batch, dtype=torch.int32, device=dev), w.ctx0,
                     Kp0)
    reps = []
    for r in range(a.replicas):
        reps.append(dict(
            K=K0.clone(), V=V0.clone(), Kp=Kp0.clone(),
            cnt=torch.zeros((w.batch, w.n_imp_heads), dtype=torch.int32, device=dev),
            bits=torch.zeros((w.batch, w.n_imp_heads, tbl.bitmap_words(shape)),
                             dtype=torch.int32, device=dev),
            keep=torch.zeros(w.batch, dtype=torch.int32, device=dev)))
    del K0, V0, Kp0
    ws = tbl.alloc_workspace(shape, params, dev)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device=dev)
    q, qi = inp.q.to(dev), inp.q_imp.to(dev)
    kn, vn = inp.k_new.to(dev), inp.v_new.to(dev)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=q.dtype, device=dev)
    step_args = [tbl.step_args(shape, params, q=q, q_imp=qi, k_new=kn, v_new=vn, refresh=True, w=W,
                               k_cache=r["K"], v_cache=r["V"], kp_cache=r["Kp"], ctx_len=ctx,
                               softmax_scale=w.softmax_scale, sel_idx=None,
                               sel_count=r["cnt"], sel_bits=r["bits"], keep_from=r["keep"],
                               out=out)
                 for r in reps]
    torch.cuda.synchronize()

    R = len(reps)
    log(f"bench: warmup {a.warmup}, timed {a.steps} fused steps over {R} replicas")
    for s in range(a.warmup):
        tbl.decode_step(shape, params, step_args[s % R], ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(a.steps):
        tbl.decode_step(shape, params, step_args[s % R], ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / a.steps
    log(f"bench: {ms_step * 1e3:.2f} us/step")

    # dominant kernel: the gathered attention, launched alone on the same stream
    for s in range(a.warmup):
        r = reps[s % R]
        tbl.sparse_attn(shape, q, r["K"], r["V"], None, 0, None, r["keep"], ctx,
                        w.softmax_scale, out, ws, sel_bits=r["bits"])
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(a.steps):
        r = reps[s % R]
        tbl.sparse_attn(shape, q, r["K"], r["V"], None, 0, None, r["keep"], ctx,
                        w.softmax_scale, out, ws, sel_bits=r["bits"])
    e1.record(stream)
    torch.cuda.synchronize()
    ms_attn = e0.elapsed_time(e1) / a.steps

    # comparator: dense attention over the whole context at the same shape
    for s in range(a.warmup):
        r = reps[s % R]
        tbl.dense_attn(shape, q, r["K"], r["V"], ctx, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(a.steps):
        r = reps[s % R]
        tbl.dense_attn(shape, q, r["K"], r["V"], ctx, w.softmax_scale, out, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_dense = e0.elapsed_time(e1) / a.steps

    # prediction interval: a reuse step appends and projects the new token and
    # attends over the selection the last refresh left in its replica (no
    # scores, no selection); the mean step over an interval of P steps is one
    # refresh and P - 1 reuses
    P = 8
    reuse_args = [tbl.step_args(shape, params, q=q, q_imp=qi, k_new=kn, v_new=vn, refresh=False,
                                w=W, k_cache=r["K"], v_cache=r["V"], kp_cache=r["Kp"],
                                ctx_len=ctx, softmax_scale=w.softmax_scale, sel_idx=None,
                                sel_count=r["cnt"], sel_bits=r["bits"], keep_from=r["keep"],
                                out=out)
                  for r in reps]
    for s in range(a.warmup):
        tbl.decode_step(shape, params, reuse_args[s % R], ws)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(a.steps):
        tbl.decode_step(shape, params, reuse_args[s % R], ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_reuse = e0.elapsed_time(e1) / a.steps

    # A reuse step's GPU work is shorter than the time the host needs to issue
    # a step from Python, so the interval is also timed as HIP-graph replays
    # (one captured step per replica) of refresh and of reuse steps; each
    # replay must reproduce the eager output.
    def graph_ms(args_list):
        tbl.decode_step(shape, params, args_list[R - 1], ws)
        torch.cuda.synchronize()
        ref = out.clone()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for r in range(R):
                tbl.decode_step(shape, params, args_list[r], ws)
        for _ in range(2):
            out.zero_()
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref):
                raise RuntimeError("graph replay of the decode step differs from the eager step")
        n_rep = max(1, a.steps // R)
        e0.record(stream)
        for _ in range(n_rep):
            gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n_rep * R)

    ms_refresh_g = graph_ms(step_args)
    ms_reuse_g = graph_ms(reuse_args)
    ms_interval = (ms_refresh_g + (P - 1) * ms_reuse_g) / P
    log(f"bench: reuse step {ms_reuse * 1e3:.2f} us issued from Python; graph replay: refresh "
        f"{ms_refresh_g * 1e3:.2f} us, reuse {ms_reuse_g * 1e3:.2f} us; interval of {P}: mean "
        f"step {ms_interval * 1e3:.2f} us, {ms_dense / ms_interval:.2f}x dense attention")

    mlp = {tok: mlp_leg(w, tok, R, a.warmup, a.steps) for tok in (w.batch, BATCHED_8K.batch)}

    uniq, logical = unique_rows(reps[0]["bits"], w, w.ctx)
    row_bytes = w.head_dim * w.elt_bytes
    gather_bytes = uniq * 2 * row_bytes
    kp_bytes = w.ctx * w.n_kv_heads * w.d_imp * w.elt_bytes
    step_bytes = kp_bytes + gather_bytes
    attn_gbs = gather_bytes / (ms_attn * 1e-3) / 1e9
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    dense_bytes = w.ctx * w.n_kv_heads * 2 * row_bytes
    dense_gbs = dense_bytes / (ms_dense * 1e-3) / 1e9
    log(f"bench: attention {ms_attn * 1e3:.2f} us, {attn_gbs:.0f} GB/s; step {step_gbs:.0f} GB/s "
        f"({uniq} unique rows, {logical} logical)")
    log(f"bench: dense attention {ms_dense * 1e3:.2f} us, {dense_gbs:.0f} GB/s; "
        f"sparse step / dense attention = {ms_dense / ms_step:.2f}x")

    if a.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    offload = None if a.no_offload else offload_leg(max(4, min(a.steps, 20)))

    del reps, step_args, reuse_args, ws
    torch.cuda.empty_cache()
    proj = projection_leg(w, 20)

    per_workload = {w.name: {"workload": w.name, "timed_unit": "1 fused step", "unit": "steps/s",
                        "value": 1e3 / ms_step, "us_per_unit": ms_step * 1e3,
                        "graph_us_per_unit": ms_refresh_g * 1e3, "timing": "eager launches",
                        "algorithmic_bytes": step_bytes, "achieved": step_gbs,
                        "frac": step_gbs / PEAK_HBM_GBS}}
    if not a.no_configs:
        per_workload[TINY_F32.name] = single_step_leg(TINY_F32, a.steps)
        per_workload[BATCHED_8K.name] = layers_leg(BATCHED_8K, max(3, a.steps // 20))
        per_workload[INTERVAL_16K.name] = interval_leg(INTERVAL_16K)
        per_workload[LONG_128K.name] = single_step_leg(LONG_128K, a.steps)

    cpu = None
    if not a.no_cpu_baseline:
        for name in list(per_workload):
            log(f"bench: timing the CPU oracle on {name}")
            per_workload[name]["cpu_baseline"] = cpu_baseline(BY_NAME[name], a.cpu_seconds)
        cpu = per_workload[w.name]["cpu_baseline"]

    line = {
        "metric": METRIC,
        "value": 1e3 / ms_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) K/V/queries, 1% planted heavy tokens; bf16 caches)",
        "config": {"workload": w.name, "batch": w.batch, "ctx": w.ctx,
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "imp_heads": w.n_imp_heads, "head_dim": w.head_dim, "d_imp": w.d_imp,
                   "budget": w.budget, "radius": w.radius, "interval": w.interval,
                   "n_sink": w.n_sink, "n_local": w.n_local,
                   "storage": w.dtype, "replicas": R},
        "roofline": {"bound": "hbm", "kernel": "attn_kernel (tb_sparse_attn)",
                     "achieved": attn_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": attn_gbs / PEAK_HBM_GBS, "traffic": measured_traffic(),
                     "algorithmic_bytes": gather_bytes, "us_per_launch": ms_attn * 1e3,
                     "step": {"algorithmic_bytes": step_bytes, "achieved": step_gbs,
                              "frac": step_gbs / PEAK_HBM_GBS}},
        "step_hbm": {"algorithmic_bytes": step_bytes, "achieved": step_gbs,
                     "frac": step_gbs / PEAK_HBM_GBS, "unique_rows": uniq,
                     "logical_rows": logical},
        "dense_attention": {"kernel": "dense_kernel (tb_dense_attn)", "us_per_launch": ms_dense * 1e3,
                            "algorithmic_bytes": dense_bytes, "achieved": dense_gbs,
                            "frac": dense_gbs / PEAK_HBM_GBS,
                            "speedup_of_sparse_step": ms_dense / ms_step},
        "prediction_interval": {"interval": P, "timing": "HIP-graph replay",
                                "refresh_step_us": ms_refresh_g * 1e3,
                                "reuse_step_us": ms_reuse_g * 1e3,
                                "reuse_step_us_issued_from_python": ms_reuse * 1e3,
                                "mean_step_us": ms_interval * 1e3,
                                "speedup_vs_dense_attention": ms_dense / ms_interval},
        "predictor_mlp": {str(k): v for k, v in mlp.items()},
        "projection": proj,
        "offload": offload,
        "configs": per_workload,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
