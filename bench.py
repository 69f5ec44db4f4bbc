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
  dense_attention  the dense decode-attention kernel over the whole context at
                the same shape (the baseline of the pages' speedup claims);
  predictor_mlp the importance-query producer MLP (weight-streaming bound);
  offload       a 256K-context step with K/V in pinned host memory against
                dense attention over the same offloaded caches;
  cpu_baseline  the fp64 C oracle's decode step on the host (1 thread), on a
                bounded number of steps.
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
from query_aware_kv_amd.workloads import (BATCHED_8K, INTERVAL_16K, LLAMA_32K,  # noqa: E402
                                          LONG_128K, OFFLOAD_256K)

PEAK_HBM_GBS = 8000.0
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


def workload_leg(w, launches: int) -> dict:
    """One layer's fused step of another workload, HBM resident: refresh
    steps (and, with a prediction interval, reuse steps), each timed over
    `launches` eager launches with HIP events.  Cache replicas (one GB in
    all) rotate between launches so the 256 MB MALL cannot carry a step's
    rows over to the next.  Bytes = projected keys of the context + unique
    gathered K/V rows per KV group (from the library's own bitmaps)."""
    dev = "cuda:0"
    pre = synth.prefill(w)
    inp = synth.step_inputs(w, 0, pre)
    shape = tbl.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.n_imp_heads, w.head_dim,
                           w.d_imp, w.ctx_cap, synth.torch_dtype(w))
    params = tbl.make_params(w.budget, w.radius, w.n_sink, w.n_local)
    K0, V0, W = pre.K.to(dev), pre.V.to(dev), pre.W.to(dev)
    Kp0 = torch.zeros((w.batch, w.n_kv_heads, w.ctx_cap, w.d_imp), dtype=K0.dtype, device=dev)
    tbl.project_keys(shape, K0, W, torch.zeros(w.batch, dtype=torch.int32, device=dev), w.ctx0,
                     Kp0)
    per = (K0.numel() + V0.numel() + Kp0.numel()) * K0.element_size()
    R = max(2, -(-(1 << 30) // per))
    reps = [dict(K=K0.clone(), V=V0.clone(), Kp=Kp0.clone(),
                 cnt=torch.zeros((w.batch, w.n_imp_heads), dtype=torch.int32, device=dev),
                 bits=torch.zeros((w.batch, w.n_imp_heads, tbl.bitmap_words(shape)),
                                  dtype=torch.int32, device=dev),
                 keep=torch.zeros(w.batch, dtype=torch.int32, device=dev)) for _ in range(R)]
    del K0, V0, Kp0
    ws = tbl.alloc_workspace(shape, params, dev)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device=dev)
    q, qi = inp.q.to(dev), inp.q_imp.to(dev)
    kn, vn = inp.k_new.to(dev), inp.v_new.to(dev)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=q.dtype, device=dev)

    def args(r, refresh):
        return tbl.step_args(shape, params, q=q, q_imp=qi, k_new=kn, v_new=vn, refresh=refresh,
                             w=W, k_cache=r["K"], v_cache=r["V"], kp_cache=r["Kp"], ctx_len=ctx,
                             softmax_scale=w.softmax_scale, sel_idx=None, sel_count=r["cnt"],
                             sel_bits=r["bits"], keep_from=r["keep"], out=out)

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(arg_list):
        for i in range(max(R, 10)):
            tbl.decode_step(shape, params, arg_list[i % R], ws)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(launches):
            tbl.decode_step(shape, params, arg_list[i % R], ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches

    ms_refresh = timed([args(r, True) for r in reps])
    uniq = sum(unique_rows(reps[0]["bits"][b:b + 1], w, w.ctx)[0] for b in range(w.batch))
    row = w.head_dim * w.elt_bytes
    kp_bytes = w.batch * w.n_kv_heads * w.ctx * w.d_imp * w.elt_bytes
    by = kp_bytes + uniq * 2 * row
    res = {"batch": w.batch, "ctx": w.ctx, "budget": w.budget, "radius": w.radius,
           "interval": w.interval, "replicas": R, "refresh_step_us": ms_refresh * 1e3,
           "unique_rows": uniq, "unique_row_fraction": uniq / (w.batch * w.n_kv_heads * w.ctx),
           "algorithmic_bytes": by, "achieved": by / (ms_refresh * 1e-3) / 1e9,
           "frac": by / (ms_refresh * 1e-3) / 1e9 / PEAK_HBM_GBS}
    msg = (f"bench: {w.name}: refresh step {ms_refresh * 1e3:.1f} us, {by / 1e6:.0f} MB, "
           f"{res['achieved']:.0f} GB/s")
    if w.interval > 1:
        ms_reuse = timed([args(r, False) for r in reps])
        by_r = uniq * 2 * row + w.batch * w.n_kv_heads * w.d_imp * w.elt_bytes
        ms_mean = (ms_refresh + (w.interval - 1) * ms_reuse) / w.interval
        by_mean = (by + (w.interval - 1) * by_r) / w.interval
        res.update({"reuse_step_us": ms_reuse * 1e3, "mean_step_us": ms_mean * 1e3,
                    "mean_achieved": by_mean / (ms_mean * 1e-3) / 1e9,
                    "mean_frac": by_mean / (ms_mean * 1e-3) / 1e9 / PEAK_HBM_GBS})
        msg += (f"; reuse step {ms_reuse * 1e3:.1f} us; mean over {w.interval}: "
                f"{ms_mean * 1e3:.1f} us, {res['mean_achieved']:.0f} GB/s")
    log(msg)
    del reps, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, pre, inp, seconds: float, max_steps: int) -> dict:
    import oracle as orc
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    K = f64(pre.K[0])
    Kp = np.zeros((w.n_kv_heads, w.ctx_cap, w.d_imp))
    Kp[:, :w.ctx0] = orc.project(K[:, :w.ctx0], f64(pre.W), orc.BF16)  # set-up, not timed
    st = orc.SequenceState(K, f64(pre.V[0]), Kp, w.n_imp_heads, w.budget, w.radius)
    args = (f64(pre.W), f64(inp.q[0]), f64(inp.q_imp[0]))
    kn, vn = f64(inp.k_new[0]), f64(inp.v_new[0])
    n = 0
    t0 = time.perf_counter()
    while n < max_steps:
        orc.decode_step(st, *args, w.ctx, orc.BF16, True, w.softmax_scale, k_new=kn, v_new=vn)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} decode steps of the 32K-context workload (append+project, score, "
                      f"top-B, attend; fp64 C oracle, single thread, {dt:.1f} s)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--n-sink", type=int, default=0,
                    help="tokens always kept at the start of the context (sink buffer)")
    ap.add_argument("--n-local", type=int, default=0,
                    help="most recent tokens always kept (local window)")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the 256K CPU-offloaded K/V leg")
    ap.add_argument("--other-workloads", action="store_true",
                    help="also time one layer of the batch-16 8K, batch-4 16K interval and "
                         "128K workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (for HBM counter scaling)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {a.gpus}); "
              "sharding is described in the design notes but not built", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    w = replace(LLAMA_32K, n_sink=a.n_sink, n_local=a.n_local)
    dev = "cuda:0"
    torch.cuda.set_device(0)
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

    # the importance-query producer MLP at the step's batch: Llama-3-8B hidden
    # size, inner width 1024, four consumer slots of this shape's heads
    mshape = tbl.make_mlp_shape(w.batch, 4096, 1024, 4, w.n_imp_heads, w.d_imp, q.dtype,
                                tbl.TB_ACT_SILU)
    n_out = 4 * w.n_imp_heads * w.d_imp
    mins = [synth.mlp_inputs(w.batch, 4096, 1024, n_out, q.dtype, 40 + r) for r in range(R)]
    mdev = [(m.h.to(dev), m.w1.to(dev), m.w2.to(dev)) for m in mins]
    mws = tbl.alloc_mlp_workspace(mshape, dev)
    q_pred = torch.empty((4, w.batch, w.n_imp_heads, w.d_imp), dtype=q.dtype, device=dev)
    for s in range(a.warmup):
        tbl.predict_queries(mshape, *mdev[s % R], q_pred, mws)
    torch.cuda.synchronize()
    # Two short launches per call take less GPU time than the host needs to
    # issue them, so the calls (one per replica) are captured in a HIP graph
    # and the graph is replayed: the figure is the GPU's time per call.  A
    # replay must reproduce the eager call's output.
    q_eager = q_pred.clone()
    tbl.predict_queries(mshape, *mdev[R - 1], q_eager, mws)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(R):
            tbl.predict_queries(mshape, *mdev[r], q_pred, mws)
    torch.cuda.synchronize()
    n_rep = max(1, a.steps // R)
    for _ in range(2):
        q_pred.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(q_pred, q_eager):
            raise RuntimeError("graph replay of tb_predict_queries differs from the eager call")
    e0.record(stream)
    for _ in range(n_rep):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_mlp = e0.elapsed_time(e1) / (n_rep * R)
    mlp_bytes = (4096 * 1024 + 1024 * n_out) * w.elt_bytes
    mlp_gbs = mlp_bytes / (ms_mlp * 1e-3) / 1e9
    log(f"bench: importance-query MLP {ms_mlp * 1e3:.2f} us, {mlp_gbs:.0f} GB/s")

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

    others = None
    if a.other_workloads:
        others = {wl.name: workload_leg(wl, 100) for wl in (BATCHED_8K, INTERVAL_16K, LONG_128K)}

    cpu = None
    if not a.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        cpu = cpu_baseline(w, pre, inp, a.cpu_seconds, 200)

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
                     "algorithmic_bytes": gather_bytes, "us_per_launch": ms_attn * 1e3},
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
        "predictor_mlp": {"kernel": "two layer launches (tb_predict_queries), HIP-graph replay",
                          "shape": {"tokens": w.batch, "hidden": 4096, "inner": 1024,
                                    "slots": 4, "imp_heads": w.n_imp_heads, "d_imp": w.d_imp},
                          "us_per_call": ms_mlp * 1e3, "algorithmic_bytes": mlp_bytes,
                          "achieved": mlp_gbs, "frac": mlp_gbs / PEAK_HBM_GBS},
        "offload": offload,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
