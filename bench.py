#!/usr/bin/env python3
"""Decode-step benchmark for libmla on one MI355X.

A step is one pass of the whole hot path over one batch: plan, absorb_q,
split-KV attention, then the log-sum-exp combine and absorb_out (one fused
call), for every sequence of the workload.  Inputs are seeded synthetic
tensors already resident in HBM.  The same line also reports, measured on
their own: the cache append of the step's new tokens and the prefill of a
4 x 4096-token batch (--no-prefill skips it), the step over the workload's
FP8-cache twin (--no-fp8), and the offline weight folds with the fused
products that replace absorb_q and absorb_out (--no-folds).
Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-prefill]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "batch64_1k8k_bf16"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
KERNEL_SOURCES = ["mla_latent_kv_14_amd/csrc/decode_mfma.hip", "mla_latent_kv_14_amd/csrc/common.h",
                  "mla_latent_kv_14_amd/csrc/mfma_util.h"]
PREFILL_WORKLOAD = "prefill_4x4k_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attention_batch64_1k8k_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_work(prob):
    """Bytes and flops the attention kernel must move / do for one launch.

    Bytes: every visible cache row once (d_c + d_rope elements, one byte each
    for an FP8 cache), the absorbed queries, the block-table entries used, the
    sequence lengths, and the latent output o (float32).  Split partials are
    implementation overhead and not counted.  Flops: 2 * (d_c + d_rope) for
    the score plus 2 * d_c for the weighted sum, per visible (query row,
    token) pair.
    """
    wl = prob.wl
    esz = 4 if wl.dtype == "f32" else 2
    D = wl.d_c + wl.d_rope
    L = prob.seq_lens.astype(np.int64)
    rows_bytes = int(L.sum()) * D * (1 if prob.fp8 else esz)
    q_bytes = wl.batch * wl.q_len * wl.heads * D * esz
    table_bytes = int(((L + wl.block_size - 1) // wl.block_size).sum()) * 4 + wl.batch * 4
    o_bytes = wl.batch * wl.q_len * wl.heads * wl.d_c * 4
    visible = sum(int((L - wl.q_len + j + 1).sum()) for j in range(wl.q_len))
    flops = 2 * wl.heads * visible * (D + wl.d_c)
    return rows_bytes + q_bytes + table_bytes + o_bytes, flops


def tokens_of(prob):
    """New tokens one decode step produces: B * q_len."""
    return prob.wl.batch * prob.wl.q_len


def append_work(prob, d_model):
    """Bytes and flops of one cache append: the two projection weights, the
    hidden states, the written rows and the table entries and lengths read;
    2 * d_model flops per written element."""
    wl = prob.wl
    esz = 4 if wl.dtype == "f32" else 2
    D = wl.d_c + wl.d_rope
    M = wl.batch * wl.q_len
    nbytes = (D * d_model + M * d_model + M * D) * esz + M * 4 + wl.batch * 4
    return nbytes, 2 * M * D * d_model


def prefill_work(prob):
    """Flops of one prefill call: the attention over the visible (query, key)
    pairs, (d_nope + d_rope + d_v) multiply-adds each per head, and the
    up-projection of every token's latent to per-head keys and values."""
    wl = prob.wl
    causal_pairs = sum(int(L) * (int(L) + 1) // 2 for L in prob.seq_lens)
    attn = 2 * wl.heads * causal_pairs * (wl.d_nope + wl.d_rope + wl.d_v)
    up = 2 * prob.total_tokens * wl.d_c * wl.heads * (wl.d_nope + wl.d_v)
    return attn, up


def source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        p = os.path.join(ROOT, rel)
        if os.path.exists(p):
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per attention launch from committed rocprofv3 counters, if they match this source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash() or rec.get("workload") != workload_name:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(prob, budget_s=15.0, max_s=30.0):
    """Time the float64 oracle on the first sequences of the same workload."""
    from oracle import mla_oracle as orc

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    wl = prob.wl
    cache = prob.cache.float().numpy() if wl.dtype == "bf16" else prob.cache.numpy()
    qn, qr = prob.f64("q_nope"), prob.f64("q_rope")
    wuk, wuv = prob.f64("w_uk"), prob.f64("w_uv")
    done, tokens_ctx = 0, 0
    t0 = time.perf_counter()
    for b in range(wl.batch):
        sel = [(b, h) for h in range(wl.heads)]
        orc.mla_decode_reference(qn, qr, cache, prob.block_table, prob.seq_lens, wuk, wuv, prob.scale, wl.d_c,
                                 select=sel)
        done += 1
        tokens_ctx += int(prob.seq_lens[b])
        el = time.perf_counter() - t0
        if el >= budget_s or el >= max_s:
            break
    el = time.perf_counter() - t0
    return {
        "value": done * wl.q_len / el,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{done} of {wl.batch} sequences ({tokens_ctx} context tokens), all {wl.heads} heads, "
                   f"float64 non-absorbed route, {el:.1f} s"),
    }


FOLD_D_IN = 1536  # query latent width: the input of the fused query weight


def measure_folds(prob, r, stream, K, warmup):
    """The offline folds and the fused products, with the unfolded route beside them.

    Fused query: q_cat = [W~_Q x ; q^R] replaces (W_in x, then absorb_q).
    Fused output: y = W~^O o replaces (absorb_out, then W^O u).  The unfolded
    route's plain projections W_in x and W^O u are not libmla calls: they run
    as torch.matmul (hipBLASLt) here, for comparison only.  Algorithmic bytes
    of a fused product: its weight, its inputs and its output once.
    """
    import torch

    from mla_latent_kv_14_amd import binding as libmla
    from mla_latent_kv_14_amd.inputs import make_fold_inputs

    wl = prob.wl
    dev = "cuda:0"
    fi = make_fold_inputs(prob, d_in=FOLD_D_IN)
    d = r.dims
    M, H, D = wl.batch * wl.q_len, wl.heads, wl.d_c + wl.d_rope
    x, w_in, w_o, o = (t.to(dev) for t in (fi.x, fi.w_in, fi.w_o, fi.o))
    w_uk, w_uv, q_rope = (t.to(dev) for t in (prob.w_uk, prob.w_uv, prob.q_rope))
    dt = w_in.dtype
    wq = torch.empty((H, wl.d_c, fi.d_in), dtype=dt, device=dev)
    wo = torch.empty((fi.d_out, H * wl.d_c), dtype=dt, device=dev)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    fold_q = lambda: libmla.mla_fold_query_weight(d, fi.d_in, w_in, w_uk, wq)
    fold_o = lambda: libmla.mla_fold_output_weight(d, fi.d_out, w_o, w_uv, wo)
    fold_q()
    fold_o()
    fold_q_us, fold_o_us = timed(fold_q, 2), timed(fold_o, 2)

    q_cat = torch.empty((wl.batch, wl.q_len, H, D), dtype=dt, device=dev)
    ws = torch.empty((max(libmla.mla_fused_output_workspace_bytes(d, fi.d_out), 4) // 4,), dtype=torch.float32,
                     device=dev)
    y = torch.empty((wl.batch, wl.q_len, fi.d_out), dtype=dt, device=dev)
    fq = lambda: libmla.mla_fused_query(d, fi.d_in, x, q_rope, wq, q_cat)
    fo = lambda: libmla.mla_fused_output(d, fi.d_out, o, wo, y, ws)
    q_nope = torch.empty((M, H * wl.d_nope), dtype=dt, device=dev)
    u = torch.empty((wl.batch, wl.q_len, H, wl.d_v), dtype=dt, device=dev)
    y2 = torch.empty((M, fi.d_out), dtype=dt, device=dev)
    w_uq = w_in.reshape(H * wl.d_nope, fi.d_in)

    def unfolded_q():
        torch.matmul(x.reshape(M, fi.d_in), w_uq.t(), out=q_nope)
        libmla.mla_absorb_q(d, q_nope.view(wl.batch, wl.q_len, H, wl.d_nope), q_rope, w_uk, q_cat)

    def unfolded_o():
        libmla.mla_absorb_out(d, o, w_uv, u)
        torch.matmul(u.view(M, H * wl.d_v), w_o.t(), out=y2)

    for fn in (fq, fo, unfolded_q, unfolded_o):
        for _ in range(warmup):
            fn()
    fq_us, fo_us = timed(fq, K), timed(fo, K)
    uq_us, uo_us = timed(unfolded_q, K), timed(unfolded_o, K)
    esz = 2 if dt == torch.bfloat16 else 4
    q_bytes = wq.numel() * esz + x.numel() * esz + q_rope.numel() * esz + q_cat.numel() * esz
    o_bytes = wo.numel() * esz + o.numel() * 4 + y.numel() * esz
    res = {
        "d_in": fi.d_in, "d_out": fi.d_out,
        "fold_query_ms": fold_q_us / 1e3, "fold_output_ms": fold_o_us / 1e3,
        "fused_query": {"us": fq_us, "alg_bytes": q_bytes, "gbs": q_bytes / (fq_us * 1e-6) / 1e9,
                        "hbm_frac": q_bytes / (fq_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                        "weight_bytes": wq.numel() * esz},
        "fused_output": {"us": fo_us, "alg_bytes": o_bytes, "gbs": o_bytes / (fo_us * 1e-6) / 1e9,
                         "hbm_frac": o_bytes / (fo_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "weight_bytes": wo.numel() * esz},
        "unfolded_query_us": uq_us, "unfolded_output_us": uo_us,
        "unfolded_note": "W_in x and W^O u by torch.matmul (hipBLASLt), absorb_q / absorb_out by libmla",
    }
    log(f"bench: folds: fused query {fq_us:.1f} us ({res['fused_query']['gbs']:.0f} GB/s) vs unfolded {uq_us:.1f} us;"
        f" fused output {fo_us:.1f} us ({res['fused_output']['gbs']:.0f} GB/s) vs unfolded {uo_us:.1f} us;"
        f" folds {fold_q_us / 1e3:.2f} + {fold_o_us / 1e3:.2f} ms offline")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time HIP-graph replays instead of eager launches")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache twin of the workload")
    ap.add_argument("--no-folds", action="store_true", help="skip the weight folds and fused products")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libmla has no multi-GPU path (whole sequences would shard "
              "across GPUs with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mla_latent_kv_14_amd.inputs import (WORKLOADS, make_append_inputs, make_fold_inputs, make_prefill_problem,
                                             make_problem, workload)
    from mla_latent_kv_14_amd.runner import DecodeRunner, PrefillRunner

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    torch.cuda.set_device(0)
    wl = workload(args.workload)
    log(f"bench: generating {wl.name} ...")
    prob = make_problem(wl, args.seed)
    r = DecodeRunner(prob, device="cuda:0")
    stream = torch.cuda.current_stream()
    log(f"bench: B={wl.batch} H={wl.heads} Lq={wl.q_len} tokens={prob.total_tokens} splits={r.num_splits}")

    calls = [("plan", r.plan), ("absorb_q", r.absorb_q), ("decode", r.decode_planned),
             ("combine_absorb_out", r.combine_absorb_out)]
    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    log("bench: warmup done")
    K = args.steps

    # per-call breakdown: eager calls bracketed by events on the library's stream
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for n, _ in calls}
    for i in range(K):
        for n, fn in calls:
            ev[n][i][0].record(stream)
            fn()
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    per_call_us = {n: 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n, _ in calls}

    # the timed region: K steps back to back, four eager launches per step with
    # nothing between them (--graph replays HIP graphs of the same steps
    # instead; on this stack that measured slower)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.graph:
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K):
            for _, fn in calls:
                fn()
        end.record(stream)
    else:
        # one graph holds G consecutive steps; K/G replays run exactly K steps
        G = max(d for d in range(1, min(K, 10) + 1) if K % d == 0)
        g = r.capture(G)
        g.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K // G):
            g.replay()
        end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    log(f"bench: {ms_step * 1e3:.1f} us/step ({'graph' if args.graph else 'eager'}); per call, eager (us): " +
        ", ".join(f"{n}={v:.1f}" for n, v in per_call_us.items()))

    # the attention kernel's own duration: K launches back to back between two
    # events on its stream, so that each launch's dispatch overlaps the previous
    # kernel (the per-call events above also hold that latency); the roofline
    # below divides by this
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for i in range(K):
        r.decode_planned()
    d1.record(stream)
    torch.cuda.synchronize()
    decode_kernel_us = 1e3 * d0.elapsed_time(d1) / K
    log(f"bench: attention kernel {decode_kernel_us:.1f} us per launch (back to back)")

    # the cache append (the step just before attention in a decode loop),
    # timed on its own: K back-to-back calls; it rewrites the same slots
    app = make_append_inputs(prob)
    r.setup_append(app)
    for _ in range(args.warmup):
        r.cache_append()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a0.record(stream)
    for i in range(K):
        r.cache_append()
    a1.record(stream)
    torch.cuda.synchronize()
    append_us = 1e3 * a0.elapsed_time(a1) / K
    ap_bytes, ap_flops = append_work(prob, app.d_model)
    log(f"bench: cache append {append_us:.1f} us/call (d_model={app.d_model})")

    # prefill (the non-absorbed forward over whole sequences), its own workload
    prefill = None
    if not args.no_prefill:
        pprob = make_prefill_problem(workload(PREFILL_WORKLOAD))
        pr = PrefillRunner(pprob, device="cuda:0")
        for _ in range(2):
            pr.prefill()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        KP = 5
        torch.cuda.synchronize()
        p0.record(stream)
        for i in range(KP):
            pr.prefill()
        p1.record(stream)
        torch.cuda.synchronize()
        pms = p0.elapsed_time(p1) / KP
        f_attn, f_up = prefill_work(pprob)
        prefill = {"workload": PREFILL_WORKLOAD, "tokens": pprob.total_tokens, "heads": pprob.wl.heads,
                   "causal": True, "ms_per_call": pms, "tokens_per_s": pprob.total_tokens / (pms * 1e-3),
                   "attn_tflop": f_attn / 1e12, "upproject_tflop": f_up / 1e12,
                   "tflops": (f_attn + f_up) / (pms * 1e-3) / 1e12,
                   "mfma_frac": (f_attn + f_up) / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
        log(f"bench: prefill {PREFILL_WORKLOAD}: {pms:.2f} ms, {prefill['tflops']:.0f} TFLOP/s")
        del pr

    # the same step over an FP8 (E4M3) cache: the workload's FP8 twin (same
    # draws, codes of value / kv_scale)
    fp8 = None
    twin = wl.name.replace("_bf16", "_fp8")
    if not args.no_fp8 and not prob.fp8 and twin in WORKLOADS:
        fprob = make_problem(workload(twin), args.seed)
        fr = DecodeRunner(fprob, device="cuda:0")
        fcalls = [fr.plan, fr.absorb_q, fr.decode_planned, fr.combine_absorb_out]
        for _ in range(args.warmup):
            for fn in fcalls:
                fn()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record(stream)
        for i in range(K):
            for fn in fcalls:
                fn()
        f1.record(stream)
        torch.cuda.synchronize()
        f_step = f0.elapsed_time(f1) / K
        torch.cuda.synchronize()
        f0.record(stream)
        for i in range(K):
            fr.decode_planned()
        f1.record(stream)
        torch.cuda.synchronize()
        f_kernel_us = 1e3 * f0.elapsed_time(f1) / K
        f_bytes, _ = algorithmic_work(fprob)
        fp8 = {"workload": twin, "kv_scale": fprob.kv_scale, "ms_per_step": f_step,
               "tokens_per_s": tokens_of(fprob) / (f_step * 1e-3), "attention_kernel_us": f_kernel_us,
               "alg_bytes_per_launch": f_bytes, "gbs": f_bytes / (f_kernel_us * 1e-6) / 1e9,
               "hbm_frac": f_bytes / (f_kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
               "cache_bytes": int(fprob.cache.numel()), "num_splits": fr.num_splits}
        log(f"bench: FP8 cache ({twin}): {f_step * 1e3:.1f} us/step, attention {f_kernel_us:.1f} us")
        del fr

    folds = None
    if not args.no_folds:
        folds = measure_folds(prob, r, stream, K, args.warmup)

    alg_bytes, flops = algorithmic_work(prob)
    dec_s = decode_kernel_us * 1e-6
    achieved_gbs = alg_bytes / dec_s / 1e9
    achieved_tflops = flops / dec_s / 1e12
    tokens = wl.batch * wl.q_len
    traffic = measured_traffic(wl.name)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(prob)

    rec = {
        "metric": "MLA decode tokens/s + TFLOP/s & HBM GB/s vs roofline, B=64 H=128 ctx 1K-8K",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "q_len": wl.q_len, "d_c": wl.d_c,
                   "d_rope": wl.d_rope, "d_nope": wl.d_nope, "d_v": wl.d_v, "block_size": wl.block_size,
                   "context_tokens": prob.total_tokens, "lengths": " ".join(str(x) for x in wl.lengths),
                   "num_splits": r.num_splits},
        "roofline": {"kernel": "mla_decode attention", "kernel_us": decode_kernel_us, "bound": "hbm",
                     "achieved": achieved_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "alg_bytes_per_launch": alg_bytes,
                     "mfma_tflops": achieved_tflops, "mfma_frac": achieved_tflops / MFMA_BF16_PEAK_TFLOPS},
        "per_call_us": per_call_us,
        "launch": "hip_graph" if args.graph else "eager",
        "step_tflops": flops / (ms_step * 1e-3) / 1e12,
        "step_gbs": alg_bytes / (ms_step * 1e-3) / 1e9,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "fp8_cache": fp8,
        "weight_folds": folds,
        "cache_append": {"us_per_call": append_us, "d_model": app.d_model, "alg_bytes": ap_bytes,
                         "gbs": ap_bytes / (append_us * 1e-6) / 1e9,
                         "hbm_frac": ap_bytes / (append_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "tflops": ap_flops / (append_us * 1e-6) / 1e12},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
