#!/usr/bin/env python3
"""Decode-step benchmark for libmla on one MI355X.

A step is one pass of the whole hot path over one batch: absorb_q with the
split-KV plan (one launch), the split-KV attention, then the log-sum-exp
combine and absorb_out (one fused call), for every sequence of the workload.  Inputs are seeded synthetic
tensors already resident in HBM.

Timing is cold: before every timed step (or call) a flush kernel reads
1 GiB of an unrelated buffer, outside the timed events, so that the 256 MB
last-level cache and the L2s hold none of the step's data (and no dirty
lines) and the cache rows come from HBM.  Times come from HIP events on
the library's stream: per sample, (flush, step) minus a flush alone, each
between two events, so that the event pair's own cost cancels; the line
reports their mean (which `value` uses), p10, p50 and p90, for the step and
for the attention kernel alone (whose mean the roofline uses).  Warm
back-to-back numbers are reported separately and labelled as such.

The line also carries: the roofs this chip sustains, measured by the
measurement kernels of libmla_roofs.so (a streaming HBM read over 4 GiB and a
register-only bf16 matrix-core loop), next to the published peaks; the
attention kernel's roofline against both; the other decode workloads (one
sequence of 4096, four of 131,072, and the 2-token batch of 128 at 16 heads)
timed the same way; and, measured on their own, the cache append, the
prefill of 4 x 4096 tokens (--no-prefill), the step over the FP8-cache twin
(--no-fp8) and the weight folds with their fused products (--no-folds).
Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-configs]
                    [--cold-only] [--no-prefill] [--no-fp8] [--no-folds]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "batch64_1k8k_bf16"
OTHER_WORKLOADS = ["single_4k_bf16", "long128k_bf16", "mtp2_lognormal_bf16"]
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FLUSH_BYTES = 1 << 30  # read before every cold timing: four times the 256 MB last-level cache
READ_PEAK_BYTES = 4 << 30  # streamed by the HBM read measurement
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


def stats(times_us):
    a = np.asarray(times_us, dtype=np.float64)
    return {"mean": float(a.mean()), "p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


class Timer:
    """Cold and warm timing on one stream with HIP events (torch.cuda.Event records on the given stream).

    The flush READS 1 GiB (plain loads, which allocate in the L2s and the last-level cache), so that the
    caches hold only clean lines of an unrelated buffer.  A flush that writes would leave up to 288 MB of
    dirty lines whose write-back lands inside the next timed kernel; write_flush = True does that, for
    the comparison the line reports."""

    def __init__(self, stream, flush_buf):
        import torch
        from mla_latent_kv_14_amd import roofs

        self.torch, self.roofs = torch, roofs
        self.stream, self.flush_buf = stream, flush_buf
        self.sink = torch.zeros(max(roofs.read_grid(), 1) + 64, dtype=torch.int32, device=flush_buf.device)
        self.write_flush = False

    def flush(self):
        if self.write_flush:
            self.roofs.flush(self.flush_buf, self.stream)
        else:
            self.roofs.hbm_read(self.flush_buf, self.sink, False, self.stream)

    def cold_net(self, fn, n):
        """n cold samples of fn without the event pair's own cost (us): each sample times (flush, fn) and then a
        flush alone, each between two events and each after a flush that leaves the caches clean, and takes the
        difference."""
        torch = self.torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        torch.cuda.synchronize()
        for e in ev:
            self.flush()
            e[0].record(self.stream)
            self.flush()
            fn()
            e[1].record(self.stream)
            self.flush()
            e[2].record(self.stream)
            self.flush()
            e[3].record(self.stream)
        torch.cuda.synchronize()
        return [1e3 * (e[0].elapsed_time(e[1]) - e[2].elapsed_time(e[3])) for e in ev]

    def cold(self, fn, n):
        """n calls of fn, each after a flush that is outside its events; returns the per-call times (us)."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            self.flush()
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return [1e3 * a.elapsed_time(b) for a, b in ev]

    def cold_split(self, fns, n):
        """n cold steps of the calls fns (flush, then an event between consecutive calls): per-call times."""
        torch = self.torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n)]
        torch.cuda.synchronize()
        for row in ev:
            self.flush()
            row[0].record(self.stream)
            for k, fn in enumerate(fns):
                fn()
                row[k + 1].record(self.stream)
        torch.cuda.synchronize()
        return [[1e3 * row[k].elapsed_time(row[k + 1]) for row in ev] for k in range(len(fns))]

    def warm(self, fn, n):
        """n calls back to back between two events; returns the mean time per call (us)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(n):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n


def measure_roofs(timer):
    """What the chip sustains: a cold streaming read of 4 GiB (plain and non-temporal loads, the faster
    kept), a register-only bf16 matrix-core loop, and the cost of an event pair around an empty kernel."""
    import torch
    from mla_latent_kv_14_amd import roofs

    dev = "cuda:0"
    out = {}
    try:
        buf = torch.empty(READ_PEAK_BYTES // 4, dtype=torch.int32, device=dev)
    except RuntimeError:
        buf = torch.empty((READ_PEAK_BYTES // 4) // 4, dtype=torch.int32, device=dev)
    buf.fill_(1)
    sink = torch.zeros(max(roofs.read_grid(), 1) + 64, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * 4
    best = 0.0
    for nt in (False, True):
        roofs.hbm_read(buf, sink, nt, timer.stream)  # warm-up of the code path
        t = stats(timer.cold(lambda: roofs.hbm_read(buf, sink, nt, timer.stream), 5))
        gbs = nbytes / (t["p50"] * 1e-6) / 1e9
        out["hbm_read_nt" if nt else "hbm_read"] = {"bytes": nbytes, "us_p50": t["p50"], "gbs": gbs}
        best = max(best, gbs)
    out["hbm_read_gbs"] = best
    del buf
    msink = torch.zeros(roofs.mfma_grid() * 4 + 64, dtype=torch.int32, device=dev)
    iters = 20000
    flops = roofs.mfma_bf16(iters, msink, timer.stream)
    t = stats(timer.cold(lambda: roofs.mfma_bf16(iters, msink, timer.stream), 5))
    out["mfma_bf16"] = {"flops": flops, "us_p50": t["p50"], "tflops": flops / (t["p50"] * 1e-6) / 1e12}
    out["mfma_bf16_tflops"] = out["mfma_bf16"]["tflops"]
    e = stats(timer.cold(lambda: roofs.empty(timer.stream), 20))
    out["event_pair_empty_kernel_us"] = e["p50"]
    log(f"bench: roofs: HBM read {best:.0f} GB/s (spec {HBM_PEAK_GBS:.0f}), bf16 MFMA "
        f"{out['mfma_bf16_tflops']:.0f} TFLOP/s (spec {MFMA_BF16_PEAK_TFLOPS:.0f}), event pair + empty kernel "
        f"{e['p50']:.1f} us")
    return out


def roofline(alg_bytes, flops, kernel_us, peaks, traffic=None, kernel="mla_decode attention"):
    """Both roofs for one kernel.  The bound is the roof whose floor is the longer time at the published
    peaks (arithmetic intensity against the published ridge point); frac is against that roof's published
    peak, frac_measured against what libmla_roofs measured on this chip."""
    s = kernel_us * 1e-6
    gbs = alg_bytes / s / 1e9
    tflops = flops / s / 1e12
    ai = flops / alg_bytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "hbm" if ai < ridge else "mfma"
    hbm_m, mfma_m = peaks.get("hbm_read_gbs"), peaks.get("mfma_bf16_tflops")
    rec = {"kernel": kernel, "kernel_us": kernel_us, "bound": bound,
           "achieved": gbs if bound == "hbm" else tflops,
           "peak": HBM_PEAK_GBS if bound == "hbm" else MFMA_BF16_PEAK_TFLOPS,
           "unit": "GB/s" if bound == "hbm" else "TFLOP/s", "traffic": traffic,
           "alg_bytes_per_launch": alg_bytes, "flops_per_launch": flops, "arith_intensity": ai,
           "ridge_spec": ridge,
           "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
           "hbm_frac_measured": gbs / hbm_m if hbm_m else None,
           "mfma_tflops": tflops, "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
           "mfma_frac_measured": tflops / mfma_m if mfma_m else None}
    rec["frac"] = rec["hbm_frac"] if bound == "hbm" else rec["mfma_frac"]
    rec["frac_measured"] = rec["hbm_frac_measured"] if bound == "hbm" else rec["mfma_frac_measured"]
    return rec


def measure_decode(prob, timer, K, warmup, peaks, cold_only=False, traffic=None, label=None):
    """Cold steps, cold per-call breakdown, cold attention-kernel launches (and warm figures unless
    cold_only) for one decode workload."""
    import torch
    from mla_latent_kv_14_amd.runner import DecodeRunner

    wl = prob.wl
    r = DecodeRunner(prob, device="cuda:0")
    calls = [("absorb_q_plan", r.absorb_q_plan), ("decode", r.decode_planned),
             ("combine_absorb_out", r.combine_absorb_out)]

    def step():
        for _, fn in calls:
            fn()

    for _ in range(warmup):
        if cold_only:
            timer.flush()
        step()
    torch.cuda.synchronize()
    step_t = stats(timer.cold_net(step, K))
    per_call = timer.cold_split([fn for _, fn in calls], K)
    per_call = {n: stats(t) for (n, _), t in zip(calls, per_call)}
    kern = stats(timer.cold(r.decode_planned, K))
    kern_net = stats(timer.cold_net(r.decode_planned, K))
    kern_mean = kern_net["mean"]
    alg_bytes, flops = algorithmic_work(prob)
    rec = {"workload": label or wl.name, "batch": wl.batch, "heads": wl.heads, "q_len": wl.q_len,
           "context_tokens": prob.total_tokens, "num_splits": r.num_splits,
           "step_us": step_t, "per_call_us": per_call,
           "attention_kernel_us": dict(kern_net, with_event_pair=kern,
                                       note="each sample: (flush, kernel) minus a flush alone, each between two "
                                            "events and after a clean flush, so the event pair's own cost cancels; "
                                            "its mean is the roofline's kernel time; with_event_pair: the kernel "
                                            "alone between two events"),
           "tokens_per_s": wl.batch * wl.q_len / (step_t["mean"] * 1e-6),
           "roofline": roofline(alg_bytes, flops, kern_mean, peaks, traffic)}
    if not cold_only:
        timer.write_flush = True
        rec["attention_after_write_flush_us"] = stats(timer.cold(r.decode_planned, K))["mean"]
        timer.write_flush = False
    if not cold_only:
        rec["warm"] = {"step_us": timer.warm(step, K), "attention_kernel_us": timer.warm(r.decode_planned, K),
                       "note": "back-to-back launches with caches warm; not used for any roofline figure"}
    rl = rec["roofline"]
    log(f"bench: {rec['workload']}: step {step_t['mean']:.1f} us cold (p10 {step_t['p10']:.1f}, p90 "
        f"{step_t['p90']:.1f}); attention {kern_mean:.1f} us cold (events {kern['mean']:.1f}, after a write flush "
        f"{rec.get('attention_after_write_flush_us', 0):.1f}) = {rl['hbm_gbs']:.0f} GB/s "
        f"({100 * rl['hbm_frac']:.1f}% HBM spec, {100 * (rl['hbm_frac_measured'] or 0):.1f}% measured), "
        f"{rl['mfma_tflops']:.0f} TFLOP/s ({100 * rl['mfma_frac']:.1f}% MFMA spec)")
    return rec, r


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


def measure_folds(prob, r, timer, K, warmup):
    """The offline folds and the fused products, with the unfolded route beside them (cold calls).

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

    fold_q = lambda: libmla.mla_fold_query_weight(d, fi.d_in, w_in, w_uk, wq)
    fold_o = lambda: libmla.mla_fold_output_weight(d, fi.d_out, w_o, w_uv, wo)
    fold_q()
    fold_o()
    fold_q_us, fold_o_us = stats(timer.cold(fold_q, 2))["mean"], stats(timer.cold(fold_o, 2))["mean"]

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
    fq_us, fo_us = stats(timer.cold(fq, K))["mean"], stats(timer.cold(fo, K))["mean"]
    uq_us, uo_us = stats(timer.cold(unfolded_q, K))["mean"], stats(timer.cold(unfolded_o, K))["mean"]
    esz = 2 if dt == torch.bfloat16 else 4
    q_bytes = wq.numel() * esz + x.numel() * esz + q_rope.numel() * esz + q_cat.numel() * esz
    o_bytes = wo.numel() * esz + o.numel() * 4 + y.numel() * esz
    res = {
        "d_in": fi.d_in, "d_out": fi.d_out, "timing": "cold",
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
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other decode workloads")
    ap.add_argument("--cold-only", action="store_true",
                    help="main workload only, every launch cold (warm-up included): for kernel traces")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache twin of the workload")
    ap.add_argument("--no-folds", action="store_true", help="skip the weight folds and fused products")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libmla has no multi-GPU path (whole sequences would shard "
              "across GPUs with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mla_latent_kv_14_amd.inputs import WORKLOADS, make_append_inputs, make_prefill_problem, make_problem, workload
    from mla_latent_kv_14_amd.runner import PrefillRunner

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0")
    timer = Timer(stream, flush_buf)
    K, W = args.steps, args.warmup
    cold_only = args.cold_only

    peaks = {} if cold_only else measure_roofs(timer)
    if cold_only:
        # two 1 GiB write flushes: a kernel of known write size beside the 1 GiB read flushes, so that
        # HBM byte counters taken over this run can be calibrated
        timer.roofs.flush(flush_buf, stream)
        timer.roofs.flush(flush_buf, stream)
        torch.cuda.synchronize()

    wl = workload(args.workload)
    log(f"bench: generating {wl.name} ...")
    prob = make_problem(wl, args.seed)
    traffic = measured_traffic(wl.name)
    main_rec, r = measure_decode(prob, timer, K, W, peaks, cold_only=cold_only, traffic=traffic)
    log(f"bench: B={wl.batch} H={wl.heads} Lq={wl.q_len} tokens={prob.total_tokens} splits={r.num_splits}")

    configs = []
    if not args.no_configs and not cold_only:
        for name in OTHER_WORKLOADS:
            if name == wl.name:
                continue
            p2 = make_problem(workload(name))
            rec2, r2 = measure_decode(p2, timer, min(K, 20), min(W, 3), peaks)
            configs.append(rec2)
            del r2, p2
            torch.cuda.empty_cache()

    append = None
    if not cold_only:
        # the cache append (the step just before attention in a decode loop),
        # timed on its own, cold; it rewrites the same slots every call
        app = make_append_inputs(prob)
        r.setup_append(app)
        for _ in range(W):
            r.cache_append()
        at = stats(timer.cold_net(r.cache_append, K))
        ap_bytes, ap_flops = append_work(prob, app.d_model)
        append = {"us": at, "with_event_pair_us": stats(timer.cold(r.cache_append, K)), "launches": 2,
                  "d_model": app.d_model, "alg_bytes": ap_bytes,
                  "gbs": ap_bytes / (at["mean"] * 1e-6) / 1e9,
                  "hbm_frac": ap_bytes / (at["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                  "tflops": ap_flops / (at["mean"] * 1e-6) / 1e12}
        log(f"bench: cache append {at['mean']:.1f} us/call cold (d_model={app.d_model})")

    prefill = None
    if not args.no_prefill and not cold_only:
        pprob = make_prefill_problem(workload(PREFILL_WORKLOAD))
        pr = PrefillRunner(pprob, device="cuda:0")
        for _ in range(2):
            pr.prefill()
        pt = stats(timer.cold(pr.prefill, 5))
        pms = pt["mean"] / 1e3
        f_attn, f_up = prefill_work(pprob)
        prefill = {"workload": PREFILL_WORKLOAD, "tokens": pprob.total_tokens, "heads": pprob.wl.heads,
                   "causal": True, "ms_per_call": pms, "us": pt, "tokens_per_s": pprob.total_tokens / (pms * 1e-3),
                   "attn_tflop": f_attn / 1e12, "upproject_tflop": f_up / 1e12,
                   "tflops": (f_attn + f_up) / (pms * 1e-3) / 1e12,
                   "mfma_frac": (f_attn + f_up) / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                   "mfma_frac_measured": ((f_attn + f_up) / (pms * 1e-3) / 1e12 / peaks["mfma_bf16_tflops"]
                                          if peaks.get("mfma_bf16_tflops") else None)}
        log(f"bench: prefill {PREFILL_WORKLOAD}: {pms:.2f} ms cold, {prefill['tflops']:.0f} TFLOP/s")
        del pr, pprob
        torch.cuda.empty_cache()

    fp8 = None
    twin = wl.name.replace("_bf16", "_fp8")
    if not args.no_fp8 and not cold_only and not prob.fp8 and twin in WORKLOADS:
        fprob = make_problem(workload(twin), args.seed)
        fp8, fr = measure_decode(fprob, timer, K, W, peaks)
        fp8["kv_scale"] = fprob.kv_scale
        fp8["cache_bytes"] = int(fprob.cache.numel())
        del fr, fprob
        torch.cuda.empty_cache()

    folds = None
    if not args.no_folds and not cold_only:
        folds = measure_folds(prob, r, timer, min(K, 20), W)

    cpu = None
    if not args.no_cpu_baseline and not cold_only:
        log("bench: timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(prob)

    ms_step = main_rec["step_us"]["mean"] / 1e3
    tokens = wl.batch * wl.q_len
    alg_bytes, flops = algorithmic_work(prob)
    rec = {
        "metric": "MLA decode tokens/s + TFLOP/s & HBM GB/s vs roofline, B=64 H=128 ctx 1K-8K",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "timing": ("cold: a 1 GiB read flush before every timed step; per step, (flush, step) minus a flush alone, "
                   "each between two HIP events on the library's stream; value = tokens / mean"),
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "q_len": wl.q_len, "d_c": wl.d_c,
                   "d_rope": wl.d_rope, "d_nope": wl.d_nope, "d_v": wl.d_v, "block_size": wl.block_size,
                   "context_tokens": prob.total_tokens, "lengths": " ".join(str(x) for x in wl.lengths),
                   "num_splits": r.num_splits},
        "roofline": main_rec["roofline"],
        "step_us": main_rec["step_us"],
        "attention_kernel_us": main_rec["attention_kernel_us"],
        "per_call_us": main_rec["per_call_us"],
        "warm": main_rec.get("warm"),
        "step_tflops": flops / (ms_step * 1e-3) / 1e12,
        "step_gbs": alg_bytes / (ms_step * 1e-3) / 1e9,
        "measured_roofs": peaks,
        "configs": configs,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "fp8_cache": fp8,
        "weight_folds": folds,
        "cache_append": append,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
