"""Device-resident buffers for one decode problem plus the three-launch step.

Allocation and upload use torch (device memory only); every step of the
computation is a libmla call.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as libmla
from .inputs import Problem


class DecodeRunner:
    """Holds a problem's inputs, workspace and outputs on one device."""

    def __init__(self, prob: Problem, device="cuda", num_splits: Optional[int] = None):
        self.prob = prob
        wl = prob.wl
        self.device = torch.device(device)
        self.dims = libmla.make_dims(wl.batch, wl.q_len, wl.heads, wl.d_c, wl.d_rope, wl.d_nope, wl.d_v,
                                     wl.block_size, prob.max_blocks, prob.num_blocks,
                                     torch.float32 if wl.dtype == "f32" else torch.bfloat16)
        dev = self.device
        self.cache = prob.cache.to(dev)
        self.q_nope = prob.q_nope.to(dev)
        self.q_rope = prob.q_rope.to(dev)
        self.w_uk = prob.w_uk.to(dev)
        self.w_uv = prob.w_uv.to(dev)
        self.block_table = torch.from_numpy(np.ascontiguousarray(prob.block_table)).to(dev)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(prob.seq_lens)).to(dev)
        self.fp8 = prob.fp8  # the cache holds E4M3 codes standing for prob.kv_scale * value
        if num_splits is None:
            sizing = libmla.mla_decode_num_splits_fp8 if self.fp8 else libmla.mla_decode_num_splits
            num_splits = sizing(self.dims, int(prob.seq_lens.max()), prob.total_tokens)
        self.num_splits = int(num_splits)
        B, Lq, H = wl.batch, wl.q_len, wl.heads
        st = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        self.q_cat = torch.empty((B, Lq, H, wl.d_c + wl.d_rope), dtype=st, device=dev)
        ws_bytes = libmla.mla_decode_workspace_bytes(self.dims, self.num_splits)
        self.workspace = torch.empty(ws_bytes // 4, dtype=torch.int32, device=dev)
        self.o_partial = torch.empty((B, Lq, H, self.num_splits, wl.d_c), dtype=st, device=dev)  # storage type
        self.lse_partial = torch.empty((B, Lq, H, self.num_splits), dtype=torch.float32, device=dev)
        self.o = torch.empty((B, Lq, H, wl.d_c), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Lq, H), dtype=torch.float32, device=dev)
        self.u = torch.empty((B, Lq, H, wl.d_v), dtype=st, device=dev)

    def setup_append(self, app):
        """Upload the inputs of a cache append (``inputs.AppendInputs``) and size its workspace."""
        dev = self.device
        self.app = app
        self.h = app.h.to(dev)
        self.w_dkv = app.w_dkv.to(dev)
        self.w_kr = app.w_kr.to(dev)
        nbytes = libmla.mla_cache_append_workspace_bytes(self.dims, app.d_model)
        self.append_ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=dev) if nbytes else None

    def cache_append(self, stream=None):
        """Write the new tokens' rows [W^DKV h | RoPE(W^KR h)] into self.cache (as E4M3 codes of
        row / kv_scale for an FP8 cache)."""
        if self.fp8:
            libmla.mla_cache_append_fp8(self.dims, self.app.d_model, self.h, self.w_dkv, self.w_kr,
                                        self.app.rope_base, self.prob.kv_scale, self.block_table, self.seq_lens,
                                        self.cache, self.append_ws, stream)
        else:
            libmla.mla_cache_append(self.dims, self.app.d_model, self.h, self.w_dkv, self.w_kr, self.app.rope_base,
                                    self.block_table, self.seq_lens, self.cache, self.append_ws, stream)

    def absorb_q(self, stream=None):
        libmla.mla_absorb_q(self.dims, self.q_nope, self.q_rope, self.w_uk, self.q_cat, stream)

    def decode(self, stream=None):
        if self.fp8:
            libmla.mla_decode_fp8(self.dims, self.q_cat, self.cache, self.prob.kv_scale, self.block_table,
                                  self.seq_lens, self.prob.scale, self.num_splits, self.workspace, self.o_partial,
                                  self.lse_partial, stream)
        else:
            libmla.mla_decode(self.dims, self.q_cat, self.cache, self.block_table, self.seq_lens, self.prob.scale,
                              self.num_splits, self.workspace, self.o_partial, self.lse_partial, stream)

    def plan(self, stream=None):
        planner = libmla.mla_decode_plan_fp8 if self.fp8 else libmla.mla_decode_plan
        planner(self.dims, self.seq_lens, self.num_splits, self.workspace, stream)

    def decode_planned(self, stream=None):
        if self.fp8:
            libmla.mla_decode_planned_fp8(self.dims, self.q_cat, self.cache, self.prob.kv_scale, self.block_table,
                                          self.prob.scale, self.num_splits, self.workspace, self.o_partial,
                                          self.lse_partial, stream)
        else:
            libmla.mla_decode_planned(self.dims, self.q_cat, self.cache, self.block_table, self.prob.scale,
                                      self.num_splits, self.workspace, self.o_partial, self.lse_partial, stream)

    def combine(self, stream=None):
        libmla.mla_combine(self.dims, self.num_splits, self.o_partial, self.lse_partial, self.o, self.lse, stream)

    def absorb_out(self, stream=None):
        libmla.mla_absorb_out(self.dims, self.o, self.w_uv, self.u, stream)

    def combine_absorb_out(self, keep_latent=False, stream=None):
        """Merge the splits and apply W_UV in one call (the latent output is
        written to self.o only when asked, or when the call is not fused)."""
        fused = libmla.mla_combine_absorb_out_fused(self.dims, self.num_splits)
        libmla.mla_combine_absorb_out(self.dims, self.num_splits, self.o_partial, self.lse_partial, self.w_uv, self.u,
                                      self.o if (keep_latent or not fused) else None,
                                      self.lse if (keep_latent or not fused) else None, stream)

    def absorb_q_plan(self, stream=None):
        """absorb_q and the plan in one launch (the planner runs as one more workgroup)."""
        fn = libmla.mla_absorb_q_plan_fp8 if self.fp8 else libmla.mla_absorb_q_plan
        fn(self.dims, self.q_nope, self.q_rope, self.w_uk, self.q_cat, self.seq_lens, self.num_splits,
           self.workspace, stream)

    def fused_step(self, stream=None):
        """One decode step as the bench runs it: absorb_q with the plan, attention, fused merge + W_UV
        (three launches)."""
        self.absorb_q_plan(stream)
        self.decode_planned(stream)
        self.combine_absorb_out(stream=stream)

    def capture(self, steps=1):
        """Record `steps` consecutive fused_steps into one HIP graph
        (torch.cuda.CUDAGraph) and return it.

        The libmla calls enqueue kernels only (no memsets, no allocation), so
        the graph holds exactly the three kernels of each step."""
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            self.fused_step()  # warm-up on the capture stream
        torch.cuda.current_stream(self.device).wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.fused_step()
        return g

    def step(self, stream=None):
        """One full decode step: absorb_q -> decode -> combine -> absorb_out."""
        self.absorb_q(stream)
        self.decode(stream)
        self.combine(stream)
        self.absorb_out(stream)


class PrefillRunner:
    """Device-resident buffers for one prefill problem and the mla_prefill call."""

    def __init__(self, prob, device="cuda", causal=True):
        self.prob = prob
        wl = prob.wl
        self.device = torch.device(device)
        self.causal = bool(causal)
        st = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        self.dims = libmla.make_dims(wl.batch, 1, wl.heads, wl.d_c, wl.d_rope, wl.d_nope, wl.d_v, 1, 1, 1, st)
        dev = self.device
        T = prob.total_tokens
        self.cu = torch.from_numpy(np.ascontiguousarray(prob.cu_seqlens)).to(dev)
        self.q_nope, self.q_rope = prob.q_nope.to(dev), prob.q_rope.to(dev)
        self.c_kv, self.k_rope = prob.c_kv.to(dev), prob.k_rope.to(dev)
        self.w_uk, self.w_uv = prob.w_uk.to(dev), prob.w_uv.to(dev)
        self.max_seqlen = max(int(prob.seq_lens.max()), 1)
        nbytes = libmla.mla_prefill_workspace_bytes(self.dims, T)
        self.workspace = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
        self.u = torch.empty((T, wl.heads, wl.d_v), dtype=st, device=dev)
        self.lse = torch.empty((T, wl.heads), dtype=torch.float32, device=dev)

    def prefill(self, stream=None):
        libmla.mla_prefill(self.dims, self.prob.total_tokens, self.max_seqlen, self.cu, self.q_nope, self.q_rope,
                           self.c_kv, self.k_rope, self.w_uk, self.w_uv, self.prob.scale, self.causal, self.u,
                           self.workspace, self.lse, stream)
