"""Seeded synthetic workloads for absorbed MLA decode over a paged latent cache.

This module only draws numbers and lays them out; it performs none of the
attention arithmetic.  It is the one piece shared by the HIP path (tests,
bench) and the CPU oracle, which both receive the arrays it returns.

Shapes follow DeepSeek-V2/V3 attention: n_h = 128 heads, per-head content
width d_h = 128, KV latent width d_c = 512 and decoupled RoPE width 64
("DeepSeek-V2 Multi-Head Latent Attention" knowledge note, Query Compression
table; "DeepSeek-V3 MLA: Multi-Head Latent Attention Guide", Core
Architecture section 1).  Every cache row holds ``[c_kv (d_c) | k_rope
(d_rope)]``, the two quantities that page's cache rule keeps per token.

Recipe:
  * one ``numpy.random.Generator(PCG64(seed))`` per problem, draws in the
    order: lengths, block permutation, cache, q_nope, q_rope, W_UK, W_UV;
  * values are drawn in float64, cast to float32 and, for bf16 problems,
    rounded once to bf16 (round-to-nearest-even through torch);
  * latents, rope keys and queries ~ N(0, 1); W_UK and W_UV ~ N(0, 1)/sqrt(d_c)
    (d_c is the fan-in of k = W c);
  * the paged pool holds exactly sum_b ceil(L_b / bs) blocks whose physical
    order is a random permutation; table rows are padded with -1;
  * cache slots past a sequence's length in its last block are poisoned
    (NaN by default) because nothing may read them.

Cache-append inputs (``make_append_inputs``) come from a second generator,
``PCG64([seed, 0xA99E])``, so adding them moves none of the draws above:
hidden states h ~ N(0, 1) of width d_model (7168 for the DeepSeek-V3 shapes,
the input width of the Guide's MLA topology figure), then W^DKV and W^KR ~
N(0, 1)/sqrt(d_model) (fan-in d_model), rounded like the rest.

FP8 cache workloads (``cache_dtype="fp8"``) draw exactly the same numbers;
the cache values are then stored as E4M3 codes of value / kv_scale, clipped
to +-448 and rounded by torch's float8_e4m3fn cast (round to nearest even),
so each code stands for kv_scale times its value.  kv_scale = 0.0175 puts
7.8 standard deviations at the top of the format's range.  Poisoned slots
hold the NaN code 0x7F ("nan") or the codes of +-448 ("big").

Prefill problems (``make_prefill_problem``, the prefill_* workloads) come
from ``PCG64([seed, 0x9F11])``: lengths by the workload's distribution, then
the tokens' latents c ~ N(0, 1), RoPE keys ~ N(0, 1), q_nope, q_rope ~ N(0, 1)
per (token, head), then W_UK, W_UV ~ N(0, 1)/sqrt(d_c); the tokens of all
sequences are packed in sequence order.

Weight-fold inputs (``make_fold_inputs``) come from ``PCG64([seed, 0xF01D])``:
the query projection's input x ~ N(0, 1) of width d_in (1536, the query
latent width of the DeepSeek-V2/V3 shapes), the per-head content query
projection W_in ~ N(0, 1)/sqrt(d_in) [H, d_nope, d_in], the output projection
W^O ~ N(0, 1)/sqrt(H d_v) [d_out, H d_v] (d_out = the model width, 7168), and
a merged latent attention output o ~ N(0, 1)/4 in float32 [B, Lq, H, d_c] (a
softmax-weighted mean of unit-variance latent rows, so well under 1).
``synthetic_fused_output_weight`` draws a stand-in for W~^O ~ N(0, 1)/256
[d_out, H d_c] from ``PCG64([seed, 0xF01E])`` for the full-size product test,
where folding the real weight in float64 would take minutes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "Problem", "make_problem", "workload", "AppendInputs", "make_append_inputs",
           "PrefillProblem", "make_prefill_problem", "FoldInputs", "make_fold_inputs", "synthetic_fused_output_weight"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named decode workload: dimensions plus the length distribution."""

    name: str
    dtype: str  # "f32" or "bf16": storage type of q, cache and weights
    batch: int
    heads: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    q_len: int
    block_size: int
    lengths: tuple  # ("fixed", (L0, L1, ...)) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    seed_base: int
    d_model: int = 7168  # hidden width h feeding the cache append
    cache_dtype: str = "same"  # "same" (the storage type) or "fp8" (E4M3 codes)
    kv_scale: float = 1.0  # FP8 cache: a code stands for kv_scale * its value

    @property
    def row_width(self) -> int:
        return self.d_c + self.d_rope

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(d_nope + d_rope); the caller always passes it
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)


FP8_KV_SCALE = 0.0175  # 448 * 0.0175 = 7.84: the E4M3 range covers 7.8 sigma of N(0, 1) latents

WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", "f32", 2, 8, 64, 16, 32, 32, 1, 16, ("fixed", (37, 200)), 1000, 96),
        Workload("single_4k_bf16", "bf16", 1, 128, 512, 64, 128, 128, 1, 64, ("fixed", (4096,)), 2000),
        Workload("batch64_1k8k_bf16", "bf16", 64, 128, 512, 64, 128, 128, 1, 64, ("uniform", 1024, 8192), 3000),
        Workload("long128k_bf16", "bf16", 4, 128, 512, 64, 128, 128, 1, 64, ("fixed", (131072,) * 4), 4000),
        Workload("mtp2_lognormal_bf16", "bf16", 128, 16, 512, 64, 128, 128, 2, 64,
                 ("lognormal", 2048, 1.0, 64, 32768), 5000),
        # FP8 (E4M3) latent cache: the same draws as their bf16 twins
        Workload("tiny_f32_fp8", "f32", 2, 8, 64, 16, 32, 32, 1, 16, ("fixed", (37, 200)), 1000, 96, "fp8",
                 FP8_KV_SCALE),
        Workload("single_4k_fp8", "bf16", 1, 128, 512, 64, 128, 128, 1, 64, ("fixed", (4096,)), 2000, 7168, "fp8",
                 FP8_KV_SCALE),
        Workload("batch64_1k8k_fp8", "bf16", 64, 128, 512, 64, 128, 128, 1, 64, ("uniform", 1024, 8192), 3000,
                 7168, "fp8", FP8_KV_SCALE),
        Workload("mtp2_lognormal_fp8", "bf16", 128, 16, 512, 64, 128, 128, 2, 64,
                 ("lognormal", 2048, 1.0, 64, 32768), 5000, 7168, "fp8", FP8_KV_SCALE),
        # prefill (whole sequences as queries; q_len and block_size unused)
        Workload("prefill_tiny_f32", "f32", 3, 4, 64, 16, 32, 32, 1, 16, ("fixed", (5, 1, 70)), 6000, 96),
        Workload("prefill_4x4k_bf16", "bf16", 4, 128, 512, 64, 128, 128, 1, 64, ("fixed", (4096,) * 4), 7000),
        Workload("prefill_mixed_bf16", "bf16", 8, 128, 512, 64, 128, 128, 1, 64, ("uniform", 128, 4096), 8000),
    ]
}


def workload(name: str, **overrides) -> Workload:
    """Return a named workload, optionally with fields replaced (smaller test sizes)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


@dataclasses.dataclass
class Problem:
    """One drawn problem.  Tensors live on the CPU in the storage dtype."""

    wl: Workload
    seed: int
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, MB], -1 padded
    cache: torch.Tensor  # [NB, bs, d_c + d_rope]
    q_nope: torch.Tensor  # [B, Lq, H, d_nope]
    q_rope: torch.Tensor  # [B, Lq, H, d_rope]
    w_uk: torch.Tensor  # [H, d_nope, d_c]
    w_uv: torch.Tensor  # [H, d_v, d_c]

    @property
    def num_blocks(self) -> int:
        return int(self.cache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def scale(self) -> float:
        return self.wl.scale

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    @property
    def fp8(self) -> bool:
        return self.wl.cache_dtype == "fp8"

    @property
    def kv_scale(self) -> float:
        return float(self.wl.kv_scale)

    def f64(self, name: str) -> np.ndarray:
        """A stored tensor upcast exactly to float64 (what the oracle consumes).
        An FP8 cache holds codes, not values: the oracle decodes those itself."""
        if name == "cache" and self.fp8:
            raise ValueError("the FP8 cache holds E4M3 codes; decode them with the oracle")
        return getattr(self, name).to(torch.float64).numpy()


def _draw_lengths(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = wl.lengths[0]
    if kind == "fixed":
        vals = np.asarray(wl.lengths[1], dtype=np.int64)
        if vals.size != wl.batch:
            vals = np.resize(vals, wl.batch)
    elif kind == "uniform":
        lo, hi = wl.lengths[1], wl.lengths[2]
        vals = rng.integers(lo, hi, size=wl.batch, endpoint=True)
    elif kind == "lognormal":
        median, sigma, lo, hi = wl.lengths[1:]
        vals = np.clip(np.rint(np.exp(math.log(median) + sigma * rng.standard_normal(wl.batch))), lo, hi)
    else:
        raise ValueError(f"unknown length distribution {kind!r}")
    vals = vals.astype(np.int64)
    if (vals < wl.q_len).any():
        raise ValueError("every sequence must hold at least q_len tokens")
    return vals.astype(np.int32)


def _store(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_problem(wl: Workload, seed: Optional[int] = None, *, poison: Optional[str] = "nan",
                 seq_lens: Optional[np.ndarray] = None) -> Problem:
    """Draw one problem.  ``seed`` defaults to the workload's base seed.

    ``seq_lens`` overrides the drawn lengths (edge-case tests); the RNG still
    draws them first so the rest of the stream does not move.
    ``poison`` fills never-visible cache slots: "nan", "big" (+-1e4) or None.
    """
    seed = wl.seed_base if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = _draw_lengths(wl, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
        if lens.shape != (wl.batch,) or (lens < wl.q_len).any():
            raise ValueError("bad seq_lens override")
    bs = wl.block_size
    nblk = (lens.astype(np.int64) + bs - 1) // bs
    nb_total = int(nblk.sum())
    mb = int(nblk.max()) if wl.batch else 0
    perm = rng.permutation(nb_total).astype(np.int32)
    table = np.full((wl.batch, max(mb, 1)), -1, dtype=np.int32)
    pos = 0
    for b in range(wl.batch):
        table[b, : nblk[b]] = perm[pos: pos + nblk[b]]
        pos += nblk[b]

    D = wl.row_width
    if wl.cache_dtype == "fp8":
        vals = np.clip(rng.standard_normal((nb_total, bs, D)) / wl.kv_scale, -448.0, 448.0)
        cache = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        cache = _store(rng.standard_normal((nb_total, bs, D)), wl.dtype)
    q_nope = _store(rng.standard_normal((wl.batch, wl.q_len, wl.heads, wl.d_nope)), wl.dtype)
    q_rope = _store(rng.standard_normal((wl.batch, wl.q_len, wl.heads, wl.d_rope)), wl.dtype)
    inv = 1.0 / math.sqrt(wl.d_c)
    w_uk = _store(rng.standard_normal((wl.heads, wl.d_nope, wl.d_c)) * inv, wl.dtype)
    w_uv = _store(rng.standard_normal((wl.heads, wl.d_v, wl.d_c)) * inv, wl.dtype)

    if poison is not None:
        for b in range(wl.batch):
            tail = int(lens[b]) % bs
            if tail:
                blk = int(table[b, nblk[b] - 1])
                if wl.cache_dtype == "fp8":
                    if poison == "nan":
                        cache[blk, tail:, :] = 0x7F
                    elif poison == "big":
                        codes = torch.full((bs - tail, D), 0x7E, dtype=torch.uint8)
                        codes[1::2] = 0xFE
                        cache[blk, tail:, :] = codes
                    else:
                        raise ValueError(f"unknown poison {poison!r}")
                elif poison == "nan":
                    cache[blk, tail:, :] = float("nan")
                elif poison == "big":
                    sign = torch.ones(bs - tail, D)
                    sign[1::2] = -1.0
                    cache[blk, tail:, :] = (1e4 * sign).to(cache.dtype)
                else:
                    raise ValueError(f"unknown poison {poison!r}")
    return Problem(wl, seed, lens, table, cache, q_nope, q_rope, w_uk, w_uv)


ROPE_BASE = 10000.0  # the apply_rope base of the DeepSeek V4 Pro MLA module


@dataclasses.dataclass
class AppendInputs:
    """Inputs of one cache append.  Tensors live on the CPU in the storage dtype."""

    d_model: int
    h: torch.Tensor  # [B, Lq, d_model]
    w_dkv: torch.Tensor  # [d_c, d_model]
    w_kr: torch.Tensor  # [d_rope, d_model]
    rope_base: float = ROPE_BASE

    def f64(self, name: str) -> np.ndarray:
        return getattr(self, name).to(torch.float64).numpy()


def make_append_inputs(prob: Problem, d_model: Optional[int] = None) -> AppendInputs:
    """Draw the hidden states and projection weights of the new tokens of ``prob``."""
    wl = prob.wl
    d_model = wl.d_model if d_model is None else int(d_model)
    rng = np.random.Generator(np.random.PCG64([prob.seed, 0xA99E]))
    h = _store(rng.standard_normal((wl.batch, wl.q_len, d_model)), wl.dtype)
    inv = 1.0 / math.sqrt(d_model)
    w_dkv = _store(rng.standard_normal((wl.d_c, d_model)) * inv, wl.dtype)
    w_kr = _store(rng.standard_normal((wl.d_rope, d_model)) * inv, wl.dtype)
    return AppendInputs(d_model, h, w_dkv, w_kr)


@dataclasses.dataclass
class PrefillProblem:
    """One drawn prefill problem: whole sequences, tokens packed.  CPU tensors, storage dtype."""

    wl: Workload
    seed: int
    seq_lens: np.ndarray  # int32 [B]
    cu_seqlens: np.ndarray  # int32 [B + 1]
    q_nope: torch.Tensor  # [T, H, d_nope]
    q_rope: torch.Tensor  # [T, H, d_rope]
    c_kv: torch.Tensor  # [T, d_c]
    k_rope: torch.Tensor  # [T, d_rope]
    w_uk: torch.Tensor  # [H, d_nope, d_c]
    w_uv: torch.Tensor  # [H, d_v, d_c]

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def scale(self) -> float:
        return self.wl.scale

    def f64(self, name: str) -> np.ndarray:
        return getattr(self, name).to(torch.float64).numpy()


def make_prefill_problem(wl: Workload, seed: Optional[int] = None, seq_lens: Optional[np.ndarray] = None) -> PrefillProblem:
    """Draw one prefill problem; ``seq_lens`` overrides the drawn lengths (drawn first all the same)."""
    seed = wl.seed_base if seed is None else seed
    rng = np.random.Generator(np.random.PCG64([seed, 0x9F11]))
    lens = _draw_lengths(wl, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
        if lens.shape != (wl.batch,) or (lens < 0).any():
            raise ValueError("bad seq_lens override")
    cu = np.concatenate([[0], np.cumsum(lens.astype(np.int64))]).astype(np.int32)
    T = int(cu[-1])
    c_kv = _store(rng.standard_normal((T, wl.d_c)), wl.dtype)
    k_rope = _store(rng.standard_normal((T, wl.d_rope)), wl.dtype)
    q_nope = _store(rng.standard_normal((T, wl.heads, wl.d_nope)), wl.dtype)
    q_rope = _store(rng.standard_normal((T, wl.heads, wl.d_rope)), wl.dtype)
    inv = 1.0 / math.sqrt(wl.d_c)
    w_uk = _store(rng.standard_normal((wl.heads, wl.d_nope, wl.d_c)) * inv, wl.dtype)
    w_uv = _store(rng.standard_normal((wl.heads, wl.d_v, wl.d_c)) * inv, wl.dtype)
    return PrefillProblem(wl, seed, lens, cu, q_nope, q_rope, c_kv, k_rope, w_uk, w_uv)


@dataclasses.dataclass
class FoldInputs:
    """Inputs of the weight folds and the fused products.  CPU tensors, storage dtype (o: float32)."""

    d_in: int
    d_out: int
    x: torch.Tensor  # [B, Lq, d_in]
    w_in: torch.Tensor  # [H, d_nope, d_in]
    w_o: torch.Tensor  # [d_out, H * d_v]
    o: torch.Tensor  # [B, Lq, H, d_c] float32

    def f64(self, name: str) -> np.ndarray:
        return getattr(self, name).to(torch.float64).numpy()


def make_fold_inputs(prob: Problem, d_in: int = 1536, d_out: Optional[int] = None) -> FoldInputs:
    """Draw the fold inputs belonging to ``prob`` (its q_rope, W_UK and W_UV complete them)."""
    wl = prob.wl
    d_out = wl.d_model if d_out is None else int(d_out)
    rng = np.random.Generator(np.random.PCG64([prob.seed, 0xF01D]))
    x = _store(rng.standard_normal((wl.batch, wl.q_len, d_in)), wl.dtype)
    w_in = _store(rng.standard_normal((wl.heads, wl.d_nope, d_in)) / math.sqrt(d_in), wl.dtype)
    w_o = _store(rng.standard_normal((d_out, wl.heads * wl.d_v)) / math.sqrt(wl.heads * wl.d_v), wl.dtype)
    o = torch.from_numpy((rng.standard_normal((wl.batch, wl.q_len, wl.heads, wl.d_c)) / 4).astype(np.float32))
    return FoldInputs(d_in, d_out, x, w_in, w_o, o)


def synthetic_fused_output_weight(prob: Problem, d_out: int) -> torch.Tensor:
    """A stand-in fused output weight [d_out, H d_c] in the storage dtype, drawn in float32 row blocks."""
    wl = prob.wl
    rng = np.random.Generator(np.random.PCG64([prob.seed, 0xF01E]))
    K = wl.heads * wl.d_c
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = torch.empty((d_out, K), dtype=dt)
    step = 256
    for r in range(0, d_out, step):
        n = min(step, d_out - r)
        blk = rng.standard_normal((n, K), dtype=np.float32) / np.float32(256.0)
        out[r:r + n] = torch.from_numpy(blk).to(dt)
    return out
