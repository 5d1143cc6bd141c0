"""CPU oracle for MLA decode over a paged latent cache -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this module.  The library never calls it and shares no code with it.

Everything here is plain float64 NumPy.  The main routine takes the
*non-absorbed* route: it up-projects every cached latent into per-head keys
and values, then runs textbook softmax attention.  That is the formulation of

  * "Deconstructing DeepSeek V4 Pro: Optimizing Multi-Head Latent Attention
    and Auxiliary-Loss-Free Load Balancing" -- Mathematical Formulation
    (K^C = c W_UK, V^C = c W_UV), Decoupled RoPE (K_t = [c W_UK, R(x W_KR)])
    and the forward pass of its PyTorch module (scale 1/sqrt(d_head+d_rope),
    softmax over the keys, weighted sum of the values);
  * "DeepSeek-V3 MLA: Multi-Head Latent Attention Guide" -- Core Architecture
    section 1 (k^C = W^UK c, v^C = W^UV c, W^UK in R^{(n_h d_h) x d_c}),
    section 3 (q = [q^C; q^R], k = [k^C; k^R] with one k^R shared by all
    heads) and its absorbed decode step, which appends the new token's latent
    before scoring so that the current token is part of the context;
  * "DeepSeek-V2 Multi-Head Latent Attention" knowledge note -- cache rule
    (only c^KV and k^R are cached per token).

Readings taken where the pages leave a step open: weights are stored
W_UK[h] in R^{d_nope x d_c}, W_UV[h] in R^{d_v x d_c} (a Linear weight
viewed per head); q_rope and the cached k_rope
are already rotated; sequence lengths include the q_len new tokens; for
q_len > 1, query j sees keys t <= L - q_len + j; lse is the natural-log
log-sum-exp of the *scaled* scores; a split with no visible key has
lse = -inf and contributes nothing to a merge.

Parity status: every function below is pinned in tests/test_oracle.py
against an independent route (absorbed algebra, a library attention routine,
pure-Python brute force, closed forms, or figures printed on the pages).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "gather_rows",
    "mla_decode_reference",
    "absorb_q_reference",
    "absorb_out_reference",
    "lse_merge_reference",
    "latent_attention_partial_reference",
    "cache_elements_per_token",
    "cache_bytes",
    "rope_reference",
    "cache_rows_reference",
    "cache_append_reference",
    "prefill_reference",
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "fp8_cache_values",
    "cache_append_fp8_reference",
    "fold_query_weight_reference",
    "fused_query_reference",
    "fold_output_weight_reference",
    "fused_output_reference",
]


def gather_rows(cache: np.ndarray, block_table: np.ndarray, b: int, length: int) -> np.ndarray:
    """Rows 0..length-1 of sequence b from a paged pool.

    Token t of sequence b sits in physical block block_table[b, t // bs] at
    slot t % bs.  Paging is not on the pages (they keep one contiguous tensor
    per sequence); this is its plain definition.
    """
    bs = cache.shape[1]
    rows = [cache[int(block_table[b, t // bs]), t % bs, :] for t in range(length)]
    return np.stack(rows, axis=0) if rows else np.zeros((0, cache.shape[2]), dtype=cache.dtype)


def _softmax_stats(s: np.ndarray):
    """Textbook softmax over the last axis with max subtraction (no mask, no extras)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def mla_decode_reference(q_nope, q_rope, cache, block_table, seq_lens, w_uk, w_uv, scale, d_c,
                         select=None):
    """Decode attention for every (sequence, new token, head), non-absorbed.

    Shapes: q_nope [B,Lq,H,d_n], q_rope [B,Lq,H,d_r], cache [NB,bs,d_c+d_r],
    block_table [B,MB], seq_lens [B], w_uk [H,d_n,d_c], w_uv [H,d_v,d_c].

    Returns (u [B,Lq,H,d_v], o [B,Lq,H,d_c], lse [B,Lq,H]) in float64:
      u   -- the per-head attention output sum_j p_j v_j (the primary result);
      o   -- the latent-weighted sum sum_j p_j c_j (secondary, for intermediates);
      lse -- log sum_j exp(score_j) of the scaled scores (secondary).
    ``select`` (optional iterable of (b, h)) restricts the work to those
    pairs, for spot checks at full size; every other entry is left NaN.
    The cache may be any array type that indexes like [block, slot, :].
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, Lq, H, _ = q_nope.shape
    d_v = w_uv.shape[1]
    u = np.full((B, Lq, H, d_v), np.nan)
    o = np.full((B, Lq, H, d_c), np.nan)
    lse = np.full((B, Lq, H), np.nan)
    wanted = None if select is None else {}
    if select is not None:
        for b, h in select:
            wanted.setdefault(int(b), []).append(int(h))
    for b in range(B):
        if wanted is not None and b not in wanted:
            continue
        L = int(seq_lens[b])
        if L < Lq or L > block_table.shape[1] * cache.shape[1]:
            raise ValueError(f"sequence {b}: length {L} outside [q_len, max_blocks * block_size]")
        rows = np.asarray(gather_rows(cache, block_table, b, L), dtype=np.float64)
        c = rows[:, :d_c]  # cached latent c^KV for every context token
        k_rope = rows[:, d_c:]  # cached, already-rotated shared RoPE key k^R
        for h in (range(H) if wanted is None else wanted[b]):
            k_content = c @ w_uk[h].T  # k^C_{t,h} = W^UK_h c_t       -> [L, d_n]
            v = c @ w_uv[h].T  # v^C_{t,h} = W^UV_h c_t             -> [L, d_v]
            keys = np.concatenate([k_content, k_rope], axis=1)  # k_{t,h} = [k^C; k^R]
            for j in range(Lq):
                last = L - Lq + j  # query j sees keys 0..last
                q = np.concatenate([q_nope[b, j, h], q_rope[b, j, h]])  # q = [q^C; q^R]
                s = scale * (keys[: last + 1] @ q)
                p, lse_bjh = _softmax_stats(s[None, :])
                p = p[0]
                u[b, j, h] = p @ v[: last + 1]
                o[b, j, h] = p @ c[: last + 1]
                lse[b, j, h] = lse_bjh[0]
    return u, o, lse


def absorb_q_reference(q_nope, q_rope, w_uk):
    """q_cat[b,j,h] = [ (W^UK_h)^T q^C_{b,j,h} ; q^R_{b,j,h} ].

    The absorbed content query of "DeepSeek-V3 MLA: Multi-Head Latent
    Attention Guide", Matrix Absorption Trick section 2 (Folding W^UK into
    Query Projection), written out as a per-head matrix-vector product.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    B, Lq, H, _ = q_nope.shape
    d_c = w_uk.shape[2]
    out = np.zeros((B, Lq, H, d_c + q_rope.shape[3]))
    for h in range(H):
        out[:, :, h, :d_c] = q_nope[:, :, h, :] @ w_uk[h]  # sum_n q[n] W[h,n,c]
        out[:, :, h, d_c:] = q_rope[:, :, h, :]
    return out


def absorb_out_reference(o, w_uv):
    """u[b,j,h] = W^UV_h o[b,j,h]: the same guide, section 3 (Absorbing W^UV)."""
    o = np.asarray(o, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    H = o.shape[2]
    u = np.zeros(o.shape[:3] + (w_uv.shape[1],))
    for h in range(H):
        u[:, :, h, :] = o[:, :, h, :] @ w_uv[h].T
    return u


def latent_attention_partial_reference(q_cat, rows, scale, d_c, visible):
    """Softmax attention of absorbed queries over a subset of latent rows.

    q_cat [R, D] absorbed queries, rows [T, D] latent rows, visible [R, T]
    boolean mask.  Returns (o [R, d_c], lse [R]) with o normalised over the
    visible rows only; a query that sees nothing gets o = 0, lse = -inf.
    Scores are q_cat . row (the guide's score on latents: content part
    q~ . c plus RoPE part q^R . k^R) times ``scale``.
    """
    q_cat = np.asarray(q_cat, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    R = q_cat.shape[0]
    o = np.zeros((R, d_c))
    lse = np.full(R, -np.inf)
    for r in range(R):
        idx = np.nonzero(visible[r])[0]
        if idx.size == 0:
            continue
        s = scale * (rows[idx] @ q_cat[r])
        p, l = _softmax_stats(s[None, :])
        o[r] = p[0] @ rows[idx, :d_c]
        lse[r] = l[0]
    return o, lse


def lse_merge_reference(o_parts, lse_parts):
    """Merge normalised partial outputs over disjoint key sets.

    o_parts [..., S, d], lse_parts [..., S].  Returns (o [..., d], lse [...])
    with lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
    Parts with lse_s = -inf hold no keys and are skipped (their o_s is never
    read).  If every part is empty the result is o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    lead = lse_parts.shape[:-1]
    S = lse_parts.shape[-1]
    d = o_parts.shape[-1]
    o = np.zeros(lead + (d,))
    lse = np.full(lead, -np.inf)
    for idx in np.ndindex(*lead):
        live = [s for s in range(S) if np.isfinite(lse_parts[idx + (s,)])]
        if not live:
            continue
        m = max(lse_parts[idx + (s,)] for s in live)
        z = sum(math.exp(lse_parts[idx + (s,)] - m) for s in live)
        total = m + math.log(z)
        lse[idx] = total
        o[idx] = sum(math.exp(lse_parts[idx + (s,)] - total) * o_parts[idx + (s,)] for s in live)
    return o, lse


def cache_elements_per_token(kind: str, *, n_h=128, d_h=128, d_c=512, d_rope=64, n_kv=8) -> int:
    """Cached elements per token per layer.

    MLA keeps c^KV and k^R: d_c + d_rope.  MHA keeps K and V for every head:
    2 n_h d_h.  GQA keeps K and V for n_kv heads: 2 n_kv d_h.
    """
    if kind == "mla":
        return d_c + d_rope
    if kind == "mha":
        return 2 * n_h * d_h
    if kind == "gqa":
        return 2 * n_kv * d_h
    raise ValueError(kind)


def cache_bytes(kind: str, tokens: int, bytes_per_element: int, layers: int = 1, **dims) -> int:
    """Bytes of cache for ``tokens`` tokens over ``layers`` layers."""
    return cache_elements_per_token(kind, **dims) * tokens * bytes_per_element * layers


def rope_reference(x, pos, base=10000.0):
    """Rotary position embedding of the last axis of x at integer positions pos.

    "Deconstructing DeepSeek V4 Pro ..." -- the apply_rope helper of its MLA
    module: element pairs (x[2p], x[2p+1]) are rotated by the angle
    theta_p = pos / base^(2p / d) with d the width of the last axis:
        out[2p]   = x[2p] cos(theta_p) - x[2p+1] sin(theta_p)
        out[2p+1] = x[2p+1] cos(theta_p) + x[2p] sin(theta_p)
    x has shape [..., d] and pos broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even width")
    pos = np.asarray(pos, dtype=np.float64)[..., None]  # [..., 1]
    p = np.arange(d // 2, dtype=np.float64)
    theta = pos / np.power(float(base), 2.0 * p / d)  # [..., d/2]
    c, s_ = np.cos(theta), np.sin(theta)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s_
    out[..., 1::2] = x1 * c + x0 * s_
    return out


def cache_rows_reference(h, w_dkv, w_kr, pos, base=10000.0):
    """Cache rows [c^KV | k^R] of hidden states h at positions pos.

    c^KV_t = W^DKV h_t and k^R_t = RoPE_t(W^KR h_t): "DeepSeek-V3 MLA:
    Multi-Head Latent Attention Guide", Core Architecture section 1 (joint KV
    compression) and section 3 (decoupled RoPE key); the weights are Linear
    weights, W^DKV in R^{d_c x d} and W^KR in R^{d_rope x d} (the V4 Pro
    module's W_dkv and W_kr).  h has shape [..., d]; returns [..., d_c + d_rope].
    """
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(w_dkv, dtype=np.float64).T
    k = rope_reference(h @ np.asarray(w_kr, dtype=np.float64).T, pos, base)
    return np.concatenate([c, k], axis=-1)


def cache_append_reference(cache, block_table, seq_lens, h, w_dkv, w_kr, base=10000.0):
    """The paged cache after writing the rows of the q_len new tokens.

    Sequence b holds seq_lens[b] tokens including its q_len new ones (the
    Guide's decode step appends the new latent before scoring); new token j
    sits at position t = seq_lens[b] - q_len + j, in physical block
    block_table[b, t // bs] at slot t % bs, and its row is
    cache_rows_reference(h[b, j], ..., pos=t).  Every other slot is left as
    it was.  Returns a float64 copy of the cache.
    """
    out = np.array(cache, dtype=np.float64, copy=True)
    h = np.asarray(h, dtype=np.float64)
    B, Lq, _ = h.shape
    bs = out.shape[1]
    for b in range(B):
        for j in range(Lq):
            t = int(seq_lens[b]) - Lq + j
            if t < 0:
                raise ValueError("a sequence is shorter than q_len")
            row = cache_rows_reference(h[b, j], w_dkv, w_kr, t, base)
            out[int(block_table[b, t // bs]), t % bs, :] = row
    return out



def prefill_reference(q_nope, q_rope, c_kv, k_rope, cu_seqlens, w_uk, w_uv, scale, causal=True, select=None):
    """Non-absorbed MLA attention over whole sequences (prefill, training forward).

    "Deconstructing DeepSeek V4 Pro ..." -- the forward pass of its MLA module
    -- and "DeepSeek-V3 MLA: Multi-Head Latent Attention Guide" -- forward_train:
    every token's latent is up-projected per head,
        K_{t,h} = [W^UK_h c_t ; k^R_t],   V_{t,h} = W^UV_h c_t,
    and u_{j,h} = softmax_t(scale q_{j,h} . K_{t,h}) V_{t,h} over the tokens of
    j's own sequence, q_{j,h} = [q^C_{j,h} ; q^R_{j,h}].  Both pages' code
    scores every key of the sequence; causal=True (the default) takes the
    decoder's reading that token j sees the keys t <= j, as the decode step
    does, and causal=False is the code as printed.

    Tokens of all sequences are packed: sequence b is rows cu_seqlens[b] ..
    cu_seqlens[b+1] - 1 of q_nope [T,H,d_n], q_rope [T,H,d_r], c_kv [T,d_c]
    and k_rope [T,d_r] (already rotated).  w_uk [H,d_n,d_c], w_uv [H,d_v,d_c].
    Returns (u [T,H,d_v], lse [T,H]) in float64, lse the natural-log
    log-sum-exp of the scaled, masked scores.  ``select`` (iterable of
    (token, head)) restricts the work to those pairs; the rest is NaN.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, _ = q_nope.shape
    d_v = w_uv.shape[1]
    u = np.full((T, H, d_v), np.nan)
    lse = np.full((T, H), np.nan)
    wanted = None
    if select is not None:
        wanted = {}
        for t, h in select:
            wanted.setdefault(int(h), set()).add(int(t))
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 <= s0:
            continue
        c = c_kv[s0:s1]
        for h in range(H):
            rows = range(s0, s1) if wanted is None else sorted(t for t in wanted.get(h, ()) if s0 <= t < s1)
            if not rows:
                continue
            keys = np.concatenate([c @ w_uk[h].T, k_rope[s0:s1]], axis=1)  # K_{t,h}, [L, d_n + d_r]
            vals = c @ w_uv[h].T  # V_{t,h}, [L, d_v]
            for t in rows:
                j = t - s0  # position of the query inside its sequence
                q = np.concatenate([q_nope[t, h], q_rope[t, h]])
                n_vis = j + 1 if causal else s1 - s0  # keys 0 .. n_vis - 1
                sc = scale * (keys[:n_vis] @ q)
                p, lse_t = _softmax_stats(sc[None, :])
                u[t, h] = p[0] @ vals[:n_vis]
                lse[t, h] = lse_t[0]
    return u, lse


# --------------------------------------------------------------------------
# FP8 (E4M3) latent cache.  "Deconstructing DeepSeek V4 Pro", Practical
# Deployment (quantization strategies): the compressed latent tolerates FP8
# (E4M3/E5M2), which brings a token's cached row below a kilobyte; "DeepSeek-V3
# MLA: Multi-Head Latent Attention Guide", Core Architecture: the 576 cached
# values per token are kept in fp8 or bf16.  The pages name the format only;
# the readings taken here are: the whole row [c^KV | k^R] is E4M3 (576 bytes),
# one float scale per cache (a stored code q stands for scale * value(q)), and
# encoding rounds to the nearest code with ties to the even code, saturating
# at +-448 so that a finite latent never becomes NaN.

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Values (float64) of E4M3 codes, from the format's definition (OCP 8-bit
    floating point, E4M3): bit 7 is the sign, bits 6..3 the exponent with bias
    7, bits 2..0 the mantissa.  Exponent field 0 holds the subnormals
    m/8 * 2^-6; otherwise the value is (1 + m/8) * 2^(e-7).  The code with all
    six exponent and mantissa bits set is NaN; there are no infinities, so the
    largest magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, val)


def e4m3_encode(x):
    """E4M3 code (uint8) nearest to x, ties to the even code, saturating:
    magnitudes of 448 and above give the code of +-448.  -0.0 keeps its sign
    bit; NaN gives the NaN code 0x7F.  Written as a nearest-neighbour search
    over the 127 non-negative finite values."""
    x = np.asarray(x, dtype=np.float64)
    table = e4m3_decode(np.arange(0x7F))  # codes 0x00..0x7E: 0 .. 448, increasing
    a = np.minimum(np.abs(np.where(np.isnan(x), 0.0, x)), E4M3_MAX)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, len(table) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = pick | np.where(np.signbit(x), 0x80, 0)
    return np.where(np.isnan(x), 0x7F, code).astype(np.uint8)


def fp8_cache_values(codes, kv_scale):
    """The latent cache an E4M3 code cache stands for: kv_scale * value(code),
    float64, same shape.  Decoding over it is mla_decode_reference unchanged."""
    return float(kv_scale) * e4m3_decode(codes)


def cache_append_fp8_reference(codes, block_table, seq_lens, h, w_dkv, w_kr, kv_scale, base=10000.0,
                               row_dtype=np.float64):
    """The E4M3 code cache after writing the rows of the q_len new tokens: the
    row of new token j of sequence b is cache_rows_reference(...) at position
    seq_lens[b] - q_len + j, divided by kv_scale and encoded with
    e4m3_encode.  ``row_dtype`` is the precision in which the row value meets
    the rounding decision (float64 by default; float32 to take the decision in
    the kernel's precision).  Every other code is left as it was."""
    out = np.array(codes, dtype=np.uint8, copy=True)
    h = np.asarray(h, dtype=np.float64)
    B, Lq, _ = h.shape
    bs = out.shape[1]
    for b in range(B):
        for j in range(Lq):
            pos = int(seq_lens[b]) - Lq + j  # position of new token j
            if pos < 0:
                raise ValueError("a sequence is shorter than q_len")
            row = cache_rows_reference(h[b, j], w_dkv, w_kr, pos, base).astype(row_dtype)
            out[int(block_table[b, pos // bs]), pos % bs, :] = e4m3_encode(row / row_dtype(kv_scale))
    return out


# --------------------------------------------------------------------------
# Offline weight folds.  "DeepSeek-V3 MLA: Multi-Head Latent Attention
# Guide", Matrix Absorption Trick section 3: the final output W^O [u_1; ...;
# u_nh] equals W~^O [o_1; ...; o_nh], W~^O being W^O multiplied offline by the
# heads' up-projections W^UV_i; "Deconstructing DeepSeek V4 Pro", Practical
# Deployment: the query projection and W^UK^T can likewise be multiplied into
# one fused query weight before serving.  Readings: the query projection is
# given per head as W_in[h] in R^{d_nope x d_in} (the content part of the
# query up-projection W^UQ of the query latent c^Q, d_in = d_c' = 1536 in the
# Guide's module and the V2 note's table, or a projection of the hidden state
# itself), so the fused weight is W~_Q[h] = W^UK_h^T W_in[h] in
# R^{d_c x d_in}; W^O in R^{d_out x (n_h d_v)} acts on the heads' outputs
# concatenated in head order, so W~^O = W^O blockdiag(W^UV_1, ..., W^UV_nh) in
# R^{d_out x (n_h d_c)}.


def fold_query_weight_reference(w_in, w_uk):
    """W~_Q[h] = (W^UK_h)^T W_in[h]: w_in [H, d_nope, d_in], w_uk [H, d_nope, d_c] -> [H, d_c, d_in]."""
    w_in = np.asarray(w_in, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    return np.stack([w_uk[h].T @ w_in[h] for h in range(w_in.shape[0])])


def fused_query_reference(x, q_rope, w_fused):
    """q_cat[b,j,h] = [W~_Q[h] x[b,j] ; q^R_{b,j,h}]: x [B, Lq, d_in], q_rope [B, Lq, H, d_rope],
    w_fused [H, d_c, d_in] -> [B, Lq, H, d_c + d_rope] (what mla_absorb_q gives from q^C = W_in x)."""
    x = np.asarray(x, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    w_fused = np.asarray(w_fused, dtype=np.float64)
    B, Lq, _ = x.shape
    H, d_c, _ = w_fused.shape
    out = np.zeros((B, Lq, H, d_c + q_rope.shape[3]))
    out[:, :, :, d_c:] = q_rope  # the RoPE part passes through
    for h in range(H):
        out[:, :, h, :d_c] = x @ w_fused[h].T
    return out


def fold_output_weight_reference(w_o, w_uv, rows=None):
    """W~^O = W^O blockdiag(W^UV_h): w_o [d_out, H d_v], w_uv [H, d_v, d_c] -> [d_out, H d_c];
    column block h is W^O[:, h d_v:(h+1) d_v] W^UV_h.  ``rows`` restricts the result to those rows."""
    w_o = np.asarray(w_o, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    if rows is not None:
        w_o = w_o[np.asarray(rows)]
    H, d_v, d_c = w_uv.shape
    return np.concatenate([w_o[:, h * d_v:(h + 1) * d_v] @ w_uv[h] for h in range(H)], axis=1)


def fused_output_reference(o, w_fused):
    """y[b,j] = W~^O [o_{b,j,1}; ...; o_{b,j,H}]: o [B, Lq, H, d_c], w_fused [d_out, H d_c] -> [B, Lq, d_out]."""
    o = np.asarray(o, dtype=np.float64)
    w_fused = np.asarray(w_fused, dtype=np.float64)
    B, Lq, H, d_c = o.shape
    return o.reshape(B, Lq, H * d_c) @ w_fused.T
