"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes the oracle module as an argument so that the mutation
tests can run the same pins against deliberately broken copies of it.  A pin
raises AssertionError (or any exception) when the oracle is wrong.

Independent routes used here:
  * the absorbed algebra of "DeepSeek-V3 MLA: Multi-Head Latent Attention
    Guide" (Matrix Absorption Trick, sections 2 and 3): scores on latents and
    W^UV applied after the weighted sum -- a different computation that the
    page shows equal to the non-absorbed one;
  * torch.nn.functional.scaled_dot_product_attention in float64 on the CPU,
    fed with keys and values materialised here;
  * pure-Python scalar loops on tiny inputs;
  * closed forms (length-1 context, zero query, constant latent rows);
  * invariances (physical block permutation, causal reduction for q_len = 2);
  * the log-sum-exp merge identity over a split of the keys;
  * for the cache append: RoPE as multiplication by a unit complex number
    (numpy complex arithmetic, angle from logarithms), RoPE's defining
    relative-position property, 2 x 2 rotation matrices in scalar loops, and
    the paging invariant that only the new tokens' slots change;
  * for the prefill: the absorbed algebra per query token, torch's float64
    scaled_dot_product_attention with is_causal, scalar loops, the decode
    oracle on every prefix (a causal prefill row is a decode step), the key
    permutation invariance of the unmasked form, and the one-key closed form;
  * for the FP8 (E4M3) cache: torch's float8_e4m3fn conversions (a library
    implementation of the same format), values the format's definition fixes
    (1, 2, 1.5, 448, the smallest normal and subnormal, -0), a pure-Python
    nearest-code search over all finite codes, and the float cache append
    rounded through torch;
  * for the weight folds: the unfolded route of the same pages (W_in x, then
    the absorbed query; W^UV after the latent sum, then W^O) through the
    pinned absorb_q / absorb_out references and plain matrix products, and
    scalar loops on tiny sizes.
"""
from __future__ import annotations

import math

import numpy as np
import torch

RTOL = 1e-11
ATOL = 1e-12


class Tiny:
    """A tiny paged problem built from contiguous per-sequence rows.

    The contiguous rows are kept, so routes below never go through the
    oracle's own gather.
    """

    def __init__(self, seed=0, B=2, Lq=2, H=3, d_c=8, d_r=4, d_n=5, d_v=5, bs=4, lens=(5, 11),
                 zero_query=False, const_rows=False):
        rng = np.random.default_rng(seed)
        self.B, self.Lq, self.H, self.d_c, self.d_r, self.d_n, self.d_v, self.bs = B, Lq, H, d_c, d_r, d_n, d_v, bs
        self.lens = np.asarray(lens, dtype=np.int64)
        D = d_c + d_r
        self.rows = []
        for L in self.lens:
            r = rng.standard_normal((int(L), D))
            if const_rows:
                r[:] = r[0]
            self.rows.append(r)
        nblk = [int(math.ceil(L / bs)) for L in self.lens]
        nb = sum(nblk)
        perm = rng.permutation(nb)
        self.table = np.full((B, max(nblk)), -1, dtype=np.int64)
        self.cache = np.full((nb, bs, D), np.nan)
        k = 0
        for b in range(B):
            for i in range(nblk[b]):
                pb = perm[k]
                k += 1
                self.table[b, i] = pb
                seg = self.rows[b][i * bs:(i + 1) * bs]
                self.cache[pb, : seg.shape[0]] = seg
        self.q_nope = rng.standard_normal((B, Lq, H, d_n))
        self.q_rope = rng.standard_normal((B, Lq, H, d_r))
        if zero_query:
            self.q_nope[:] = 0.0
            self.q_rope[:] = 0.0
        self.w_uk = rng.standard_normal((H, d_n, d_c)) / math.sqrt(d_c)
        self.w_uv = rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c)
        self.scale = 1.0 / math.sqrt(d_n + d_r)

    def run(self, orc, **kw):
        return orc.mla_decode_reference(self.q_nope, self.q_rope, self.cache, self.table, self.lens,
                                        self.w_uk, self.w_uv, self.scale, self.d_c, **kw)


def _close(a, b, rtol=RTOL, atol=ATOL):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


def pin_absorbed_route(orc, seed=0):
    """u, o, lse equal the absorbed-algebra computation on the contiguous rows."""
    p = Tiny(seed)
    u, o, lse = p.run(orc)
    for b in range(p.B):
        L = int(p.lens[b])
        c = p.rows[b][:, : p.d_c]
        kr = p.rows[b][:, p.d_c:]
        for h in range(p.H):
            for j in range(p.Lq):
                n = L - p.Lq + j + 1
                q_abs = np.einsum("n,nc->c", p.q_nope[b, j, h], p.w_uk[h])
                s = (c[:n] @ q_abs + kr[:n] @ p.q_rope[b, j, h]) * p.scale
                w = np.exp(s - s.max())
                z = w.sum()
                o_ref = (w / z) @ c[:n]
                _close(o[b, j, h], o_ref)
                _close(u[b, j, h], p.w_uv[h] @ o_ref)
                _close(lse[b, j, h], s.max() + math.log(z))


def pin_library_sdpa(orc, seed=1):
    """u equals torch's float64 scaled_dot_product_attention on materialised K and V."""
    p = Tiny(seed, H=4, lens=(9, 6))
    u, _, _ = p.run(orc)
    for b in range(p.B):
        L = int(p.lens[b])
        c = torch.from_numpy(p.rows[b][:, : p.d_c])
        kr = torch.from_numpy(p.rows[b][:, p.d_c:])
        wk = torch.from_numpy(p.w_uk)
        wv = torch.from_numpy(p.w_uv)
        K = torch.cat([torch.einsum("tc,hnc->htn", c, wk), kr.unsqueeze(0).expand(p.H, L, p.d_r)], dim=2)
        V = torch.einsum("tc,hvc->htv", c, wv)
        Q = torch.cat([torch.from_numpy(p.q_nope[b]), torch.from_numpy(p.q_rope[b])], dim=2).transpose(0, 1)
        mask = torch.zeros(p.Lq, L, dtype=torch.bool)
        for j in range(p.Lq):
            mask[j, : L - p.Lq + j + 1] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q.contiguous(), K.contiguous(), V.contiguous(), attn_mask=mask, scale=p.scale)
        _close(u[b], ref.transpose(0, 1).numpy())


def pin_bruteforce(orc, seed=2):
    """u equals scalar pure-Python loops on a tiny problem."""
    p = Tiny(seed, B=2, Lq=2, H=2, d_c=3, d_r=2, d_n=2, d_v=2, bs=2, lens=(3, 4))
    u, _, _ = p.run(orc)
    for b in range(p.B):
        L = int(p.lens[b])
        for h in range(p.H):
            for j in range(p.Lq):
                n = L - p.Lq + j + 1
                scores = []
                for t in range(n):
                    row = [float(x) for x in p.rows[b][t]]
                    acc = 0.0
                    for a in range(p.d_n):
                        k_a = sum(float(p.w_uk[h, a, cc]) * row[cc] for cc in range(p.d_c))
                        acc += float(p.q_nope[b, j, h, a]) * k_a
                    for r in range(p.d_r):
                        acc += float(p.q_rope[b, j, h, r]) * row[p.d_c + r]
                    scores.append(acc * p.scale)
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                z = sum(ex)
                for vv in range(p.d_v):
                    val = 0.0
                    for t in range(n):
                        v_t = sum(float(p.w_uv[h, vv, cc]) * float(p.rows[b][t][cc]) for cc in range(p.d_c))
                        val += ex[t] / z * v_t
                    assert abs(u[b, j, h, vv] - val) <= 1e-12 + 1e-11 * abs(val), (b, j, h, vv)


def pin_length_one(orc, seed=3):
    """A one-token context returns that token's value exactly (p = 1)."""
    p = Tiny(seed, Lq=1, lens=(1, 1))
    u, o, _ = p.run(orc)
    for b in range(p.B):
        c0 = p.rows[b][0, : p.d_c]
        for h in range(p.H):
            _close(o[b, 0, h], c0, rtol=0, atol=0)
            _close(u[b, 0, h], p.w_uv[h] @ c0)


def pin_zero_query(orc, seed=4):
    """A zero query gives uniform attention: u is the mean value over visible keys."""
    p = Tiny(seed, zero_query=True)
    u, _, lse = p.run(orc)
    for b in range(p.B):
        L = int(p.lens[b])
        for h in range(p.H):
            v = p.rows[b][:, : p.d_c] @ p.w_uv[h].T
            for j in range(p.Lq):
                n = L - p.Lq + j + 1
                _close(u[b, j, h], v[:n].mean(axis=0))
                _close(lse[b, j, h], math.log(n))


def pin_constant_rows(orc, seed=5):
    """When every latent row is the same vector, softmax weights sum to one so o is that vector."""
    p = Tiny(seed, const_rows=True)
    _, o, _ = p.run(orc)
    for b in range(p.B):
        _close(o[b], np.broadcast_to(p.rows[b][0, : p.d_c], o[b].shape))


def pin_block_permutation(orc, seed=6):
    """Re-placing the physical blocks (and the table with them) changes nothing, bit for bit."""
    p = Tiny(seed)
    u1, o1, l1 = p.run(orc)
    rng = np.random.default_rng(seed + 100)
    nb = p.cache.shape[0]
    perm = rng.permutation(nb)
    cache2 = np.empty_like(p.cache)
    cache2[perm] = p.cache
    table2 = np.where(p.table >= 0, perm[np.maximum(p.table, 0)], -1)
    u2, o2, l2 = orc.mla_decode_reference(p.q_nope, p.q_rope, cache2, table2, p.lens, p.w_uk, p.w_uv,
                                          p.scale, p.d_c)
    assert np.array_equal(u1, u2) and np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_causal_reduction(orc, seed=7):
    """For q_len = 2, query 0 equals a q_len = 1 run over the first L - 1 tokens."""
    p = Tiny(seed, Lq=2)
    u2, o2, l2 = p.run(orc)
    u1, o1, l1 = orc.mla_decode_reference(p.q_nope[:, :1], p.q_rope[:, :1], p.cache, p.table, p.lens - 1,
                                          p.w_uk, p.w_uv, p.scale, p.d_c)
    _close(u2[:, 0], u1[:, 0])
    _close(o2[:, 0], o1[:, 0])
    _close(l2[:, 0], l1[:, 0])
    # and query 1 sees one more key than query 0, so the two must differ
    assert not np.allclose(u2[:, 0], u2[:, 1])


def pin_merge(orc, seed=8):
    """Splitting the keys into parts and merging (o_s, lse_s) gives the whole; empty parts count zero."""
    p = Tiny(seed, Lq=2, lens=(7, 10))
    _, o, lse = p.run(orc)
    q_cat = np.concatenate([np.einsum("bjhn,hnc->bjhc", p.q_nope, p.w_uk), p.q_rope], axis=3)
    for b in range(p.B):
        L = int(p.lens[b])
        bounds = [0, 2, 2, L // 2 + 1, L, L]  # includes empty parts
        qs = q_cat[b].reshape(p.Lq * p.H, -1)
        o_parts, l_parts = [], []
        for s0, s1 in zip(bounds[:-1], bounds[1:]):
            vis = np.zeros((p.Lq * p.H, s1 - s0), dtype=bool)
            for j in range(p.Lq):
                last = L - p.Lq + j
                for h in range(p.H):
                    vis[j * p.H + h] = np.arange(s0, s1) <= last
            op, lp = orc.latent_attention_partial_reference(qs, p.rows[b][s0:s1], p.scale, p.d_c, vis)
            o_parts.append(op)
            l_parts.append(lp)
        om, lm = orc.lse_merge_reference(np.stack(o_parts, axis=1), np.stack(l_parts, axis=1))
        _close(om.reshape(p.Lq, p.H, p.d_c), o[b])
        _close(lm.reshape(p.Lq, p.H), lse[b])
    # all-empty merge is (0, -inf)
    om, lm = orc.lse_merge_reference(np.full((1, 2, 3), np.nan), np.full((1, 2), -np.inf))
    assert np.all(om == 0) and np.all(np.isneginf(lm))


def pin_absorb_q(orc, seed=9):
    """q_cat . [c; k^R] equals the materialised score k^C . q^C + k^R . q^R (page's associativity)."""
    p = Tiny(seed, d_n=7)
    q_cat = orc.absorb_q_reference(p.q_nope, p.q_rope, p.w_uk)
    assert q_cat.shape == (p.B, p.Lq, p.H, p.d_c + p.d_r)
    for b in range(p.B):
        rows = p.rows[b]
        for h in range(p.H):
            k_c = rows[:, : p.d_c] @ p.w_uk[h].T
            for j in range(p.Lq):
                direct = k_c @ p.q_nope[b, j, h] + rows[:, p.d_c:] @ p.q_rope[b, j, h]
                _close(rows @ q_cat[b, j, h], direct)


def pin_absorb_out(orc, seed=10):
    """W^UV applied to o equals the weighted sum of materialised values (u from the non-absorbed route)."""
    p = Tiny(seed, d_v=6)
    u, o, _ = p.run(orc)
    _close(orc.absorb_out_reference(o, p.w_uv), u)


def pin_select(orc, seed=11):
    """Restricting to chosen (b, h) pairs reproduces exactly those entries of the full run."""
    p = Tiny(seed)
    u, o, lse = p.run(orc)
    sel = [(1, 2), (0, 0)]
    us, os_, ls = p.run(orc, select=sel)
    for b, h in sel:
        assert np.array_equal(us[b, :, h], u[b, :, h]) and np.array_equal(ls[b, :, h], lse[b, :, h])
    assert np.isnan(us[0, :, 1]).all()


def pin_rope_complex(orc, seed=12):
    """RoPE of pair p is multiplication of x[2p] + i x[2p+1] by exp(i pos base^(-2p/d))."""
    rng = np.random.default_rng(seed)
    d, base = 16, 10000.0
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 1000, 131071])
    z = x[:, 0::2] + 1j * x[:, 1::2]
    p = np.arange(d // 2)
    ang = pos[:, None] * np.exp(-(2.0 * p / d) * math.log(base))
    zr = z * np.exp(1j * ang)
    want = np.empty_like(x)
    want[:, 0::2], want[:, 1::2] = zr.real, zr.imag
    _close(orc.rope_reference(x, pos, base), want, rtol=1e-9, atol=1e-9)


def pin_rope_relative(orc, seed=13):
    """<RoPE_m(q), RoPE_n(k)> = <RoPE_{m-n}(q), k>; norms of pairs are kept; position 0 is the identity."""
    rng = np.random.default_rng(seed)
    d = 8
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in [(5, 2), (17, 17), (3, 40)]:
        lhs = orc.rope_reference(q, m) @ orc.rope_reference(k, n)
        rhs = orc.rope_reference(q, m - n) @ k
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(rhs))
    r = orc.rope_reference(q, 123)
    _close(r[0::2] ** 2 + r[1::2] ** 2, q[0::2] ** 2 + q[1::2] ** 2)
    assert np.array_equal(orc.rope_reference(q, 0), q)


def pin_cache_rows_bruteforce(orc, seed=14):
    """Cache rows from scalar loops: c_n = sum_k W^DKV[n, k] h[k], k^R from explicit 2 x 2 rotations."""
    rng = np.random.default_rng(seed)
    d, d_c, d_r = 6, 5, 4
    h = rng.standard_normal(d)
    w_dkv, w_kr = rng.standard_normal((d_c, d)), rng.standard_normal((d_r, d))
    pos = 9
    want = []
    for n in range(d_c):
        want.append(sum(float(w_dkv[n, k]) * float(h[k]) for k in range(d)))
    kr = [sum(float(w_kr[n, k]) * float(h[k]) for k in range(d)) for n in range(d_r)]
    for pp in range(d_r // 2):
        th = pos / (10000.0 ** (2.0 * pp / d_r))
        rot = [[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]]
        a, b = kr[2 * pp], kr[2 * pp + 1]
        want += [rot[0][0] * a + rot[0][1] * b, rot[1][0] * a + rot[1][1] * b]
    _close(orc.cache_rows_reference(h, w_dkv, w_kr, pos), np.array(want))


def pin_cache_append(orc, seed=15):
    """Appending writes exactly the q_len new tokens' slots (through the table), nothing else; the
    decode over the appended cache equals the decode over contiguous rows with the new rows put last."""
    p = Tiny(seed, B=2, Lq=2, lens=(5, 11))
    rng = np.random.default_rng(seed + 100)
    d = 7
    h = rng.standard_normal((p.B, p.Lq, d))
    w_dkv, w_kr = rng.standard_normal((p.d_c, d)), rng.standard_normal((p.d_r, d))
    new = orc.cache_append_reference(p.cache, p.table, p.lens, h, w_dkv, w_kr)
    touched = np.zeros(p.cache.shape[:2], dtype=bool)
    for b in range(p.B):
        for j in range(p.Lq):
            t = int(p.lens[b]) - p.Lq + j
            touched[p.table[b, t // p.bs], t % p.bs] = True
            p.rows[b][t] = orc.cache_rows_reference(h[b, j], w_dkv, w_kr, t)
    same = ~touched
    assert np.array_equal(np.isnan(new[same]), np.isnan(p.cache[same]))
    assert np.array_equal(np.nan_to_num(new[same]), np.nan_to_num(p.cache[same]))
    p.cache = new
    u, o, lse = p.run(orc)
    # the absorbed algebra on the contiguous rows (which now hold the new rows)
    for b in range(p.B):
        L = int(p.lens[b])
        for j in range(p.Lq):
            rows = p.rows[b][: L - p.Lq + j + 1]
            for hh in range(p.H):
                qc = p.w_uk[hh].T @ p.q_nope[b, j, hh]
                s = p.scale * (rows[:, : p.d_c] @ qc + rows[:, p.d_c:] @ p.q_rope[b, j, hh])
                e = np.exp(s - s.max())
                _close(o[b, j, hh], (e / e.sum()) @ rows[:, : p.d_c])


class TinyPrefill:
    """Packed sequences for the prefill oracle (contiguous rows, no paging)."""

    def __init__(self, seed=20, H=3, d_c=8, d_r=4, d_n=5, d_v=5, lens=(5, 1, 7)):
        rng = np.random.default_rng(seed)
        self.H, self.d_c, self.d_r, self.d_n, self.d_v = H, d_c, d_r, d_n, d_v
        self.lens = np.asarray(lens, dtype=np.int64)
        self.cu = np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int64)
        T = int(self.cu[-1])
        self.c = rng.standard_normal((T, d_c))
        self.kr = rng.standard_normal((T, d_r))
        self.q_nope = rng.standard_normal((T, H, d_n))
        self.q_rope = rng.standard_normal((T, H, d_r))
        self.w_uk = rng.standard_normal((H, d_n, d_c)) / math.sqrt(d_c)
        self.w_uv = rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c)
        self.scale = 1.0 / math.sqrt(d_n + d_r)

    def run(self, orc, causal=True, **kw):
        return orc.prefill_reference(self.q_nope, self.q_rope, self.c, self.kr, self.cu, self.w_uk, self.w_uv,
                                     self.scale, causal=causal, **kw)


def pin_prefill_absorbed(orc, seed=20):
    """Prefill u and lse equal the absorbed algebra token by token (q~ = W_UK^T q^C, scores on the
    latents, W_UV applied after the latent-weighted sum), causal and unmasked."""
    p = TinyPrefill(seed)
    for causal in (True, False):
        u, lse = p.run(orc, causal=causal)
        for b in range(len(p.lens)):
            s0, s1 = int(p.cu[b]), int(p.cu[b + 1])
            for t in range(s0, s1):
                vis = slice(s0, t + 1) if causal else slice(s0, s1)
                for h in range(p.H):
                    q_abs = np.einsum("n,nc->c", p.q_nope[t, h], p.w_uk[h])
                    sc = (p.c[vis] @ q_abs + p.kr[vis] @ p.q_rope[t, h]) * p.scale
                    w = np.exp(sc - sc.max())
                    z = w.sum()
                    _close(u[t, h], p.w_uv[h] @ ((w / z) @ p.c[vis]))
                    _close(lse[t, h], sc.max() + math.log(z))


def pin_prefill_sdpa(orc, seed=21):
    """Prefill u equals torch's float64 scaled_dot_product_attention (is_causal for the causal form)."""
    p = TinyPrefill(seed, H=4, lens=(9, 3, 6))
    for causal in (True, False):
        u, _ = p.run(orc, causal=causal)
        for b in range(len(p.lens)):
            s0, s1 = int(p.cu[b]), int(p.cu[b + 1])
            L = s1 - s0
            c = torch.from_numpy(p.c[s0:s1])
            kr = torch.from_numpy(p.kr[s0:s1])
            K = torch.cat([torch.einsum("tc,hnc->htn", c, torch.from_numpy(p.w_uk)),
                           kr.unsqueeze(0).expand(p.H, L, p.d_r)], dim=2)
            V = torch.einsum("tc,hvc->htv", c, torch.from_numpy(p.w_uv))
            Q = torch.cat([torch.from_numpy(p.q_nope[s0:s1]), torch.from_numpy(p.q_rope[s0:s1])], dim=2).transpose(0, 1)
            ref = torch.nn.functional.scaled_dot_product_attention(Q.contiguous(), K.contiguous(), V.contiguous(),
                                                                   is_causal=causal, scale=p.scale)
            _close(u[s0:s1], ref.transpose(0, 1).numpy())


def pin_prefill_bruteforce(orc, seed=22):
    """Prefill u equals scalar pure-Python loops on a tiny problem."""
    p = TinyPrefill(seed, H=2, d_c=3, d_r=2, d_n=2, d_v=2, lens=(3, 2))
    u, _ = p.run(orc)
    for b in range(len(p.lens)):
        s0, s1 = int(p.cu[b]), int(p.cu[b + 1])
        for t in range(s0, s1):
            for h in range(p.H):
                scores = []
                for k in range(s0, t + 1):
                    acc = 0.0
                    for n in range(p.d_n):
                        kc = sum(p.w_uk[h, n, i] * p.c[k, i] for i in range(p.d_c))
                        acc += p.q_nope[t, h, n] * kc
                    for r in range(p.d_r):
                        acc += p.q_rope[t, h, r] * p.kr[k, r]
                    scores.append(acc * p.scale)
                mx = max(scores)
                ws = [math.exp(x - mx) for x in scores]
                z = sum(ws)
                for v in range(p.d_v):
                    val = 0.0
                    for k, w in zip(range(s0, t + 1), ws):
                        val += w / z * sum(p.w_uv[h, v, i] * p.c[k, i] for i in range(p.d_c))
                    assert abs(u[t, h, v] - val) <= 1e-11 * max(1.0, abs(val)), (t, h, v)


def pin_prefill_matches_decode(orc, seed=23):
    """A causal prefill row is a decode step: row t equals the decode oracle over the prefix
    0..t of its sequence, with that token as the single new query (blocks in order)."""
    p = TinyPrefill(seed, lens=(6, 4))
    u, lse = p.run(orc)
    bs = 2
    for b in range(len(p.lens)):
        s0, s1 = int(p.cu[b]), int(p.cu[b + 1])
        for t in range(s0, s1):
            n = t - s0 + 1
            rows = np.concatenate([p.c[s0:t + 1], p.kr[s0:t + 1]], axis=1)
            nb = (n + bs - 1) // bs
            cache = np.full((nb, bs, rows.shape[1]), np.nan)
            for i in range(n):
                cache[i // bs, i % bs] = rows[i]
            table = np.arange(nb).reshape(1, nb)
            ud, _, ld = orc.mla_decode_reference(p.q_nope[t][None, None], p.q_rope[t][None, None], cache, table,
                                                 np.array([n]), p.w_uk, p.w_uv, p.scale, p.d_c)
            _close(u[t], ud[0, 0])
            _close(lse[t], ld[0, 0])


def pin_prefill_key_permutation(orc, seed=24):
    """Without the mask, permuting a sequence's keys and values together (its c and k^R rows)
    changes nothing; with the mask, the first token's output depends on the first key only."""
    p = TinyPrefill(seed)
    u, lse = p.run(orc, causal=False)
    rng = np.random.default_rng(seed)
    q = TinyPrefill(seed)
    for b in range(len(p.lens)):
        s0, s1 = int(p.cu[b]), int(p.cu[b + 1])
        perm = s0 + rng.permutation(s1 - s0)
        q.c[s0:s1] = p.c[perm]
        q.kr[s0:s1] = p.kr[perm]
    u2, lse2 = q.run(orc, causal=False)
    _close(u2, u, rtol=1e-10, atol=1e-11)
    _close(lse2, lse, rtol=1e-10, atol=1e-11)
    uc, lc = p.run(orc, causal=True)
    for b in range(len(p.lens)):
        t = int(p.cu[b])
        for h in range(p.H):
            _close(uc[t, h], p.w_uv[h] @ p.c[t])  # one visible key: weight 1
            k = np.concatenate([p.w_uk[h] @ p.c[t], p.kr[t]])
            _close(lc[t, h], p.scale * float(np.concatenate([p.q_nope[t, h], p.q_rope[t, h]]) @ k))


def pin_prefill_select(orc, seed=25):
    """Restricting the prefill to chosen (token, head) pairs reproduces those entries."""
    p = TinyPrefill(seed)
    u, lse = p.run(orc)
    sel = [(0, 1), (5, 0), (11, 2), (7, 1)]
    us, ls = p.run(orc, select=sel)
    for t, h in sel:
        _close(us[t, h], u[t, h])
        _close(ls[t, h], lse[t, h])
    assert np.isnan(us[1, 0]).all()


# ------------------------------------------------------------------ FP8 (E4M3) cache

def pin_e4m3_decode_library(orc, seed=30):
    """Every one of the 256 codes decodes to what torch's float8_e4m3fn dtype gives."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert int(np.isnan(got).sum()) == 2  # 0x7F and 0xFF only


def pin_e4m3_known_values(orc, seed=31):
    """Values the format's definition fixes (sign 1 bit, exponent 4 bits with bias 7, mantissa 3 bits)."""
    table = {0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x07: 7.0 * 2.0 ** -9, 0x00: 0.0, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5, 0x77: 240.0}
    for code, val in table.items():
        assert orc.e4m3_decode(np.array([code]))[0] == val, hex(code)
    z = orc.e4m3_decode(np.array([0x80]))[0]
    assert z == 0.0 and np.signbit(z)
    assert orc.E4M3_MAX == 448.0


def _e4m3_nearest_bruteforce(x, values):
    """Nearest finite code by scanning every code, ties to the even code, saturating, -0 and NaN kept."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = min(abs(x), 448.0)
    best, best_d = None, None
    for code in range(0x7F):
        d = abs(a - values[code])
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return best | sign


def pin_e4m3_encode_bruteforce(orc, seed=32):
    """Encoding equals a scalar nearest-code search, on random values, exact midpoints, tiny and huge values."""
    rng = np.random.default_rng(seed)
    values = [float(v) for v in torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn)
              .to(torch.float64).numpy()]
    xs = list(rng.standard_normal(300) * 40.0) + list(rng.standard_normal(100) * 0.01)
    for c in range(0x7E):  # midpoints of neighbouring codes (ties) and points just off them
        mid = 0.5 * (values[c] + values[c + 1])
        xs += [mid, -mid, math.nextafter(mid, 0.0), math.nextafter(mid, 1e9)]
    xs += [448.0, 449.0, 463.9, 464.0, 500.0, 1e9, -1e9, 0.0, -0.0, 1e-30, -1e-30, float("nan")]
    got = orc.e4m3_encode(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == _e4m3_nearest_bruteforce(x, values), (x, int(g))


def pin_e4m3_encode_library(orc, seed=33):
    """Inside the finite range the encoding equals torch's round-to-nearest-even cast to float8_e4m3fn."""
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.standard_normal(20000) * 60.0, rng.standard_normal(5000) * 1e-3])
    x = x[np.abs(x) < 440.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(x), ref)


def pin_fp8_cache_values(orc, seed=34):
    """The cache an FP8 code cache stands for is scale * the library-decoded value of each code."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(3, 4, 5)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scale = 0.0123
    ref = scale * torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _close(orc.fp8_cache_values(codes, scale), ref)


def pin_cache_append_fp8(orc, seed=35):
    """The FP8 append writes, into exactly the new tokens' slots, the float append's rows divided by the
    scale and rounded by torch's float8_e4m3fn cast (within the finite range)."""
    rng = np.random.default_rng(seed)
    B, Lq, d, d_c, d_r, bs, NB = 2, 2, 12, 6, 4, 4, 7
    h = rng.standard_normal((B, Lq, d))
    w_dkv = rng.standard_normal((d_c, d)) / math.sqrt(d)
    w_kr = rng.standard_normal((d_r, d)) / math.sqrt(d)
    table = np.array([[3, 0, 5], [6, 1, 2]])
    lens = np.array([6, 9])
    codes = rng.integers(0, 0x7E, size=(NB, bs, d_c + d_r)).astype(np.uint8)
    scale = 0.037
    got = orc.cache_append_fp8_reference(codes, table, lens, h, w_dkv, w_kr, scale)
    ref_float = orc.cache_append_reference(np.zeros((NB, bs, d_c + d_r)), table, lens, h, w_dkv, w_kr)
    written = np.zeros((NB, bs), dtype=bool)
    for b in range(B):
        for j in range(Lq):
            t = int(lens[b]) - Lq + j
            blk, slot = int(table[b, t // bs]), t % bs
            written[blk, slot] = True
            row = ref_float[blk, slot] / scale
            assert np.abs(row).max() < 440.0
            want = torch.from_numpy(row).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(got[blk, slot], want)
    assert np.array_equal(got[~written], codes[~written])


# ------------------------------------------------------------------ offline weight folds

class TinyFold:
    def __init__(self, seed, H=3, d_n=4, d_v=5, d_c=6, d_r=2, d_in=7, d_out=8, B=2, Lq=2):
        rng = np.random.default_rng(seed)
        self.w_in = rng.standard_normal((H, d_n, d_in))
        self.w_uk = rng.standard_normal((H, d_n, d_c))
        self.w_uv = rng.standard_normal((H, d_v, d_c))
        self.w_o = rng.standard_normal((d_out, H * d_v))
        self.x = rng.standard_normal((B, Lq, d_in))
        self.q_rope = rng.standard_normal((B, Lq, H, d_r))
        self.o = rng.standard_normal((B, Lq, H, d_c))


def pin_fused_query_equals_unfolded(orc, seed=40):
    """Fused query weight on x equals the unfolded route: q^C = W_in x per head, then absorb_q."""
    p = TinyFold(seed)
    q_nope = np.einsum("hnd,bjd->bjhn", p.w_in, p.x)
    ref = orc.absorb_q_reference(q_nope, p.q_rope, p.w_uk)
    got = orc.fused_query_reference(p.x, p.q_rope, orc.fold_query_weight_reference(p.w_in, p.w_uk))
    _close(got, ref)


def pin_fused_output_equals_unfolded(orc, seed=41):
    """Fused output weight on the latent sums equals W^O applied to the heads' u = W^UV o, concatenated."""
    p = TinyFold(seed)
    u = orc.absorb_out_reference(p.o, p.w_uv)  # [B, Lq, H, d_v]
    ref = u.reshape(u.shape[0], u.shape[1], -1) @ p.w_o.T
    got = orc.fused_output_reference(p.o, orc.fold_output_weight_reference(p.w_o, p.w_uv))
    _close(got, ref)


def pin_folds_bruteforce(orc, seed=42):
    """Both folds against scalar loops, and the row-restricted output fold against the whole."""
    p = TinyFold(seed)
    H, d_n, d_in = p.w_in.shape
    d_c = p.w_uk.shape[2]
    fq = orc.fold_query_weight_reference(p.w_in, p.w_uk)
    for h in range(H):
        for c in range(d_c):
            for i in range(d_in):
                _close(fq[h, c, i], sum(p.w_uk[h, n, c] * p.w_in[h, n, i] for n in range(d_n)))
    fo = orc.fold_output_weight_reference(p.w_o, p.w_uv)
    d_out = p.w_o.shape[0]
    d_v = p.w_uv.shape[1]
    for r in range(d_out):
        for h in range(H):
            for c in range(d_c):
                want = sum(p.w_o[r, h * d_v + v] * p.w_uv[h, v, c] for v in range(d_v))
                _close(fo[r, h * d_c + c], want)
    _close(orc.fold_output_weight_reference(p.w_o, p.w_uv, rows=[5, 1]), fo[[5, 1]])
    y = orc.fused_output_reference(p.o, fo)
    for b in range(p.o.shape[0]):
        for j in range(p.o.shape[1]):
            for r in range(d_out):
                _close(y[b, j, r], sum(fo[r, h * d_c + c] * p.o[b, j, h, c] for h in range(H) for c in range(d_c)))


ALL_PINS = [
    pin_absorbed_route,
    pin_library_sdpa,
    pin_bruteforce,
    pin_length_one,
    pin_zero_query,
    pin_constant_rows,
    pin_block_permutation,
    pin_causal_reduction,
    pin_merge,
    pin_absorb_q,
    pin_absorb_out,
    pin_select,
    pin_rope_complex,
    pin_rope_relative,
    pin_cache_rows_bruteforce,
    pin_cache_append,
    pin_prefill_absorbed,
    pin_prefill_sdpa,
    pin_prefill_bruteforce,
    pin_prefill_matches_decode,
    pin_prefill_key_permutation,
    pin_prefill_select,
    pin_e4m3_decode_library,
    pin_e4m3_known_values,
    pin_e4m3_encode_bruteforce,
    pin_e4m3_encode_library,
    pin_fp8_cache_values,
    pin_cache_append_fp8,
    pin_fused_query_equals_unfolded,
    pin_fused_output_equals_unfolded,
    pin_folds_bruteforce,
]
