"""GPU parity when scores span far more than the kernels' fast-path headroom.

The softmax of both attention kernels works against a reference maximum
taken from the first key tile of each piece of work, and recomputes the piece
against each row's observed maximum when a later score exceeds that reference
by more than 64 log2 units.  A plain softmax ("Deconstructing DeepSeek V4
Pro", the forward pass of its MLA module; "DeepSeek-V3 MLA: Multi-Head Latent
Attention Guide", the absorbed decode step) is exact for any spread of
scores, so these inputs plant keys whose score for one chosen (query, head)
lies about 200 log2 units above every other score of that row, always past
the first 32-key tile of the piece that holds them.  Without the recompute
exp2 of such a score overflows float32 and the row turns to inf/NaN, so a
finite result that matches the oracle shows the recompute ran and is exact.

The planted key has k^R = 32 q^R of the chosen row at d_rope = 64 (128 q^R
at d_rope = 16; a power of two, so it is exact in bf16), which adds about
2000 to that raw score.  The
chosen row then attends almost only to the planted key, so its output is
W^UV c of that key: entries of order one (several units), compared to the
same tolerances as every other case (bf16: max-abs 2e-2 and relative L2
1e-2; float32 max-abs 1e-5), except that the bf16 element bar on u adds
2^-7 |u| for the two bf16 roundings such outputs go through (the decode's
split partial and u; the prefill's V and u).  Every element of u and lse is
compared.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_latent_kv_14_amd.inputs import make_prefill_problem, make_problem, workload
from mla_latent_kv_14_amd.runner import DecodeRunner, PrefillRunner
from oracle import mla_oracle as orc
from tests.gpu_common import assert_parity, metrics, replay_schedule, require_gpu, say, to64

pytestmark = pytest.mark.gpu

GAMMA_NUM = 2048.0  # planted k^R = (GAMMA_NUM / d_rope) q^R of the chosen row: 32 q^R at d_rope = 64
SUB = 32  # tokens per key tile of the attention kernels


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def _plants(prob):
    """(b, t, j, h): token t of sequence b gets k^R = GAMMA * q^R[b, j, h].  Tokens 40 (second tile of the
    first piece), the middle and the last one visible to query j; lengths are chosen so that the last token
    sits at least 32 tokens into its 64-aligned piece."""
    wl = prob.wl
    out = []
    for b in range(wl.batch):
        L = int(prob.seq_lens[b])
        for k, t in enumerate(sorted({min(40, L - 1), L // 2 + 40, L - 1})):
            if t >= L or t < SUB:
                continue
            j = wl.q_len - 1 if t == L - 1 else (k % wl.q_len)
            if t > L - wl.q_len + j:
                continue
            qq = prob.q_rope[b, j].float().pow(2).sum(-1)  # |q^R|^2 per head: take the k-th largest
            h = int(torch.argsort(qq, descending=True)[k % wl.heads])
            out.append((b, t, j, h))
    return out


def _plant_decode(prob, plants):
    wl = prob.wl
    bs, d_c = wl.block_size, wl.d_c
    for (b, t, j, h) in plants:
        blk, slot = int(prob.block_table[b, t // bs]), t % bs
        kr = (GAMMA_NUM / wl.d_rope) * prob.q_rope[b, j, h].float()
        if prob.fp8:
            codes = torch.clamp(kr / prob.kv_scale, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
            prob.cache[blk, slot, d_c:] = codes
        else:
            prob.cache[blk, slot, d_c:] = kr.to(prob.cache.dtype)


def _decode_oracle(prob):
    cache = (orc.fp8_cache_values(prob.cache.numpy(), prob.kv_scale) if prob.fp8 else
             prob.cache.float().numpy() if prob.cache.dtype == torch.bfloat16 else prob.cache.numpy())
    return orc.mla_decode_reference(prob.f64("q_nope"), prob.f64("q_rope"), cache, prob.block_table, prob.seq_lens,
                                    prob.f64("w_uk"), prob.f64("w_uv"), prob.scale, prob.wl.d_c)


def _check_planted_past_first_tile(ws, plants, lens):
    """Token 40 and the last token lie at least one key tile into the piece of the schedule that holds them
    (the middle plant may or may not; either way the result must be exact)."""
    hdr, segs, _ = replay_schedule(ws)
    past = 0
    for (b, t, _, _) in plants:
        owners = [(t0, t1) for (_, bb, t0, t1, _, _, _) in segs if bb == b and t0 <= t < t1]
        assert len(owners) == hdr["hg"], (b, t, owners)  # one piece per head group
        for (t0, _) in owners:
            if t - t0 >= SUB:
                past += 1
            else:
                assert t not in (40, int(lens[b]) - 1), f"planted token {t} of sequence {b} is in its piece's first tile"
    say(f"  {past} of {len(plants) * hdr['hg']} (planted key, head group) pairs lie past the first tile of "
        f"their piece")


def _check_lse(gpu, ref, dtype):
    """lse reaches several hundred on the planted rows, where float32 itself resolves only about 3e-5: the
    float32 bar is 1e-5 plus 1e-6 of |lse| (a few float32 roundings of the value); bf16 keeps max-abs 2e-2."""
    err = np.abs(gpu - ref)
    say(f"  lse: max_abs={err.max():.3e} (max |lse| {np.abs(ref).max():.1f})")
    assert np.isfinite(gpu).all()
    if dtype == "f32":
        assert (err <= 1e-5 + 1e-6 * np.abs(ref)).all()
    else:
        assert err.max() <= 2e-2


def _decode_case(wl, seed, num_splits=None):
    prob = make_problem(wl, seed)
    plants = _plants(prob)
    _plant_decode(prob, plants)
    say(f"case {wl.name} H={wl.heads} Lq={wl.q_len} lens={prob.seq_lens.tolist()} splits={num_splits} "
        f"plants={plants}")
    r = DecodeRunner(prob, num_splits=num_splits)
    r.step()
    torch.cuda.synchronize()
    _check_planted_past_first_tile(r.workspace.cpu().numpy(), plants, prob.seq_lens)
    u, o, lse = _decode_oracle(prob)
    # the planted rows are far outside the fast path's range
    q = prob.f64("q_rope")
    for (b, t, j, h) in plants:
        assert (GAMMA_NUM / wl.d_rope) * float(q[b, j, h] @ q[b, j, h]) * prob.scale * np.log2(np.e) > 140
    _check_decode_u(to64(r.u), u, wl.dtype, "u")
    _check_lse(to64(r.lse), lse, wl.dtype)
    mo, ro = metrics(to64(r.o), o)
    say(f"  o: max_abs={mo:.3e} rel_l2={ro:.3e}")
    assert ro <= 1e-2
    r.u.fill_(0)
    r.combine_absorb_out()  # the fused merge + W_UV route over the same partials
    torch.cuda.synchronize()
    _check_decode_u(to64(r.u), u, wl.dtype, "u (fused merge)")


def _check_decode_u(got, u, dtype, what):
    """A planted row attends to one key and returns W^UV c of that key: entries of order one (several units),
    where the bf16 path rounds twice, the split's partial o_s and u itself, half a step (2^-9 relative) each.
    As for the prefill below, the bf16 bar per element is the workloads' 2e-2 plus 2^-7 |u| for those two
    roundings (a factor 2 of margin), with relative L2 1e-2 over the whole output; float32 keeps 1e-5."""
    if dtype == "f32":
        assert_parity(got, u, dtype, what)
        return
    max_abs, rel = metrics(got, u)
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} max|u|={np.abs(u).max():.2f}")
    assert np.isfinite(got).all() and rel <= 1e-2
    over = np.abs(got - u) - (2e-2 + 2.0 ** -7 * np.abs(u))
    if (over > 0).any():
        idx = tuple(int(x) for x in np.unravel_index(np.argmax(over), over.shape))
        say(f"  worst element {idx}: gpu {got[idx]:.5f} oracle {u[idx]:.5f}; {int((over > 0).sum())} over")
    assert (over <= 0).all()


LENS = (700, 2100, 300)  # (L - 1) mod 64 >= 32 for each


@pytest.mark.parametrize("num_splits", [None, 1, 5])
def test_decode_bf16_h128_far_scores(num_splits):
    """128 query rows (four waves of 32 rows)."""
    _decode_case(workload("single_4k_bf16", batch=3, lengths=("fixed", LENS)), 71, num_splits)


@pytest.mark.parametrize("heads,q_len", [(64, 1), (32, 2)])
def test_decode_bf16_64_rows_far_scores(heads, q_len):
    """64 query rows (pairs of waves split the output columns)."""
    _decode_case(workload("mtp2_lognormal_bf16", batch=3, heads=heads, q_len=q_len, lengths=("fixed", LENS)), 72)


@pytest.mark.parametrize("heads,q_len", [(16, 2), (8, 2), (20, 1)])
def test_decode_bf16_32_rows_far_scores(heads, q_len):
    """32 or fewer query rows (the four waves split the output columns)."""
    _decode_case(workload("mtp2_lognormal_bf16", batch=3, heads=heads, q_len=q_len, lengths=("fixed", LENS)), 73)


def test_decode_f32_far_scores():
    """The portable float32 kernel (its online softmax rescales; the case pins it all the same)."""
    _decode_case(workload("tiny_f32", batch=3, lengths=("fixed", (100, 250, 37))), 74)


@pytest.mark.parametrize("heads,q_len", [(128, 1), (16, 2)])
def test_decode_fp8_far_scores(heads, q_len):
    """FP8 cache.  kv_scale = 0.25 gives the codes room for the planted keys (up to 112)."""
    wl = workload("single_4k_fp8", batch=3, heads=heads, q_len=q_len, kv_scale=0.25, lengths=("fixed", LENS))
    _decode_case(wl, 75)


# ------------------------------------------------------------------ prefill

def _prefill_case(wl, seed, causal):
    prob = make_prefill_problem(wl, seed)
    cu = prob.cu_seqlens
    plants = []
    for b in range(wl.batch):
        s0, L = int(cu[b]), int(prob.seq_lens[b])
        for k, t in enumerate(sorted({40, L // 2 + 33, L - 2})):
            if t < SUB or t >= L:
                continue
            i = min(L - 1, t + 5 * k)  # the chosen query sees the key in the causal form too
            qq = prob.q_rope[s0 + i].float().pow(2).sum(-1)
            h = int(torch.argsort(qq, descending=True)[k % wl.heads])
            plants.append((s0 + t, s0 + i, h))
    for (t, i, h) in plants:
        prob.k_rope[t] = ((GAMMA_NUM / wl.d_rope) * prob.q_rope[i, h].float()).to(prob.k_rope.dtype)
    say(f"case {wl.name} H={wl.heads} lens={prob.seq_lens.tolist()} causal={causal} plants={plants}")
    r = PrefillRunner(prob, causal=causal)
    r.prefill()
    torch.cuda.synchronize()
    u, lse = orc.prefill_reference(prob.f64("q_nope"), prob.f64("q_rope"), prob.f64("c_kv"), prob.f64("k_rope"),
                                   prob.cu_seqlens, prob.f64("w_uk"), prob.f64("w_uv"), prob.scale, causal=causal)
    got = to64(r.u)
    max_abs, rel = metrics(got, u)
    say(f"  u: max_abs={max_abs:.3e} rel_l2={rel:.3e} max|u|={np.abs(u).max():.2f}")
    # A prefill row that attends to one key returns that key's V = W^UV c, entries of order one, and the bf16
    # path rounds V (the up-projection output) and u to bf16, half a step (2^-9 relative) each: the bar per
    # element is the workload's 2e-2 plus 2^-7 |u| for those two roundings (with a factor 2 of margin).
    assert np.isfinite(got).all() and rel <= 1e-2
    over = np.abs(got - u) - (2e-2 + 2.0 ** -7 * np.abs(u))
    if (over > 0).any():
        t, h, c = (int(x) for x in np.unravel_index(np.argmax(over), over.shape))
        say(f"  worst element: token {t} head {h} col {c}: gpu {got[t, h, c]:.5f} oracle {u[t, h, c]:.5f}; "
            f"{int((over > 0).sum())} elements over; lse gpu {float(r.lse[t, h]):.4f} oracle {lse[t, h]:.4f}")
    assert (over <= 0).all()
    _check_lse(to64(r.lse), lse, wl.dtype)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_bf16_far_scores(causal):
    wl = workload("prefill_mixed_bf16", batch=3, heads=16, lengths=("fixed", (300, 700, 65)))
    _prefill_case(wl, 81, causal)


def test_prefill_bf16_h128_far_scores():
    wl = workload("prefill_mixed_bf16", batch=2, lengths=("fixed", (520, 90)))
    _prefill_case(wl, 82, True)
