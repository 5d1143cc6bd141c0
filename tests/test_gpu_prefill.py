"""GPU parity of the prefill (mla_prefill) against the float64 oracle.

u: float32 storage max-abs 1e-5; bf16 storage max-abs 2e-2 and relative L2
1e-2.  lse (float32): max-abs 1e-5 for float32 storage, 2e-2 for bf16 (the
bf16 path rounds the up-projected keys to bf16, which moves scores by a few
thousandths).  Small cases compare every element; full-size workloads compare
sampled (token, head) pairs that the oracle computes one by one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_latent_kv_14_amd.inputs import make_prefill_problem, workload
from mla_latent_kv_14_amd.runner import PrefillRunner
from oracle import mla_oracle as orc
from tests.gpu_common import assert_parity, metrics, require_gpu, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def _oracle(prob, causal, select=None):
    return orc.prefill_reference(prob.f64("q_nope"), prob.f64("q_rope"), prob.f64("c_kv"), prob.f64("k_rope"),
                                 prob.cu_seqlens, prob.f64("w_uk"), prob.f64("w_uv"), prob.scale, causal=causal,
                                 select=select)


def _run(prob, causal):
    wl = prob.wl
    say(f"case {wl.name} B={wl.batch} H={wl.heads} lens={prob.seq_lens.tolist()[:10]} causal={causal}")
    r = PrefillRunner(prob, causal=causal)
    r.prefill()
    torch.cuda.synchronize()
    return r


def _check_lse(gpu, ref, dtype, what="lse"):
    m, _ = metrics(gpu, ref)
    say(f"  {what}: max_abs={m:.3e}")
    assert m <= (1e-5 if dtype == "f32" else 2e-2), f"{what}: max_abs {m:.3e}"


def _full_check(prob, causal=True):
    r = _run(prob, causal)
    u, lse = _oracle(prob, causal)
    assert_parity(to64(r.u), u, prob.wl.dtype, "u")
    _check_lse(to64(r.lse), lse, prob.wl.dtype)
    return r


# ------------------------------------------------------------------ small, every element

@pytest.mark.parametrize("causal", [True, False])
def test_prefill_tiny_f32(causal):
    _full_check(make_prefill_problem(workload("prefill_tiny_f32")), causal)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_bf16_ragged(causal):
    # lengths around the 32-key tiles and 256-query blocks, one single token
    wl = workload("prefill_mixed_bf16", batch=6, heads=8, lengths=("fixed", (1, 31, 33, 255, 257, 600)))
    _full_check(make_prefill_problem(wl, 8100), causal)


def test_prefill_bf16_h128():
    wl = workload("prefill_mixed_bf16", batch=2, heads=128, lengths=("fixed", (70, 300)))
    _full_check(make_prefill_problem(wl, 8200))


def test_prefill_bf16_empty_sequence():
    wl = workload("prefill_mixed_bf16", batch=4, heads=4, lengths=("fixed", (40, 1, 1, 90)))
    prob = make_prefill_problem(wl, 8300, seq_lens=np.array([40, 0, 1, 90]))
    _full_check(prob)


def test_prefill_portable_and_mfma_agree(monkeypatch):
    wl = workload("prefill_mixed_bf16", batch=3, heads=4, lengths=("fixed", (5, 130, 290)))
    prob = make_prefill_problem(wl, 8400)
    r_m = _full_check(prob)
    u_m = r_m.u.clone()
    monkeypatch.setenv("MLA_KERNELS", "portable")
    r_p = _full_check(prob)
    m, rel = metrics(to64(u_m), to64(r_p.u))
    say(f"  mfma vs portable: max_abs={m:.3e} rel_l2={rel:.3e}")
    assert m <= 2e-2 and rel <= 1e-2


def test_prefill_rows_equal_decode_steps():
    """A causal prefill row is a decode step over its prefix: the last token of
    each sequence against mla_decode over a paged cache holding the sequence."""
    from mla_latent_kv_14_amd.inputs import make_problem
    from mla_latent_kv_14_amd.runner import DecodeRunner
    wl = workload("prefill_mixed_bf16", batch=3, heads=16, lengths=("fixed", (64, 129, 700)))
    pp = make_prefill_problem(wl, 8500)
    rp = _run(pp, True)
    dw = workload("single_4k_bf16", batch=3, heads=16, lengths=("fixed", tuple(int(x) for x in pp.seq_lens)))
    dp = make_problem(dw, 8500, poison=None)
    # put the prefill problem's rows and last queries into the decode problem
    bs = dw.block_size
    for b in range(wl.batch):
        s0, s1 = int(pp.cu_seqlens[b]), int(pp.cu_seqlens[b + 1])
        rows = torch.cat([pp.c_kv[s0:s1], pp.k_rope[s0:s1]], dim=1)
        for t in range(s1 - s0):
            dp.cache[int(dp.block_table[b, t // bs]), t % bs] = rows[t]
        dp.q_nope[b, 0] = pp.q_nope[s1 - 1]
        dp.q_rope[b, 0] = pp.q_rope[s1 - 1]
    dp.w_uk.copy_(pp.w_uk)
    dp.w_uv.copy_(pp.w_uv)
    rd = DecodeRunner(dp)
    rd.step()
    torch.cuda.synchronize()
    last = [int(pp.cu_seqlens[b + 1]) - 1 for b in range(wl.batch)]
    m, rel = metrics(to64(rp.u[last]), to64(rd.u[:, 0]))
    say(f"  prefill last rows vs decode: max_abs={m:.3e} rel_l2={rel:.3e}")
    assert m <= 2e-2 and rel <= 1e-2


# ------------------------------------------------------------------ full size, sampled

def _sampled(name, n_tok=24, seed=None, causal=True):
    prob = make_prefill_problem(workload(name), seed)
    r = _run(prob, causal)
    rng = np.random.default_rng(7)
    T, H = prob.total_tokens, prob.wl.heads
    toks = set(int(x) for x in rng.integers(0, T, size=n_tok))
    for b in range(prob.wl.batch):  # first, block-edge and last tokens of every sequence
        s0, s1 = int(prob.cu_seqlens[b]), int(prob.cu_seqlens[b + 1])
        toks.update(t for t in (s0, s0 + 255, s0 + 256, s1 - 1) if s0 <= t < s1)
    sel = [(t, int(h)) for t in sorted(toks) for h in rng.choice(H, size=2, replace=False)]
    u, lse = _oracle(prob, causal, select=sel)
    ti = [t for t, _ in sel]
    hi = [h for _, h in sel]
    assert_parity(to64(r.u[ti, hi]), u[ti, hi], prob.wl.dtype, "u (sampled)")
    _check_lse(to64(r.lse[ti, hi]), lse[ti, hi], prob.wl.dtype, "lse (sampled)")


def test_prefill_full_4x4k():
    _sampled("prefill_4x4k_bf16")


def test_prefill_full_mixed():
    _sampled("prefill_mixed_bf16")


def test_prefill_full_mixed_noncausal():
    _sampled("prefill_mixed_bf16", n_tok=12, causal=False)


# ------------------------------------------------------------------ repeatability

@pytest.mark.parametrize("name,heads", [("prefill_4x4k_bf16", 128), ("prefill_mixed_bf16", 5)])
def test_prefill_repeatable(name, heads):
    """Three calls on the same inputs give the same bits: the up-projected workspace, u and lse.  H = 128
    runs the 256 x 256 up-projection tiles, H = 5 (an odd head count) the 128 x 128 ones.  (Both once
    staged their output tile in LDS and let other waves read it without waiting for the writes to land,
    which made a few 16-byte pieces of the workspace differ from call to call.)"""
    prob = make_prefill_problem(workload(name, heads=heads))
    r = PrefillRunner(prob)
    outs = []
    for _ in range(3):
        r.workspace.zero_()
        r.u.zero_()
        r.lse.zero_()
        r.prefill()
        torch.cuda.synchronize()
        outs.append((r.workspace.clone(), r.u.clone(), r.lse.clone()))
    for k in (1, 2):
        nws = int((outs[k][0] != outs[0][0]).sum())
        say(f"  {name} H={heads}: call {k}: {nws} workspace words differ")
        assert nws == 0 and torch.equal(outs[k][1], outs[0][1]) and torch.equal(outs[k][2], outs[0][2])
