"""CPU tests of the seeded workload generator (shapes, determinism, paging layout)."""
import math

import numpy as np
import pytest
import torch

from mla_latent_kv_14_amd.inputs import WORKLOADS, make_problem, workload


def test_deterministic_by_seed():
    wl = workload("tiny_f32")
    a, b = make_problem(wl, 7), make_problem(wl, 7)
    c = make_problem(wl, 8)
    assert torch.equal(a.q_nope, b.q_nope) and np.array_equal(a.block_table, b.block_table)
    assert not torch.equal(a.q_nope, c.q_nope)


@pytest.mark.parametrize("name", ["tiny_f32", "single_4k_bf16"])
def test_shapes_and_dtypes(name):
    wl = WORKLOADS[name]
    p = make_problem(wl)
    D = wl.d_c + wl.d_rope
    assert p.cache.shape[1:] == (wl.block_size, D)
    assert p.q_nope.shape == (wl.batch, wl.q_len, wl.heads, wl.d_nope)
    assert p.q_rope.shape == (wl.batch, wl.q_len, wl.heads, wl.d_rope)
    assert p.w_uk.shape == (wl.heads, wl.d_nope, wl.d_c)
    assert p.w_uv.shape == (wl.heads, wl.d_v, wl.d_c)
    want = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    assert all(t.dtype == want for t in (p.cache, p.q_nope, p.q_rope, p.w_uk, p.w_uv))
    assert p.scale == pytest.approx(1 / math.sqrt(wl.d_nope + wl.d_rope))


def test_tiny_lengths_and_table():
    p = make_problem(WORKLOADS["tiny_f32"])
    assert list(p.seq_lens) == [37, 200]
    bs = p.wl.block_size
    nblk = [(int(L) + bs - 1) // bs for L in p.seq_lens]
    used = np.concatenate([p.block_table[b, :n] for b, n in enumerate(nblk)])
    assert sorted(used.tolist()) == list(range(p.num_blocks))  # a permutation, no duplicates
    for b, n in enumerate(nblk):
        assert (p.block_table[b, n:] == -1).all()
    # the physical order is shuffled
    assert used.tolist() != list(range(p.num_blocks))


def test_poisoned_tail_only():
    p = make_problem(WORKLOADS["tiny_f32"])
    bs = p.wl.block_size
    for b, L in enumerate(p.seq_lens):
        L = int(L)
        last = int(p.block_table[b, (L - 1) // bs])
        tail = L % bs
        if tail:
            assert torch.isnan(p.cache[last, tail:]).all()
            assert not torch.isnan(p.cache[last, :tail]).any()


def test_uniform_and_lognormal_lengths():
    wl3 = workload("batch64_1k8k_bf16", batch=64)
    rng_lens = make_problem(workload("batch64_1k8k_bf16", d_c=8, d_rope=4, d_nope=4, d_v=4, heads=2)).seq_lens
    assert rng_lens.min() >= 1024 and rng_lens.max() <= 8192 and len(rng_lens) == wl3.batch
    p5 = make_problem(workload("mtp2_lognormal_bf16", d_c=8, d_rope=4, d_nope=4, d_v=4, heads=2))
    assert p5.seq_lens.min() >= 64 and p5.seq_lens.max() <= 32768
    assert 1000 < np.median(p5.seq_lens) < 4000


def test_weight_scale():
    p = make_problem(workload("single_4k_bf16"))
    std = p.w_uk.float().std().item()
    assert abs(std * math.sqrt(512) - 1.0) < 0.02
