"""GPU test of mla_decode_noalloc, the decode entry point that allocates nothing (its work schedule lives
in a library-owned device array): through the C ABI it must give exactly what mla_decode gives with a
caller workspace, on two calls in a row, the second with a smaller batch, and its merged output must meet
the workload tolerances against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_latent_kv_14_amd import binding as libmla
from mla_latent_kv_14_amd.inputs import make_problem, workload
from mla_latent_kv_14_amd.runner import DecodeRunner
from oracle import mla_oracle as orc
from tests.gpu_common import assert_parity, require_gpu, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def _both(prob):
    """(partials of mla_decode with a workspace, partials of mla_decode_noalloc) for one problem."""
    r = DecodeRunner(prob)
    r.absorb_q()
    r.o_partial.fill_(float("nan"))
    r.lse_partial.fill_(float("nan"))
    r.decode()
    torch.cuda.synchronize()
    ref_o, ref_l = r.o_partial.clone(), r.lse_partial.clone()
    r.o_partial.fill_(float("nan"))
    r.lse_partial.fill_(float("nan"))
    libmla.mla_decode_noalloc(r.dims, r.q_cat, r.cache, r.block_table, r.seq_lens, prob.scale, r.num_splits,
                              r.o_partial, r.lse_partial)
    torch.cuda.synchronize()
    return r, (ref_o, ref_l), (r.o_partial.clone(), r.lse_partial.clone())


def _same(ref, got):
    ref_o, ref_l = ref
    got_o, got_l = got
    assert torch.equal(ref_l, got_l), "lse partials differ"
    used = torch.isfinite(ref_l)  # unused splits leave o unwritten
    assert torch.equal(ref_o[used], got_o[used]), "o partials differ"


def test_noalloc_matches_workspace_decode_twice():
    wl_a = workload("single_4k_bf16", batch=5, lengths=("fixed", (1, 63, 700, 2100, 4097)))
    wl_b = workload("single_4k_bf16", batch=2, lengths=("fixed", (300, 65)))
    for wl, seed in ((wl_a, 91), (wl_b, 92)):  # the second call is smaller: the array keeps the first's schedule
        prob = make_problem(wl, seed)
        say(f"case noalloc B={wl.batch} lens={prob.seq_lens.tolist()}")
        r, ref, got = _both(prob)
        _same(ref, got)
        # merged and projected, the no-allocation partials meet the workload tolerances
        r.combine()
        r.absorb_out()
        torch.cuda.synchronize()
        u, _, _ = orc.mla_decode_reference(prob.f64("q_nope"), prob.f64("q_rope"), prob.cache.float().numpy(),
                                           prob.block_table, prob.seq_lens, prob.f64("w_uk"), prob.f64("w_uv"),
                                           prob.scale, wl.d_c)
        assert_parity(to64(r.u), u, wl.dtype, "u from the no-allocation partials")


def test_noalloc_small_row_groups_and_float32():
    """The other kernel shapes: 32 query rows (q_len 2, 16 heads) on the matrix cores, and float32 storage on
    the portable kernel."""
    for wl, seed in ((workload("mtp2_lognormal_bf16", batch=4, lengths=("fixed", (2, 129, 700, 3000))), 93),
                     (workload("tiny_f32"), 94)):
        prob = make_problem(wl, seed)
        say(f"case noalloc {wl.name} B={wl.batch}")
        _, ref, got = _both(prob)
        _same(ref, got)
