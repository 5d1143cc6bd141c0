"""GPU parity of decode over an FP8 (E4M3) latent cache, against the float64 oracle.

The oracle decodes the codes (kv_scale times each code's value, its own E4M3
decoder) and runs the unchanged decode reference.  E4M3 values are exact in
bf16 and float32, so the tolerances are those of the queries' storage type:
float32 max-abs 1e-5; bf16 max-abs 2e-2 and relative L2 1e-2.  Small cases
and the full-size workloads compare every element.  With kv_scale = 1 and
one schedule the FP8 path must equal, bit for bit, the bf16 path run on a
bf16 cache holding the same values.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from mla_latent_kv_14_amd import binding as libmla
from mla_latent_kv_14_amd.inputs import make_problem, workload
from mla_latent_kv_14_amd.runner import DecodeRunner
from oracle import mla_oracle as orc
from tests.gpu_common import assert_parity, metrics, replay_schedule, require_gpu, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def _values(prob):
    return orc.fp8_cache_values(prob.cache.numpy(), prob.kv_scale)


def _oracle(prob, select=None):
    return orc.mla_decode_reference(prob.f64("q_nope"), prob.f64("q_rope"), _values(prob), prob.block_table,
                                    prob.seq_lens, prob.f64("w_uk"), prob.f64("w_uv"), prob.scale, prob.wl.d_c,
                                    select=select)


def _run(prob, num_splits=None, fused=False):
    r = DecodeRunner(prob, num_splits=num_splits)
    if fused:
        r.fused_step()
    else:
        r.step()
    torch.cuda.synchronize()
    return r


def _full_check(prob, num_splits=None, fused=False):
    wl = prob.wl
    say(f"case {wl.name} seed={prob.seed} B={wl.batch} H={wl.heads} Lq={wl.q_len} "
        f"lens={prob.seq_lens.tolist()[:8]} splits={num_splits} fused={fused}")
    r = _run(prob, num_splits, fused)
    u, o, lse = _oracle(prob)
    assert_parity(to64(r.u), u, wl.dtype, "u")
    if not fused:
        if wl.dtype == "f32":
            assert_parity(to64(r.o), o, "f32", "o")
            assert_parity(to64(r.lse), lse, "f32", "lse")
        else:
            mo, ro = metrics(to64(r.o), o)
            ml, _ = metrics(to64(r.lse), lse)
            say(f"  o: max_abs={mo:.3e} rel_l2={ro:.3e}  lse: max_abs={ml:.3e}")
            assert ro <= 1e-2 and ml <= 2e-2
    return r


# ------------------------------------------------------------------ small, every element

@pytest.mark.parametrize("seed", [1000, 1001])
def test_fp8_tiny_f32(seed):
    _full_check(make_problem(workload("tiny_f32_fp8"), seed))


def test_fp8_tiny_f32_poison_big():
    _full_check(make_problem(workload("tiny_f32_fp8"), 1003, poison="big"))


def test_fp8_bf16_ragged_h128():
    # lengths around the 32-token sub-tiles and 64-token blocks
    wl = workload("single_4k_fp8", batch=7, lengths=("fixed", (1, 31, 33, 63, 65, 200, 1000)))
    _full_check(make_problem(wl, 2101))


@pytest.mark.parametrize("heads,q_len", [(64, 1), (16, 2), (32, 1), (8, 2)])
def test_fp8_row_groups(heads, q_len):
    wl = workload("mtp2_lognormal_fp8", batch=4, heads=heads, q_len=q_len, lengths=("fixed", (2, 65, 300, 1100)))
    _full_check(make_problem(wl, 2102))


def test_fp8_poison_big():
    wl = workload("single_4k_fp8", batch=3, lengths=("fixed", (5, 70, 700)))
    _full_check(make_problem(wl, 2103, poison="big"))


@pytest.mark.parametrize("splits", [1, 3, 64, None])
def test_fp8_split_sweep(splits):
    wl = workload("single_4k_fp8", batch=3, lengths=("fixed", (40, 900, 2100)))
    _full_check(make_problem(wl, 2104), num_splits=splits)


def test_fp8_fused_step():
    wl = workload("single_4k_fp8", batch=4, lengths=("fixed", (64, 500, 1500, 3000)))
    _full_check(make_problem(wl, 2105), fused=True)


def test_fp8_partials_against_oracle():
    """Each split written by mla_decode_fp8 equals attention over that split's decoded rows."""
    wl = workload("single_4k_fp8", batch=3, lengths=("fixed", (1, 300, 1030)))
    p = make_problem(wl, 2106)
    r = DecodeRunner(p, num_splits=4)
    r.absorb_q()
    r.decode()
    torch.cuda.synchronize()
    hdr, segs, _ = replay_schedule(r.workspace.cpu().numpy())
    assert hdr["error"] == 0 and hdr["B"] == wl.batch
    q_cat = to64(r.q_cat)
    cache = _values(p)
    o_part, lse_part = to64(r.o_partial), to64(r.lse_partial)
    H, d_c = wl.heads, wl.d_c
    Hg = H // hdr["hg"]  # head groups each hold their own pieces
    seen = set()
    for (_, b, t0, t1, s, ns, g) in segs:
        L = int(p.seq_lens[b])
        hs = slice(g * Hg, (g + 1) * Hg)
        rows = orc.gather_rows(cache, p.block_table, b, L)[t0:t1]
        vis = np.ones((Hg, t1 - t0), dtype=bool)
        o_ref, l_ref = orc.latent_attention_partial_reference(q_cat[b].reshape(H, -1)[hs], rows, p.scale, d_c, vis)
        got_l = lse_part[b, :, :, s].reshape(-1)[hs]
        got_o = o_part[b, :, :, s].reshape(H, d_c)[hs]
        assert np.abs(got_l - l_ref).max() <= 2e-2
        assert np.abs(got_o - o_ref).max() <= 2e-2
        _, rel = metrics(got_o, o_ref)
        assert rel <= 1e-2
        seen.add((b, s))
        for s2 in range(ns, r.num_splits):
            assert np.isneginf(lse_part[b, :, :, s2].reshape(-1)[hs]).all()
    assert {b for b, _ in seen} == set(range(wl.batch))


def test_fp8_matrix_core_and_portable_kernels_agree(monkeypatch):
    wl = workload("single_4k_fp8", batch=5, lengths=("fixed", (1, 63, 65, 1000, 2049)))
    p = make_problem(wl, 2107)
    r1 = _run(p)
    monkeypatch.setenv("MLA_KERNELS", "portable")
    r2 = _run(p)
    monkeypatch.delenv("MLA_KERNELS")
    u_ref, _, _ = _oracle(p)
    assert_parity(to64(r1.u), u_ref, "bf16", "u matrix-core")
    assert_parity(to64(r2.u), u_ref, "bf16", "u portable")
    mx, rel = metrics(to64(r1.o), to64(r2.o))
    say(f"  o matrix-core vs portable: max_abs={mx:.3e} rel={rel:.3e}")
    assert rel <= 1e-2


@pytest.mark.parametrize("name,lens", [("single_4k_fp8", (1, 33, 700, 2500)),
                                       ("mtp2_lognormal_fp8", (2, 64, 129, 900))])
def test_fp8_equals_bf16_cache_of_the_same_values(name, lens):
    """With kv_scale = 1 every cached value is exactly a bf16 value and nothing is rescaled, so the
    FP8 path (copy of the codes, conversion in LDS) must give exactly the bf16 path's result on a
    bf16 cache holding those values: partials, lse and u, bit for bit."""
    wl = workload(name, batch=len(lens), lengths=("fixed", lens), kv_scale=1.0)
    p8 = make_problem(wl, 2108)
    vals = torch.from_numpy(p8.cache.numpy()).view(torch.float8_e4m3fn).to(torch.float32) * wl.kv_scale
    pb = dataclasses.replace(p8, wl=dataclasses.replace(wl, cache_dtype="same"), cache=vals.to(torch.bfloat16))
    assert torch.equal(pb.cache.float()[~torch.isnan(vals)], vals[~torch.isnan(vals)])
    splits = DecodeRunner(p8).num_splits
    rb = _run(pb, splits)
    # the same schedule for both: the bf16 planner's (either planner's schedule serves either call)
    r8 = DecodeRunner(p8, num_splits=splits)
    r8.absorb_q()
    libmla.mla_decode_plan(r8.dims, r8.seq_lens, r8.num_splits, r8.workspace)
    r8.decode_planned()
    r8.combine()
    r8.absorb_out()
    torch.cuda.synchronize()
    for what in ("o_partial", "lse_partial", "o", "lse", "u"):
        a, b = getattr(r8, what), getattr(rb, what)
        if what == "o_partial":  # unused splits are never written
            used = torch.isfinite(r8.lse_partial)
            a, b = a[used], b[used]
        diff = (a.float() - b.float()).abs()
        say(f"  {what}: identical={torch.equal(a, b)} max_abs_diff={float(diff.max()):.3e} "
            f"differing={int((diff > 0).sum())}/{diff.numel()}")
        assert torch.equal(a, b), what


# ------------------------------------------------------------------ full size, every element

def _full_size_check(name, seed=None):
    wl = workload(name)
    p = make_problem(wl, seed)
    say(f"case {name} full size: seed={p.seed} B={wl.batch} tokens={p.total_tokens}")
    r = _run(p, fused=True)
    u_gpu = to64(r.u)
    u_ref, _, _ = _oracle(p)
    assert_parity(u_gpu, u_ref, wl.dtype, f"u {name} (every element)")


def test_fp8_full_single_4k():
    _full_size_check("single_4k_fp8")


def test_fp8_full_batch64_1k8k():
    _full_size_check("batch64_1k8k_fp8")


def test_fp8_full_mtp2_lognormal():
    _full_size_check("mtp2_lognormal_fp8")


# ------------------------------------------------------------------ FP8 append

def _slots(prob):
    wl = prob.wl
    out = []
    for b in range(wl.batch):
        for j in range(wl.q_len):
            t = int(prob.seq_lens[b]) - wl.q_len + j
            out.append((int(prob.block_table[b, t // wl.block_size]), t % wl.block_size, t))
    return out


def _e4m3_half_step(v):
    """Half the spacing of E4M3 values around |v| (3 mantissa bits; subnormal spacing 2^-9)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    return 2.0 ** (e - 4)


def _sum_bound(app, rows_h, d_c):
    """d_model 2^-24 sum_k |h_k| |w_k| per element (float32 sums in any order), RoPE pairs added."""
    w = np.concatenate([app.f64("w_dkv"), app.f64("w_kr")], axis=0)
    t = np.abs(rows_h) @ np.abs(w).T
    pair = t[:, d_c::2] + t[:, d_c + 1::2]
    t[:, d_c::2] = pair
    t[:, d_c + 1::2] = pair
    return app.d_model * 2.0 ** -24 * t


def _append_fp8_check(prob):
    from mla_latent_kv_14_amd.inputs import make_append_inputs
    wl = prob.wl
    app = make_append_inputs(prob)
    say(f"case FP8 append {wl.name} B={wl.batch} Lq={wl.q_len} d_model={app.d_model} "
        f"lens={prob.seq_lens.tolist()[:8]}")
    r = DecodeRunner(prob)
    r.setup_append(app)
    before = r.cache.clone()
    r.cache_append()
    torch.cuda.synchronize()
    after = r.cache
    slots = _slots(prob)
    blk = torch.tensor([s[0] for s in slots], device=after.device)
    slot = torch.tensor([s[1] for s in slots], device=after.device)
    got = after[blk, slot].cpu().numpy()
    h = app.f64("h").reshape(wl.batch * wl.q_len, app.d_model)
    pos = np.array([s[2] for s in slots], dtype=np.int64)
    v64 = orc.cache_rows_reference(h, app.f64("w_dkv"), app.f64("w_kr"), pos, app.rope_base) / prob.kv_scale
    assert np.abs(v64).max() < orc.E4M3_MAX  # no saturation in these inputs
    ref32 = orc.cache_append_fp8_reference(prob.cache.numpy(), prob.block_table, prob.seq_lens, app.f64("h"),
                                           app.f64("w_dkv"), app.f64("w_kr"), prob.kv_scale, app.rope_base,
                                           row_dtype=np.float32)
    ref_codes = ref32[[s[0] for s in slots], [s[1] for s in slots]]
    exact = float((got == ref_codes).mean())
    lim = _e4m3_half_step(v64) + _sum_bound(app, h, wl.d_c) / prob.kv_scale
    worst = float(np.max(np.abs(orc.e4m3_decode(got) - v64) / lim))
    say(f"  codes equal to the oracle's float32 decision: {100 * exact:.3f}%; worst error / bound = {worst:.3f}")
    assert exact >= 0.995
    assert worst <= 1.0
    mask = torch.ones(before.shape[:2], dtype=torch.bool, device=before.device)
    mask[blk, slot] = False
    assert torch.equal(after[mask], before[mask]), "the FP8 append wrote outside the new tokens' slots"
    return r, app


def test_fp8_append_tiny_f32():
    _append_fp8_check(make_problem(workload("tiny_f32_fp8"), 1000))


def test_fp8_append_bf16_ragged():
    wl = workload("single_4k_fp8", batch=6, lengths=("fixed", (1, 31, 33, 64, 65, 1000)))
    _append_fp8_check(make_problem(wl, 2110))


def test_fp8_append_mtp2_block_edges():
    wl = workload("mtp2_lognormal_fp8", batch=5, lengths=("fixed", (2, 64, 65, 129, 700)))
    _append_fp8_check(make_problem(wl, 2111))


def test_fp8_append_full_batch64():
    _append_fp8_check(make_problem(workload("batch64_1k8k_fp8")))


def test_fp8_append_portable_and_mfma_agree(monkeypatch):
    wl = workload("single_4k_fp8", batch=3, lengths=("fixed", (5, 70, 700)))
    p = make_problem(wl, 2112)
    r1, _ = _append_fp8_check(p)
    monkeypatch.setenv("MLA_KERNELS", "portable")
    r2, _ = _append_fp8_check(p)
    monkeypatch.delenv("MLA_KERNELS")
    same = float((r1.cache == r2.cache).float().mean())
    say(f"  matrix-core vs portable append: {100 * same:.4f}% of codes equal")
    assert same >= 0.999


def test_fp8_append_then_decode():
    """The FP8 decode reads the codes the FP8 append wrote: the GPU's append + decode against the oracle's
    append (its own codes, float32 decisions) + decode over the decoded cache."""
    from mla_latent_kv_14_amd.inputs import make_append_inputs
    wl = workload("single_4k_fp8", batch=4, lengths=("fixed", (1, 70, 640, 3000)))
    p = make_problem(wl, 2113)
    app = make_append_inputs(p)
    r = DecodeRunner(p)
    r.setup_append(app)
    r.cache_append()
    r.step()
    torch.cuda.synchronize()
    codes = orc.cache_append_fp8_reference(p.cache.numpy(), p.block_table, p.seq_lens, app.f64("h"),
                                           app.f64("w_dkv"), app.f64("w_kr"), p.kv_scale, app.rope_base,
                                           row_dtype=np.float32)
    u, _, _ = orc.mla_decode_reference(p.f64("q_nope"), p.f64("q_rope"), orc.fp8_cache_values(codes, p.kv_scale),
                                       p.block_table, p.seq_lens, p.f64("w_uk"), p.f64("w_uv"), p.scale, wl.d_c)
    assert_parity(to64(r.u), u, wl.dtype, "u after FP8 append")
