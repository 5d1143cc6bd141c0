"""GPU parity: libmla (through its C ABI) against the float64 CPU oracle.

Small cases and the full-size workloads (the shapes and launch configuration
the bench times, the two largest batches at three seeds) compare every output
element; the margins are printed for each.
Tolerances: float32 storage max-abs 1e-5; bf16 storage max-abs 2e-2 and
relative L2 1e-2.
"""
from __future__ import annotations

import math

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


def _oracle(prob, select=None):
    cache = prob.cache.float().numpy() if prob.cache.dtype == torch.bfloat16 else prob.cache.numpy()
    return orc.mla_decode_reference(prob.f64("q_nope"), prob.f64("q_rope"), cache, prob.block_table, prob.seq_lens,
                                    prob.f64("w_uk"), prob.f64("w_uv"), prob.scale, prob.wl.d_c, select=select)


def _run(prob, num_splits=None):
    """Four-call step, then the fused merge + W_UV call, which must give the same u bit for bit."""
    r = DecodeRunner(prob, num_splits=num_splits)
    r.step()
    torch.cuda.synchronize()
    u_steps = r.u.clone()
    r.u.fill_(0)
    r.combine_absorb_out()
    torch.cuda.synchronize()
    assert torch.equal(r.u, u_steps), "mla_combine_absorb_out differs from mla_combine + mla_absorb_out"
    return r


def _full_check(prob, num_splits=None, check_intermediate=True):
    say(f"case {prob.wl.name} seed={prob.seed} B={prob.wl.batch} H={prob.wl.heads} Lq={prob.wl.q_len} "
        f"lens={prob.seq_lens.tolist()[:8]} splits={num_splits}")
    r = _run(prob, num_splits)
    u, o, lse = _oracle(prob)
    assert_parity(to64(r.u), u, prob.wl.dtype, "u")
    if check_intermediate:
        if prob.wl.dtype == "f32":
            assert_parity(to64(r.o), o, "f32", "o")
            assert_parity(to64(r.lse), lse, "f32", "lse")
        else:
            mo, ro = metrics(to64(r.o), o)
            ml, _ = metrics(to64(r.lse), lse)
            say(f"  o: max_abs={mo:.3e} rel_l2={ro:.3e}  lse: max_abs={ml:.3e}")
            assert ro <= 1e-2 and ml <= 2e-2
    return r


# ------------------------------------------------------------------ small, every element

@pytest.mark.parametrize("seed", [1000, 1001, 1002])
def test_tiny_f32(seed):
    _full_check(make_problem(workload("tiny_f32"), seed))


def test_tiny_f32_poison_big():
    _full_check(make_problem(workload("tiny_f32"), 1003, poison="big"))


def test_bf16_ragged_h128():
    wl = workload("single_4k_bf16", batch=5, lengths=("fixed", (1, 63, 65, 200, 1000)))
    _full_check(make_problem(wl, 7))


def test_bf16_mtp2_h16_ragged():
    wl = workload("mtp2_lognormal_bf16", batch=8, lengths=("fixed", (2, 3, 64, 65, 127, 128, 129, 700)))
    _full_check(make_problem(wl, 11))


@pytest.mark.parametrize("heads,q_len", [(64, 1), (32, 2), (8, 2), (20, 1), (32, 1)])
def test_bf16_row_groups(heads, q_len):
    """64 query rows per sequence (two waves per 32-row group split the score
    contraction) and 32 or fewer (four waves split it; 20 leaves rows past R
    in the group): every element against the oracle."""
    wl = workload("mtp2_lognormal_bf16", batch=6, heads=heads, q_len=q_len,
                  lengths=("fixed", (2, 63, 65, 129, 700, 2049)))
    _full_check(make_problem(wl, 13))


def test_bf16_poison_big():
    wl = workload("single_4k_bf16", batch=2, lengths=("fixed", (70, 300)))
    _full_check(make_problem(wl, 12, poison="big"))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, None, 64])
def test_split_sweep(splits):
    wl = workload("single_4k_bf16", batch=3, lengths=("fixed", (2100, 64, 130)))
    r = _full_check(make_problem(wl, 21), num_splits=splits, check_intermediate=False)
    hdr, segs, _ = replay_schedule(r.workspace.cpu().numpy())
    per_seq = {}
    for (_, b, t0, t1, s, ns, g) in segs:
        per_seq.setdefault((b, g), []).append((t0, t1, s, ns))
    for b, L in enumerate(r.prob.seq_lens):
        for g in range(hdr["hg"]):  # each head group covers the sequence on its own
            pieces = sorted(per_seq[(b, g)])
            assert pieces[0][0] == 0 and pieces[-1][1] == L
            assert all(p[1] == q[0] for p, q in zip(pieces, pieces[1:]))  # contiguous, no overlap
            assert [p[2] for p in pieces] == list(range(len(pieces)))
            assert len(pieces) == pieces[0][3] <= r.num_splits


@pytest.mark.parametrize("batch", [256, 257, 600])
def test_many_sequences(batch):
    """More sequences than the planner has threads: its prefix sum runs over
    several windows and its searches read the sums from the workspace.  Every
    element against the oracle, and the schedule's sums against the lengths."""
    rng = np.random.default_rng(batch)
    lens = tuple(int(x) for x in rng.integers(1, 200, size=batch))
    wl = workload("mtp2_lognormal_bf16", batch=batch, q_len=1, lengths=("fixed", lens))
    r = _full_check(make_problem(wl, 17), check_intermediate=False)
    hdr, segs, got = replay_schedule(r.workspace.cpu().numpy())
    assert hdr["B"] == batch and hdr["error"] == 0
    assert np.array_equal(got, r.prob.seq_lens)
    covered = {}
    for (_, b, t0, t1, _, _, _) in segs:
        covered[b] = covered.get(b, 0) + (t1 - t0)
    assert covered == {b: int(L) for b, L in enumerate(r.prob.seq_lens)}


def test_block_permutation_bit_identical():
    wl = workload("single_4k_bf16", batch=3, lengths=("fixed", (700, 129, 1500)))
    p = make_problem(wl, 31)
    r1 = _run(p)
    u1 = r1.u.clone()
    rng = np.random.default_rng(5)
    perm = rng.permutation(p.num_blocks)
    cache2 = torch.empty_like(p.cache)
    cache2[torch.from_numpy(perm)] = p.cache
    p.block_table = np.where(p.block_table >= 0, perm[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    p.cache = cache2
    r2 = _run(p)
    assert torch.equal(u1, r2.u)


@pytest.mark.parametrize("name,lens", [("single_4k_bf16", (1, 63, 65, 200, 1000, 4097)),
                                       ("mtp2_lognormal_bf16", (2, 3, 64, 65, 700, 2049))])
def test_matrix_core_and_portable_kernels_agree(name, lens, monkeypatch):
    """Both HIP decode kernels on the same inputs (each is also checked against the oracle)."""
    wl = workload(name, batch=len(lens), lengths=("fixed", lens))
    p = make_problem(wl, 51)
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


# ------------------------------------------------------------------ individual entry points

@pytest.mark.parametrize("name,batch", [("tiny_f32", 3), ("single_4k_bf16", 3), ("single_4k_bf16", 70),
                                        ("mtp2_lognormal_bf16", 40)])
def test_absorb_q_against_oracle(name, batch):
    wl = workload(name, batch=batch, lengths=("fixed", tuple(range(5, 5 + batch))))
    p = make_problem(wl, 41)
    r = DecodeRunner(p)
    r.absorb_q()
    torch.cuda.synchronize()
    ref = orc.absorb_q_reference(p.f64("q_nope"), p.f64("q_rope"), p.f64("w_uk"))
    got = to64(r.q_cat)
    tol = (2.0 ** -8) * np.abs(ref) + 1e-5 if wl.dtype == "bf16" else 1e-5 + 1e-6 * np.abs(ref)
    err = np.abs(got - ref)
    say(f"  absorb_q {name}: max_abs={err.max():.3e}")
    assert (err <= tol).all()


@pytest.mark.parametrize("name,batch", [("tiny_f32", 3), ("single_4k_bf16", 3), ("single_4k_bf16", 70),
                                        ("mtp2_lognormal_bf16", 40)])
def test_absorb_out_against_oracle(name, batch):
    wl = workload(name, batch=batch, lengths=("fixed", tuple(range(5, 5 + batch))))
    p = make_problem(wl, 42)
    r = DecodeRunner(p)
    g = torch.Generator().manual_seed(3)
    o = torch.randn(r.o.shape, generator=g, dtype=torch.float32)
    r.o.copy_(o)
    r.absorb_out()
    torch.cuda.synchronize()
    ref = orc.absorb_out_reference(o.double().numpy(), p.f64("w_uv"))
    got = to64(r.u)
    tol = (2.0 ** -8) * np.abs(ref) + 1e-5 if wl.dtype == "bf16" else 1e-5 + 1e-6 * np.abs(ref)
    err = np.abs(got - ref)
    say(f"  absorb_out {name}: max_abs={err.max():.3e}")
    assert (err <= tol).all()


@pytest.mark.parametrize("name,lens", [("tiny_f32", (37, 200)), ("single_4k_bf16", (1, 70, 640, 3000))])
def test_combine_absorb_out_keeps_latent(name, lens):
    """With o_latent and lse requested, the one-call route writes exactly what mla_combine writes."""
    wl = workload(name, batch=len(lens), lengths=("fixed", lens))
    r = DecodeRunner(make_problem(wl, 51), num_splits=5)
    r.absorb_q()
    r.decode()
    r.combine()
    r.absorb_out()
    torch.cuda.synchronize()
    o1, l1, u1 = r.o.clone(), r.lse.clone(), r.u.clone()
    r.o.fill_(7.0)
    r.lse.fill_(7.0)
    r.u.fill_(0)
    r.combine_absorb_out(keep_latent=True)
    torch.cuda.synchronize()
    assert torch.equal(r.o, o1) and torch.equal(r.lse, l1) and torch.equal(r.u, u1)


def test_graph_replay_matches_eager():
    """The step captured in a HIP graph replays to the eager result, with eager work and input changes between replays."""
    wl = workload("single_4k_bf16", batch=3, lengths=("fixed", (700, 129, 1500)))
    p = make_problem(wl, 61)
    r = DecodeRunner(p)
    r.fused_step()
    torch.cuda.synchronize()
    u_ref = r.u.clone()
    g = r.capture()
    torch.cuda.synchronize()
    for k in range(3):
        r.u.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r.u, u_ref), f"replay {k} differs from the eager step"
        _ = (torch.arange(4096, device=r.u.device, dtype=torch.float32) * k).sum().item()  # eager work between replays
    # new inputs in place: the graph reads them at replay
    r.q_nope.mul_(-1)
    r.fused_step()
    torch.cuda.synchronize()
    u2 = r.u.clone()
    assert not torch.equal(u2, u_ref)
    r.u.fill_(0)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(r.u, u2)


@pytest.mark.parametrize("batch,q_len,S", [(1, 1, 65), (1, 1, 9), (4, 1, 200), (5, 1, 17), (17, 1, 8), (8, 2, 33),
                                          (64, 1, 8), (70, 1, 3)])
def test_merge_row_groups_and_many_splits(batch, q_len, S):
    """Merge of random partials for every tile shape of the merge kernels (1 to 32 rows per tile, so 32 to 1
    block groups per row) and split counts past one block of eight: o and lse against the oracle's
    log-sum-exp merge, and the fused merge + W_UV bit-identical to the two-kernel route."""
    wl = workload("single_4k_bf16", batch=batch, q_len=q_len, heads=8, lengths=("fixed", (64,) * batch))
    p = make_problem(wl, 44)
    r = DecodeRunner(p, num_splits=S)
    assert libmla.mla_combine_absorb_out_fused(r.dims, S) == 1
    g = torch.Generator().manual_seed(S * 1000 + batch)
    o_part = torch.randn(r.o_partial.shape, generator=g).to(r.o_partial.dtype)
    lse_part = torch.randn(r.lse_partial.shape, generator=g) * 4
    drop = torch.rand(r.lse_partial.shape, generator=g) < 0.2  # empty splits anywhere
    lse_part[drop] = -math.inf
    lse_part[0, 0, 0, :] = -math.inf  # a row with no keys
    o_part[drop] = float("nan")  # never read
    r.o_partial.copy_(o_part)
    r.lse_partial.copy_(lse_part)
    r.combine()
    r.absorb_out()
    torch.cuda.synchronize()
    o1, l1, u1 = r.o.clone(), r.lse.clone(), r.u.clone()
    o_ref, lse_ref = orc.lse_merge_reference(o_part.double().numpy(), lse_part.double().numpy())
    got_o, got_l = to64(o1), to64(l1)
    fin = np.isfinite(lse_ref)
    assert np.all(np.isneginf(got_l[~fin])) and np.all(got_o[~fin] == 0)
    err_l = np.abs(got_l[fin] - lse_ref[fin]).max()
    err_o = np.abs(got_o - o_ref).max()
    say(f"  merge B={batch} Lq={q_len} S={S}: lse max_abs {err_l:.2e}, o max_abs {err_o:.2e}")
    assert err_l <= 1e-5 and err_o <= 1e-5
    r.o.fill_(7.0)
    r.lse.fill_(7.0)
    r.u.fill_(0)
    r.combine_absorb_out(keep_latent=True)
    torch.cuda.synchronize()
    assert torch.equal(r.o, o1) and torch.equal(r.lse, l1) and torch.equal(r.u, u1)
    r.u.fill_(0)
    r.combine_absorb_out()  # without the latent outputs
    torch.cuda.synchronize()
    assert torch.equal(r.u, u1)


def test_combine_against_oracle():
    wl = workload("single_4k_bf16", batch=2, heads=4, lengths=("fixed", (5, 6)))
    p = make_problem(wl, 43)
    S = 5
    r = DecodeRunner(p, num_splits=S)
    g = torch.Generator().manual_seed(4)
    o_part = torch.randn(r.o_partial.shape, generator=g).to(r.o_partial.dtype)  # partials are in the storage type
    lse_part = torch.randn(r.lse_partial.shape, generator=g) * 3
    lse_part[0, 0, 0, :] = -math.inf  # a row with no keys at all
    lse_part[0, 0, 1, 1:3] = -math.inf  # some empty splits
    lse_part[1, 0, 2, 4] = 80.0  # a dominant split
    o_part[0, 0, 1, 1:3] = float("nan")  # empty splits' o is never read
    r.o_partial.copy_(o_part)
    r.lse_partial.copy_(lse_part)
    r.combine()
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.lse_merge_reference(o_part.double().numpy(), lse_part.double().numpy())
    got_o, got_l = to64(r.o), to64(r.lse)
    assert np.isneginf(got_l[0, 0, 0]) and np.all(got_o[0, 0, 0] == 0)
    fin = np.isfinite(lse_ref)
    assert np.abs(got_l[fin] - lse_ref[fin]).max() <= 1e-5
    assert np.abs(got_o - o_ref).max() <= 1e-5


@pytest.mark.parametrize("name,lens", [("tiny_f32", (37, 200)), ("single_4k_bf16", (1, 300, 1030)),
                                       ("mtp2_lognormal_bf16", (2, 65, 640))])
def test_decode_partials_against_oracle(name, lens):
    """Each split written by mla_decode equals softmax attention over exactly that split's rows."""
    wl = workload(name, batch=len(lens), lengths=("fixed", lens))
    p = make_problem(wl, 44)
    r = DecodeRunner(p, num_splits=4)
    r.absorb_q()
    r.decode()
    torch.cuda.synchronize()
    hdr, segs, lens_ws = replay_schedule(r.workspace.cpu().numpy())
    assert hdr["error"] == 0 and hdr["B"] == wl.batch
    q_cat = to64(r.q_cat)  # the kernel's own input, so only the decode step is under test
    cache = p.cache.float().numpy()
    o_part, lse_part = to64(r.o_partial), to64(r.lse_partial)
    Lq, H, d_c = wl.q_len, wl.heads, wl.d_c
    Hg = H // hdr["hg"]  # head groups (q_len = 1 only) each hold their own pieces
    seen = set()
    for (_, b, t0, t1, s, ns, g) in segs:
        L = int(p.seq_lens[b])
        sel = np.arange(Lq * H) if hdr["hg"] == 1 else np.arange(g * Hg, (g + 1) * Hg)
        rows = orc.gather_rows(cache, p.block_table, b, L)[t0:t1]
        vis = np.zeros((Lq * H, t1 - t0), dtype=bool)
        for j in range(Lq):
            vis[j * H:(j + 1) * H] = (np.arange(t0, t1) <= L - Lq + j)[None, :]
        o_ref, l_ref = orc.latent_attention_partial_reference(q_cat[b].reshape(Lq * H, -1)[sel], rows, p.scale, d_c,
                                                              vis[sel])
        got_l = lse_part[b, :, :, s].reshape(-1)[sel]
        got_o = o_part[b, :, :, s].reshape(Lq * H, d_c)[sel]
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(got_l), fin)
        tol = 1e-5 if wl.dtype == "f32" else 2e-2
        assert np.abs(got_l[fin] - l_ref[fin]).max() <= tol
        if fin.any():
            assert np.abs(got_o[fin] - o_ref[fin]).max() <= tol
            _, rel = metrics(got_o[fin], o_ref[fin])
            assert rel <= (1e-6 if wl.dtype == "f32" else 1e-2)
        seen.add((b, s))
        for s2 in range(ns, r.num_splits):  # unused splits are marked empty
            assert np.isneginf(lse_part[b, :, :, s2].reshape(-1)[sel]).all()
    assert {b for b, _ in seen} == set(range(wl.batch))


# ------------------------------------------------------------------ full-size workloads, every element

def _full_size_check(name, seed=None):
    """A full-size workload in the launch configuration the bench times (automatic split count, the fused
    merge + W_UV call), every element of u against the oracle at the workload tolerances; lse (max-abs
    2e-2) and the merged latent output o (relative L2 1e-2) in full as well."""
    wl = workload(name)
    p = make_problem(wl, seed)
    say(f"case {name} full size: seed={p.seed} B={wl.batch} H={wl.heads} Lq={wl.q_len} tokens={p.total_tokens}")
    r = _run(p)
    say(f"  splits={r.num_splits}")
    u_gpu, o_gpu, lse_gpu = to64(r.u), to64(r.o), to64(r.lse)
    u_ref, o_ref, lse_ref = _oracle(p)
    assert_parity(u_gpu, u_ref, wl.dtype, f"u {name} seed {p.seed} (every element)")
    ml, rl = metrics(lse_gpu, lse_ref)
    mo, ro = metrics(o_gpu, o_ref)
    say(f"  lse: max_abs={ml:.3e} rel_l2={rl:.3e}  o: max_abs={mo:.3e} rel_l2={ro:.3e}")
    assert np.isfinite(lse_gpu).all() and ml <= 2e-2, f"lse max_abs {ml:.3e}"
    assert ro <= 1e-2, f"o rel_l2 {ro:.3e}"
    return r


def test_full_single_4k():
    _full_size_check("single_4k_bf16")


@pytest.mark.parametrize("k", [0, 1, 2])
def test_full_batch64_1k8k(k):
    _full_size_check("batch64_1k8k_bf16", 3000 + k)


def test_full_long128k():
    """All four 131,072-token sequences, all 128 heads."""
    _full_size_check("long128k_bf16")


@pytest.mark.parametrize("k", [0, 1, 2])
def test_full_mtp2_lognormal(k):
    _full_size_check("mtp2_lognormal_bf16", 5000 + k)


def test_choose_splits_equals_num_splits():
    """mla_choose_splits over host lengths (or a length bound) gives mla_decode_num_splits of their max and sum."""
    from mla_latent_kv_14_amd import binding as libmla
    bf = libmla.make_dims(64, 1, 128, 512, 64, 128, 128, 64, 128, 8192, torch.bfloat16)
    lens = np.random.default_rng(0).integers(1024, 8192, size=64, endpoint=True).astype(np.int32)
    assert libmla.mla_choose_splits(bf, lens) == libmla.mla_decode_num_splits(bf, int(lens.max()), int(lens.sum()))
    assert libmla.mla_choose_splits_fp8(bf, lens) == libmla.mla_decode_num_splits_fp8(bf, int(lens.max()),
                                                                                     int(lens.sum()))
    assert libmla.mla_choose_splits(bf, None, 4096) == libmla.mla_decode_num_splits(bf, 4096, 64 * 4096)
    big = lens.copy()
    big[3], big[4] = 1 << 30, -5  # clamped into [0, MB * block_size]
    clamp = np.clip(big.astype(np.int64), 0, 128 * 64)
    assert libmla.mla_choose_splits(bf, big) == libmla.mla_decode_num_splits(bf, int(clamp.max()), int(clamp.sum()))


@pytest.mark.parametrize("batch,heads,q_len,max_len", [(1, 128, 1, 4096), (2, 128, 1, 4096), (3, 128, 1, 2100),
                                                        (4, 128, 1, 4096), (1, 64, 1, 4096), (5, 64, 1, 4096),
                                                        (1, 16, 2, 4096), (16, 128, 1, 8192)])
def test_head_groups(batch, heads, q_len, max_len):
    """With q_len = 1 and 64 or 128 heads, a batch whose largest possible tile count (B x max_blocks x
    block_size / 64) fits the CUs twice or four times over is scheduled in groups of 32 heads: the schedule
    header records the grouping, every (sequence, group) pair covers its sequence once, and u matches the
    oracle in every element."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wl = workload("single_4k_bf16", batch=batch, heads=heads, q_len=q_len,
                  lengths=("fixed", tuple(max_len - 97 * i for i in range(batch))))
    p = make_problem(wl, 83)
    max_tiles = batch * -(-p.max_blocks * wl.block_size // 64)
    expect = 0
    if q_len == 1 and heads in (64, 128):
        while expect < (2 if heads == 128 else 1) and (max_tiles << (expect + 1)) <= cus:
            expect += 1
    r = _full_check(p, check_intermediate=False)
    hdr, segs, lens = replay_schedule(r.workspace.cpu().numpy())
    say(f"  {cus} CUs, at most {max_tiles} tiles: {hdr['hg']} head groups, splits={r.num_splits}")
    assert hdr["hg"] == 1 << expect and hdr["B"] == batch and hdr["error"] == 0
    assert np.array_equal(lens, p.seq_lens)
    covered = {}
    for (_, b, t0, t1, _, _, g) in segs:
        covered[(b, g)] = covered.get((b, g), 0) + (t1 - t0)
    assert covered == {(b, g): int(p.seq_lens[b]) for b in range(batch) for g in range(hdr["hg"])}


@pytest.mark.parametrize("name,over", [
    ("single_4k_bf16", dict(batch=5, lengths=("fixed", (1, 70, 640, 3000, 129)))),
    ("single_4k_bf16", dict(batch=1, lengths=("fixed", (3000,)))),  # four head groups
    ("mtp2_lognormal_bf16", dict(batch=6, lengths=("fixed", (2, 64, 65, 66, 129, 700)))),
    ("single_4k_fp8", dict(batch=3, lengths=("fixed", (5, 900, 4096)))),
    ("single_4k_fp8", dict(batch=2, lengths=("fixed", (900, 2500)))),  # two head groups
    ("tiny_f32", {}),
])
def test_absorb_q_plan_equals_two_calls(name, over):
    """mla_absorb_q_plan (the planner as one more workgroup of the absorb_q launch) writes the same q_cat and
    the same schedule as mla_absorb_q followed by mla_decode_plan, bit for bit; float32 storage takes the
    portable two-launch route through the same entry point."""
    p = make_problem(workload(name, **over), 71)
    r = DecodeRunner(p)
    outs = []
    for fused in (False, True):
        r.workspace.fill_(-7)
        r.q_cat.zero_()
        if fused:
            r.absorb_q_plan()
        else:
            r.plan()
            r.absorb_q()
        torch.cuda.synchronize()
        outs.append((r.workspace.clone(), r.q_cat.clone()))
    assert torch.equal(outs[0][0], outs[1][0]), "schedule differs"
    assert torch.equal(outs[0][1].view(torch.int16) if outs[0][1].dtype == torch.bfloat16 else outs[0][1],
                       outs[1][1].view(torch.int16) if outs[1][1].dtype == torch.bfloat16 else outs[1][1])
    r.decode_planned()
    r.combine_absorb_out()
    torch.cuda.synchronize()
    u1 = r.u.clone()
    r.u.zero_()
    r.fused_step()
    torch.cuda.synchronize()
    assert torch.equal(r.u, u1)
