"""Helpers shared by the GPU tests: device guard, comparisons, schedule replay."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from mla_latent_kv_14_amd import binding as libmla

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2


def require_gpu():
    """Fail (never skip) when the library or the GPU is missing on a GPU run."""
    if not os.path.exists(libmla.LIB_PATH):
        raise RuntimeError("libmla.so is not built; GPU tests need the HIP library")
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    libmla.load()


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def metrics(gpu: np.ndarray, ref: np.ndarray):
    diff = gpu - ref
    max_abs = float(np.nanmax(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_parity(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values on the GPU"
    max_abs, rel = metrics(gpu, ref)
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: max_abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max_abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{what}: rel_l2 {rel:.3e} > {BF16_REL_L2}"


def pack_fused_weight(w: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """The fragment order the header defines for a fused weight viewed as [n x k]: element (r, c) moves to
    ((r/32)(k/64) + c/64) 2048 + ((c%64)/16) 512 + (((c%16)/8) 32 + r%32) 8 + c%8 (a pure reordering)."""
    return (w.reshape(n // 32, 32, k // 64, 4, 2, 8).permute(0, 2, 3, 4, 1, 5).contiguous()
            .reshape(w.shape))


def unpack_fused_weight(w: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """Inverse of pack_fused_weight."""
    return (w.reshape(n // 32, k // 64, 4, 2, 32, 8).permute(0, 4, 1, 2, 3, 5).contiguous()
            .reshape(w.shape))


PLAN_TILE = 64


WS_HEADER = 16
WS_CU = WS_HEADER + 4 * 1024  # the per-workgroup first-segment words come first


def replay_schedule(ws: np.ndarray):
    """Host replay of the planner's schedule read back from the workspace.

    Header words: chunk, groups, total, maxn, splits, error, B, empty, ov,
    hg_log2.  With head groups (hg = 2^hg_log2 > 1, q_len = 1 only) the
    schedule's B counts (sequence, head group) pairs: entry e is group
    e % hg of sequence e // hg and covers heads [g H / hg, (g + 1) H / hg).
    Entry e occupies [cu[e], cu[e+1]) of the schedule line: ov overhead
    tiles (none for an empty sequence), then its real tiles.  Workgroup w
    owns line tiles [w*chunk, (w+1)*chunk).
    Returns (header dict with the batch B and the group count hg, list of
    segments (w, b, tok_begin, tok_end, split, nsplits, g), lengths per sequence).
    """
    chunk, groups, total, maxn, splits, err, B, empty, ov, hgl = (int(x) for x in ws[:10])
    cu = ws[WS_CU:WS_CU + B + 1].astype(np.int64)
    lens = ws[WS_CU + B + 1:WS_CU + 2 * B + 1].astype(np.int64)
    # the line: entry b takes ceil(len / tile) real tiles, plus ov when it has any
    n = -(-lens // PLAN_TILE)
    n = n + np.where(n > 0, ov, 0)
    assert cu[0] == 0 and np.array_equal(np.diff(cu), n) and cu[B] == total, "schedule prefix sums"
    segs = []
    if chunk > 0:
        for w in range(groups):
            t0, t1 = w * chunk, min((w + 1) * chunk, total)
            for b in range(B):
                if cu[b + 1] == cu[b]:
                    continue
                rs = cu[b] + ov
                lo, hi = max(t0, rs), min(t1, cu[b + 1])
                if lo >= hi:
                    continue
                first = rs // chunk
                segs.append((w, b >> hgl, int((lo - rs) * PLAN_TILE), int(min((hi - rs) * PLAN_TILE, lens[b])),
                             int(w - first), int((cu[b + 1] - 1) // chunk - first + 1), b & ((1 << hgl) - 1)))
    else:
        for b in range(B):
            segs.append((b % groups, b >> hgl, 0, int(lens[b]), 0, 1, b & ((1 << hgl) - 1)))
    if chunk > 0:  # each workgroup's first segment, as the planner precomputes it for the attention kernels
        for w in range(min(groups, 1024)):
            t = w * chunk
            b = int(np.searchsorted(cu, t, side="right")) - 1 if t < total else B
            while b < B and cu[b + 1] <= t:
                b += 1
            want = (b, int(cu[b]), int(cu[b + 1]), int(lens[b])) if b < B else (B, 0, 0, 0)
            got = tuple(int(x) for x in ws[WS_HEADER + 4 * w:WS_HEADER + 4 * w + 4])
            assert got == want, f"first segment of workgroup {w}: {got} != {want}"
    hdr = dict(chunk=chunk, groups=groups, total=total, maxn=maxn, splits=splits, error=err, B=B >> hgl,
               empty=empty, ov=ov, hg=1 << hgl)
    return hdr, segs, lens[::1 << hgl]
