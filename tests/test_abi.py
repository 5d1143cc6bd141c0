"""CPU tests of the C-ABI library: it loads, exports what the header declares,
and rejects invalid arguments before touching the device."""
import ctypes
import os
import subprocess
import sys

import pytest

from mla_latent_kv_14_amd import binding as libmla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(libmla.LIB_PATH), reason="libmla.so not built")

FAKE = 0x7F0000001000  # aligned, never dereferenced: every call below fails validation first


def _dims(**kw):
    base = dict(batch=2, q_len=1, num_heads=8, d_c=64, d_rope=16, d_nope=32, d_v=32, block_size=16,
                max_blocks_per_seq=13, num_blocks=16, dtype=libmla.MLA_F32)
    base.update(kw)
    return libmla.mla_dims(**base)


def test_header_symbols_exported():
    lib = libmla.load()
    names = libmla.header_symbols()
    assert {"mla_absorb_q", "mla_decode", "mla_combine", "mla_absorb_out"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_exported_symbols_match_header_exactly():
    out = subprocess.run(["nm", "-D", "--defined-only", libmla.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T mla_" in l})
    assert exported == libmla.header_symbols()


def test_status_and_version():
    lib = libmla.load()
    assert lib.mla_version() >= 100
    for s in (0, -1, -2, -3, -4):
        assert lib.mla_status_str(s)
    assert libmla.status_str(-1) == "invalid argument"
    assert libmla.status_str(libmla.MLA_ERR_WORKSPACE) == "workspace too small"


def test_workspace_bytes_is_host_only():
    n = libmla.mla_decode_workspace_bytes(_dims(batch=1000), 8)
    assert n % 256 == 0 and n >= (8 + 2 * 1000 + 1) * 4


def _call(name, *args):
    return getattr(libmla.load(), name)(*args)


P = ctypes.c_void_p


@pytest.mark.parametrize("mut,expect", [
    ({"batch": 0}, libmla.MLA_ERR_INVALID_ARG),
    ({"num_heads": -1}, libmla.MLA_ERR_INVALID_ARG),
    ({"dtype": 7}, libmla.MLA_ERR_UNSUPPORTED),
    ({"d_c": 60}, libmla.MLA_ERR_UNSUPPORTED),
    ({"d_rope": 12}, libmla.MLA_ERR_UNSUPPORTED),
    ({"q_len": 9}, libmla.MLA_ERR_UNSUPPORTED),
    ({"d_c": 1024, "d_rope": 72}, libmla.MLA_ERR_UNSUPPORTED),
])
def test_bad_dims_rejected(mut, expect):
    d = _dims(**mut)
    assert _call("mla_absorb_q", ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == expect
    assert _call("mla_combine", ctypes.byref(d), 2, P(FAKE), P(FAKE), P(FAKE), None, None) == expect
    assert _call("mla_absorb_out", ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), None) == expect
    sz = ctypes.c_size_t(0)
    assert _call("mla_decode_workspace_bytes", ctypes.byref(d), 2, ctypes.byref(sz)) == expect


def test_null_dims():
    assert _call("mla_absorb_q", None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == libmla.MLA_ERR_INVALID_ARG


def _decode(d, **over):
    args = dict(q_cat=P(FAKE), cache=P(FAKE), table=P(FAKE), lens=P(FAKE), scale=0.1, splits=4, ws=P(FAKE),
                ws_bytes=1 << 20, o=P(FAKE), lse=P(FAKE))
    args.update(over)
    return _call("mla_decode", ctypes.byref(d), args["q_cat"], args["cache"], args["table"], args["lens"],
                 ctypes.c_float(args["scale"]), args["splits"], args["ws"], args["ws_bytes"], args["o"],
                 args["lse"], None)


@pytest.mark.parametrize("over", [
    {"q_cat": None}, {"cache": None}, {"table": None}, {"lens": None}, {"ws": None}, {"o": None}, {"lse": None},
    {"cache": P(FAKE + 4)}, {"o": P(FAKE + 8)},
    {"splits": 0}, {"splits": 5000}, {"scale": 0.0}, {"scale": float("nan")}, {"scale": -1.0},
])
def test_decode_invalid_args(over):
    assert _decode(_dims(), **over) == libmla.MLA_ERR_INVALID_ARG


def test_decode_workspace_too_small():
    d = _dims()
    need = libmla.mla_decode_workspace_bytes(d, 4)
    assert _decode(d, ws_bytes=8) == libmla.MLA_ERR_WORKSPACE
    assert _decode(d, ws_bytes=need - 1) == libmla.MLA_ERR_WORKSPACE
    f = "mla_decode_plan"
    assert _call(f, ctypes.byref(d), P(FAKE), 4, P(FAKE), need - 4, None) == libmla.MLA_ERR_WORKSPACE
    f = "mla_decode_planned"
    assert _call(f, ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), ctypes.c_float(0.1), 4, P(FAKE), 16, P(FAKE),
                 P(FAKE), None) == libmla.MLA_ERR_WORKSPACE


def test_absorb_null_and_misaligned():
    d = _dims()
    assert _call("mla_absorb_q", ctypes.byref(d), None, P(FAKE), P(FAKE), P(FAKE), None) == -1
    assert _call("mla_absorb_q", ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE + 2), P(FAKE), None) == -1
    assert _call("mla_absorb_out", ctypes.byref(d), P(FAKE), None, P(FAKE), None) == -1
    assert _call("mla_combine", ctypes.byref(d), 0, P(FAKE), P(FAKE), P(FAKE), None, None) == -1
    assert _call("mla_combine", ctypes.byref(d), 2, P(FAKE), P(FAKE), P(FAKE), P(FAKE + 4), None) == -1


def test_combine_absorb_out_args():
    d = _dims()
    f = "mla_combine_absorb_out"
    assert _call(f, ctypes.byref(d), 0, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, None) == -1
    assert _call(f, ctypes.byref(d), 2, None, P(FAKE), P(FAKE), P(FAKE), None, None, None) == -1
    assert _call(f, ctypes.byref(d), 2, P(FAKE), P(FAKE), P(FAKE), None, None, None, None) == -1
    assert _call(f, ctypes.byref(d), 2, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE + 4), None, None) == -1
    assert _call(f, ctypes.byref(d), 2, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE + 4), None) == -1
    # float32 storage has no fused kernel: without o_latent there is no intermediate
    d32 = _dims(dtype=0, d_c=64, d_rope=16, d_nope=32, d_v=32)
    assert _call(f, ctypes.byref(d32), 2, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, None) == -2


def test_combine_absorb_out_fused_predicate():
    lib = libmla.load()
    d = _dims(dtype=libmla.MLA_BF16, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128, block_size=64)
    assert lib.mla_combine_absorb_out_fused(ctypes.byref(d), 8) == 1
    assert lib.mla_combine_absorb_out_fused(ctypes.byref(d), 64) == 1
    assert lib.mla_combine_absorb_out_fused(ctypes.byref(d), 65) == 1  # any split count
    assert lib.mla_combine_absorb_out_fused(ctypes.byref(d), 4096) == 1
    assert lib.mla_combine_absorb_out_fused(ctypes.byref(d), 4097) == 0  # past the split limit: invalid
    assert lib.mla_combine_absorb_out_fused(ctypes.byref(d), 0) == 0
    d32 = _dims(dtype=0, d_c=64, d_rope=16, d_nope=32, d_v=32)
    assert lib.mla_combine_absorb_out_fused(ctypes.byref(d32), 8) == 0
    assert lib.mla_combine_absorb_out_fused(None, 8) == 0


def test_num_splits_args():
    d = _dims()
    out = ctypes.c_int32(0)
    assert _call("mla_decode_num_splits", ctypes.byref(d), 0, 10, ctypes.byref(out)) == -1
    assert _call("mla_decode_num_splits", ctypes.byref(d), 100, 10, ctypes.byref(out)) == -1
    assert _call("mla_decode_num_splits", ctypes.byref(d), 100, 200, None) == -1


def test_choose_splits_invalid_args():
    # valid calls query the device's compute units (GPU test); invalid ones fail before that
    import numpy as np
    bf = _dims(dtype=libmla.MLA_BF16, batch=64, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
               block_size=64, max_blocks_per_seq=128, num_blocks=8192)
    out = ctypes.c_int32(0)
    for fn in ("mla_choose_splits", "mla_choose_splits_fp8"):
        assert _call(fn, ctypes.byref(bf), None, 0, ctypes.byref(out)) == -1
        assert _call(fn, ctypes.byref(bf), None, 100, None) == -1
        zeros = np.zeros(64, dtype=np.int32)
        assert _call(fn, ctypes.byref(bf), zeros.ctypes.data_as(ctypes.c_void_p), 0, ctypes.byref(out)) == -1
        assert _call(fn, None, None, 100, ctypes.byref(out)) == -1
    with pytest.raises(ValueError):
        libmla.mla_choose_splits(bf, np.ones(3, dtype=np.int32))


def test_binding_refuses_host_tensors():
    import torch
    d = _dims()
    with pytest.raises(ValueError):
        libmla.mla_combine(d, 2, torch.zeros(2 * 8 * 2 * 64), torch.zeros(2 * 8 * 2), torch.zeros(2 * 8 * 64))


def test_missing_library_fails_loudly(tmp_path):
    # a fresh interpreter with the library path pointed elsewhere must raise, not fall back
    code = ("import mla_latent_kv_14_amd.binding as L; L.LIB_PATH = '/nonexistent/libmla.so'\n"
            "try:\n    L.load()\nexcept RuntimeError as e:\n    print('raised')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in r.stdout


def test_cache_append_workspace_bytes():
    bf = _dims(dtype=libmla.MLA_BF16, batch=64, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
               block_size=64)
    n = libmla.mla_cache_append_workspace_bytes(bf, 7168)
    assert n % 256 == 0 and n >= 64 * 576 * 4  # float32 partials, at least one split
    assert libmla.mla_cache_append_workspace_bytes(bf, 7168 + 8) == 0  # not a multiple of 128: portable kernel
    assert libmla.mla_cache_append_workspace_bytes(_dims(), 96) == 0  # float32 storage: portable kernel
    out = ctypes.c_size_t(0)
    for dm in (0, -1, 1 << 17):
        assert _call("mla_cache_append_workspace_bytes", ctypes.byref(bf), dm, ctypes.byref(out)) == -1
    assert _call("mla_cache_append_workspace_bytes", ctypes.byref(bf), 7168, None) == -1


def _append(d, **over):
    args = dict(d_model=96, h=P(FAKE), w_dkv=P(FAKE), w_kr=P(FAKE), base=10000.0, table=P(FAKE), lens=P(FAKE),
                cache=P(FAKE), ws=P(FAKE), ws_bytes=1 << 24)
    args.update(over)
    return _call("mla_cache_append", ctypes.byref(d), args["d_model"], args["h"], args["w_dkv"], args["w_kr"],
                 ctypes.c_float(args["base"]), args["table"], args["lens"], args["cache"], args["ws"],
                 args["ws_bytes"], None)


@pytest.mark.parametrize("over", [
    {"h": None}, {"w_dkv": None}, {"w_kr": None}, {"table": None}, {"lens": None}, {"cache": None},
    {"h": P(FAKE + 2)}, {"cache": P(FAKE + 8)}, {"d_model": 0}, {"d_model": 1 << 17},
    {"base": 0.0}, {"base": -2.0}, {"base": float("nan")}, {"base": float("inf")},
])
def test_cache_append_invalid_args(over):
    assert _append(_dims(), **over) == libmla.MLA_ERR_INVALID_ARG


def test_cache_append_workspace_checked():
    bf = _dims(dtype=libmla.MLA_BF16, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128, block_size=64)
    need = libmla.mla_cache_append_workspace_bytes(bf, 256)
    assert need > 0
    assert _append(bf, d_model=256, ws=None) == -1
    assert _append(bf, d_model=256, ws_bytes=need - 1) == libmla.MLA_ERR_WORKSPACE
    assert _append(bf, d_model=256, ws=P(FAKE + 4)) == -1


def test_prefill_workspace_bytes():
    bf = _dims(dtype=libmla.MLA_BF16, batch=4, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
    n = libmla.mla_prefill_workspace_bytes(bf, 16384)
    assert n >= 16384 * (128 * 256 + 64) * 2 and n % 256 == 0
    out = ctypes.c_size_t(0)
    assert _call("mla_prefill_workspace_bytes", ctypes.byref(bf), 0, ctypes.byref(out)) == -1
    assert _call("mla_prefill_workspace_bytes", ctypes.byref(bf), 16, None) == -1


def _prefill(d, **over):
    args = dict(T=100, maxlen=60, cu=P(FAKE), qn=P(FAKE), qr=P(FAKE), c=P(FAKE), kr=P(FAKE), wk=P(FAKE),
                wv=P(FAKE), scale=0.1, causal=1, out=P(FAKE), lse=None, ws=P(FAKE), ws_bytes=1 << 30)
    args.update(over)
    return _call("mla_prefill", ctypes.byref(d), args["T"], args["maxlen"], args["cu"], args["qn"], args["qr"],
                 args["c"], args["kr"], args["wk"], args["wv"], ctypes.c_float(args["scale"]), args["causal"],
                 args["out"], args["lse"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over", [
    {"cu": None}, {"qn": None}, {"qr": None}, {"c": None}, {"kr": None}, {"wk": None}, {"wv": None},
    {"out": None}, {"ws": None}, {"qn": P(FAKE + 2)}, {"lse": P(FAKE + 4)},
    {"T": 0}, {"maxlen": 0}, {"maxlen": 101}, {"causal": 2}, {"causal": -1},
    {"scale": 0.0}, {"scale": float("nan")}, {"scale": float("inf")},
])
def test_prefill_invalid_args(over):
    assert _prefill(_dims(), **over) == libmla.MLA_ERR_INVALID_ARG


def test_prefill_workspace_too_small():
    assert _prefill(_dims(), ws_bytes=1024) == libmla.MLA_ERR_WORKSPACE


def test_prefill_grid_limit():
    # batch * heads * ceil(max_seqlen / 256) workgroups of 512 threads past 2^32 - 1: rejected before any launch
    bf = _dims(dtype=libmla.MLA_BF16, batch=1024, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
    T = 60000
    need = libmla.mla_prefill_workspace_bytes(bf, T)
    assert need < 1 << 32
    assert _prefill(bf, T=T, maxlen=16384, ws_bytes=need) == libmla.MLA_ERR_UNSUPPORTED


def test_prefill_bf16_workspace_limit():
    # the matrix-core kernels address the workspace with 32-bit offsets
    bf = _dims(dtype=libmla.MLA_BF16, batch=1, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
    T = 70000
    need = libmla.mla_prefill_workspace_bytes(bf, T)
    assert need >= 1 << 32
    assert _prefill(bf, T=T, maxlen=T, ws_bytes=need) == libmla.MLA_ERR_UNSUPPORTED


def test_fused_output_workspace_bytes():
    bf = _dims(dtype=libmla.MLA_BF16, batch=64, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
               block_size=64)
    n = libmla.mla_fused_output_workspace_bytes(bf, 7168)
    assert n % 256 == 0 and n >= 64 * 7168 * 4  # float32 partials, at least one split
    assert libmla.mla_fused_output_workspace_bytes(bf, 7168 + 32) == 0  # not a multiple of 64: portable kernel
    assert libmla.mla_fused_output_workspace_bytes(_dims(), 64) == 0  # float32 storage: portable kernel
    out = ctypes.c_size_t(0)
    for dout in (0, -1, 1 << 17):
        assert _call("mla_fused_output_workspace_bytes", ctypes.byref(bf), dout, ctypes.byref(out)) == -1
    assert _call("mla_fused_output_workspace_bytes", ctypes.byref(bf), 7168, None) == -1


@pytest.mark.parametrize("over", [
    {"a": None}, {"b": None}, {"c": None}, {"a": P(FAKE + 2)}, {"c": P(FAKE + 8)}, {"n": 0}, {"n": 1 << 17},
])
@pytest.mark.parametrize("fn", ["mla_fold_query_weight", "mla_fold_output_weight"])
def test_fold_invalid_args(fn, over):
    args = dict(n=96, a=P(FAKE), b=P(FAKE), c=P(FAKE))
    args.update(over)
    assert _call(fn, ctypes.byref(_dims()), args["n"], args["a"], args["b"], args["c"], None) == -1


@pytest.mark.parametrize("over", [
    {"x": None}, {"w": None}, {"q": None}, {"r": None}, {"x": P(FAKE + 4)}, {"d_in": 0}, {"d_in": 1 << 17},
])
def test_fused_query_invalid_args(over):
    args = dict(d_in=96, x=P(FAKE), r=P(FAKE), w=P(FAKE), q=P(FAKE))
    args.update(over)
    assert _call("mla_fused_query", ctypes.byref(_dims()), args["d_in"], args["x"], args["r"], args["w"],
                 args["q"], None) == -1


@pytest.mark.parametrize("over", [
    {"o": None}, {"w": None}, {"y": None}, {"o": P(FAKE + 4)}, {"d_out": 0}, {"d_out": 1 << 17},
    {"ws": None}, {"ws": P(FAKE + 4)}, {"ws_bytes": 0},
])
def test_fused_output_invalid_args(over):
    bf = _dims(dtype=libmla.MLA_BF16, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128, block_size=64)
    args = dict(d_out=256, o=P(FAKE), w=P(FAKE), y=P(FAKE), ws=P(FAKE), ws_bytes=1 << 24)
    args.update(over)
    expect = libmla.MLA_ERR_WORKSPACE if over.get("ws_bytes") == 0 else libmla.MLA_ERR_INVALID_ARG
    assert _call("mla_fused_output", ctypes.byref(bf), args["d_out"], args["o"], args["w"], args["y"], args["ws"],
                 args["ws_bytes"], None) == expect


def test_fused_weight_packed_predicates():
    bf = _dims(dtype=libmla.MLA_BF16, batch=64, num_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
               block_size=64)
    assert libmla.mla_fused_query_weight_packed(bf, 1536)
    assert not libmla.mla_fused_query_weight_packed(bf, 1536 + 32)  # d_in not a multiple of 64
    assert libmla.mla_fused_output_weight_packed(bf, 7168)
    assert not libmla.mla_fused_output_weight_packed(bf, 7168 + 64)  # d_out not a multiple of 256
    assert not libmla.mla_fused_query_weight_packed(_dims(), 128)  # float32 storage: row-major
    assert not libmla.mla_fused_output_weight_packed(_dims(), 256)
    for bad in (0, -5, 1 << 17):
        assert not libmla.mla_fused_query_weight_packed(bf, bad)
        assert not libmla.mla_fused_output_weight_packed(bf, bad)


def test_fused_products_row_limit():
    big = _dims(batch=1 << 20, q_len=8)  # 8M rows: past the fused products' limit
    assert _call("mla_fused_query", ctypes.byref(big), 96, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == \
        libmla.MLA_ERR_UNSUPPORTED
    assert _call("mla_fused_output", ctypes.byref(big), 64, P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1 << 40, None) == \
        libmla.MLA_ERR_UNSUPPORTED


# ------------------------------------------------------------------ measurement library (libmla_roofs.so)

def _roofs_header_symbols():
    import re
    from mla_latent_kv_14_amd import roofs
    with open(roofs.HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_roofs_\w+)\s*\(", text, flags=re.M)))


def test_roofs_exports_match_header():
    from mla_latent_kv_14_amd import roofs
    if not os.path.exists(roofs.LIB_PATH):
        pytest.skip("libmla_roofs.so not built")
    out = subprocess.run(["nm", "-D", "--defined-only", roofs.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T mla_" in l})
    assert exported == _roofs_header_symbols()
    assert {"mla_roofs_flush", "mla_roofs_hbm_read", "mla_roofs_mfma_bf16"} <= set(exported)


def test_roofs_invalid_args():
    from mla_latent_kv_14_amd import roofs
    if not os.path.exists(roofs.LIB_PATH):
        pytest.skip("libmla_roofs.so not built")
    lib = roofs.load()
    assert lib.mla_roofs_flush(None, 1 << 20, None) == -1
    assert lib.mla_roofs_flush(P(FAKE), 15, None) == -1
    assert lib.mla_roofs_flush(P(FAKE + 4), 1 << 20, None) == -1
    assert lib.mla_roofs_hbm_read(P(FAKE), 0, 0, P(FAKE), 1 << 20, None) == -1
    assert lib.mla_roofs_hbm_read(P(FAKE), 1 << 20, 0, None, 1 << 20, None) == -1
    flops = ctypes.c_double(0)
    assert lib.mla_roofs_mfma_bf16(0, P(FAKE), 1 << 20, ctypes.byref(flops), None) == -1
    assert lib.mla_roofs_mfma_bf16(10, P(FAKE), 1 << 20, None, None) == -1


def test_decode_noalloc_host_checks():
    """The allocation-free decode validates like mla_decode, and refuses batches past its array's capacity."""
    def call(d, **over):
        a = dict(q_cat=P(FAKE), cache=P(FAKE), table=P(FAKE), lens=P(FAKE), scale=0.1, splits=4, o=P(FAKE),
                 lse=P(FAKE))
        a.update(over)
        return _call("mla_decode_noalloc", ctypes.byref(d), a["q_cat"], a["cache"], a["table"], a["lens"],
                     ctypes.c_float(a["scale"]), a["splits"], a["o"], a["lse"], None)
    d = _dims()
    for over in ({"q_cat": None}, {"lens": None}, {"o": P(FAKE + 4)}, {"splits": 0}, {"scale": float("nan")}):
        assert call(d, **over) == libmla.MLA_ERR_INVALID_ARG
    assert call(_dims(batch=65537)) == libmla.MLA_ERR_WORKSPACE
    assert call(_dims(dtype=9)) == libmla.MLA_ERR_UNSUPPORTED


def _absorb_q_plan(d, fn="mla_absorb_q_plan", **over):
    args = dict(q_nope=P(FAKE), q_rope=P(FAKE), w_uk=P(FAKE), q_cat=P(FAKE), lens=P(FAKE), splits=4, ws=P(FAKE),
                ws_bytes=1 << 20)
    args.update(over)
    return _call(fn, ctypes.byref(d), args["q_nope"], args["q_rope"], args["w_uk"], args["q_cat"], args["lens"],
                 args["splits"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("fn", ["mla_absorb_q_plan", "mla_absorb_q_plan_fp8"])
@pytest.mark.parametrize("over", [
    {"q_nope": None}, {"w_uk": None}, {"q_cat": None}, {"lens": None}, {"ws": None}, {"q_cat": P(FAKE + 4)},
    {"splits": 0}, {"splits": 5000},
])
def test_absorb_q_plan_invalid_args(fn, over):
    """Every argument of both halves is checked before anything is enqueued (no GPU is touched here)."""
    assert _absorb_q_plan(_dims(), fn, **over) == libmla.MLA_ERR_INVALID_ARG


def test_absorb_q_plan_workspace_too_small():
    d = _dims()
    need = libmla.mla_decode_workspace_bytes(d, 4)
    assert _absorb_q_plan(d, ws_bytes=need - 4) == libmla.MLA_ERR_WORKSPACE
    assert _absorb_q_plan(d, "mla_absorb_q_plan_fp8", ws_bytes=8) == libmla.MLA_ERR_WORKSPACE
