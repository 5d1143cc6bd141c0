"""CPU tests of the float64 oracle against its pins, the pages' figures, and planted mistakes."""
from __future__ import annotations

import json
import os
import types

import numpy as np
import pytest

from oracle import mla_oracle as orc
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(orc)


def _footprint_value(e):
    dims = {}
    if "n_kv" in e:
        dims["n_kv"] = e["n_kv"]
    q = e["quantity"]
    if q == "elements":
        return orc.cache_elements_per_token(e["kind"], **dims)
    if q == "bytes":
        return orc.cache_bytes(e["kind"], e["tokens"], e["bytes_per_element"], e.get("layers", 1), **dims)
    if q == "reduction_vs":
        return 100.0 * (1.0 - orc.cache_elements_per_token("mla") / orc.cache_elements_per_token(e["versus"]))
    if q == "relative_to":
        return 100.0 * orc.cache_elements_per_token("mla") / orc.cache_elements_per_token(e["versus"])
    if q == "ratio_to_dh":
        return orc.cache_elements_per_token("mla") / e["d_h"]
    raise KeyError(q)


def _golden_entries():
    with open(os.path.join(GOLDEN, "cache_footprint.json")) as f:
        return json.load(f)["entries"]


@pytest.mark.parametrize("entry", _golden_entries(), ids=lambda e: e["name"])
def test_cache_footprint_matches_pages(entry):
    v = _footprint_value(entry)
    if "printed_kb" in entry:
        assert abs(v / 1e3 - entry["printed_kb"]) <= entry["abs_tol_kb"]
    elif "printed_gb" in entry:
        assert abs(v / 1e9 - entry["printed_gb"]) <= entry["abs_tol_gb"]
    elif "printed_gib" in entry:
        assert abs(v / 2**30 - entry["printed_gib"]) <= entry["abs_tol_gib"]
    elif entry.get("rel_tol", None) == 0:
        assert v == entry["printed"]
    else:
        assert abs(v - entry["printed"]) <= entry["abs_tol"]


def test_oracle_rejects_bad_lengths():
    p = pins.Tiny(0)
    with pytest.raises(ValueError):
        orc.mla_decode_reference(p.q_nope, p.q_rope, p.cache, p.table, np.array([1, 11]), p.w_uk, p.w_uv,
                                 p.scale, p.d_c)  # L < q_len
    with pytest.raises(ValueError):
        orc.mla_decode_reference(p.q_nope, p.q_rope, p.cache, p.table, np.array([5, 13]), p.w_uk, p.w_uv,
                                 p.scale, p.d_c)  # L > max_blocks * bs


# ---- planted mistakes: each mutation of the oracle must be caught by some pin ----

_SRC = open(orc.__file__).read()

MUTATIONS = {
    "drop_rope_term": ("keys = np.concatenate([k_content, k_rope], axis=1)",
                       "keys = np.concatenate([k_content, 0.0 * k_rope], axis=1)"),
    "swap_uk_uv": ("k_content = c @ w_uk[h].T", "k_content = c @ w_uv[h].T"),
    "causal_off_by_one": ("last = L - Lq + j  #", "last = L - Lq + j - 1  #"),
    "no_causal_mask": ("last = L - Lq + j  #", "last = L - 1  #"),
    "missing_scale": ("s = scale * (keys[: last + 1] @ q)", "s = keys[: last + 1] @ q"),
    "log2_lse": ("return e / z, (m + np.log(z))[..., 0]", "return e / z, (m + np.log2(z))[..., 0]"),
    "gather_wrong_slot": ("cache[int(block_table[b, t // bs]), t % bs, :]",
                          "cache[int(block_table[b, t // bs]), (t + 1) % bs, :]"),
    "gather_wrong_block": ("cache[int(block_table[b, t // bs]), t % bs, :]",
                           "cache[int(block_table[b, t // bs - (t >= bs)]), t % bs, :]"),
    "o_uses_one_row_less": ("o[b, j, h] = p @ c[: last + 1]", "o[b, j, h] = p[:-1] @ c[: last]"),
    "merge_unnormalised": ("math.exp(lse_parts[idx + (s,)] - total) * o_parts[idx + (s,)]",
                           "math.exp(lse_parts[idx + (s,)] - m) * o_parts[idx + (s,)]"),
    "absorb_q_rope_dropped": ("out[:, :, h, d_c:] = q_rope[:, :, h, :]", "out[:, :, h, d_c:] = 0.0"),
    "absorb_out_transposed": ("u[:, :, h, :] = o[:, :, h, :] @ w_uv[h].T",
                              "u[:, :, h, :] = (w_uv[h] @ o[:, :, h, :].reshape(-1, o.shape[3]).T).T.reshape(u[:, :, h, :].shape)[..., ::-1]"),
    "partial_scale_dropped": ("s = scale * (rows[idx] @ q_cat[r])", "s = rows[idx] @ q_cat[r]"),
    "rope_sign_flipped": ("out[..., 0::2] = x0 * c - x1 * s_", "out[..., 0::2] = x0 * c + x1 * s_"),
    "rope_half_split_pairs": ("x0, x1 = x[..., 0::2], x[..., 1::2]", "x0, x1 = x[..., : d // 2], x[..., d // 2:]"),
    "rope_exponent_wrong": ("theta = pos / np.power(float(base), 2.0 * p / d)", "theta = pos / np.power(float(base), p / d)"),
    "append_position_off_by_one": ("t = int(seq_lens[b]) - Lq + j\n", "t = int(seq_lens[b]) - Lq + j + 1\n"),
    "append_rope_dropped": ("k = rope_reference(h @ np.asarray(w_kr, dtype=np.float64).T, pos, base)",
                            "k = h @ np.asarray(w_kr, dtype=np.float64).T"),
    "append_wdkv_transposed": ("c = h @ np.asarray(w_dkv, dtype=np.float64).T",
                               "c = (np.asarray(w_dkv, dtype=np.float64) @ np.resize(h, np.asarray(w_dkv).shape[1]))[..., : np.asarray(w_dkv).shape[0]] * 0 + h[..., : np.asarray(w_dkv).shape[0]]"),
    "prefill_causal_off_by_one": ("n_vis = j + 1 if causal else s1 - s0", "n_vis = j + 2 if causal else s1 - s0"),
    "prefill_rope_dropped": ("keys = np.concatenate([c @ w_uk[h].T, k_rope[s0:s1]], axis=1)",
                             "keys = np.concatenate([c @ w_uk[h].T, 0.0 * k_rope[s0:s1]], axis=1)"),
    "prefill_values_from_w_uk": ("vals = c @ w_uv[h].T", "vals = c @ w_uk[h].T"),
    "prefill_global_position": ("j = t - s0  #", "j = t  #"),
    "prefill_missing_scale": ("sc = scale * (keys[:n_vis] @ q)", "sc = keys[:n_vis] @ q"),
    "prefill_rope_query_dropped": ("q = np.concatenate([q_nope[t, h], q_rope[t, h]])\n                n_vis",
                                   "q = np.concatenate([q_nope[t, h], 0.0 * q_rope[t, h]])\n                n_vis"),
    "e4m3_bias_8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "e4m3_subnormal_scale": ("m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    "e4m3_nan_whole_top_binade": ("np.where((e == 15) & (m == 7), np.nan, val)", "np.where(e == 15, np.nan, val)"),
    "e4m3_ties_up": ("np.where(lo % 2 == 0, lo, hi)", "hi"),
    "e4m3_sign_dropped": ("code = pick | np.where(np.signbit(x), 0x80, 0)", "code = pick"),
    "e4m3_nan_on_overflow": ("return np.where(np.isnan(x), 0x7F, code).astype(np.uint8)",
                             "return np.where(np.isnan(x) | (np.abs(x) >= 464), 0x7F, code).astype(np.uint8)"),
    "fp8_scale_inverted": ("return float(kv_scale) * e4m3_decode(codes)", "return e4m3_decode(codes) / float(kv_scale)"),
    "append_fp8_scale_multiplied": ("e4m3_encode(row / row_dtype(kv_scale))", "e4m3_encode(row * row_dtype(kv_scale))"),
    "append_fp8_wrong_slot": ("out[int(block_table[b, pos // bs]), pos % bs, :] = e4m3_encode(",
                              "out[int(block_table[b, pos // bs]), (pos + 1) % bs, :] = e4m3_encode("),
    "append_fp8_position_off_by_one": ("pos = int(seq_lens[b]) - Lq + j  #", "pos = int(seq_lens[b]) - Lq + j - 1  #"),
    "fold_query_rows_reversed": ("np.stack([w_uk[h].T @ w_in[h] for h in range(w_in.shape[0])])",
                                 "np.stack([(w_uk[h].T @ w_in[h])[::-1] for h in range(w_in.shape[0])])"),
    "fused_query_rope_dropped": ("out[:, :, :, d_c:] = q_rope  #", "out[:, :, :, d_c:] = 0.0 * q_rope  #"),
    "fold_output_wrong_block": ("w_o[:, h * d_v:(h + 1) * d_v] @ w_uv[h] for h in range(H)",
                                "w_o[:, h * d_v:(h + 1) * d_v] @ w_uv[(h + 1) % H] for h in range(H)"),
    "fused_output_columns_reversed": ("return o.reshape(B, Lq, H * d_c) @ w_fused.T",
                                      "return o.reshape(B, Lq, H * d_c) @ w_fused[:, ::-1].T"),
}


def _mutant(old, new):
    assert _SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("mla_oracle_mutant")
    exec(compile(_SRC.replace(old, new), "mla_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure means the pin noticed
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
