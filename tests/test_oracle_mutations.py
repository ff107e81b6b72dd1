"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each one.  This is what makes the pins meaningful: a dropped term, a
wrong sign, an off-by-one or a transposed mapping must fail at least one."""

import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.decode as odec
import oracle.resolve as ores
import test_oracle as T


def _pins():
    """Run a compact selection of pins; return the names of those that fail."""
    failed = []
    checks = [
        ("bruteforce", lambda: [T.test_bruteforce_agrees(k) for k in T.CASES[::3]]),
        ("golden", lambda: [T.test_golden_row_sets(c) for c in T.GOLDEN_CASES]),
        ("sdpa", lambda: T.test_wide_window_equals_sdpa_causal("TND")),
        ("uniform", lambda: (T.test_uniform_attention_swa_decode_closed_form(),
                             T.test_uniform_attention_with_sink())),
        ("lse", T.test_lse_against_scipy_logsumexp),
        ("fp8", T.test_fp8_decoder_matches_torch_all_codes),
        ("fp16", T.test_fp16_decoder_matches_torch_all_codes),
        ("packed", lambda: T.test_packed_equals_float_on_dequantised_values("int8_packed", 64)),
        ("packed_value", lambda: T.test_packed_value_tensor_equals_float_value_on_dequantised_codes(
            "fp8_e4m3_packed", 0)),
        ("layout", lambda: T.test_layout_and_block_permutation_invariance("csa")),
        ("sink", T.test_sink_closed_form),
        ("merge", T.test_split_merge_equals_unsplit),
        ("cp", T.test_cp_split_invariance),
        ("block_sdpa", lambda: T.test_block_topk_covering_the_prefix_equals_sdpa_causal(8)),
    ]
    for name, fn in checks:
        try:
            with np.errstate(all="ignore"):
                fn()
        except Exception:
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _pins() == []


_orig_ori_visible = ores.ori_visible
_orig_cmp_visible = ores.cmp_visible
_orig_attend = oatt.attend
_orig_phys = ores.physical_row
_orig_fp8 = odec.fp8_e4m3fn_to_f64
_orig_packed = odec.decode_packed
_orig_block_tokens = ores.block_tokens
_orig_fp16 = odec.fp16_to_f64
_orig_packed_value = odec.decode_packed_value


def _band_exclusive(mode, j, p, n, left, right):
    if mode == 4 and left >= 0 and j == p - left:
        return False
    return _orig_ori_visible(mode, j, p, n, left, right)


def _cmp_strict(mode, j, p_c, n, ratio):
    if mode == 3:
        return 0 <= j < n and (j + 1) * ratio < p_c + 1
    return _orig_cmp_visible(mode, j, p_c, n, ratio)


def _no_scale(q, K, V, scale, sinks=None):
    return _orig_attend(q, K, V, 1.0, sinks)


def _sink_negated(q, K, V, scale, sinks=None):
    return _orig_attend(q, K, V, scale, None if sinks is None else -np.asarray(sinks))


def _sink_in_lse(q, K, V, scale, sinks=None):
    O, lse, tot = _orig_attend(q, K, V, scale, sinks)
    return O, tot, tot


def _pa_transposed(P, side, b, j):
    if P.params["layout_kv"] == "PA_BSND":
        bs = int(P.params["%s_block_size" % side])
        table = np.asarray(P.arrays["%s_block_table" % side])
        nblk = table.shape[1]
        return int(table[b, (j % bs) % nblk]) * bs + (j // bs) % bs
    return _orig_phys(P, side, b, j)


def _fp8_bias8(codes):
    return _orig_fp8(codes) / 2.0


def _packed_scale_tiles_swapped(rows_u8, rope_dim, fmt):
    rows = np.array(rows_u8, copy=True)
    so = 512 + 2 * rope_dim
    sc = rows[:, so:so + 16].copy().reshape(-1, 4, 4)
    rows[:, so:so + 16] = sc[:, ::-1, :].reshape(-1, 16)
    return _orig_packed(rows, rope_dim, fmt)


def _v_from_rope(q, K, V, scale, sinks=None):
    return _orig_attend(q, K, K[:, -V.shape[1]:], scale, sinks)


def _fp16_bias16(bits):
    return _orig_fp16(bits) * 0.5                       # exponent bias 16 instead of 15


def _packed_value_ignored(value_u8, key_rows_u8, rope_dim, fmt):
    return _orig_packed(key_rows_u8, rope_dim, fmt)[1]  # V from the key's own codes


def _packed_value_one_scale(value_u8, key_rows_u8, rope_dim, fmt):
    rows = np.array(key_rows_u8, copy=True)
    so = 512 + 2 * rope_dim
    sc = rows[:, so:so + 4].copy()
    for t in range(1, 4):                               # every tile takes tile 0's scale
        rows[:, so + 4 * t:so + 4 * t + 4] = sc
    return _orig_packed_value(value_u8, rows, rope_dim, fmt)


def _block_offset_dropped(v, sbs):
    return [v + u for u in range(sbs)]                  # forgets the block stride


MUTANTS = {
    "window_left_edge_exclusive": (ores, "ori_visible", _band_exclusive),
    "cmp_causal_strict": (ores, "cmp_visible", _cmp_strict),
    "dropped_softmax_scale": (oatt, "attend", _no_scale),
    "sink_sign_flipped": (oatt, "attend", _sink_negated),
    "sink_counted_in_lse": (oatt, "attend", _sink_in_lse),
    "paged_mapping_transposed": (ores, "physical_row", _pa_transposed),
    "fp8_exponent_bias_off_by_one": (odec, "fp8_e4m3fn_to_f64", _fp8_bias8),
    "packed_scale_tiles_reversed": (oatt, "decode_packed", _packed_scale_tiles_swapped),
    "value_taken_from_wrong_columns": (oatt, "attend", _v_from_rope),
    "block_offset_dropped": (ores, "block_tokens", _block_offset_dropped),
    "fp16_exponent_bias_off_by_one": (odec, "fp16_to_f64", _fp16_bias16),
    "packed_value_tensor_ignored": (oatt, "decode_packed_value", _packed_value_ignored),
    "packed_value_one_scale_for_all_tiles": (oatt, "decode_packed_value", _packed_value_one_scale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    if mod is oatt and attr == "attend":
        monkeypatch.setattr(oracle, "attend", fn)
    failed = _pins()
    assert failed, "mutant %s passed every pin" % name
