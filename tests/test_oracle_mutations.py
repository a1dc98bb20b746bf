"""Planted mistakes: each mutant copy of the oracle (built on the CPU from its source with one
plausible error) must fail at least one of the pins, showing that the pins constrain the oracle."""
import inspect
import types

import numpy as np
import pytest

from oracle import mla_oracle as O
import tests.test_oracle_attention as TA
import tests.test_oracle_codec_norms as TC
import tests.test_oracle_next as TN
import tests.test_oracle_tolerance as TT

MUTANTS = {
    "rope_sign": ("ra = a * c - b * s", "ra = a * c + b * s",
                  [(TC, "test_rope_hand_case"), (TA, "test_query_path_matches_torch_complex_route")]),
    "kv_halves_swapped": ("return w[:, :NOPE, :], w[:, NOPE:, :]", "return w[:, V_DIM:, :], w[:, :V_DIM, :]",
                          [(TA, "test_value_half_is_last_rows_of_each_head")]),
    "query_heads_transposed": ("q = q.reshape(q.shape[0], n_heads, QK)",
                               "q = q.reshape(q.shape[0], QK, n_heads).transpose(0, 2, 1).copy()",
                               [(TA, "test_query_path_shape_and_head_column_ownership")]),
    "rotary_score_dropped": ("s = scale * (q_lat @ c.T + np.asarray(q_pe, np.float64) @ pe.T)",
                             "s = scale * (q_lat @ c.T)",
                             [(TA, "test_decode_matches_torch_sdpa")]),
    "scale_dropped": ("s = scale * (q_lat @ c.T + np.asarray(q_pe, np.float64) @ pe.T)",
                      "s = (q_lat @ c.T + np.asarray(q_pe, np.float64) @ pe.T)",
                      [(TA, "test_decode_matches_torch_sdpa")]),
    "absorb_through_value_half": ("uk, _ = wkv_b_heads(bf16_decode(wkv_b_bits), q.shape[0])",
                                  "_, uk = wkv_b_heads(bf16_decode(wkv_b_bits), q.shape[0])",
                                  [(TA, "test_absorbed_equals_expanded")]),
    "causal_diagonal_dropped": ("s = scale * (k[: t + 1] @ q_h[r])", "s = scale * (k[: max(t, 1)] @ q_h[r])",
                                [(TA, "test_prefill_first_row_future_rows_and_sdpa")]),
    "rms_sum_not_mean": ("m2 = np.mean(x * x, axis=-1, keepdims=True)", "m2 = np.sum(x * x, axis=-1, keepdims=True)",
                         [(TC, "test_rmsnorm_hand_case"), (TC, "test_rmsnorm_unit_rms_and_eps_shrink")]),
    "layernorm_unbiased": ("var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)",
                           "var = np.var(x, axis=-1, ddof=1, keepdims=True)",
                           [(TC, "test_layernorm_hand_case")]),
    "combine_weight_sign": ("w = np.where(np.isfinite(ls), np.exp(ls - safe_M), 0.0)",
                            "w = np.where(np.isfinite(ls), np.exp(safe_M - ls), 0.0)",
                            [(TA, "test_split_partition_invariance")]),
    "bf16_truncates": ("r = np.rint(flat[fin] * np.exp2(-q)) * np.exp2(q)",
                       "r = np.trunc(flat[fin] * np.exp2(-q)) * np.exp2(q)",
                       [(TC, "test_bf16_encode_matches_torch_on_fp32_values")]),
    "kv_split_rotary_first": ("lat, _ = rms_norm(a[:, :KV_LORA], kv_gamma, eps)",
                              "lat, _ = rms_norm(a[:, ROPE:], kv_gamma, eps)",
                              [(TN, "test_kv_side_split_order")]),
    "cache_position_shifted": ("pos = int(start_pos[b]) + t", "pos = int(start_pos[b]) + t + 1",
                               [(TN, "test_cache_append_rows_and_decode_roundtrip")]),
    "topk_mask_ignored": ("mask[idx[(idx >= 0) & (idx < L)]] = 0.0", "mask[:] = 0.0",
                          [(TN, "test_topk_equals_dense_decode_over_gathered_rows")]),
    "prefix_offset_dropped": ("t = q_offset + r", "t = r",
                              [(TN, "test_prefix_prefill_equals_tail_of_whole_prefill")]),
    "wo_flatten_value_major": ("x = x.reshape(x.shape[0], -1)",
                               "x = x.transpose(0, 2, 1).reshape(x.shape[0], -1)",
                               [(TN, "test_output_proj_width_flatten_order_and_library")]),
    "gain_ignored": ("y = np.asarray(gamma, dtype=np.float64) * (x * inv)", "y = (x * inv) + 0 * np.asarray(gamma)",
                     [(TA, "test_query_path_matches_torch_complex_route")]),
    "lse_in_log2": ("return (p @ c) / l, (m + np.log(l))[:, 0]", "return (p @ c) / l, (m + np.log2(l))[:, 0]",
                    [(TA, "test_decode_matches_torch_sdpa"), (TA, "test_decode_special_cases")]),
    "combine_lse_without_max": ("lse = np.where(tot > 0, safe_M + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)",
                                "lse = np.where(tot > 0, np.log(np.where(tot > 0, tot, 1.0)), -np.inf)",
                                [(TA, "test_split_partition_invariance")]),
    "prefill_scale_dropped": ("s = scale * (k[: t + 1] @ q_h[r])", "s = (k[: t + 1] @ q_h[r])",
                              [(TA, "test_prefill_first_row_future_rows_and_sdpa")]),
    "prefill_rotary_key_dropped": ("k = np.concatenate([k_nope_h, k_pe], axis=1)",
                                   "k = np.concatenate([k_nope_h, 0 * k_pe], axis=1)",
                                   [(TA, "test_prefill_first_row_future_rows_and_sdpa"),
                                    (TA, "test_prefill_row_equals_decode_over_prefix")]),
    "expand_value_from_key_half": ("v = np.stack([c @ uv[h].T for h in heads], axis=1)",
                                   "v = np.stack([c @ uk[h].T for h in heads], axis=1)",
                                   [(TA, "test_prefill_row_equals_decode_over_prefix"),
                                    (TA, "test_prefill_first_row_future_rows_and_sdpa")]),
    "kv_rotary_key_not_rotated": ("pe = rope_rotate(a[:, KV_LORA:], np.asarray(rope_cs, np.float64))",
                                  "pe = a[:, KV_LORA:] + 0 * np.asarray(rope_cs, np.float64)[:, :1, 0]",
                                  [(TN, "test_kv_side_rotary_key")]),
    "kv_norm_gain_ignored": ("lat, _ = rms_norm(a[:, :KV_LORA], kv_gamma, eps)",
                             "lat, _ = rms_norm(a[:, :KV_LORA], np.ones(KV_LORA), eps)",
                             [(TN, "test_kv_side_latent_norm_and_library")]),
    "topk_first_position_unselectable": ("mask[idx[(idx >= 0) & (idx < L)]] = 0.0",
                                         "mask[idx[(idx >= 1) & (idx < L)]] = 0.0",
                                         [(TN, "test_topk_all_positions_is_dense_decode"),
                                          (TN, "test_topk_special_cases")]),
    "wo_not_transposed": ("return _maybe_round(x @ w.T, staged)",
                          "return _maybe_round(x @ w.reshape(w.shape[1], w.shape[0]), staged)",
                          [(TN, "test_output_proj_width_flatten_order_and_library")]),
    "decode_magnitude_scale_dropped": ("return scale * np.max(np.abs(q_lat) @ c.T", "return np.max(np.abs(q_lat) @ c.T",
                                       [(TT, "test_decode_magnitude_hand_case"),
                                        (TT, "test_decode_magnitude_scaling_sign_and_zero_query")]),
    "decode_magnitude_signed_terms": ("np.max(np.abs(q_lat) @ c.T + np.abs(q[:, NOPE:]) @ pe.T, axis=1)",
                                      "np.max(q_lat @ c.T + q[:, NOPE:] @ pe.T, axis=1)",
                                      [(TT, "test_decode_magnitude_hand_case"),
                                       (TT, "test_decode_magnitude_scaling_sign_and_zero_query")]),
    "prefill_magnitude_scale_dropped": ("mag[j, i] = scale * np.max(", "mag[j, i] = np.max(",
                                        [(TT, "test_prefill_magnitude_hand_case_and_causal_range"),
                                         (TT, "test_prefill_magnitude_scaling_sign_future_rows_and_zero_query")]),
    "prefill_magnitude_sees_next_key": ("np.max(k[: off + r + 1] @ np.abs(q[r, h]))",
                                        "np.max(k[: off + r + 2] @ np.abs(q[r, h]))",
                                        [(TT, "test_prefill_magnitude_hand_case_and_causal_range"),
                                         (TT, "test_prefill_magnitude_scaling_sign_future_rows_and_zero_query")]),
}


def _mutant(old, new):
    src = inspect.getsource(O)
    assert src.count(old) == 1, old
    m = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), m.__dict__)
    return m


def _call(fn):
    sig = inspect.signature(fn)
    if not sig.parameters:
        fn()
        return
    # parametrised pins: run every parameter set of the pin
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    names, values = marks[0].args
    names = [n.strip() for n in names.split(",")]
    for v in values:
        v = v if isinstance(v, (tuple, list)) and len(names) > 1 else (v,)
        fn(**dict(zip(names, v)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    old, new, pins = MUTANTS[name]
    m = _mutant(old, new)
    caught = []
    for mod, pin in pins:
        monkeypatch.setattr(mod, "O", m)
        try:
            with np.errstate(all="ignore"):
                _call(getattr(mod, pin))
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin)
        finally:
            monkeypatch.setattr(mod, "O", O)
    assert caught, f"mutant {name} survived {pins}"


def test_unmutated_source_passes_the_same_pins():
    m = _mutant("import numpy as np", "import numpy as np")
    for _, (old, new, pins) in MUTANTS.items():
        for mod, pin in pins:
            orig = mod.O
            mod.O = m
            try:
                _call(getattr(mod, pin))
            finally:
                mod.O = orig
