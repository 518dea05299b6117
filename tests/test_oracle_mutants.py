"""Planted-mistake check for the oracle's pins.

Each case copies the oracle's source, plants one plausible mistake (a dropped
term, a wrong index, a reversed order, a wrong rounding rule) and runs a few
pins against the copy on the CPU.  At least one pin must fail, which shows the
pins constrain that part of the oracle.  The real oracle is never modified.
"""

import json
import os
import types

import numpy as np
import pytest

import tests.test_oracle_fp8_rows as FR
import tests.test_oracle_nonfinite as NF
import tests.test_oracle_numerics as NUM
import tests.test_oracle_routing as RT
import tests.test_oracle_scales as SC

HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(os.path.dirname(HERE), "oracle", "epdc_oracle.py")
with open(SRC_PATH) as f:
    SRC = f.read()
with open(os.path.join(HERE, "golden", "hand_worked_tiny.json")) as f:
    GOLDEN = json.load(f)


def make_mutant(old, new):
    """Copy of the oracle with ``old`` replaced by ``new`` (str or lists)."""
    olds = [old] if isinstance(old, str) else old
    news = [new] if isinstance(new, str) else new
    src = SRC
    for o, n in zip(olds, news):
        assert src.count(o) >= 1, f"mutation anchor not found: {o!r}"
        src = src.replace(o, n, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pin(module, name, *args):
    return (module, name, args)


ROUTING_PINS = [
    pin(RT, "test_hand_worked_metadata", GOLDEN),
    pin(RT, "test_layout_equals_lexsort", "tiny"),
    pin(RT, "test_layout_invariants_skewed"),
    pin(RT, "test_chunk_bounds_cases", GOLDEN),
]
REGROUP_PINS = [
    pin(RT, "test_regroup_equals_stable_sort_and_bincount", 4),
    pin(RT, "test_regroup_groups_are_segments_end_to_end"),
    pin(RT, "test_regroup_brute_force_tiny"),
    pin(RT, "test_regroup_restore_is_weighted_sum"),
]
PARTIAL_PINS = [
    pin(NUM, "test_combine_partials_counts_each_destination_once"),
    pin(NUM, "test_combine_partials_within_1ulp_of_exact_sum"),
    pin(NUM, "test_combine_partials_single_destination_is_copy"),
    pin(NUM, "test_combine_biases_are_added"),
]
COMBINE_PINS = [
    pin(NUM, "test_combine_hand_worked", GOLDEN),
    pin(NUM, "test_combine_order_is_k_ascending"),
    pin(NUM, "test_combine_rounds_product_before_sum"),
    pin(NUM, "test_combine_identity_round_trip_within_1ulp"),
    pin(NUM, "test_combine_k1_weight1_is_copy_and_unrouted_is_zero"),
]
FORMAT_PINS = [
    pin(NUM, "test_bf16_rne_matches_torch"),
    pin(NUM, "test_e4m3_encode_matches_torch"),
    pin(NUM, "test_e4m3_hand_cases", GOLDEN),
    pin(NUM, "test_quantize_hand_row", GOLDEN),
    pin(NUM, "test_quantize_properties"),
]
SCALE_PINS = [
    pin(SC, "test_pow2_is_the_smallest_power_at_or_above"),
    pin(SC, "test_ue8m0_bytes_match_torch_e8m0_on_powers_of_two"),
    pin(SC, "test_ue8m0_small_scales_clamp_to_the_lowest_code"),
    pin(SC, "test_packing_is_a_little_endian_int_view"),
    pin(SC, "test_scale_formats_hand_worked"),
    pin(SC, "test_pow2_and_ue8m0_codes_against_torch"),
    pin(SC, "test_batched_fp8_is_the_gather_of_quantized_rows"),
]
NONFINITE_PINS = [
    pin(NF, "test_bf16_nan_is_the_canonical_quiet_nan"),
    pin(NF, "test_e4m3_nan_code_and_saturation"),
    pin(NF, "test_nan_elements_do_not_move_amax"),
    pin(NF, "test_all_nan_group_keeps_its_nans"),
    pin(NF, "test_infinite_group_gets_an_infinite_scale"),
]
FP8_ROW_PINS = [
    pin(FR, "test_dequantize_matches_torch_decode_times_scale"),
    pin(FR, "test_dequantize_hand_row"),
    pin(FR, "test_dequantize_rounds_the_float32_product_once_to_bf16"),
    pin(FR, "test_dispatch_permute_fp8_is_each_send_row_quantized"),
    pin(FR, "test_dispatch_permute_fp8_follows_any_row_order"),
]
BATCHED_PINS = [
    pin(RT, "test_batched_equals_stable_argsort", 0, 32),
    pin(RT, "test_hand_worked_permute_and_batched", GOLDEN),
]

MUTANTS = {
    "chunk_last_no_remainder": (
        "end = num_tokens if i == chunks - 1 else (i + 1) * size",
        "end = (i + 1) * size", ROUTING_PINS),
    "owner_strided_not_contiguous": (
        "dest = np.where(idx >= 0, idx // El, -1).astype(np.int32)",
        "dest = np.where(idx >= 0, idx % P, -1).astype(np.int32)", ROUTING_PINS),
    "tokens_descending_in_segment": (
        "for t in np.flatnonzero(is_in_rank[:, p]):",
        "for t in np.flatnonzero(is_in_rank[:, p])[::-1]:", ROUTING_PINS),
    "local_id_not_rebased": (
        "send_idx[n, owned] = idx[t, owned] - p * El",
        "send_idx[n, owned] = idx[t, owned]", ROUTING_PINS),
    "weights_copied_on_all_slots": (
        "send_w[n, owned] = w[t, owned]",
        "send_w[n] = w[t]", ROUTING_PINS),
    "counts_per_slot_not_per_token": (
        "is_in_rank[:, p] = (dest == p).any(axis=1)",
        "is_in_rank[:, p] = np.minimum((dest == p).sum(axis=1), 1) * 0 + (dest == p).sum(axis=1)",
        ROUTING_PINS),
    "combine_k_descending": (
        "for k in range(K):\n        r = row[:, k]",
        "for k in reversed(range(K)):\n        r = row[:, k]", COMBINE_PINS),
    "combine_unweighted": (
        "prod = (w[m, k][:, None] * bf16_to_f32(y[r[m]])).astype(np.float32)",
        "prod = bf16_to_f32(y[r[m]]).astype(np.float32)", COMBINE_PINS),
    "combine_f64_accumulate": (
        ["acc = np.zeros((T, H), dtype=np.float32)",
         "acc[m] = (acc[m] + prod).astype(np.float32)"],
        ["acc = np.zeros((T, H), dtype=np.float64)",
         "acc[m] = acc[m] + prod"], COMBINE_PINS),
    "combine_fused_multiply_add": (
        ["prod = (w[m, k][:, None] * bf16_to_f32(y[r[m]])).astype(np.float32)",
         "acc[m] = (acc[m] + prod).astype(np.float32)"],
        ["prod = w[m, k][:, None].astype(np.float64) * bf16_to_f32(y[r[m]])",
         "acc[m] = (acc[m] + prod).astype(np.float32)"], COMBINE_PINS),
    "combine_truncating_bf16": (
        "pick_upper = (rem > half) | ((rem == half) & ~lower_even)",
        "pick_upper = rem < 0", COMBINE_PINS + FORMAT_PINS[:1]),
    "bf16_ties_away": (
        "pick_upper = (rem > half) | ((rem == half) & ~lower_even)",
        "pick_upper = rem >= half", FORMAT_PINS),
    "e4m3_ties_away": (
        "take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))",
        "take_hi = d_hi <= d_lo", FORMAT_PINS),
    "e4m3_bias_8": (
        "(1.0 + m / 8.0) * 2.0 ** (e - 7.0)",
        "(1.0 + m / 8.0) * 2.0 ** (e - 8.0)", FORMAT_PINS),
    "fp8_scale_from_max_not_448": (
        "scale = (amax / np.float32(FP8_MAX)).astype(np.float32)",
        "scale = (amax / np.float32(240.0)).astype(np.float32)", FORMAT_PINS),
    "fp8_group_64": ("FP8_GROUP = 128", "FP8_GROUP = 64", FORMAT_PINS),
    "fp8_zero_group_sign": (
        "zero_group = np.where(np.isnan(g), np.uint8(0x7F), np.uint8(0))",
        "zero_group = np.where(np.isnan(g), np.uint8(0x7F), np.uint8(0x80))", FORMAT_PINS),
    "bf16_nan_rounded_like_finite": (
        "return np.where(is_nan, np.uint16(0x7FC0), out).astype(np.uint16)",
        "return out.astype(np.uint16)", NONFINITE_PINS),
    "e4m3_nan_saturates": (
        "return np.where(np.isnan(mag), 0x7F, code).astype(np.uint8)",
        "return np.where(np.isnan(mag), 0x7E, code).astype(np.uint8)", NONFINITE_PINS),
    "fp8_amax_propagates_nan": (
        "amax = np.where(np.isnan(g), np.float32(0.0), np.abs(g)).max(axis=2)",
        "amax = np.abs(g).max(axis=2)", NONFINITE_PINS),
    "fp8_zero_group_drops_nan": (
        "zero_group = np.where(np.isnan(g), np.uint8(0x7F), np.uint8(0))",
        "zero_group = np.uint8(0)", NONFINITE_PINS),
    "ue8m0_infinite_scale_clamped": (
        "b = np.where(np.isinf(p64), 255, b)",
        "b = np.where(np.isinf(p64), 254, b)", NONFINITE_PINS),
    "pow2_infinite_scale_finite": (
        "p = np.where(fin, p, s64)",
        "p = np.where(fin, p, 1.0)", NONFINITE_PINS),
    "regroup_no_padding": (
        "    padded = [-(-int(c) // A) * A for c in counts]",
        "    padded = [int(c) for c in counts]", REGROUP_PINS),
    "regroup_rows_descending": (
        "        rows = [r for r in range(R) if grp[r] == g and (idx[r] == e).any()]",
        "        rows = [r for r in range(R - 1, -1, -1) if grp[r] == g and (idx[r] == e).any()]",
        REGROUP_PINS),
    "regroup_groups_ignored": (
        "        rows = [r for r in range(R) if grp[r] == g and (idx[r] == e).any()]",
        "        rows = [r for r in range(R) if (idx[r] == e).any()] if g == 0 else []",
        REGROUP_PINS),
    "regroup_weight_of_first_slot_wrong": (
        "            perm_w[n] = w[r, k]",
        "            perm_w[n] = w[r, 0]", REGROUP_PINS),
    "regroup_offset_off_by_one": (
        "            n = offsets[b] + s",
        "            n = offsets[b] + s + (1 if b else 0)", REGROUP_PINS),
    "partials_duplicates_counted": (
        "            if r < 0 or r in seen:",
        "            if r < 0:", PARTIAL_PINS),
    "partials_weighted_by_accident": (
        "            acc[t] = (acc[t] + bf16_to_f32(y[r])).astype(np.float32)",
        "            acc[t] = (acc[t] + 0.5 * bf16_to_f32(y[r])).astype(np.float32)",
        PARTIAL_PINS),
    "bias_dropped": (
        "    for b in biases:\n        acc = (acc + bf16_to_f32(np.asarray(b, dtype=np.uint16)))",
        "    for b in biases[:0]:\n        acc = (acc + bf16_to_f32(np.asarray(b, dtype=np.uint16)))",
        PARTIAL_PINS),
    "bias_subtracted": (
        "acc = (acc + bf16_to_f32(np.asarray(b, dtype=np.uint16))).astype(np.float32)",
        "acc = (acc - bf16_to_f32(np.asarray(b, dtype=np.uint16))).astype(np.float32)",
        PARTIAL_PINS),
    "pow2_rounds_down": (
        "p = np.where(m == 0.5, s64, np.ldexp(1.0, e))",
        "p = np.where(m == 0.5, s64, np.ldexp(1.0, e - 1))", SCALE_PINS),
    "pow2_exact_powers_doubled": (
        "p = np.where(m == 0.5, s64, np.ldexp(1.0, e))",
        "p = np.ldexp(1.0, e)", SCALE_PINS),
    "ue8m0_bias_128": ("UE8M0_BIAS = 127", "UE8M0_BIAS = 128", SCALE_PINS),
    "ue8m0_not_clamped": (
        "np.clip(e + UE8M0_BIAS, 0, 254)", "(e + UE8M0_BIAS) % 256", SCALE_PINS),
    "ue8m0_packed_big_endian": (
        "word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)",
        "word = b[..., 3] | (b[..., 2] << 8) | (b[..., 1] << 16) | (b[..., 0] << 24)",
        SCALE_PINS),
    "ue8m0_quantizes_with_unclamped_power": (
        "scale = np.where(amax > 0, ue8m0_decode(byte), np.float32(0.0)).astype(np.float32)",
        "scale = round_scale_pow2(scale)", SCALE_PINS),
    "batched_fp8_scale_of_next_token": (
        "            b_scale[e, slot] = sc[t]",
        "            b_scale[e, slot] = sc[min(t + 1, T - 1)]", SCALE_PINS),
    "batched_fp8_padding_scale_one": (
        "    b_scale = np.zeros((El, M, sc.shape[1]), dtype=sc.dtype)",
        "    b_scale = np.ones((El, M, sc.shape[1]), dtype=sc.dtype)", SCALE_PINS),
    "dequant_scale_of_neighbouring_group": (
        "prod = (vals * np.asarray(scales, dtype=np.float32)[:, :, None]).astype(np.float32)",
        "prod = (vals * np.roll(np.asarray(scales, dtype=np.float32), 1, axis=1)[:, :, None])"
        ".astype(np.float32)", FP8_ROW_PINS),
    "dequant_scale_rounded_to_bf16_first": (
        "prod = (vals * np.asarray(scales, dtype=np.float32)[:, :, None]).astype(np.float32)",
        "prod = (vals * bf16_to_f32(f32_to_bf16(np.asarray(scales, dtype=np.float32)))"
        "[:, :, None]).astype(np.float32)", FP8_ROW_PINS),
    "dequant_sign_dropped": (
        "vals = e4m3_decode(q).astype(np.float32)",
        "vals = np.abs(e4m3_decode(q)).astype(np.float32)", FP8_ROW_PINS),
    "dequant_groups_interleaved": (
        "vals = e4m3_decode(q).astype(np.float32).reshape(R, H // FP8_GROUP, FP8_GROUP)",
        "vals = e4m3_decode(q).astype(np.float32).reshape(R, FP8_GROUP, H // FP8_GROUP)"
        ".transpose(0, 2, 1)", FP8_ROW_PINS),
    "permute_fp8_gathers_by_row_not_token": (
        "rows = np.asarray(send_token_idx, dtype=np.int64)",
        "rows = np.arange(len(send_token_idx), dtype=np.int64) % len(q)", FP8_ROW_PINS),
    "permute_fp8_scales_of_another_row": (
        "return q[rows].copy(), s[rows].copy()",
        "return q[rows].copy(), s[np.sort(rows)].copy()", FP8_ROW_PINS),
    "batched_slots_descending": (
        "tokens = np.flatnonzero(hit_slots.any(axis=1))",
        "tokens = np.flatnonzero(hit_slots.any(axis=1))[::-1]", BATCHED_PINS),
    "batched_row_stride_wrong": (
        "token_row[t, hit_slots[t]] = e * M + slot",
        "token_row[t, hit_slots[t]] = e * (M - 1) + slot", BATCHED_PINS),
    "batched_padding_not_zero": (
        "b_x = np.zeros((El, M, H), dtype=np.uint16)",
        "b_x = np.ones((El, M, H), dtype=np.uint16)", BATCHED_PINS),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    old, new, pins = MUTANTS[name]
    mod = make_mutant(old, new)
    failures = []
    for module, fn, args in pins:
        monkeypatch.setattr(module, "O", mod)
        try:
            getattr(module, fn)(*args)
        except (AssertionError, ValueError, IndexError) as e:   # the pin fired
            failures.append((fn, type(e).__name__))
    assert failures, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_all_pins(monkeypatch):
    mod = make_mutant("FP8_GROUP = 128", "FP8_GROUP = 128")
    for module, fn, args in (ROUTING_PINS + COMBINE_PINS + FORMAT_PINS + BATCHED_PINS +
                             PARTIAL_PINS + REGROUP_PINS + SCALE_PINS + FP8_ROW_PINS):
        monkeypatch.setattr(module, "O", mod)
        getattr(module, fn)(*args)
