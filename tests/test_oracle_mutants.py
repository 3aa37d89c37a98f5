"""Planted mistakes: each test copies oracle.c, plants one plausible mistake
(a dropped term, a wrong index or sign, a wrong rounding rule), builds the copy
on the CPU and checks that at least one of the oracle's pins now fails.  This is
the evidence that the pins constrain every part of the oracle.
"""
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as obuild

from . import test_oracle_dispatch_combine as tdc
from . import test_oracle_formats as tf
from . import test_oracle_layout as tl
from . import test_oracle_ll as tll
from . import test_oracle_variants as tv

MUTANTS = {
    # layout: k walked backwards -> duplicate experts in a row get swapped slots
    "k_order": ("for (int32_t k = 0; k < K; k++) {\n      int32_t e = topk_idx[(int64_t)t * K + k];\n      if (e < 0 || e >= E) {",
                "for (int32_t k = K - 1; k >= 0; k--) {\n      int32_t e = topk_idx[(int64_t)t * K + k];\n      if (e < 0 || e >= E) {"),
    # layout: padding rounds down instead of up
    "pad_round": ("int32_t padded = (cnt + A - 1) / A * A;", "int32_t padded = cnt / A * A + (cnt % A ? 1 : 0);"),
    # layout: expert -> rank map taken modulo instead of quotient
    "rank_map": ("is_token_in_rank[(int64_t)t * R + e / L] = 1;", "is_token_in_rank[(int64_t)t * R + e % R] = 1;"),
    # layout: source rank taken modulo
    "src_map": ("int32_t src = t / T;", "int32_t src = t % R;"),
    # layout: -1 entries not skipped in the counts
    "minus_one": ("      if (e == -1) continue;\n", "      if (e == -1) e = 0;\n"),
    # combine: accumulator overwritten (dropped term)
    "dropped_term": ("acc = acc + p;", "acc = p;"),
    # combine: weight index transposed
    "weight_index": ("float p = topk_weights[(int64_t)t * K + k] * v;", "float p = topk_weights[(int64_t)k * N + t] * v;"),
    # combine: sign slip
    "sign": ("acc = acc + p;", "acc = acc - p;"),
    # bf16: ties away from zero
    "bf16_ties": ("if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;", "if (lo >= 0x8000u) hi += 1u;"),
    # e4m3: ties away from zero in the normal range
    "e4m3_ties": ("double m = nearbyint((2.0 * fr - 1.0) * 8.0);", "double m = round((2.0 * fr - 1.0) * 8.0);"),
    # e4m3: wrong exponent bias
    "e4m3_bias": ("return (uint8_t)(s | (uint8_t)(((E + 7) << 3) | (int)m));", "return (uint8_t)(s | (uint8_t)(((E + 8) << 3) | (int)m));"),
    # e4m3: subnormal step off by a factor of two
    "e4m3_sub": ("double m = nearbyint(a * 512.0);", "double m = nearbyint(a * 256.0);"),
    # quantiser: scale against the wrong constant
    "fp8_scale": ("float scale = amax / 448.0f;", "float scale = amax / 480.0f;"),
    # quantiser: group stride wrong (first element of each group missed)
    "fp8_amax": ("for (int32_t i = 0; i < 128; i++) {\n      float a = fabsf", "for (int32_t i = 1; i < 128; i++) {\n      float a = fabsf"),
    # low-latency layout: counters not reset per source
    "ll_reset": ("    for (int32_t e = 0; e < E; e++) cnt[e] = 0;\n    for (int32_t t = s * T;",
                 "    for (int32_t t = s * T;"),
    # low-latency layout: source-major instead of expert-major sub-blocks
    "ll_slot": ("slot_of[q] = ((e * R) + s) * M + cnt[e];", "slot_of[q] = ((s * E) + e) * M + cnt[e];"),
    # low-latency layout: overflow check off by one
    "ll_overflow": ("if (cnt[e] >= M) {", "if (cnt[e] > M) {"),
    # quantiser: no rescale where 448/amax overflows (zeros become NaN, small
    # values saturate to +-amax)
    "fp8_tiny": ("if (isinf(inv)) {", "if (0) {"),
    # quantiser: the rescale applied to the inverse but not to the values
    "fp8_tiny_vals": ("float v = ldexpf(oracle_bf16_to_f32(xrow[128 * g + i]), pre);",
                      "float v = oracle_bf16_to_f32(xrow[128 * g + i]);"),
    # fp8 dispatch: scales copied to the wrong row
    "fp8_copy": ("memcpy(recv_scales + (int64_t)s * G, sc", "memcpy(recv_scales + (int64_t)t * G, sc"),
    # pre-quantised pass-through: scales taken from the wrong token row
    "q_scales": ("memcpy(recv_scales + (int64_t)s * G, scales + (int64_t)t * G",
                 "memcpy(recv_scales + (int64_t)s * G, scales + (int64_t)k * G"),
    # zero padding: the whole region cleared instead of its tail
    "zp_start": ("for (int64_t s = (int64_t)off[e] + count[e]; s < off[e + 1]; s++)",
                 "for (int64_t s = (int64_t)off[e]; s < off[e + 1]; s++)"),
    # running statistics overwritten instead of accumulated
    "stats": ("stats[e] += count[e];", "stats[e] = count[e];"),
}


def _pins(orc):
    """Every oracle pin, as (name, callable)."""
    yield "golden", lambda: tl.test_worked_example_golden(orc)
    yield "lesson14", lambda: tl.test_lesson14_simulator_end_to_end(orc)
    for trial in range(40):
        yield f"brute{trial}", (lambda tr=trial: tl.test_bruteforce_tiny(orc, tr))
    yield "invariants", lambda: tl.test_invariants(orc, 2, 0)
    yield "e4m3_decode", lambda: tf.test_e4m3_decode_all_codes(orc)
    yield "e4m3_exh", lambda: tf.test_e4m3_encode_exhaustive_bf16_times_inv(orc, 448.0 / 3.0)
    yield "e4m3_torch", lambda: tf.test_e4m3_encode_matches_torch_in_range(orc)
    yield "bf16_torch", lambda: tf.test_bf16_round_matches_torch(orc)
    yield "fp8_closed", lambda: tf.test_quantize_amax_maps_to_448_and_error_bound(orc)
    yield "fp8_pow2", lambda: tf.test_quantize_codes_invariant_under_power_of_two_scaling(orc)
    for w in tdc.CASES:
        yield f"copy_{w.name}", (lambda w=w: tdc.test_dispatch_bf16_is_row_copy(orc, w))
        yield f"rand_{w.name}", (lambda w=w: tdc.test_combine_random_expert_outputs(orc, w))
    for w in tdc.CASES[:2]:
        yield f"ident_{w.name}", (lambda w=w: tdc.test_identity_round_trip_bf16(orc, w))
    yield "fp8_rt", lambda: tdc.test_fp8_dispatch_and_identity_round_trip(orc)
    yield "ll_golden", lambda: tll.test_ll_golden(orc)
    for trial in range(30):
        yield f"ll_brute{trial}", (lambda tr=trial: tll.test_ll_bruteforce(orc, tr))
    for trial in range(3):
        yield f"ll_compact{trial}", (lambda tr=trial: tll.test_ll_agrees_with_compact_layout(orc, tr))
    for w in tv.CASES:
        yield f"q_brute_{w.name}", (lambda w=w: tv.test_prequantized_passthrough_bruteforce(orc, w))
        yield f"zp_{w.name}", (lambda w=w: tv.test_zero_padding_bruteforce(orc, w, True))
        yield f"stats_{w.name}", (lambda w=w: tv.test_cumulative_stats_are_a_histogram(orc, w))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / "oracle_mutant.c"
    cpath.write_text(mutated)
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", *obuild.CFLAGS, str(cpath), obuild.MT_SRC, "-o", str(so), *obuild.LIBS],
                   check=True)
    caught = []
    with oracle.swapped(str(so)):
        for pin, fn in _pins(oracle):
            try:
                with np.errstate(all="ignore"):
                    fn()
            except (AssertionError, ValueError, IndexError) as ex:   # noqa: PERF203
                caught.append(pin)
                break
    assert caught, f"planted mistake '{name}' passed every pin"


def test_unmutated_copy_passes_all_pins(tmp_path):
    so = tmp_path / "liboracle_copy.so"
    shutil.copy(obuild.SRC, tmp_path / "o.c")
    subprocess.run(["gcc", *obuild.CFLAGS, str(tmp_path / "o.c"), obuild.MT_SRC, "-o", str(so),
                    *obuild.LIBS], check=True)
    with oracle.swapped(str(so)):
        for _, fn in _pins(oracle):
            fn()
