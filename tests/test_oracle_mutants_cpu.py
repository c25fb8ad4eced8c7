"""The pins catch plausible mistakes in the oracle: each case below copies
oracle/oracle.c with one deliberate slip (a wrong rounding tie rule, an
unfused SAXPY, a ReLU that keeps -0, a gather index that wraps at 2^64, an
approximate square root, an abs that rewrites NaN payloads, an add-scalar
that rounds alpha to bfloat16 first, a bfloat16 narrowing that does not
quiet NaNs, a binary16 overflow threshold at 65504, a widening that keeps
signalling NaNs, a bias indexed by row, a view that ignores negative
strides), builds it with the oracle's own flags, points the oracle at the
copy and runs the pins that should notice: every one must fail.  The real
oracle is restored afterwards.  CPU only; nothing here touches a GPU."""
import os
import subprocess

import pytest

import oracle
from oracle import build as oracle_build
from tests import test_oracle as pins

MUTANTS = {
    "ties_round_up": (
        "if (rem > half || (rem == half && (q & 1u))) q += 1u;",
        "if (rem >= half) q += 1u;",
        [pins.test_f16_rounding_closed_forms, pins.test_add_f16_exact_rational]),
    "saxpy_unfused": (
        "for (size_t i = 0; i < n; ++i) y[i] = fmaf(alpha, x[i], y[i]);",
        "for (size_t i = 0; i < n; ++i) y[i] = alpha * x[i] + y[i];",
        [pins.test_saxpy_is_fused_not_two_roundings, pins.test_saxpy_exact_rational]),
    "relu_keeps_negative_zero": (
        "        if (v > 0.0f)      y[i] = v;",
        "        if (v >= 0.0f)     y[i] = v;",
        [pins.test_relu_vs_numpy_maximum]),
    "gather_index_wraps_at_2_64": (
        "unsigned __int128 p = (unsigned __int128)stride * (unsigned __int128)i;",
        "unsigned __int128 p = (unsigned __int128)(stride * i);",
        [pins.test_gather_large_index_products_exact]),
    "sqrt_not_correctly_rounded": (
        "for (size_t i = 0; i < n; ++i) y[i] = sqrtf(x[i]);",
        "for (size_t i = 0; i < n; ++i) y[i] = 1.0f / (1.0f / sqrtf(x[i]));",
        [pins.test_sqrt_f32_vs_numpy_and_exact_root]),
    "abs_rewrites_nan_payloads": (
        "for (size_t i = 0; i < n; ++i) d[i] = s[i] & 0x7fffffffu;",
        "for (size_t i = 0; i < n; ++i) d[i] = (s[i] & 0x7fffffffu) > 0x7f800000u ? "
        "0x7fc00000u : (s[i] & 0x7fffffffu);",
        [pins.test_abs_vs_library_and_bit_identity]),
    "add_scalar_rounds_alpha_first": (
        "y[i] = oracle_f32_to_bf16(oracle_bf16_to_f32(x[i]) + alpha);",
        "y[i] = oracle_f32_to_bf16(oracle_bf16_to_f32(x[i]) + "
        "oracle_bf16_to_f32(oracle_f32_to_bf16(alpha)));",
        [lambda: pins.test_scalar_maps16_vs_library_and_exact_rational("bf16")]),
    # (moving the threshold by one ulp is no mistake: at exactly 65520 the
    # normal path's rounding carries into the exponent and also gives inf)
    "f16_overflow_threshold_at_65504": (
        "if (a >= 0x477ff000u) {",
        "if (a >= 0x477fe000u) {",
        [pins.test_add_f16_overflow_threshold, pins.test_f16_rounding_closed_forms]),
    "f16_widening_keeps_signalling_nans": (
        "        if (m != 0) out |= 0x00400000u;",
        "",
        [pins.test_f16_widen_all_patterns]),
    "bias_indexed_by_row": (
        "y[r * cols + c] = relu1(x[r * cols + c] + bias[c]);",
        "y[r * cols + c] = relu1(x[r * cols + c] + bias[r % cols]);",
        [pins.test_bias_relu_vs_numpy_broadcast]),
    "view_ignores_negative_strides": (
        "d[r * cols + c] = s[(int64_t)r * stride_r + (int64_t)c * stride_c];",
        "d[r * cols + c] = s[(int64_t)r * (stride_r < 0 ? -stride_r : stride_r) + "
        "(int64_t)c * (stride_c < 0 ? -stride_c : stride_c)];",
        [pins.test_copy2d_vs_numpy_strided_views]),
    "bf16_nan_not_quieted": (
        "return (uint16_t)((u >> 16) | 0x0040u);",
        "return (uint16_t)(u >> 16);",
        [pins.test_f32_to_bf16_structured_sweep_vs_torch]),
}


@pytest.fixture
def swap_oracle():
    """Point the oracle package at another library; restore it afterwards."""
    real = oracle._LIB_PATH

    def use(path):
        oracle._lib = None
        oracle._LIB_PATH = path
        oracle._load()
    yield use
    oracle._lib = None
    oracle._LIB_PATH = real
    oracle._load()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, tmp_path, swap_oracle):
    old, new, catchers = MUTANTS[name]
    src = open(oracle_build.SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {old}"
    mutant = tmp_path / f"oracle_{name}.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / f"liboracle_{name}.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-o", str(lib), str(mutant), "-lm"], check=True)
    swap_oracle(str(lib))
    for pin in catchers:
        with pytest.raises(AssertionError):
            pin()


def test_the_real_oracle_passes_the_same_pins(swap_oracle):
    """Control: the unmutated source, built the same way, passes them all."""
    swap_oracle(oracle_build.LIB)
    for _, _, catchers in MUTANTS.values():
        for pin in catchers:
            pin()
