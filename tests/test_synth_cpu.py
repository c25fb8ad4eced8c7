"""The seeded input recipe: what each draw produces and that the workloads
have the shapes, seeds and offsets they are described with."""
import numpy as np

import synth


def test_uniform_is_exact_multiples_of_2_pow_minus_23_in_the_half_open_interval():
    x = synth.uniform_pm1(synth.rng(1), 1 << 20)
    assert x.dtype == np.float32
    assert float(x.min()) >= -1.0 and float(x.max()) < 1.0
    k = x.astype(np.float64) * (1 << 23)
    assert np.array_equal(k, np.round(k))                 # exact multiples of 2^-23
    assert not np.any(np.signbit(x) & (x == 0))           # no -0.0
    assert not np.any((x != 0) & (np.abs(x) < np.finfo(np.float32).tiny))   # no subnormals


def test_draws_are_reproducible_and_seed_dependent():
    a = synth.make_inputs("add_f32", 4096, 7)
    b = synth.make_inputs("add_f32", 4096, 7)
    c = synth.make_inputs("add_f32", 4096, 8)
    assert np.array_equal(a["a"], b["a"]) and np.array_equal(a["b"], b["b"])
    assert not np.array_equal(a["a"], c["a"])
    assert not np.array_equal(a["a"], a["b"])            # A drawn before B, one generator


def test_normal_and_absnormal():
    g1, g2 = synth.rng(3), synth.rng(3)
    x = synth.normal01(g1, 1 << 16)
    y = synth.absnormal(g2, 1 << 16)
    assert x.dtype == np.float32 and abs(float(x.mean())) < 0.02
    assert np.array_equal(y.view(np.uint32), x.view(np.uint32) & 0x7FFFFFFF)


def test_16_bit_inputs_are_rne_casts_of_the_fp32_draw():
    u = synth.uniform_pm1(synth.rng(104), 1 << 12)
    f16 = synth.make_inputs("add_f16", 1 << 12, 104)["a"]
    assert f16.dtype == np.uint16
    assert np.array_equal(f16, u.astype(np.float16).view(np.uint16))
    bf = synth.make_inputs("add_bf16", 1 << 12, 104)["a"]
    # bfloat16 keeps the top 16 bits after RNE: widening back is within half an ulp
    back = (bf.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back.astype(np.float64) - u) <= np.abs(u) * 2.0 ** -8 + 1e-45)


def test_workloads_match_their_descriptions():
    w = synth.WORKLOADS
    assert w["cfg1_add_f32_2e20"].n == 1 << 20
    assert w["cfg2_add_f32_2e28p3_offA1"].n == (1 << 28) + 3
    assert w["cfg2_add_f32_2e28p3_offA1"].offsets == {"a": 1}
    assert w["cfg3_saxpy_f32_32M"].n == 1 << 25 and w["cfg3_saxpy_f32_32M"].alpha == 2.5
    assert w["cfg5b_gather_f32_2e26_s2"].stride == 2
    for name, wl in w.items():
        assert wl.name == name and wl.description
        assert wl.op in synth.OP_INPUTS
        if wl.op == "copy2d_f32":
            sr, sc, base, off = wl.view
            rows = wl.n // wl.cols
            assert rows * wl.cols == wl.n
            hi = off + max(0, (rows - 1) * sr) + max(0, (wl.cols - 1) * sc)
            assert hi < base                               # the view stays inside its base
        if wl.op == "bias_relu_f32":
            assert wl.n % wl.cols == 0
