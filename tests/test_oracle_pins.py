"""Pins of the CPU oracle to facts outside itself (no GPU).

Each pin is a plain function that raises AssertionError when the oracle is
wrong.  ``test_pins_hold`` runs them against the oracle; ``test_pins_catch``
plants plausible mistakes in the oracle (on the CPU, by monkeypatching its
module) and checks that at least one pin fails for each of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.qmv_oracle as Q
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _hex_words(rows):
    return np.array([[int(h, 16) for h in row] for row in rows], dtype=np.uint32)


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------
def pin_golden_words():
    g = _load("packing.json")
    for case in g["words"]:
        bits = case["bits"]
        word = np.array([[int(case["word"], 16)]], dtype=np.uint32)
        K = 32 // bits
        got = Q.unpack_words(word, bits, K)[0].tolist()
        assert got == case["codes"], (case, got)
        assert Q.pack_words(np.array([case["codes"]]), bits)[0, 0] == int(case["word"], 16)


def pin_golden_t5():
    g = _load("packing.json")
    for case in g["t5_bytes"]:
        # one byte placed first in a gs=64 group: its digits are codes 0..4
        data = np.zeros((1, 13), dtype=np.uint8)
        data[0, 0] = case["byte"]
        got = Q.t5_unpack(data, 64, 64)[0, :5].tolist()
        assert got == case["digits"], (case, got)
    for gs, nbytes in g["t5_group_bytes"].items():
        assert Q.t5_group_bytes(int(gs)) == nbytes


def pin_article_facts():
    # section 二 path 1: 32 one-bit values per uint32 (and 16 two-bit ones)
    assert Q.pack_words(np.ones((1, 32), np.uint8), 1).shape == (1, 1)
    assert Q.pack_words(np.ones((1, 16), np.uint8), 2).shape == (1, 1)
    # section 二 path 3: 13/26 bytes per 64/128 group; ~1.585 bit per weight is
    # log2(3), the information content of a ternary digit; the storage is 1.625
    for gs in (64, 128):
        assert Q.t5_group_bytes(gs) * 8 / gs == pytest.approx(1.625)
    assert math.log2(3) == pytest.approx(1.585, abs=5e-4)
    # section 二 path 3 puts t5's memory about a quarter below 2-bit uint32
    # weights; that holds when t5 stores one fp16 scale per group and 2-bit
    # stores scale + bias:
    for gs, lo, hi in ((64, 0.2, 0.26), (128, 0.2, 0.26)):
        t5 = Q.algorithmic_bytes("t5", 0, 1, 1024 * gs, gs, bias_stored=False)
        u2 = Q.algorithmic_bytes("u2", 0, 1, 1024 * gs, gs, bias_stored=True)
        assert lo < 1 - t5 / u2 < hi
    # the largest valid t5 byte is 3^5 - 1
    assert Q.T5_MAX_BYTE == 3 ** 5 - 1


def pin_golden_qmv_u2():
    g = _load("worked_qmv.json")["u2"]
    K, gs = g["K"], g["group_size"]
    w = _hex_words(g["words"])
    s = np.array(g["scales"], np.float16)
    b = np.array(g["biases"], np.float16)
    x = np.array([[r["first_group"]] * 64 + [r["second_group"]] * 64 for r in g["x_rows"]], np.float16)
    y, _ = Q.qmv_reference("u2", x, w, s, b, K, gs)
    assert y.tolist() == g["y"], y


def pin_golden_qmv_t5():
    g = _load("worked_qmv.json")["t5"]
    data = np.array(g["bytes"], np.uint8)
    s = np.array(g["scales"], np.float16)
    x = np.arange(64, dtype=np.float16)[None, :]
    y, _ = Q.qmv_reference("t5", x, data, s, None, g["K"], g["group_size"])
    assert y.tolist() == g["y"], y


def pin_golden_dequant_rne():
    for case in _load("worked_qmv.json")["dequant_rne"]:
        s = np.array([[int(case["scale_f16"], 16)]], np.uint16).view(np.float16)
        codes = np.full((1, 64), case["q"], np.uint8)
        b = np.array([[case["bias"]]], np.float64)
        got = Q.dequant_f16(codes, s, b, 64)[0, 0].view(np.uint16)
        assert int(got) == int(case["f16"], 16), (case, hex(int(got)))


def pin_roundtrip():
    rng = np.random.default_rng(1)
    for bits in (1, 2):
        c = rng.integers(0, 2 ** bits, size=(5, 256)).astype(np.uint8)
        assert (Q.unpack_words(Q.pack_words(c, bits), bits, 256) == c).all()
    for gs in (64, 128):
        c = rng.integers(0, 3, size=(5, 2 * gs)).astype(np.uint8)
        data = Q.t5_pack(c, gs)
        assert data.shape == (5, 2 * Q.t5_group_bytes(gs))
        assert (Q.t5_unpack(data, 2 * gs, gs) == c).all()
        # padding digits are zero, so the last byte of a group is small
        tail = data.reshape(5, 2, -1)[:, :, -1]
        assert tail.max() < 3 ** (gs - 5 * (Q.t5_group_bytes(gs) - 1))
        assert data.max() <= Q.T5_MAX_BYTE


def pin_scalar_vs_vector():
    rng = np.random.default_rng(2)
    for bits in (1, 2):
        words = synth.draw_words(rng, 3, 128, bits)
        assert Q.unpack_words(words, bits, 128).tolist() == Q.unpack_words_scalar(words, bits, 128)
    for gs in (64, 128):
        data = synth.draw_t5_bytes(rng, 3, 2 * gs, gs)
        assert Q.t5_unpack(data, 2 * gs, gs).tolist() == Q.t5_unpack_scalar(data, 2 * gs, gs)


def _tiny_case(fmt, M, N, K, gs, seed, bias="stored"):
    rng = np.random.default_rng(seed)
    if fmt == "t5":
        codes = rng.integers(0, 3, size=(N, K)).astype(np.uint8)
        w = Q.t5_pack(codes, gs)
    else:
        codes = rng.integers(0, 2 ** Q.bits_of(fmt), size=(N, K)).astype(np.uint8)
        w = Q.pack_words(codes, Q.bits_of(fmt))
    s = synth.draw_scales(rng, N, K // gs)
    b = synth.draw_biases(rng, N, K // gs) if bias == "stored" else None
    x = synth.draw_x(rng, M, K)
    return codes, w, s, b, x


def pin_exact_rational():
    """The fp64 oracle rounds the exact (rational) result, for every format,
    group size, stored and implied biases."""
    for fmt, gs, bias, seed in (("u1", 64, "stored", 3), ("u2", 64, "stored", 4),
                                ("u2", 128, "implied", 5), ("t5", 64, "implied", 6),
                                ("t5", 128, "stored", 7), ("u1", 128, "implied", 8)):
        M, N, K = 2, 3, 2 * gs
        codes, w, s, b, x = _tiny_case(fmt, M, N, K, gs, seed, bias)
        y, mass = Q.qmv_reference(fmt, x, w, s, b, K, gs)
        if b is None:  # implied bias, written out independently of the oracle
            r = {"u1": Fraction(1, 2), "u2": Fraction(3, 2), "t5": Fraction(1)}[fmt]
            bf = [[-Fraction(float(v)) * r for v in row] for row in s]
        else:
            bf = [[Fraction(float(v)) for v in row] for row in b]
        for m in range(M):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    g = k // gs
                    acc += Fraction(float(x[m][k])) * (Fraction(float(s[n][g])) * int(codes[n][k]) + bf[n][g])
                assert abs(Fraction(float(y[m, n])) - acc) <= Fraction(2 * K) * Fraction(2.0 ** -52) * Fraction(float(mass[m, n])) + Fraction(1, 2 ** 60)


def pin_brute_force():
    codes, w, s, b, x = _tiny_case("u2", 3, 4, 128, 64, 9)
    y, _ = Q.qmv_reference("u2", x, w, s, b, 128, 64)
    yb = Q.qmv_brute(x, codes, s, b.astype(np.float64), 64)
    assert np.allclose(y, np.array(yb), rtol=1e-12, atol=1e-12)


def pin_one_hot():
    """x = e_k selects weight column k: y[n] = s[n][k//gs]*q[n][k] + b[n][k//gs]
    exactly (a single nonzero product); checked at group edges."""
    for fmt, gs in (("u1", 64), ("u2", 128), ("t5", 64), ("t5", 128)):
        K = 3 * gs
        codes, w, s, b, _ = _tiny_case(fmt, 1, 5, K, gs, 10)
        for k in (0, gs - 1, gs, 2 * gs + 7, K - 1):
            x = np.zeros((1, K), np.float16)
            x[0, k] = 1.0
            y, _ = Q.qmv_reference(fmt, x, w, s, b, K, gs)
            g = k // gs
            expect = [float(s[n, g]) * int(codes[n, k]) + float(b[n, g]) for n in range(5)]
            assert y[0].tolist() == expect, (fmt, gs, k)


def pin_constant_codes():
    """All codes equal c: y = sum_g (s_g*c + b_g) * X_g with X_g the group sum
    of x; with s = 0, y = sum_g b_g X_g whatever the codes are."""
    gs, K, N = 64, 256, 3
    rng = np.random.default_rng(11)
    x = synth.draw_x(rng, 2, K)
    s = synth.draw_scales(rng, N, K // gs)
    b = synth.draw_biases(rng, N, K // gs)
    X = x.astype(np.float64).reshape(2, K // gs, gs).sum(-1)
    for c in (0, 1, 3):
        w = Q.pack_words(np.full((N, K), c, np.uint8), 2)
        y, _ = Q.qmv_reference("u2", x, w, s, b, K, gs)
        expect = X @ (s.astype(np.float64) * c + b.astype(np.float64)).T
        assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)
    w = Q.pack_words(rng.integers(0, 4, (N, K)).astype(np.uint8), 2)
    y, _ = Q.qmv_reference("u2", x, w, np.zeros_like(s), b, K, gs)
    assert np.allclose(y, X @ b.astype(np.float64).T, rtol=1e-12, atol=1e-12)


def pin_sym_identity():
    """Symmetric variant == affine variant with the explicit bias -s*r (article
    section 二 path 2); exact because the generator trims 2-bit scales."""
    for fmt in ("u1", "u2"):
        inp = synth.make_inputs(fmt, 2, 6, 256, 64, "sym", seed=12)
        r = {"u1": 0.5, "u2": 1.5}[fmt]
        explicit = (-(inp.scales.astype(np.float64)) * r).astype(np.float16)
        assert (explicit.astype(np.float64) == -inp.scales.astype(np.float64) * r).all()
        y_sym, _ = Q.qmv_reference(fmt, inp.x, inp.w, inp.scales, None, 256, 64)
        y_asym, _ = Q.qmv_reference(fmt, inp.x, inp.w, inp.scales, explicit, 256, 64)
        assert (y_sym == y_asym).all()


def pin_t5_equals_u2():
    """t5 codes repacked as 2-bit words give the same product."""
    inp = synth.make_inputs("t5", 3, 7, 384, 128, "t5", seed=13)
    codes = Q.t5_unpack(inp.w, 384, 128)
    words = Q.pack_words(codes, 2)
    bias = (-inp.scales.astype(np.float64)).astype(np.float16)
    y5, _ = Q.qmv_reference("t5", inp.x, inp.w, inp.scales, None, 384, 128)
    y2, _ = Q.qmv_reference("u2", inp.x, words, inp.scales, bias, 384, 128)
    assert np.allclose(y5, y2, rtol=1e-13, atol=1e-13)


def pin_invalid_t5_rejected():
    bad = np.zeros((1, 13), np.uint8)
    bad[0, 3] = 243
    with pytest.raises(ValueError):
        Q.t5_unpack(bad, 64, 64)


def pin_tolerance_rule():
    y_ref = np.array([[1.0, -2.0]])
    mass = np.array([[10.0, 10.0]])
    # bound = 1e-3*10 + 1e-3*|y_ref| = 0.011 and 0.012
    ok, worst = Q.check_close(y_ref + np.array([[0.0109, -0.0119]]), y_ref, mass)
    assert ok and 0.99 < worst < 1.0
    ok, _ = Q.check_close(y_ref + np.array([[0.0112, 0.0]]), y_ref, mass)
    assert not ok
    ok, _ = Q.check_close(y_ref + np.array([[0.0, 0.0122]]), y_ref, mass)
    assert not ok
    ok, _ = Q.check_close(np.array([[np.nan, -2.0]]), y_ref, mass)
    assert not ok


def pin_abs_mass():
    """The bound's scale term is the sum of the element-wise absolute
    products (hand-worked values in tests/golden/abs_mass.json), not the
    absolute sum, not the product of the norms, not a sum with signed x."""
    g = _load("abs_mass.json")
    c = g["plain"]
    x = np.array(c["x"], np.float16)
    W = np.array(c["w"], np.float64)
    assert Q.abs_mass(x, W).tolist() == [[c["mass"]]]
    assert Q.qmv_f64(x, W).tolist() == [[c["y"]]]
    c = g["u2"]
    K, gs = c["K"], c["group_size"]
    codes = np.full((1, K), c["codes_rest"], np.uint8)
    codes[0, :4] = c["codes_head"]
    x = np.zeros((1, K), np.float16)
    x[0, :4] = c["x_head"]
    y, mass = Q.qmv_reference("u2", x, Q.pack_words(codes, 2), np.array([[c["scale"]]], np.float16),
                              np.array([[c["bias"]]], np.float16), K, gs)
    assert y.tolist() == [[c["y"]]] and mass.tolist() == [[c["mass"]]], (y, mass)
    c = g["t5"]
    K, gs = c["K"], c["group_size"]
    x = np.zeros((1, K), np.float16)
    x[0, :6] = c["x_head"]
    y, mass = Q.qmv_reference("t5", x, np.array([c["bytes"]], np.uint8), np.array([[c["scale"]]], np.float16),
                              None, K, gs)
    assert y.tolist() == [[c["y"]]] and mass.tolist() == [[c["mass"]]], (y, mass)
    # invariants: one-hot x gives |w_k|; the mass bounds |y|; it does not see signs
    rng = np.random.default_rng(14)
    W = rng.uniform(-1, 1, (4, 64))
    xr = synth.draw_x(rng, 3, 64)
    m = Q.abs_mass(xr, W)
    assert (m >= np.abs(Q.qmv_f64(xr, W)) - 1e-12).all()
    assert np.array_equal(m, Q.abs_mass(-xr, W)) and np.array_equal(m, Q.abs_mass(xr, -W))
    e = np.zeros((1, 64), np.float16)
    e[0, 9] = 1.0
    assert np.array_equal(Q.abs_mass(e, W)[0], np.abs(W[:, 9]))


PINS = [pin_golden_words, pin_golden_t5, pin_article_facts, pin_golden_qmv_u2, pin_golden_qmv_t5,
        pin_golden_dequant_rne, pin_roundtrip, pin_scalar_vs_vector, pin_exact_rational,
        pin_brute_force, pin_one_hot, pin_constant_codes, pin_sym_identity, pin_t5_equals_u2,
        pin_invalid_t5_rejected, pin_tolerance_rule, pin_abs_mass]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pins_hold(pin):
    pin()


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin.
# ---------------------------------------------------------------------------
def _msb_first_unpack(words, bits, K):
    words = np.asarray(words, dtype=np.uint32)
    k = np.arange(K)
    shift = (32 - bits - (k * bits) % 32).astype(np.uint32)
    return ((words[:, (k * bits) // 32] >> shift) & np.uint32((1 << bits) - 1)).astype(np.uint8)


def _msd_first_t5(data, K, gs):
    data = np.asarray(data, dtype=np.uint8)
    gb = Q.t5_group_bytes(gs)
    k = np.arange(K)
    g, r = divmod(k, gs)
    j, i = divmod(r, 5)
    return ((data[:, g * gb + j].astype(np.int64) // (3 ** (4 - i))) % 3).astype(np.uint8)


def _t5_wrong_group_bytes(gs):
    return gs // 5


def _bias_sign(fmt, scales, biases):
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if biases is None:
        return s * Q.sym_ratio(fmt)
    return -np.asarray(biases, dtype=np.float16).astype(np.float64)


def _wrong_ratio(fmt):
    return 1.0 if fmt == "t5" else float(2 ** Q.bits_of(fmt) - 1)


def _group_off_by_one(codes, scales, biases_f64, gs):
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), gs, axis=1)
    b = np.repeat(np.asarray(biases_f64, dtype=np.float64), gs, axis=1)
    s = np.roll(s, -1, axis=1)
    return s * codes.astype(np.float64) + b


def _transposed(x, W64):
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    Wt = W64.reshape(W64.shape[1], W64.shape[0]) if W64.shape[0] != W64.shape[1] else W64.T
    return x64 @ Wt if Wt.shape[0] == x64.shape[1] else x64 @ W64.T[::-1]


def _drop_bias(codes, scales, biases_f64, gs):
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), gs, axis=1)
    return s * codes.astype(np.float64)


def _f32_dequant(codes, scales, biases_f64, gs):
    return Q.dequant_f64(codes, scales, biases_f64, gs).astype(np.float32).astype(np.float16)


def _half_up_round(codes, scales, biases_f64, gs):
    v = Q.dequant_f64(codes, scales, biases_f64, gs)
    lo = v.astype(np.float16)
    hi = np.nextafter(lo, np.float16(np.inf))
    return np.where(np.abs(hi.astype(np.float64) - v) <= np.abs(v - lo.astype(np.float64)), hi, lo)


def _loose_tolerance(y_ref, mass):
    return 1e-2 * mass + 1e-3 * np.abs(y_ref)


def _mass_of_sum(x, W64):
    return np.abs(Q.qmv_f64(x, W64))


def _mass_product_of_norms(x, W64):
    xa = np.abs(np.asarray(x, dtype=np.float16).astype(np.float64)).sum(axis=1, keepdims=True)
    return xa * np.abs(W64).sum(axis=1)[None, :]


def _mass_signed_x(x, W64):
    return np.asarray(x, dtype=np.float16).astype(np.float64) @ np.abs(W64).T


MUTANTS = {
    "msb_first_words": ("unpack_words", _msb_first_unpack),
    "msd_first_t5": ("t5_unpack", _msd_first_t5),
    "t5_group_bytes": ("t5_group_bytes", _t5_wrong_group_bytes),
    "bias_sign": ("effective_biases", _bias_sign),
    "sym_ratio": ("sym_ratio", _wrong_ratio),
    "group_index": ("dequant_f64", _group_off_by_one),
    "transposed_product": ("qmv_f64", _transposed),
    "dropped_bias": ("dequant_f64", _drop_bias),
    "half_up_rounding": ("dequant_f16", _half_up_round),
    "loose_tolerance": ("tolerance", _loose_tolerance),
    "mass_of_sum": ("abs_mass", _mass_of_sum),
    "mass_product_of_norms": ("abs_mass", _mass_product_of_norms),
    "mass_signed_x": ("abs_mass", _mass_signed_x),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(Q, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (Exception, pytest.fail.Exception):  # any failure counts as detection
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
