"""CPU emulation of the decode kernels' activation staging (no GPU).

The decode kernels multiply each packed code in place: a code masked inside
a 16-bit half at bit offset e reads as the fp16 subnormal q * 2^(e-24), and
the activation it meets is staged in fp16 as x * 2^(c-e), where c is a
power-of-two exponent chosen per 64-code chunk of x.  Every fp16 x fp16
product is exact in fp32, so the only rounding the staging adds is the fp16
rounding of x * 2^(c-e).  This module emulates that rounding in numpy (the
products and sums in fp64) and checks the result against the oracle's
acceptance rule, |y - y_ref| <= 1e-3 * sum_k |x_k w_k| + 1e-3 * |y_ref|, for
activation rows of every magnitude the fp16 input can hold.

The chunk exponent: with E the fp16 exponent field of the chunk's largest
|x|, c = min(29 - E, 15), which puts that value in [2^14, 2^15) (or scales
the chunk by 2^15 when it is smaller than 1/2); a fixed c = 0 is the rule
that fails for small activations, and the test checks that it does, so
that the emulation is known to see the problem.
"""
import numpy as np
import pytest

import oracle
import synth

KS = (5120, 17408)


def code_offsets(fmt, K, gs):
    """Bit offset e of every code inside its 16-bit half, and the 64-code
    chunk it is staged in (t5 128-groups: halves of 65 and 63 codes)."""
    k = np.arange(K)
    if fmt == "u2":
        j = k % 16
        p = j & 7
        e = 2 * np.where(p < 5, p, p - 5)
        chunk = k // 64
    elif fmt == "u1":
        j = k % 32
        p = j & 15
        e = np.where(p < 10, p, p - 10)
        chunk = k // 64
    else:
        r = k % gs
        e = 2 * (r % 5) if gs == 64 else 2 * (np.where(r >= 65, r - 65, r) % 5)
        chunk = (k // gs) * (gs // 64) + ((r >= 65) if gs == 128 else 0)
    return e.astype(np.int64), chunk.astype(np.int64)


def chunk_exponent(x16, chunk, rule):
    """Per (row, chunk) exponent c; rule 'fixed' = 0, 'chunk' = the kernels'."""
    M = x16.shape[0]
    nch = int(chunk.max()) + 1
    if rule == "fixed":
        return np.zeros((M, nch), np.int64)
    mag = (x16.view(np.uint16) & 0x7FFF).astype(np.int64)
    amax = np.zeros((M, nch), np.int64)
    for m in range(M):
        np.maximum.at(amax[m], chunk, mag[m])
    E = amax >> 10
    return np.minimum(29 - E, 15)


def staged_product(fmt, x16, w, scales, biases, K, gs, rule):
    """y as the kernels form it, with the staging rounding emulated exactly
    (fp16 rounding of x*2^(c-e)) and everything else in fp64."""
    e, chunk = code_offsets(fmt, K, gs)
    c = chunk_exponent(x16, chunk, rule)  # [M][nch]
    ce = c[:, chunk] - e[None, :]          # [M][K]
    x64 = x16.astype(np.float64)
    staged = (x64 * np.exp2(ce)).astype(np.float16).astype(np.float64)
    x_eff = staged * np.exp2(-ce)          # what the products see
    codes = oracle.codes_of(fmt, w, K, gs).astype(np.float64)
    s = np.repeat(scales.astype(np.float64), gs, axis=1)
    b = np.repeat(oracle.effective_biases(fmt, scales, biases), gs, axis=1)
    # products: s*q against the staged x, the bias against the exact x sum
    return x_eff @ (s * codes).T + x64 @ b.T


def rows_of(kind, rng, M, K):
    z = rng.standard_normal((M, K))
    if kind.startswith("normal"):
        j = int(kind.split("_")[1])
        return (z * 2.0 ** -j).astype(np.float16)
    if kind == "constant_sign":
        return (np.abs(z) * 1.8e-4).astype(np.float16)
    if kind == "wide_range":
        return (z * np.exp2(-rng.uniform(0, 24, size=(M, K)))).astype(np.float16)
    raise ValueError(kind)


KINDS = ("normal_0", "normal_8", "normal_12", "normal_14", "normal_16", "constant_sign", "wide_range")


@pytest.mark.parametrize("fmt,gs", [("u1", 64), ("u2", 64), ("u2", 128), ("t5", 64), ("t5", 128)])
@pytest.mark.parametrize("K", KS)
def test_chunk_exponent_staging_within_tolerance(fmt, gs, K):
    rng = np.random.default_rng(K + gs)
    variant = "t5" if fmt == "t5" else "asym"
    inp = synth.make_inputs(fmt, 1, 48, K, gs, variant, seed=41)
    for kind in KINDS:
        x = rows_of(kind, rng, 3, K)
        y = staged_product(fmt, x, inp.w, inp.scales, inp.biases, K, gs, "chunk")
        y_ref, mass = oracle.qmv_reference(fmt, x, inp.w, inp.scales, inp.biases, K, gs)
        ok, worst = oracle.check_close(y, y_ref, mass)
        assert ok, f"{fmt} gs{gs} K{K} {kind}: worst err/tol {worst:.3g}"
        # the staging error itself stays far below the bound
        assert worst < 0.05, f"{fmt} gs{gs} K{K} {kind}: worst err/tol {worst:.3g}"


@pytest.mark.parametrize("fmt,gs", [("u1", 64), ("u2", 64), ("t5", 128)])
def test_fixed_exponent_staging_fails_small_rows(fmt, gs):
    """The emulation sees the problem a fixed exponent has: rows of fp16
    activations near 2^-16 break the bound."""
    K = 5120
    rng = np.random.default_rng(3)
    variant = "t5" if fmt == "t5" else "asym"
    inp = synth.make_inputs(fmt, 1, 48, K, gs, variant, seed=42)
    x = rows_of("normal_16", rng, 3, K)
    y = staged_product(fmt, x, inp.w, inp.scales, inp.biases, K, gs, "fixed")
    y_ref, mass = oracle.qmv_reference(fmt, x, inp.w, inp.scales, inp.biases, K, gs)
    ok, worst = oracle.check_close(y, y_ref, mass)
    assert not ok and worst > 1.5, worst


def test_chunk_exponent_scale_invariant():
    """Scaling a row by a power of two (within the fp16 normal range) scales
    the emulated result by exactly that power."""
    K, gs = 5120, 64
    rng = np.random.default_rng(5)
    inp = synth.make_inputs("u2", 1, 16, K, gs, "asym", seed=43)
    # magnitudes in [2^-4, 4): every x * 2^-j below stays a normal fp16 number
    x = (rng.choice([-1.0, 1.0], size=(2, K)) * np.exp2(rng.uniform(-4, 2, size=(2, K)))).astype(np.float16)
    y0 = staged_product("u2", x, inp.w, inp.scales, np.zeros_like(inp.biases), K, gs, "chunk")
    for j in (1, 4, 9):
        xs = (x.astype(np.float64) * 2.0 ** -j).astype(np.float16)
        assert np.array_equal(xs.astype(np.float64) * 2.0 ** j, x.astype(np.float64))
        yj = staged_product("u2", xs, inp.w, inp.scales, np.zeros_like(inp.biases), K, gs, "chunk")
        assert np.array_equal(yj * 2.0 ** j, y0), j
