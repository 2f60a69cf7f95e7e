"""GPU parity: every entry point of the C ABI against the fp64 oracle.

Tolerance (reading R5): |y - y_ref| <= 1e-3*sum_k|x_k w_k| + 1e-3*|y_ref|.
Dequantized weights and codes are compared bit for bit.  Cross-variant
identities (wide row == single-row call, symmetric == affine with the
explicit bias) are bit-identical by construction of the kernels.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import BITS, assert_close, dev, make, reference, run_entry, to_np, torch_mod

pytestmark = pytest.mark.gpu

# a shape spanning several 1024-code K tiles with a ragged last tile, and a
# row count that is not a multiple of any workgroup's rows
MID = dict(N=333, K=2560)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


# ------------------------------------------------------------------ tiny
def test_tiny_config():
    """M=1, N=512, K=512, 1-bit, gs=64 (the small decode case)."""
    inp = make("u1", 1, 512, 512, 64, "asym", seed=0)
    for entry in ("qmv", "qmv_wide"):
        print(f"tiny {entry}", flush=True)
        assert_close(run_entry(entry, inp), inp, what=entry)


# ------------------------------------------------------------------ uint32 formats
@pytest.mark.parametrize("fmt", ["u1", "u2"])
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5])
def test_wide_asym(fmt, gs, M):
    inp = make(fmt, M, MID["N"], MID["K"], gs, "asym", seed=1)
    print(f"wide {fmt} gs{gs} M{M}", flush=True)
    assert_close(run_entry("qmv_wide", inp), inp, what=f"qmv_wide {fmt} gs{gs} M{M}")


@pytest.mark.parametrize("fmt", ["u1", "u2"])
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M", [1, 3, 5])
def test_sym(fmt, gs, M):
    inp = make(fmt, M, MID["N"], MID["K"], gs, "sym", seed=2)
    print(f"sym {fmt} gs{gs} M{M}", flush=True)
    y = run_entry("qmv_sym", inp)
    assert_close(y, inp, what="qmv_sym")
    # the bias tensor is never read: a NaN-filled one changes nothing
    y_poison = run_entry("qmv_sym", inp, poison_bias=True)
    assert np.array_equal(y, y_poison)
    # bit-identical to the affine kernel with the explicit bias -s*r
    r = oracle.sym_ratio(fmt)
    explicit = (-inp.scales.astype(np.float64) * r).astype(np.float16)
    y_aff = run_entry("qmv_wide", inp, b=dev(explicit))
    assert np.array_equal(y, y_aff)


@pytest.mark.parametrize("fmt", ["u1", "u2", "t5"])
@pytest.mark.parametrize("gs", [64, 128])
def test_wide_rows_equal_single_row_calls(fmt, gs):
    """Row m of a wide call is bit-identical to M separate M=1 calls, and to
    the per-row entry point with all M rows."""
    torch = torch_mod()
    inp = make(fmt, 5, MID["N"], MID["K"], gs, seed=3)
    wide = "t5_qmv_wide" if fmt == "t5" else "qmv_wide"
    per_row = "t5_qmv" if fmt == "t5" else "qmv"
    y = run_entry(wide, inp)
    y_rows = run_entry(per_row, inp)
    assert np.array_equal(y, y_rows)
    xd = dev(inp.x)
    for m in range(5):
        one = make(fmt, 1, MID["N"], MID["K"], gs, seed=3)
        one.x = inp.x[m:m + 1].copy()
        one.w, one.scales, one.biases = inp.w, inp.scales, inp.biases
        ym = run_entry(wide, one, x=xd[m:m + 1].contiguous())
        assert np.array_equal(y[m], ym[0]), f"row {m}"
    del torch


@pytest.mark.parametrize("fmt", ["u1", "u2"])
def test_per_row_entry_any_m(fmt):
    inp = make(fmt, 7, 130, 1024, 64, "asym", seed=4)
    assert_close(run_entry("qmv", inp), inp, what="qmv M=7")


# ------------------------------------------------------------------ t5
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5])
def test_t5_wide(gs, M):
    inp = make("t5", M, MID["N"], MID["K"], gs, "t5", seed=5)
    print(f"t5 wide gs{gs} M{M}", flush=True)
    assert_close(run_entry("t5_qmv_wide", inp), inp, what=f"t5_qmv_wide gs{gs} M{M}")


@pytest.mark.parametrize("gs", [64, 128])
def test_t5_explicit_bias(gs):
    inp = make("t5", 3, MID["N"], MID["K"], gs, "asym", seed=6)
    assert_close(run_entry("t5_qmv_wide", inp), inp, what="t5 asym wide")
    assert_close(run_entry("t5_qmv", inp), inp, what="t5 asym per-row")


@pytest.mark.parametrize("gs", [64, 128])
def test_t5_equals_2bit(gs):
    """The same codes (in {0,1,2}) as t5 bytes and as 2-bit words, with the
    same scales and bias -scale, give the same product (within tolerance)."""
    inp = make("t5", 4, MID["N"], MID["K"], gs, "t5", seed=7)
    codes = oracle.t5_unpack(inp.w, inp.K, gs)
    words = oracle.pack_words(codes, 2)
    bias = (-inp.scales.astype(np.float64)).astype(np.float16)
    y5 = run_entry("t5_qmv_wide", inp)
    u2 = make("u2", 4, MID["N"], MID["K"], gs, "asym", seed=7)
    u2.x, u2.w, u2.scales, u2.biases = inp.x, words, inp.scales, bias
    y2 = run_entry("qmv_wide", u2)
    y_ref, mass = reference(inp)
    ok, worst = oracle.check_close(y5, y2, mass)
    assert ok, worst


# ------------------------------------------------------------------ edges
@pytest.mark.parametrize("fmt,gs,K", [("u1", 64, 64), ("u2", 64, 64), ("u2", 128, 128),
                                      ("u1", 128, 128), ("t5", 64, 256), ("t5", 128, 256)])
@pytest.mark.parametrize("N", [1, 17])
def test_minimum_sizes(fmt, gs, K, N):
    for M in (1, 5):
        inp = make(fmt, M, N, K, gs, seed=8)
        entry = "t5_qmv_wide" if fmt == "t5" else "qmv_wide"
        assert_close(run_entry(entry, inp), inp, what=f"{fmt} N{N} K{K} M{M}")


def test_one_hot_columns_exact():
    """x = e_k returns fp16(s*q + b) of column k exactly (one product)."""
    inp = make("u2", 1, 200, 1024, 64, "asym", seed=9)
    codes = oracle.unpack_words(inp.w, 2, 1024)
    for k in (0, 63, 64, 511, 1023):
        x = np.zeros((1, 1024), np.float16)
        x[0, k] = 1.0
        inp.x = x
        y = run_entry("qmv_wide", inp)
        g = k // 64
        expect = (inp.scales[:, g].astype(np.float64) * codes[:, k] + inp.biases[:, g].astype(np.float64)).astype(np.float16)
        assert np.array_equal(y[0].astype(np.float16), expect), k


def test_repeat_is_deterministic():
    inp = make("t5", 5, 1000, 5120, 128, seed=10)
    ys = [run_entry("t5_qmv_wide", inp) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[1], ys[2])


# ------------------------------------------------------------------ full sizes, sampled rows
def _sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(N, 48), replace=False).tolist())
    rows.update({0, 1, N - 2, N - 1})
    return np.array(sorted(rows))


@pytest.mark.parametrize("shape", list(synth.PROJECTION_SHAPES))
@pytest.mark.parametrize("fmt,gs,M", [("u2", 64, 1), ("u1", 128, 1), ("u2", 128, 5), ("t5", 128, 1),
                                      ("t5", 64, 4)])
def test_full_size_sampled(shape, fmt, gs, M):
    N, K = synth.PROJECTION_SHAPES[shape]
    inp = make(fmt, M, N, K, gs, seed=11)
    entry = "t5_qmv_wide" if fmt == "t5" else "qmv_wide"
    print(f"full {shape} {fmt} gs{gs} M{M}", flush=True)
    y = run_entry(entry, inp)
    assert np.all(np.isfinite(y))
    assert_close(y, inp, rows=_sample_rows(N, 12), what=f"{shape} {fmt}")


def test_full_size_sym_2bit_gate_m5():
    N, K = synth.PROJECTION_SHAPES["gate"]
    inp = make("u2", 5, N, K, 64, "sym", seed=13)
    y = run_entry("qmv_sym", inp)
    assert_close(y, inp, rows=_sample_rows(N, 14), what="gate sym M5")


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("fmt", ["u1", "u2", "t5"])
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("bias", ["stored", "implied"])
def test_dequant_bit_exact(fmt, gs, bias):
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    variant = "asym" if bias == "stored" else ("t5" if fmt == "t5" else "sym")
    inp = make(fmt, 1, 300, 2560 if fmt != "t5" else 2560, gs, variant, seed=15)
    out = bq.dequant(dev(inp.w), dev(inp.scales), dev(inp.biases), BITS[fmt], gs, inp.K)
    torch.cuda.synchronize()
    codes = oracle.codes_of(fmt, inp.w, inp.K, gs)
    expect = oracle.dequant_f16(codes, inp.scales, oracle.effective_biases(fmt, inp.scales, inp.biases), gs)
    got = to_np(out)
    assert np.array_equal(got.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("fmt", ["u1", "u2", "t5"])
def test_codes_bit_exact(fmt):
    """With scale 1 and bias 0 the dequantized weights are the codes."""
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    inp = make(fmt, 1, 257, 1024, 64, "asym", seed=16)
    ones = np.ones_like(inp.scales)
    zeros = np.zeros_like(inp.scales)
    out = bq.dequant(dev(inp.w), dev(ones), dev(zeros), BITS[fmt], 64, inp.K)
    torch.cuda.synchronize()
    codes = oracle.codes_of(fmt, inp.w, inp.K, 64)
    assert np.array_equal(to_np(out).astype(np.int64), codes.astype(np.int64))


def test_dequant_rounding_ties():
    """Exact ties of scale*q + bias round to even (e.g. 3*fp16(0.1))."""
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    N, K = 64, 256
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 4, size=(N, K)).astype(np.uint8)
    w = oracle.pack_words(codes, 2)
    s = np.full((N, K // 64), 0.1, np.float16)
    b = rng.uniform(-1, 1, size=(N, K // 64)).astype(np.float16)
    b[:, 0] = 0
    out = bq.dequant(dev(w), dev(s), dev(b), 2, 64, K)
    torch.cuda.synchronize()
    expect = oracle.dequant_f16(codes, s, b.astype(np.float64), 64)
    assert np.array_equal(to_np(out).view(np.uint16), expect.view(np.uint16))


# ------------------------------------------------------------------ t5 qmm (prefill)
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,N,K", [(17, 200, 512), (32, 333, 2560), (130, 129, 1024), (1, 40, 256)])
def test_t5_qmm(gs, M, N, K):
    inp = make("t5", M, N, K, gs, "t5", seed=18)
    print(f"qmm gs{gs} M{M} N{N} K{K}", flush=True)
    assert_close(run_entry("t5_qmm", inp), inp, what=f"t5_qmm gs{gs} M{M}")


def test_t5_qmm_explicit_bias():
    inp = make("t5", 48, 160, 1024, 128, "asym", seed=19)
    assert_close(run_entry("t5_qmm", inp), inp, what="t5_qmm asym")


def test_t5_qmm_matches_wide():
    inp = make("t5", 5, MID["N"], MID["K"], 128, "t5", seed=20)
    y_mm = run_entry("t5_qmm", inp)
    y_mv = run_entry("t5_qmv_wide", inp)
    _, mass = reference(inp)
    ok, worst = oracle.check_close(y_mm, y_mv, mass)
    assert ok, worst


# Shapes for which the tile choice takes each route above 32 rows: 32 x 64
# and 64 x 64 tiles with four steps per iteration and x one iteration ahead
# (40 x 4096, 80 x 8192), 64 x 64 tiles two iterations ahead (40 and 50 rows
# of wide N; 50 x 1000 with 6 K steps, no multiple of four), 128 x 64 tiles
# two iterations ahead (the rest; 100 x 200 with 2 K steps, as many
# iterations as the prefetch depth); ragged row and column counts; checked
# on sampled output columns.
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,N,K", [(20, 65536, 256), (40, 4096, 256), (80, 8192, 256), (40, 17408, 256),
                                   (50, 65536, 256), (50, 1000, 384), (80, 17408, 256), (100, 65536, 256),
                                   (100, 200, 128), (160, 12288, 256), (600, 17408, 1024)])
def test_t5_qmm_tile_shapes(gs, M, N, K):
    inp = make("t5", M, N, K, gs, "t5", seed=23)
    print(f"qmm tiles gs{gs} M{M} N{N} K{K}", flush=True)
    y = run_entry("t5_qmm", inp)
    assert np.all(np.isfinite(y))
    assert_close(y, inp, rows=_sample_rows(N, 24), what=f"t5_qmm tiles gs{gs} M{M}")


def test_t5_qmm_tile_shapes_explicit_bias():
    inp = make("t5", 300, 16384, 512, 64, "asym", seed=25)
    y = run_entry("t5_qmm", inp)
    assert_close(y, inp, rows=_sample_rows(16384, 26), what="t5_qmm tiles asym")


# With one-hot activation rows every output is a single fp16 weight times
# 1.0, accumulated alone in fp32: exact.  Reading back all N x K weights this
# way checks every code, every K step and every tile of the fused product bit
# for bit, with enough tiles that two workgroups share a CU (512 and more).
@pytest.mark.parametrize("M,N,K,gs,variant", [(20, 65536, 256, 64, "t5"), (20, 65536, 256, 128, "t5"),
                                              (100, 65536, 256, 64, "t5"), (32, 65536, 512, 64, "asym"),
                                              (300, 16384, 512, 128, "t5"), (600, 17408, 768, 64, "t5"),
                                              # several K steps per pipeline iteration: 32 x 64 tiles
                                              # (4 steps), 64 x 64 tiles in one round (4 steps)
                                              (32, 1024, 1024, 128, "t5"), (24, 2048, 512, 64, "asym"),
                                              (64, 4096, 768, 64, "t5"), (48, 2048, 1024, 128, "asym"),
                                              # iteration counts that are not whole rounds of the
                                              # small-M prefetch (10 and 7 steps)
                                              (32, 2048, 640, 64, "t5"), (16, 1024, 448, 64, "asym"),
                                              # a single K step: fewer iterations than the
                                              # prefetch depth of 128 x 64 tiles
                                              (100, 200, 64, 64, "t5")])
def test_t5_qmm_one_hot_rows_read_exact_weights(M, N, K, gs, variant):
    import bit_quantized_decode_qmv_amd as bq
    inp = make("t5", M, N, K, gs, variant, seed=31)
    codes = oracle.codes_of("t5", inp.w, K, gs)
    W16 = oracle.dequant_f16(codes, inp.scales, oracle.effective_biases("t5", inp.scales, inp.biases), gs)
    wd, sd, bd = dev(inp.w), dev(inp.scales), dev(inp.biases)
    print(f"qmm one-hot gs{gs} M{M} N{N} K{K} {variant}", flush=True)
    for base in range(0, K, M):
        ks = np.arange(base, min(base + M, K))
        x = np.zeros((M, K), np.float16)
        x[np.arange(len(ks)), ks] = 1.0
        y = to_np(bq.t5_qmm(dev(x), wd, sd, gs, biases=bd))
        want = W16[:, ks].T
        bad = np.argwhere(y[:len(ks)] != want)
        assert len(bad) == 0, (f"K columns {base}..{base + len(ks) - 1}: {len(bad)} weights differ, e.g. "
                               + ", ".join(f"W[{n}][{ks[m]}] {y[m, n]!r} != {want[m, n]!r}" for m, n in bad[:6]))
        assert not y[len(ks):].any()


# Products with at most 32 rows request x and weight bytes four iterations
# ahead and walk K in whole rounds of four iterations.  K step counts of 10,
# 7 and 21 (K 640, 448, 1344) give iteration counts that are not whole
# rounds (one or two steps per iteration), including fewer than four.
@pytest.mark.parametrize("M,N,K,gs", [(32, 1000, 640, 64), (32, 1000, 640, 128), (20, 515, 448, 64),
                                      (9, 4100, 1344, 64), (32, 300, 128, 128)])
@pytest.mark.parametrize("variant", ["t5", "asym"])
def test_t5_qmm_small_m_partial_rounds(M, N, K, gs, variant):
    inp = make("t5", M, N, K, gs, variant, seed=33)
    print(f"qmm small-M rounds gs{gs} M{M} N{N} K{K} {variant}", flush=True)
    y = run_entry("t5_qmm", inp)
    assert np.all(np.isfinite(y))
    assert_close(y, inp, what=f"t5_qmm small M gs{gs} M{M} K{K} {variant}")


@pytest.mark.parametrize("shape", ["gate", "down"])
@pytest.mark.parametrize("M", [32, 512, 2048])
def test_t5_qmm_full_size_sampled(shape, M):
    """The prefill configurations the benchmark times (gs 128, gate and
    down, M 32 / 512 / 2048), checked on sampled output columns."""
    N, K = synth.PROJECTION_SHAPES[shape]
    inp = make("t5", M, N, K, 128, "t5", seed=21)
    print(f"qmm full {shape} M{M}", flush=True)
    y = run_entry("t5_qmm", inp)
    assert np.all(np.isfinite(y))
    assert_close(y, inp, rows=_sample_rows(N, 22), what=f"qmm {shape}")
