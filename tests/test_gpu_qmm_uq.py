"""GPU parity of bq_qmm, the fused 1/2-bit prefill product, against the fp64
oracle, and a bit-exact readout of every weight it uses."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, dev, make, run_entry, to_np, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


def _sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(N, 40), replace=False).tolist())
    rows.update({0, N - 1})
    return np.array(sorted(rows))


# shapes that reach every route of the tile choice, ragged M and N: 32-row
# tiles (M <= 32); 32 x 64 and 64 x 64 tiles with four steps per iteration
# (130 x 129, 80 x 8192); 64 x 64 tiles two iterations ahead (40 x 17408;
# 50 x 1000 with 6 K steps); 128 x 64 (100 and 160 rows; 100 x 200 with 2 K
# steps), 256 x 64 (300 x 8000) and 256 x 128 tiles (600 and 520 rows), two
# iterations ahead
@pytest.mark.parametrize("fmt", ["u1", "u2"])
@pytest.mark.parametrize("variant", ["asym", "sym"])
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,N,K", [(1, 40, 256), (17, 200, 512), (20, 65536, 256), (40, 17408, 256),
                                   (50, 1000, 384), (80, 8192, 256), (130, 129, 1024), (100, 65536, 256),
                                   (100, 200, 128), (160, 12288, 256), (300, 8000, 512), (520, 130, 384),
                                   (600, 17408, 1024)])
def test_qmm_parity(fmt, variant, gs, M, N, K):
    inp = make(fmt, M, N, K, gs, variant, seed=90)
    print(f"qmm {fmt} {variant} gs{gs} M{M} N{N} K{K}", flush=True)
    y = run_entry("qmm", inp)
    assert np.all(np.isfinite(y))
    rows = None if N <= 2048 else _sample_rows(N, 91)
    assert_close(y, inp, rows=rows, what=f"qmm {fmt} {variant} gs{gs} M{M}")


# small-M products (at most 32 rows) walk K in whole rounds of four
# iterations: step counts of 10, 7 and 21 leave partial rounds
@pytest.mark.parametrize("fmt,gs,variant,M,N,K", [("u2", 64, "asym", 32, 1000, 640), ("u1", 128, "sym", 32, 1000, 640),
                                                  ("u2", 64, "sym", 20, 515, 448), ("u1", 64, "asym", 9, 4100, 1344)])
def test_qmm_small_m_partial_rounds(fmt, gs, variant, M, N, K):
    inp = make(fmt, M, N, K, gs, variant, seed=93)
    print(f"qmm small-M rounds {fmt} {variant} gs{gs} M{M} N{N} K{K}", flush=True)
    y = run_entry("qmm", inp)
    assert np.all(np.isfinite(y))
    assert_close(y, inp, what=f"qmm small M {fmt} {variant} gs{gs} M{M} K{K}")


# one-hot activation rows read every weight back exactly (one product each)
@pytest.mark.parametrize("fmt,gs,variant,M,N,K", [("u2", 64, "asym", 20, 65536, 256), ("u1", 128, "sym", 20, 65536, 256),
                                                  ("u2", 128, "sym", 100, 65536, 256), ("u1", 64, "asym", 32, 65536, 512),
                                                  ("u2", 64, "sym", 300, 16384, 512),
                                                  # 256 x 64 and 256 x 128 tiles
                                                  ("u1", 128, "sym", 300, 4096, 512), ("u2", 64, "asym", 520, 2048, 768),
                                                  # a single K step (fewer iterations than the prefetch depth)
                                                  ("u2", 64, "asym", 100, 200, 64), ("u1", 64, "sym", 600, 130, 64),
                                                  # several K steps per pipeline iteration (32 x 64, 64 x 64)
                                                  ("u2", 128, "asym", 32, 1024, 1024), ("u1", 64, "sym", 24, 2048, 512),
                                                  ("u2", 64, "asym", 64, 4096, 768), ("u1", 128, "asym", 48, 2048, 1024)])
def test_qmm_one_hot_rows_read_exact_weights(fmt, gs, variant, M, N, K):
    import bit_quantized_decode_qmv_amd as bq
    inp = make(fmt, M, N, K, gs, variant, seed=92)
    codes = oracle.codes_of(fmt, inp.w, K, gs)
    W16 = oracle.dequant_f16(codes, inp.scales, oracle.effective_biases(fmt, inp.scales, inp.biases), gs)
    wd, sd, bd = dev(inp.w), dev(inp.scales), dev(inp.biases)
    bits = 1 if fmt == "u1" else 2
    print(f"qmm one-hot {fmt} gs{gs} {variant} M{M} N{N} K{K}", flush=True)
    for base in range(0, K, M):
        ks = np.arange(base, min(base + M, K))
        x = np.zeros((M, K), np.float16)
        x[np.arange(len(ks)), ks] = 1.0
        y = to_np(bq.qmm(dev(x), wd, sd, bits, gs, biases=bd))
        want = W16[:, ks].T
        bad = np.argwhere(y[:len(ks)] != want)
        assert len(bad) == 0, (f"K columns {base}..{base + len(ks) - 1}: {len(bad)} weights differ, e.g. "
                               + ", ".join(f"W[{n}][{ks[m]}] {y[m, n]!r} != {want[m, n]!r}" for m, n in bad[:6]))
        assert not y[len(ks):].any()


@pytest.mark.parametrize("shape", ["gate", "down"])
@pytest.mark.parametrize("fmt", ["u1", "u2"])
@pytest.mark.parametrize("M", [32, 64, 2048])
def test_qmm_full_size_sampled(shape, fmt, M):
    N, K = synth.PROJECTION_SHAPES[shape]
    inp = make(fmt, M, N, K, 128, "asym", seed=93)
    print(f"qmm full {shape} {fmt} M{M}", flush=True)
    y = run_entry("qmm", inp)
    assert np.all(np.isfinite(y))
    assert_close(y, inp, rows=_sample_rows(N, 94), what=f"qmm {shape} {fmt}")


def test_qmm_rows_match_wide():
    """The fused product and five-row wide passes agree within the tolerance
    (different accumulation orders, same weights)."""
    inp = make("u2", 5, 333, 2560, 64, "asym", seed=95)
    y_mm = run_entry("qmm", inp)
    y_w = run_entry("qmv_wide", inp)
    y_ref, mass = oracle.qmv_reference("u2", inp.x, inp.w, inp.scales, inp.biases, inp.K, inp.group_size)
    ok, worst = oracle.check_close(y_mm, y_w, mass)
    assert ok, worst
