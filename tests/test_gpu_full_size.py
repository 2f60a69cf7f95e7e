"""GPU parity of the decode calls at the full projection sizes.

Every (format, group size, bias kind) of the decode workloads on all seven
projection shapes of a hidden=5120 decoder, for every M = 1..5: the same
kernel instances the benchmark times (their rows per unit and prefetch
depth depend on the shape and M).  Checked against the fp64 oracle on about
512 sampled rows per shape -- at least one per workgroup (the sampling
stride is below every workgroup's row count) plus the first and last rows
-- with the acceptance rule |y - y_ref| <= 1e-3*sum_k|x_k w_k| +
1e-3*|y_ref|.  Row m of every wide call is also compared bit for bit with a
single-row call on that row (no sum of the kernels depends on M).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import BITS, dev, make, to_np, torch_mod

pytestmark = pytest.mark.gpu

CELLS = [(fmt, gs, variant) for fmt in ("u1", "u2") for gs in (64, 128) for variant in ("asym", "sym")] + \
        [("t5", gs, "t5") for gs in (64, 128)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


def sample_rows(N, seed, per=512):
    """About `per` rows: one at a random offset in each window of N // per
    rows (N // per is at most half of any workgroup's rows), plus the
    first two and last two rows."""
    rng = np.random.default_rng(seed)
    step = max(1, N // per)
    starts = np.arange(0, N, step)
    rows = starts + rng.integers(0, step, size=len(starts))
    rows = rows[rows < N]
    return np.unique(np.concatenate([rows, [0, 1, N - 2, N - 1]]))


def call(fmt, variant, xd, wd, sd, bd, gs):
    import bit_quantized_decode_qmv_amd as bq
    if fmt == "t5":
        return bq.t5_qmv_wide(xd, wd, sd, gs)
    if variant == "sym":
        return bq.qmv_sym(xd, wd, sd, BITS[fmt], gs)
    return bq.qmv_wide(xd, wd, sd, bd, BITS[fmt], gs)


@pytest.mark.parametrize("shape", list(synth.PROJECTION_SHAPES))
@pytest.mark.parametrize("fmt,gs,variant", CELLS, ids=lambda c: str(c))
def test_full_size_every_m(fmt, gs, variant, shape):
    torch = torch_mod()
    N, K = synth.PROJECTION_SHAPES[shape]
    inp = make(fmt, 5, N, K, gs, variant, seed=61)
    rows = sample_rows(N, 62)
    y_ref, mass = oracle.qmv_reference(fmt, inp.x, inp.w, inp.scales, inp.biases, K, gs, rows)
    xd, wd, sd, bd = dev(inp.x), dev(inp.w), dev(inp.scales), dev(inp.biases)
    single = []
    for m in range(5):
        y1 = call(fmt, variant, xd[m:m + 1].contiguous(), wd, sd, bd, gs)
        single.append(to_np(y1)[0])
    for M in range(1, 6):
        print(f"full {shape} {fmt} gs{gs} {variant} M{M}", flush=True)
        y = to_np(call(fmt, variant, xd[:M].contiguous(), wd, sd, bd, gs)).astype(np.float64)
        torch.cuda.synchronize()
        assert np.all(np.isfinite(y))
        ok, worst = oracle.check_close(y[:, rows], y_ref[:M], mass[:M])
        assert ok, f"{shape} {fmt} gs{gs} {variant} M{M}: worst err/tol {worst:.3g}"
        for m in range(M):
            assert np.array_equal(y[m].astype(np.float16), single[m]), f"M{M} row {m} != single-row call"


@pytest.mark.parametrize("fmt,gs,variant", [("t5", 64, "t5"), ("t5", 128, "t5"), ("u2", 64, "asym"), ("u2", 128, "sym")],
                         ids=lambda c: str(c))
@pytest.mark.parametrize("M", [3, 5])
def test_long_shape_ragged_rows(fmt, gs, variant, M):
    """A gate-like shape three rows short of a multiple of four (17405 x
    5120): the 12-wave instances (4-row units for t5 at M >= 3, 2-row units
    for 2-bit) with a last workgroup of 65 rows, so its last row-group is
    partial.  Sampled rows plus the last 12, against the oracle, and every
    row bit for bit against single-row calls."""
    N, K = 17405, 5120
    inp = make(fmt, M, N, K, gs, variant, seed=63)
    rows = np.unique(np.concatenate([sample_rows(N, 64), np.arange(N - 12, N)]))
    y_ref, mass = oracle.qmv_reference(fmt, inp.x, inp.w, inp.scales, inp.biases, K, gs, rows)
    xd, wd, sd, bd = dev(inp.x), dev(inp.w), dev(inp.scales), dev(inp.biases)
    print(f"ragged {fmt} gs{gs} {variant} M{M} N{N}", flush=True)
    y = to_np(call(fmt, variant, xd, wd, sd, bd, gs)).astype(np.float64)
    assert np.all(np.isfinite(y))
    ok, worst = oracle.check_close(y[:, rows], y_ref, mass)
    assert ok, f"ragged {fmt} gs{gs} {variant} M{M}: worst err/tol {worst:.3g}"
    for m in range(M):
        y1 = to_np(call(fmt, variant, xd[m:m + 1].contiguous(), wd, sd, bd, gs))[0]
        assert np.array_equal(y[m].astype(np.float16), y1), f"M{M} row {m} != single-row call"
