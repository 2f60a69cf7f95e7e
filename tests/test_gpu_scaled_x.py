"""GPU parity at every activation scale.

The decode kernels stage x in fp16 scaled by a per-chunk power of two; the
result must stay within the acceptance bound, |y - y_ref| <= 1e-3 *
sum_k |x_k w_k| + 1e-3 * |y_ref|, whatever the magnitude of x: rows of
N(0,1) scaled by 2^-8 .. 2^-16 (at 2^-16 every value is an fp16
subnormal), constant-sign rows of about 1.8e-4, rows spanning 2^24 in
magnitude, and large rows (2^8).  Scaling a row by a power of two that
keeps it normal scales the output by exactly that power.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import assert_close, dev, make, run_entry, torch_mod

pytestmark = pytest.mark.gpu

MID = dict(N=333, K=2560)
KINDS = ("n2m8", "n2m12", "n2m14", "n2m16", "const_sign", "wide_range", "n2p8")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


def scaled_rows(kind, M, K, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, K))
    if kind.startswith("n2m"):
        return (z * 2.0 ** -int(kind[3:])).astype(np.float16)
    if kind == "n2p8":
        return (z * 2.0 ** 8).astype(np.float16)
    if kind == "const_sign":
        return (np.abs(z) * 1.8e-4).astype(np.float16)
    if kind == "wide_range":
        return (z * np.exp2(-rng.uniform(0, 24, size=(M, K)))).astype(np.float16)
    raise ValueError(kind)


def entry_of(fmt):
    return "t5_qmv_wide" if fmt == "t5" else "qmv_wide"


@pytest.mark.parametrize("fmt,gs", [("u1", 64), ("u1", 128), ("u2", 64), ("u2", 128), ("t5", 64), ("t5", 128)])
@pytest.mark.parametrize("M", [1, 5])
def test_scaled_rows_mid(fmt, gs, M):
    inp = make(fmt, M, MID["N"], MID["K"], gs, seed=51)
    for i, kind in enumerate(KINDS):
        inp.x = scaled_rows(kind, M, inp.K, 52 + i)
        print(f"scaled {fmt} gs{gs} M{M} {kind}", flush=True)
        assert_close(run_entry(entry_of(fmt), inp), inp, what=f"{fmt} gs{gs} M{M} {kind}")


@pytest.mark.parametrize("fmt,gs", [("u1", 64), ("u2", 64), ("u2", 128), ("t5", 64), ("t5", 128)])
@pytest.mark.parametrize("shape", ["gate", "down"])
def test_scaled_rows_full_size(fmt, gs, shape):
    N, K = synth.PROJECTION_SHAPES[shape]
    inp = make(fmt, 5, N, K, gs, seed=53)
    rng = np.random.default_rng(54)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 96, replace=False)]))
    for M in (1, 5):
        for i, kind in enumerate(("n2m12", "n2m16", "const_sign", "wide_range")):
            inp.x = scaled_rows(kind, M, K, 55 + i)
            print(f"scaled full {shape} {fmt} gs{gs} M{M} {kind}", flush=True)
            assert_close(run_entry(entry_of(fmt), inp), inp, rows=rows, what=f"{shape} {fmt} M{M} {kind}")


@pytest.mark.parametrize("fmt,gs", [("u1", 64), ("u2", 128), ("t5", 64), ("t5", 128)])
def test_power_of_two_scaling_is_exact(fmt, gs):
    """y(x * 2^-j) * 2^j == y(x) bit for bit while x * 2^-j stays normal and
    the output stays a normal fp16 number (bias 0, so that the bias term
    scales too)."""
    inp = make(fmt, 3, MID["N"], MID["K"], gs, seed=56)
    if inp.biases is not None:
        inp.biases = np.zeros_like(inp.biases)
    rng = np.random.default_rng(57)
    inp.x = (rng.choice([-1.0, 1.0], size=(3, inp.K)) *
             np.exp2(rng.uniform(-2, 2, size=(3, inp.K)))).astype(np.float16)
    y0 = run_entry(entry_of(fmt), inp)
    for j in (1, 5, 10):
        xs = (inp.x.astype(np.float64) * 2.0 ** -j).astype(np.float16)
        yj = run_entry(entry_of(fmt), inp, x=dev(xs))
        big = np.abs(y0) >= 2.0 ** (-14 + j)  # y0 * 2^-j still normal in fp16
        assert np.array_equal((yj * 2.0 ** j)[big], y0[big]), j
