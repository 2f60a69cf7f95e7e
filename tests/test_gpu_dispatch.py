"""GPU tests of the dispatcher (bq_linear) and of the symmetric-bias check
(bq_sym_check), through the C ABI.

Routing follows the "oMLX Bonsai 自定义内核" article, section 二 (kernels
chosen by bits and the number of rows M; t5 prefill with M > 16 on the fused
product) and section 三 (1/2-bit layers in decode on the fast kernels); the
symmetric variant applies when bias = -scale * ratio holds (section 二 path
2).  Every result is checked against the fp64 oracle with the tolerance
rule, and against the entry point the route names, bit for bit.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, dev, make, to_np

pytestmark = pytest.mark.gpu

N, K = 333, 2560


def _bq():
    import torch

    import bit_quantized_decode_qmv_amd as bq
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bq.load_library()
    return bq, torch


def _qw(bq, inp, biases="stored"):
    b = dev(inp.biases) if biases == "stored" else biases
    return bq.QuantizedWeight(dev(inp.w), dev(inp.scales), b, {"u1": 1, "u2": 2, "t5": 0}[inp.fmt],
                              inp.group_size)


@pytest.mark.parametrize("fmt,gs", [("u2", 64), ("u1", 128)])
@pytest.mark.parametrize("M", [1, 5, 7, 12])
def test_linear_affine_matches_oracle_and_wide_passes(fmt, gs, M):
    bq, torch = _bq()
    inp = make(fmt, M, N, K, gs, "asym")
    qw = _qw(bq, inp)
    assert qw.sym is False  # random biases
    x = dev(inp.x)
    y = to_np(bq.linear(x, qw)).astype(np.float64)
    torch.cuda.synchronize()
    assert_close(y, inp, what=f"linear {fmt} gs{gs} M{M}")
    # the same bits as the wide kernel on each pass of five rows
    for m0 in range(0, M, 5):
        yp = to_np(bq.qmv_wide(x[m0:m0 + 5].contiguous(), qw.w, qw.scales, qw.biases, qw.bits, gs))
        assert np.array_equal(y[m0:m0 + 5].astype(np.float16).view(np.uint16), yp.view(np.uint16))


@pytest.mark.parametrize("fmt", ["u1", "u2"])
@pytest.mark.parametrize("M", [3, 9])
def test_linear_sym_route_and_check(fmt, M):
    bq, torch = _bq()
    inp = make(fmt, M, N, K, 64, "sym")
    r = oracle.sym_ratio(fmt)
    explicit = (-inp.scales.astype(np.float64) * r).astype(np.float16)
    qw = _qw(bq, inp, biases=dev(explicit))
    assert qw.sym is True  # every bias is -scale * ratio exactly
    x = dev(inp.x)
    y_sym = to_np(bq.linear(x, qw))
    y_aff = to_np(bq.linear(x, qw, sym=False))
    torch.cuda.synchronize()
    # the symmetric route skips the bias read and gives the same bits
    assert np.array_equal(y_sym.view(np.uint16), y_aff.view(np.uint16))
    assert_close(y_sym.astype(np.float64), inp, what=f"linear sym {fmt} M{M}")
    # and without any bias tensor the layer is symmetric by definition
    qn = _qw(bq, inp, biases=None)
    assert qn.sym is True
    assert np.array_equal(to_np(bq.linear(x, qn)).view(np.uint16), y_sym.view(np.uint16))


def test_sym_check_rejects_near_misses():
    bq, torch = _bq()
    inp = make("u2", 1, N, K, 64, "sym")
    s = dev(inp.scales)
    exact = (-inp.scales.astype(np.float64) * 1.5).astype(np.float16)
    assert bq.sym_check(s, dev(exact), 2, 64) is True
    # the ratio belongs to the bit width: 1-bit's 0.5 does not match
    assert bq.sym_check(s, dev(exact), 1, 64) is False
    # one bias one fp16 step away
    off = exact.copy()
    off.view(np.uint16)[N // 2, 7] += 1
    assert bq.sym_check(s, dev(off), 2, 64) is False
    # a NaN bias, and a NaN scale
    nan_b = exact.copy()
    nan_b[N - 1, -1] = np.float16(np.nan)
    assert bq.sym_check(s, dev(nan_b), 2, 64) is False
    nan_s = inp.scales.copy()
    nan_s[0, 0] = np.float16(np.nan)
    assert bq.sym_check(dev(nan_s), dev(exact), 2, 64) is False
    # random affine biases
    a = make("u2", 1, N, K, 64, "asym")
    assert bq.sym_check(dev(a.scales), dev(a.biases), 2, 64) is False
    # t5: bias = -scale
    t = make("t5", 1, N, K, 64)
    assert bq.sym_check(dev(t.scales), dev((-t.scales.astype(np.float64)).astype(np.float16)), 0, 64) is True


def test_sym_check_untrimmed_scales_are_not_symmetric_for_2bit():
    # -1.5*s is not an fp16 value for most untrimmed scales: its rounding is
    # not the implied bias, and the check must say so
    bq, torch = _bq()
    inp = make("u2", 1, N, K, 64, "asym")
    rounded = (-inp.scales.astype(np.float64) * 1.5).astype(np.float16)
    assert bq.sym_check(dev(inp.scales), dev(rounded), 2, 64) is False


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M", [4, 16, 17, 37])
def test_linear_t5_routes(gs, M):
    bq, torch = _bq()
    inp = make("t5", M, N, K, gs)
    qw = _qw(bq, inp, biases=None)
    x = dev(inp.x)
    y = to_np(bq.linear(x, qw))
    torch.cuda.synchronize()
    assert_close(y.astype(np.float64), inp, what=f"linear t5 gs{gs} M{M}")
    route, passes = bq.bq_linear_route(M, N, bq.BITS_T5)
    if route == "t5_qmm":
        ref = to_np(bq.t5_qmm(x, qw.w, qw.scales, gs))
        assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))
    else:
        for m0 in range(0, M, 5):
            yp = to_np(bq.t5_qmv_wide(x[m0:m0 + 5].contiguous(), qw.w, qw.scales, gs))
            assert np.array_equal(y[m0:m0 + 5].view(np.uint16), yp.view(np.uint16))


def test_linear_t5_stored_bias_and_sym_flag():
    bq, torch = _bq()
    inp = make("t5", 6, N, K, 64, "asym")  # general affine t5: biases stored and read
    qw = _qw(bq, inp)
    assert qw.sym is False
    y = to_np(bq.linear(dev(inp.x), qw)).astype(np.float64)
    torch.cuda.synchronize()
    assert_close(y, inp, what="linear t5 stored bias")
    # forcing the flag implies -scale and ignores the stored biases
    ys = to_np(bq.linear(dev(inp.x), qw, sym=True))
    yn = to_np(bq.linear(dev(inp.x), _qw(bq, inp, biases=None)))
    assert np.array_equal(ys.view(np.uint16), yn.view(np.uint16))


@pytest.mark.parametrize("fmt,gs", [("u2", 64), ("u1", 128)])
@pytest.mark.parametrize("M,NN", [(17, 8192), (16, 8192), (40, 5120), (64, 17408)])
def test_linear_1_2_bit_prefill_routes(fmt, gs, M, NN):
    """From 17 rows with enough tiles bq_linear takes the fused product and
    gives its bits; otherwise five-row wide passes."""
    bq, torch = _bq()
    inp = make(fmt, M, NN, 1024, gs, "asym", seed=101)
    bits = 1 if fmt == "u1" else 2
    qw = _qw(bq, inp)
    qw._sym = False  # the affine route (the random biases are not symmetric)
    x = dev(inp.x)
    y = to_np(bq.linear(x, qw))
    torch.cuda.synchronize()
    assert_close(y.astype(np.float64), inp, rows=None if NN <= 2048 else np.arange(0, NN, 97),
                 what=f"linear {fmt} M{M} N{NN}")
    route, passes = bq.bq_linear_route(M, NN, bits)
    if route == "qmm":
        ref = to_np(bq.qmm(x, qw.w, qw.scales, bits, gs, biases=qw.biases))
    else:
        ref = np.concatenate([to_np(bq.qmv_wide(x[m0:m0 + 5].contiguous(), qw.w, qw.scales, qw.biases, bits, gs))
                              for m0 in range(0, M, 5)])
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16)), route


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,NN", [(17, 8192), (16, 8192), (17, 5120), (40, 5120), (17, 4032), (23, 1024),
                                  (24, 1024)])
def test_linear_t5_prefill_routes(gs, M, NN):
    """t5 from 17 rows takes the fused product when it has 64 tiles of
    32 x 64 (17 x 8192, 17 x 5120, 40 x 5120), or 16 tiles from 24 rows
    (24 x 1024), and gives its bits; otherwise (16 rows, 17 x 4032 with 63
    tiles, 23 x 1024) five-row wide passes."""
    bq, torch = _bq()
    inp = make("t5", M, NN, 1024, gs, seed=102)
    qw = _qw(bq, inp, biases=None)
    x = dev(inp.x)
    y = to_np(bq.linear(x, qw))
    torch.cuda.synchronize()
    assert_close(y.astype(np.float64), inp, rows=np.arange(0, NN, 97), what=f"linear t5 M{M} N{NN}")
    route, passes = bq.bq_linear_route(M, NN, bq.BITS_T5)
    tiles = (NN + 63) // 64 * ((M + 31) // 32)
    expect = "t5_qmm" if M >= 17 and (tiles >= 64 or (M >= 24 and tiles >= 16)) else "t5_qmv_wide"
    assert route == expect
    if route == "t5_qmm":
        ref = to_np(bq.t5_qmm(x, qw.w, qw.scales, gs))
    else:
        ref = np.concatenate([to_np(bq.t5_qmv_wide(x[m0:m0 + 5].contiguous(), qw.w, qw.scales, gs))
                              for m0 in range(0, M, 5)])
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16)), route


# With a workspace (bq_linear_ws) the fused product takes every call from
# the prefill row count on, whatever its tile count (its K split keeps few
# tiles fast): 1024 columns are 16 tiles, which bq_linear sends to passes.
@pytest.mark.parametrize("fmt,variant,sym", [("t5", "t5", False), ("u2", "asym", False), ("u1", "sym", True)])
@pytest.mark.parametrize("M", [5, 16, 17, 32])
def test_linear_ws_routes(fmt, variant, sym, M):
    bq, torch = _bq()
    NN, KK, gs = 1024, 2560, 64
    inp = make(fmt, M, NN, KK, gs, variant)
    qw = _qw(bq, inp)
    x = dev(inp.x)
    bits = {"u1": 1, "u2": 2, "t5": 0}[fmt]
    need = bq.bq_qmm_workspace(M, NN, KK, bits, gs)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    y = to_np(bq.linear(x, qw, sym=sym, workspace=ws))
    torch.cuda.synchronize()
    assert_close(y.astype(np.float64), inp, what=f"linear_ws {fmt} M{M}")
    prefill = M >= (bq.T5_QMM_MIN_M if fmt == "t5" else bq.QMM_MIN_M)
    if prefill:
        b = None if sym else qw.biases
        want = (bq.t5_qmm_ws(x, qw.w, qw.scales, gs, biases=b, workspace=ws) if fmt == "t5"
                else bq.qmm_ws(x, qw.w, qw.scales, bits, gs, biases=b, workspace=ws))
    else:
        want = bq.linear(x, qw, sym=sym)
    assert np.array_equal(y.view(np.uint16), to_np(want).view(np.uint16))
    # no workspace: exactly bq_linear
    y0 = to_np(bq.linear(x, qw, sym=sym))
    yn = torch.empty((M, NN), dtype=torch.float16, device="cuda:0")
    bq.bq_linear_ws(x.data_ptr(), qw.w.data_ptr(), qw.scales.data_ptr(),
                    qw.biases.data_ptr() if qw.biases is not None else None, yn.data_ptr(), M, NN, KK, bits, gs,
                    bq.LINEAR_SYM if sym else 0, None, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(yn).view(np.uint16), y0.view(np.uint16))
    # the binding's own workspace gives the same bits
    ya = to_np(bq.linear(x, qw, sym=sym, workspace="auto"))
    assert np.array_equal(ya.view(np.uint16), y.view(np.uint16))
