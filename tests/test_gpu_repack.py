"""GPU parity of bq_t5_repack (1/2-bit code words -> t5 bytes) against the
oracle's t5 packing, bit for bit, and of the repacked layer's products."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import BITS, assert_close, dev, make, run_entry, to_np, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


def _ternary_codes(N, K, gs, bits, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 3 if bits == 2 else 2, size=(N, K)).astype(np.uint8)


def _repack(words, bits, gs, K):
    import bit_quantized_decode_qmv_amd as bq
    out, ternary = bq.t5_repack(dev(words), bits, gs, K)
    return to_np(out), ternary


@pytest.mark.parametrize("bits", [1, 2])
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("N,K", [(1, 256), (333, 2560), (64, 5120)])
def test_repack_bit_exact(bits, gs, N, K):
    codes = _ternary_codes(N, K, gs, bits, seed=40 + N)
    words = oracle.pack_words(codes, bits)
    print(f"repack u{bits} gs{gs} N{N} K{K}", flush=True)
    got, ternary = _repack(words, bits, gs, K)
    assert ternary
    assert np.array_equal(got, oracle.t5_pack(codes, gs))
    assert np.array_equal(oracle.t5_unpack(got, K, gs), codes)


@pytest.mark.parametrize("gs", [64, 128])
def test_repack_flags_code_3(gs):
    N, K = 50, 1024
    codes = _ternary_codes(N, K, gs, 2, seed=50)
    codes[7, 0] = 3
    codes[49, K - 1] = 3
    codes[20, 300] = 3
    got, ternary = _repack(oracle.pack_words(codes, 2), 2, gs, K)
    assert not ternary
    # code 3 becomes digit 2; every byte stays a valid t5 byte
    assert np.array_equal(got, oracle.t5_pack(np.minimum(codes, 2), gs))


def test_repack_single_code_3_anywhere_is_seen():
    N, K, gs = 3, 256, 64
    for pos in (0, 31, 32, 255):
        codes = np.zeros((N, K), np.uint8)
        codes[2, pos] = 3
        _, ternary = _repack(oracle.pack_words(codes, 2), 2, gs, K)
        assert not ternary, pos


def test_repack_full_size_sampled_rows():
    N, K = synth.PROJECTION_SHAPES["gate"]
    gs = 128
    codes = _ternary_codes(N, K, gs, 2, seed=51)
    got, ternary = _repack(oracle.pack_words(codes, 2), 2, gs, K)
    assert ternary
    rows = np.array(sorted({0, 1, N // 2, N - 2, N - 1} | set(np.random.default_rng(52).choice(N, 40).tolist())))
    assert np.array_equal(got[rows], oracle.t5_pack(codes[rows], gs))


@pytest.mark.parametrize("gs", [64, 128])
def test_repacked_layer_products(gs):
    """A 2-bit layer with ternary codes and bias -scale, repacked: the t5
    layer drops the biases (implied -scale) and its products match the
    oracle; with other biases they are kept."""
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    M, N, K = 3, 333, 2560
    inp = make("u2", M, N, K, gs, "asym", seed=53)
    codes = _ternary_codes(N, K, gs, 2, seed=54)
    inp.w = oracle.pack_words(codes, 2)
    inp.biases = (-inp.scales.astype(np.float64)).astype(np.float16)  # exact
    qw = bq.QuantizedWeight(dev(inp.w), dev(inp.scales), dev(inp.biases), 2, gs)
    q5 = qw.to_t5()
    assert q5.bits == bq.BITS_T5 and q5.biases is None
    xd = dev(inp.x)
    y5 = to_np(bq.linear(xd, q5)).astype(np.float64)
    assert_close(y5, inp, what="repacked t5, implied bias")
    y2 = run_entry("qmv_wide", inp)
    assert_close(y2, inp, what="2-bit source layer")
    # biases that are not -scale stay with the layer
    inp.biases = make("u2", M, N, K, gs, "asym", seed=55).biases
    qw = bq.QuantizedWeight(dev(inp.w), dev(inp.scales), dev(inp.biases), 2, gs)
    q5 = qw.to_t5()
    assert q5.biases is not None
    y5 = to_np(bq.linear(xd, q5)).astype(np.float64)
    assert_close(y5, inp, what="repacked t5, stored bias")
    del torch


def test_to_t5_refuses_code_3():
    import bit_quantized_decode_qmv_amd as bq
    N, K, gs = 4, 256, 64
    codes = np.full((N, K), 3, np.uint8)
    s = np.full((N, K // gs), 0.01, np.float16)
    qw = bq.QuantizedWeight(dev(oracle.pack_words(codes, 2)), dev(s), dev(-s), 2, gs)
    with pytest.raises(ValueError, match="code 3"):
        qw.to_t5()
