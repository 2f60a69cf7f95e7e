"""GPU parity through the C ABI with pointers that are only 4-byte aligned,
and t5 rows that are not whole dwords.

The boundary requires 4-byte alignment of W and of the decode calls' x,
scales and biases, and 2-byte alignment of fp16 outputs; every decode entry
point is called here with each of its arrays 4 bytes past a 256-byte
boundary (y also 2 bytes past), with scale arrays whose byte size is not a
multiple of 4, and compared with the fp64 oracle.  t5 weights are checked
for K a multiple of the group size only (rows of 65 and 78 bytes) on the
decode, prefill and dequant entries.
"""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import BITS, make, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


class Placed:
    """A device copy of a numpy array starting `off` bytes past a 256-byte
    boundary (the allocation is padded so the array fits)."""

    def __init__(self, a, off):
        torch = torch_mod()
        raw = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
        self.buf = torch.zeros(raw.size + 512, dtype=torch.uint8, device="cuda:0")
        base = self.buf.data_ptr()
        self.start = (-base) % 256 + off
        self.buf[self.start:self.start + raw.size] = torch.from_numpy(raw.copy()).to("cuda:0")
        self.ptr = base + self.start
        self.nbytes = raw.size

    def read(self, dtype, shape):
        torch = torch_mod()
        torch.cuda.synchronize()
        return self.buf[self.start:self.start + self.nbytes].cpu().numpy().view(dtype).reshape(shape)


def run_placed(entry, inp, offs, y_off=4):
    """Calls the C entry point with every array at its offset; returns y."""
    import bit_quantized_decode_qmv_amd as bq
    lib = bq.load_library()
    M, N, K, gs = inp.M, inp.N, inp.K, inp.group_size
    x = Placed(inp.x, offs)
    w = Placed(inp.w, offs)
    s = Placed(inp.scales, offs)
    b = Placed(inp.biases, offs) if inp.biases is not None else None
    y = Placed(np.zeros((M, N), np.float16), y_off)
    st = getattr(lib, "bq_" + entry)(x.ptr, w.ptr, s.ptr, b.ptr if b is not None else None, y.ptr, M, N, K,
                                     BITS[inp.fmt], gs, ctypes.c_void_p(torch_mod().cuda.current_stream().cuda_stream))
    assert st == 0, (entry, st)
    return y.read(np.float16, (M, N)).astype(np.float64)


def check(y, inp, what):
    y_ref, mass = oracle.qmv_reference(inp.fmt, inp.x, inp.w, inp.scales, inp.biases, inp.K, inp.group_size)
    ok, worst = oracle.check_close(y, y_ref, mass)
    assert ok, f"{what}: worst err/tol {worst:.3g}"


DECODE = [("qmv", "u2", "asym"), ("qmv_wide", "u1", "asym"), ("qmv_wide", "u2", "asym"), ("qmv_sym", "u2", "sym"),
          ("qmv_sym", "u1", "sym"), ("t5_qmv", "t5", "t5"), ("t5_qmv_wide", "t5", "t5"), ("t5_qmv_wide", "t5", "asym")]


@pytest.mark.parametrize("entry,fmt,variant", DECODE)
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("N,K", [(333, 2560), (77, 640)])
@pytest.mark.parametrize("M", [1, 3, 5])
def test_decode_four_byte_offsets(entry, fmt, variant, gs, N, K, M):
    inp = make(fmt, M, N, K, gs, variant, seed=71)
    print(f"align {entry} {fmt} {variant} gs{gs} N{N} K{K} M{M}", flush=True)
    for offs, y_off in ((4, 4), (12, 2), (8, 6)):
        check(run_placed(entry, inp, offs, y_off), inp, f"{entry} {fmt} gs{gs} offsets {offs}/{y_off}")


@pytest.mark.parametrize("gs,K", [(64, 320), (64, 448), (128, 384), (128, 640)])
@pytest.mark.parametrize("M", [1, 2, 5])
@pytest.mark.parametrize("variant", ["t5", "asym"])
def test_t5_rows_not_whole_dwords_decode(gs, K, M, variant):
    for N in (1, 7, 333):
        inp = make("t5", M, N, K, gs, variant, seed=72)
        print(f"t5 rows gs{gs} K{K} M{M} N{N} {variant}", flush=True)
        check(run_placed("t5_qmv_wide", inp, 4, 2), inp, f"t5 gs{gs} K{K} N{N} M{M}")
        check(run_placed("t5_qmv", inp, 0, 0), inp, f"t5 per-row gs{gs} K{K} N{N} M{M}")


@pytest.mark.parametrize("gs,K", [(64, 320), (128, 384)])
@pytest.mark.parametrize("M,N", [(20, 200), (40, 8192), (17, 129)])
def test_t5_rows_not_whole_dwords_qmm(gs, K, M, N):
    inp = make("t5", M, N, K, gs, "t5", seed=73)
    print(f"t5 qmm rows gs{gs} K{K} M{M} N{N}", flush=True)
    check(run_placed("t5_qmm", inp, 0, 2), inp, f"t5_qmm gs{gs} K{K} M{M}")


@pytest.mark.parametrize("fmt,gs,K", [("u1", 64, 640), ("u2", 128, 640), ("t5", 64, 320), ("t5", 128, 384),
                                      ("t5", 64, 1024)])
@pytest.mark.parametrize("bias", ["stored", "implied"])
@pytest.mark.parametrize("y_off", [0, 2, 4])
def test_dequant_any_output_alignment(fmt, gs, K, bias, y_off):
    import bit_quantized_decode_qmv_amd as bq
    lib = bq.load_library()
    N = 37
    variant = "asym" if bias == "stored" else ("t5" if fmt == "t5" else "sym")
    inp = make(fmt, 1, N, K, gs, variant, seed=74)
    w = Placed(inp.w, 4)
    s = Placed(inp.scales, 2)
    b = Placed(inp.biases, 2) if inp.biases is not None else None
    y = Placed(np.zeros((N, K), np.float16), y_off)
    st = lib.bq_dequant(None, w.ptr, s.ptr, b.ptr if b is not None else None, y.ptr, 0, N, K, BITS[fmt], gs,
                        ctypes.c_void_p(torch_mod().cuda.current_stream().cuda_stream))
    assert st == 0, st
    got = y.read(np.float16, (N, K))
    codes = oracle.codes_of(fmt, inp.w, K, gs)
    expect = oracle.dequant_f16(codes, inp.scales, oracle.effective_biases(fmt, inp.scales, inp.biases), gs)
    assert np.array_equal(got.view(np.uint16), expect.view(np.uint16))
