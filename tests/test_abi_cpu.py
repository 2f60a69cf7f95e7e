"""The C ABI library loads and exports what include/bq.h declares, and every
entry point rejects invalid arguments with its documented status before it
touches the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import bit_quantized_decode_qmv_amd as bq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bq.h")

OK, NULL, BITS, GROUP, SHAPE, MRANGE, ALIGN = 0, -1, -2, -3, -4, -5, -6
HIP_ERR = -7

# The calls below pass fake device addresses and must all be refused by
# argument validation.  On a machine with a GPU a call that got past
# validation would launch a kernel on those addresses, so there these tests
# do not run at all.
GPU_PRESENT = os.path.exists("/dev/kfd")


class _NoLaunch:
    """The library, with every entry point checked not to have reached a
    launch: without a GPU a launch returns BQ_ERR_HIP."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        fn = getattr(self._lib, name)
        if not name.startswith("bq_") or name in ("bq_abi_version", "bq_strerror", "bq_linear_route",
                                                  "bq_spec_verify_workspace", "bq_qmm_workspace"):
            return fn

        def checked(*args):
            st = fn(*args)
            assert st != HIP_ERR, f"{name}{args} passed validation and tried to launch"
            return st
        return checked


@pytest.fixture(scope="module")
def lib():
    if GPU_PRESENT:
        pytest.skip("fake-pointer validation tests run only on machines without a GPU")
    if not os.path.exists(bq.LIB_PATH):
        pytest.fail("libbq.so is not built: run __graft_entry__.build() first")
    return _NoLaunch(bq.load_library())


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|int)\s+(bq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(bq.ALL_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.bq_abi_version() == bq.ABI_VERSION == 10


def test_strerror_covers_every_status(lib):
    msgs = {s: bq.strerror(s) for s in range(-9, 1)}
    assert len(set(msgs.values())) == 10
    assert bq.strerror(-99) == "unknown bq status"


def test_abi_mismatch_is_an_error(tmp_path, monkeypatch):
    monkeypatch.setattr(bq, "ABI_VERSION", 999)
    with pytest.raises(ImportError, match="ABI version"):
        bq.load_library(bq.LIB_PATH)


def test_missing_library_is_an_error(tmp_path):
    with pytest.raises(ImportError, match="not built"):
        bq.load_library(str(tmp_path / "libbq.so"))


# fake, aligned, never dereferenced device addresses: validation fails first
P = 0x10000
PX, PW, PS, PB, PY = P, 2 * P, 3 * P, 4 * P, 5 * P


def call(lib, name, x=PX, w=PW, s=PS, b=PB, y=PY, M=1, N=8, K=256, bits=2, gs=64):
    return getattr(lib, name)(x, w, s, b, y, M, N, K, bits, gs, None)


U_ENTRIES = ["bq_qmv", "bq_qmv_wide", "bq_qmv_sym", "bq_qmm"]
T5_ENTRIES = ["bq_t5_qmv", "bq_t5_qmv_wide", "bq_t5_qmm"]


@pytest.mark.parametrize("name", U_ENTRIES + T5_ENTRIES + ["bq_dequant"])
def test_null_pointers(lib, name):
    bits = 0 if name in T5_ENTRIES else 2
    for kw in ("w", "s", "y"):
        assert call(lib, name, bits=bits, **{kw: None}) == NULL
    if name != "bq_dequant":
        assert call(lib, name, bits=bits, x=None) == NULL


@pytest.mark.parametrize("name", ["bq_qmv", "bq_qmv_wide"])
def test_affine_entries_need_biases(lib, name):
    assert call(lib, name, b=None) == NULL


@pytest.mark.parametrize("name", U_ENTRIES)
def test_bits_uint32_entries(lib, name):
    for bits in (0, 3, 4, 8, -1):
        assert call(lib, name, bits=bits) == BITS


@pytest.mark.parametrize("name", T5_ENTRIES)
def test_bits_t5_entries(lib, name):
    for bits in (1, 2, 3):
        assert call(lib, name, bits=bits) == BITS


def test_bits_dequant(lib):
    for bits in (3, 4, -1):
        assert call(lib, "bq_dequant", bits=bits) == BITS


@pytest.mark.parametrize("name", U_ENTRIES + T5_ENTRIES + ["bq_dequant"])
def test_group_size(lib, name):
    bits = 0 if name in T5_ENTRIES else 2
    for gs in (0, 32, 96, 256):
        assert call(lib, name, bits=bits, gs=gs) == GROUP


@pytest.mark.parametrize("name", U_ENTRIES + T5_ENTRIES + ["bq_dequant"])
def test_shapes(lib, name):
    bits = 0 if name in T5_ENTRIES else 2
    assert call(lib, name, bits=bits, N=0) == SHAPE
    assert call(lib, name, bits=bits, N=-3) == SHAPE
    assert call(lib, name, bits=bits, K=0) == SHAPE
    assert call(lib, name, bits=bits, K=320, gs=128) == SHAPE
    assert call(lib, name, bits=bits, K=(1 << 30) + 1024) == SHAPE
    assert call(lib, name, bits=bits, N=1, K=(1 << 26) + 1024) == SHAPE
    assert call(lib, name, bits=bits, N=8192, K=1 << 20) == SHAPE  # packed rows past 2^30 bytes
    if name not in ("bq_t5_qmm", "bq_qmm", "bq_dequant"):
        # a workgroup's scale rows no longer fit LDS
        assert call(lib, name, bits=bits, N=2, K=4093 * 64 + (192 if name in T5_ENTRIES else 0)) == SHAPE


@pytest.mark.parametrize("name", U_ENTRIES + T5_ENTRIES)
def test_m_range(lib, name):
    bits = 0 if name in T5_ENTRIES else 2
    assert call(lib, name, bits=bits, M=0) == MRANGE
    assert call(lib, name, bits=bits, M=-1) == MRANGE
    wide = name in ("bq_qmv_wide", "bq_qmv_sym", "bq_t5_qmv_wide")
    # M = 6 is valid for the per-row and qmm entry points; a misaligned y
    # stops those calls after the M check, before any launch
    assert call(lib, name, bits=bits, M=6, y=PY + 1) == (MRANGE if wide else ALIGN)


@pytest.mark.parametrize("name", U_ENTRIES + T5_ENTRIES + ["bq_dequant"])
def test_alignment(lib, name):
    bits = 0 if name in T5_ENTRIES else 2
    assert call(lib, name, bits=bits, w=PW + 2) == ALIGN
    assert call(lib, name, bits=bits, s=PS + 1) == ALIGN
    assert call(lib, name, bits=bits, y=PY + 1) == ALIGN
    if name != "bq_dequant":
        assert call(lib, name, bits=bits, x=PX + 1) == ALIGN


def test_qmm_x_vector_alignment(lib):
    # the prefill products stage x with 16-byte loads that write LDS
    assert call(lib, "bq_t5_qmm", bits=0, x=PX + 8) == ALIGN
    assert call(lib, "bq_qmm", bits=1, x=PX + 8) == ALIGN
    assert call(lib, "bq_t5_qmm", bits=0, x=PX + 4) == ALIGN


@pytest.mark.parametrize("name", ["bq_qmv", "bq_qmv_wide", "bq_qmv_sym", "bq_t5_qmv", "bq_t5_qmv_wide"])
def test_decode_dword_alignment(lib, name):
    # the decode kernels read x, scales and biases as dwords (any 4-byte
    # aligned address; the GPU tests run 4-byte offsets)
    bits = 0 if name in T5_ENTRIES else 2
    assert call(lib, name, bits=bits, x=PX + 2) == ALIGN
    assert call(lib, name, bits=bits, s=PS + 2) == ALIGN
    if name != "bq_qmv_sym":  # sym never reads the bias pointer
        assert call(lib, name, bits=bits, b=PB + 2) == ALIGN


PWS = 6 * P  # fake workspace


def call_ws(lib, name, ws=PWS, ws_bytes=1 << 24, **kw):
    x, w, sc, b, y = (kw.pop(k, d) for k, d in (("x", PX), ("w", PW), ("s", PS), ("b", PB), ("y", PY)))
    M, N, K, bits, gs = (kw.pop(k, d) for k, d in (("M", 1), ("N", 8), ("K", 256), ("bits", 2), ("gs", 64)))
    assert not kw
    return getattr(lib, name)(x, w, sc, b, y, M, N, K, bits, gs, ws, ws_bytes, None)


@pytest.mark.parametrize("name,bits", [("bq_t5_qmm_ws", 0), ("bq_qmm_ws", 2)])
def test_split_prefill_entries_validate(lib, name, bits):
    """The K-split products check the arguments of bq_t5_qmm / bq_qmm, then
    a 16-byte aligned workspace, before any launch."""
    for kw in ("w", "s", "y", "x"):
        assert call_ws(lib, name, bits=bits, **{kw: None}) == NULL
    assert call_ws(lib, name, bits=1 if bits == 0 else 0) == BITS
    assert call_ws(lib, name, bits=bits, gs=96) == GROUP
    assert call_ws(lib, name, bits=bits, K=320, gs=128) == SHAPE
    assert call_ws(lib, name, bits=bits, M=0) == MRANGE
    assert call_ws(lib, name, bits=bits, x=PX + 8) == ALIGN
    assert call_ws(lib, name, bits=bits, y=PY + 1) == ALIGN
    for off in (4, 8, 12):
        assert call_ws(lib, name, bits=bits, ws=PWS + off) == ALIGN


def test_linear_ws_validates(lib):
    def lw(flags=0, ws=PWS, M=20, bits=0, **kw):
        x, w, sc, b, y = (kw.pop(k, d) for k, d in (("x", PX), ("w", PW), ("s", PS), ("b", PB), ("y", PY)))
        return lib.bq_linear_ws(x, w, sc, b, y, M, 8, 256, bits, 64, flags, ws, 1 << 20, None)
    assert lw(flags=4) == -8  # BQ_ERR_FLAGS
    assert lw(ws=PWS + 8) == ALIGN  # prefill rows: the split product checks its workspace
    assert lw(w=None) == NULL
    assert lw(bits=2, b=None) == NULL  # stored biases required without the symmetric flag
    assert lw(bits=2, x=PX + 8) == ALIGN
    assert lw(M=0) == MRANGE
    assert lw(M=3, ws=PWS + 8, y=PY + 1) == ALIGN  # decode rows: bq_linear's checks
    assert lw(M=3, bits=3) == BITS


def test_split_prefill_workspace_size(lib):
    import ctypes
    n = ctypes.c_size_t(7)

    def ws(M, N, K, bits=0, gs=128):
        assert lib.bq_qmm_workspace(M, N, K, bits, gs, ctypes.byref(n)) == OK
        return n.value

    slice_ = lambda M, N: (M * N + 3) // 4 * 4 * 4
    # few tiles (5120 columns: 80 of 64) at M <= 32: a split of 2..8 shares
    for M, N in ((32, 5120), (17, 5120), (1, 1024), (5, 333)):
        b = ws(M, N, 17408)
        assert b % slice_(M, N) == 0 and 2 <= b // slice_(M, N) <= 8, (M, N, b)
    assert ws(17, 1000, 2560, bits=2, gs=64) % slice_(17, 1000) == 0
    # no split above 32 rows, nor where one K iteration leaves nothing to share
    assert ws(33, 5120, 17408) == 0
    assert ws(32, 5120, 64, bits=1, gs=64) == 0
    assert bq.bq_qmm_workspace(32, 5120, 17408, 0, 128) == ws(32, 5120, 17408)
    assert lib.bq_qmm_workspace(32, 8, 256, 3, 64, ctypes.byref(n)) == BITS
    assert lib.bq_qmm_workspace(32, 8, 256, 2, 96, ctypes.byref(n)) == GROUP
    assert lib.bq_qmm_workspace(32, 8, 320, 2, 128, ctypes.byref(n)) == SHAPE
    assert lib.bq_qmm_workspace(32, 0, 256, 2, 64, ctypes.byref(n)) == SHAPE
    assert lib.bq_qmm_workspace(0, 8, 256, 2, 64, ctypes.byref(n)) == MRANGE
    assert lib.bq_qmm_workspace(1, 8, 256, 2, 64, None) == NULL


def test_binding_raises_with_status(lib):
    with pytest.raises(bq.BQError) as ei:
        bq.bq_qmv_wide(PX, PW, PS, PB, PY, 6, 8, 256, 2, 64)
    assert ei.value.status == MRANGE and "BQ_ERR_M" in str(ei.value)


def test_binding_tensor_helpers_refuse_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 64, dtype=torch.float16)
    w = torch.zeros(1, 4, dtype=torch.int32)
    s = torch.zeros(1, 1, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        bq.qmv_wide(x, w, s, s, 2, 64)


# ---------------------------------------------------------------- dispatcher
def test_linear_routes():
    gate, down = 17408, 5120
    # bits 1/2: passes of up to five rows through the wide or symmetric kernel
    for bits in (1, 2):
        for M in (1, 2, 5):
            assert bq.bq_linear_route(M, gate, bits) == ("qmv_wide", 1)
            assert bq.bq_linear_route(M, gate, bits, bq.LINEAR_SYM) == ("qmv_sym", 1)
        assert bq.bq_linear_route(6, gate, bits) == ("qmv_wide", 2)
        assert bq.bq_linear_route(16, gate, bits) == ("qmv_wide", 4)
        # the fused product from 17 rows when there are 128 tiles of 32 x 64
        assert bq.QMM_MIN_M == 17 and bq.QMM_MIN_TILES == 128
        assert bq.bq_linear_route(17, gate, bits) == ("qmm", 1)
        assert bq.bq_linear_route(17, gate, bits, bq.LINEAR_SYM) == ("qmm", 1)
        assert bq.bq_linear_route(17, down, bits) == ("qmv_wide", 4)      # 80 tiles
        assert bq.bq_linear_route(32, down, bits) == ("qmv_wide", 7)
        assert bq.bq_linear_route(33, down, bits) == ("qmm", 1)           # 160 tiles
        assert bq.bq_linear_route(17, 64 * 128, bits) == ("qmm", 1)
        assert bq.bq_linear_route(17, 64 * 127, bits) == ("qmv_wide", 4)
        assert bq.bq_linear_route(2048, down, bits) == ("qmm", 1)
    # t5: wide passes below 17 rows, the fused product from 17 (M > 16)
    # when there are enough tiles of 32 x 64
    assert bq.T5_QMM_MIN_M == 17
    for M in (1, 5):
        assert bq.bq_linear_route(M, gate, bq.BITS_T5) == ("t5_qmv_wide", 1)
        assert bq.bq_linear_route(M, gate, bq.BITS_T5, bq.LINEAR_SYM) == ("t5_qmv_wide", 1)
    assert bq.bq_linear_route(16, gate, bq.BITS_T5) == ("t5_qmv_wide", 4)
    # t5 takes the fused product on fewer tiles: 64 tiles, or 16 from 24 rows
    assert (bq.T5_QMM_MIN_TILES, bq.T5_QMM_FEW_MIN_M, bq.T5_QMM_FEW_TILES) == (64, 24, 16)
    assert bq.bq_linear_route(17, gate, bq.BITS_T5) == ("t5_qmm", 1)
    assert bq.bq_linear_route(17, 64, bq.BITS_T5) == ("t5_qmv_wide", 4)    # 1 tile
    assert bq.bq_linear_route(17, down, bq.BITS_T5) == ("t5_qmm", 1)       # 80 tiles
    assert bq.bq_linear_route(17, 64 * 64, bq.BITS_T5) == ("t5_qmm", 1)    # 64 tiles
    assert bq.bq_linear_route(17, 64 * 63, bq.BITS_T5) == ("t5_qmv_wide", 4)
    assert bq.bq_linear_route(17, 1024, bq.BITS_T5) == ("t5_qmv_wide", 4)  # 16 tiles
    assert bq.bq_linear_route(23, 1024, bq.BITS_T5) == ("t5_qmv_wide", 5)
    assert bq.bq_linear_route(24, 1024, bq.BITS_T5) == ("t5_qmm", 1)
    assert bq.bq_linear_route(24, 64 * 15, bq.BITS_T5) == ("t5_qmv_wide", 5)  # 15 tiles
    assert bq.bq_linear_route(33, down, bq.BITS_T5) == ("t5_qmm", 1)       # 160 tiles
    assert bq.bq_linear_route(512, gate, bq.BITS_T5) == ("t5_qmm", 1)


def test_linear_route_errors(lib):
    assert lib.bq_linear_route(0, 8, 2, 0, None) == MRANGE
    assert lib.bq_linear_route(-4, 8, 2, 0, None) == MRANGE
    assert lib.bq_linear_route(1, 0, 2, 0, None) == SHAPE
    assert lib.bq_linear_route(1, 8, 3, 0, None) == BITS
    with pytest.raises(bq.BQError):
        bq.bq_linear_route(0, 8, 2)


FLAGS = -8


def lcall(lib, x=PX, w=PW, s=PS, b=PB, y=PY, M=1, N=8, K=256, bits=2, gs=64, flags=0):
    return lib.bq_linear(x, w, s, b, y, M, N, K, bits, gs, flags, None)


def test_linear_validates_before_launch(lib):
    assert lcall(lib, flags=2) == FLAGS
    assert lcall(lib, flags=-1) == FLAGS
    assert lcall(lib, M=0) == MRANGE
    assert lcall(lib, bits=3) == BITS
    assert lcall(lib, gs=32) == GROUP
    assert lcall(lib, N=0) == SHAPE
    assert lcall(lib, x=None) == NULL
    assert lcall(lib, b=None) == NULL            # stored bias required without the sym flag
    assert lcall(lib, x=PX + 2) == ALIGN
    assert lcall(lib, s=PS + 2) == ALIGN
    # t5 routes: wide below 17 rows (or with few output tiles), qmm from 17; both validate first
    assert lcall(lib, bits=0, K=192, b=None, x=PX + 2) == ALIGN
    assert lcall(lib, bits=0, M=17, N=8192, K=192, b=None, x=PX + 8) == ALIGN
    assert lcall(lib, bits=0, M=17, w=None, b=None) == NULL
    # the 1/2-bit fused route validates too, and needs stored biases without the sym flag
    assert lcall(lib, M=17, N=8192, b=None) == NULL
    assert lcall(lib, M=17, N=8192, x=PX + 8) == ALIGN
    assert lcall(lib, M=17, N=8192, flags=1, y=PY + 1) == ALIGN


def test_sym_check_validates(lib):
    vp = PX + 64
    assert lib.bq_sym_check(None, PB, 8, 256, 2, 64, vp, None) == NULL
    assert lib.bq_sym_check(PS, None, 8, 256, 2, 64, vp, None) == NULL
    assert lib.bq_sym_check(PS, PB, 8, 256, 2, 64, None, None) == NULL
    assert lib.bq_sym_check(PS, PB, 8, 256, 3, 64, vp, None) == BITS
    assert lib.bq_sym_check(PS, PB, 8, 256, 2, 96, vp, None) == GROUP
    assert lib.bq_sym_check(PS, PB, 0, 256, 2, 64, vp, None) == SHAPE
    assert lib.bq_sym_check(PS, PB, 8, 200, 2, 64, vp, None) == SHAPE
    assert lib.bq_sym_check(PS + 1, PB, 8, 256, 2, 64, vp, None) == ALIGN
    assert lib.bq_sym_check(PS, PB, 8, 256, 2, 64, vp + 2, None) == ALIGN


def test_t5_repack_validates(lib):
    fp = PX + 64
    rp = lambda w=PW, o=PY, N=8, K=256, bits=2, gs=64, flag=fp: lib.bq_t5_repack(w, o, N, K, bits, gs, flag, None)
    assert rp(w=None) == NULL
    assert rp(o=None) == NULL
    assert rp(flag=None) == NULL
    for bits in (0, 3, 4, -1):
        assert rp(bits=bits) == BITS
    for gs in (0, 32, 96, 256):
        assert rp(gs=gs) == GROUP
    assert rp(N=0) == SHAPE
    assert rp(K=0) == SHAPE
    assert rp(K=320, gs=128) == SHAPE
    assert rp(K=(1 << 26) + 256) == SHAPE
    assert rp(N=8192, K=1 << 20) == SHAPE      # input rows past 2^30 bytes
    assert rp(K=192) == ALIGN                  # t5 rows must be whole dwords
    assert rp(K=384, gs=128) == ALIGN
    assert rp(w=PW + 2) == ALIGN
    assert rp(o=PY + 2) == ALIGN
    assert rp(flag=fp + 2) == ALIGN


def test_t5_repack_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="GPU"):
        bq.t5_repack(torch.zeros(4, 16, dtype=torch.int32), 2, 64, 256)


WORKSPACE_ERR = -9


def test_spec_workspace_size(lib):
    import ctypes
    n = ctypes.c_size_t(0)
    assert lib.bq_spec_verify_workspace(4, 7, 151936, ctypes.byref(n)) == OK
    assert n.value >= 4 * 8 * 8 + 4 * 4
    assert bq.bq_spec_verify_workspace(4, 7, 151936) == n.value
    assert lib.bq_spec_verify_workspace(0, 7, 100, ctypes.byref(n)) == SHAPE
    assert lib.bq_spec_verify_workspace(1, -1, 100, ctypes.byref(n)) == SHAPE
    assert lib.bq_spec_verify_workspace(1, 1025, 100, ctypes.byref(n)) == SHAPE
    assert lib.bq_spec_verify_workspace(1, 1, 0, ctypes.byref(n)) == SHAPE
    assert lib.bq_spec_verify_workspace(1, 1, 1, None) == NULL


def test_spec_verify_validates(lib):
    D, A, T, W = PX, PW, PS, PB  # fake, aligned addresses
    big = 1 << 20

    def sv(lg=PY, dt=1, d=D, B=2, L=3, V=1000, a=A, n=A + 64, t=T, w=W, wb=big):
        return lib.bq_spec_decode_verify(lg, dt, d, B, L, V, a, n, t, w, wb, None)
    assert sv(lg=None) == NULL
    assert sv(d=None) == NULL
    assert sv(a=None) == NULL
    assert sv(n=None) == NULL
    for dt in (0, 3, -1):
        assert sv(dt=dt) == BITS
    assert sv(B=0) == SHAPE
    assert sv(L=-1) == SHAPE
    assert sv(L=1025) == SHAPE
    assert sv(V=0) == SHAPE
    assert sv(B=1 << 20, L=1000, V=1 << 20) == SHAPE     # grid past 2^31 workgroups
    assert sv(w=None) == WORKSPACE_ERR
    assert sv(wb=16) == WORKSPACE_ERR
    assert sv(lg=PY + 1) == ALIGN
    assert sv(lg=PY + 2, dt=2) == ALIGN                   # fp32 logits need 4 bytes
    assert sv(d=D + 2) == ALIGN
    assert sv(a=A + 2) == ALIGN
    assert sv(n=A + 66) == ALIGN
    assert sv(t=T + 2) == ALIGN
    assert sv(w=W + 4) == ALIGN


SCRATCH_ERR = -10


def test_spec_verify_noalloc_validates(lib):
    """The allocation-free verify call checks the same arguments and refuses,
    before any launch, a call whose scratch exceeds its static array."""
    import ctypes
    D, A, T = PX, PW, PS

    def sv(lg=PY, dt=1, d=D, B=2, L=3, V=1000, a=A, n=A + 64, t=T):
        return lib.bq_spec_decode_verify_noalloc(lg, dt, d, B, L, V, a, n, t, None)
    assert sv(lg=None) == NULL
    assert sv(d=None) == NULL
    assert sv(a=None) == NULL
    assert sv(n=None) == NULL
    for dt in (0, 3):
        assert sv(dt=dt) == BITS
    assert sv(B=0) == SHAPE
    assert sv(L=1025) == SHAPE
    assert sv(lg=PY + 1) == ALIGN
    assert sv(t=T + 2) == ALIGN
    # scratch: a key line and a count line per row of B*(L+1), a count line
    # per sequence
    limit = 2 * 1024 * 1024
    n = ctypes.c_size_t(0)
    assert lib.bq_spec_verify_workspace(4096, 15, 1000, ctypes.byref(n)) == OK and n.value > limit
    assert sv(B=4096, L=15) == SCRATCH_ERR
    assert lib.bq_spec_verify_workspace(256, 15, 1000, ctypes.byref(n)) == OK and n.value <= limit
    assert bq.STATUS[SCRATCH_ERR] == "BQ_ERR_SCRATCH"
    assert "scratch" in bq.strerror(SCRATCH_ERR)
