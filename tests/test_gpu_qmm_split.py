"""GPU parity of the K-split prefill products (bq_t5_qmm_ws, bq_qmm_ws)
through the C ABI: several workgroups share the K iterations of an output
tile, store fp32 partial tiles to the caller's workspace, and a second
kernel adds them in a fixed order.  Checked against the fp64 oracle, bit for
bit on one-hot activation rows, for a fixed result across calls, and for
the unsplit result when the workspace is missing or too small."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import BITS, assert_close, dev, make, to_np, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


def _split_call(inp, x=None, ws_bytes=None, workspace="alloc"):
    """One call of the split entry point of inp's format; returns (y, the
    workspace bytes bq_qmm_workspace asked for)."""
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    M, N, K, gs = inp.M, inp.N, inp.K, inp.group_size
    bits = BITS[inp.fmt]
    xd = x if x is not None else dev(inp.x)
    wd, sd, bd = dev(inp.w), dev(inp.scales), dev(inp.biases)
    need = bq.bq_qmm_workspace(M, N, K, bits, gs)
    nbytes = need if ws_bytes is None else ws_bytes
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda:0") if workspace == "alloc" else None
    y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fn = bq.bq_t5_qmm_ws if inp.fmt == "t5" else bq.bq_qmm_ws
    fn(xd.data_ptr(), wd.data_ptr(), sd.data_ptr(), bd.data_ptr() if bd is not None else None, y.data_ptr(),
       M, N, K, bits, gs, ws.data_ptr() if ws is not None else None, nbytes if ws is not None else 0,
       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return to_np(y), need


def _unsplit(inp):
    import bit_quantized_decode_qmv_amd as bq
    xd, wd, sd, bd = dev(inp.x), dev(inp.w), dev(inp.scales), dev(inp.biases)
    if inp.fmt == "t5":
        y = bq.t5_qmm(xd, wd, sd, inp.group_size, biases=bd)
    else:
        y = bq.qmm(xd, wd, sd, BITS[inp.fmt], inp.group_size, biases=bd)
    torch_mod().cuda.synchronize()
    return to_np(y)


# ragged N, 1 to 32 rows, K step counts that the share count does not
# divide (43 and 21 steps over 8 and 7 shares), both group sizes and bias
# kinds
CASES = [("t5", "t5", 64, 17, 1000, 2560), ("t5", "asym", 128, 32, 333, 2560), ("t5", "t5", 128, 1, 200, 4608),
         ("t5", "t5", 64, 5, 1000, 2752), ("u2", "asym", 64, 32, 1000, 2560), ("u1", "sym", 128, 17, 333, 2560),
         ("u2", "sym", 64, 24, 1000, 2752), ("u1", "asym", 64, 9, 4100, 1344)]


@pytest.mark.parametrize("fmt,variant,gs,M,N,K", CASES)
def test_split_parity(fmt, variant, gs, M, N, K):
    inp = make(fmt, M, N, K, gs, variant, seed=110)
    print(f"split qmm {fmt} {variant} gs{gs} M{M} N{N} K{K}", flush=True)
    y, need = _split_call(inp)
    assert need > 0, "these shapes are meant to split"
    assert np.all(np.isfinite(y))
    assert_close(y.astype(np.float64), inp, what=f"split {fmt} {variant} gs{gs} M{M} N{N} K{K}")
    # the partials are added in a fixed order: the same bits every call
    y2, _ = _split_call(inp)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("fmt,variant,gs,M,N,K", [("t5", "t5", 64, 32, 1000, 640), ("t5", "asym", 128, 20, 515, 1280),
                                                  ("u2", "asym", 64, 32, 1000, 640), ("u1", "sym", 128, 16, 300, 1024)])
def test_split_one_hot_rows_read_exact_weights(fmt, variant, gs, M, N, K):
    """With one-hot activation rows each output is one weight: the share
    holding it gives the weight exactly and the others exact zeros, so the
    split result is every weight bit for bit."""
    inp = make(fmt, M, N, K, gs, variant, seed=111)
    codes = oracle.codes_of(fmt, inp.w, K, gs)
    W16 = oracle.dequant_f16(codes, inp.scales, oracle.effective_biases(fmt, inp.scales, inp.biases), gs)
    print(f"split one-hot {fmt} {variant} gs{gs} M{M} N{N} K{K}", flush=True)
    for base in range(0, K, M):
        ks = np.arange(base, min(base + M, K))
        x = np.zeros((M, K), np.float16)
        x[np.arange(len(ks)), ks] = 1.0
        y, need = _split_call(inp, x=dev(x))
        assert need > 0
        want = W16[:, ks].T
        bad = np.argwhere(y[:len(ks)] != want)
        assert len(bad) == 0, (f"K columns {base}..{base + len(ks) - 1}: {len(bad)} weights differ, e.g. "
                               + ", ".join(f"W[{n}][{ks[m]}] {y[m, n]!r} != {want[m, n]!r}" for m, n in bad[:6]))
        assert not y[len(ks):].any()


@pytest.mark.parametrize("fmt,variant", [("t5", "t5"), ("u2", "asym")])
def test_missing_or_small_workspace_gives_the_unsplit_product(fmt, variant):
    inp = make(fmt, 32, 1000, 2560, 64, variant, seed=112)
    ref = _unsplit(inp)
    y_null, need = _split_call(inp, workspace=None)
    assert need > 0
    assert np.array_equal(y_null.view(np.uint16), ref.view(np.uint16))
    # room for fewer shares only: a smaller split or none, each within the tolerance
    for nbytes in (need - 16, (need // 2) & ~15, 16):
        y, _ = _split_call(inp, ws_bytes=nbytes)
        assert_close(y.astype(np.float64), inp, what=f"split with {nbytes} of {need} workspace bytes")
    y16, _ = _split_call(inp, ws_bytes=16)
    assert np.array_equal(y16.view(np.uint16), ref.view(np.uint16))


def _sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(N, 40), replace=False).tolist())
    rows.update({0, N - 1})
    return np.array(sorted(rows))


@pytest.mark.parametrize("shape", ["q", "k", "o", "gate", "down"])
@pytest.mark.parametrize("fmt,variant,M", [("t5", "t5", 32), ("u2", "asym", 17)])
def test_split_full_size_sampled(shape, fmt, variant, M):
    """The projection shapes of a hidden = 5120 decoder, gs 128, where the
    split applies (every one at M <= 32), on sampled output columns."""
    N, K = synth.PROJECTION_SHAPES[shape]
    inp = make(fmt, M, N, K, 128, variant, seed=113)
    print(f"split full {fmt} {shape} M{M}", flush=True)
    y, need = _split_call(inp)
    assert need > 0
    assert np.all(np.isfinite(y))
    assert_close(y.astype(np.float64), inp, rows=_sample_rows(N, 114), what=f"split {fmt} {shape} M{M}")


def test_binding_allocates_the_workspace():
    import bit_quantized_decode_qmv_amd as bq
    inp = make("t5", 24, 1000, 1280, 64, "t5", seed=115)
    y_c, _ = _split_call(inp)
    y_b = to_np(bq.t5_qmm_ws(dev(inp.x), dev(inp.w), dev(inp.scales), 64))
    assert np.array_equal(y_c.view(np.uint16), y_b.view(np.uint16))
    inp = make("u1", 24, 1000, 1280, 64, "asym", seed=116)
    y_c, _ = _split_call(inp)
    y_b = to_np(bq.qmm_ws(dev(inp.x), dev(inp.w), dev(inp.scales), 1, 64, biases=dev(inp.biases)))
    assert np.array_equal(y_c.view(np.uint16), y_b.view(np.uint16))


def test_graph_replays_match_eager_calls():
    """The split products (and decode calls beside them) captured in one
    graph give the eager bits on every replay, with eager work and
    synchronizations between the replays (the workspace is reused by
    replays and eager calls alike)."""
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    stream = lambda: torch.cuda.current_stream().cuda_stream
    cases = [make("t5", 24, 1000, 2560, 128, "t5", seed=117), make("u2", 32, 700, 1280, 64, "asym", seed=118),
             make("t5", 5, 1000, 2560, 64, "t5", seed=119), make("u2", 3, 700, 1280, 64, "asym", seed=120)]
    ins = [(dev(c.x), dev(c.w), dev(c.scales), dev(c.biases)) for c in cases]
    outs = [torch.zeros((c.M, c.N), dtype=torch.float16, device="cuda:0") for c in cases]
    need = max(bq.bq_qmm_workspace(c.M, c.N, c.K, BITS[c.fmt], c.group_size) for c in cases[:2])
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")

    def launch_all():
        for c, (x, w, s, b), y in zip(cases, ins, outs):
            args = (x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr() if b is not None else None, y.data_ptr(),
                    c.M, c.N, c.K, BITS[c.fmt], c.group_size)
            if c.M > 5:
                fn = bq.bq_t5_qmm_ws if c.fmt == "t5" else bq.bq_qmm_ws
                fn(*args, ws.data_ptr(), need, stream())
            else:
                fn = bq.bq_t5_qmv_wide if c.fmt == "t5" else bq.bq_qmv_wide
                fn(*args, stream())

    launch_all()
    torch.cuda.synchronize()
    eager = [to_np(y).copy() for y in outs]
    for c, y in zip(cases, eager):
        assert_close(y.astype(np.float64), c, what=f"eager {c.fmt} M{c.M}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch_all()
    for r in range(3):
        for y in outs:
            y.zero_()
        launch_all()  # eager calls on the same workspace between replays
        torch.cuda.synchronize()
        for y in outs:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for c, y, e in zip(cases, outs, eager):
            assert np.array_equal(to_np(y).view(np.uint16), e.view(np.uint16)), f"replay {r}: {c.fmt} M{c.M}"
