"""GPU parity of bq_spec_decode_verify against the oracle: accepted lengths,
next tokens and target tokens are integers and must match exactly."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import bit_quantized_decode_qmv_amd as bq
    bq.load_library()


def _run(logits, draft, workspace=None):
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to("cuda:0")
    dr = torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).to("cuda:0")
    a, n, t = bq.spec_decode_verify(lg, dr, workspace=workspace)
    torch.cuda.synchronize()
    return a.cpu().numpy(), n.cpu().numpy(), t.cpu().numpy()


def _check(logits, draft, workspace=None, what=""):
    a, n, t = _run(logits, draft, workspace)
    ra, rn, rt = oracle.spec_verify(logits, draft)
    assert np.array_equal(t, rt), f"{what}: target tokens differ"
    assert np.array_equal(a, ra), f"{what}: accepted {a} != {ra}"
    assert np.array_equal(n, rn), f"{what}: next {n} != {rn}"


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("B,L,V", [(1, 0, 1), (1, 1, 17), (3, 4, 8192), (3, 4, 8193), (2, 7, 32000),
                                   (8, 4, synth.QWEN_VOCAB), (1, 16, synth.QWEN_VOCAB)])
def test_spec_verify_planted(dtype, B, L, V):
    s = synth.make_spec_inputs(B, L, V, dtype=dtype, seed=60 + B + L)
    print(f"spec B{B} L{L} V{V} {np.dtype(dtype).name}", flush=True)
    _check(s.logits, s.draft, what=f"B{B} L{L} V{V}")
    a, _, _ = _run(s.logits, s.draft)
    assert np.array_equal(a, s.agree)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_spec_verify_ties_and_specials(dtype):
    """Integer-valued logits give many equal maxima (the lowest index wins);
    rows with -0/+0 ties, infinities and NaN follow the same rules as the
    oracle."""
    rng = np.random.default_rng(61)
    B, L, V = 4, 5, 20000
    lg = rng.integers(-3, 4, size=(B, L + 1, V)).astype(dtype)
    lg[0, 0] = -0.0
    lg[0, 0, 12345] = 0.0
    lg[0, 0, 777] = -0.0                      # -0 and +0 tie: 0 is the first
    lg[1, 2, 9000] = np.inf
    lg[1, 2, 9001] = np.inf
    lg[2, 3, 19999] = np.nan                  # NaN beats +inf and every number
    lg[2, 3, 5] = np.inf
    lg[3, :, :] = -np.inf
    lg[3, 1, 15000] = np.nan
    lg[3, 1, 16000] = np.nan
    t_ref = oracle.target_tokens(lg)
    draft = t_ref[:, :L].astype(np.int32).copy()
    draft[1, 2] += 1                          # sequence 1 rejected at position 2
    _check(lg, draft, what="ties")


def test_spec_verify_workspace_reuse():
    """One workspace serves calls of different shapes back to back; each call
    leaves it zero for the next."""
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    need = max(bq.bq_spec_verify_workspace(8, 7, synth.QWEN_VOCAB), bq.bq_spec_verify_workspace(2, 3, 1000))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for i, (B, L, V) in enumerate([(8, 7, synth.QWEN_VOCAB), (2, 3, 1000), (8, 7, synth.QWEN_VOCAB),
                                   (1, 0, 5)]):
        s = synth.make_spec_inputs(B, L, V, dtype=np.float16, seed=70 + i)
        _check(s.logits, s.draft, workspace=ws, what=f"call {i}")
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0


def test_spec_verify_all_accepted_and_first_rejected():
    B, L, V = 6, 7, 50000
    s = synth.make_spec_inputs(B, L, V, dtype=np.float32, seed=80, agree=[0, 7, 3, 7, 0, 6])
    a, n, t = _run(s.logits, s.draft)
    assert a.tolist() == [0, 7, 3, 7, 0, 6]
    assert np.array_equal(n, s.planted[np.arange(B), a])


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("V", [7, 9, 8193, 20011])
def test_spec_verify_maximum_kinds(dtype, V):
    """Rows whose maximum is each kind of value the kernel tells apart: a
    positive or negative normal number (also repeated, and at the first and
    last index), a subnormal, the most negative finite value, -inf, a zero;
    rows start at every offset within a 16-byte block (odd V)."""
    rng = np.random.default_rng(62 + V)
    fi = np.finfo(dtype)
    B, L = 3, 6
    rows = B * (L + 1)
    lg = (rng.standard_normal((rows, V)) * 3).astype(dtype)
    sub = fi.smallest_subnormal
    lg[0] = -np.abs(lg[0]) - 1                          # negative normal maximum
    lg[0, V // 2] = -0.5
    lg[1, :] = -np.abs(lg[1]) - 1                       # maximum at the first index
    lg[1, 0] = -0.25
    lg[2, :] = -np.abs(lg[2]) - 1                       # maximum at the last index
    lg[2, V - 1] = -0.125
    lg[3] = -np.abs(lg[3])                              # subnormal maximum, repeated
    lg[3, V // 3] = sub * 3
    lg[3, V - 1] = sub * 3
    lg[4] = -fi.max                                     # the most negative finite value everywhere
    lg[5] = -fi.max
    lg[5, V // 2:] = -np.inf                            # ... and -inf after it
    lg[6] = -np.inf                                     # -inf everywhere: index 0
    lg[7] = -np.abs(lg[7]) - 1                          # a zero maximum: -0 first, then +0
    lg[7, V - 1] = 0.0
    lg[7, min(3, V - 2)] = -0.0
    lg[8] = np.abs(lg[8]) + 1                           # repeated positive maximum
    lg[8, [V - 1, V // 2, 1]] = 7.0
    lg[9] = -np.abs(lg[9]) - 1                          # -fmax beside a normal maximum
    lg[9, 0] = -fi.max
    lg[9, V - 1] = -2.0
    lg[10, :] = sub                                     # subnormal everywhere
    lg = lg.reshape(B, L + 1, V)
    t_ref = oracle.target_tokens(lg)
    draft = t_ref[:, :L].astype(np.int32).copy()
    draft[2, 4] += 1
    print(f"spec maximum kinds V{V} {np.dtype(dtype).name}", flush=True)
    _check(lg, draft, what=f"maximum kinds V{V}")
