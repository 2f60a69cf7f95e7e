"""GPU check of the allocation-free verify entry point through the C ABI.

bq_spec_decode_verify_noalloc must give exactly the outputs of
bq_spec_decode_verify (caller workspace) -- accepted lengths, next tokens and
target tokens are integers -- on consecutive calls that share its static
scratch, the second with a smaller input, and both must match the oracle.
"""
import ctypes

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


def _both(lib, logits, draft):
    """(noalloc outputs, workspace outputs), each (accepted, next, targets)."""
    torch = torch_mod()
    B, rows, V = logits.shape
    L = rows - 1
    dt = 1 if logits.dtype == np.float16 else 2
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to("cuda:0")
    dr = torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).to("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for kind in ("noalloc", "workspace"):
        a = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
        n = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
        t = torch.full((B, rows), -7, dtype=torch.int32, device="cuda:0")
        dp = dr.data_ptr() if L > 0 else None
        if kind == "noalloc":
            st = lib.bq_spec_decode_verify_noalloc(lg.data_ptr(), dt, dp, B, L, V, a.data_ptr(), n.data_ptr(),
                                                   t.data_ptr(), stream)
        else:
            nb = ctypes.c_size_t(0)
            assert lib.bq_spec_verify_workspace(B, L, V, ctypes.byref(nb)) == 0
            ws = torch.zeros(nb.value, dtype=torch.uint8, device="cuda:0")
            st = lib.bq_spec_decode_verify(lg.data_ptr(), dt, dp, B, L, V, a.data_ptr(), n.data_ptr(), t.data_ptr(),
                                           ws.data_ptr(), nb.value, stream)
        assert st == 0, (kind, st)
        torch.cuda.synchronize()
        outs.append((a.cpu().numpy(), n.cpu().numpy(), t.cpu().numpy()))
    return outs


def test_noalloc_matches_workspace_call_twice_then_smaller():
    import bit_quantized_decode_qmv_amd as bq
    lib = bq.load_library()
    cases = [(8, 7, synth.QWEN_VOCAB, np.float16), (2, 3, 32000, np.float32), (5, 0, 777, np.float16)]
    for i, (B, L, V, dtype) in enumerate(cases):
        print(f"noalloc call {i}: B{B} L{L} V{V} {np.dtype(dtype).name}", flush=True)
        s = synth.make_spec_inputs(B, L, V, dtype=dtype, seed=90 + i)
        (na, nn, nt), (wa, wn, wt) = _both(lib, s.logits, s.draft)
        assert np.array_equal(na, wa) and np.array_equal(nn, wn) and np.array_equal(nt, wt), f"call {i}"
        ra, rn, rt = oracle.spec_verify(s.logits, s.draft)
        assert np.array_equal(na, ra) and np.array_equal(nn, rn) and np.array_equal(nt, rt), f"call {i} vs oracle"


def test_noalloc_refuses_oversized_call_without_launch():
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    lib = bq.load_library()
    B, L, V = 4096, 15, 16
    lg = torch.zeros((B, L + 1, V), dtype=torch.float16, device="cuda:0")
    dr = torch.zeros((B, L), dtype=torch.int32, device="cuda:0")
    a = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    n = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    st = lib.bq_spec_decode_verify_noalloc(lg.data_ptr(), 1, dr.data_ptr(), B, L, V, a.data_ptr(), n.data_ptr(),
                                           None, None)
    torch.cuda.synchronize()
    assert st == -10
    assert int(a.min()) == -7 and int(a.max()) == -7  # nothing ran
