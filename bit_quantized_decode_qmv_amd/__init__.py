"""Low-bit weight-quantized decode QMV for MI355X (gfx950).

Thin binding over the C ABI of ``libbq.so`` (declared in ``include/bq.h``):
argument marshalling only -- every step of the product runs in the HIP
kernels.  PyTorch is used for device memory and streams.

Two layers:

* ``bq_*`` functions with the C names and C arguments (integers for
  pointers and the stream); they raise :class:`BQError` on a nonzero status.
* tensor helpers (``qmv``, ``qmv_wide``, ``qmv_sym``, ``t5_qmv``,
  ``t5_qmv_wide``, ``t5_qmm``, ``dequant``, ``linear``, ``sym_check``) that
  check devices, dtypes and contiguity, allocate the output and pass the
  current stream, and :class:`QuantizedWeight`, a layer's packed weights
  with its symmetric-bias check done once.

The library is loaded on first use; a missing build or an ABI mismatch is an
error (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

ABI_VERSION = 10
BITS_T5 = 0
MAX_WIDE_M = 5
LINEAR_SYM = 1
T5_QMM_MIN_M = 17
T5_QMM_MIN_TILES = 64
T5_QMM_FEW_MIN_M = 24
T5_QMM_FEW_TILES = 16
QMM_MIN_M = 17
QMM_MIN_TILES = 128
DTYPE_F16 = 1
DTYPE_F32 = 2
SPEC_MAX_DRAFT = 1024
ROUTES = {1: "qmv_wide", 2: "qmv_sym", 3: "t5_qmv_wide", 4: "t5_qmm", 5: "qmm"}

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libbq.so")

ENTRY_POINTS = ("bq_qmv", "bq_qmv_wide", "bq_qmv_sym", "bq_t5_qmv", "bq_t5_qmv_wide",
                "bq_t5_qmm", "bq_dequant", "bq_qmm")
DISPATCH_POINTS = ("bq_linear", "bq_linear_route", "bq_sym_check", "bq_t5_repack", "bq_spec_verify_workspace",
                   "bq_spec_decode_verify", "bq_spec_decode_verify_noalloc", "bq_qmm_workspace", "bq_t5_qmm_ws",
                   "bq_qmm_ws", "bq_linear_ws")
ALL_SYMBOLS = ("bq_abi_version", "bq_strerror") + ENTRY_POINTS + DISPATCH_POINTS

STATUS = {
    0: "BQ_OK", -1: "BQ_ERR_NULL", -2: "BQ_ERR_BITS", -3: "BQ_ERR_GROUP", -4: "BQ_ERR_SHAPE",
    -5: "BQ_ERR_M", -6: "BQ_ERR_ALIGN", -7: "BQ_ERR_HIP", -8: "BQ_ERR_FLAGS", -9: "BQ_ERR_WORKSPACE",
    -10: "BQ_ERR_SCRATCH",
}


class BQError(RuntimeError):
    def __init__(self, status: int, message: str, entry: str):
        super().__init__(f"{entry}: {STATUS.get(status, status)} ({message})")
        self.status = status
        self.entry = entry


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libbq.so once and check its ABI version."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    lib.bq_abi_version.restype = ctypes.c_int
    lib.bq_abi_version.argtypes = []
    lib.bq_strerror.restype = ctypes.c_char_p
    lib.bq_strerror.argtypes = [ctypes.c_int]
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ENTRY_POINTS:
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.bq_linear.restype = ctypes.c_int
    lib.bq_linear.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.bq_linear_route.restype = ctypes.c_int
    lib.bq_linear_route.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_int)]
    lib.bq_sym_check.restype = ctypes.c_int
    lib.bq_sym_check.argtypes = [vp, vp, i, i, i, i, vp, vp]
    lib.bq_t5_repack.restype = ctypes.c_int
    lib.bq_t5_repack.argtypes = [vp, vp, i, i, i, i, vp, vp]
    lib.bq_spec_verify_workspace.restype = ctypes.c_int
    lib.bq_spec_verify_workspace.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_size_t)]
    lib.bq_spec_decode_verify.restype = ctypes.c_int
    lib.bq_spec_decode_verify.argtypes = [vp, i, vp, i, i, i, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bq_spec_decode_verify_noalloc.restype = ctypes.c_int
    lib.bq_spec_decode_verify_noalloc.argtypes = [vp, i, vp, i, i, i, vp, vp, vp, vp]
    lib.bq_linear_ws.restype = ctypes.c_int
    lib.bq_linear_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, ctypes.c_size_t, vp]
    lib.bq_qmm_workspace.restype = ctypes.c_int
    lib.bq_qmm_workspace.argtypes = [i, i, i, i, i, ctypes.POINTER(ctypes.c_size_t)]
    for name in ("bq_t5_qmm_ws", "bq_qmm_ws"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, ctypes.c_size_t, vp]
    ver = lib.bq_abi_version()
    if ver != ABI_VERSION:
        raise ImportError(f"{p} has ABI version {ver}, this binding needs {ABI_VERSION}")
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().bq_strerror(status).decode()


def _call(name: str, x, w, scales, biases, y, M, N, K, bits, group_size, stream) -> int:
    lib = load_library()
    st = getattr(lib, name)(x, w, scales, biases, y, M, N, K, bits, group_size, stream)
    if st != 0:
        raise BQError(st, lib.bq_strerror(st).decode(), name)
    return st


def _c_entry(name):
    def fn(x, w, scales, biases, y, M, N, K, bits, group_size, stream=None):
        return _call(name, x, w, scales, biases, y, M, N, K, bits, group_size, stream)
    fn.__name__ = name
    fn.__doc__ = f"C entry point {name} of include/bq.h (pointers and stream as integers)."
    return fn


bq_qmv = _c_entry("bq_qmv")
bq_qmv_wide = _c_entry("bq_qmv_wide")
bq_qmv_sym = _c_entry("bq_qmv_sym")
bq_t5_qmv = _c_entry("bq_t5_qmv")
bq_t5_qmv_wide = _c_entry("bq_t5_qmv_wide")
bq_t5_qmm = _c_entry("bq_t5_qmm")
bq_dequant = _c_entry("bq_dequant")
bq_qmm = _c_entry("bq_qmm")


def bq_abi_version() -> int:
    return load_library().bq_abi_version()


def _raise_if(st: int, name: str) -> int:
    if st < 0:
        raise BQError(st, load_library().bq_strerror(st).decode(), name)
    return st


def bq_linear(x, w, scales, biases, y, M, N, K, bits, group_size, flags, stream=None):
    """C entry point bq_linear of include/bq.h (pointers and stream as integers)."""
    return _raise_if(load_library().bq_linear(x, w, scales, biases, y, M, N, K, bits, group_size, flags,
                                               stream), "bq_linear")


def bq_linear_ws(x, w, scales, biases, y, M, N, K, bits, group_size, flags, workspace, workspace_bytes,
                 stream=None):
    """C entry point bq_linear_ws of include/bq.h (pointers and stream as integers)."""
    return _raise_if(load_library().bq_linear_ws(x, w, scales, biases, y, M, N, K, bits, group_size, flags,
                                                  workspace, workspace_bytes, stream), "bq_linear_ws")


def bq_linear_route(M, N, bits, flags=0):
    """(route name, passes) bq_linear takes for (M, N, bits, flags); host only."""
    passes = ctypes.c_int(0)
    st = _raise_if(load_library().bq_linear_route(M, N, bits, flags, ctypes.byref(passes)), "bq_linear_route")
    return ROUTES[st], passes.value


def bq_sym_check(scales, biases, N, K, bits, group_size, flag, stream=None):
    """C entry point bq_sym_check of include/bq.h (flag: device int pointer)."""
    return _raise_if(load_library().bq_sym_check(scales, biases, N, K, bits, group_size, flag, stream),
                     "bq_sym_check")


def bq_t5_repack(w, w_t5, N, K, bits, group_size, flag, stream=None):
    """C entry point bq_t5_repack of include/bq.h (flag: device int pointer)."""
    return _raise_if(load_library().bq_t5_repack(w, w_t5, N, K, bits, group_size, flag, stream), "bq_t5_repack")


def bq_spec_verify_workspace(B, L, V):
    """Workspace bytes bq_spec_decode_verify needs (host only)."""
    n = ctypes.c_size_t(0)
    _raise_if(load_library().bq_spec_verify_workspace(B, L, V, ctypes.byref(n)), "bq_spec_verify_workspace")
    return n.value


def bq_spec_decode_verify(logits, logits_dtype, draft, B, L, V, accepted, next_token, target_tokens, workspace,
                          workspace_bytes, stream=None):
    """C entry point bq_spec_decode_verify of include/bq.h (pointers as integers)."""
    return _raise_if(load_library().bq_spec_decode_verify(logits, logits_dtype, draft, B, L, V, accepted, next_token,
                                                          target_tokens, workspace, workspace_bytes, stream),
                     "bq_spec_decode_verify")


def bq_spec_decode_verify_noalloc(logits, logits_dtype, draft, B, L, V, accepted, next_token, target_tokens,
                                  stream=None):
    """C entry point bq_spec_decode_verify_noalloc of include/bq.h (pointers as
    integers): the verify call without a workspace (static scratch inside
    the library; no allocation)."""
    return _raise_if(load_library().bq_spec_decode_verify_noalloc(logits, logits_dtype, draft, B, L, V, accepted,
                                                                  next_token, target_tokens, stream),
                     "bq_spec_decode_verify_noalloc")


def bq_qmm_workspace(M, N, K, bits, group_size):
    """Workspace bytes the K-split prefill products want (0: no split; host only)."""
    n = ctypes.c_size_t(0)
    _raise_if(load_library().bq_qmm_workspace(M, N, K, bits, group_size, ctypes.byref(n)), "bq_qmm_workspace")
    return n.value


def bq_t5_qmm_ws(x, w, scales, biases, y, M, N, K, bits, group_size, workspace, workspace_bytes, stream=None):
    """C entry point bq_t5_qmm_ws of include/bq.h (pointers and stream as integers)."""
    return _raise_if(load_library().bq_t5_qmm_ws(x, w, scales, biases, y, M, N, K, bits, group_size, workspace,
                                                  workspace_bytes, stream), "bq_t5_qmm_ws")


def bq_qmm_ws(x, w, scales, biases, y, M, N, K, bits, group_size, workspace, workspace_bytes, stream=None):
    """C entry point bq_qmm_ws of include/bq.h (pointers and stream as integers)."""
    return _raise_if(load_library().bq_qmm_ws(x, w, scales, biases, y, M, N, K, bits, group_size, workspace,
                                               workspace_bytes, stream), "bq_qmm_ws")


# ---------------------------------------------------------------------------
# torch helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _check(t, name, dtype, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _run(name, x, w, scales, biases, bits, group_size, out, M, N, K, out_shape):
    torch = _torch()
    dev = w.device
    _check(w, "w", torch.uint8 if bits == BITS_T5 else torch.int32, dev)
    _check(scales, "scales", torch.float16, dev)
    if biases is not None:
        _check(biases, "biases", torch.float16, dev)
    if x is not None:
        _check(x, "x", torch.float16, dev)
    if out is None:
        out = torch.empty(out_shape, dtype=torch.float16, device=dev)
    else:
        _check(out, "out", torch.float16, dev)
        if tuple(out.shape) != tuple(out_shape):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(out_shape)}")
    _call(name, x.data_ptr() if x is not None else None, w.data_ptr(), scales.data_ptr(),
          biases.data_ptr() if biases is not None else None, out.data_ptr(), M, N, K, bits,
          group_size, _stream_handle(dev))
    return out


def _shapes(x, scales, group_size):
    M, K = x.shape
    N = scales.shape[0]
    if scales.shape[1] * group_size != K:
        raise ValueError("scales must be [N][K/group_size]")
    return M, N, K


def qmv(x, w, scales, biases, bits: int, group_size: int, out=None):
    """y = x . W^T, each row of x an independent pass over W (bits 1 or 2)."""
    M, N, K = _shapes(x, scales, group_size)
    return _run("bq_qmv", x, w, scales, biases, bits, group_size, out, M, N, K, (M, N))


def qmv_wide(x, w, scales, biases, bits: int, group_size: int, out=None):
    """y = x . W^T for 1..5 rows sharing one read of W (bits 1 or 2)."""
    M, N, K = _shapes(x, scales, group_size)
    return _run("bq_qmv_wide", x, w, scales, biases, bits, group_size, out, M, N, K, (M, N))


def qmv_sym(x, w, scales, bits: int, group_size: int, out=None, biases=None):
    """Symmetric variant: bias implied as -scale*(2^bits-1)/2, never read."""
    M, N, K = _shapes(x, scales, group_size)
    return _run("bq_qmv_sym", x, w, scales, biases, bits, group_size, out, M, N, K, (M, N))


def t5_qmv(x, w, scales, group_size: int, biases=None, out=None):
    """t5 ternary weights, each row of x an independent pass."""
    M, N, K = _shapes(x, scales, group_size)
    return _run("bq_t5_qmv", x, w, scales, biases, BITS_T5, group_size, out, M, N, K, (M, N))


def t5_qmv_wide(x, w, scales, group_size: int, biases=None, out=None):
    """t5 ternary weights, 1..5 rows sharing one read of W."""
    M, N, K = _shapes(x, scales, group_size)
    return _run("bq_t5_qmv_wide", x, w, scales, biases, BITS_T5, group_size, out, M, N, K, (M, N))


def t5_qmm(x, w, scales, group_size: int, biases=None, out=None):
    """t5 prefill product on the matrix cores (any M)."""
    M, N, K = _shapes(x, scales, group_size)
    return _run("bq_t5_qmm", x, w, scales, biases, BITS_T5, group_size, out, M, N, K, (M, N))


def qmm(x, w, scales, bits: int, group_size: int, biases=None, out=None):
    """Fused 1/2-bit prefill product y = x . W^T (biases None: implied
    -scale*(2^bits-1)/2)."""
    M, N, K = _shapes(x, scales, group_size)
    return _run("bq_qmm", x, w, scales, biases, bits, group_size, out, M, N, K, (M, N))


def _run_ws(name, x, w, scales, biases, bits, group_size, out, workspace):
    torch = _torch()
    M, N, K = _shapes(x, scales, group_size)
    dev = w.device
    _check(w, "w", torch.uint8 if bits == BITS_T5 else torch.int32, dev)
    _check(scales, "scales", torch.float16, dev)
    _check(x, "x", torch.float16, dev)
    if biases is not None:
        _check(biases, "biases", torch.float16, dev)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    else:
        _check(out, "out", torch.float16, dev)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    if workspace is None:
        need = bq_qmm_workspace(M, N, K, bits, group_size)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    elif workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    fn = bq_t5_qmm_ws if name == "bq_t5_qmm_ws" else bq_qmm_ws
    fn(x.data_ptr(), w.data_ptr(), scales.data_ptr(), biases.data_ptr() if biases is not None else None,
       out.data_ptr(), M, N, K, bits, group_size, workspace.data_ptr() if workspace is not None else None,
       workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream_handle(dev))
    return out


def t5_qmm_ws(x, w, scales, group_size: int, biases=None, out=None, workspace=None):
    """t5 prefill product with K split over a workspace (a device tensor of
    at least bq_qmm_workspace bytes, 16-byte aligned; None: allocated here)."""
    return _run_ws("bq_t5_qmm_ws", x, w, scales, biases, BITS_T5, group_size, out, workspace)


def qmm_ws(x, w, scales, bits: int, group_size: int, biases=None, out=None, workspace=None):
    """1/2-bit prefill product with K split over a workspace (as t5_qmm_ws)."""
    return _run_ws("bq_qmm_ws", x, w, scales, biases, bits, group_size, out, workspace)


def dequant(w, scales, biases, bits: int, group_size: int, K: int, out=None):
    """fp16 [N][K] weights, each the correctly rounded scale*q + bias."""
    N = scales.shape[0]
    return _run("bq_dequant", None, w, scales, biases, bits, group_size, out, 0, N, K, (N, K))


def sym_check(scales, biases, bits: int, group_size: int) -> bool:
    """True when every bias equals -scale*ratio exactly (ratio (2^bits-1)/2,
    t5: 1), checked on the GPU; waits for the result."""
    torch = _torch()
    dev = scales.device
    _check(scales, "scales", torch.float16, dev)
    _check(biases, "biases", torch.float16, dev)
    if tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("scales and biases must have the same shape")
    N, G = scales.shape
    flag = torch.empty(1, dtype=torch.int32, device=dev)
    bq_sym_check(scales.data_ptr(), biases.data_ptr(), N, G * group_size, bits, group_size, flag.data_ptr(),
                 _stream_handle(dev))
    return bool(flag.item())


def t5_repack(w, bits: int, group_size: int, K: int):
    """t5 bytes of a 1/2-bit code tensor (int32 words [N][K*bits/32]) and
    whether every code was 0..2 (then the repack is exact); waits for the
    flag."""
    torch = _torch()
    dev = w.device
    _check(w, "w", torch.int32, dev)
    N = w.shape[0]
    if w.dim() != 2 or w.shape[1] * 32 != K * bits:
        raise ValueError(f"w has shape {tuple(w.shape)}, expected ({N}, {K * bits // 32})")
    out = torch.empty((N, (K // group_size) * ((group_size + 4) // 5)), dtype=torch.uint8, device=dev)
    flag = torch.empty(1, dtype=torch.int32, device=dev)
    bq_t5_repack(w.data_ptr(), out.data_ptr(), N, K, bits, group_size, flag.data_ptr(), _stream_handle(dev))
    return out, bool(flag.item())


def spec_decode_verify(logits, draft, workspace=None, targets: bool = True):
    """Greedy verification of L draft tokens per sequence against the target
    logits [B][L+1][V] (fp16 or fp32): (accepted [B], next_token [B],
    target tokens [B][L+1] or None), int32 tensors.  workspace: a zeroed
    uint8 tensor of at least bq_spec_verify_workspace bytes, reused across
    calls (each call leaves it zero); allocated here when None."""
    torch = _torch()
    dev = logits.device
    if logits.dtype not in (torch.float16, torch.float32):
        raise TypeError(f"logits must be float16 or float32, got {logits.dtype}")
    _check(logits, "logits", logits.dtype, dev)
    if logits.dim() != 3:
        raise ValueError("logits must be [B][L+1][V]")
    B, rows, V = logits.shape
    L = rows - 1
    _check(draft, "draft", torch.int32, dev)
    if tuple(draft.shape) != (B, L):
        raise ValueError(f"draft has shape {tuple(draft.shape)}, expected {(B, L)}")
    need = bq_spec_verify_workspace(B, L, V)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", torch.uint8, dev)
    accepted = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    tgt = torch.empty((B, rows), dtype=torch.int32, device=dev) if targets else None
    bq_spec_decode_verify(logits.data_ptr(), DTYPE_F16 if logits.dtype == torch.float16 else DTYPE_F32,
                          draft.data_ptr() if L > 0 else None, B, L, V, accepted.data_ptr(), nxt.data_ptr(),
                          tgt.data_ptr() if tgt is not None else None, workspace.data_ptr(), workspace.numel(),
                          _stream_handle(dev))
    return accepted, nxt, tgt


class QuantizedWeight:
    """One layer's packed weights: w (int32 words for bits 1/2, uint8 t5
    bytes), fp16 scales [N][K/gs], fp16 biases or None (implied bias).  The
    symmetric-bias check runs once, on first use."""

    def __init__(self, w, scales, biases, bits: int, group_size: int):
        self.w, self.scales, self.biases = w, scales, biases
        self.bits, self.group_size = bits, group_size
        self.N = scales.shape[0]
        self.K = scales.shape[1] * group_size
        self._sym = None if biases is not None else True

    @property
    def sym(self) -> bool:
        if self._sym is None:
            self._sym = sym_check(self.scales, self.biases, self.bits, self.group_size)
        return self._sym


    def to_t5(self) -> "QuantizedWeight":
        """The same layer in t5 bytes (bits 1/2 with stored biases and codes
        0..2 only).  The biases are dropped when every one equals -scale
        (the t5 implied bias), else kept."""
        if self.bits == BITS_T5:
            return self
        if self.biases is None:
            raise ValueError("to_t5 needs stored biases (the implied 1/2-bit bias is not -scale)")
        w5, ternary = t5_repack(self.w, self.bits, self.group_size, self.K)
        if not ternary:
            raise ValueError("the layer has code 3, which t5 cannot hold")
        implied = sym_check(self.scales, self.biases, BITS_T5, self.group_size)
        return QuantizedWeight(w5, self.scales, None if implied else self.biases, BITS_T5, self.group_size)


def linear(x, qw: QuantizedWeight, out=None, sym: Optional[bool] = None, workspace=None):
    """y = x . W^T for any number of rows, routed as bq_linear does (bits
    1/2: the fused qmm from QMM_MIN_M rows when the product has
    QMM_MIN_TILES tiles, else passes of up to 5 rows through the wide or
    symmetric kernel; t5: wide passes below T5_QMM_MIN_M rows, the fused
    qmm from there when the product has T5_QMM_MIN_TILES tiles, or
    T5_QMM_FEW_TILES from T5_QMM_FEW_MIN_M rows).  sym
    defaults to the layer's checked symmetric-bias property.  workspace:
    None (bq_linear), a device tensor, or "auto" (allocated here, of the
    bq_qmm_workspace size): routed as bq_linear_ws, the fused product with
    K split from QMM_MIN_M / T5_QMM_MIN_M rows."""
    use_sym = qw.sym if sym is None else sym
    M, K = x.shape
    if K != qw.K:
        raise ValueError(f"x has K = {K}, the weight {qw.K}")
    torch = _torch()
    dev = qw.w.device
    _check(qw.w, "w", torch.uint8 if qw.bits == BITS_T5 else torch.int32, dev)
    _check(qw.scales, "scales", torch.float16, dev)
    if qw.biases is not None:
        _check(qw.biases, "biases", torch.float16, dev)
    _check(x, "x", torch.float16, dev)
    if out is None:
        out = torch.empty((M, qw.N), dtype=torch.float16, device=dev)
    else:
        _check(out, "out", torch.float16, dev)
        if tuple(out.shape) != (M, qw.N):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, qw.N)}")
    args = (x.data_ptr(), qw.w.data_ptr(), qw.scales.data_ptr(),
            qw.biases.data_ptr() if qw.biases is not None else None, out.data_ptr(), M, qw.N, qw.K, qw.bits,
            qw.group_size, LINEAR_SYM if use_sym else 0)
    if workspace is None:
        bq_linear(*args, _stream_handle(dev))
        return out
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be None, 'auto' or a tensor, got {workspace!r}")
        need = bq_qmm_workspace(M, qw.N, qw.K, qw.bits, qw.group_size)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    bq_linear_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(dev))
    return out


__all__ = [
    "ABI_VERSION", "ALL_SYMBOLS", "BITS_T5", "BQError", "DISPATCH_POINTS", "ENTRY_POINTS", "LIB_PATH",
    "LINEAR_SYM", "MAX_WIDE_M", "QMM_MIN_M", "QMM_MIN_TILES", "QuantizedWeight", "ROUTES", "T5_QMM_FEW_MIN_M", "T5_QMM_FEW_TILES", "T5_QMM_MIN_M", "T5_QMM_MIN_TILES", "bq_abi_version", "bq_dequant",
    "bq_linear", "bq_linear_route", "bq_qmm", "bq_qmv", "bq_qmv_sym", "bq_qmv_wide", "bq_sym_check", "bq_t5_qmm",
    "bq_t5_qmv", "bq_t5_qmv_wide", "dequant", "linear", "load_library", "qmm", "qmv", "qmv_sym", "qmv_wide",
    "DTYPE_F16", "DTYPE_F32", "SPEC_MAX_DRAFT", "bq_spec_decode_verify", "bq_spec_decode_verify_noalloc",
    "bq_spec_verify_workspace", "bq_qmm_workspace", "bq_qmm_ws", "bq_t5_qmm_ws", "qmm_ws", "t5_qmm_ws",
    "bq_linear_ws",
    "bq_t5_repack", "spec_decode_verify", "strerror", "sym_check", "t5_qmm", "t5_qmv", "t5_qmv_wide", "t5_repack",
]
