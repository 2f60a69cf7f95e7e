"""Plain CPU oracle for group-wise affine low-bit QMV (fp64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library; both are fed by the generators in ``synth``.

Source of the method ("the article"): the web article "oMLX Bonsai
自定义内核: Qwen 系列快速 QMV 路径完整解析" (cnnetsun.cn).  Sections cited:

* section 一 -- single-token decode reads every weight once and is
  memory-bandwidth bound;
* section 二, path 1 (qmv_fast) -- 1-bit affine weights packed 32 to a
  uint32, unpacked by shifting and dotted with the activation; 1-bit prefill
  dequantizes to float16 and then multiplies;
* section 二, path 2 (qmv_wide) -- M = 2..5 activation rows share one read
  of the weights; the symmetric variant applies when bias = -scale * ratio
  and then the bias tensor is not read;
* section 二, path 3 (t5) -- ternary codes {0,1,2} stored in uint8, 13/26
  bytes per weight group, about 1.585 bit per weight.

Readings where the article is silent:

* R1 weight matrix is ``W[N][K]`` (output x input, the QuantizedLinear
  convention); groups of ``gs`` consecutive weights along K share one fp16
  scale and one fp16 bias: ``w = scale * q + bias``; ``y = x @ W^T``.
* R2 uint32 packing is LSB-first along K: code k lives in word
  ``k*bits // 32`` at bit ``(k*bits) % 32``.
* R3 t5: the ``ceil(gs/5)`` bytes of a group hold its codes five to a byte,
  least-significant base-3 digit first (code ``5j+i`` of the group is digit
  ``i`` of byte ``j``); unused digits of the last byte are zero.
* R4 symmetric ratio: ``r = (2^bits - 1) / 2`` (0.5 for 1-bit, 1.5 for
  2-bit), i.e. the codes are centred; t5 with no stored bias uses
  ``bias = -scale`` (r = 1), giving weights in {-s, 0, +s}.
* R5 acceptance: ``|y - y_ref| <= 1e-3 * sum_k |x_k w_k| + 1e-3 * |y_ref|``.

Every function computes in float64 from exactly converted fp16 inputs.
"""
from __future__ import annotations

import math

import numpy as np

T5_MAX_BYTE = 242  # 3^5 - 1


# --------------------------------------------------------------------------
# Formats
# --------------------------------------------------------------------------
def bits_of(fmt: str) -> int:
    return {"u1": 1, "u2": 2}[fmt]


def t5_group_bytes(group_size: int) -> int:
    """Bytes per t5 group: five codes per byte, the last byte partly used
    (13 bytes for 64 weights, 26 for 128 -- article, section 二 path 3)."""
    return -(-group_size // 5)


def sym_ratio(fmt: str) -> float:
    """Ratio r of the symmetric identity bias = -scale * r (reading R4)."""
    if fmt == "t5":
        return 1.0
    return (2 ** bits_of(fmt) - 1) / 2.0


# --------------------------------------------------------------------------
# uint32 packing (article section 二 path 1; reading R2)
# --------------------------------------------------------------------------
def unpack_words(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Codes ``[N][K]`` (uint8) from LSB-first uint32 words ``[N][K*bits/32]``."""
    words = np.asarray(words, dtype=np.uint32)
    k = np.arange(K)
    word_idx = (k * bits) // 32
    shift = ((k * bits) % 32).astype(np.uint32)
    mask = np.uint32((1 << bits) - 1)
    return ((words[:, word_idx] >> shift) & mask).astype(np.uint8)


def unpack_words_scalar(words, bits: int, K: int):
    """Pure-Python loop version of :func:`unpack_words` (tiny inputs only)."""
    out = []
    for row in words:
        codes = []
        for k in range(K):
            word = int(row[(k * bits) // 32])
            codes.append((word >> ((k * bits) % 32)) & ((1 << bits) - 1))
        out.append(codes)
    return out


def pack_words(codes: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of :func:`unpack_words`."""
    codes = np.asarray(codes, dtype=np.uint64)
    N, K = codes.shape
    per = 32 // bits
    if K % per:
        raise ValueError("K must fill whole words")
    if codes.max(initial=0) >= (1 << bits):
        raise ValueError("code out of range")
    c = codes.reshape(N, K // per, per)
    words = np.zeros((N, K // per), dtype=np.uint64)
    for i in range(per):
        words |= c[:, :, i] << np.uint64(i * bits)
    return words.astype(np.uint32)


# --------------------------------------------------------------------------
# t5 ternary bytes (article section 二 path 3; reading R3)
# --------------------------------------------------------------------------
def t5_unpack(data: np.ndarray, K: int, group_size: int) -> np.ndarray:
    """Codes ``[N][K]`` in {0,1,2} from t5 bytes ``[N][(K/gs)*ceil(gs/5)]``."""
    data = np.asarray(data, dtype=np.uint8)
    if data.size and int(data.max()) > T5_MAX_BYTE:
        raise ValueError("t5 byte above 242 is not a valid base-3 word")
    gb = t5_group_bytes(group_size)
    k = np.arange(K)
    g, r = divmod(k, group_size)
    j, i = divmod(r, 5)
    byte = data[:, g * gb + j].astype(np.int64)
    return ((byte // (3 ** i)) % 3).astype(np.uint8)


def t5_unpack_scalar(data, K: int, group_size: int):
    """Pure-Python loop version of :func:`t5_unpack` (tiny inputs only)."""
    gb = t5_group_bytes(group_size)
    out = []
    for row in data:
        codes = []
        for k in range(K):
            g, r = divmod(k, group_size)
            j, i = divmod(r, 5)
            b = int(row[g * gb + j])
            if b > T5_MAX_BYTE:
                raise ValueError("invalid t5 byte")
            for _ in range(i):
                b //= 3
            codes.append(b % 3)
        out.append(codes)
    return out


def t5_pack(codes: np.ndarray, group_size: int) -> np.ndarray:
    """Inverse of :func:`t5_unpack`; unused digits of a group's last byte are 0."""
    codes = np.asarray(codes, dtype=np.int64)
    N, K = codes.shape
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    if codes.size and (codes.min() < 0 or codes.max() > 2):
        raise ValueError("t5 codes must be in {0,1,2}")
    gb = t5_group_bytes(group_size)
    G = K // group_size
    padded = np.zeros((N, G, gb * 5), dtype=np.int64)
    padded[:, :, :group_size] = codes.reshape(N, G, group_size)
    digits = padded.reshape(N, G, gb, 5)
    weights = 3 ** np.arange(5)
    return (digits * weights).sum(axis=-1).astype(np.uint8).reshape(N, G * gb)


# --------------------------------------------------------------------------
# Codes of any format
# --------------------------------------------------------------------------
def codes_of(fmt: str, w: np.ndarray, K: int, group_size: int) -> np.ndarray:
    if fmt == "t5":
        return t5_unpack(w, K, group_size)
    return unpack_words(w, bits_of(fmt), K)


def effective_biases(fmt: str, scales: np.ndarray, biases) -> np.ndarray:
    """fp64 biases: the stored ones, or the implied ``-scale * r`` when none is
    stored (symmetric variant, article section 二 path 2; t5, reading R4)."""
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if biases is None:
        return -s * sym_ratio(fmt)
    return np.asarray(biases, dtype=np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# Dequantization (article section 二 path 1: w = scale * q + bias per group)
# --------------------------------------------------------------------------
def dequant_f64(codes: np.ndarray, scales: np.ndarray, biases_f64: np.ndarray,
                group_size: int) -> np.ndarray:
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), group_size, axis=1)
    b = np.repeat(np.asarray(biases_f64, dtype=np.float64), group_size, axis=1)
    return s * codes.astype(np.float64) + b


def dequant_f16(codes, scales, biases_f64, group_size) -> np.ndarray:
    """fp16 weights, each rounded once (to nearest even) from the exact value."""
    return dequant_f64(codes, scales, biases_f64, group_size).astype(np.float16)


def weights_f64(fmt: str, w, scales, biases, K: int, group_size: int, rows=None) -> np.ndarray:
    """Dequantized fp64 weight rows (all rows, or the listed ``rows``)."""
    if rows is not None:
        w = np.asarray(w)[rows]
        scales = np.asarray(scales)[rows]
        biases = None if biases is None else np.asarray(biases)[rows]
    codes = codes_of(fmt, w, K, group_size)
    return dequant_f64(codes, scales, effective_biases(fmt, scales, biases), group_size)


# --------------------------------------------------------------------------
# The product (article section 一 / 二: y = x . W^T over fp16 activations)
# --------------------------------------------------------------------------
def qmv_f64(x: np.ndarray, W64: np.ndarray) -> np.ndarray:
    """``y[m][n] = sum_k x[m][k] * W[n][k]`` in fp64."""
    return np.asarray(x, dtype=np.float16).astype(np.float64) @ W64.T


def abs_mass(x: np.ndarray, W64: np.ndarray) -> np.ndarray:
    """``sum_k |x[m][k] * W[n][k]|`` -- the scale of the acceptance bound
    (reading R5): the sum of the element-wise absolute products."""
    return np.abs(np.asarray(x, dtype=np.float16).astype(np.float64)) @ np.abs(W64).T


def qmv_reference(fmt: str, x, w, scales, biases, K: int, group_size: int, rows=None):
    """(y_ref, mass) for all output rows or the listed ``rows``."""
    W64 = weights_f64(fmt, w, scales, biases, K, group_size, rows)
    return qmv_f64(x, W64), abs_mass(x, W64)


def qmv_brute(x, codes, scales, biases_f64, group_size):
    """Scalar triple loop (tiny inputs): y[m][n] = sum_k x*(s*q+b)."""
    M, K = len(x), len(x[0])
    N = len(codes)
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                g = k // group_size
                wk = float(scales[n][g]) * float(codes[n][k]) + float(biases_f64[n][g])
                acc += float(x[m][k]) * wk
            y[m][n] = acc
    return y


# --------------------------------------------------------------------------
# Acceptance (reading R5)
# --------------------------------------------------------------------------
RTOL_MASS = 1e-3
RTOL_VALUE = 1e-3


def tolerance(y_ref: np.ndarray, mass: np.ndarray) -> np.ndarray:
    return RTOL_MASS * mass + RTOL_VALUE * np.abs(y_ref)


def check_close(y, y_ref, mass):
    """Returns (ok, worst_ratio): ratio = |y - y_ref| / tolerance, worst over
    all elements; ok iff every element is finite and within tolerance."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return False, math.inf
    tol = tolerance(y_ref, mass)
    ratio = np.abs(y - y_ref) / np.maximum(tol, np.finfo(np.float64).tiny)
    worst = float(ratio.max(initial=0.0))
    return worst <= 1.0, worst


# --------------------------------------------------------------------------
# Byte accounting (article section 四: weights + scales + biases +
# activations, implied biases count 0) -- plus the fp16 output y.
# --------------------------------------------------------------------------
def algorithmic_bytes(fmt: str, M: int, N: int, K: int, group_size: int,
                      bias_stored: bool) -> int:
    G = K // group_size
    if fmt == "t5":
        wbytes = N * G * t5_group_bytes(group_size)
    else:
        wbytes = N * K * bits_of(fmt) // 8
    sb = N * G * 2 * (2 if bias_stored else 1)
    return wbytes + sb + M * K * 2 + M * N * 2
