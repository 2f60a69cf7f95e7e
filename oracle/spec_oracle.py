"""Plain CPU oracle for speculative-decoding verification.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library.

Source: the web article "oMLX Bonsai 自定义内核: Qwen 系列快速 QMV 路径完整
解析", section 三: ``spec_decode_verify`` fuses three steps into one kernel --
compare the draft tokens, count the accepted length, produce the correction
token.  The article gives no formulas; the reading taken here (R10) is
greedy verification:

* ``t[i] = argmax_v logits[i][v]`` for the L+1 positions the target model
  scored (the L draft positions and the one after them); among equal maxima
  the lowest index, ``-0 == +0``, and a NaN counts as the largest value (the
  first NaN wins) -- numpy's ``argmax`` convention;
* accepted length ``a`` = the first ``i < L`` with ``draft[i] != t[i]``, or
  ``L`` when every draft token matches;
* next token ``t[a]``: the correction token, or the bonus token when all
  draft tokens were accepted.

The argmax decides an integer from floating point, so it compares the
logits in their own precision (fp16 and fp32 values convert exactly to
fp64, which preserves their order).
"""
from __future__ import annotations

import numpy as np


def target_tokens(logits: np.ndarray) -> np.ndarray:
    """``argmax`` over the last axis of ``[B][L+1][V]`` logits (int64)."""
    lg = np.asarray(logits)
    return np.argmax(lg.astype(np.float64), axis=-1)


def spec_verify(logits: np.ndarray, draft: np.ndarray):
    """(accepted [B], next_token [B], targets [B][L+1]) for ``[B][L+1][V]``
    logits and ``[B][L]`` draft tokens."""
    t = target_tokens(logits)
    draft = np.asarray(draft).reshape(t.shape[0], t.shape[1] - 1)
    B, rows = t.shape
    L = rows - 1
    accepted = np.full(B, L, dtype=np.int64)
    for b in range(B):
        for i in range(L):
            if draft[b, i] != t[b, i]:
                accepted[b] = i
                break
    nxt = t[np.arange(B), accepted]
    return accepted, nxt, t


def spec_verify_scalar(logits, draft):
    """Pure-Python loops of :func:`spec_verify` (tiny inputs only): a linear
    scan for each argmax with NaN as the largest value and ``>`` so that the
    first of equal values stays."""
    import math
    out_a, out_n, out_t = [], [], []
    for b, rows in enumerate(logits):
        ts = []
        for row in rows:
            best_i, best_v = 0, row[0]
            for i, v in enumerate(row):
                bv = float(best_v)
                fv = float(v)
                if math.isnan(bv):
                    continue
                if math.isnan(fv) or fv > bv:
                    best_i, best_v = i, v
            ts.append(best_i)
        L = len(rows) - 1
        a = L
        for i in range(L):
            if int(draft[b][i]) != ts[i]:
                a = i
                break
        out_a.append(a)
        out_n.append(ts[a])
        out_t.append(ts)
    return out_a, out_n, out_t
