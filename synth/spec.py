"""Seeded inputs for speculative-decoding verification: target logits with a
planted winner per position and draft tokens that follow the winners for a
chosen number of positions.  Holds no arithmetic of the method: the winners
are planted (the winning logit is set above the range the others are drawn
from), not computed.  The vocabulary size of the workload is Qwen's,
151936."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QWEN_VOCAB = 151936


@dataclass
class SpecInputs:
    logits: np.ndarray   # [B][L+1][V] float16 or float32
    draft: np.ndarray    # [B][L] int32
    planted: np.ndarray  # [B][L+1] the planted winners
    agree: np.ndarray    # [B] how many leading draft tokens equal the winners


def make_spec_inputs(B: int, L: int, V: int, dtype=np.float16, seed: int = 0, agree=None) -> SpecInputs:
    """Logits uniform in [-1, 1), one entry per row set to 2 (the planted
    winner); draft[b][i] is the winner for i < agree[b], a different token
    at i = agree[b] (when < L) and uniform after that."""
    rng = np.random.default_rng(seed)
    logits = rng.uniform(-1.0, 1.0, size=(B, L + 1, V)).astype(dtype)
    planted = rng.integers(0, V, size=(B, L + 1)).astype(np.int64)
    logits[np.arange(B)[:, None], np.arange(L + 1)[None, :], planted] = 2.0
    if agree is None:
        agree = rng.integers(0, L + 1, size=B)
    agree = np.asarray(agree, dtype=np.int64).reshape(B)
    draft = rng.integers(0, V, size=(B, L)).astype(np.int32)
    for b in range(B):
        a = int(agree[b])
        draft[b, :a] = planted[b, :a]
        if a < L and V > 1:
            draft[b, a] = (planted[b, a] + 1 + rng.integers(0, V - 1)) % V
    return SpecInputs(logits, draft, planted, agree)
