"""Pins of the speculative-verification oracle (CPU): worked cases whose
answer follows from the definition by inspection, invariants, the scalar
loop against the vectorized version, and planted mistakes that some pin must
catch."""
import numpy as np
import pytest

import oracle.spec_oracle as S
import synth


def pin_hand_cases():
    # B = 1, L = 3, V = 4: targets 2, 0, 3, 1 by inspection
    lg = np.array([[[0.1, 0.2, 0.9, 0.0],
                    [0.5, -1.0, 0.25, 0.0],
                    [0.0, 0.0, 0.0, 0.125],
                    [-2.0, 3.0, 1.0, 2.5]]], dtype=np.float16)
    a, n, t = S.spec_verify(lg, np.array([[2, 0, 1]]))
    assert t.tolist() == [[2, 0, 3, 1]]
    assert (a.tolist(), n.tolist()) == ([2], [3])          # rejected at 2, correction 3
    a, n, _ = S.spec_verify(lg, np.array([[2, 0, 3]]))
    assert (a.tolist(), n.tolist()) == ([3], [1])          # all accepted, bonus token 1
    a, n, _ = S.spec_verify(lg, np.array([[1, 0, 3]]))
    assert (a.tolist(), n.tolist()) == ([0], [2])          # first token rejected


def pin_no_draft():
    lg = np.array([[[1.0, 5.0, 2.0]], [[7.0, 5.0, 2.0]]], dtype=np.float32)
    a, n, t = S.spec_verify(lg, np.zeros((2, 0), np.int32))
    assert a.tolist() == [0, 0] and n.tolist() == [1, 0]


def pin_ties_zero_nan_inf():
    row = lambda *v: np.array(v, dtype=np.float32)
    cases = [
        (row(1, 3, 3, 2), 1),                      # equal maxima: the lowest index
        (row(-0.0, 0.0, -1), 0),                   # -0 == +0
        (row(0.0, -0.0, -1), 0),
        (row(-np.inf, -np.inf), 0),
        (row(1, np.inf, 2, np.inf), 1),
        (row(1, np.nan, 2, np.nan), 1),            # NaN is the largest, first NaN wins
        (row(np.inf, 3, np.nan), 2),
        (row(-5, -4, -4.5), 1),
    ]
    for r, want in cases:
        lg = r.reshape(1, 1, -1)
        assert S.target_tokens(lg).tolist() == [[want]], (r, want)
        assert S.target_tokens(lg.astype(np.float16)).tolist() == [[want]], (r, want)


def pin_scalar_equals_vector():
    rng = np.random.default_rng(3)
    for trial in range(40):
        B, L, V = rng.integers(1, 4), rng.integers(0, 5), rng.integers(1, 7)
        lg = rng.integers(-2, 3, size=(B, L + 1, V)).astype(np.float32)   # many ties
        lg[rng.random(lg.shape) < 0.05] = np.nan
        draft = rng.integers(0, V, size=(B, L))
        a, n, t = S.spec_verify(lg, draft)
        a2, n2, t2 = S.spec_verify_scalar(lg.tolist(), draft.tolist())
        assert a.tolist() == a2 and n.tolist() == n2 and t.tolist() == t2


def pin_invariants_on_planted_inputs():
    for seed in range(5):
        s = synth.make_spec_inputs(4, 6, 500, seed=seed)
        a, n, t = S.spec_verify(s.logits, s.draft)
        assert np.array_equal(t, s.planted)
        assert np.array_equal(a, s.agree)
        for b in range(4):
            assert np.array_equal(s.draft[b, :a[b]], t[b, :a[b]])
            if a[b] < 6:
                assert s.draft[b, a[b]] != t[b, a[b]]
            assert n[b] == t[b, a[b]]


PINS = [pin_hand_cases, pin_no_draft, pin_ties_zero_nan_inf, pin_scalar_equals_vector,
        pin_invariants_on_planted_inputs]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_spec_pins_hold(pin):
    pin()


# planted mistakes
def _last_of_ties(logits):
    lg = np.asarray(logits).astype(np.float64)
    V = lg.shape[-1]
    return V - 1 - np.argmax(lg[..., ::-1], axis=-1)


def _nan_ignored(logits):
    lg = np.asarray(logits).astype(np.float64)
    return np.nanargmax(np.where(np.isnan(lg), -np.inf, lg), axis=-1)


def _accept_one_more(logits, draft):
    a, n, t = ORIGINAL(logits, draft)
    L = t.shape[1] - 1
    a = np.minimum(a + 1, L)
    return a, t[np.arange(t.shape[0]), a], t


def _next_is_draft(logits, draft):
    a, n, t = ORIGINAL(logits, draft)
    d = np.asarray(draft).reshape(t.shape[0], -1)
    L = t.shape[1] - 1
    n = np.where(a < L, d[np.arange(t.shape[0]), np.minimum(a, max(L - 1, 0))] if L else n, n)
    return a, n, t


ORIGINAL = S.spec_verify
MUTANTS = {
    "last_of_ties": ("target_tokens", _last_of_ties),
    "nan_ignored": ("target_tokens", _nan_ignored),
    "accept_one_more": ("spec_verify", _accept_one_more),
    "next_is_draft": ("spec_verify", _next_is_draft),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_spec_pins_catch(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(S, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
