"""The pins must reject plausible mistakes.

Each mutant is a copy of an oracle function with one mistake planted in it (on
the CPU, in this file only).  The closed-form checks used by the pin tests must
flag every mutant; if one slipped through, the pins would not be pinning it.
"""
import numpy as np
import pytest

import oracle
from test_oracle_pins import closed_form_ns, p_scalar, rel, semi_orthogonal


def _ns_mutant(kind):
    a0, b0, c0 = oracle.NS_COEFFS

    def ns(Y, steps=5, coeffs=oracle.NS_COEFFS, eps=oracle.NS_EPS):
        a, b, c = coeffs
        Y = np.asarray(Y, np.float64)
        tall = Y.shape[0] > Y.shape[1]
        X = Y.T if (tall and kind != "no_orient") else Y
        if kind == "spectral_once":
            X = X / (np.linalg.norm(X, 2) + eps)
        else:
            X = X / (np.linalg.norm(X) + eps)
        for _ in range(steps):
            if kind == "spectral_each":
                X = X / np.linalg.norm(X, 2)
            A = X @ X.T
            if kind == "drop_c":
                B = b * A
            elif kind == "sign_b":
                B = -b * A + c * (A @ A)
            elif kind == "c_times_A":
                B = b * A + c * A
            else:
                B = b * A + c * (A @ A)
            if kind == "xb":
                X = a * X + X @ B if X.shape[0] == X.shape[1] else a * X + B @ X
            elif kind == "drop_a":
                X = B @ X
            else:
                X = a * X + B @ X
        return X.T if (tall and kind != "no_orient") else X
    return ns


@pytest.mark.parametrize("kind", ["drop_c", "sign_b", "c_times_A", "xb", "drop_a",
                                  "spectral_once", "spectral_each"])
def test_closed_form_rejects_ns_mutants(kind):
    rng = np.random.default_rng(21)
    worst = 0.0
    with np.errstate(all="ignore"):
        for shape in [(9, 9), (6, 14), (14, 6)]:
            Y = rng.standard_normal(shape)
            e = rel(_ns_mutant(kind)(Y), closed_form_ns(Y))
            worst = np.inf if not np.isfinite(e) else max(worst, e)
    assert worst > 1e-3, f"mutant {kind} not detected"


def test_closed_form_accepts_unmutated_copy():
    rng = np.random.default_rng(21)
    for shape in [(9, 9), (6, 14), (14, 6)]:
        Y = rng.standard_normal(shape)
        assert rel(_ns_mutant("none")(Y), closed_form_ns(Y)) < 1e-12


def test_momentum_pin_rejects_old_buffer_lookahead():
    # Using the old buffer in the look-ahead gives U_1 = (1 - mu) g, not (1 - mu^2) g.
    g = np.ones((2, 2))
    mu = float(np.float32(0.95))
    _, U = oracle.nesterov_momentum(g, np.zeros_like(g), 0.95)
    wrong = g + mu * (np.zeros_like(g) - g)
    assert rel(U, (1 - mu ** 2) * g) < 1e-15
    assert rel(wrong, (1 - mu ** 2) * g) > 0.3


def test_view_pin_rejects_column_slices():
    rng = np.random.default_rng(22)
    R, C, v = 8, 16, 4
    stored = rng.standard_normal((R, C))
    good = oracle.ns_batched(stored[None], view_blocks=v)[0]
    cols = np.concatenate([oracle.newton_schulz(stored[:, k * 4:(k + 1) * 4]) for k in range(v)],
                          axis=1)
    assert rel(cols, good) > 1e-2
    # and the correct reading equals per-block closed forms of the contiguous blocks
    blocks = stored.reshape(-1).reshape(v, R, C // v)
    want = np.stack([closed_form_ns(b) for b in blocks]).reshape(R, C)
    assert rel(good, want) < 1e-12


def test_aspect_pin_rejects_inverted_ratio():
    # 4 x 1 stored shape: the right factor is 2; max(1, C/R)^0.5 would give 1.
    P = np.zeros((4, 1))
    O = np.ones((4, 1))
    got = oracle.muon_update(P, O, lr=1.0, weight_decay=0.0)
    assert np.all(got == -2.0)
    assert p_scalar(1.0, oracle.NS_COEFFS, 5) != pytest.approx(1.0, abs=0.1)
    Q = semi_orthogonal(rng := np.random.default_rng(1), 4, 8)
    assert rel(oracle.newton_schulz(Q, eps=0.0), p_scalar(0.5, oracle.NS_COEFFS, 5) * Q) < 1e-12
