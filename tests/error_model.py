"""bf16 error model of the GPU path (test infrastructure, CPU only).

The HIP kernels round to bf16 (nearest, ties to even) at every stored
output: the cast of the update U to the first iterate, the Gram matrix A,
the polynomial B' = aI + bA + cA A, and each new iterate.  Their fp32
accumulation is far more precise than bf16 (about sqrt(K) 2^-24 against
2^-9), so the GPU result should sit where a pipeline with those roundings
and exact accumulation puts it.  This module is that pipeline: the quintic
Newton-Schulz iteration of the parameter-golf walkthrough, Part 1
(A = X X^T, B = bA + cA A, X = aX + BX, after X / (|X|_F + eps)), with the
coefficients of the "Muon Custom Sizing" walkthrough, section 2.3, written
the way the kernels arrange it:

* the Frobenius normalisation is folded into the first iteration: the Gram
  stores the unscaled A0 = X X^T and yields s^2 = trace(X X^T) (the sum of
  the squares of the bf16 values X holds; for ACCURATE those of the hi plane),
  the polynomial forms a I + b s^-2 A0 + c s^-4 A0 A0 and B X scales by s^-1,
  so X0 = U / s is never rounded (with zero iterations the update is U / s
  with s from U itself);
* aX rides on B''s diagonal (aX + BX = (aI + B) X), so a is rounded with B;
* FAST keeps every operand in bf16; ACCURATE keeps B' and X as bf16 hi + lo
  pairs and forms B' X as Bh Xh + Bh Xl + Bl Xh (the Gram uses Xh only).

With rounding switched off the model is the method itself (an exact rewrite),
which tests/test_error_model_cpu.py checks against the fp64 oracle.  Mutants
(truncation instead of round-to-nearest, a dropped lo pass) show how far a
precision regression moves the predicted error.
"""
from __future__ import annotations

import numpy as np

COEFFS = (3.4445, -4.7750, 2.0315)
EPS = 1e-7


def round_bf16(x):
    """float64 -> nearest bf16 value (8 significant bits, ties to even)."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def trunc_bf16(x):
    """float64 -> bf16 by truncation toward zero (a mutant: not what the GPU does)."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


def no_rounding(x):
    return np.asarray(x, np.float64)


def ns_model(U, steps: int = 5, coeffs=COEFFS, eps: float = EPS, precision: str = "fast",
             rnd=round_bf16, drop_lo: bool = False):
    """Predicted GPU output O for one NS block U (float64 values of what the
    kernels read: bf16 x for NS-only calls, the fp32 update for a step).
    Returns O in U's orientation."""
    a, b, c = coeffs
    Y = np.asarray(U, np.float64)
    tall = Y.shape[0] > Y.shape[1]
    if tall:
        Y = Y.T
    m = Y.shape[0]
    eye = np.eye(m)
    if precision == "fast":
        X = rnd(Y)
        s = np.sqrt(np.sum(X * X)) + eps           # trace(X X^T): the squares of the values X holds
        for t in range(steps):
            sc = 1.0 / s if t == 0 else 1.0
            A = rnd(X @ X.T)
            B = rnd(a * eye + b * sc * sc * A + c * sc ** 4 * (A @ A))
            X = rnd((B @ X) * sc)
        O = X
    else:
        Xh = rnd(Y)
        Xl = 0.0 * Xh if drop_lo else rnd(Y - Xh)
        s = np.sqrt(np.sum(Xh * Xh)) + eps         # trace(Xh Xh^T): the Gram reads the hi plane
        for t in range(steps):
            sc = 1.0 / s if t == 0 else 1.0
            A = rnd(Xh @ Xh.T)
            v = a * eye + b * sc * sc * A + c * sc ** 4 * (A @ A)
            Bh = rnd(v)
            Bl = 0.0 * Bh if drop_lo else rnd(v - Bh)
            v = (Bh @ Xh + Bh @ Xl + Bl @ Xh) * sc
            Xh = rnd(v)
            Xl = 0.0 * Xh if drop_lo else rnd(v - Xh)
        O = rnd(Xh + Xl)
    if steps == 0:
        # the prep's sums of squares: of the bf16 values (FAST), of U (ACCURATE)
        O = rnd(X / s) if precision == "fast" else rnd((Xh + Xl) / (np.sqrt(np.sum(Y * Y)) + eps))
    return O.T if tall else O


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
