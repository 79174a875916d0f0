"""fp64 CPU oracle for the batched Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the test suite, the smoke check and the benchmark's CPU-baseline leg call
it.  It shares no code with the HIP library (no kernels, headers, constants or
helpers); the two meet only in the seeded inputs of the `workloads` module.

Everything is computed in float64 with numpy; `@` (BLAS dgemm) is the only
library primitive used as a step.  There is no blocking, fusion or reordering
beyond what the definitions below state.

Sources (page title, then section):
  [CS]  "Muon Custom Sizing" walkthrough of the modded-nanogpt 124M record
        (2025-09-23): section 1 (Muon = SGD-momentum, then Newton-Schulz
        orthogonalisation of each 2-D update), section 2.3 (attn weights viewed
        as 4 independent blocks before NS; the quintic constants; 5 iterations),
        section 3.1 (the (hdim, 4*dim) -> (4, hdim, dim) contiguous view),
        section 4 (momentum lerp forms, decoupled weight decay lr*wd*wd_mul,
        effective lr lr*max(1, rows/cols)^0.5*lr_mul).
  [PG]  parameter-golf train_gpt.py walkthrough, Part 1 "how the Muon optimizer
        works": the zeropower_via_newtonschulz5 body (cast, Frobenius
        normalisation, A = X X^T, B = b A + c A A, X = a X + B X) and the
        max(1, m/n)^0.5 aspect correction.

Readings where the pages are silent or garbled (each also listed in the design doc):
  R1  The NS update is X <- aX + (bA + cA^2)X with A = X X^T, as the PG code
      states; the CS prose form of it lost its plus signs in extraction.
  R2  The input is normalised once, by its Frobenius norm, before the loop (PG
      code).  The CS prose says "spectral norm each time"; the code form wins
      because it is the one that the rest of both pages supports.
  R3  The normaliser is ||Y||_F + eps with eps = 1e-7 (not printed); a zero
      block therefore maps to zero.
  R4  A block with more rows than columns is processed transposed (wide side
      as the inner dimension); in exact arithmetic this gives the same result.
  R5  Normalisation is per NS block: with the attn view each of the 4 blocks
      has its own norm.
  R6  The attn view is the row-major reinterpretation of a stored R x C matrix
      as view_blocks contiguous blocks of R x (C / view_blocks).
  R7  The aspect factor uses the stored parameter shape (R, C).
  R8  Momentum uses the lerp forms of CS section 4 for every workload; the
      look-ahead uses the updated buffer.  Without Nesterov the update
      direction is the buffer itself.
  R9  Weight decay is decoupled and uses the base lr: P <- P(1 - lr wd wd_mul)
      - lr max(1,R/C)^0.5 lr_mul O.
  R10 Scalars cross the C ABI as float32, so the oracle rounds lr, weight
      decay, momentum, lr_mul and wd_mul through float32 before using them in
      float64.  The NS coefficients are used as the decimal values printed.

Every function here is pinned by tests against closed forms and invariants
(SVD closed form of the iteration, rank-1 and scaled-orthogonal special cases,
momentum closed forms, hand-computed update values); none is parity unpinned.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

# [CS] section 2.3: quintic coefficients (a, b, c) and 5 iterations.
NS_COEFFS: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315)
NS_STEPS: int = 5
NS_EPS: float = 1e-7  # reading R3


def _f32(x: float) -> float:
    """Round a Python scalar through float32 (reading R10)."""
    return float(np.float32(x))


def nesterov_momentum(grad, buf, momentum: float, nesterov: bool = True):
    """One momentum update, [CS] section 4.

    buf <- buf + (1 - mu) (grad - buf)      (buffer lerp towards the gradient)
    upd <- grad + mu (buf_new - grad)       (Nesterov look-ahead, reading R8)
    Returns (buf_new, upd) in float64.
    """
    g = np.asarray(grad, dtype=np.float64)
    m = np.asarray(buf, dtype=np.float64)
    mu = _f32(momentum)
    m_new = m + (1.0 - mu) * (g - m)
    if nesterov:
        upd = g + mu * (m_new - g)
    else:
        upd = m_new
    return m_new, upd


def view_blocks_of(stored: np.ndarray, view_blocks: int) -> np.ndarray:
    """Reading R6: a stored R x C matrix as view_blocks contiguous R x (C/view_blocks) blocks."""
    R, C = stored.shape
    if C % view_blocks != 0:
        raise ValueError("cols must be divisible by view_blocks")
    return np.ascontiguousarray(stored).reshape(view_blocks, R, C // view_blocks)


def unview_blocks(blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    return np.ascontiguousarray(blocks).reshape(rows, cols)


def newton_schulz(Y, steps: int = NS_STEPS, coeffs: Tuple[float, float, float] = NS_COEFFS,
                  eps: float = NS_EPS) -> np.ndarray:
    """Quintic Newton-Schulz orthogonalisation of one block, [PG] Part 1.

    X = Y / (||Y||_F + eps)                  (readings R2, R3)
    repeat `steps` times:
        A = X X^T
        B = b A + c A A
        X = a X + B X
    A tall block is processed as its transpose (reading R4).
    """
    Y = np.asarray(Y, dtype=np.float64)
    if Y.ndim != 2:
        raise ValueError("newton_schulz expects a 2-D block")
    a, b, c = coeffs
    tall = Y.shape[0] > Y.shape[1]
    X = Y.T if tall else Y
    X = X / (np.linalg.norm(X) + eps)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def ns_batched(X, view_blocks: int = 1, steps: int = NS_STEPS,
               coeffs: Tuple[float, float, float] = NS_COEFFS, eps: float = NS_EPS) -> np.ndarray:
    """NS of every block of a stored batch [B, R, C] (attn view per reading R6)."""
    X = np.asarray(X, dtype=np.float64)
    Bn, R, C = X.shape
    out = np.empty_like(X)
    for i in range(Bn):
        blocks = view_blocks_of(X[i], view_blocks)
        ob = np.stack([newton_schulz(blk, steps, coeffs, eps) for blk in blocks])
        out[i] = unview_blocks(ob, R, C)
    return out


def aspect_factor(rows: int, cols: int) -> float:
    """max(1, rows/cols)^0.5 of the stored shape, [PG] Part 1 and [CS] section 4."""
    return max(1.0, rows / cols) ** 0.5


def muon_update(P, O, lr: float, weight_decay: float, lr_mul: float = 1.0,
                wd_mul: float = 1.0) -> np.ndarray:
    """P <- P (1 - lr wd wd_mul) - lr max(1,R/C)^0.5 lr_mul O, [CS] section 4 (reading R9)."""
    P = np.asarray(P, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    R, C = P.shape[-2:]
    lr, wd, lrm, wdm = _f32(lr), _f32(weight_decay), _f32(lr_mul), _f32(wd_mul)
    return P - (lr * wd * wdm) * P - (lr * aspect_factor(R, C) * lrm) * O


def muon_step(P, G, M, *, lr: float, weight_decay: float, momentum: float,
              nesterov: bool = True, lr_mul: float = 1.0, wd_mul: float = 1.0,
              view_blocks: int = 1, ns_steps: int = NS_STEPS,
              coeffs: Tuple[float, float, float] = NS_COEFFS, eps: float = NS_EPS):
    """One Muon step on a stored batch [B, R, C].

    P: parameters, G: gradients (already decoded to float), M: momentum buffers.
    Returns (P_new, M_new, O) in float64, where O is the orthogonalised update
    (before lr and aspect scaling).
    """
    P = np.asarray(P, dtype=np.float64)
    M_new, U = nesterov_momentum(G, M, momentum, nesterov)
    O = ns_batched(U, view_blocks, ns_steps, coeffs, eps)
    P_new = np.stack([muon_update(P[i], O[i], lr, weight_decay, lr_mul, wd_mul)
                      for i in range(P.shape[0])])
    return P_new, M_new, O
