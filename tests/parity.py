"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (per NS block unless stated):
  * relative Frobenius error of the NS output      <= 2e-2
  * max |sigma_i(O_gpu) - sigma_i(O_ref)|            <= 5e-2 (both sorted)
  * momentum buffer, relative Frobenius per matrix  <= 1e-6
  * parameters: |P_gpu - P_ref|_F <= sum over steps of 2e-2 |lr_eff O_ref|_F
                                     + 4 * steps * 2^-24 * max |P|_F
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads

NS_REL_TOL = 2e-2
SIGMA_TOL = 5e-2
MOMENTUM_TOL = 1e-6


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def torch_bf16_to_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def singular_values(block: np.ndarray) -> np.ndarray:
    b = np.asarray(block, np.float64)
    if b.shape[0] > b.shape[1]:
        b = b.T
    ev = np.linalg.eigvalsh(b @ b.T)
    return np.sqrt(np.clip(ev, 0.0, None))[::-1]


def block_errors(got_stored: np.ndarray, ref_stored: np.ndarray, view_blocks: int, sigma: bool = True):
    """Per NS block (rel_fro, sigma_dev) for one stored matrix."""
    out = []
    gb = oracle.view_blocks_of(np.asarray(got_stored, np.float64), view_blocks)
    rb = oracle.view_blocks_of(np.asarray(ref_stored, np.float64), view_blocks)
    for g, r in zip(gb, rb):
        nr = np.linalg.norm(r)
        rel = np.linalg.norm(g - r) / nr if nr > 0 else np.linalg.norm(g)
        sd = float(np.max(np.abs(singular_values(g) - singular_values(r)))) if sigma else 0.0
        out.append((float(rel), sd))
    return out


def assert_ns_close(got_stored, ref_stored, view_blocks=1, tol=NS_REL_TOL, sigma_tol=SIGMA_TOL,
                    sigma=True, label=""):
    errs = block_errors(got_stored, ref_stored, view_blocks, sigma)
    worst_rel = max(e[0] for e in errs)
    worst_sig = max(e[1] for e in errs)
    assert worst_rel <= tol, f"{label}: relative Frobenius error {worst_rel:.3e} > {tol}"
    assert worst_sig <= sigma_tol, f"{label}: singular-value deviation {worst_sig:.3e} > {sigma_tol}"
    return worst_rel, worst_sig


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))
