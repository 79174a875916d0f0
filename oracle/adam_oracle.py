"""fp64 CPU oracle for the AdamW step of the non-matrix parameters.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the test suite, the smoke check and the benchmark's CPU-baseline leg call
it.  It shares no code with the HIP library; the two meet only in the seeded
inputs of the `workloads` module.

Everything is computed in float64 with numpy element-wise operations, in the
order the page lists them.

Sources (page title, then section):
  [DA]  The article on moving the Adam gradient reduce-scatter of
        modded-nanogpt's DistAdam into a backward hook (record of 2025-10-31),
        "change two: step() walks the parameter groups and parameters in
        reverse": the per-parameter body of DistAdam.step -- the step count is
        incremented first; weight decay is decoupled and applied first,
        p *= 1 - lr lr_mul wd wd_mul (only when wd != 0); the two moments are
        updated as exp_avg = beta1 exp_avg + (1 - beta1) g and
        exp_avg_sq = beta2 exp_avg_sq + (1 - beta2) g^2; with
        bias1 = 1 - beta1^t and bias2 = 1 - beta2^t the parameter moves by
        -lr lr_mul (bias2^0.5 / bias1) exp_avg / (sqrt(exp_avg_sq) + eps).
  [CS]  "Muon Custom Sizing" walkthrough of the modded-nanogpt 124M record,
        section 4: the DistAdam that steps the scalar, head and embedding
        parameters uses lr 0.008, betas (0.8, 0.95), eps 1e-8.

Readings where the pages leave a step open (each also listed in the design doc):
  A1  eps is added to sqrt(exp_avg_sq) before the bias correction of the
      second moment, which the page folds into the step size.  torch's AdamW
      adds eps after dividing by sqrt(bias2), so the two agree exactly only
      when eps is replaced by eps / sqrt(bias2) (pinned against torch).
  A2  One GPU holds the whole parameter: the page's rank slice
      param[rank * rows / world : ...] is the full tensor here.
  A3  Gradients arrive in bf16 (as for Muon); parameters and both moments are
      fp32.  Scalars cross the C ABI as float32, so lr, the betas, eps, the
      weight decay and the per-tensor multipliers are rounded through float32
      before use in float64 (as reading R10 of the Muon oracle).
  A4  t is the tensor's step count after the increment (t >= 1), kept by the
      caller; a tensor whose moments start at zero starts at t = 1.

Every function here is pinned by tests against closed forms (sign-descent
first step and constant-gradient trajectories at eps = 0, decay-only steps at
g = 0) and against torch.optim.AdamW in float64; none is parity unpinned.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

# [CS] section 4: the 124M record's DistAdam settings.
ADAM_LR = 0.008
ADAM_BETAS: Tuple[float, float] = (0.8, 0.95)
ADAM_EPS = 1e-8


def _f32(x: float) -> float:
    """A scalar as the C ABI sees it (A3)."""
    return float(np.float32(x))


def adam_scalars(t: int, *, lr: float, beta1: float, beta2: float, weight_decay: float,
                 lr_mul: float = 1.0, wd_mul: float = 1.0) -> Tuple[float, float]:
    """[DA] per-parameter constants of one step: (decay factor, step size).

    decay = 1 - lr lr_mul wd wd_mul (1 when wd == 0);
    step size = lr lr_mul (1 - beta2^t)^0.5 / (1 - beta1^t).
    """
    if t < 1:
        raise ValueError("t is the step count after the increment (t >= 1)")
    lr_eff = _f32(lr) * _f32(lr_mul)
    wd = _f32(weight_decay)
    decay = 1.0 - lr_eff * wd * _f32(wd_mul) if wd != 0.0 else 1.0
    b1, b2 = _f32(beta1), _f32(beta2)
    bias1 = 1.0 - b1 ** t
    bias2 = 1.0 - b2 ** t
    return decay, lr_eff * (bias2 ** 0.5 / bias1)


def adamw_step(p, g, exp_avg, exp_avg_sq, *, t: int, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float, lr_mul: float = 1.0, wd_mul: float = 1.0):
    """[DA] one AdamW step of one parameter; returns (p, exp_avg, exp_avg_sq) in float64.

    Inputs are not modified.  `g` holds the gradient values (already decoded
    from bf16 by the caller).
    """
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(exp_avg, np.float64)
    v = np.asarray(exp_avg_sq, np.float64)
    b1, b2, e = _f32(beta1), _f32(beta2), _f32(eps)
    decay, step_size = adam_scalars(t, lr=lr, beta1=beta1, beta2=beta2, weight_decay=weight_decay,
                                    lr_mul=lr_mul, wd_mul=wd_mul)
    # weight decay first
    p = p * decay
    # running averages
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    # bias-corrected step
    denom = np.sqrt(v) + e
    p = p - step_size * (m / denom)
    return p, m, v
