"""Pins of the AdamW oracle against closed forms and an independent library
implementation (torch.optim.AdamW, float64 on the CPU), plus planted mistakes
that the pins must reject.  No GPU."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_oracle_pins import _read_golden

B1, B2 = oracle.ADAM_BETAS


def _f32(x):
    return float(np.float32(x))


def test_constants_match_pages():
    h = _read_golden("hyperparameters.txt")
    assert oracle.ADAM_LR == h["adam_lr"]
    assert oracle.ADAM_BETAS == (h["adam_beta1"], h["adam_beta2"])
    assert oracle.ADAM_EPS == h["adam_eps"]


def test_adam_workload_matches_pages():
    h = _read_golden("hyperparameters.txt")
    wl = workloads.ADAM_WORKLOADS["gpt124m_adam"]
    assert (wl.lr, wl.betas, wl.eps) == (h["adam_lr"], (h["adam_beta1"], h["adam_beta2"]), h["adam_eps"])
    shapes = dict(wl.tensors)
    vocab, dim = int(h["model_vocab_size"]), int(h["model_dim"])
    assert shapes["embed"] == (vocab, dim) and shapes["lm_head"] == (vocab, dim)
    assert shapes["scalars"] == (4 * int(h["model_num_layers"]),)


def test_scalars_closed_form():
    # t = 1: bias1 = 1 - b1, bias2 = 1 - b2 -> step = lr sqrt(1 - b2) / (1 - b1)
    d, s = oracle.adam_scalars(1, lr=0.008, beta1=B1, beta2=B2, weight_decay=0.0)
    b1, b2 = _f32(B1), _f32(B2)
    assert d == 1.0
    assert s == pytest.approx(_f32(0.008) * (1 - b2) ** 0.5 / (1 - b1), rel=1e-15)
    # t large: both corrections -> 1, step -> lr lr_mul; decay = 1 - lr lr_mul wd wd_mul
    d, s = oracle.adam_scalars(10_000, lr=0.01, beta1=B1, beta2=B2, weight_decay=0.1, lr_mul=2.0, wd_mul=0.5)
    assert s == pytest.approx(_f32(0.01) * 2.0, rel=1e-12)
    assert d == pytest.approx(1 - _f32(0.01) * 2.0 * _f32(0.1) * 0.5, rel=1e-15)
    with pytest.raises(ValueError):
        oracle.adam_scalars(0, lr=0.01, beta1=B1, beta2=B2, weight_decay=0.0)


def test_first_step_is_sign_descent_at_eps_zero():
    # From zero moments: m = (1-b1) g, v = (1-b2) g^2, so with eps = 0 the move is
    # lr sqrt(1-b2)/(1-b1) * (1-b1) g / (sqrt(1-b2) |g|) = lr sign(g), after the decay.
    rng = np.random.default_rng(1)
    p0 = rng.standard_normal(257)
    g = rng.standard_normal(257) * np.exp(rng.uniform(-8, 8, 257))
    lr, wd = 0.008, 0.05
    p, m, v = oracle.adamw_step(p0, g, np.zeros(257), np.zeros(257), t=1, lr=lr, beta1=B1, beta2=B2,
                                eps=0.0, weight_decay=wd)
    d = 1 - _f32(lr) * _f32(wd)
    np.testing.assert_allclose(p, d * p0 - _f32(lr) * np.sign(g), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(m, (1 - _f32(B1)) * g, rtol=1e-15)
    np.testing.assert_allclose(v, (1 - _f32(B2)) * g * g, rtol=1e-15)


def test_constant_gradient_trajectory_closed_form():
    # Constant g from zero moments: m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2, so at
    # eps = 0 every step moves by lr lr_mul sign(g); with decay d the recurrence
    # p_t = d p_{t-1} - s gives p_T = d^T p_0 - s (1 - d^T) / (1 - d).
    rng = np.random.default_rng(2)
    n, T = 64, 9
    p0 = rng.standard_normal(n)
    g = rng.standard_normal(n)
    m = np.zeros(n)
    v = np.zeros(n)
    p = p0
    lr, lr_mul, wd, wd_mul = 0.02, 1.5, 0.1, 0.25
    for t in range(1, T + 1):
        p, m, v = oracle.adamw_step(p, g, m, v, t=t, lr=lr, beta1=B1, beta2=B2, eps=0.0,
                                    weight_decay=wd, lr_mul=lr_mul, wd_mul=wd_mul)
        b1, b2 = _f32(B1), _f32(B2)
        np.testing.assert_allclose(m, (1 - b1 ** t) * g, rtol=1e-13)
        np.testing.assert_allclose(v, (1 - b2 ** t) * g * g, rtol=1e-13)
    s = _f32(lr) * _f32(lr_mul)
    d = 1 - s * _f32(wd) * _f32(wd_mul)
    expect = d ** T * p0 - s * np.sign(g) * (1 - d ** T) / (1 - d)
    np.testing.assert_allclose(p, expect, rtol=1e-12, atol=1e-14)


def test_zero_gradient_only_decays():
    rng = np.random.default_rng(3)
    p0 = rng.standard_normal(100)
    p, m, v = p0, np.zeros(100), np.zeros(100)
    for t in range(1, 6):
        p, m, v = oracle.adamw_step(p, np.zeros(100), m, v, t=t, lr=0.01, beta1=B1, beta2=B2, eps=1e-8,
                                    weight_decay=0.2)
    d = 1 - _f32(0.01) * _f32(0.2)
    np.testing.assert_allclose(p, d ** 5 * p0, rtol=1e-14)
    assert not m.any() and not v.any()
    # wd == 0 leaves the parameter exactly in place
    p1, _, _ = oracle.adamw_step(p0, np.zeros(100), np.zeros(100), np.zeros(100), t=1, lr=0.01, beta1=B1,
                                 beta2=B2, eps=1e-8, weight_decay=0.0)
    assert np.array_equal(p1, p0)


def _torch_adamw(p0, grads, *, lr, betas, eps_per_step, weight_decay):
    """torch.optim.AdamW in float64, one optimizer step per gradient."""
    p = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=lr, betas=betas, eps=eps_per_step[0], weight_decay=weight_decay,
                            foreach=False)
    for g, e in zip(grads, eps_per_step):
        opt.param_groups[0]["eps"] = e
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("eps", [0.0, 1e-8, 1e-3])
def test_matches_torch_adamw(eps):
    # torch adds eps after dividing sqrt(v) by sqrt(bias2); the page adds it before
    # folding sqrt(bias2) into the step size (reading A1), i.e. torch with
    # eps_t = eps / sqrt(bias2_t).  At eps = 0 the two are the same formula.
    rng = np.random.default_rng(4)
    n, T = 300, 6
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 10 ** rng.uniform(-4, 0) for _ in range(T)]
    lr, lr_mul, wd, wd_mul = 0.008, 0.5, 0.02, 2.0
    b1, b2 = _f32(B1), _f32(B2)
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        p, m, v = oracle.adamw_step(p, g, m, v, t=t, lr=lr, beta1=B1, beta2=B2, eps=eps, weight_decay=wd,
                                    lr_mul=lr_mul, wd_mul=wd_mul)
    eps_t = [_f32(eps) / (1 - b2 ** t) ** 0.5 for t in range(1, T + 1)]
    tp, tm, tv = _torch_adamw(p0, grads, lr=_f32(lr) * _f32(lr_mul), betas=(b1, b2), eps_per_step=eps_t,
                              weight_decay=_f32(wd) * _f32(wd_mul))
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(p, tp, rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------- planted mistakes
def _mutant(kind):
    def step(p, g, m, v, *, t, lr, beta1, beta2, eps, weight_decay, lr_mul=1.0, wd_mul=1.0):
        b1, b2, e = _f32(beta1), _f32(beta2), _f32(eps)
        s = _f32(lr) * _f32(lr_mul)
        d = 1 - s * _f32(weight_decay) * _f32(wd_mul)
        if kind != "decay_last":
            p = p * d
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        bias1, bias2 = 1 - b1 ** t, 1 - b2 ** t
        if kind == "no_sqrt_bias2":
            step_size = s * bias2 / bias1
        elif kind == "no_bias1":
            step_size = s * bias2 ** 0.5
        elif kind == "swap_betas":
            step_size = s * (1 - b1 ** t) ** 0.5 / (1 - b2 ** t)
        else:
            step_size = s * bias2 ** 0.5 / bias1
        if kind == "eps_in_sqrt":
            denom = np.sqrt(v + e)
        else:
            denom = np.sqrt(v) + e
        upd = step_size * m / denom
        p = p - upd
        if kind == "decay_last":
            p = p * d
        if kind == "decay_base_lr":
            p = p + s * _f32(weight_decay) * _f32(wd_mul) * p - _f32(lr) * _f32(weight_decay) * _f32(wd_mul) * p
        return p, m, v
    return step


@pytest.mark.parametrize("kind", ["decay_last", "no_sqrt_bias2", "no_bias1", "swap_betas", "eps_in_sqrt",
                                  "decay_base_lr"])
def test_pins_reject_adam_mutants(kind):
    rng = np.random.default_rng(5)
    n, T = 200, 5
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 1e-3 for _ in range(T)]
    lr, lr_mul, wd, wd_mul, eps = 0.008, 0.5, 0.3, 2.0, 1e-3
    f = _mutant(kind)
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        p, m, v = f(p, g, m, v, t=t, lr=lr, beta1=B1, beta2=B2, eps=eps, weight_decay=wd, lr_mul=lr_mul,
                    wd_mul=wd_mul)
    b2 = _f32(B2)
    eps_t = [_f32(eps) / (1 - b2 ** t) ** 0.5 for t in range(1, T + 1)]
    tp, _, _ = _torch_adamw(p0, grads, lr=_f32(lr) * _f32(lr_mul), betas=(_f32(B1), b2), eps_per_step=eps_t,
                            weight_decay=_f32(wd) * _f32(wd_mul))
    assert np.max(np.abs(p - tp)) > 1e-7, f"mutant {kind} not detected"


def test_unmutated_copy_passes_the_same_check():
    rng = np.random.default_rng(5)
    n, T = 200, 5
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 1e-3 for _ in range(T)]
    lr, lr_mul, wd, wd_mul, eps = 0.008, 0.5, 0.3, 2.0, 1e-3
    f = _mutant("none")
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        p, m, v = f(p, g, m, v, t=t, lr=lr, beta1=B1, beta2=B2, eps=eps, weight_decay=wd, lr_mul=lr_mul,
                    wd_mul=wd_mul)
    b2 = _f32(B2)
    eps_t = [_f32(eps) / (1 - b2 ** t) ** 0.5 for t in range(1, T + 1)]
    tp, _, _ = _torch_adamw(p0, grads, lr=_f32(lr) * _f32(lr_mul), betas=(_f32(B1), b2), eps_per_step=eps_t,
                            weight_decay=_f32(wd) * _f32(wd_mul))
    assert np.max(np.abs(p - tp)) < 1e-12
