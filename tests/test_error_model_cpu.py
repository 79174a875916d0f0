"""CPU checks of the bf16 error model (tests/error_model.py).

* Without rounding the model is the method: an exact rewrite of the oracle's
  iteration (normalisation folded into the first iteration, aI carried by B',
  hi + lo splits summing to the value), equal to it to float64 rounding.
* With round-to-nearest-even it predicts errors in the range the survey's
  NumPy probes found (FAST about 1e-2 at 768x3072; ACCURATE below it; FAST
  near the 2e-2 bar on a 1/i spectrum, where ACCURATE stays far below).
* The two precision regressions the GPU band tests must catch move the
  prediction well outside a 1.33x band: truncation instead of round-to-nearest,
  and ACCURATE with its lo pass dropped.
"""
import numpy as np
import pytest

import error_model as em
import oracle
import workloads


def _gauss(shape, seed, std=1e-2):
    bits = workloads.gaussian_bits(shape, seed=seed, std=std)
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def _spectral(m, n, seed):
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((m, m)))
    v, _ = np.linalg.qr(rng.standard_normal((n, m)))
    g = (u * (1.0 / np.arange(1, m + 1))) @ v.T
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(g.astype(np.float32))).astype(np.float64)


@pytest.mark.parametrize("shape", [(64, 128), (96, 300), (300, 96), (128, 128)])
@pytest.mark.parametrize("precision", ["fast", "accurate"])
def test_unrounded_model_is_the_oracle(shape, precision):
    Y = _gauss(shape, seed=shape[0] + shape[1])
    got = em.ns_model(Y, precision=precision, rnd=em.no_rounding)
    want = oracle.newton_schulz(Y)
    assert em.rel_fro(got, want) < 1e-12


def test_unrounded_model_zero_steps_is_normalisation():
    Y = _gauss((64, 160), seed=3)
    for precision in ("fast", "accurate"):
        got = em.ns_model(Y, steps=0, precision=precision, rnd=em.no_rounding)
        assert em.rel_fro(got, oracle.newton_schulz(Y, steps=0)) < 1e-14


def test_round_bf16_is_rne():
    # 1 + 2^-8 is halfway between bf16 1 and 1 + 2^-7: ties go to the even (1);
    # 1 + 3 * 2^-8 ties to 1 + 2^-6 (even mantissa); a hair above a tie rounds up
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8), 3.0, 0.0])
    np.testing.assert_array_equal(em.round_bf16(x), [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0, 3.0, 0.0])
    # agrees with the fp32 -> bf16 encoder on float32 inputs
    v = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    np.testing.assert_array_equal(em.round_bf16(v.astype(np.float64)),
                                  workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v)))


def test_predicted_levels_match_the_survey_probes():
    Y = _gauss((768, 3072), seed=7)
    ref = oracle.newton_schulz(Y)
    e_fast = em.rel_fro(em.ns_model(Y), ref)
    e_acc = em.rel_fro(em.ns_model(Y, precision="accurate"), ref)
    assert 5e-3 < e_fast < 1.5e-2
    assert e_acc < 0.6 * e_fast
    # a 1/i spectrum: FAST near the 2e-2 bar (the survey's probes, normalisation
    # folded: 1.8e-2 at 512x1792, 2.1e-2 at 2048x7168), ACCURATE far below it
    S = _spectral(256, 896, seed=5)
    ref = oracle.newton_schulz(S)
    e_fast = em.rel_fro(em.ns_model(S), ref)
    e_acc = em.rel_fro(em.ns_model(S, precision="accurate"), ref)
    assert e_fast > 1.2e-2 and e_acc < 4e-3 and e_fast > 4 * e_acc


def test_regressions_leave_the_band():
    Y = _gauss((256, 768), seed=11)
    ref = oracle.newton_schulz(Y)
    e = em.rel_fro(em.ns_model(Y), ref)
    assert em.rel_fro(em.ns_model(Y, rnd=em.trunc_bf16), ref) > 1.5 * e
    S = _spectral(256, 896, seed=13)
    ref = oracle.newton_schulz(S)
    e_acc = em.rel_fro(em.ns_model(S, precision="accurate"), ref)
    assert em.rel_fro(em.ns_model(S, precision="accurate", drop_lo=True), ref) > 3 * e_acc
