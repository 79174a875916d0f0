"""Pins for the fp64 oracle: closed forms, special cases and invariants.

Each test checks the oracle against something other than its own code path:
the SVD closed form of the iteration (NS acts on each singular value through
the scalar polynomial p(s) = a s + b s^3 + c s^5), rank-1 and scaled-orthogonal
special cases, momentum closed forms for a constant gradient, hand-computed
update values, and the constants printed on the pages (tests/golden/).
"""
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [float(v) for v in vals] if len(vals) > 1 else float(vals[0])
    return out


def p_scalar(s, coeffs, steps):
    """Scalar quintic applied `steps` times (the map NS applies to each singular value)."""
    a, b, c = coeffs
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def closed_form_ns(Y, coeffs=oracle.NS_COEFFS, steps=oracle.NS_STEPS, eps=oracle.NS_EPS):
    U, sig, Vt = np.linalg.svd(np.asarray(Y, np.float64), full_matrices=False)
    s = np.sqrt(np.sum(sig ** 2)) + eps
    return (U * p_scalar(sig / s, coeffs, steps)[None, :]) @ Vt


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def semi_orthogonal(rng, m, n):
    """m x n (m <= n) with orthonormal rows."""
    q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return q.T


# ---------------------------------------------------------------- constants
def test_constants_match_pages():
    g = _read_golden("ns_coefficients.txt")
    assert oracle.NS_COEFFS == (g["a"], g["b"], g["c"])
    assert oracle.NS_STEPS == int(g["steps"])
    # p(1) = a + b + c = 0.701 (arithmetic on the printed constants)
    assert p_scalar(1.0, oracle.NS_COEFFS, 1) == pytest.approx(0.701, abs=1e-12)


def test_workload_shapes_match_pages():
    g = _read_golden("custom_sizing_groups.txt")
    wl = workloads.get_workload("gpt124m")
    by = {gr.name: gr for gr in wl.groups}
    assert by["gate"].count == g["smear_gate"] + g["attn_gate"]
    assert by["attn"].count == g["attn"] and by["mlp"].count == g["mlp"]
    assert wl.n_matrices == g["total"] == sum(g["group_sizes"])
    for name in ("attn", "mlp"):
        assert (by[name].rows, by[name].cols) == (g["stored_rows"], g["stored_cols"])
    assert by["attn"].view_blocks == g["view_blocks"]
    assert by["attn"].block_shape == (768, 768)
    h = _read_golden("hyperparameters.txt")
    assert wl.lr == h["record_lr"] and wl.weight_decay == h["record_weight_decay"]
    assert wl.momentum == h["record_momentum"]
    gq = workloads.get_workload("gqa_small")
    assert gq.lr == h["matrix_lr"]
    assert gq.momentum_at(0) == pytest.approx(h["warmup_start"])
    assert gq.momentum_at(int(h["warmup_steps"])) == pytest.approx(h["warmup_end"])
    assert gq.momentum_at(250) == pytest.approx(0.5 * (h["warmup_start"] + h["warmup_end"]))
    t = workloads.get_workload("tiny")
    assert (t.lr, t.weight_decay, t.momentum) == (
        h["muon_default_lr"], h["muon_default_weight_decay"], h["muon_default_momentum"])


# ---------------------------------------------------------------- NS closed form
@pytest.mark.parametrize("shape", [(8, 8), (6, 10), (10, 6), (16, 48), (33, 17), (64, 128), (1, 12)])
@pytest.mark.parametrize("seed", [0, 1])
def test_ns_matches_svd_closed_form(shape, seed):
    rng = np.random.default_rng(seed)
    Y = rng.standard_normal(shape)
    got = oracle.newton_schulz(Y)
    assert rel(got, closed_form_ns(Y)) < 1e-12


@pytest.mark.parametrize("coeffs,steps", [((1.0, 0.0, 0.0), 1), ((0.0, 1.0, 0.0), 1),
                                          ((0.0, 0.0, 1.0), 1), ((0.3, -0.7, 1.9), 2),
                                          (oracle.NS_COEFFS, 1), (oracle.NS_COEFFS, 3)])
def test_ns_closed_form_each_term(coeffs, steps):
    # Isolating a, b and c one at a time catches a dropped or mis-signed term,
    # and the square non-symmetric input catches X B in place of B X.
    rng = np.random.default_rng(7)
    for shape in [(9, 9), (5, 13), (13, 5)]:
        Y = rng.standard_normal(shape)
        got = oracle.newton_schulz(Y, steps=steps, coeffs=coeffs)
        assert rel(got, closed_form_ns(Y, coeffs, steps)) < 1e-12


def test_ns_zero_steps_is_frobenius_normalisation():
    Y = np.random.default_rng(3).standard_normal((7, 11)) * 5.0
    got = oracle.newton_schulz(Y, steps=0)
    assert np.linalg.norm(got) == pytest.approx(1.0, abs=1e-7)
    assert rel(got, Y / np.linalg.norm(Y)) < 1e-7


def test_ns_rank1_gate():
    # A 1 x n block has one singular value, equal to its norm: O = p^5(1) g/||g||.
    g = np.random.default_rng(11).standard_normal((1, 12))
    k = p_scalar(1.0, oracle.NS_COEFFS, 5)
    assert k == pytest.approx(0.6964364, abs=1e-7)
    got = oracle.newton_schulz(g, eps=0.0)
    np.testing.assert_allclose(got, k * g / np.linalg.norm(g), rtol=1e-12, atol=1e-15)
    got_eps = oracle.newton_schulz(g)  # eps = 1e-7 shifts the singular value by ~3e-8
    np.testing.assert_allclose(got_eps, k * g / np.linalg.norm(g), rtol=1e-6)


@pytest.mark.parametrize("m,n,expected", [(64, 128, 0.68814), (16, 64, None), (32, 32, None)])
def test_ns_scaled_semi_orthogonal(m, n, expected):
    # Y = alpha Q with orthonormal rows: every normalised singular value is 1/sqrt(m).
    rng = np.random.default_rng(m + n)
    Q = semi_orthogonal(rng, m, n)
    k = p_scalar(1.0 / np.sqrt(m), oracle.NS_COEFFS, 5)
    if expected is not None:
        assert k == pytest.approx(expected, abs=1e-5)
    for alpha in (1e-3, 1.0, 37.0):
        got = oracle.newton_schulz(alpha * Q, eps=0.0)
        assert rel(got, k * Q) < 1e-12
        got_t = oracle.newton_schulz(alpha * Q.T, eps=0.0)
        assert rel(got_t, k * Q.T) < 1e-12


def test_ns_zero_block_maps_to_zero():
    assert np.all(oracle.newton_schulz(np.zeros((4, 9))) == 0.0)


def test_ns_transpose_equivariance():
    Y = np.random.default_rng(5).standard_normal((12, 30))
    assert rel(oracle.newton_schulz(Y.T), oracle.newton_schulz(Y).T) < 1e-13


def test_ns_orthogonal_equivariance():
    rng = np.random.default_rng(6)
    Y = rng.standard_normal((10, 24))
    Q1, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    Q2, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    lhs = oracle.newton_schulz(Q1 @ Y @ Q2.T)
    rhs = Q1 @ oracle.newton_schulz(Y) @ Q2.T
    assert rel(lhs, rhs) < 1e-12


def test_ns_odd_and_scale_invariant():
    Y = np.random.default_rng(8).standard_normal((8, 20))
    base = oracle.newton_schulz(Y, eps=0.0)
    assert rel(oracle.newton_schulz(-Y, eps=0.0), -base) < 1e-14
    assert rel(oracle.newton_schulz(1e4 * Y, eps=0.0), base) < 1e-12


def test_ns_singular_value_band():
    # Normalised singular values of a 64 x 256 Gaussian lie in about [0.06, 0.19],
    # well above 1.5e-3, so after 5 steps they sit in [0.6798, 1.2024] (inside the
    # [0.6, 1.25] band).
    Y = np.random.default_rng(9).standard_normal((64, 256))
    s = np.linalg.svd(oracle.newton_schulz(Y), compute_uv=False)
    assert s.min() > 0.6798 - 1e-6 and s.max() < 1.2024 + 1e-6
    assert s.min() >= 0.6 and s.max() <= 1.25


# ---------------------------------------------------------------- attn view
def test_attn_view_is_contiguous_row_major_blocks():
    # Stored 16 x 32 matrix viewed as 4 blocks of 16 x 8: block k occupies the
    # contiguous elements [k*128, (k+1)*128), i.e. stored rows 4k..4k+3.
    rng = np.random.default_rng(12)
    R, C, v = 16, 32, 4
    blocks = []
    for k in range(v):
        Q = semi_orthogonal(rng, C // v, R).T  # 16 x 8, orthonormal columns
        blocks.append((k + 1.5) * Q)
    stored = np.concatenate([b.reshape(-1) for b in blocks]).reshape(R, C)
    # the view really is the stored rows 4k..4k+3
    np.testing.assert_array_equal(oracle.view_blocks_of(stored, v)[2].reshape(-1),
                                  stored[8:12].reshape(-1))
    out = oracle.ns_batched(stored[None], view_blocks=v, eps=0.0)[0]
    k5 = p_scalar(1.0 / np.sqrt(C // v), oracle.NS_COEFFS, 5)
    want = np.concatenate([(k5 * b / (k + 1.5)).reshape(-1) for k, b in enumerate(blocks)]).reshape(R, C)
    assert rel(out, want) < 1e-12
    # the column-slice reading gives something else
    col = np.concatenate([oracle.newton_schulz(stored[:, k * 8:(k + 1) * 8], eps=0.0)
                          for k in range(v)], axis=1)
    assert rel(col, want) > 1e-2


# ---------------------------------------------------------------- momentum
def test_momentum_constant_gradient_closed_form():
    g = np.random.default_rng(13).standard_normal((3, 5))
    mu = 0.95
    muf = float(np.float32(mu))
    M = np.zeros_like(g)
    for t in range(1, 7):
        M, U = oracle.nesterov_momentum(g, M, mu, nesterov=True)
        np.testing.assert_allclose(M, (1 - muf ** t) * g, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(U, (1 - muf ** (t + 1)) * g, rtol=1e-13, atol=1e-15)


def test_momentum_schedule_closed_form_and_plain():
    g = np.random.default_rng(14).standard_normal((4, 4))
    wl = workloads.get_workload("gqa_small")
    M = np.zeros_like(g)
    prod = 1.0
    for t in range(6):
        mu = wl.momentum_at(t)
        muf = float(np.float32(mu))
        prod *= muf
        M, U = oracle.nesterov_momentum(g, M, mu)
        np.testing.assert_allclose(M, (1 - prod) * g, rtol=1e-12)
        np.testing.assert_allclose(U, (1 - muf * prod) * g, rtol=1e-12)
    M2, U2 = oracle.nesterov_momentum(g, 0.5 * g, 0.9, nesterov=False)
    np.testing.assert_array_equal(U2, M2)
    np.testing.assert_allclose(M2, (0.5 + 0.5 * (1 - float(np.float32(0.9)))) * g, rtol=1e-15)


def test_momentum_uses_float32_rounded_coefficient():
    g = np.ones((1, 1))
    M, _ = oracle.nesterov_momentum(g, np.zeros((1, 1)), 0.95)
    assert M[0, 0] == 1.0 - float(np.float32(0.95))
    assert M[0, 0] != pytest.approx(0.05, abs=1e-9)


# ---------------------------------------------------------------- update
@pytest.mark.parametrize("R,C,lr_mul,wd_mul,expected", [
    (4, 1, 1.0, 1.0, 0.75),     # 2(1 - 0.5*0.25) - 0.5*2*1
    (1, 4, 1.0, 1.0, 1.25),     # aspect 1
    (4, 4, 2.0, 2.0, 0.5),      # 2(1 - 0.25) - 0.5*1*2*1
    (9, 1, 1.0, 0.0, 0.5),      # aspect 3, no decay: 2 - 0.5*3
])
def test_update_hand_computed(R, C, lr_mul, wd_mul, expected):
    P = np.full((R, C), 2.0)
    O = np.ones((R, C))
    got = oracle.muon_update(P, O, lr=0.5, weight_decay=0.25, lr_mul=lr_mul, wd_mul=wd_mul)
    np.testing.assert_array_equal(got, np.full((R, C), expected))


def test_full_step_closed_form():
    # G = alpha Q (orthonormal rows), zero buffer: U = (1 - mu^2) alpha Q, so
    # O = p^5(1/sqrt(m)) Q and P' = P(1 - lr wd) - lr aspect O.
    rng = np.random.default_rng(15)
    m, n = 16, 40
    Q = semi_orthogonal(rng, m, n)
    for R, C, Qs in [(m, n, Q), (n, m, Q.T)]:
        G = (0.3 * Qs)[None]
        P = rng.standard_normal((1, R, C))
        M = np.zeros_like(G)
        P1, M1, O = oracle.muon_step(P, G, M, lr=0.25, weight_decay=0.5, momentum=0.95,
                                     eps=0.0)
        k = p_scalar(1.0 / np.sqrt(m), oracle.NS_COEFFS, 5)
        assert rel(O[0], k * Qs) < 1e-12
        asp = max(1.0, R / C) ** 0.5
        assert rel(P1[0], P[0] * (1 - 0.125) - 0.25 * asp * k * Qs) < 1e-13
        np.testing.assert_allclose(M1, (1 - float(np.float32(0.95))) * G, rtol=1e-15)


# ---------------------------------------------------------------- input encoder
def test_bf16_encoder_round_to_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8),
                  3.4e38, np.inf, -0.0, 1e-40], dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    back = workloads.bf16_bits_to_f32(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even (mantissa ...0)
    assert back[2] == 1 + 4 * 2 ** -8          # tie -> even (mantissa ...0)
    assert back[3] == 1 + 2 * 2 ** -8          # above the tie -> up
    assert back[4] == -1.0
    assert np.isinf(back[5])                   # rounds past the largest finite bf16
    assert np.isinf(back[6]) and bits[7] == 0x8000
    assert abs(back[8] - 1e-40) < 2 ** -133 * 2
    nanb = workloads.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(workloads.bf16_bits_to_f32(nanb))[0]
