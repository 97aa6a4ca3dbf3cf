"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a closed
form (SVD, eigen-decomposition of the small Gram matrix, unrolled momentum
sum), a value printed on a page (tests/golden), an invariant, or brute force
on tiny inputs.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
A, B, C = 3.4445, -4.7750, 2.0315


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f_scalar(x, steps=5, schedule=None):
    """Odd quintic of "Muon Optimizer 정리", Newton-Schulz section, iterated on a scalar."""
    x = np.asarray(x, dtype=np.float64)
    for t in range(steps):
        a, b, c = schedule[t] if schedule is not None else (A, B, C)
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def svd_closed_form(m, steps=5, schedule=None):
    """Z = U f^steps(Sigma / ||M||_F) V^T: the polynomial acts on singular values only."""
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    nu = np.sqrt(np.sum(s ** 2))
    return (u * f_scalar(s / nu, steps, schedule)[None, :]) @ vt


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# Momentum
# ----------------------------------------------------------------------------

def test_momentum_constant_gradient_closed_form():
    # Unrolled eq. (1): with a constant gradient, M_k = G (1 - mu^k) / (1 - mu).
    g = rng(0).standard_normal((5, 7))
    mu = 0.95
    m = np.zeros_like(g)
    for k in range(1, 12):
        m = O.momentum_update(m, g, mu)
        np.testing.assert_allclose(m, g * (1 - mu ** k) / (1 - mu), rtol=1e-13, atol=1e-14)


def test_momentum_unrolled_sum_varying_gradients():
    r = rng(1)
    mu = 0.9
    gs = [r.standard_normal((3, 4)) for _ in range(6)]
    m = np.zeros((3, 4))
    for g in gs:
        m = O.momentum_update(m, g, mu)
    expect = sum(mu ** (len(gs) - 1 - t) * gs[t] for t in range(len(gs)))
    np.testing.assert_allclose(m, expect, rtol=1e-13, atol=1e-14)


def test_momentum_stored_rounding_bf16():
    g = np.array([[1.0, 3.0]])
    m = O.momentum_update(np.array([[2.0 ** -8, 0.0]]), g, 1.0, "bf16")
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa -> 1.0.
    assert m[0, 0] == 1.0 and m[0, 1] == 3.0


# ----------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------

def test_round_bf16_ties_and_torch_agreement():
    assert O.round_to_dtype(np.array([1 + 2.0 ** -8]), "bf16")[0] == 1.0
    assert O.round_to_dtype(np.array([1 + 3 * 2.0 ** -8]), "bf16")[0] == 1 + 2.0 ** -6
    assert O.round_to_dtype(np.array([-(1 + 3 * 2.0 ** -8)]), "bf16")[0] == -(1 + 2.0 ** -6)
    assert np.isinf(O.round_to_dtype(np.array([3.5e38]), "bf16")[0])
    # Against torch's float32 -> bfloat16 conversion (one rounding from float32).
    x32 = (rng(2).standard_normal(20000) * np.exp(rng(3).uniform(-80, 80, 20000))).astype(np.float32)
    x32 = np.concatenate([x32, np.float32([1e-40, -3e-39, 2.0 ** -130, 0.0])])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_dtype(x32.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------------------
# Newton-Schulz
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(4, 16), (16, 4), (7, 7), (9, 30), (33, 5), (1, 12), (12, 1)])
def test_ns_matches_svd_closed_form(shape):
    m = rng(hash(shape) % 1000).standard_normal(shape) * np.exp(rng(5).uniform(-2, 2, shape[1]))[None, :]
    z = O.newton_schulz(m)
    np.testing.assert_allclose(z, svd_closed_form(m), rtol=0, atol=1e-11)


def test_ns_rank_deficient_matches_svd():
    r = rng(6)
    m = r.standard_normal((10, 3)) @ r.standard_normal((3, 25))
    np.testing.assert_allclose(O.newton_schulz(m), svd_closed_form(m), atol=1e-11)


def test_ns_rank_one_is_scaled_normalised_input():
    # One singular value equal to ||M||_F: Z = f^5(1) * M / ||M||_F.
    r = rng(7)
    m = np.outer(r.standard_normal(6), r.standard_normal(11))
    f5_1 = f_scalar(1.0)
    assert abs(f5_1 - 0.6964364094697522) < 1e-12
    np.testing.assert_allclose(O.newton_schulz(m), f5_1 * m / np.linalg.norm(m), atol=1e-13)


def test_ns_width_one_column_is_normalised_vector():
    # "From PCG to Muon", "6. Muon Reshaping": width 1 just normalises the vector.
    v = rng(8).standard_normal((40, 1))
    np.testing.assert_allclose(O.newton_schulz(v), f_scalar(1.0) * v / np.linalg.norm(v), atol=1e-13)


def test_ns_tall_uses_small_gram_eigendecomposition():
    # N x 2: the iteration is a polynomial in the 2 x 2 Gram matrix G^T G
    # ("From PCG to Muon", "Muon's Gram Matrix").  Z = X V diag(f(s)/s) V^T,
    # with X = G / ||G||_F and G^T G / ||G||^2 = V diag(s^2) V^T.
    g = rng(9).standard_normal((500, 2)) * np.array([3.0, 0.1])
    x = g / np.linalg.norm(g)
    lam, v = np.linalg.eigh(x.T @ x)
    s = np.sqrt(lam)
    z = x @ (v * (f_scalar(s) / s)[None, :]) @ v.T
    np.testing.assert_allclose(O.newton_schulz(g), z, atol=1e-12)


def test_ns_worked_example_directions_kept_magnitudes_equalised():
    gold = _golden("sitech_worked_example.json")
    sig = np.array(gold["input_singular_values"])
    r = rng(10)
    u, _ = np.linalg.qr(r.standard_normal((3, 3)))
    v, _ = np.linalg.qr(r.standard_normal((5, 3)))
    g = (u * sig[None, :]) @ v.T
    z = O.newton_schulz(g)
    core = u.T @ z @ v                     # diagonal iff singular vectors are kept
    np.testing.assert_allclose(core - np.diag(np.diag(core)), 0.0, atol=1e-12)
    out = np.diag(core)
    np.testing.assert_allclose(out, f_scalar(sig / np.linalg.norm(sig)), atol=1e-12)
    # "approximately 1": every value within the 5-step band around 1.
    assert np.all(out > 0.68) and np.all(out < 1.21)
    np.testing.assert_allclose(out, gold["output_singular_values_approx"], atol=0.32)


def test_ns_invariances():
    r = rng(11)
    m = r.standard_normal((6, 9))
    z = O.newton_schulz(m)
    np.testing.assert_allclose(O.newton_schulz(m.T), z.T, atol=1e-13)
    np.testing.assert_allclose(O.newton_schulz(7.5 * m), z, atol=1e-13)
    p, _ = np.linalg.qr(r.standard_normal((6, 6)))
    q, _ = np.linalg.qr(r.standard_normal((9, 9)))
    np.testing.assert_allclose(O.newton_schulz(p @ m @ q), p @ z @ q, atol=1e-12)


def test_ns_inner_product_positive():
    # <M, Z> = sum sigma_i f^5(sigma_i / nu) > 0: Z is a descent direction.
    m = rng(12).standard_normal((8, 20))
    s = np.linalg.svd(m, compute_uv=False)
    ip = np.sum(m * O.newton_schulz(m))
    assert ip > 0
    np.testing.assert_allclose(ip, np.sum(s * f_scalar(s / np.linalg.norm(s))), rtol=1e-12)


def test_ns_zero_input_and_zero_steps():
    assert np.all(O.newton_schulz(np.zeros((3, 4))) == 0)
    m = rng(13).standard_normal((3, 4))
    np.testing.assert_allclose(O.newton_schulz(m, steps=0), m / np.linalg.norm(m), atol=1e-15)


def test_ns_singular_value_band():
    # For singular values not far below the largest, five steps land in [0.68, 1.21].
    r = rng(14)
    u, _ = np.linalg.qr(r.standard_normal((20, 20)))
    v, _ = np.linalg.qr(r.standard_normal((30, 20)))
    sig = np.exp(np.linspace(0, np.log(0.05), 20))
    z = O.newton_schulz((u * sig) @ v.T)
    s = np.linalg.svd(z, compute_uv=False)
    assert s.min() > 0.68 and s.max() < 1.21


def test_ns_schedule_matches_per_iteration_polynomials():
    sched = [(4.0, -5.0, 2.0), (3.5, -4.5, 1.9), (3.0, -3.2, 1.2), (2.5, -2.0, 0.6), (1.9, -1.3, 0.4)]
    m = rng(15).standard_normal((5, 12))
    np.testing.assert_allclose(O.newton_schulz(m, 5, schedule=sched),
                               svd_closed_form(m, 5, sched), atol=1e-11)
    const = [(A, B, C)] * 5
    np.testing.assert_array_equal(O.newton_schulz(m, 5, schedule=const), O.newton_schulz(m))


# ----------------------------------------------------------------------------
# Energies and the float32 pairwise tree
# ----------------------------------------------------------------------------

def test_pairwise_tree_brute_force_small():
    f = np.float32
    p = rng(16).uniform(0, 1, 9).astype(np.float32)
    assert O.pairwise_sum_f32(p[:1]) == p[0]
    assert O.pairwise_sum_f32(p[:2]) == f(p[0] + p[1])
    assert O.pairwise_sum_f32(p[:3]) == f(f(p[0] + p[1]) + p[2])
    assert O.pairwise_sum_f32(p[:4]) == f(f(p[0] + p[1]) + f(p[2] + p[3]))
    left = f(f(p[0] + p[1]) + f(p[2] + p[3]))
    assert O.pairwise_sum_f32(p[:6]) == f(left + f(p[4] + p[5]))
    assert O.pairwise_sum_f32(p[:7]) == f(left + f(f(p[4] + p[5]) + p[6]))
    eight = f(left + f(f(p[4] + p[5]) + f(p[6] + p[7])))
    assert O.pairwise_sum_f32(p[:8]) == eight
    assert O.pairwise_sum_f32(p[:9]) == f(eight + p[8])
    assert O.pairwise_sum_f32(np.zeros(0)) == 0


def test_pairwise_tree_differs_from_sequential_somewhere():
    # Guards against a tree silently replaced by a left-to-right sum.
    r = rng(17)
    diffs = 0
    for _ in range(50):
        p = r.uniform(0, 1, 100).astype(np.float32)
        seq = np.float32(0)
        for v in p:
            seq = np.float32(seq + v)
        diffs += O.pairwise_sum_f32(p) != seq
    assert diffs > 0


@pytest.mark.parametrize("shape", [(4, 16), (37, 300), (300, 37), (1, 1), (2, 1025)])
def test_energies_tree_within_bound_of_float64(shape):
    x = (rng(18).standard_normal(shape) * 3).astype(np.float32).astype(np.float64)
    r32, c32 = O.energies_f32_tree(x)
    r64, c64 = O.energies_f64(x)
    m, n = shape
    depth_r = int(np.ceil(np.log2(max(n, 1)))) + 1
    depth_c = int(np.ceil(np.log2(max(m, 1)))) + 1
    u = 2.0 ** -24
    assert np.all(np.abs(r32 - r64) <= depth_r * u * r64 + 1e-45)
    assert np.all(np.abs(c32 - c64) <= depth_c * u * c64 + 1e-45)
    assert r32.dtype == np.float32 and c32.shape == (n,)


# ----------------------------------------------------------------------------
# Dimuon conditioning
# ----------------------------------------------------------------------------

def test_conditioning_problem4_printed_values():
    gold = _golden("dimuon_problem4.json")
    e = np.array(gold["relative_energy"])
    d = O.conditioning(e, gold["eps"])
    np.testing.assert_array_equal(np.round(d, gold["factor_printed_decimals"]), gold["factor_printed"])
    with np.errstate(divide="ignore"):
        d0 = O.conditioning(e, 0.0)
    assert np.isinf(d0[3])
    np.testing.assert_array_equal(np.round(d0[:3], gold["factor_without_floor_decimals"]),
                                  gold["factor_without_floor_printed"][:3])


def test_conditioning_caps_per_side_and_total():
    gold = _golden("dimuon_problem4.json")
    r = rng(19)
    for _ in range(20):
        er = r.exponential(1.0, 50) * (r.uniform(size=50) > 0.2)
        ec = r.exponential(1.0, 70) ** 6
        dr, dc = O.conditioning(er), O.conditioning(ec)
        assert dr.max() <= gold["max_factor_per_side"] * (1 + 1e-12)
        assert dc.max() <= gold["max_factor_per_side"] * (1 + 1e-12)
        assert np.outer(dr, dc).max() <= gold["max_factor_both_sides"] * (1 + 1e-12)
        assert dr.min() >= (1 + 1e-4) ** -0.25 * (1 - 1e-15)


def test_conditioning_zero_rows_hit_floor_and_first_step_off():
    e = np.array([4.0, 0.0, 1.0, 0.0])
    d = O.conditioning(e)
    np.testing.assert_allclose(d[[1, 3]], 10.0, rtol=1e-15)
    assert d[0] == (1 + 1e-4) ** -0.25
    np.testing.assert_array_equal(O.conditioning(np.zeros(5)), np.ones(5))


def test_conditioning_relative_to_largest():
    # Scaling all energies leaves the factors unchanged (relative energy).
    e = rng(20).exponential(1.0, 30)
    np.testing.assert_allclose(O.conditioning(e), O.conditioning(1e5 * e), rtol=1e-13)


# ----------------------------------------------------------------------------
# Whole steps
# ----------------------------------------------------------------------------

def _mats(shape, seed):
    r = rng(seed)
    return (0.02 * r.standard_normal(shape), r.standard_normal(shape), r.standard_normal(shape))


@pytest.mark.parametrize("shape", [(4, 16), (16, 4), (6, 6)])
def test_dimuon_first_step_is_muon_bitwise(shape):
    w, g, _ = _mats(shape, 21)
    zero = np.zeros(shape)
    a = O.muon_step(w, g, zero, lr=0.01, mu=0.95)
    b = O.dimuon_step(w, g, zero, lr=0.01, mu=0.95)
    np.testing.assert_array_equal(a.o, b.o)
    np.testing.assert_array_equal(a.w, b.w)
    np.testing.assert_array_equal(a.m, b.m)
    np.testing.assert_array_equal(b.d_r, 1.0)


@pytest.mark.parametrize("shape", [(5, 12), (12, 5)])
def test_dimuon_matches_svd_closed_form(shape):
    w, g, mp = _mats(shape, 22)
    mp = mp * np.exp(rng(23).uniform(-3, 3, shape[1]))[None, :]
    res = O.dimuon_step(w, g, mp, lr=0.02, mu=0.9)
    er = (mp ** 2).sum(1)
    ec = (mp ** 2).sum(0)
    dr = (er / er.max() + 1e-4) ** -0.25
    dc = (ec / ec.max() + 1e-4) ** -0.25
    y = dr[:, None] * (0.9 * mp + g) * dc[None, :]
    u, s, vt = np.linalg.svd(y, full_matrices=False)
    fs = f_scalar(s / np.linalg.norm(s))
    p = dr[:, None] * ((u * fs) @ vt) * dc[None, :]
    o = p * (np.linalg.norm(fs) / np.linalg.norm(p))
    # Energies are summed in float32 by the oracle: factors agree to ~1e-7.
    np.testing.assert_allclose(res.o, o, atol=2e-6)
    np.testing.assert_allclose(np.linalg.norm(res.o), np.linalg.norm(fs), rtol=1e-6)
    np.testing.assert_allclose(res.w, w - 0.02 * res.o, atol=1e-15)


def test_dimuon_factors_come_from_previous_momentum():
    # With mu = 0 the new momentum no longer holds M_prev, yet Dimuon's step
    # still depends on it through the energies; Muon's does not.
    w, g, mp = _mats((6, 10), 24)
    mp2 = mp * np.linspace(0.1, 3, 10)[None, :]
    a = O.dimuon_step(w, g, mp, lr=0.1, mu=0.0)
    b = O.dimuon_step(w, g, mp2, lr=0.1, mu=0.0)
    assert np.max(np.abs(a.o - b.o)) > 1e-3
    np.testing.assert_array_equal(O.muon_step(w, g, mp, lr=0.1, mu=0.0).o,
                                  O.muon_step(w, g, mp2, lr=0.1, mu=0.0).o)


def test_toy_dimuon_rebalances_columns():
    ctx = _golden("dimuon_toy_context.json")
    def share(o):
        col = (o ** 2).sum(0)
        return col[-4:].sum() / col.sum()
    for seed in range(8):
        m = W.lora_toy(seed).mats[0]
        w, g, mp = (t.double().numpy() for t in (m.w, m.g, m.m_prev))
        mu_res = O.muon_step(w, g, mp, lr=0.01, mu=0.95)
        di_res = O.dimuon_step(w, g, mp, lr=0.01, mu=0.95)
        assert share(di_res.o) < share(mu_res.o)
        s = np.linalg.svd(di_res.o, compute_uv=False)
        assert s.max() / s.min() > 1.8       # no longer near-orthogonal
    # Adam's first step keeps only signs: four of sixteen columns get 4/16.
    sgn = np.sign(g)
    assert share(sgn) == ctx["top4_share_adam_first_step"]


def test_update_closed_form_with_decay_and_scale():
    # Rows of Q orthonormal: every singular value of M = alpha * Q is alpha,
    # so Z = f^5(1/sqrt(k)) * Q.
    r = rng(25)
    q, _ = np.linalg.qr(r.standard_normal((20, 4)))
    q = q.T                                    # 4 x 20, orthonormal rows
    w = 0.02 * r.standard_normal((4, 20))
    res = O.muon_step(w, 3.0 * q, np.zeros((4, 20)), lr=0.05, mu=0.95,
                      weight_decay=0.1, scale=0.7)
    z = f_scalar(0.5) * q
    np.testing.assert_allclose(res.o, z, atol=1e-13)
    np.testing.assert_allclose(res.w, w - 0.05 * (0.7 * z + 0.1 * w), atol=1e-15)


def test_nesterov_input_closed_form():
    g = rng(26).standard_normal((3, 8))
    mu = 0.95
    m = np.zeros_like(g)
    for k in range(1, 6):
        res = O.muon_step(np.zeros_like(g), g, m, lr=1.0, mu=mu, nesterov=True)
        m = res.m
        v = g + mu * g * (1 - mu ** k) / (1 - mu)
        np.testing.assert_allclose(res.o, svd_closed_form(v), atol=1e-12)


def test_weight_dtype_rounding():
    w, g, mp = _mats((3, 5), 27)
    res = O.muon_step(w, g, mp, lr=0.02, mu=0.95, w_dtype="bf16", mom_dtype="bf16")
    np.testing.assert_array_equal(res.w, O.round_to_dtype(res.w, "bf16"))
    np.testing.assert_array_equal(res.m, O.round_to_dtype(0.95 * mp + g, "bf16"))
