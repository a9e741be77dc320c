"""Pins of the oracle's elementary pieces against things other than itself:
libm's exp, SciPy's spherical harmonics, quadrature orthonormality, the
logistic function, Adam's first-step closed form."""
import math

import numpy as np
import pytest
import scipy.special as sps


def ulp_diff(a, b):
    """Distance in float32 ulps between float32 a and the float64 reference b."""
    a = a.astype(np.float64)
    spacing = np.spacing(np.abs(b).astype(np.float32)).astype(np.float64)
    return np.abs(a - b) / spacing


def test_exp_cw_within_2ulp_of_libm(oracle_lib):
    x = np.linspace(-87.0, 88.0, 2_000_001, dtype=np.float32)
    y = oracle_lib.exp_cw(x)
    ref = np.exp(x.astype(np.float64))
    assert ulp_diff(y, ref).max() <= 2.0


def test_exp_falloff_within_1ulp_of_libm(oracle_lib):
    # a dense sweep of [-6, 0] plus every f32 in three windows: around 0, around
    # a rounding boundary of k (x log2 e = -0.5) and at the bottom of the range
    x = np.linspace(-6.0, 0.0, 3_000_001, dtype=np.float32)
    wins = []
    for c in (np.float32(-1e-6), np.float32(-0.5 / 1.4426950408889634), np.float32(-5.9999)):
        u = c.view(np.uint32)
        wins.append(np.arange(u - 200_000, u + 200_000, dtype=np.uint32).view(np.float32))
    x = np.concatenate([x] + wins)
    x = x[(x >= -6.0) & (x <= 0.0)]
    y = oracle_lib.exp_falloff(x)
    assert ulp_diff(y, np.exp(x.astype(np.float64))).max() <= 1.0


def test_exp_falloff_never_exceeds_one(oracle_lib):
    # G <= 1 on [-6, 0], as exp is there: alpha = o G never exceeds o, so the
    # clamp at 0.99 binds only for opacities above it.  A dense sweep, the f32
    # values next to 0 and to the steps of k (where the reduced argument
    # changes sign), every one checked.
    x = np.linspace(-6.0, 0.0, 3_000_001, dtype=np.float32)
    wins = [np.arange(0x80000000, 0x80000000 + 400_000, dtype=np.uint32).view(np.float32)]
    for k in range(1, 9):
        c = np.float32(-(k - 0.5) * math.log(2.0))
        u = c.view(np.uint32)
        wins.append(np.arange(u - 50_000, u + 50_000, dtype=np.uint32).view(np.float32))
    x = np.concatenate([x] + wins)
    x = x[(x >= -6.0) & (x <= 0.0)]
    y = oracle_lib.exp_falloff(x)
    assert (y <= np.float32(1.0)).all()
    assert (y[np.abs(x) < 1e-8] == np.float32(1.0)).all()


def test_exp_falloff_clamp_keeps_every_skip_decision(oracle_lib):
    y = oracle_lib.exp_falloff(np.array([0.0, -0.0, 0.5, 1e30, -6.0, -6.5, -87.0, -1e30], np.float32))
    assert y[0] == 1.0 and y[1] == 1.0 and y[2] == 1.0 and y[3] == 1.0
    assert y[5] == y[4] and y[6] == y[4] and y[7] == y[4]
    # below -6 the value stands in for exp(x) < exp(-6): any opacity <= 1 times
    # it stays under the 1/255 threshold, so the entry is skipped either way,
    # while the largest power that can be included (-ln 255) is inside the range
    assert np.float32(1.0) * y[4] < np.float32(1.0) / np.float32(255.0)
    assert -np.log(255.0) > -6.0


def test_exp_cw_special_values(oracle_lib):
    x = np.array([0.0, -0.0, -87.5, -1e30, 89.0, np.inf, -np.inf, 1.0], np.float32)
    y = oracle_lib.exp_cw(x)
    assert y[0] == 1.0 and y[1] == 1.0
    assert y[2] == 0.0 and y[3] == 0.0 and y[6] == 0.0
    assert np.isinf(y[4]) and np.isinf(y[5])
    assert ulp_diff(y[7:8], np.array([math.e])).max() <= 1.0
    assert np.isnan(oracle_lib.exp_cw(np.array([np.nan], np.float32))[0])


def test_exp_cw_monotone_on_negative_range(oracle_lib):
    # the rasterizer only evaluates exp at power <= 0
    x = np.linspace(-87.0, 0.0, 1_000_001, dtype=np.float32)
    y = oracle_lib.exp_cw(x)
    assert np.all(np.diff(y) >= 0)


def real_sh_scipy(deg, dirs):
    """Real orthonormal SH without the Condon-Shortley phase, built from
    SciPy's complex harmonics (which include that phase)."""
    x, y, z = dirs[:, 0], dirs[:, 1], dirs[:, 2]
    theta = np.arccos(np.clip(z, -1, 1))
    phi = np.arctan2(y, x)
    cols = []
    for l in range(deg + 1):
        for m in range(-l, l + 1):
            if m == 0:
                cols.append(sps.sph_harm_y(l, 0, theta, phi).real)
            elif m > 0:
                cols.append(math.sqrt(2) * (-1) ** m * sps.sph_harm_y(l, m, theta, phi).real)
            else:
                cols.append(math.sqrt(2) * (-1) ** m * sps.sph_harm_y(l, -m, theta, phi).imag)
    return np.stack(cols, axis=1)


@pytest.mark.parametrize("deg", [0, 1, 2, 3])
def test_sh_basis_matches_scipy(oracle_lib, deg):
    rng = np.random.default_rng(7)
    d = rng.normal(size=(500, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    Y = oracle_lib.sh_basis(deg, d, np.float64)
    np.testing.assert_allclose(Y, real_sh_scipy(deg, d), rtol=0, atol=1e-12)
    Y32 = oracle_lib.sh_basis(deg, d.astype(np.float32), np.float32)
    np.testing.assert_allclose(Y32, Y, rtol=0, atol=3e-6)


def test_sh_basis_orthonormal_by_quadrature(oracle_lib):
    # Gauss-Legendre in cos(theta) x uniform phi integrates degree <= 6 exactly
    nt, nph = 12, 16
    ct, wt = np.polynomial.legendre.leggauss(nt)
    ph = np.arange(nph) * 2 * np.pi / nph
    CT, PH = np.meshgrid(ct, ph, indexing="ij")
    st = np.sqrt(1 - CT ** 2)
    d = np.stack([st * np.cos(PH), st * np.sin(PH), CT], axis=-1).reshape(-1, 3)
    w = (wt[:, None] * np.full(nph, 2 * np.pi / nph)[None, :]).reshape(-1)
    Y = oracle_lib.sh_basis(3, d, np.float64)
    gram = (Y * w[:, None]).T @ Y
    np.testing.assert_allclose(gram, np.eye(16), atol=1e-12)


def test_adam_first_step_closed_form(oracle_lib):
    rng = np.random.default_rng(3)
    g = rng.normal(size=1000) * 10.0 ** rng.uniform(-8, 2, size=1000)
    g[:5] = 0.0
    theta = rng.normal(size=1000)
    lr, eps = 1e-3, 1e-15
    p, m, v = oracle_lib.adam(g, theta, np.zeros(1000), np.zeros(1000), step=1, lr=lr, eps=eps)
    np.testing.assert_allclose(p - theta, -lr * g / (np.abs(g) + eps), rtol=1e-9, atol=1e-18)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-14)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-14)


def test_adam_second_step_moves_along_moments(oracle_lib):
    # two steps with a constant gradient: bias-corrected moments equal g and g^2
    g = np.array([1e-3, -2.0, 5.0])
    theta = np.zeros(3)
    p, m, v = oracle_lib.adam(g, theta, np.zeros(3), np.zeros(3), step=1, lr=0.1, eps=0.0)
    p2, _, _ = oracle_lib.adam(g, p, m, v, step=2, lr=0.1, eps=0.0)
    np.testing.assert_allclose(p2, -0.2 * np.sign(g), rtol=1e-12)
