"""Pins for the oracle's Spectral Score Smoothing (step 2).

AudioKV article, section 2.2: F = rfft(s); cumulative energy E(k); the
smallest k* with E(k*) >= rho E(L/2); low-pass mask with cutoff k*; blend
s_hat = (1 - alpha) s + alpha irfft(F * mask).  Pins: numpy's FFT as the
library routine, closed forms for sinusoidal rows, and the algebraic
invariants that any plausible slip (inclusive/exclusive cutoff, a missing
factor 2 on paired bins, a wrong blend weight, a dropped 1/L) breaks.
"""
import numpy as np
import pytest

from oracle import oracle as O

LENGTHS = [1, 2, 3, 4, 5, 8, 16, 17, 64, 100, 256]


@pytest.mark.parametrize("L", LENGTHS)
def test_direct_dft_matches_numpy_rfft(L):
    s = np.random.default_rng(L).random(L)
    F = O.dft(s)
    ref = np.fft.rfft(s)
    assert F.shape == ref.shape
    np.testing.assert_allclose(F, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(s).sum()))


@pytest.mark.parametrize("L", [2, 3, 8, 9, 64, 100])
def test_lowpass_matches_numpy_irfft_for_every_cutoff(L):
    s = np.random.default_rng(100 + L).standard_normal(L)
    n = L // 2
    F = np.fft.rfft(s)
    for ks in sorted({0, 1, n // 2, max(0, n - 1), n}):
        _, got_ks, _, lp = O.sss(s, 1.0, 0.7, kstar=ks)
        assert got_ks == ks
        ref = np.fft.irfft(np.where(np.arange(n + 1) <= ks, F, 0), n=L)
        np.testing.assert_allclose(lp, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L", [16, 64, 1024, 100, 999, 3001])
@pytest.mark.parametrize("c,a,f", [(1.0, 0.5, 3), (0.2, 1.0, 5), (0.0, 1.0, 1), (1.0, 1.0, 7)])
def test_cosine_closed_form(L, c, a, f):
    # s = c + a cos(2 pi f j / L), 0 < f < L/2: F_0 = L c, F_f = a L / 2, rest 0.
    # E(0) = (Lc)^2, E(n) = (Lc)^2 + (aL/2)^2  =>  k* = 0 iff c^2 >= rho (c^2 + a^2/4),
    # else k* = f, and the low-pass is the constant c or s itself.
    j = np.arange(L)
    s = c + a * np.cos(2 * np.pi * f * j / L)
    for rho in (0.3, 0.7, 0.95):
        sh, ks, E, lp = O.sss(s, 0.5, rho)
        want = 0 if c * c >= rho * (c * c + a * a / 4) else f
        assert ks == want
        np.testing.assert_allclose(lp, np.full(L, c) if want == 0 else s, atol=1e-12)
        np.testing.assert_allclose(E[-1], L * L * (c * c + a * a / 4), rtol=1e-12)


def test_two_tone_closed_form_cutoffs():
    # s = c + a cos(2 pi f j/L) + b sin(2 pi g j/L), f < g < L/2.
    L, f, g = 128, 4, 20
    j = np.arange(L)
    c, a, b = 1.0, 1.2, 0.8
    s = c + a * np.cos(2 * np.pi * f * j / L) + b * np.sin(2 * np.pi * g * j / L)
    e0, ef, eg = c * c, a * a / 4, b * b / 4
    tot = e0 + ef + eg
    low = c + a * np.cos(2 * np.pi * f * j / L)
    for rho, want, want_lp in [(e0 / tot - 1e-9, 0, np.full(L, c)),
                               ((e0 + ef) / tot - 1e-9, f, low),
                               ((e0 + ef) / tot + 1e-9, g, s)]:
        sh, ks, _, lp = O.sss(s, 0.25, rho)
        assert ks == want, (rho, ks)
        np.testing.assert_allclose(lp, want_lp, atol=1e-12)
        np.testing.assert_allclose(sh, 0.75 * s + 0.25 * want_lp, atol=1e-12)


def test_nyquist_bin_closed_form():
    # s_j = c + a (-1)^j puts energy a^2 L^2 into the Nyquist bin only.
    L, c, a = 32, 1.0, 2.0
    s = c + a * (-1.0) ** np.arange(L)
    sh, ks, _, lp = O.sss(s, 1.0, 0.9)
    assert ks == L // 2
    np.testing.assert_allclose(lp, s, atol=1e-12)
    sh, ks, _, lp = O.sss(s, 1.0, 0.1)
    assert ks == 0
    np.testing.assert_allclose(lp, np.full(L, c), atol=1e-12)


def test_alpha_zero_is_identity_bit_exact():
    s = np.random.default_rng(7).random(512)
    sh, _, _, _ = O.sss(s, 0.0, 0.7)
    assert np.array_equal(sh, s)


@pytest.mark.parametrize("L", [64, 1024, 4096])
def test_constant_row_passes_unchanged(L):
    for c in (0.5, 1.0 / 1024, 3.0):
        s = np.full(L, c)
        sh, ks, _, lp = O.sss(s, 0.5, 0.7)
        assert ks == 0
        assert np.array_equal(lp, s)
        assert np.array_equal(sh, s)


def test_sum_preserved_and_scale_equivariance():
    rng = np.random.default_rng(8)
    s = rng.random(256)
    sh, ks, _, _ = O.sss(s, 0.6, 0.7)
    assert sh.sum() == pytest.approx(s.sum(), rel=1e-12)
    sh2, ks2, _, _ = O.sss(3.5 * s, 0.6, 0.7)
    assert ks2 == ks
    np.testing.assert_allclose(sh2, 3.5 * sh, rtol=1e-11)


def test_cutoff_monotone_in_rho():
    s = np.random.default_rng(9).random(512) ** 4
    ks = [O.sss(s, 0.5, rho)[1] for rho in np.linspace(0.05, 1.0, 40)]
    assert all(a <= b for a, b in zip(ks, ks[1:]))


def test_full_energy_full_blend_reconstructs():
    s = np.random.default_rng(10).random(128)
    sh, ks, _, _ = O.sss(s, 1.0, 1.0)
    np.testing.assert_allclose(sh, s, atol=1e-12)


def test_circular_shift_commutes():
    rng = np.random.default_rng(11)
    s = rng.random(256) + np.sin(np.arange(256) / 9.0)
    sh, ks, _, _ = O.sss(s, 0.5, 0.8)
    for m in (1, 17, 100):
        sh_m, ks_m, _, _ = O.sss(np.roll(s, m), 0.5, 0.8)
        assert ks_m == ks
        np.testing.assert_allclose(sh_m, np.roll(sh, m), atol=1e-12)


def test_lowpass_linear_for_fixed_cutoff():
    rng = np.random.default_rng(12)
    a, b = rng.random(64), rng.random(64)
    lpa = O.sss(a, 1.0, 0.7, kstar=5)[3]
    lpb = O.sss(b, 1.0, 0.7, kstar=5)[3]
    lpab = O.sss(a + b, 1.0, 0.7, kstar=5)[3]
    np.testing.assert_allclose(lpab, lpa + lpb, atol=1e-13)


def test_energy_is_parseval_total():
    # E(n) counts each bin once (one-sided, unweighted, as written).
    s = np.random.default_rng(13).random(100)
    _, _, E, _ = O.sss(s, 0.5, 0.7)
    F = np.fft.rfft(s)
    assert E[-1] == pytest.approx(np.sum(np.abs(F) ** 2), rel=1e-12)
    assert np.all(np.diff(E) >= 0)
