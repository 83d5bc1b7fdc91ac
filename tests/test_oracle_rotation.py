"""Pins for the oracle's calibration: covariance, eigh, order, signs.

Any R with R^T R = I and R^T Sigma R diagonal with ascending diagonal is the
ascending eigendecomposition, so checking those invariants pins it (up to the
sign rule, checked separately).  A covariance built from a known orthogonal
matrix and spectrum gives a closed form for the eigenvalues and vectors.
"""
import numpy as np

from oracle import mla_oracle as O
from workloads import synth as S


def test_covariance_matches_scalar_loops():
    rng = np.random.default_rng(10)
    c = rng.standard_normal((7, 5)).astype(np.float32)
    sig = O.latent_covariance(c)
    for i in range(5):
        for j in range(5):
            want = sum(float(c[t, i]) * float(c[t, j]) for t in range(7)) / 7
            assert abs(sig[i, j] - want) <= 1e-14 * max(1.0, abs(want))


def test_closed_form_spectrum_and_vectors():
    rng = np.random.default_rng(11)
    r = 24
    q = S.haar_orthogonal(rng, r)
    e = np.exp(rng.uniform(np.log(1e-4), 0, size=r))
    sigma = (q * e) @ q.T
    # feed Sigma through "calibration tokens" whose covariance is exactly it:
    # c = sqrt(n) * Sigma^(1/2) rows, so that c^T c / n == Sigma
    n = r
    half = (q * np.sqrt(e)) @ q.T
    c = np.sqrt(n) * half
    R, lam, V = O.calibrate_rotation(c)
    order = np.argsort(e)
    np.testing.assert_allclose(lam, e[order], rtol=1e-9, atol=1e-15)
    # each column equals +-the matching column of q
    dots = np.abs(np.sum(V * q[:, order], axis=0))
    np.testing.assert_allclose(dots, 1.0, atol=1e-9)


def test_rotation_invariants_workload1():
    w = S.WORKLOADS[1]
    st = S.streams(1)
    m = S.latent_model(w, st)
    c = S.calib_latents(w, st, m)
    R, lam, V = O.calibrate_rotation(c)
    sigma = O.latent_covariance(c)
    r = w.kv_lora_rank
    assert np.max(np.abs(V.T @ V - np.eye(r))) <= 1e-12
    R64 = R.astype(np.float64)
    assert np.max(np.abs(R64.T @ R64 - np.eye(r))) <= 1e-6
    assert np.all(np.diff(lam) >= 0)
    d = V.T @ sigma @ V
    off = d - np.diag(np.diag(d))
    assert np.max(np.abs(off)) <= 1e-12 * np.max(np.abs(sigma))
    np.testing.assert_allclose(np.diag(d), lam, rtol=1e-10, atol=1e-15)
    # statistical sanity: the sample trace follows the configured spectrum
    # (E tr = sum eig; sd = sqrt(2 sum eig^2 / N) for Gaussian latents)
    sd = np.sqrt(2.0 * np.sum(m.eig ** 2) / w.n_calib)
    assert abs(lam.sum() - m.eig.sum()) < 5 * sd


def test_sign_rule():
    v = np.array([[0.6, -0.8, 0.5],
                  [-0.8, -0.6, -0.5],
                  [0.0, 0.0, 0.0]])
    c = O.canonical_signs(v)
    # column 0: largest |.| is row 1 (-0.8) -> flipped
    assert c[:, 0].tolist() == [-0.6, 0.8, -0.0]
    # column 1: row 0 (-0.8) -> flipped
    assert c[:, 1].tolist() == [0.8, 0.6, -0.0]
    # column 2: tie between rows 0 and 1; the lower row decides (+0.5) -> kept
    assert c[:, 2].tolist() == [0.5, -0.5, 0.0]


def test_rotation_apply_is_bf16_of_R():
    rng = np.random.default_rng(12)
    R = rng.standard_normal((16, 16)).astype(np.float32)
    Ra = O.rotation_apply(R)
    import torch
    want = torch.from_numpy(R).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(Ra, want)


def test_rotate_exact_then_single_rounding():
    """z32 is the exact dot product rounded once to fp32 (checked with
    Python's exact rational arithmetic on a few tokens)."""
    from fractions import Fraction
    rng = np.random.default_rng(13)
    r = 16
    c = S.to_bf16_values(rng.standard_normal((3, r)).astype(np.float32))
    Ra = O.rotation_apply(rng.standard_normal((r, r)).astype(np.float32) / 4)
    z = O.rotate(c, Ra)
    for t in range(3):
        for j in range(r):
            exact = sum(Fraction(float(c[t, i])) * Fraction(float(Ra[i, j]))
                        for i in range(r))
            assert z[t, j] == np.float32(float(exact))
