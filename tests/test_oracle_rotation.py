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


# ---------------------------------------------------------------------------
# up-projection-aware rotation (a reading of the open refinement)
# ---------------------------------------------------------------------------

def _orthonormal_rows_weights(rng, H, d, r):
    """W_UK / W_UV whose stacked rows are orthonormal columns' transposes:
    sum_h W[h]^T W[h] = I (needs H * d >= r)."""
    q, _ = np.linalg.qr(rng.standard_normal((H * d, r)))
    return q.reshape(H, d, r)


def test_weighted_rotation_reduces_to_plain_for_isotropic_upprojection():
    """G proportional to the identity: the weighted rotation is the OSCAR rotation."""
    rng = np.random.default_rng(21)
    r, n = 32, 400
    c = rng.standard_normal((n, r)) * np.exp(np.linspace(-3, 0, r))
    w_uk = _orthonormal_rows_weights(rng, 4, 8, r) * 3.0   # sum W^T W = 9 I
    w_uv = _orthonormal_rows_weights(rng, 4, 8, r) * 3.0
    g = O.upprojection_metric(w_uk, w_uv)
    assert np.allclose(g, np.eye(r), atol=1e-12)
    _, lam_p, R_p = O.calibrate_rotation(c)
    _, lam_w, R_w = O.calibrate_rotation_weighted(c, w_uk, w_uv)
    assert np.allclose(R_w, R_p, atol=1e-10)
    assert np.allclose(lam_w, lam_p / (1.0 + O.METRIC_RIDGE), rtol=1e-10)


def test_weighted_rotation_commuting_closed_form():
    """Sigma = Q diag(s) Q^T and G = Q diag(g) Q^T share eigenvectors, so
    Sigma_w = Q diag(s / (g + ridge)) Q^T: the columns are Q's, ordered by
    s / g ascending."""
    rng = np.random.default_rng(22)
    r = 12
    Q, _ = np.linalg.qr(rng.standard_normal((r, r)))
    s = np.exp(rng.uniform(-4, 0, r))
    gdiag = rng.uniform(0.1, 3.0, r)
    # latents with covariance exactly Q diag(s) Q^T: a whitened sample
    n = 3 * r
    x = rng.standard_normal((n, r))
    x = x @ np.linalg.inv(np.linalg.cholesky(x.T @ x / n)).T     # x^T x / n = I
    c = (x * np.sqrt(s)) @ Q.T
    # weights with G = Q diag(g) Q^T: W_UK rows = diag(sqrt(g)) Q^T, W_UV = 0
    w_uk = (np.sqrt(gdiag)[:, None] * Q.T).reshape(1, r, r)
    w_uv = np.zeros((1, 1, r))
    _, lam, R = O.calibrate_rotation_weighted(c, w_uk, w_uv)
    gn = gdiag * (r / gdiag.sum())                  # the metric's scaling
    wv = s / (gn + O.METRIC_RIDGE)
    order = np.argsort(wv)
    assert np.allclose(lam, wv[order], rtol=1e-9)
    for j, k in enumerate(order):
        assert abs(abs(R[:, j] @ Q[:, k]) - 1.0) < 1e-9


def test_weighted_rotation_invariants():
    rng = np.random.default_rng(23)
    w = S.WORKLOADS[0]
    st = S.streams(0)
    model = S.latent_model(w, st)
    c = S.calib_latents(w, st, model)
    w_uk, w_uv = S.weights(w, st)
    R32, lam, R = O.calibrate_rotation_weighted(c, w_uk, w_uv)
    r = R.shape[0]
    assert np.max(np.abs(R.T @ R - np.eye(r))) < 1e-12
    assert np.all(np.diff(lam) >= 0)
    # R diagonalises (G + ridge)^(-1/2) Sigma (G + ridge)^(-1/2), built here from its parts
    g = O.upprojection_metric(w_uk, w_uv)
    ev, evec = np.linalg.eigh(g)
    gh = evec @ np.diag(1.0 / np.sqrt(ev + O.METRIC_RIDGE)) @ evec.T
    assert np.max(np.abs(np.linalg.inv(gh @ gh) - (g + O.METRIC_RIDGE * np.eye(len(g))))) < 1e-8
    cc = np.asarray(c, np.float64)
    sw = gh @ (cc.T @ cc / cc.shape[0]) @ gh
    d = R.T @ sw @ R
    off = d - np.diag(np.diag(d))
    assert np.max(np.abs(off)) < 1e-10 * np.max(np.abs(sw))
    assert np.allclose(np.diag(d), lam, rtol=1e-9, atol=1e-14)
    # sign rule
    for j in range(r):
        assert R[np.argmax(np.abs(R[:, j])), j] > 0
    assert R32.dtype == np.float32


def test_weighted_rotation_effect_on_upprojected_error():
    """What the weighting is for (a directional check, not a pin): with an
    up-projection that amplifies a few latent directions, the INT2 error of
    the reconstruction, counted in the up-projection's metric, is lower with
    the weighted rotation than with the unweighted one."""
    rng = np.random.default_rng(24)
    r, G = 64, 16
    w = S.WORKLOADS[0]
    st = S.streams(0)
    model = S.latent_model(w, st)
    c_cal = S.calib_latents(w, st, model)
    c_test = model.sample(rng, 512)
    # up-projection: random, with 8 latent directions amplified 30x
    w_uk = rng.standard_normal((4, 32, r)) / 8
    w_uv = rng.standard_normal((4, 32, r)) / 8
    boost = np.ones(r)
    boost[rng.choice(r, 8, replace=False)] = 30.0
    Qb, _ = np.linalg.qr(rng.standard_normal((r, r)))
    amp = Qb @ np.diag(boost) @ Qb.T
    w_uk, w_uv = w_uk @ amp, w_uv @ amp
    g = O.upprojection_metric(w_uk, w_uv)

    def err(R32):
        Ra = O.rotation_apply(R32)
        alpha, _ = O.fit_clip(c_cal, R32, G)
        q = O.quantize_cache(c_test, Ra, alpha, G)
        zh = O.dequantize(q["codes"], q["scale_h"], q["zero_h"], G)
        e = O.unrotate(zh, Ra) - np.asarray(c_test, np.float64)
        return float(np.mean(np.einsum("ni,ij,nj->n", e, g, e)))

    e_plain = err(O.calibrate_rotation(c_cal)[0])
    e_weighted = err(O.calibrate_rotation_weighted(c_cal, w_uk, w_uv)[0])
    print(f"up-projected INT2 error: unweighted {e_plain:.4g}, weighted {e_weighted:.4g}")
    assert e_weighted < e_plain


def test_upprojection_metric_is_the_reconstruction_norm():
    """e^T G e is the squared size of the up-projected error, summed over
    heads' key and value parts (explicit per-head products), scaled by
    r / (sum of squared weights)."""
    rng = np.random.default_rng(25)
    H, dn, dv, r = 3, 5, 7, 11
    w_uk = rng.standard_normal((H, dn, r))
    w_uv = rng.standard_normal((H, dv, r))
    g = O.upprojection_metric(w_uk, w_uv)
    scale = r / (np.sum(w_uk ** 2) + np.sum(w_uv ** 2))
    for _ in range(5):
        e = rng.standard_normal(r)
        direct = sum(np.sum((w_uk[h] @ e) ** 2) + np.sum((w_uv[h] @ e) ** 2) for h in range(H))
        assert np.isclose(e @ g @ e, scale * direct, rtol=1e-12)
