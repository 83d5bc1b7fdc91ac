"""Pins for the OSCAR full-attention (grouped-query) oracle.

* Plain GQA attention against torch's scaled_dot_product_attention on the
  CPU in fp64 (KV heads expanded by the test, draft mask built by the test).
* The rotated-space form equals plain attention on the un-rotated entries
  (associativity) to 1e-12.
* query_covariance against a scalar loop; score_weights against its closed
  form at scale 0 (uniform causal attention: harmonic sums) and against the
  total mass each (query, head) pair contributes; value_covariance with equal
  weights against the plain uncentred covariance.
* K rotation, plain reading (the default, eigenvectors of the query
  covariance): for queries built with an exactly known covariance Q L Q^T it
  is Q with its columns ordered by ascending L (signs by the rule) and its
  eigenvalues are sorted L; it does not depend on the keys; the mean square
  score error of any key error e over the calibration queries equals the
  eigenvalue-weighted sum of e's rotated channels squared.
* K rotation, query-metric refinement: for axis-aligned queries and keys the
  signed permutation that sorts the axes by ascending key variance over
  query variance (the closed form of the metric-weighted covariance when
  both are diagonal); with isotropic queries the keys' own covariance basis.
* Both: orthogonal, ascending, sign rule.
* Directional (not a strict pin): with anisotropic queries, INT2 keys
  quantised in the query-metric basis give a smaller score error than keys
  quantised in their own covariance basis.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import gqa_oracle as Q
from oracle import mla_oracle as O


def _qkv(seed, n_q=4, n_kv=2, n=24, d=16, q_axes=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_q, n, d))
    if q_axes is not None:
        q = q * q_axes
    k = rng.standard_normal((n_kv, n, d))
    v = rng.standard_normal((n_kv, n, d))
    return q, k, v


@pytest.mark.parametrize("tq,causal", [(1, True), (3, True), (3, False)])
def test_gqa_attention_matches_sdpa(tq, causal):
    rng = np.random.default_rng(1)
    n_q, n_kv, L, d = 6, 2, 19, 8
    q = rng.standard_normal((tq, n_q, d))
    k = rng.standard_normal((n_kv, L, d))
    v = rng.standard_normal((n_kv, L, d))
    scale = 0.3
    out, lse = Q.gqa_attention(q, k, v, scale, causal)
    G = n_q // n_kv
    kk = torch.from_numpy(np.repeat(k, G, axis=0))          # [H_q, L, d]
    vv = torch.from_numpy(np.repeat(v, G, axis=0))
    qq = torch.from_numpy(q.transpose(1, 0, 2))              # [H_q, tq, d]
    mask = torch.ones(tq, L, dtype=torch.bool)
    if causal:
        for t in range(tq):
            mask[t, L - tq + t + 1:] = False
    ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    assert np.allclose(out, ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)
    s = scale * np.einsum("gtd,gld->gtl", qq.numpy(), kk.numpy())
    s = np.where(mask.numpy()[None], s, -np.inf)
    m = s.max(-1)
    ref_lse = m + np.log(np.exp(s - m[..., None]).sum(-1))
    assert np.allclose(lse, ref_lse.T, rtol=1e-12, atol=1e-12)


def test_rotated_form_equals_plain():
    rng = np.random.default_rng(2)
    n_q, n_kv, L, d = 4, 2, 30, 16
    q = rng.standard_normal((2, n_q, d))
    zk = rng.standard_normal((n_kv, L, d))
    zv = rng.standard_normal((n_kv, L, d))
    rk = np.stack([O.rotation_apply(Q.rotation_from_covariance(np.cov(rng.standard_normal((d, 40))))[0])
                   for _ in range(n_kv)])
    rv = np.stack([O.rotation_apply(Q.rotation_from_covariance(np.cov(rng.standard_normal((d, 40))))[0])
                   for _ in range(n_kv)])
    out_r, lse_r = Q.rotated_attention(q, zk, zv, rk, rv, 0.25, causal=True)
    out_p, lse_p = Q.gqa_attention(q, Q.unrotate_heads(zk, rk), Q.unrotate_heads(zv, rv), 0.25, causal=True)
    assert np.allclose(out_r, out_p, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse_r, lse_p, rtol=1e-12, atol=1e-12)


def test_query_covariance_scalar_loop():
    q, _, _ = _qkv(3, n_q=4, n_kv=2, n=5, d=3)
    got = Q.query_covariance(q, 2)
    for h in range(2):
        ref = np.zeros((3, 3))
        for g in (2 * h, 2 * h + 1):
            for i in range(5):
                for a in range(3):
                    for b in range(3):
                        ref[a, b] += q[g, i, a] * q[g, i, b]
        assert np.allclose(got[h], ref / 10, rtol=1e-14, atol=1e-15)


def test_score_weights_closed_forms():
    q, k, _ = _qkv(4, n_q=6, n_kv=3, n=20, d=8)
    w = Q.score_weights(q, k, 0.4)
    assert np.allclose(w.sum(axis=1), 20 * 2, rtol=1e-12)    # each (query, head) adds 1
    w0 = Q.score_weights(q, k, 0.0)                          # uniform causal attention
    harmonic = np.array([sum(1.0 / (i + 1) for i in range(t, 20)) for t in range(20)])
    assert np.allclose(w0, 2 * harmonic[None], rtol=1e-12)


def test_value_covariance_equal_weights():
    _, _, v = _qkv(5, n_kv=2, n=15, d=6)
    got = Q.value_covariance(v, np.full((2, 15), 3.0))
    for h in range(2):
        assert np.allclose(got[h], v[h].T @ v[h] / 15, rtol=1e-12)


def test_k_rotation_for_axis_aligned_queries():
    qax = np.array([3.0, 0.5, 2.0, 0.1, 1.0, 5.0])
    kax = np.array([1.0, 2.0, 0.3, 0.2, 3.0, 1.5])      # ratios to the queries all distinct
    q, k, v = _qkv(6, n_q=2, n_kv=1, n=4000, d=6, q_axes=qax)
    k = k * kax
    rk, ek, rv, ev, _ = Q.calibrate(q, k, v, 0.3, k_rotation=Q.K_QUERY_METRIC)
    order = np.argsort(kax ** 2 / qax ** 2)                  # ascending key / query variance
    perm = np.abs(rk[0].astype(np.float64))
    assert np.allclose(perm, np.eye(6)[:, order], atol=0.05)
    for r, e in ((rk[0], ek[0]), (rv[0], ev[0])):
        assert np.all(np.diff(e) >= 0)
        assert np.abs(r.astype(np.float64).T @ r - np.eye(6)).max() <= 1e-6
        assert np.allclose(O.canonical_signs(r.astype(np.float64)), r, atol=1e-7)


def test_isotropic_queries_give_key_covariance_basis():
    _, k, v = _qkv(8, n_q=2, n_kv=1, n=48, d=8)
    q = np.stack([np.tile(np.eye(8), (6, 1)) * 2.0 for _ in range(2)])    # Sigma_q = I / 2 exactly
    assert np.allclose(Q.query_covariance(q, 1)[0], 0.5 * np.eye(8))
    rk, ek, _, _, _ = Q.calibrate(q, k, v, 0.3, k_rotation=Q.K_QUERY_METRIC)
    r_self, e_self = Q.rotation_from_covariance(Q.key_covariance(k)[0])
    assert np.allclose(rk[0], r_self, atol=1e-5)
    assert np.allclose(ek[0], e_self / (1 + Q.METRIC_RIDGE), rtol=1e-9)   # M scaled to I


def test_query_aware_k_rotation_reduces_score_error():
    rng = np.random.default_rng(7)
    d, n = 64, 2048
    axes = np.exp(np.linspace(np.log(0.05), np.log(3.0), d))[rng.permutation(d)]
    q = rng.standard_normal((2, n, d)) * axes
    k = (rng.standard_normal((1, n, d)) * np.exp(np.linspace(0, -3, d))).astype(np.float32)
    k = O.bf16_round(k)[None][0]
    v = rng.standard_normal((1, n, d))
    rk, _, _, _, _ = Q.calibrate(q, k, v, 0.1, k_rotation=Q.K_QUERY_METRIC)
    r_self, _, _ = O.calibrate_rotation(k[0])                # K's own covariance basis

    def score_err(r):
        ra = O.rotation_apply(r)
        alpha, _ = O.fit_clip(k[0], r, 16)
        qz = O.quantize_cache(k[0], ra, alpha, 16)
        k_hat = O.dequantize(qz["codes"], qz["scale_h"], qz["zero_h"], 16) @ ra.astype(np.float64).T
        return np.mean(((q[0] @ (k[0].astype(np.float64) - k_hat).T)) ** 2)

    assert score_err(rk[0]) < score_err(r_self)


def _queries_with_covariance(basis, lam, n_q):
    """Queries [n_q, d, d] whose query covariance is exactly basis diag(lam)
    basis^T: every query head holds the rows sqrt(d lam_j) basis[:, j]."""
    d = basis.shape[0]
    rows = (np.sqrt(d * lam)[:, None] * basis.T)            # row j = sqrt(d lam_j) q_j
    return np.stack([rows] * n_q)


def test_plain_k_rotation_is_the_query_covariance_basis():
    rng = np.random.default_rng(11)
    d = 12
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.exp(rng.uniform(-3, 2, d))
    q = _queries_with_covariance(basis, lam, 2)
    assert np.allclose(Q.query_covariance(q, 1)[0], basis @ np.diag(lam) @ basis.T, atol=1e-12)
    _, k, v = _qkv(12, n_q=2, n_kv=1, n=d, d=d)
    rk, ek, _, _, _ = Q.calibrate(q, k, v, 0.2)
    order = np.argsort(lam)
    assert np.allclose(ek[0], lam[order], rtol=1e-10)
    expect = O.canonical_signs(basis[:, order])
    assert np.abs(rk[0].astype(np.float64) - expect).max() <= 1e-6
    # the keys do not enter the plain reading
    rk2, ek2, _, _, _ = Q.calibrate(q, 3.0 * k[:, ::-1], v, 0.2)
    assert np.array_equal(rk2, rk) and np.array_equal(ek2, ek)


def test_plain_k_rotation_weights_score_error_by_eigenvalue():
    q, k, v = _qkv(13, n_q=4, n_kv=2, n=64, d=8, q_axes=np.array([3.0, 0.2, 1.0, 0.5, 2.0, 0.1, 1.5, 0.7]))
    rk, ek, _, _, _ = Q.calibrate(q, k, v, 0.2)
    rng = np.random.default_rng(14)
    for h in range(2):
        r = rk[h].astype(np.float64)
        assert np.abs(r.T @ r - np.eye(8)).max() <= 1e-6
        assert np.all(np.diff(ek[h]) >= 0)
        assert np.allclose(O.canonical_signs(r), r, atol=1e-7)
        e = rng.standard_normal(8)
        qs = q[2 * h:2 * h + 2].reshape(-1, 8)               # the head's two query heads
        direct = np.mean((qs @ e) ** 2)
        weighted = np.sum(ek[h] * (r.T @ e) ** 2)
        assert np.isclose(direct, weighted, rtol=1e-6)
