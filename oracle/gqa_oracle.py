"""Plain CPU oracle for OSCAR on full-attention (grouped-query) layers.

TEST INFRASTRUCTURE ONLY, like ``oracle/mla_oracle.py`` (whose number-format,
eigh, sign and quantiser functions it reuses): it may be imported, called or
executed only by ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline``; the HIP library shares nothing with it.

Written from [OSCAR-MLA] (OSCAR issue #10, "MLA model support (GLM-5.1 /
DeepSeek-style)", the maintainer's reply, part "How the rotation adapts to the
latent", first point): for full-attention models OSCAR fits two
covariance-aware rotations per layer that act per KV head - a
query-covariance rotation for K and a score-weighted V-covariance rotation
for V.  Everything the page leaves open is marked "Reading:".

Layout: H_q query heads, H_kv KV heads, query head g reads KV head
g // (H_q / H_kv); head dimension d for queries, keys and values.
Calibration inputs are head-major: q [H_q, N, d], k and v [H_kv, N, d]; they
are one calibration sequence of N tokens.

Parity status: the readings (the order of the eigenvectors, the causal
score weights) are pinned by closed forms, invariants and brute force, not
against the pages, which print no numbers for this path.
"""
from __future__ import annotations

import numpy as np

from oracle import mla_oracle as O

F64 = np.float64


def group_of(n_q, n_kv):
    """Query heads per KV head (grouped-query attention)."""
    assert n_q % n_kv == 0
    return n_q // n_kv


def query_covariance(q_cal, n_kv) -> np.ndarray:
    """Per KV head: the uncentred covariance of the queries that read it.

    Sigma_q[h] = (1 / (N G)) sum over calibration tokens i and the G query
    heads g of KV head h of q_{g,i} q_{g,i}^T, fp64.  The score error a
    quantisation error e of a key causes is q . e, with mean square
    e^T Sigma_q e: this is the metric the K rotation is fitted to.
    """
    q = np.asarray(q_cal, F64)
    n_q, n, d = q.shape
    G = group_of(n_q, n_kv)
    out = np.zeros((n_kv, d, d))
    for h in range(n_kv):
        rows = q[h * G:(h + 1) * G].reshape(G * n, d)
        out[h] = rows.T @ rows / (G * n)
    return out


def score_weights(q_cal, k_cal, scale) -> np.ndarray:
    """Attention mass each calibration key receives, per KV head, fp64.

    Reading: the calibration tokens form one sequence under causal
    self-attention (query i sees keys 0..i); w[h, t] = sum over queries
    i >= t and the G query heads g of KV head h of softmax_t(scale
    q_{g,i} . k_{h,t}).  Each (query, head) pair contributes a total of 1.
    """
    q = np.asarray(q_cal, F64)
    k = np.asarray(k_cal, F64)
    n_q, n, _ = q.shape
    n_kv = k.shape[0]
    G = group_of(n_q, n_kv)
    w = np.zeros((n_kv, n))
    for g in range(n_q):
        h = g // G
        s = scale * (q[g] @ k[h].T)                     # [query i, key t]
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        w[h] += (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
    return w


def value_covariance(v_cal, w) -> np.ndarray:
    """Score-weighted V covariance per KV head: sum_t w_t v_t v_t^T / sum_t w_t."""
    v = np.asarray(v_cal, F64)
    w = np.asarray(w, F64)
    return np.einsum("ht,htd,hte->hde", w, v, v) / w.sum(axis=1)[:, None, None]


def key_covariance(k_cal) -> np.ndarray:
    """Per KV head: the uncentred covariance of its calibration keys, fp64."""
    k = np.asarray(k_cal, F64)
    return np.einsum("hnd,hne->hde", k, k) / k.shape[1]


METRIC_RIDGE = 1e-8


def metric_weighted(sigma_data, metric) -> np.ndarray:
    """M^(-1/2) Sigma M^(-1/2), with M scaled to mean eigenvalue 1 and a
    ridge so directions no query reads stay finite (the same whitening as the
    up-projection-aware latent rotation)."""
    m = np.asarray(metric, F64)
    m = m * (m.shape[0] / np.trace(m))
    lam, vec = np.linalg.eigh(m)
    s = (vec / np.sqrt(np.maximum(lam, 0.0) + METRIC_RIDGE)) @ vec.T
    w = s @ np.asarray(sigma_data, F64) @ s
    return 0.5 * (w + w.T)


def rotation_from_covariance(sigma):
    """Eigenvectors by ascending eigenvalue, signs as the MLA rotation.

    Reading: the same order and sign rule as the latent rotation, so the
    directions of smallest weight share the first INT2 groups.
    Returns (R fp32 [d, d], eigenvalues fp64 [d]).
    """
    lam, vec = np.linalg.eigh(np.asarray(sigma, F64))
    vec = O.canonical_signs(vec)
    return vec.astype(np.float32), lam


K_QUERY_COVARIANCE = 0   # the K rotation's plain reading (the default)
K_QUERY_METRIC = 1       # the refinement: key covariance in the query metric


def calibrate(q_cal, k_cal, v_cal, scale, k_rotation=K_QUERY_COVARIANCE):
    """Both rotations of every KV head.

    "A query-covariance rotation for K", plain reading (K_QUERY_COVARIANCE):
    the eigenvectors of the query covariance Sigma_q of the KV head's query
    heads, ascending.  A key error e costs the score error q . e, of mean
    square e^T Sigma_q e; in this basis that is the eigenvalue-weighted sum of
    the rotated channels' squared errors, so channels of equal weight share
    the INT2 groups.  The refinement (K_QUERY_METRIC) also follows where the
    keys vary: the eigenvectors of Sigma_q^(-1/2) Sigma_k Sigma_q^(-1/2)
    (Sigma_k the keys' own covariance, Sigma_q scaled to mean eigenvalue 1),
    ascending - the construction of the up-projection-aware latent rotation,
    with the queries in the role of the up-projection.
    "A score-weighted V-covariance rotation": the eigenvectors of the value
    covariance weighted by the attention mass each calibration token
    receives, ascending.
    Returns (R_k [H_kv, d, d], eig_k [H_kv, d], R_v, eig_v, w).
    """
    assert k_rotation in (K_QUERY_COVARIANCE, K_QUERY_METRIC)
    n_kv = np.asarray(k_cal).shape[0]
    sq = query_covariance(q_cal, n_kv)
    sk = key_covariance(k_cal)
    w = score_weights(q_cal, k_cal, scale)
    sv = value_covariance(v_cal, w)
    rk, ek, rv, ev = [], [], [], []
    for h in range(n_kv):
        sk_h = sq[h] if k_rotation == K_QUERY_COVARIANCE else metric_weighted(sk[h], sq[h])
        r, e = rotation_from_covariance(sk_h)
        rk.append(r)
        ek.append(e)
        r, e = rotation_from_covariance(sv[h])
        rv.append(r)
        ev.append(e)
    return np.stack(rk), np.stack(ek), np.stack(rv), np.stack(ev), w


def quantize_heads(x, r_apply, alpha, group):
    """INT2 entries of head-major rows x [H_kv, n, d] in each head's rotated
    basis (the MLA quantiser per head).  Returns a list of per-head dicts."""
    return [O.quantize_cache(np.asarray(x[h], np.float32), r_apply[h], alpha[h], group)
            for h in range(np.asarray(x).shape[0])]


def dequantize_heads(q_list, group) -> np.ndarray:
    """z_hat [H_kv, n, d] (rotated basis), fp64."""
    return np.stack([O.dequantize(q["codes"], q["scale_h"], q["zero_h"], group) for q in q_list])


def gqa_attention(q, k, v, scale, causal=True):
    """Plain grouped-query decode attention, fp64.

    q [Tq, H_q, d]; k, v [H_kv, L, d] (un-rotated).  The Tq queries are the
    last Tq positions; with ``causal`` query t sees keys 0 .. L - Tq + t.
    Returns (out [Tq, H_q, d], lse [Tq, H_q]) with the natural-log lse.
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    tq, n_q, _ = q.shape
    n_kv, L, _ = k.shape
    G = group_of(n_q, n_kv)
    out = np.zeros((tq, n_q, v.shape[2]))
    lse = np.full((tq, n_q), -np.inf)
    for t in range(tq):
        n_vis = O.visible_len(L, tq, t, causal)
        if n_vis <= 0:
            continue
        for g in range(n_q):
            h = g // G
            s = scale * (k[h, :n_vis] @ q[t, g])
            m = s.max()
            e = np.exp(s - m)
            out[t, g] = (e / e.sum()) @ v[h, :n_vis]
            lse[t, g] = m + np.log(e.sum())
    return out, lse


def rotated_attention(q, zk_hat, zv_hat, rk_apply, rv_apply, scale, causal=True):
    """The rotated-space form the GPU computes, fp64.

    With k_hat = z_k_hat R_k^T and v_hat = z_v_hat R_v^T (R = the applied bf16
    rotations), q . k_hat = (q R_k) . z_k_hat and sum p v_hat =
    (sum p z_v_hat) R_v^T: the query is rotated once, the output un-rotated
    once, and attention runs on the cached entries directly.
    """
    q = np.asarray(q, F64)
    rk = np.asarray(rk_apply, F64)
    rv = np.asarray(rv_apply, F64)
    n_kv = rk.shape[0]
    G = group_of(q.shape[1], n_kv)
    q_t = np.stack([q[:, g] @ rk[g // G] for g in range(q.shape[1])], axis=1)
    o_z, lse = gqa_attention(q_t, zk_hat, zv_hat, scale, causal)
    out = np.stack([o_z[:, g] @ rv[g // G].T for g in range(q.shape[1])], axis=1)
    return out, lse


def unrotate_heads(z_hat, r_apply) -> np.ndarray:
    """x_hat [H_kv, n, d] = z_hat R_apply^T per head."""
    return np.einsum("hnd,hed->hne", np.asarray(z_hat, F64), np.asarray(r_apply, F64))
