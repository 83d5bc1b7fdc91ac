"""Pins for the oracle's sparse (indexer) decode.

The pages name the sparse-attention indexer of GLM-5.3-Flash's latent layers
and its cached key, nothing more, so the score, the selection and the sparse
attention follow a reading (see the oracle).  What pins that reading here:

* ``index_scores`` equals a scalar loop over Python-level fp32 operations in
  the stated order (brute force), and the fp64 dot product within the fp32
  accumulation bound;
* ``index_topk`` equals an independent sort on Python tuples (value, -0
  below +0, lower index first) over small inputs full of ties, and has the
  selection properties on random ones;
* sparse attention over every token is dense attention, bit for bit, and over
  a subset it equals dense attention with the other tokens' scores set to
  minus infinity (a separately written masked softmax).
"""
import math

import numpy as np
import pytest

from oracle import mla_oracle as O


def _bf16(rng, shape):
    return O.bf16_round(rng.standard_normal(shape).astype(np.float32))


def test_index_scores_brute_force():
    rng = np.random.default_rng(5)
    q = _bf16(rng, 12)
    k = _bf16(rng, (9, 12))
    got = O.index_scores(q, k)
    for t in range(9):
        acc = np.float32(0.0)
        for e in range(12):
            acc = np.float32(acc + np.float32(np.float32(k[t, e]) * np.float32(q[e])))
        assert got[t] == acc and got.dtype == np.float32


def test_index_scores_close_to_exact_dot():
    rng = np.random.default_rng(6)
    q = _bf16(rng, 64)
    k = _bf16(rng, (500, 64))
    got = O.index_scores(q, k).astype(np.float64)
    exact = k.astype(np.float64) @ q.astype(np.float64)
    bound = 64 * np.finfo(np.float32).eps * (np.abs(k.astype(np.float64)) @ np.abs(q.astype(np.float64)))
    assert np.all(np.abs(got - exact) <= bound)


def _brute_topk(scores, k):
    items = []
    for t, v in enumerate(scores.tolist()):
        neg_zero = 1 if (v == 0.0 and math.copysign(1.0, v) < 0) else 0
        items.append((-v, neg_zero, t))
    items.sort()
    return sorted(t for _, _, t in items[:k])


@pytest.mark.parametrize("seed", range(6))
def test_index_topk_matches_independent_sort(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 40))
    scores = rng.choice(np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0], np.float32), size=L)
    for k in (1, 2, 5, L - 1, L, L + 3):
        if k < 1:
            continue
        assert O.index_topk(scores, k).tolist() == _brute_topk(scores, k)


def test_index_topk_properties():
    rng = np.random.default_rng(7)
    scores = rng.standard_normal(5000).astype(np.float32)
    scores[100:120] = scores[3]             # ties
    sel = O.index_topk(scores, 777)
    assert len(sel) == 777 and np.all(np.diff(sel) > 0)
    mask = np.zeros(len(scores), bool)
    mask[sel] = True
    assert scores[mask].min() >= scores[~mask].max()
    thr = scores[mask].min()
    tied = np.nonzero(scores == thr)[0]
    taken = tied[mask[tied]]
    # among tokens with the threshold score, the lower indices are taken
    assert np.all(taken <= tied[~mask[tied]].min()) if (~mask[tied]).any() else True


def _attn_case(seed, L=50, H=3, r=16, d_n=8, d_r=4, d_v=5):
    rng = np.random.default_rng(seed)
    qn = rng.standard_normal((1, H, d_n))
    qr = rng.standard_normal((1, H, d_r))
    wuk = rng.standard_normal((H, d_n, r)) / np.sqrt(r)
    wuv = rng.standard_normal((H, d_v, r)) / np.sqrt(r)
    R, _, _ = O.calibrate_rotation(rng.standard_normal((4 * r, r)) * np.linspace(0.1, 2, r))
    Ra = O.rotation_apply(R)
    zh = rng.standard_normal((L, r))
    kr = rng.standard_normal((L, d_r))
    return qn, qr, wuk, wuv, zh, kr, Ra, O.default_softmax_scale(d_n, d_r)


def test_sparse_over_all_tokens_is_dense():
    qn, qr, wuk, wuv, zh, kr, Ra, sc = _attn_case(1)
    L = zh.shape[0]
    o_s, l_s = O.sparse_absorbed_attention(qn, qr, wuk, wuv, zh, kr, Ra, sc, np.arange(L))
    o_d, l_d = O.absorbed_attention(qn, qr, wuk, wuv, zh, kr, Ra, sc, causal=False)
    assert np.array_equal(o_s, o_d) and np.array_equal(l_s, l_d)


def test_sparse_equals_masked_dense():
    qn, qr, wuk, wuv, zh, kr, Ra, sc = _attn_case(2)
    L = zh.shape[0]
    sel = np.sort(np.random.default_rng(3).choice(L, 17, replace=False))
    o_s, l_s = O.sparse_absorbed_attention(qn, qr, wuk, wuv, zh, kr, Ra, sc, sel)
    # masked dense, written out: decompress the latent, score every token,
    # minus infinity outside the selection
    c_hat = zh @ Ra.astype(np.float64).T
    keep = np.zeros(L, bool)
    keep[sel] = True
    for h in range(qn.shape[1]):
        s = sc * (c_hat @ (wuk[h].T @ qn[0, h]) + kr @ qr[0, h])
        s = np.where(keep, s, -np.inf)
        m = s.max()
        e = np.exp(s - m)
        ref = wuv[h] @ ((e / e.sum()) @ c_hat)
        assert np.allclose(o_s[0, h], ref, rtol=1e-12, atol=1e-14)
        assert abs(l_s[0, h] - (m + np.log(e.sum()))) <= 1e-12
