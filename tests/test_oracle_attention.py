"""Pins for the oracle's attention forms.

* The absorbed, full-head and rotated-space forms are three different
  computations of one quantity (associativity); they must agree to 1e-12 in
  fp64 (the shard page reports about 1e-13 for its own offline check).
* The full-head form is checked against torch's scaled_dot_product_attention
  on the CPU in fp64, with K and V built by the test itself.
* A signed-permutation rotation (exact in bf16) checks the orientation of the
  un-rotation against plain attention on the un-rotated latent.
* Split-K with any chunking equals the single pass.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mla_oracle as O
from workloads import synth as S


def _case(seed, L=40, tq=1, H=3, r=24, d_n=8, d_r=4, d_v=6, quantized=True):
    rng = np.random.default_rng(seed)
    qn = rng.standard_normal((tq, H, d_n))
    qr = rng.standard_normal((tq, H, d_r))
    wuk = rng.standard_normal((H, d_n, r)) / np.sqrt(r)
    wuv = rng.standard_normal((H, d_v, r)) / np.sqrt(r)
    c = rng.standard_normal((L, r)).astype(np.float32)
    R, _, _ = O.calibrate_rotation(rng.standard_normal((4 * r, r)) * np.linspace(0.1, 2, r))
    Ra = O.rotation_apply(R)
    if quantized:
        q = O.quantize_cache(c, Ra, np.full(r // 4, 0.9, np.float32), 4)
        zh = O.dequantize(q["codes"], q["scale_h"], q["zero_h"], 4)
    else:
        zh = c.astype(np.float64) @ Ra.astype(np.float64)
    kr = rng.standard_normal((L, d_r))
    scale = O.default_softmax_scale(d_n, d_r)
    return qn, qr, wuk, wuv, zh, kr, Ra, scale


@pytest.mark.parametrize("tq,causal", [(1, True), (4, True), (4, False)])
@pytest.mark.parametrize("quantized", [True, False])
def test_three_forms_agree(tq, causal, quantized):
    args = _case(20 + tq, tq=tq, quantized=quantized)
    a, la = O.absorbed_attention(*args, causal=causal)
    f, lf = O.full_head_attention(*args, causal=causal)
    r, lr = O.rotated_attention(*args, causal=causal)
    for x in (f, r):
        assert np.max(np.abs(x - a)) <= 1e-12 * np.max(np.abs(a))
    for x in (lf, lr):
        assert np.max(np.abs(x - la)) <= 1e-12 * np.max(np.abs(la))


@pytest.mark.parametrize("tq,causal", [(1, True), (3, True), (3, False)])
def test_full_head_matches_torch_sdpa(tq, causal):
    qn, qr, wuk, wuv, zh, kr, Ra, scale = _case(30 + tq, L=33, tq=tq)
    out, lse = O.full_head_attention(qn, qr, wuk, wuv, zh, kr, Ra, scale, causal)
    # build K, V, Q here, independently of the oracle
    c_hat = zh @ Ra.astype(np.float64).T                # un-rotated latent
    H = qn.shape[1]
    L = zh.shape[0]
    for h in range(H):
        k = np.concatenate([c_hat @ wuk[h].T, kr], axis=1)    # [L, d_n + d_r]
        v = c_hat @ wuv[h].T
        q = np.concatenate([qn[:, h], qr[:, h]], axis=1)      # [tq, d]
        mask = None
        if causal:
            pos = np.arange(L)[None, :]
            lim = (L - tq + np.arange(tq))[:, None]
            mask = torch.from_numpy(pos <= lim)
        want = F.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None],
            torch.from_numpy(v)[None], attn_mask=mask, scale=scale)[0].numpy()
        assert np.max(np.abs(out[:, h] - want)) <= 1e-12 * np.max(np.abs(want))
        s = scale * (q @ k.T)
        if causal:
            s = np.where(mask.numpy(), s, -np.inf)
        want_lse = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
        np.testing.assert_allclose(lse[:, h], want_lse, rtol=1e-13, atol=1e-13)


def test_orientation_with_signed_permutation():
    """R_apply = signed permutation (exact in bf16): attention over the rotated
    cache equals plain MLA attention over the original latent."""
    rng = np.random.default_rng(40)
    r, L, H, d_n, d_r, d_v = 12, 17, 2, 5, 3, 4
    perm = rng.permutation(r)
    P = np.zeros((r, r), np.float32)
    P[np.arange(r), perm] = rng.choice([-1.0, 1.0], size=r)
    c = rng.standard_normal((L, r))
    z = c @ P                                       # rotated latent, exact
    qn = rng.standard_normal((1, H, d_n))
    qr = rng.standard_normal((1, H, d_r))
    wuk = rng.standard_normal((H, d_n, r))
    wuv = rng.standard_normal((H, d_v, r))
    kr = rng.standard_normal((L, d_r))
    scale = 0.3
    out, _ = O.absorbed_attention(qn, qr, wuk, wuv, z, kr, P, scale)
    for h in range(H):
        s = scale * ((c @ wuk[h].T) @ qn[0, h] + kr @ qr[0, h])
        p = np.exp(s - s.max())
        p /= p.sum()
        want = wuv[h] @ (p @ c)
        np.testing.assert_allclose(out[0, h], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 5, 16, 39])
def test_split_k_equals_single_pass(chunk):
    args = _case(50, L=40, tq=4)
    a, la = O.rotated_attention(*args, causal=True)
    b, lb = O.rotated_attention(*args, causal=True, chunk=chunk)
    assert np.max(np.abs(a - b)) <= 1e-13 * np.max(np.abs(a))
    assert np.max(np.abs(la - lb)) <= 1e-13 * np.max(np.abs(la))


def test_split_k_fully_masked_chunk():
    """A chunk that a draft query cannot see contributes nothing."""
    args = _case(51, L=12, tq=4)
    parts = O.rotated_partials(*args, chunks=[(0, 9), (9, 10), (10, 12)],
                               causal=True)
    m, l, o = parts[2]
    # positions 10, 11 are visible only to queries t >= 2
    assert np.all(l[:2] == 0) and np.all(np.isneginf(m[:2]))
    out, lse, _ = O.combine_partials(parts, args[3], args[6])
    want, wl = O.rotated_attention(*args, causal=True)
    assert np.max(np.abs(out - want)) <= 1e-13 * np.max(np.abs(want))
