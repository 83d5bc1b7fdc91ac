"""Plain CPU oracle for INT2 rotated-latent MLA decode.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: it may
be imported, called or executed only by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The HIP library never links or calls it, and it shares no code, header, table
or helper with the HIP path.

Everything here is written from three web pages:

* [OSCAR-MLA]  OSCAR issue #10, "MLA model support (GLM-5.1 / DeepSeek-style)",
  the maintainer's reply, part "How the rotation adapts to the latent": one
  rotation per MLA layer, fitted on the shared latent c_kv; covariance
  c_kv^T c_kv over calibration tokens; eigh; eigenvectors ordered by ascending
  eigenvalue so that low-variance directions share INT2 groups; clip
  thresholds fitted on the rotated latent; the cache holds the rotated,
  quantised latent and the kv_b_proj up-projection runs on the dequantised
  latent.
* [SHARD-MLA]  shard PR #5, "GLM-5.2 speculative drafting ... + opt-in
  MLA-latent KV cache", TL;DR item 2: the DeepSeek "absorb" form caches the
  latent plus one shared rope key and attends in latent space; it was checked
  equal to full-head attention offline with errors near 1e-13.
* [LLMH-SIZE]  llm-helper PR #64, "hf: size GLM-5.3-Flash's KV cache from its
  latent layers only", PR description: a latent layer stores kv_lora_rank +
  qk_rope_head_dim (+ index_head_dim) values per token.

Precision: fp64 everywhere, except the INT2 quantiser, which runs step by step
in IEEE fp32 (numpy float32 element-wise operations: one rounding per
operation, never a fused multiply-add) because the codes it decides are
compared bit for bit.  Readings of points the pages leave open are marked
"Reading:" and are listed in the design notes of the repository.

Parity status per function (what pins it is in tests/test_oracle_*.py):
all functions below are pinned, except ``fit_clip``'s choice of objective and
grid (the pages print no clip values: parity unpinned against the pages; the
search itself is pinned by brute force) and ``calibrate_rotation_weighted``'s
weighting (a reading of a refinement the pages only name: parity unpinned
against the pages; its reduction to the unweighted rotation, a closed form
and its invariants are pinned).  The sparse decode functions
(``index_scores``, ``index_topk``, ``sparse_absorbed_attention``) follow a
reading of an indexer the pages only name: pinned by brute force, sorting and
the reduction to dense attention, unpinned against the pages.  The rope-key
variant (``quantize_rope_key`` and its entry layout) follows a reading of
designs the pages only name: pinned by brute force, closed forms and
hand-worked bytes, unpinned against the pages.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------


def bf16_round(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returned as float32 arrays holding exactly representable bf16 values.
    Reading: the rotation is applied in bf16 (see ``rotation_apply``).
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    bits = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    out = rounded.astype(np.uint32).view(F32)
    # NaN payloads survive as NaN; infinities are unchanged by the rounding.
    return np.where(np.isnan(a), a, out)


def fp16_round(x) -> np.ndarray:
    """Round float32 values to IEEE binary16 (ties to even); returns float16."""
    return np.asarray(x, dtype=F32).astype(np.float16)


# --------------------------------------------------------------------------
# Calibration: covariance, eigh, ascending order  [OSCAR-MLA]
# --------------------------------------------------------------------------


def latent_covariance(c_cal) -> np.ndarray:
    """Uncentred latent covariance over the calibration tokens, fp64.

    [OSCAR-MLA] writes the estimate as c_kv^T c_kv.  Reading: no mean is
    removed (the page writes none); the 1/N factor only scales the reported
    eigenvalues and leaves the eigenvectors unchanged.
    """
    c = np.asarray(c_cal, dtype=F64)
    n = c.shape[0]
    if n == 0:
        raise ValueError("no calibration tokens")
    return (c.T @ c) / n


def canonical_signs(v) -> np.ndarray:
    """Fix each eigenvector's sign: its largest-magnitude entry is positive.

    Reading: the pages are silent on signs (any sign is an eigenvector); ties
    in magnitude go to the lowest row index.
    """
    v = np.array(v, dtype=F64, copy=True)
    for j in range(v.shape[1]):
        i = int(np.argmax(np.abs(v[:, j])))  # first maximum = lowest row
        if v[i, j] < 0:
            v[:, j] = -v[:, j]
    return v


def calibrate_rotation(c_cal):
    """One orthogonal [r x r] rotation per layer, columns by ascending eigenvalue.

    [OSCAR-MLA]: eigendecompose the latent covariance and order the
    eigenvectors by ascending eigenvalue so that low-variance directions land
    in the same INT2 groups.  Column j of R is the eigenvector of the j-th
    smallest eigenvalue.  Returns (R as float32, eigenvalues as float64,
    R as float64).
    """
    sigma = latent_covariance(c_cal)
    lam, vec = np.linalg.eigh(sigma)  # LAPACK, eigenvalues ascending
    order = np.argsort(lam, kind="stable")
    lam = lam[order]
    vec = canonical_signs(vec[:, order])
    return vec.astype(F32), lam, vec


def upprojection_metric(w_uk, w_uv) -> np.ndarray:
    """Latent-space metric of the kv_b_proj up-projection, fp64.

    [OSCAR-MLA] (closing paragraph, the open refinement): make the latent
    rotation aware of the kv_b_proj up-projection, i.e. shape the INT2 error
    in the latent directions that matter most after reconstruction.  The
    up-projection maps a latent error e to the per-head key parts W_UK[h] e
    and value parts W_UV[h] e, whose total squared size is e^T G e with
    G = sum_h (W_UK[h]^T W_UK[h] + W_UV[h]^T W_UV[h]).
    w_uk [H, d_n, r], w_uv [H, d_v, r].  Reading: keys and values weigh
    equally and queries are not modelled; G is scaled to mean eigenvalue 1
    (trace r), which leaves every eigenvector below unchanged.
    """
    r = np.asarray(w_uk).shape[-1]
    a = np.asarray(w_uk, dtype=F64).reshape(-1, r)
    b = np.asarray(w_uv, dtype=F64).reshape(-1, r)
    g = a.T @ a + b.T @ b
    return g * (r / np.trace(g))


METRIC_RIDGE = 1e-8   # added to G's eigenvalues (G has mean eigenvalue 1)


def metric_inv_sqrt(g) -> np.ndarray:
    """(G + ridge I)^(-1/2) of the symmetric positive semi-definite metric (eigh, fp64).

    Reading: a ridge of 1e-8 of the mean eigenvalue keeps latent directions
    the up-projection ignores finite (they get the largest weighted variance
    and end in the coarsest groups).
    """
    lam, vec = np.linalg.eigh(np.asarray(g, dtype=F64))
    return (vec / np.sqrt(np.maximum(lam, 0.0) + METRIC_RIDGE)) @ vec.T


def calibrate_rotation_weighted(c_cal, w_uk, w_uv):
    """Up-projection-aware rotation (reading of the open refinement).

    [OSCAR-MLA] names, without fixing it, a rotation aware of the kv_b_proj
    up-projection that shapes the INT2 error toward the latent directions
    that matter least after reconstruction.  Reading: take the eigenvectors,
    by ascending eigenvalue and with calibrate_rotation's sign rule, of
    Sigma_w = G^(-1/2) Sigma G^(-1/2), the latent covariance measured against
    the up-projection's metric G.  Directions the up-projection amplifies get
    a small weighted variance and share the first, finest INT2 groups; those
    it ignores come last.  The result is orthogonal, so the cache format, the
    clip fit and decode are unchanged, and for G proportional to the identity
    it is the unweighted rotation.  (Of the weightings tried on synthetic
    up-projections that amplify a few latent directions, this one gave the
    lowest reconstruction error in G's metric; G^(1/2) Sigma G^(1/2) made it
    worse than no weighting.)  Parity unpinned against the pages.
    Returns (R float32, eigenvalues of Sigma_w float64, R float64).
    """
    sigma = latent_covariance(c_cal)
    s = metric_inv_sqrt(upprojection_metric(w_uk, w_uv))
    sw = s @ sigma @ s
    sw = 0.5 * (sw + sw.T)
    lam, vec = np.linalg.eigh(sw)
    order = np.argsort(lam, kind="stable")
    lam = lam[order]
    vec = canonical_signs(vec[:, order])
    return vec.astype(F32), lam, vec


def rotation_apply(r_fp32) -> np.ndarray:
    """The rotation actually applied: bf16(R), round to nearest even.

    Reading: the pages do not fix the precision of the applied rotation; the
    same bf16 matrix rotates the latent, un-rotates it and is folded into the
    absorb weights, so every consumer sees one matrix.
    """
    return bf16_round(r_fp32)


def rotate(c, r_apply) -> np.ndarray:
    """z = c . R_apply per token, computed in fp64 and rounded once to fp32.

    Products of bf16/fp32 values are exact in fp64; the sum is rounded once
    to fp32, the value the quantiser sees.
    """
    return (np.asarray(c, dtype=F64) @ np.asarray(r_apply, dtype=F64)).astype(F32)


# --------------------------------------------------------------------------
# INT2 group quantiser  [OSCAR-MLA]
# --------------------------------------------------------------------------


def group_params(z32, alpha, group, levels=3):
    """Per-(token, group) clip thresholds and fp16 side information, fp32.

    z32:   [n, r] float32 rotated latents.
    alpha: [r/G] clip ratios, one per group (Reading: the fitted clip
           threshold is a ratio of each token's group half-range around its
           mid-point; alpha = 1 is plain asymmetric min-max INT2).
    Per (token, group), in this order, each step rounded to fp32:
      mx, mn = max, min of the group
      mid = 0.5 * (mx + mn);  half = 0.5 * (mx - mn)
      lo = mid - (alpha * half);  hi = mid + (alpha * half)
      scale32 = (hi - lo) / levels   (levels = 3 for INT2 codes 0..3)
      scale_h = fp16(scale32);  zero_h = fp16(lo)
    Returns scale_h, zero_h (float16 [n, r/G]) and scale32, lo (float32, the
    values before the fp16 rounding).
    """
    z32 = np.asarray(z32, dtype=F32)
    n, r = z32.shape
    if r % group:
        raise ValueError("kv_lora_rank must be a multiple of the group size")
    ng = r // group
    a = np.asarray(alpha, dtype=F32).reshape(1, ng)
    zg = z32.reshape(n, ng, group)
    mx = zg.max(axis=2)
    mn = zg.min(axis=2)
    mid = F32(0.5) * (mx + mn)
    half = F32(0.5) * (mx - mn)
    ah = a * half
    lo = mid - ah
    hi = mid + ah
    scale32 = (hi - lo) / F32(levels)
    return fp16_round(scale32), fp16_round(lo), scale32, lo


def codes_from_params(z32, scale_h, zero_h, group, levels=3):
    """Codes of each channel from its group's fp16 scale and zero, fp32.

      u = (z - zero_h) / scale_h   (u = 0 when scale_h == 0)
      code = min(levels, max(0, rint(u)))   rint: ties to even; NaN -> 0
    (levels = 3: the INT2 codes of the latent)
    Reading: the stored fp16 scale and zero are the ones used to quantise, so
    the stored side information and the codes agree.
    Returns codes [n, r] uint8 and u [n, r] float32.
    """
    z32 = np.asarray(z32, dtype=F32)
    n, r = z32.shape
    ng = r // group
    zg = z32.reshape(n, ng, group)
    s = np.asarray(scale_h).astype(F32)[:, :, None]
    z0 = np.asarray(zero_h).astype(F32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (zg - z0) / s
    u = np.where(s == 0, F32(0.0), u).astype(F32)
    code = np.clip(np.rint(u), F32(0.0), F32(levels))
    code = np.where(np.isnan(code), F32(0.0), code)
    return code.astype(np.uint8).reshape(n, r), u.reshape(n, r)


def quantize_groups(z32, alpha, group):
    """Clip + INT2-quantise rotated latents group by group, in IEEE fp32.

    ``group_params`` then ``codes_from_params``.  Returns codes [n, r] uint8
    in 0..3, scale_h and zero_h [n, r/G] float16, and u [n, r] float32 (the
    pre-rounding code value, for boundary bands).
    """
    scale_h, zero_h, _, _ = group_params(z32, alpha, group)
    codes, u = codes_from_params(z32, scale_h, zero_h, group)
    return codes, scale_h, zero_h, u


def pack_codes(codes) -> np.ndarray:
    """Four 2-bit codes per byte: channel 4k+i sits at bits 2i..2i+1 of byte k."""
    c = np.asarray(codes, dtype=np.uint8)
    n, r = c.shape
    if r % 4:
        raise ValueError("channel count must be a multiple of 4")
    q = c.reshape(n, r // 4, 4).astype(np.uint16)
    b = q[:, :, 0] | (q[:, :, 1] << 2) | (q[:, :, 2] << 4) | (q[:, :, 3] << 6)
    return b.astype(np.uint8)


def unpack_codes(packed, r) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    n = p.shape[0]
    out = np.empty((n, r), dtype=np.uint8)
    for i in range(4):
        out[:, i::4] = (p[:, : r // 4] >> (2 * i)) & 3
    return out


def dequantize(codes, scale_h, zero_h, group) -> np.ndarray:
    """z_hat = zero + scale * code, in fp64, from the stored fp16 side info."""
    c = np.asarray(codes, dtype=F64)
    n, r = c.shape
    s = np.repeat(np.asarray(scale_h, dtype=F64), group, axis=1)
    z = np.repeat(np.asarray(zero_h, dtype=F64), group, axis=1)
    return z + s * c


def quantize_cache(c, r_apply, alpha, group):
    """Append path for a block of tokens: rotate, clip, quantise, pack.

    Returns a dict with packed codes [n, r/4] uint8, scale_zero [n, r/G, 2]
    float16 (scale first), unpacked codes, u, the fp32 rotated latent and the
    pre-rounding scale32 and lo.
    """
    z32 = rotate(c, r_apply)
    scale_h, zero_h, scale32, lo = group_params(z32, alpha, group)
    codes, u = codes_from_params(z32, scale_h, zero_h, group)
    sz = np.stack([scale_h, zero_h], axis=-1)
    return dict(packed=pack_codes(codes), scale_zero=sz, codes=codes, u=u,
                z32=z32, scale_h=scale_h, zero_h=zero_h, scale32=scale32,
                lo=lo)


# --------------------------------------------------------------------------
# Clip fit  [OSCAR-MLA: thresholds fitted on the rotated latent]
# --------------------------------------------------------------------------

DEFAULT_ALPHA_GRID = tuple(F32(1.0 - 0.05 * k) for k in range(11))


def group_sse(z32, alpha_value, group) -> np.ndarray:
    """Per-group squared INT2 error over all tokens at one clip ratio, fp64."""
    z32 = np.asarray(z32, dtype=F32)
    ng = z32.shape[1] // group
    alpha = np.full(ng, alpha_value, dtype=F32)
    codes, scale_h, zero_h, _ = quantize_groups(z32, alpha, group)
    zh = dequantize(codes, scale_h, zero_h, group)
    err = (z32.astype(F64) - zh) ** 2
    return err.reshape(err.shape[0], ng, group).sum(axis=(0, 2))


def fit_clip(c_cal, r_fp32, group, grid=DEFAULT_ALPHA_GRID):
    """Per-group clip ratio minimising the squared error of the rotated latent.

    Reading: the pages say only that clip thresholds are fitted on the rotated
    latent.  Objective: sum over calibration tokens of (z - z_hat)^2 per
    group; exhaustive search over ``grid``; exact ties go to the larger ratio.
    Returns (alpha [r/G] float32, sse [r/G, len(grid)] float64).
    """
    z32 = rotate(c_cal, rotation_apply(r_fp32))
    grid = [F32(g) for g in grid]
    sse = np.stack([group_sse(z32, g, group) for g in grid], axis=1)
    ng = sse.shape[0]
    alpha = np.empty(ng, dtype=F32)
    for gi in range(ng):
        best_a, best_e = None, None
        for a, e in zip(grid, sse[gi]):
            if best_e is None or e < best_e or (e == best_e and a > best_a):
                best_a, best_e = a, e
        alpha[gi] = best_a
    return alpha, sse


# --------------------------------------------------------------------------
# Attention  [SHARD-MLA absorb form; OSCAR-MLA up-projection on z_hat]
# --------------------------------------------------------------------------


def visible_len(L, tq, t, causal):
    """Tokens query t of a Tq-token window may see.

    Reading: the Tq queries are the last Tq cache positions of the sequence
    (drafts included in L); with ``causal`` query t sees positions
    0 .. L - Tq + t, otherwise all L positions.
    """
    return (L - tq + t + 1) if causal else L


def _softmax_stats(s):
    m = np.max(s)
    e = np.exp(s - m)
    l = np.sum(e)
    return e / l, m + np.log(l)


def unrotate(z_hat, r_apply) -> np.ndarray:
    """c_hat_tau = R_apply z_hat_tau (columns); rows: c_hat = z_hat R_apply^T."""
    return np.asarray(z_hat, dtype=F64) @ np.asarray(r_apply, dtype=F64).T


def absorbed_attention(q_nope, q_rope, w_uk, w_uv, z_hat, k_rope, r_apply,
                       scale, causal=True):
    """Absorbed MLA decode for one sequence, fp64  [SHARD-MLA].

    q_nope [Tq, H, d_n]; q_rope [Tq, H, d_r]; w_uk [H, d_n, r];
    w_uv [H, d_v, r]; z_hat [L, r] dequantised rotated latent;
    k_rope [L, d_r]; r_apply [r, r].
    Per head: q_lat = W_UK[h]^T q_nope; s_tau = scale (q_lat . c_hat_tau +
    q_rope . k_rope_tau); p = softmax(s); out = W_UV[h] sum_tau p_tau c_hat_tau.
    Returns (out [Tq, H, d_v], lse [Tq, H]).
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    k_rope = np.asarray(k_rope, F64)
    c_hat = unrotate(z_hat, r_apply)
    L = c_hat.shape[0]
    tq, nh, _ = q_nope.shape
    out = np.zeros((tq, nh, w_uv.shape[1]))
    lse = np.full((tq, nh), -np.inf)
    for t in range(tq):
        n_vis = visible_len(L, tq, t, causal)
        if n_vis <= 0:
            continue
        for h in range(nh):
            q_lat = w_uk[h].T @ q_nope[t, h]
            s = scale * (c_hat[:n_vis] @ q_lat + k_rope[:n_vis] @ q_rope[t, h])
            p, lse[t, h] = _softmax_stats(s)
            out[t, h] = w_uv[h] @ (p @ c_hat[:n_vis])
    return out, lse


def full_head_attention(q_nope, q_rope, w_uk, w_uv, z_hat, k_rope, r_apply,
                        scale, causal=True):
    """Reference full-head form: decompress per-head K and V, then attend.

    k_tau[h] = [W_UK[h] c_hat_tau ; k_rope_tau], v_tau[h] = W_UV[h] c_hat_tau,
    q = [q_nope ; q_rope]; out = sum_tau softmax(scale q . k_tau) v_tau.
    This is the decompressed path the absorb form replaces [SHARD-MLA].
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    k_rope = np.asarray(k_rope, F64)
    c_hat = unrotate(z_hat, r_apply)
    L = c_hat.shape[0]
    tq, nh, _ = q_nope.shape
    out = np.zeros((tq, nh, w_uv.shape[1]))
    lse = np.full((tq, nh), -np.inf)
    for h in range(nh):
        k_nope = c_hat @ w_uk[h].T          # [L, d_n]
        v = c_hat @ w_uv[h].T               # [L, d_v]
        k = np.concatenate([k_nope, k_rope], axis=1)
        for t in range(tq):
            n_vis = visible_len(L, tq, t, causal)
            if n_vis <= 0:
                continue
            q = np.concatenate([q_nope[t, h], q_rope[t, h]])
            s = scale * (k[:n_vis] @ q)
            p, lse[t, h] = _softmax_stats(s)
            out[t, h] = p @ v[:n_vis]
    return out, lse


def fold_weights(w, r_apply) -> np.ndarray:
    """W~[h] = W[h] R_apply: folds the un-rotation into a per-head weight."""
    return np.asarray(w, F64) @ np.asarray(r_apply, F64)


def rotated_partials(q_nope, q_rope, w_uk, w_uv, z_hat, k_rope, r_apply,
                     scale, chunks, causal=True):
    """Split-K partials of the rotated-space form, fp64.

    q~ = W~_UK[h]^T q_nope (W~ = W R_apply); s_tau = scale (q~ . z_hat_tau +
    q_rope . k_rope_tau).  For each token chunk [a, b): m = max s,
    l = sum exp(s - m), O = sum exp(s - m) z_hat (all over visible tokens).
    Returns lists of (m [Tq,H], l [Tq,H], O [Tq,H,r]).
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    k_rope = np.asarray(k_rope, F64)
    z_hat = np.asarray(z_hat, F64)
    wk = fold_weights(w_uk, r_apply)                  # [H, d_n, r]
    L, r = z_hat.shape
    tq, nh, _ = q_nope.shape
    q_t = np.einsum("hnr,thn->thr", wk, q_nope)       # [Tq, H, r]
    parts = []
    for a, b in chunks:
        m = np.full((tq, nh), -np.inf)
        l = np.zeros((tq, nh))
        o = np.zeros((tq, nh, r))
        for t in range(tq):
            hi = min(b, visible_len(L, tq, t, causal))
            if hi <= a:
                continue
            s = scale * (q_t[t] @ z_hat[a:hi].T + q_rope[t] @ k_rope[a:hi].T)
            m[t] = s.max(axis=1)
            e = np.exp(s - m[t][:, None])
            l[t] = e.sum(axis=1)
            o[t] = e @ z_hat[a:hi]
        parts.append((m, l, o))
    return parts


def combine_partials(parts, w_uv, r_apply):
    """Log-sum-exp merge of split-K partials, then the up-projection.

    m = max_s m_s; O = sum_s e^(m_s - m) O_s / sum_s e^(m_s - m) l_s;
    out = W~_UV[h] O;  lse = m + log(sum_s e^(m_s - m) l_s).
    """
    ms = np.stack([p[0] for p in parts])
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])
    m = ms.max(axis=0)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(ms), np.exp(ms - m[None]), 0.0)
    den = (w * ls).sum(axis=0)
    num = (w[..., None] * os_).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o_z = np.where(den[..., None] > 0, num / den[..., None], 0.0)
        lse = np.where(den > 0, m + np.log(den), -np.inf)
    wv = fold_weights(w_uv, r_apply)                  # [H, d_v, r]
    out = np.einsum("hvr,thr->thv", wv, o_z)
    return out, lse, o_z


def rotated_attention(q_nope, q_rope, w_uk, w_uv, z_hat, k_rope, r_apply,
                      scale, causal=True, chunk=None):
    """The rotated-space form the GPU computes, single pass or split-K."""
    L = np.asarray(z_hat).shape[0]
    if chunk is None or chunk >= L:
        chunks = [(0, L)]
    else:
        chunks = [(a, min(a + chunk, L)) for a in range(0, L, chunk)]
    parts = rotated_partials(q_nope, q_rope, w_uk, w_uv, z_hat, k_rope,
                             r_apply, scale, chunks, causal)
    out, lse, _ = combine_partials(parts, w_uv, r_apply)
    return out, lse


def default_softmax_scale(d_n, d_r) -> float:
    """Reading: 1/sqrt(qk_nope_head_dim + qk_rope_head_dim), no extra factor."""
    return 1.0 / np.sqrt(d_n + d_r)


# --------------------------------------------------------------------------
# Sparse decode through the indexer key  [LLMH-SIZE: the latent layers of
# GLM-5.3-Flash carry a sparse-attention indexer and cache its key]
# --------------------------------------------------------------------------


def index_scores(q_idx, k_idx) -> np.ndarray:
    """Indexer score of every cached token for one query, fp32.

    Reading (the pages name the indexer and its cached key, nothing more):
    the score of token tau is the dot product of the query's index vector
    q_idx [d_idx] with the token's cached index key k_idx [L, d_idx], both
    bf16-valued, accumulated in IEEE fp32 in channel order e = 0 .. d_idx-1
    (one rounding per addition; each bf16 x bf16 product is exact in fp32).
    """
    q = np.asarray(q_idx, dtype=F32)
    k = np.asarray(k_idx, dtype=F32)
    s = np.zeros(k.shape[0], dtype=F32)
    for e in range(k.shape[1]):
        s = (s + (k[:, e] * q[e]).astype(F32)).astype(F32)
    return s


def score_order_key(scores) -> np.ndarray:
    """Total order on fp32 scores as unsigned integers (larger = higher).

    Sign-magnitude bits mapped to an ordered integer: negative values have
    all bits flipped, non-negative ones get the sign bit set.  This is the
    float order, with -0 just below +0.
    """
    b = np.ascontiguousarray(np.asarray(scores, dtype=F32)).view(np.uint32).astype(np.uint64)
    neg = (b >> np.uint64(31)) == 1
    return np.where(neg, (~b) & np.uint64(0xFFFFFFFF), b | np.uint64(0x80000000))


def index_topk(scores, k) -> np.ndarray:
    """Token indices selected for attention, ascending.

    Reading: the k tokens of highest indexer score; equal scores go to the
    lower token index; fewer than k tokens select them all.
    """
    L = len(scores)
    if k >= L:
        return np.arange(L, dtype=np.int64)
    key = score_order_key(scores)
    order = np.lexsort((np.arange(L), -key.astype(np.float64)))  # key desc, index asc
    # key fits in 32 bits, so the float64 negation above is exact
    return np.sort(order[:k]).astype(np.int64)


def sparse_absorbed_attention(q_nope, q_rope, w_uk, w_uv, z_hat, k_rope, r_apply,
                              scale, selected):
    """Absorbed decode of one query token over the selected tokens only.

    Reading: the indexer's selection replaces the visible window; attention
    over it is the absorbed form above with the unselected tokens left out.
    q_nope [1, H, d_n], q_rope [1, H, d_r]; selected: token indices.
    """
    sel = np.asarray(selected, dtype=np.int64)
    return absorbed_attention(q_nope, q_rope, w_uk, w_uv,
                              np.asarray(z_hat)[sel], np.asarray(k_rope)[sel],
                              r_apply, scale, causal=False)


# --------------------------------------------------------------------------
# Rope-key variant: the shared rope key stored quantised  [OSCAR issue #10,
# the maintainer's later reply: two designs for the rope and the non-rope
# parts of MLA are being benchmarked; neither is described]
# --------------------------------------------------------------------------

ROPE_GROUP = 16
ROPE_BITS = 4


def quantize_rope_key(k_rope, group=ROPE_GROUP, bits=ROPE_BITS):
    """Quantise the shared rope key of each token, fp32 steps.

    Reading: the rope key is kept out of the rotation (the rotation is fitted
    on the latent c_kv only, and the rope key carries the positional
    rotation the scores need as is) and quantised on its own in groups of
    `group` consecutive dims with `bits`-bit codes, by the latent's
    quantiser with no clipping (alpha = 1: the pages fit clip thresholds on
    the rotated latent only) and 2^bits - 1 levels: mid, half, lo = mid -
    half, hi = mid + half, scale = (hi - lo) / (2^bits - 1), fp16 scale and
    zero, code = clamp(rint((x - zero) / scale), 0, 2^bits - 1).
    k_rope [n, d_r] (bf16 values) -> dict with codes [n, d_r], scale_h and
    zero_h [n, d_r/group] (float16), u, scale32, lo and x32 (the fp32 key).
    """
    x32 = np.asarray(k_rope, dtype=F32)
    n, d = x32.shape
    if d % group:
        raise ValueError("qk_rope_head_dim must be a multiple of the rope group")
    levels = (1 << bits) - 1
    alpha = np.ones(d // group, dtype=F32)
    scale_h, zero_h, scale32, lo = group_params(x32, alpha, group, levels)
    codes, u = codes_from_params(x32, scale_h, zero_h, group, levels)
    return dict(codes=codes, scale_h=scale_h, zero_h=zero_h, u=u,
                scale32=scale32, lo=lo, x32=x32)


def rope_entry_bytes(d_r, group=ROPE_GROUP, bits=ROPE_BITS):
    """Bytes of one token's quantised rope key: codes, then (scale, zero)."""
    return d_r * bits // 8 + 4 * (d_r // group)


def pack_rope_entry(codes, scale_h, zero_h):
    """Byte layout of a quantised rope key (4-bit codes): byte k holds dim
    2k in bits 0..3 and dim 2k+1 in bits 4..7; then per group its fp16
    scale and fp16 zero, little-endian.  Returns [n, rope_entry_bytes]."""
    c = np.asarray(codes, dtype=np.uint8)
    n, d = c.shape
    lo_hi = c.reshape(n, d // 2, 2).astype(np.uint16)
    code_bytes = (lo_hi[:, :, 0] | (lo_hi[:, :, 1] << 4)).astype(np.uint8)
    sz = np.stack([np.asarray(scale_h, np.float16), np.asarray(zero_h, np.float16)], axis=-1)
    side = np.ascontiguousarray(sz).view(np.uint8).reshape(n, -1)
    return np.concatenate([code_bytes, side], axis=1)


def unpack_rope_entry(entry, d_r, group=ROPE_GROUP):
    """Inverse of pack_rope_entry: codes [n, d_r], scale_h, zero_h."""
    e = np.asarray(entry, dtype=np.uint8)
    n = e.shape[0]
    cb = e[:, : d_r // 2]
    codes = np.empty((n, d_r), dtype=np.uint8)
    codes[:, 0::2] = cb & 15
    codes[:, 1::2] = cb >> 4
    sz = np.ascontiguousarray(e[:, d_r // 2: d_r // 2 + 4 * (d_r // group)]).view(np.float16)
    sz = sz.reshape(n, d_r // group, 2)
    return codes, sz[..., 0], sz[..., 1]


def dequantize_rope(codes, scale_h, zero_h, group=ROPE_GROUP):
    """k_hat = zero + scale * code, in fp64 (dequantize with the rope group)."""
    return dequantize(codes, scale_h, zero_h, group)


# --------------------------------------------------------------------------
# Cache sizing  [LLMH-SIZE; SHARD-MLA]
# --------------------------------------------------------------------------


def latent_values_per_token(kv_lora_rank, qk_rope_head_dim, index_head_dim=0):
    """Logical cache entry of one latent layer, in values per token."""
    return kv_lora_rank + qk_rope_head_dim + index_head_dim


def full_head_values_per_token(num_heads, qk_nope_head_dim, qk_rope_head_dim,
                               v_head_dim):
    """Decompressed per-head K (nope + rope) and V values per token."""
    return num_heads * (qk_nope_head_dim + qk_rope_head_dim + v_head_dim)


def int2_cache_bytes_per_token(kv_lora_rank, group, qk_rope_head_dim,
                               index_head_dim=0, rope_bits=0):
    """Physical bytes of one token in the INT2 cache (no padding).

    2-bit codes (r/4 bytes) + fp16 scale and zero per group (4 r/G bytes) +
    the rope key: bf16 (2 d_r), or with rope_bits = 4 its quantised entry
    (d_r/2 + 4 d_r/16) + bf16 indexer key (2 d_idx).
    """
    rope = 2 * qk_rope_head_dim if rope_bits == 0 else rope_entry_bytes(qk_rope_head_dim)
    return (kv_lora_rank // 4 + 4 * (kv_lora_rank // group)
            + rope + 2 * index_head_dim)
