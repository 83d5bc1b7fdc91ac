"""Parity at the full workload sizes, in the configuration the benchmark times.

For each DeepSeek-V3 / GLM-5.3-Flash shaped workload the whole cache is
built through the library exactly as ``bench.py`` builds it (same seeded
latents, rope keys, indexer keys and queries, one append of every token,
then ``mla_decode_absorbed`` with the default kernel choice).  The oracle
then re-does one seeded sequence end to end: it quantises the whole
sequence itself and computes attention for every head and query token of
that sequence (rotated-space form; the absorbed form on a seeded sample of
heads as well).  Checked:

* the sequence's INT2 codes and fp16 side info (bit-exact outside the
  1e-5 boundary band / fp16-midpoint rule), and its rope and indexer keys;
* every output row of the sequence (per-row max relative error <= 2e-3) and lse.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int2_quantized_absorbed_amd as M
from oracle import mla_oracle as O
from workloads import synth as S

from tests import gpu_cases as C
from tests.parity import LSE_TOL, OUT_RTOL, compare_append, row_rel_err

pytestmark = pytest.mark.gpu

HEADS_SAMPLED = 4


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_full_size_sampled(wid):
    w = S.WORKLOADS[wid]
    C.say(f"full-size workload {wid} ({w.name})")
    layer = C.Layer(w)
    d = layer.dims
    lens = S.seq_lens(w, layer.st)
    base, cap = S.contiguous_layout(lens)
    B, tq, H = len(lens), w.tq, w.num_heads
    lat = S.torch_latents(layer.model, cap, seed=1000 + wid, device=C.DEV)
    kr = S.torch_normal_bf16((cap, w.qk_rope_head_dim), 2000 + wid, C.DEV)
    idx = S.torch_normal_bf16((cap, w.index_head_dim), 3000 + wid, C.DEV) if w.index_head_dim else None
    cache = M.Cache(d, cap, C.DEV)
    M.mla_append_quant(d, lat, kr, idx, torch.arange(cap, dtype=torch.int64, device=C.DEV), layer.Rt_d,
                       layer.alpha_d, cache)
    qn = S.torch_normal_bf16((B, tq, H, w.qk_nope_head_dim), 4000 + wid, C.DEV)
    qr = S.torch_normal_bf16((B, tq, H, w.qk_rope_head_dim), 5000 + wid, C.DEV)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    out, lse = M.mla_decode_absorbed(d, qn, qr, layer.w_uk_f, layer.w_uv_f, cache, torch.from_numpy(base).to(C.DEV),
                                     torch.from_numpy(lens).to(C.DEV), tq, w.causal, scale)
    torch.cuda.synchronize()
    C.say(f"  GPU done: {cap} cached tokens, batch {B}, tq {tq}")

    rng = np.random.default_rng(100 + wid)
    b = int(rng.integers(B))
    heads = np.sort(rng.choice(H, HEADS_SAMPLED, replace=False))
    a, L = int(base[b]), int(lens[b])
    seg = lat[a:a + L].float().cpu().numpy()
    kr_seg = kr[a:a + L].float().cpu().numpy()

    ref = O.quantize_cache(seg, layer.R_apply, layer.alpha, w.group_size)
    stats = compare_append(cache.codes[a:a + L].cpu().numpy(), cache.scale_zero[a:a + L].cpu().numpy(), ref,
                           w.group_size)
    C.say(f"  append, sequence {b} ({L} tokens):", {k: stats[k] for k in ("n", "code_mismatch", "excused",
                                                                         "violations", "sz_diff", "sz_violations")})
    assert stats["violations"] == 0 and stats["sz_violations"] == 0, stats
    assert np.array_equal(cache.k_rope[a:a + L].float().cpu().numpy(), kr_seg)
    if idx is not None:
        assert torch.equal(cache.idx_key[a:a + L], idx[a:a + L])

    zh = O.dequantize(ref["codes"], ref["scale_h"], ref["zero_h"], w.group_size)
    # every head and every query token of the sequence, in the oracle's
    # rotated-space form (equal to the absorbed form, pinned in fp64)
    o_ref, lse_ref = O.rotated_attention(qn[b].float().cpu().numpy(), qr[b].float().cpu().numpy(), layer.w_uk,
                                         layer.w_uv, zh, kr_seg, layer.R_apply, scale, causal=w.causal)
    o_gpu = out[b].cpu().numpy()
    lse_gpu = lse[b].cpu().numpy()
    err = row_rel_err(o_gpu, o_ref)
    C.say(f"  decode, sequence {b}, all {H} heads x {tq} queries: worst row rel err {float(np.max(err)):.3e}, "
          f"lse max abs diff {float(np.max(np.abs(lse_gpu - lse_ref))):.3e}")
    assert np.all(err <= OUT_RTOL), err
    assert np.all(np.abs(lse_gpu - lse_ref) <= LSE_TOL * np.maximum(1, np.abs(lse_ref)))
    # and the oracle's absorbed form itself on a seeded sample of heads
    o_abs, _ = O.absorbed_attention(qn[b][:, heads].float().cpu().numpy(), qr[b][:, heads].float().cpu().numpy(),
                                    layer.w_uk[heads], layer.w_uv[heads], zh, kr_seg, layer.R_apply, scale,
                                    causal=w.causal)
    assert np.all(row_rel_err(o_gpu[:, heads], o_abs) <= OUT_RTOL)


def test_full_size_sparse():
    """Sparse decode at the size bench.py times it: GLM-5.3-Flash-shaped
    layer (64 heads, 64-dim indexer key), 4 x 262,144 tokens, top-2048.
    Every sequence's selection is compared with the oracle's element by
    element; the decode output of one seeded sequence (sampled heads) against
    the oracle's sparse attention over that selection."""
    w = S.WORKLOADS[4]
    top_k = 2048
    C.say(f"full-size sparse decode ({w.name}, top_k {top_k})")
    layer = C.Layer(w)
    d = layer.dims
    lens = S.seq_lens(w, layer.st)
    base, cap = S.contiguous_layout(lens)
    B, H = len(lens), w.num_heads
    lat = S.torch_latents(layer.model, cap, seed=1104, device=C.DEV)
    kr = S.torch_normal_bf16((cap, w.qk_rope_head_dim), 2104, C.DEV)
    idx = S.torch_normal_bf16((cap, w.index_head_dim), 3104, C.DEV)
    cache = M.Cache(d, cap, C.DEV)
    M.mla_append_quant(d, lat, kr, idx, torch.arange(cap, dtype=torch.int64, device=C.DEV), layer.Rt_d,
                       layer.alpha_d, cache)
    q_idx = S.torch_normal_bf16((B, w.index_head_dim), 9104, C.DEV)
    qn = S.torch_normal_bf16((B, 1, H, w.qk_nope_head_dim), 4104, C.DEV)
    qr = S.torch_normal_bf16((B, 1, H, w.qk_rope_head_dim), 5104, C.DEV)
    sb = torch.from_numpy(base).to(C.DEV)
    sel, n_sel = M.mla_index_topk(d, q_idx, cache, sb, torch.from_numpy(lens).to(C.DEV), top_k)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    out, lse = M.mla_decode_sparse(d, qn, qr, layer.w_uk_f, layer.w_uv_f, cache, sb, sel, n_sel, scale)
    torch.cuda.synchronize()
    C.say(f"  GPU done: {cap} cached tokens, batch {B}")
    sel_h, n_h = sel.cpu().numpy(), n_sel.cpu().numpy()
    q_h = q_idx.float().cpu().numpy()
    refs = []
    for b in range(B):
        a, L = int(base[b]), int(lens[b])
        ref = O.index_topk(O.index_scores(q_h[b], idx[a:a + L].float().cpu().numpy()), top_k)
        assert n_h[b] == len(ref) and np.array_equal(sel_h[b, :n_h[b]], ref), b
        refs.append(ref)
    C.say("  selections equal the oracle's for every sequence")

    rng = np.random.default_rng(104)
    b = int(rng.integers(B))
    heads = np.sort(rng.choice(H, HEADS_SAMPLED, replace=False))
    a = int(base[b])
    rows = torch.from_numpy(a + refs[b]).to(C.DEV)
    seg = lat[rows].float().cpu().numpy()
    # the selected tokens' cache entries against the oracle's quantiser (codes
    # bit-exact outside the boundary band) ...
    ref_q = O.quantize_cache(seg, layer.R_apply, layer.alpha, w.group_size)
    codes_g, sz_g = cache.codes[rows].cpu().numpy(), cache.scale_zero[rows].cpu().numpy()
    stats = compare_append(codes_g, sz_g, ref_q, w.group_size)
    assert stats["violations"] == 0 and stats["sz_violations"] == 0, stats
    # ... then attention on those entries: with 2048 tokens a code that may
    # legitimately differ at a rounding boundary (an outlier channel's step is
    # several units) would move the output by more than the decode tolerance,
    # so the decode is judged on the entries the cache holds
    zh = O.dequantize(O.unpack_codes(codes_g, w.kv_lora_rank), sz_g[..., 0].astype(np.float64),
                      sz_g[..., 1].astype(np.float64), w.group_size)
    o_ref, lse_ref = O.sparse_absorbed_attention(qn[b][:, heads].float().cpu().numpy(),
                                                 qr[b][:, heads].float().cpu().numpy(),
                                                 layer.w_uk[heads], layer.w_uv[heads], zh,
                                                 kr[rows].float().cpu().numpy(), layer.R_apply, scale,
                                                 np.arange(len(refs[b])))
    o_gpu = out[b][:, heads].cpu().numpy()
    err = row_rel_err(o_gpu, o_ref)
    C.say(f"  sparse decode, sequence {b}, heads {heads.tolist()}: worst row rel err {float(np.max(err)):.3e}")
    assert np.all(err <= OUT_RTOL), err
    lse_gpu = lse[b][:, heads].cpu().numpy()
    assert np.all(np.abs(lse_gpu - lse_ref) <= LSE_TOL * np.maximum(1, np.abs(lse_ref)))
