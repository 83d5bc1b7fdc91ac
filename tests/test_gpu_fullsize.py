"""Parity at the full workload sizes, in the configuration the benchmark times.

For each DeepSeek-V3 / GLM-5.3-Flash shaped workload the whole cache is
built through the library exactly as ``bench.py`` builds it (same seeded
latents, rope keys, indexer keys and queries, one append of every token,
then ``mla_decode_absorbed`` with the default kernel choice).  The oracle
then re-does one seeded sequence end to end: it quantises the whole
sequence itself and computes absorbed attention for a seeded sample of
heads (every query token of that sequence).  Checked:

* the sequence's INT2 codes and fp16 side info (bit-exact outside the
  1e-5 boundary band / fp16-midpoint rule), and its rope and indexer keys;
* the sampled output rows (per-row max relative error <= 2e-3) and lse.
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
    qn_b = qn[b][:, heads].float().cpu().numpy()
    qr_b = qr[b][:, heads].float().cpu().numpy()
    o_ref, lse_ref = O.absorbed_attention(qn_b, qr_b, layer.w_uk[heads], layer.w_uv[heads], zh, kr_seg,
                                          layer.R_apply, scale, causal=w.causal)
    o_gpu = out[b][:, heads].cpu().numpy()
    lse_gpu = lse[b][:, heads].cpu().numpy()
    err = row_rel_err(o_gpu, o_ref)
    C.say(f"  decode, sequence {b}, heads {heads.tolist()}: worst row rel err {float(np.max(err)):.3e}, "
          f"lse max abs diff {float(np.max(np.abs(lse_gpu - lse_ref))):.3e}")
    assert np.all(err <= OUT_RTOL), err
    assert np.all(np.abs(lse_gpu - lse_ref) <= LSE_TOL * np.maximum(1, np.abs(lse_ref)))
