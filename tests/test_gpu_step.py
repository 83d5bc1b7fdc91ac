"""The combined decode step (mla_decode_step) against the two calls it
stands for: mla_append_quant of the step's new tokens followed by
mla_decode_absorbed over the cache that holds them.  Both paths of the step
are covered: the small append run by blocks of the query-absorb launch, and
the fallback (a large append, or the vector-ALU decode) that runs the two
one after the other.  The cache bytes must be identical, and so must out and
lse (the decode kernels are the same; only their inputs could differ)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int2_quantized_absorbed_amd as M
from workloads import synth as S

from . import gpu_cases as C

pytestmark = pytest.mark.gpu

STEP_CASES = [
    # name, workload, overrides, lens, tq, causal, new tokens per sequence
    ("g32-fused", 1, dict(num_heads=16), [300, 1, 77, 1024], 1, True, 1),
    ("g16-fused", 1, dict(num_heads=16, group_size=16), [40, 513, 64], 2, True, 2),
    ("idx-fused", 4, dict(num_heads=16), [130, 65], 1, True, 1),
    ("g32-fused-2tiles", 1, dict(num_heads=16), [300, 500], 1, True, 20),  # 40 tokens: a ragged second tile
    ("idx-fused-2tiles", 4, dict(num_heads=16), [130, 65, 90], 1, True, 11),  # 33 tokens
    ("large-append", 1, dict(num_heads=16), [700, 600], 1, True, 550),   # 1100 tokens: separate append
    ("valu-decode", 0, dict(), [100, 37], 1, True, 1),                     # r = 64: vector-ALU decode
]


@pytest.mark.parametrize("name,wid,over,lens,tq,causal,new", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_equals_separate_calls(name, wid, over, lens, tq, causal, new):
    w = S.WORKLOADS[wid].with_(**over)
    C.say(f"decode_step {name} lens={lens} tq={tq} new={new}")
    layer = C.Layer(w)
    d = layer.dims
    rng = np.random.default_rng(23)
    base, cap = S.contiguous_layout(lens, 5)
    lat_all = C.latent_tensor(layer.model.sample(rng, cap), w.latent_dtype)
    kr_all = C.t_bf16(S.rope_keys(rng, cap, w.qk_rope_head_dim))
    idx_all = C.t_bf16(S.rope_keys(rng, cap, w.index_head_dim)) if w.index_head_dim else None
    # the cache before the step: every token but each sequence's last `new`
    old = np.concatenate([np.arange(base[b], base[b] + lens[b] - new) for b in range(len(lens))]).astype(np.int64)
    step = np.concatenate([np.arange(base[b] + lens[b] - new, base[b] + lens[b]) for b in range(len(lens))])
    step = step.astype(np.int64)
    old_d, step_d = torch.from_numpy(old).to(C.DEV), torch.from_numpy(step).to(C.DEV)
    caches = []
    for _ in range(2):
        c = M.Cache(d, cap, C.DEV)
        c.codes.fill_(0x5A)
        M.mla_append_quant(d, lat_all[old_d].contiguous(), kr_all[old_d].contiguous(),
                           idx_all[old_d].contiguous() if idx_all is not None else None, old_d, layer.Rt_d,
                           layer.alpha_d, c)
        caches.append(c)
    lat = lat_all[step_d].contiguous()
    kr = kr_all[step_d].contiguous()
    idx = idx_all[step_d].contiguous() if idx_all is not None else None
    st = S.streams(w.wid, 5)
    qn, qr = S.queries(w, st, batch=len(lens), tq=tq)
    qn_d, qr_d = C.t_bf16(qn), C.t_bf16(qr)
    seq_base = torch.from_numpy(base).to(C.DEV)
    seq_len = torch.from_numpy(np.asarray(lens, np.int32)).to(C.DEV)
    scale = 1.0 / float(np.sqrt(w.qk_nope_head_dim + w.qk_rope_head_dim))
    # reference: the two calls
    M.mla_append_quant(d, lat, kr, idx, step_d, layer.Rt_d, layer.alpha_d, caches[0])
    out0, lse0 = M.mla_decode_absorbed(d, qn_d, qr_d, layer.w_uk_f, layer.w_uv_f, caches[0], seq_base, seq_len, tq,
                                       causal, scale)
    # the combined step, twice in a row on the same cache (the second append
    # rewrites the same slots with the same bytes)
    for rep in range(2):
        out1, lse1 = M.mla_decode_step(d, lat, kr, idx, step_d, layer.Rt_d, layer.alpha_d, qn_d, qr_d,
                                       layer.w_uk_f, layer.w_uv_f, caches[1], seq_base, seq_len, tq, causal, scale)
        torch.cuda.synchronize()
        assert torch.equal(caches[0].codes, caches[1].codes), rep
        assert torch.equal(caches[0].scale_zero.view(torch.int16), caches[1].scale_zero.view(torch.int16)), rep
        assert torch.equal(caches[0].k_rope.view(torch.int16), caches[1].k_rope.view(torch.int16)), rep
        if idx is not None:
            assert torch.equal(caches[0].idx_key.view(torch.int16), caches[1].idx_key.view(torch.int16)), rep
        assert torch.equal(out0, out1), rep
        assert torch.equal(lse0, lse1), rep
        C.say(f"  rep {rep}: cache and outputs identical")


def test_decode_step_edge_cases():
    """No new tokens (decode only), no sequences (append only), and a fused
    append whose slot list skips tokens (negative and out-of-range slots)."""
    w = S.WORKLOADS[1].with_(num_heads=16)
    C.say("decode_step edge cases")
    layer = C.Layer(w)
    d = layer.dims
    rng = np.random.default_rng(29)
    lens = [90, 41]
    base, cap = S.contiguous_layout(lens, 5)
    lat = C.latent_tensor(layer.model.sample(rng, 6), w.latent_dtype)
    kr = C.t_bf16(S.rope_keys(rng, 6, w.qk_rope_head_dim))
    slots = torch.tensor([int(base[0]) + 89, -1, int(base[1]) + 40, cap + 7, int(base[1]) + 39, int(base[0]) + 88],
                         dtype=torch.int64, device=C.DEV)
    st = S.streams(w.wid, 9)
    qn, qr = S.queries(w, st, batch=2, tq=1)
    qn_d, qr_d = C.t_bf16(qn), C.t_bf16(qr)
    seq_base = torch.from_numpy(base).to(C.DEV)
    seq_len = torch.from_numpy(np.asarray(lens, np.int32)).to(C.DEV)
    scale = 1.0 / float(np.sqrt(w.qk_nope_head_dim + w.qk_rope_head_dim))
    fill = lambda: [M.Cache(d, cap, C.DEV) for _ in range(2)]

    # skipped slots in a fused append
    c0, c1 = fill()
    M.mla_append_quant(d, lat, kr, None, slots, layer.Rt_d, layer.alpha_d, c0)
    out0, lse0 = M.mla_decode_absorbed(d, qn_d, qr_d, layer.w_uk_f, layer.w_uv_f, c0, seq_base, seq_len, 1, True, scale)
    out1, lse1 = M.mla_decode_step(d, lat, kr, None, slots, layer.Rt_d, layer.alpha_d, qn_d, qr_d, layer.w_uk_f,
                                   layer.w_uv_f, c1, seq_base, seq_len, 1, True, scale)
    torch.cuda.synchronize()
    assert torch.equal(c0.codes, c1.codes) and torch.equal(c0.scale_zero.view(torch.int16),
                                                           c1.scale_zero.view(torch.int16))
    assert torch.equal(c0.k_rope.view(torch.int16), c1.k_rope.view(torch.int16))
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)

    # no new tokens: the decode alone
    empty_lat = torch.empty((0, w.kv_lora_rank), dtype=torch.bfloat16, device=C.DEV)
    empty_kr = torch.empty((0, w.qk_rope_head_dim), dtype=torch.bfloat16, device=C.DEV)
    empty_slots = torch.empty((0,), dtype=torch.int64, device=C.DEV)
    before = c1.codes.clone()
    out2, lse2 = M.mla_decode_step(d, empty_lat, empty_kr, None, empty_slots, layer.Rt_d, layer.alpha_d, qn_d, qr_d,
                                   layer.w_uk_f, layer.w_uv_f, c1, seq_base, seq_len, 1, True, scale)
    torch.cuda.synchronize()
    assert torch.equal(before, c1.codes)
    assert torch.equal(out2, out0) and torch.equal(lse2, lse0)

    # no sequences: the append alone
    c2, _ = fill()
    no_b = torch.empty((0,), dtype=torch.int64, device=C.DEV)
    no_l = torch.empty((0,), dtype=torch.int32, device=C.DEV)
    qn0 = torch.empty((0, 1, w.num_heads, w.qk_nope_head_dim), dtype=torch.bfloat16, device=C.DEV)
    qr0 = torch.empty((0, 1, w.num_heads, w.qk_rope_head_dim), dtype=torch.bfloat16, device=C.DEV)
    M.mla_decode_step(d, lat, kr, None, slots, layer.Rt_d, layer.alpha_d, qn0, qr0, layer.w_uk_f, layer.w_uv_f, c2,
                      no_b, no_l, 1, True, scale)
    torch.cuda.synchronize()
    assert torch.equal(c0.codes, c2.codes) and torch.equal(c0.k_rope.view(torch.int16), c2.k_rope.view(torch.int16))
    C.say("  skipped slots, decode only, append only: identical to the separate calls")
