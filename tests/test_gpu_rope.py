"""The rope-key variant on the GPU (mla_dims.rope_bits = 4: the shared rope
key stored as 4-bit groups of 16 dims with fp16 scale and zero), against
the oracle (oracle/mla_oracle.py quantize_rope_key and the attention
functions fed with the dequantised key).

* append: the latent bytes as for the bf16 rope key, and the rope entries
  (codes bit-exact outside the 1e-5 boundary band, scale / zero by the
  side-info rule) on the small-append, staged and vector-ALU append kernels;
  skipped slots untouched;
* decode over random caches with random 4-bit rope entries, on the MFMA and
  the vector-ALU split-K kernels (per-row 2e-3, lse 1e-3), and the sparse
  decode;
* mla_decode_step equals the two separate calls, bit for bit;
* end to end (append then decode) against the oracle's whole chain.
"""
import numpy as np
import pytest
import torch

import int2_quantized_absorbed_amd as M
from oracle import mla_oracle as O
from workloads import synth as S

from tests import gpu_cases as C
from tests.parity import LSE_TOL, OUT_RTOL, compare_append, compare_rope, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    torch.cuda.set_device(0)
    M.mla_set_decode_variant(0)
    yield
    torch.cuda.synchronize()
    M.mla_set_decode_variant(0)


def rope4(w: S.Workload) -> M.Dims:
    d = C.dims_of(w)
    return M.Dims(d.kv_lora_rank, d.qk_rope_head_dim, d.qk_nope_head_dim, d.v_head_dim, d.num_heads,
                  d.group_size, d.index_head_dim, rope_bits=4)


APPEND_CASES = [
    ("w1-small-8", 1, dict(), 8),
    ("w1-small-300", 1, dict(), 300),
    ("w1-staged-1500", 1, dict(), 1500),
    ("w4-idx-staged-1100", 4, dict(), 1100),
    ("w0-fp32-valu-257", 0, dict(), 257),
]


@pytest.mark.parametrize("name,wid,over,n", APPEND_CASES)
def test_append_rope_int4(name, wid, over, n):
    w = S.WORKLOADS[wid].with_(**over)
    C.say(f"append with 4-bit rope {name} n={n}")
    layer = C.Layer(w)
    d4 = rope4(w)
    rng = np.random.default_rng(17)
    c = layer.model.sample(rng, n)
    kr = S.rope_keys(rng, n, w.qk_rope_head_dim) * rng.uniform(0.05, 3.0, size=(n, 1))
    kr = S.to_bf16_values(kr)
    idx = S.rope_keys(rng, n, w.index_head_dim) if w.index_head_dim else None
    cap = n + 40
    slots = rng.permutation(cap)[:n].astype(np.int64)
    slots[::29] = -1
    cache = M.Cache(d4, cap, C.DEV)
    cache.k_rope.fill_(0xA5)
    M.mla_append_quant(d4, C.latent_tensor(c, w.latent_dtype), C.t_bf16(kr),
                       C.t_bf16(idx) if idx is not None else None, torch.from_numpy(slots).to(C.DEV),
                       layer.Rt_d, layer.alpha_d, cache)
    torch.cuda.synchronize()
    ok = (slots >= 0) & (slots < cap)
    sl = slots[ok]
    ref = O.quantize_cache(c, layer.R_apply, layer.alpha, w.group_size)
    st = compare_append(cache.codes.cpu().numpy()[sl], cache.scale_zero.cpu().numpy()[sl],
                        {k: v[ok] for k, v in ref.items()}, w.group_size)
    assert st["violations"] == 0 and st["sz_violations"] == 0, st
    rr = O.quantize_rope_key(kr[ok])
    sr = compare_rope(cache.k_rope.cpu().numpy()[sl], rr, w.qk_rope_head_dim)
    C.say(name, "latent", {k: st[k] for k in ("code_mismatch", "violations")}, "rope", sr)
    assert sr["violations"] == 0 and sr["sz_violations"] == 0, sr
    if idx is not None:
        assert np.array_equal(cache.idx_key.float().cpu().numpy()[sl], idx[ok])
    untouched = np.setdiff1d(np.arange(cap), sl)
    assert np.all(cache.k_rope.cpu().numpy()[untouched] == 0xA5)


DECODE_CASES = [
    # name, workload overrides, lens, tq, causal, variant
    ("h128-auto", dict(), [37, 700, 2049], 1, True, 0),
    ("h128-valu", dict(), [37, 700, 257], 1, True, 1),
    ("tq8-causal", dict(num_heads=16), [40, 9, 600], 8, True, 0),
    ("h16-mfma", dict(num_heads=16), [300, 1100], 1, True, 2),
    ("g16", dict(group_size=16, num_heads=32), [513], 1, True, 0),
    ("h8-g16-rows16", dict(group_size=16, num_heads=8), [700, 17], 1, True, 0),
]


def _run_decode(dims, case, entries, tq, causal, scale, layer):
    cache = C.upload_cache_rope4(dims, case, entries)
    out, lse = M.mla_decode_absorbed(dims, C.t_bf16(case["qn"]), C.t_bf16(case["qr"]), layer.w_uk_f,
                                     layer.w_uv_f, cache, torch.from_numpy(case["base"]).to(C.DEV),
                                     torch.from_numpy(case["lens"]).to(C.DEV), tq, causal, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name,over,lens,tq,causal,variant", DECODE_CASES)
def test_decode_rope_int4(name, over, lens, tq, causal, variant):
    w = S.WORKLOADS[1].with_(**over)
    C.say(f"decode with 4-bit rope {name} lens={lens} tq={tq} variant={variant}")
    layer = C.Layer(w)
    d4 = rope4(w)
    case = C.random_decode_case(w, lens, tq, seed=19)
    entries, kr_hat = C.random_rope_entries(np.random.default_rng(19), case["cap"], w.qk_rope_head_dim)
    case["kr"] = kr_hat          # the oracle attends with the dequantised rope key
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    M.mla_set_decode_variant(variant)
    out, lse = _run_decode(d4, case, entries, tq, causal, scale, layer)
    ref = C.oracle_decode(layer, case, tq, causal, scale)
    worst = 0.0
    for b, (o_ref, l_ref) in ref.items():
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lse[b]), fin)
        if fin.any():
            worst = max(worst, float(row_rel_err(out[b][fin], o_ref[fin]).max()))
            assert np.all(np.abs(lse[b][fin] - l_ref[fin]) <= LSE_TOL * np.maximum(1, np.abs(l_ref[fin])))
    C.say(f"  worst row rel err {worst:.3e}")
    assert worst <= OUT_RTOL


@pytest.mark.parametrize("new", [1, 13])
def test_decode_step_rope_int4_equals_separate_calls(new):
    """The step's new tokens (1 or 13 per sequence: one or two 32-token
    tiles) appended inside the query-absorb launch, rope keys quantised there
    too, against mla_append_quant then mla_decode_absorbed.  The cache holds
    every earlier token; the step's slots start as a fill pattern, so a
    missing write shows."""
    w = S.WORKLOADS[1]
    C.say(f"decode step with 4-bit rope, {new} new tokens per sequence")
    layer = C.Layer(w)
    d4 = rope4(w)
    lens = [900, 1301, 64]
    base, cap = S.contiguous_layout(lens)
    rng = np.random.default_rng(23)
    lat = C.t_bf16(layer.model.sample(rng, cap))
    kr = C.t_bf16(S.rope_keys(rng, cap, w.qk_rope_head_dim))
    step = np.array([int(base[b]) + L - 1 - j for b, L in enumerate(lens) for j in range(new)], np.int64)
    old = np.setdiff1d(np.arange(cap, dtype=np.int64), step)
    step_d, old_d = torch.from_numpy(step).to(C.DEV), torch.from_numpy(old).to(C.DEV)
    qn, qr = S.queries(w, S.streams(w.wid, 5), batch=len(lens), tq=1)
    qn, qr = C.t_bf16(qn), C.t_bf16(qr)
    sb, sl = torch.from_numpy(base).to(C.DEV), torch.from_numpy(np.asarray(lens, np.int32)).to(C.DEV)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    caches, outs = [], []
    for fused in (True, False):
        cache = M.Cache(d4, cap, C.DEV)
        cache.codes.fill_(0x5A)
        cache.k_rope.fill_(0x3C)
        M.mla_append_quant(d4, lat[old_d].contiguous(), kr[old_d].contiguous(), None, old_d, layer.Rt_d,
                           layer.alpha_d, cache)
        if fused:
            out, lse = M.mla_decode_step(d4, lat[step_d].contiguous(), kr[step_d].contiguous(), None, step_d,
                                         layer.Rt_d, layer.alpha_d, qn, qr, layer.w_uk_f, layer.w_uv_f, cache, sb,
                                         sl, 1, True, scale)
        else:
            M.mla_append_quant(d4, lat[step_d].contiguous(), kr[step_d].contiguous(), None, step_d, layer.Rt_d,
                               layer.alpha_d, cache)
            out, lse = M.mla_decode_absorbed(d4, qn, qr, layer.w_uk_f, layer.w_uv_f, cache, sb, sl, 1, True, scale)
        caches.append(cache)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(caches[0].k_rope, caches[1].k_rope) and torch.equal(caches[0].codes, caches[1].codes)
    assert torch.equal(caches[0].scale_zero.view(torch.int16), caches[1].scale_zero.view(torch.int16))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # the step's slots were written (the fill pattern is gone)
    assert not np.any(np.all(caches[0].codes.cpu().numpy()[step] == 0x5A, axis=1))


@pytest.mark.parametrize("heads", [128, 32])
def test_end_to_end_rope_int4(heads):
    """Append on the GPU then decode on the GPU against the oracle's whole
    chain: quantise the latent and the rope key, then absorbed attention with
    both dequantised."""
    w = S.WORKLOADS[1].with_(num_heads=heads)
    C.say(f"end to end with 4-bit rope H={heads}")
    layer = C.Layer(w)
    d4 = rope4(w)
    lens = [1500, 333]
    base, cap = S.contiguous_layout(lens)
    rng = np.random.default_rng(29)
    lat = layer.model.sample(rng, cap)
    kr = S.rope_keys(rng, cap, w.qk_rope_head_dim)
    cache = M.Cache(d4, cap, C.DEV)
    M.mla_append_quant(d4, C.t_bf16(lat), C.t_bf16(kr), None, torch.arange(cap, dtype=torch.int64, device=C.DEV),
                       layer.Rt_d, layer.alpha_d, cache)
    qn, qr = S.queries(w, S.streams(w.wid, 6), batch=len(lens), tq=1)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    out, lse = M.mla_decode_absorbed(d4, C.t_bf16(qn), C.t_bf16(qr), layer.w_uk_f, layer.w_uv_f, cache,
                                     torch.from_numpy(base).to(C.DEV),
                                     torch.from_numpy(np.asarray(lens, np.int32)).to(C.DEV), 1, True, scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    # judged on the entries the GPU wrote (checked against the oracle's
    # quantisers first): a code at a rounding boundary may legitimately differ
    codes_g, sz_g = cache.codes.cpu().numpy(), cache.scale_zero.cpu().numpy()
    rope_g = cache.k_rope.cpu().numpy()
    st = compare_append(codes_g, sz_g, O.quantize_cache(lat, layer.R_apply, layer.alpha, w.group_size),
                        w.group_size)
    sr = compare_rope(rope_g, O.quantize_rope_key(kr), w.qk_rope_head_dim)
    assert st["violations"] == 0 and sr["violations"] == 0 and sr["sz_violations"] == 0
    zh = O.dequantize(O.unpack_codes(codes_g, w.kv_lora_rank), sz_g[..., 0], sz_g[..., 1], w.group_size)
    rc, rs, rz = O.unpack_rope_entry(rope_g, w.qk_rope_head_dim)
    kh = O.dequantize_rope(rc, rs, rz)
    worst = 0.0
    for b, L in enumerate(lens):
        a = int(base[b])
        o_ref, _ = O.absorbed_attention(qn[b], qr[b], layer.w_uk, layer.w_uv, zh[a:a + L], kh[a:a + L],
                                        layer.R_apply, scale)
        worst = max(worst, float(row_rel_err(out[b], o_ref).max()))
    C.say(f"  worst row rel err {worst:.3e}")
    assert worst <= OUT_RTOL


def test_sparse_decode_rope_int4():
    w = S.WORKLOADS[4].with_(num_heads=32)
    C.say("sparse decode with 4-bit rope")
    layer = C.Layer(w)
    d4 = rope4(w)
    lens = [3000, 1200]
    case = C.random_decode_case(w, lens, 1, seed=31)
    entries, kr_hat = C.random_rope_entries(np.random.default_rng(31), case["cap"], w.qk_rope_head_dim)
    cache = C.upload_cache_rope4(d4, case, entries)
    idx = S.rope_keys(np.random.default_rng(32), case["cap"], w.index_head_dim)
    cache.idx_key.copy_(C.t_bf16(idx))
    q_idx = S.rope_keys(np.random.default_rng(33), len(lens), w.index_head_dim)
    sb = torch.from_numpy(case["base"]).to(C.DEV)
    sel, n_sel = M.mla_index_topk(d4, C.t_bf16(q_idx), cache, sb, torch.from_numpy(case["lens"]).to(C.DEV), 256)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    out, _ = M.mla_decode_sparse(d4, C.t_bf16(case["qn"]), C.t_bf16(case["qr"]), layer.w_uk_f, layer.w_uv_f, cache,
                                 sb, sel, n_sel, scale)
    torch.cuda.synchronize()
    sel_h, n_h, out = sel.cpu().numpy(), n_sel.cpu().numpy(), out.cpu().numpy()
    for b, L in enumerate(lens):
        a = int(case["base"][b])
        ref_sel = O.index_topk(O.index_scores(q_idx[b], idx[a:a + L]), 256)
        assert np.array_equal(sel_h[b, :n_h[b]], ref_sel)
        codes = O.unpack_codes(case["codes"][a:a + L], w.kv_lora_rank)
        zh = O.dequantize(codes, case["sz"][a:a + L, :, 0], case["sz"][a:a + L, :, 1], w.group_size)
        o_ref, _ = O.sparse_absorbed_attention(case["qn"][b], case["qr"][b], layer.w_uk, layer.w_uv, zh,
                                               kr_hat[a:a + L], layer.R_apply, scale, ref_sel)
        assert row_rel_err(out[b], o_ref).max() <= OUT_RTOL
