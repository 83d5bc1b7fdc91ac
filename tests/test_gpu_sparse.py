"""Sparse decode through the indexer key, GPU against the oracle.

* ``mla_index_topk``: the selected token lists are compared element by element
  with the oracle's (``index_scores`` then ``index_topk``): integer output,
  so bit-exact.  Cases: ragged lengths across several selection chunks,
  sequences shorter than, equal to and just longer than top_k, an empty one,
  top_k = 1, duplicated key rows (equal scores: the lower index wins), chunks
  longer than one scan group of the write pass, and keys drawn from a small
  pool of rows (long runs of equal scores spanning many chunks).
* ``mla_decode_sparse``: on the selection the GPU returned (itself checked
  above), outputs and lse against ``sparse_absorbed_attention`` to the decode
  tolerance, on the MFMA and on the vector-ALU kernel.
"""
import numpy as np
import pytest
import torch

import int2_quantized_absorbed_amd as M
from oracle import mla_oracle as O
from workloads import synth as S

from tests import gpu_cases as C
from tests.parity import LSE_TOL, OUT_RTOL, row_rel_err

pytestmark = pytest.mark.gpu

D_IDX = 64


def _index_case(lens, seed, dup=0, pool=0, d_idx=D_IDX):
    rng = np.random.default_rng(seed)
    base, cap = S.contiguous_layout(lens, 5)
    keys = S.bf16_normal(rng, (cap, d_idx))
    if pool:
        keys = keys[rng.integers(0, pool, size=cap)]
    if dup:
        # copy rows inside each sequence so that several tokens score equally
        for b, L in enumerate(lens):
            a = int(base[b])
            for _ in range(min(dup, L // 2)):
                i, j = rng.integers(0, L, size=2)
                keys[a + j] = keys[a + i]
    q = S.bf16_normal(rng, (len(lens), d_idx))
    return base, cap, keys, q


def _dims(H=128, d_idx=D_IDX):
    return M.Dims(512, 64, 128, 128, H, 32, d_idx)


def _run_topk(dims, lens, base, cap, keys, q, top_k):
    cache = M.Cache(dims, cap, C.DEV)
    cache.idx_key.copy_(C.t_bf16(keys))
    sel, n_sel = M.mla_index_topk(dims, C.t_bf16(q), cache, torch.from_numpy(base).to(C.DEV),
                                  torch.from_numpy(np.asarray(lens, np.int32)).to(C.DEV), top_k)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), n_sel.cpu().numpy()


TOPK_CASES = [
    ("ragged", [5000, 2049, 2048, 300, 0, 7000], 2048, 0, 0),
    ("k1", [17, 1, 999], 1, 0, 0),
    ("ties", [4096, 3000], 512, 400, 0),
    ("long", [40000], 2048, 50, 0),
    ("multigroup", [600001, 3], 2048, 3000, 0),
    ("pool", [20000, 1500], 3000, 0, 40),
]


@pytest.mark.parametrize("name,lens,top_k,dup,pool", TOPK_CASES)
def test_index_topk_matches_oracle(name, lens, top_k, dup, pool):
    C.say(f"index top-k {name} lens={lens} top_k={top_k}")
    base, cap, keys, q = _index_case(lens, 11, dup, pool)
    sel, n_sel = _run_topk(_dims(), lens, base, cap, keys, q, top_k)
    for b, L in enumerate(lens):
        a = int(base[b])
        ref = O.index_topk(O.index_scores(q[b], keys[a:a + L]), top_k)
        assert n_sel[b] == len(ref), (name, b)
        assert np.array_equal(sel[b, :len(ref)], ref), (name, b)


@pytest.mark.parametrize("lens,top_k", [([5000, 63, 1, 0, 2100], 2048), ([300, 64, 65], 7)])
def test_index_topk_128_dim_key(lens, top_k):
    # a 128-dim indexer key: four staging rounds of 16 tokens per wave
    C.say(f"index top-k, 128-dim key, lens={lens} top_k={top_k}")
    base, cap, keys, q = _index_case(lens, 12, 0, 0, d_idx=128)
    sel, n_sel = _run_topk(_dims(d_idx=128), lens, base, cap, keys, q, top_k)
    for b, L in enumerate(lens):
        a = int(base[b])
        ref = O.index_topk(O.index_scores(q[b], keys[a:a + L]), top_k)
        assert n_sel[b] == len(ref), b
        assert np.array_equal(sel[b, :len(ref)], ref), b


# (decode kernel variant, heads): 64 heads on one 64-row block, 16 heads on
# the vector-ALU and on the forced MFMA kernel, 128 heads on two row blocks
# per work item
@pytest.mark.parametrize("variant,heads", [(0, 64), (1, 16), (2, 16), (0, 128)])
def test_decode_sparse_matches_oracle(variant, heads):
    w = S.WORKLOADS[4].with_(num_heads=heads)
    lens = [3000, 700, 0, 2500]
    top_k = 1024
    C.say(f"sparse decode variant {variant} H={w.num_heads} lens={lens} top_k={top_k}")
    layer = C.Layer(w)
    d = layer.dims
    case = C.random_decode_case(w, lens, 1, seed=21)
    rng = np.random.default_rng(22)
    keys = S.bf16_normal(rng, (case["cap"], d.index_head_dim))
    q = S.bf16_normal(rng, (len(lens), d.index_head_dim))
    cache = C.upload_cache(d, case)
    cache.idx_key.copy_(C.t_bf16(keys))
    sb = torch.from_numpy(case["base"]).to(C.DEV)
    sel, n_sel = M.mla_index_topk(d, C.t_bf16(q), cache, sb, torch.from_numpy(case["lens"]).to(C.DEV), top_k)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    M.mla_set_decode_variant(variant)
    try:
        out, lse = M.mla_decode_sparse(d, C.t_bf16(case["qn"]), C.t_bf16(case["qr"]), layer.w_uk_f, layer.w_uv_f,
                                       cache, sb, sel, n_sel, scale)
        torch.cuda.synchronize()
    finally:
        M.mla_set_decode_variant(0)
    out, lse, sel_h, n_h = out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy()
    worst = 0.0
    for b, L in enumerate(lens):
        a = int(case["base"][b])
        ref_sel = O.index_topk(O.index_scores(q[b], keys[a:a + L]), top_k)
        assert n_h[b] == len(ref_sel) and np.array_equal(sel_h[b, :n_h[b]], ref_sel)
        if L == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        codes = O.unpack_codes(case["codes"][a:a + L], w.kv_lora_rank)
        zh = O.dequantize(codes, case["sz"][a:a + L, :, 0], case["sz"][a:a + L, :, 1], w.group_size)
        o_ref, l_ref = O.sparse_absorbed_attention(case["qn"][b], case["qr"][b], layer.w_uk, layer.w_uv, zh,
                                                   case["kr"][a:a + L], layer.R_apply, scale, ref_sel)
        err = row_rel_err(out[b].reshape(-1, out.shape[-1]), o_ref.reshape(-1, o_ref.shape[-1]))
        worst = max(worst, float(err.max()))
        assert np.all(np.abs(lse[b] - l_ref) <= LSE_TOL * np.maximum(1, np.abs(l_ref)))
    C.say(f"  worst row rel err {worst:.3e}")
    assert worst <= OUT_RTOL
