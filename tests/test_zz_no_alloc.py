"""The allocation-free decode (mla_decode_absorbed_noalloc) against
mla_decode_absorbed: same kernels, so the outputs must be identical bit for
bit.  Two calls in a row on the library's static scratch, the second smaller
than the first (the scratch keeps the first call's contents), each compared
with a call that brings its own workspace."""
import numpy as np
import pytest
import torch

import int2_quantized_absorbed_amd as M
from oracle import mla_oracle as O
from workloads import synth as S

from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


def _case(w, lens, tq, seed):
    layer = C.Layer(w)
    case = C.random_decode_case(w, lens, tq, seed=seed)
    cache = C.upload_cache(layer.dims, case)
    qn, qr = C.t_bf16(case["qn"]), C.t_bf16(case["qr"])
    base = torch.from_numpy(case["base"]).to(C.DEV)
    lens_d = torch.from_numpy(case["lens"]).to(C.DEV)
    return layer, cache, qn, qr, base, lens_d


def test_noalloc_decode_matches_workspace_decode():
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    M.mla_set_decode_variant(0)
    runs = [
        # a 128-head layer, 6 sequences, then a smaller 32-head one with drafts
        (S.WORKLOADS[1], [3000, 1200, 77, 2500, 640, 1], 1, 61),
        (S.WORKLOADS[1].with_(num_heads=32), [900, 33], 4, 62),
    ]
    sizes = []
    for w, lens, tq, seed in runs:
        C.say(f"noalloc decode H={w.num_heads} lens={lens} tq={tq}")
        layer, cache, qn, qr, base, lens_d = _case(w, lens, tq, seed)
        d = layer.dims
        B = len(lens)
        need = M.mla_decode_workspace_size(d, B, tq)
        assert need <= M.mla_decode_noalloc_max_workspace()
        sizes.append(need)
        scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
        ref_out, ref_lse = M.mla_decode_absorbed(d, qn, qr, layer.w_uk_f, layer.w_uv_f, cache, base, lens_d, tq,
                                                 True, scale)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        M.mla_decode_absorbed_noalloc(d, qn, qr, layer.w_uk_f, layer.w_uv_f, cache, base, lens_d, tq, True, scale,
                                      out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        C.say(f"  identical ({need} bytes of workspace)")
    assert sizes[1] < sizes[0]
