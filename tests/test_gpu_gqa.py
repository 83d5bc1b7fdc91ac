"""OSCAR on grouped-query layers, GPU against the oracle (oracle/gqa_oracle.py).

* ``gqa_calibrate``: eigenvalues of both per-KV-head problems to 1e-9
  relative and the rotations element by element to 1e-5 (fp32 output of fp64
  work; the inputs have well separated eigenvalues).
* ``gqa_prepare_rotation``: bf16(R)^T bit-exact per head.
* ``gqa_fit_clip``: the chosen ratio of every (head, group) equal to the
  oracle's ``fit_clip`` on that head, on the same rotation.
* ``gqa_append_quant``: codes and fp16 scale/zero per head and side to the
  append rule (bit-exact outside the 1e-5 boundary band, fp16 midpoint
  excuse), slots outside the cache skipped.
* ``gqa_decode``: outputs and lse against ``rotated_attention`` on the entries
  the GPU cache holds, to the decode tolerance, on the MFMA kernel (d = 128,
  at most 32 query rows per KV head) and on the vector-ALU kernel; ragged,
  empty, tile-edge and multi-query (causal and not) cases, group sizes 1
  (multi-head), 4, 8 and 16 (32 rows at tq = 2), d = 64 and 128, INT2 groups
  of 16 and 32; and the full-size shape of the benchmark on its longest and
  shortest sequences.
"""
import numpy as np
import pytest
import torch

import int2_quantized_absorbed_amd as M
from oracle import gqa_oracle as Q
from oracle import mla_oracle as O
from workloads import synth as S

from tests import gpu_cases as C
from tests.parity import LSE_TOL, OUT_RTOL, compare_append, row_rel_err

pytestmark = pytest.mark.gpu


def _scale(d):
    """The ABI takes the softmax scale as fp32: the oracle gets the same value."""
    return float(np.float32(1.0 / np.sqrt(d)))


def _calib_data(seed, hq, hkv, n, d):
    rng = np.random.default_rng(seed)
    ax = lambda lo, hi: np.exp(rng.uniform(np.log(lo), np.log(hi), d))
    q = S.to_bf16_values(rng.standard_normal((hq, n, d)) * ax(0.2, 3.0))
    k = S.to_bf16_values(rng.standard_normal((hkv, n, d)) * ax(0.1, 2.0))
    v = S.to_bf16_values(rng.standard_normal((hkv, n, d)) * ax(0.1, 2.0))
    return q, k, v


CAL_CASES = [(64, 8, 2, 256, 16), (128, 4, 4, 200, 32)]


@pytest.mark.parametrize("k_rotation", [M.GQA_K_QUERY_COVARIANCE, M.GQA_K_QUERY_METRIC])
@pytest.mark.parametrize("d,hq,hkv,n,G", CAL_CASES)
def test_gqa_calibrate_matches_oracle(d, hq, hkv, n, G, k_rotation):
    C.say(f"gqa calibrate d={d} hq={hq} hkv={hkv} n={n} k_rotation={k_rotation}")
    dims = M.GqaDims(d, hq, hkv, G, k_rotation)
    q, k, v = _calib_data(41, hq, hkv, n, d)
    scale = _scale(d)
    rk, rv, ek, ev = M.gqa_calibrate(dims, C.t_bf16(q), C.t_bf16(k), C.t_bf16(v), scale)
    ork, oek, orv, oev, _ = Q.calibrate(q, k, v, scale, k_rotation=k_rotation)
    assert np.allclose(ek, oek, rtol=1e-9, atol=1e-12)
    assert np.allclose(ev, oev, rtol=1e-9, atol=1e-12)
    assert np.abs(rk.cpu().numpy() - ork).max() <= 1e-5
    assert np.abs(rv.cpu().numpy() - orv).max() <= 1e-5


@pytest.mark.parametrize("d,hq,hkv,n,G", CAL_CASES)
def test_gqa_prepare_and_fit_clip_match_oracle(d, hq, hkv, n, G):
    dims = M.GqaDims(d, hq, hkv, G)
    q, k, v = _calib_data(43, hq, hkv, n, d)
    ork, _, orv, _, _ = Q.calibrate(q, k, v, _scale(d))
    for R, x in ((ork, k), (orv, v)):
        rt = M.gqa_prepare_rotation(dims, C.t_f32(R))
        rt_h = rt.float().cpu().numpy()
        for h in range(hkv):
            assert np.array_equal(rt_h[h], O.rotation_apply(R[h]).T)
        alpha = M.gqa_fit_clip(dims, C.t_bf16(x), rt, O.DEFAULT_ALPHA_GRID).cpu().numpy()
        for h in range(hkv):
            oa, _ = O.fit_clip(x[h], R[h], G)
            assert np.array_equal(alpha[h], oa), h


@pytest.mark.parametrize("d,hq,hkv,n,G", CAL_CASES)
def test_gqa_append_matches_oracle(d, hq, hkv, n, G):
    C.say(f"gqa append d={d} hkv={hkv}")
    dims = M.GqaDims(d, hq, hkv, G)
    q, k, v = _calib_data(47, hq, hkv, n, d)
    ork, _, orv, _, _ = Q.calibrate(q, k, v, _scale(d))
    rng = np.random.default_rng(48)
    alpha_k = np.stack([O.fit_clip(k[h], ork[h], G)[0] for h in range(hkv)])
    alpha_v = rng.choice(np.asarray(O.DEFAULT_ALPHA_GRID, np.float32), size=(hkv, d // G)).astype(np.float32)
    n_new, cap = 300, 400
    kn = S.to_bf16_values(rng.standard_normal((n_new, hkv, d)) * 1.5)
    vn = S.to_bf16_values(rng.standard_normal((n_new, hkv, d)))
    slots = rng.permutation(cap)[:n_new].astype(np.int64)
    slots[::37] = -1                                    # skipped
    cache = M.GqaCache(dims, cap, C.DEV)
    rk_t = M.gqa_prepare_rotation(dims, C.t_f32(ork))
    rv_t = M.gqa_prepare_rotation(dims, C.t_f32(orv))
    M.gqa_append_quant(dims, C.t_bf16(kn), C.t_bf16(vn), torch.from_numpy(slots).to(C.DEV), rk_t, rv_t,
                       C.t_f32(alpha_k), C.t_f32(alpha_v), cache)
    torch.cuda.synchronize()
    ok = slots >= 0
    for side, (x, R, al, codes, sz) in enumerate(((kn, ork, alpha_k, cache.k_codes, cache.k_scale_zero),
                                                   (vn, orv, alpha_v, cache.v_codes, cache.v_scale_zero))):
        codes_h, sz_h = codes.cpu().numpy(), sz.cpu().numpy()
        for h in range(hkv):
            ref = O.quantize_cache(x[ok, h, :], O.rotation_apply(R[h]), al[h], G)
            st = compare_append(codes_h[h][slots[ok]], sz_h[h][slots[ok]], ref, G)
            assert st["violations"] == 0 and st["sz_violations"] == 0, (side, h, st)
        untouched = np.setdiff1d(np.arange(cap), slots[ok])
        assert np.all(codes_h[:, untouched] == 0)


def _random_orthogonal_apply(rng, hkv, d):
    out = []
    for _ in range(hkv):
        a = rng.standard_normal((d, 2 * d))
        r, _ = Q.rotation_from_covariance(a @ a.T / (2 * d))
        out.append(O.rotation_apply(r))
    return np.stack(out)                                 # bf16-valued fp32 [hkv, d, d]


def _decode_case(dims, lens, tq, seed, gap=3):
    rng = np.random.default_rng(seed)
    d, hq, hkv, G = dims.head_dim, dims.num_q_heads, dims.num_kv_heads, dims.group_size
    base, cap = S.contiguous_layout(lens, gap)
    cap = max(cap, 1)
    kc, ksz, vc, vsz = [], [], [], []
    for _ in range(hkv):
        c, s, _ = S.random_cache(rng, cap, d, G, 2)
        kc.append(c)
        ksz.append(s)
        c, s, _ = S.random_cache(rng, cap, d, G, 2)
        vc.append(c)
        vsz.append(s)
    q = S.bf16_normal(rng, (len(lens), tq, hq, d))
    rk = _random_orthogonal_apply(rng, hkv, d)
    rv = _random_orthogonal_apply(rng, hkv, d)
    return dict(base=base, cap=cap, lens=np.asarray(lens, np.int32), kc=np.stack(kc), ksz=np.stack(ksz),
                vc=np.stack(vc), vsz=np.stack(vsz), q=q, rk=rk, rv=rv)


def _run_decode(dims, case, tq, causal, scale):
    cache = M.GqaCache(dims, case["cap"], C.DEV)
    cache.k_codes.copy_(torch.from_numpy(case["kc"]))
    cache.k_scale_zero.copy_(torch.from_numpy(case["ksz"]))
    cache.v_codes.copy_(torch.from_numpy(case["vc"]))
    cache.v_scale_zero.copy_(torch.from_numpy(case["vsz"]))
    rk_t = C.t_bf16(np.transpose(case["rk"], (0, 2, 1)))
    rv_t = C.t_bf16(np.transpose(case["rv"], (0, 2, 1)))
    out, lse = M.gqa_decode(dims, C.t_bf16(case["q"]), cache, rk_t, rv_t,
                            torch.from_numpy(case["base"]).to(C.DEV), torch.from_numpy(case["lens"]).to(C.DEV),
                            tq, causal, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check_decode(dims, case, tq, causal, scale, out, lse, seqs=None):
    d, G = dims.head_dim, dims.group_size
    worst = 0.0
    for b in (range(len(case["lens"])) if seqs is None else seqs):
        L, a = int(case["lens"][b]), int(case["base"][b])
        if L == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        deq = lambda codes, sz: np.stack([O.dequantize(O.unpack_codes(codes[h, a:a + L], d), sz[h, a:a + L, :, 0],
                                                       sz[h, a:a + L, :, 1], G) for h in range(codes.shape[0])])
        zk, zv = deq(case["kc"], case["ksz"]), deq(case["vc"], case["vsz"])
        o_ref, l_ref = Q.rotated_attention(case["q"][b], zk, zv, case["rk"], case["rv"], scale, causal)
        vis = np.isfinite(l_ref)
        assert np.all(np.isneginf(lse[b][~vis])) and np.all(out[b][~vis] == 0)
        err = row_rel_err(out[b][vis].reshape(-1, d), o_ref[vis].reshape(-1, d))
        worst = max(worst, float(err.max()))
        assert np.all(np.abs(lse[b][vis] - l_ref[vis]) <= LSE_TOL * np.maximum(1, np.abs(l_ref[vis])))
    C.say(f"  worst row rel err {worst:.3e}")
    assert worst <= OUT_RTOL


DECODE_CASES = [
    # d, hq, hkv, G, lens, tq, causal (d = 128 with at most 32 rows per KV head
    # takes the MFMA kernel under variant 0; the rest, and variant 1, the vector ALU)
    (128, 32, 8, 32, [700, 0, 1500, 33], 1, True),
    (64, 8, 8, 16, [300, 1000], 4, True),
    (128, 16, 2, 32, [257, 1100], 3, False),
    (64, 32, 4, 16, [5, 64, 2049], 2, True),
    (128, 8, 8, 16, [1, 31, 32, 33, 4000], 4, True),
    (128, 32, 2, 32, [900, 77], 2, True),
    (128, 16, 1, 32, [600, 45, 1], 1, True),    # 16 rows per KV head: the 16-row kernel's largest
    (128, 8, 4, 16, [2100, 130], 8, True),      # 2 x 8 drafts = 16 rows, G = 16
    # 40 sequences x 8 KV heads = 320 pseudo-sequences: the planner's second group
    (128, 32, 8, 32, [(53 * i) % 200 for i in range(40)], 1, True),
]


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("d,hq,hkv,G,lens,tq,causal", DECODE_CASES)
def test_gqa_decode_matches_oracle(d, hq, hkv, G, lens, tq, causal, variant):
    C.say(f"gqa decode d={d} hq={hq} hkv={hkv} G={G} lens={lens} tq={tq} causal={causal} variant={variant}")
    dims = M.GqaDims(d, hq, hkv, G)
    case = _decode_case(dims, lens, tq, seed=51)
    scale = _scale(d)
    M.mla_set_decode_variant(variant)
    try:
        out, lse = _run_decode(dims, case, tq, causal, scale)
    finally:
        M.mla_set_decode_variant(0)
    _check_decode(dims, case, tq, causal, scale, out, lse)


def test_gqa_decode_full_size():
    """The benchmark's layer shape (32 query heads, 8 KV heads, d = 128) on the
    longest and the shortest sequence of its 16k-32k draw."""
    dims = M.GqaDims(128, 32, 8, 32)
    lens = [28669, 17421]
    C.say(f"gqa decode full size lens={lens}")
    case = _decode_case(dims, lens, 1, seed=53)
    scale = _scale(128)
    out, lse = _run_decode(dims, case, 1, True, scale)
    _check_decode(dims, case, 1, True, scale, out, lse)
