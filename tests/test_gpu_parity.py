"""GPU parity: every entry point of the C ABI against the CPU oracle, on the
same seeded inputs, at sizes the oracle finishes in seconds (several tiles
plus ragged tails).  Tolerances are the ones stated in tests/parity.py."""
import numpy as np
import pytest
import torch

import int2_quantized_absorbed_amd as M
from oracle import mla_oracle as O
from workloads import synth as S
from tests import gpu_cases as C
from tests.parity import LSE_TOL, OUT_RTOL, compare_append, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    torch.cuda.set_device(0)
    M.mla_set_decode_variant(0)
    yield
    torch.cuda.synchronize()
    M.mla_set_decode_variant(0)


# ---------------------------------------------------------------------------
# calibration
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wid", [0, 1])
def test_calibrate_rotation(wid):
    w = S.WORKLOADS[wid]
    C.say(f"calibrate_rotation workload {wid}")
    st = S.streams(wid)
    model = S.latent_model(w, st)
    c = S.calib_latents(w, st, model)
    R_o, lam_o, _ = O.calibrate_rotation(c)
    R_g, lam_g = M.mla_calibrate_rotation(C.dims_of(w), C.latent_tensor(c, w.latent_dtype))
    R_g = R_g.cpu().numpy()
    np.testing.assert_allclose(lam_g, lam_o, rtol=1e-9, atol=1e-14)
    assert np.max(np.abs(R_g - R_o)) <= 2e-6
    R64 = R_g.astype(np.float64)
    assert np.max(np.abs(R64.T @ R64 - np.eye(w.kv_lora_rank))) <= 1e-6


@pytest.mark.parametrize("wid", [0, 1])
def test_calibrate_rotation_weighted(wid):
    """Up-projection-aware rotation against the oracle (same reading): columns
    equal up to sign, eigenvalues to 1e-6 relative."""
    w = S.WORKLOADS[wid]
    C.say(f"calibrate_rotation_weighted workload {wid}")
    st = S.streams(w.wid)
    model = S.latent_model(w, st)
    c_cal = S.calib_latents(w, st, model)
    w_uk, w_uv = S.weights(w, st)
    _, lam_o, R_o = O.calibrate_rotation_weighted(c_cal, w_uk, w_uv)
    d = C.dims_of(w)
    R_g, lam_g = M.mla_calibrate_rotation_weighted(d, C.latent_tensor(c_cal, w.latent_dtype), C.t_bf16(w_uk),
                                                   C.t_bf16(w_uv))
    R_g = R_g.cpu().numpy().astype(np.float64)
    assert np.allclose(lam_g, lam_o, rtol=1e-6, atol=1e-9 * np.max(np.abs(lam_o)))
    # well-separated eigenvalues: the column itself is fixed up to sign
    gaps = np.diff(lam_o)
    sep = np.ones_like(lam_o, dtype=bool)
    sep[1:] &= gaps > 1e-6 * lam_o[-1]
    sep[:-1] &= gaps > 1e-6 * lam_o[-1]
    dots = np.abs(np.sum(R_g * R_o, axis=0))
    assert np.all(dots[sep] > 1 - 1e-5), dots[sep].min()
    assert np.max(np.abs(R_g.T @ R_g - np.eye(R_g.shape[0]))) < 1e-5


def test_prepare_rotation_bit_exact():
    w = S.WORKLOADS[1]
    rng = np.random.default_rng(3)
    R = rng.standard_normal((w.kv_lora_rank, w.kv_lora_rank)).astype(np.float32)
    Rt = M.mla_prepare_rotation(C.dims_of(w), C.t_f32(R)).float().cpu().numpy()
    want = O.rotation_apply(R).T
    assert np.array_equal(Rt.view(np.uint32), np.ascontiguousarray(want).view(np.uint32))


@pytest.mark.parametrize("wid", [0, 1])
def test_fit_clip(wid):
    w = S.WORKLOADS[wid]
    C.say(f"fit_clip workload {wid}")
    layer = C.Layer(w)
    grid = list(O.DEFAULT_ALPHA_GRID)
    a_o, sse_o = O.fit_clip(layer.c_cal, layer.R, w.group_size, grid)
    a_g, sse_g = M.mla_fit_clip(layer.dims, C.latent_tensor(layer.c_cal, w.latent_dtype), layer.Rt_d, grid)
    a_g = a_g.cpu().numpy()
    np.testing.assert_allclose(sse_g, sse_o, rtol=1e-5, atol=1e-12)
    for g in range(len(a_o)):
        if a_g[g] != a_o[g]:
            best = np.sort(sse_o[g])[:2]
            assert (best[1] - best[0]) <= 1e-6 * best[0], (g, a_g[g], a_o[g], best)


def test_fold_weights():
    w = S.WORKLOADS[1].with_(num_heads=8)
    layer = C.Layer(w)
    for got, wt, tr in ((layer.w_uk_f, layer.w_uk, True), (layer.w_uv_f, layer.w_uv, False)):
        ref = O.fold_weights(wt, layer.R_apply)
        if tr:  # the K-side fold is stored [H][r][d_n]
            ref = np.ascontiguousarray(np.swapaxes(ref, 1, 2))
        g = got.float().cpu().numpy().astype(np.float64)
        # fp32 accumulation then one fp16 rounding: the accumulation error can
        # move a value across an fp16 rounding midpoint, so allow one fp16 ulp
        tol = np.abs(np.spacing(ref.astype(np.float16))).astype(np.float64) * 1.0 + 1e-6 * np.abs(ref) + 1e-8
        assert np.all(np.abs(g - ref) <= tol)


# ---------------------------------------------------------------------------
# quantise-on-append
# ---------------------------------------------------------------------------

APPEND_CASES = [
    ("w0-fp32-valu", 0, dict(), 517),
    ("w1-bf16-mfma", 1, dict(), 1000),
    ("w1-bf16-mfma-g16", 1, dict(group_size=16), 333),
    ("w4-bf16-idx", 4, dict(), 300),
    ("w1-r256", 1, dict(kv_lora_rank=256), 129),
    ("w1-r96-valu", 1, dict(kv_lora_rank=96), 70),
    # more than 1024 tokens: the LDS-staged append kernel
    ("w1-bf16-large-1500", 1, dict(), 1500),
    ("w1-bf16-large-g16-1100", 1, dict(group_size=16), 1100),
    ("w4-bf16-idx-large-1300", 4, dict(), 1300),
    ("w1-r128-large-1100", 1, dict(kv_lora_rank=128), 1100),
    ("w1-r256-large-g16-2100", 1, dict(kv_lora_rank=256, group_size=16), 2100),
    ("w1-r384-large-1030", 1, dict(kv_lora_rank=384), 1030),
    # at most 1024 tokens: the small-append kernel
    ("w1-bf16-small-8", 1, dict(), 8),
    ("w1-bf16-small-g16-37", 1, dict(group_size=16), 37),
    ("w4-bf16-idx-small-64", 4, dict(), 64),
    ("w1-r256-small-20", 1, dict(kv_lora_rank=256), 20),
]


@pytest.mark.parametrize("name,wid,over,n", APPEND_CASES)
def test_append_quant(name, wid, over, n):
    w = S.WORKLOADS[wid].with_(**over)
    C.say(f"append_quant {name} n={n}")
    layer = C.Layer(w)
    rng = np.random.default_rng(7)
    c = layer.model.sample(rng, n)
    kr = S.rope_keys(rng, n, w.qk_rope_head_dim)
    idx = S.rope_keys(rng, n, w.index_head_dim) if w.index_head_dim else None
    cap = n + 50
    slots = rng.permutation(cap)[:n].astype(np.int64)
    slots[::37] = -1                                   # skipped tokens
    slots[5] = cap + 3                                  # out of range: skipped
    cache = M.Cache(layer.dims, cap, C.DEV)
    cache.codes.fill_(0xAB)
    M.mla_append_quant(layer.dims, C.latent_tensor(c, w.latent_dtype), C.t_bf16(kr),
                       C.t_bf16(idx) if idx is not None else None, torch.from_numpy(slots).to(C.DEV),
                       layer.Rt_d, layer.alpha_d, cache)
    torch.cuda.synchronize()
    ref = O.quantize_cache(c, layer.R_apply, layer.alpha, w.group_size)
    ok = (slots >= 0) & (slots < cap)
    sl = slots[ok]
    packed = cache.codes.cpu().numpy()[sl]
    sz = cache.scale_zero.cpu().numpy()[sl]
    sub = {k: v[ok] for k, v in ref.items()}
    stats = compare_append(packed, sz, sub, w.group_size)
    C.say(name, stats)
    assert stats["violations"] == 0 and stats["sz_violations"] == 0, stats
    assert np.array_equal(cache.k_rope.float().cpu().numpy()[sl], kr[ok])
    if idx is not None:
        assert np.array_equal(cache.idx_key.float().cpu().numpy()[sl], idx[ok])
    untouched = np.setdiff1d(np.arange(cap), sl)
    assert np.all(cache.codes.cpu().numpy()[untouched] == 0xAB)


@pytest.mark.parametrize("group", [32, 16])
def test_append_small_and_large_batches_agree(group):
    """Appending tokens a few at a time (the decode step's path) writes the
    same bytes as appending them in one large call."""
    w = S.WORKLOADS[1].with_(group_size=group)
    C.say(f"append batch-size invariance G={group}")
    layer = C.Layer(w)
    rng = np.random.default_rng(11)
    n = 1500  # one call: LDS-staged kernel; pieces of at most 64: small-append kernel
    c = C.latent_tensor(layer.model.sample(rng, n), "bf16")
    kr = C.t_bf16(S.rope_keys(rng, n, w.qk_rope_head_dim))
    slots = torch.arange(n, dtype=torch.int64, device=C.DEV)
    big = M.Cache(layer.dims, n, C.DEV)
    M.mla_append_quant(layer.dims, c, kr, None, slots, layer.Rt_d, layer.alpha_d, big)
    small = M.Cache(layer.dims, n, C.DEV)
    cuts = [0, 8, 72, 73, 137, 170, 234, 298, 300] + list(range(364, n, 64)) + [n]
    for a, b in zip(cuts[:-1], cuts[1:]):
        M.mla_append_quant(layer.dims, c[a:b].clone(), kr[a:b].clone(), None, slots[a:b].clone(),
                           layer.Rt_d, layer.alpha_d, small)
    torch.cuda.synchronize()
    assert torch.equal(big.codes, small.codes)
    assert torch.equal(big.scale_zero.view(torch.int16), small.scale_zero.view(torch.int16))
    assert torch.equal(big.k_rope.view(torch.int16), small.k_rope.view(torch.int16))


def test_append_empty_is_noop():
    w = S.WORKLOADS[1]
    layer = C.Layer(w.with_(num_heads=2))
    cache = M.Cache(layer.dims, 4, C.DEV)
    M.mla_append_quant(layer.dims, torch.empty((0, 512), dtype=torch.bfloat16, device=C.DEV),
                       torch.empty((0, 64), dtype=torch.bfloat16, device=C.DEV), None,
                       torch.empty((0,), dtype=torch.int64, device=C.DEV), layer.Rt_d, layer.alpha_d, cache)
    torch.cuda.synchronize()
    assert int(cache.codes.sum()) == 0


# ---------------------------------------------------------------------------
# decode over a random cache (decode checked on its own)
# ---------------------------------------------------------------------------

DECODE_CASES = [
    # name, workload, overrides, lens, tq, causal, variant
    ("w0-valu", 0, dict(), [256], 1, True, 0),
    ("w0-ragged", 0, dict(), [1, 17, 300, 64], 1, True, 0),
    ("w1-small-auto", 1, dict(), [37, 100, 257], 1, True, 0),
    ("w1-small-valu", 1, dict(), [37, 100, 257], 1, True, 1),
    ("w3-tq8-causal", 3, dict(), [40, 9, 129], 8, True, 0),
    ("w3-tq8-causal-valu", 3, dict(), [40, 9, 129], 8, True, 1),
    ("w3-tq4-full", 3, dict(num_heads=16), [33, 70], 4, False, 0),
    ("w4-h64", 4, dict(), [200, 513], 1, True, 0),
    ("w1-h16", 1, dict(num_heads=16), [300, 31], 1, True, 0),
    ("w1-g16", 1, dict(group_size=16, num_heads=32), [129], 1, True, 0),
    ("w1-mfma-forced", 1, dict(), [1, 33, 64, 95], 1, True, 2),
    ("w1-h8-mfma-padrows", 1, dict(num_heads=8), [500], 1, True, 2),
    # at most 16 query rows: the 16-row kernel (waves over 16-token chunks)
    ("w1-h16-many-chunks", 1, dict(num_heads=16), [5000, 17, 1, 160], 1, False, 0),
    ("w1-h4-tq4-causal-mfma", 1, dict(num_heads=4), [700, 33, 4], 4, True, 2),
    ("w1-h2-tq3-mfma", 1, dict(num_heads=2), [300, 45], 3, True, 2),
    ("w1-h16-g16", 1, dict(group_size=16, num_heads=16), [777, 2049], 1, True, 0),
    ("w2-ragged-long", 2, dict(), [2049, 1500, 31, 4000], 1, True, 0),
    # 12 query rows per head at 128 heads: the merge + up-projection's 8-row
    # tiles (two per head; 24 rows, w3-tq8-causal, take its 16-row tiles)
    ("w1-12-sequences", 1, dict(), [65, 1, 400, 33, 0, 129, 1000, 64, 2, 777, 31, 96], 1, True, 0),
    # more than 256 sequences: the device planner's second group of 256
    ("w1-h4-300-sequences", 1, dict(num_heads=4), [(37 * i) % 90 for i in range(300)], 1, True, 0),
    ("w1-300-sequences", 1, dict(), [(41 * i) % 70 for i in range(300)], 1, True, 0),
    # row counts that leave padding rows in a 64-row block: 48 rows (one
    # block, its last 16 rows padding) and 96 (two blocks, the second half
    # padding), causal across the query tokens
    ("w1-h16-tq3-causal", 1, dict(num_heads=16), [200, 47], 3, True, 0),
    ("w1-h32-tq3-causal", 1, dict(num_heads=32), [150, 3, 64], 3, True, 0),
]


def _run_decode(layer, case, tq, causal, scale):
    d = layer.dims
    cache = C.upload_cache(d, case)
    out, lse = M.mla_decode_absorbed(d, C.t_bf16(case["qn"]), C.t_bf16(case["qr"]), layer.w_uk_f,
                                     layer.w_uv_f, cache, torch.from_numpy(case["base"]).to(C.DEV),
                                     torch.from_numpy(case["lens"]).to(C.DEV), tq, causal, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name,wid,over,lens,tq,causal,variant", DECODE_CASES)
def test_decode_random_cache(name, wid, over, lens, tq, causal, variant):
    w = S.WORKLOADS[wid].with_(**over)
    C.say(f"decode {name} lens={lens} tq={tq} causal={causal} variant={variant}")
    layer = C.Layer(w)
    case = C.random_decode_case(w, lens, tq, seed=11)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    M.mla_set_decode_variant(variant)
    out, lse = _run_decode(layer, case, tq, causal, scale)
    ref = C.oracle_decode(layer, case, tq, causal, scale)
    worst, worst_lse = 0.0, 0.0
    for b, (o_ref, l_ref) in ref.items():
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lse[b]), fin), name
        if (~fin).any():
            assert np.all(out[b][~fin] == 0)
        if fin.any():
            err = row_rel_err(out[b][fin], o_ref[fin])
            worst = max(worst, float(err.max()))
            lerr = np.abs(lse[b][fin] - l_ref[fin]) / np.maximum(1, np.abs(l_ref[fin]))
            worst_lse = max(worst_lse, float(lerr.max()))
    C.say(name, "worst row rel err", worst, "worst lse err", worst_lse)
    assert worst <= OUT_RTOL
    assert worst_lse <= LSE_TOL


def test_decode_edge_lengths():
    """Sequences shorter than the draft window and empty sequences."""
    w = S.WORKLOADS[3].with_(num_heads=16)
    layer = C.Layer(w)
    case = C.random_decode_case(w, [3, 0, 8, 1], 8, seed=5)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    out, lse = _run_decode(layer, case, 8, True, scale)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    ref = C.oracle_decode(layer, case, 8, True, scale, seqs=[0, 2, 3])
    for b, (o_ref, l_ref) in ref.items():
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lse[b]), fin)
        assert np.all(out[b][~fin] == 0)
        if fin.any():
            assert row_rel_err(out[b][fin], o_ref[fin]).max() <= OUT_RTOL


# ---------------------------------------------------------------------------
# the whole chain on workload 0 (calibrate -> fit -> fold -> append -> decode)
# ---------------------------------------------------------------------------

def test_end_to_end_workload0():
    w = S.WORKLOADS[0]
    C.say("end-to-end workload 0")
    st = S.streams(0)
    model = S.latent_model(w, st)
    c_cal = S.calib_latents(w, st, model)
    d = C.dims_of(w)
    # oracle chain
    R_o, _, _ = O.calibrate_rotation(c_cal)
    a_o, _ = O.fit_clip(c_cal, R_o, w.group_size)
    Ra = O.rotation_apply(R_o)
    w_uk, w_uv = S.weights(w, st)
    L = w.context
    lat = model.sample(st["cache"], L)
    kr = S.rope_keys(st["cache"], L, w.qk_rope_head_dim)
    qn, qr = S.queries(w, st)
    ref_q = O.quantize_cache(lat, Ra, a_o, w.group_size)
    zh = O.dequantize(ref_q["codes"], ref_q["scale_h"], ref_q["zero_h"], w.group_size)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    o_ref, l_ref = O.absorbed_attention(qn[0], qr[0], w_uk, w_uv, zh, kr, Ra, scale)
    # HIP chain
    cal_d = C.latent_tensor(c_cal, w.latent_dtype)
    R_g, _ = M.mla_calibrate_rotation(d, cal_d)
    Rt = M.mla_prepare_rotation(d, R_g)
    a_g, _ = M.mla_fit_clip(d, cal_d, Rt, list(O.DEFAULT_ALPHA_GRID))
    uk_f, uv_f = M.mla_fold_absorb_weights(d, C.t_bf16(w_uk), C.t_bf16(w_uv), Rt)
    cache = M.Cache(d, L, C.DEV)
    M.mla_append_quant(d, C.latent_tensor(lat, w.latent_dtype), C.t_bf16(kr), None,
                       torch.arange(L, dtype=torch.int64, device=C.DEV), Rt, a_g, cache)
    out, lse = M.mla_decode_absorbed(d, C.t_bf16(qn), C.t_bf16(qr), uk_f, uv_f, cache,
                                     torch.zeros(1, dtype=torch.int64, device=C.DEV),
                                     torch.full((1,), L, dtype=torch.int32, device=C.DEV), 1, True, scale)
    torch.cuda.synchronize()
    a_g_h = a_g.cpu().numpy()
    _, sse_o = O.fit_clip(c_cal, R_o, w.group_size)
    for g in np.nonzero(a_g_h != a_o)[0]:      # only near-ties may differ
        best = np.sort(sse_o[g])[:2]
        assert best[1] - best[0] <= 1e-6 * best[0]
    err = row_rel_err(out.cpu().numpy()[0], o_ref)
    C.say("end-to-end worst row rel err", err.max())
    assert err.max() <= OUT_RTOL
    assert np.all(np.abs(lse.cpu().numpy()[0] - l_ref) <= LSE_TOL * np.maximum(1, np.abs(l_ref)))
