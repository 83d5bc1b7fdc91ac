"""GPU parity in the numerically hard regimes, against the oracle.

* Rising scores.  The split-K kernels keep a running row maximum and only
  move it (rescaling the output accumulators) when a 32-token tile's maximum
  beats it by more than 8 log2 units.  Random caches never do that, so these
  cases make the scores climb: a rope-key channel that grows along the
  sequence with every query aligned to it (about 10 log2 units per tile), and
  flat scores that step up by 24 log2 units at seeded positions every few
  hundred tokens.  A CPU check on the same inputs confirms that the
  tile maxima really jump by more than 8 log2 units before the GPU result is
  compared.  Run on the MFMA latent kernel, the vector-ALU kernel and the
  grouped-query MFMA kernel.
* Offsets.  Latents with a seeded non-zero mean (the covariance the rotation
  is fitted on is uncentred), quantised on append and decoded; and caches
  whose groups sit far from zero (|zero| >> scale), where the kernel's fp16
  dequantised value carries a rounding of 2^-11 |z_hat| that can exceed the
  code step.
* fp16 operand range.  The MFMA kernels take q_nope (absorb), q~ * scale *
  log2(e), q_rope * scale * log2(e), the rope key and z_hat as fp16
  operands.  Queries whose scaled values reach about 0.6 of the fp16 maximum
  (65504) are decoded and compared.

Tolerances are those of tests/parity.py (per-row 2e-3, lse 1e-3).
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
from tests.test_gpu_gqa import _check_decode as gqa_check_decode
from tests.test_gpu_gqa import _decode_case as gqa_decode_case
from tests.test_gpu_gqa import _run_decode as gqa_run_decode
from tests.test_gpu_gqa import _scale as gqa_scale

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
TILE = 32
THRESHOLD = 8.0  # the kernels' lazy-rescale threshold, log2 units


@pytest.fixture(autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    torch.cuda.set_device(0)
    M.mla_set_decode_variant(0)
    yield
    torch.cuda.synchronize()
    M.mla_set_decode_variant(0)


def tile_jumps(s_log2):
    """s_log2 [rows, L] scores in log2 units.  For every row, the fraction of
    32-token tiles (after the first) whose maximum beats the running maximum
    of the earlier tiles by more than the rescale threshold, and their count."""
    rows, L = s_log2.shape
    n_t = (L + TILE - 1) // TILE
    pad = np.full((rows, n_t * TILE), -np.inf)
    pad[:, :L] = s_log2
    tmax = pad.reshape(rows, n_t, TILE).max(axis=2)
    run = np.maximum.accumulate(tmax, axis=1)
    jumps = tmax[:, 1:] > run[:, :-1] + THRESHOLD
    return float(jumps.mean()) if n_t > 1 else 0.0, int(jumps.sum())


def mla_scores_log2(layer, case, b, scale):
    """Scores of every (query, head) row of sequence b, log2 units (only to
    confirm what the inputs make the kernel do)."""
    w = layer.w
    L, a = int(case["lens"][b]), int(case["base"][b])
    codes = O.unpack_codes(case["codes"][a:a + L], w.kv_lora_rank)
    zh = O.dequantize(codes, case["sz"][a:a + L, :, 0], case["sz"][a:a + L, :, 1], w.group_size)
    wk = O.fold_weights(layer.w_uk, layer.R_apply)                       # [H, d_n, r]
    qt = np.einsum("hnr,thn->thr", wk, case["qn"][b].astype(np.float64))  # [tq, H, r]
    s = qt @ zh.T + case["qr"][b].astype(np.float64) @ case["kr"][a:a + L].astype(np.float64).T
    return (scale * LOG2E * s).reshape(-1, L)


def check_mla(layer, case, tq, causal, scale, out, lse, seqs=None):
    ref = C.oracle_decode(layer, case, tq, causal, scale, seqs)
    worst, worst_lse = 0.0, 0.0
    for b, (o_ref, l_ref) in ref.items():
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lse[b]), fin)
        assert np.all(out[b][~fin] == 0)
        if fin.any():
            worst = max(worst, float(row_rel_err(out[b][fin], o_ref[fin]).max()))
            lerr = np.abs(lse[b][fin] - l_ref[fin]) / np.maximum(1, np.abs(l_ref[fin]))
            worst_lse = max(worst_lse, float(lerr.max()))
    C.say(f"  worst row rel err {worst:.3e}, worst lse err {worst_lse:.3e}")
    assert worst <= OUT_RTOL
    assert worst_lse <= LSE_TOL


def run_mla(layer, case, tq, causal, scale):
    d = layer.dims
    cache = C.upload_cache(d, case)
    out, lse = M.mla_decode_absorbed(d, C.t_bf16(case["qn"]), C.t_bf16(case["qr"]), layer.w_uk_f, layer.w_uv_f,
                                     cache, torch.from_numpy(case["base"]).to(C.DEV),
                                     torch.from_numpy(case["lens"]).to(C.DEV), tq, causal, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def ramp_rope(case, slope=0.375, q_val=8.0):
    """Rope channels 0 and 1 of every cached token carry slope * position
    along its sequence (channel 0 its bf16 value, channel 1 the bf16 of the
    remainder, so the sum keeps rising smoothly where one bf16 value would
    step) and every query's rope channels 0 and 1 are q_val, so the scores of
    every row climb by about q_val * slope * 32 * scale * log2(e) per tile."""
    kr = case["kr"].copy()
    for b, L in enumerate(case["lens"]):
        a = int(case["base"][b])
        ramp = slope * np.arange(int(L), dtype=np.float64)
        hi = S.to_bf16_values(ramp)
        kr[a:a + int(L), 0] = hi
        kr[a:a + int(L), 1] = S.to_bf16_values(ramp - hi)
    case["kr"] = kr
    qr = case["qr"].copy()
    qr[..., 0:2] = q_val
    case["qr"] = qr
    return case


def step_positions(rng, L, lo=100, hi=500):
    """Seeded positions where the scores step up: gaps uniform in [lo, hi]."""
    pos, t = [], int(rng.integers(lo, hi))
    while t < L:
        pos.append(t)
        t += int(rng.integers(lo, hi))
    return np.asarray(pos, dtype=np.int64)


def step_rope(case, scale, height=24.0, q_val=8.0, seed=5):
    """Scores flat (the random cache's spread) with a jump of `height` log2
    units at seeded positions: rope channels 0 and 1 of a token carry the
    number of steps before it times the jump (split into bf16 value and
    remainder as in ramp_rope), every query's channels 0 and 1 are q_val.
    Each step makes one tile's maximum beat the running maximum."""
    rng = np.random.default_rng(seed)
    kr = case["kr"].copy()
    unit = height / (scale * LOG2E * 2 * q_val)
    case["steps"] = []
    for b, L in enumerate(case["lens"]):
        a = int(case["base"][b])
        pos = step_positions(rng, int(L))
        case["steps"].append(pos)
        level = unit * np.searchsorted(pos, np.arange(int(L)), side="right").astype(np.float64)
        hi = S.to_bf16_values(level)
        kr[a:a + int(L), 0] = hi
        kr[a:a + int(L), 1] = S.to_bf16_values(level - hi)
    case["kr"] = kr
    qr = case["qr"].copy()
    qr[..., 0:2] = q_val
    case["qr"] = qr
    return case


# ---------------------------------------------------------------------------
# rising scores: the lazy-rescale branch
# ---------------------------------------------------------------------------

RISE_CASES = [
    # name, workload overrides, lens, tq, causal, how, variant
    ("ramp-h128-mfma", dict(), [2049, 700, 97], 1, True, "ramp", 2),
    ("ramp-h128-long-items", dict(), [20000], 1, True, "ramp", 0),
    ("ramp-h16-mfma", dict(num_heads=16), [1500, 64, 4000], 1, True, "ramp", 2),
    ("ramp-tq8-causal-mfma", dict(num_heads=16), [900, 129], 8, True, "ramp", 2),
    ("steps-h16-rows16", dict(num_heads=16), [3000, 515], 1, True, "steps", 0),
    ("steps-h4-tq4-rows16", dict(num_heads=4), [2500, 300], 4, True, "steps", 0),
    ("ramp-h128-valu", dict(), [2049, 700, 97], 1, True, "ramp", 1),
    ("steps-h128-mfma", dict(), [3000, 515], 1, True, "steps", 2),
    ("steps-h128-long-items", dict(), [24000], 1, True, "steps", 0),
    ("steps-h32-valu", dict(num_heads=32), [3000, 515], 1, True, "steps", 1),
    ("steps-g16-mfma", dict(group_size=16, num_heads=32), [2500], 1, True, "steps", 2),
    ("steps-tq4-causal-mfma", dict(num_heads=32), [1800, 700], 4, True, "steps", 2),
]


@pytest.mark.parametrize("name,over,lens,tq,causal,how,variant", RISE_CASES)
def test_decode_rising_scores(name, over, lens, tq, causal, how, variant):
    w = S.WORKLOADS[1].with_(**over)
    C.say(f"rising scores {name} lens={lens} tq={tq} variant={variant}")
    layer = C.Layer(w)
    case = C.random_decode_case(w, lens, tq, seed=23)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    case = ramp_rope(case) if how == "ramp" else step_rope(case, scale)
    # the premise: tile maxima really jump past the threshold, many times
    fracs, counts = [], 0
    for b in range(len(lens)):
        f, n = tile_jumps(mla_scores_log2(layer, case, b, scale))
        fracs.append(f)
        counts += n
    C.say(f"  tiles whose max beats the running max by > {THRESHOLD}: {fracs} ({counts} row-tiles)")
    if how == "ramp":  # nearly every tile of a long sequence moves the maximum
        assert counts >= 10 * w.num_heads
        assert min(f for f, L in zip(fracs, lens) if L >= 512) > 0.9
    else:  # one tile per step (rows x steps, drafts share the steps)
        n_steps = sum(len(p) for p in case["steps"])
        assert counts >= 0.9 * n_steps * w.num_heads * tq
    M.mla_set_decode_variant(variant)
    out, lse = run_mla(layer, case, tq, causal, scale)
    check_mla(layer, case, tq, causal, scale, out, lse)


def _gqa_rise(dims, case, how, c_val=2.0, step=0.038, height=24.0, seed=5):
    """Group 0's zero of every K entry follows a level that grows along its
    sequence (how = "ramp": step per token; "steps": `height` log2 units at
    seeded positions) with group 0's scale 0, and every query is
    bf16(v R_k^T) with v = c_val on group 0's channels (N(0, 1) elsewhere),
    so (q R_k) . k_hat follows the level for every row."""
    d, G, Gq = dims.head_dim, dims.group_size, dims.num_q_heads // dims.num_kv_heads
    rng = np.random.default_rng(71)
    srng = np.random.default_rng(seed)
    unit = height / (gqa_scale(d) * LOG2E * c_val * G)
    ksz = case["ksz"].copy().astype(np.float64)
    case["steps"] = []
    for b, L in enumerate(case["lens"]):
        a = int(case["base"][b])
        if how == "ramp":
            level = -1.0 + step * np.arange(int(L))
        else:
            pos = step_positions(srng, int(L))
            case["steps"].append(pos)
            level = -1.0 + unit * np.searchsorted(pos, np.arange(int(L)), side="right")
        ksz[:, a:a + int(L), 0, 1] = level
        # group 0's scale 0: its z_hat is the (fp16) zero itself, so the level
        # carries no rounding of a large zero + a small step
        ksz[:, a:a + int(L), 0, 0] = 0.0
    case["ksz"] = ksz.astype(np.float16)
    q = case["q"].copy()
    B, tq, hq, _ = q.shape
    for g in range(hq):
        v = rng.standard_normal((B, tq, d))
        v[..., :G] = c_val
        q[:, :, g] = S.to_bf16_values(v @ case["rk"][g // Gq].T)
    case["q"] = q
    return case


def _gqa_scores_log2(dims, case, b, scale):
    d, G, Gq = dims.head_dim, dims.group_size, dims.num_q_heads // dims.num_kv_heads
    L, a = int(case["lens"][b]), int(case["base"][b])
    rows = []
    for g in range(dims.num_q_heads):
        h = g // Gq
        zk = O.dequantize(O.unpack_codes(case["kc"][h, a:a + L], d), case["ksz"][h, a:a + L, :, 0],
                          case["ksz"][h, a:a + L, :, 1], G)
        qr = case["q"][b, :, g].astype(np.float64) @ case["rk"][h]
        rows.append(scale * LOG2E * (qr @ zk.T))
    return np.concatenate(rows, axis=0)


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("how", ["ramp", "steps"])
def test_gqa_decode_rising_scores(how, variant):
    dims = M.GqaDims(128, 32, 8, 32)
    lens = [1500, 300, 2100]
    C.say(f"gqa rising scores {how} variant={variant}")
    case = gqa_decode_case(dims, lens, 1, seed=57)
    scale = gqa_scale(128)
    case = _gqa_rise(dims, case, how)
    counts, fracs = 0, []
    for b in range(len(lens)):
        f, n = tile_jumps(_gqa_scores_log2(dims, case, b, scale))
        counts += n
        fracs.append(f)
    C.say(f"  tiles whose max beats the running max by > {THRESHOLD}: {fracs} ({counts} row-tiles)")
    if how == "ramp":
        assert counts >= 10 * dims.num_q_heads
        assert min(f for f, L in zip(fracs, lens) if L >= 512) > 0.9
    else:
        assert counts >= 0.9 * sum(len(p) for p in case["steps"]) * dims.num_q_heads
    M.mla_set_decode_variant(variant)
    out, lse = gqa_run_decode(dims, case, 1, True, scale)
    gqa_check_decode(dims, case, 1, True, scale, out, lse)


# ---------------------------------------------------------------------------
# offsets: non-zero-mean latents, |zero| >> scale
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("heads,G", [(32, 32), (128, 32), (16, 16)])
def test_nonzero_mean_latents_append_and_decode(heads, G):
    """Latents with a mean of 5-50 standard deviations along 6 seeded
    eigen-directions: calibrated by the oracle (uncentred covariance),
    appended on the GPU (codes to the band rule), then decoded on the GPU over
    the cache it wrote and compared with the oracle's attention on those
    entries."""
    w = S.WORKLOADS[1].with_(num_heads=heads, group_size=G)
    C.say(f"non-zero-mean latents H={heads} G={G}")
    layer = C.Layer(w, mean=(6, 5.0, 50.0))
    lens = [1300, 257, 40]
    base, cap = S.contiguous_layout(lens, 2)
    rng = np.random.default_rng(31)
    lat = layer.model.sample(rng, cap)
    kr = S.rope_keys(rng, cap, w.qk_rope_head_dim)
    cache = M.Cache(layer.dims, cap, C.DEV)
    slots = np.arange(cap, dtype=np.int64)
    M.mla_append_quant(layer.dims, C.t_bf16(lat), C.t_bf16(kr), None, torch.from_numpy(slots).to(C.DEV),
                       layer.Rt_d, layer.alpha_d, cache)
    torch.cuda.synchronize()
    ref = O.quantize_cache(lat, layer.R_apply, layer.alpha, G)
    codes_g, sz_g = cache.codes.cpu().numpy(), cache.scale_zero.cpu().numpy()
    stats = compare_append(codes_g, sz_g, ref, G)
    ratio = np.abs(ref["zero_h"].astype(np.float64)) / np.maximum(ref["scale_h"].astype(np.float64), 1e-30)
    z_last = ref["z32"][:, -1].astype(np.float64)
    C.say(f"  append: {stats['code_mismatch']} code mismatches ({stats['excused']} excused), "
          f"|zero|/scale max {ratio.max():.1f}; last rotated channel mean/std "
          f"{abs(z_last.mean()) / z_last.std():.1f}")
    assert stats["violations"] == 0 and stats["sz_violations"] == 0, stats
    # the mean really shows.  The rotation is fitted on the uncentred
    # covariance, so the mean adds one rank-one term and lands in one rotated
    # channel (the largest eigenvalue, the last group): that channel sits
    # several standard deviations off zero while its group's range spans the
    # other channels, so |zero| / scale stays small on append (the
    # far-from-zero decode case below covers |zero| >> scale)
    assert abs(z_last.mean()) > 3 * z_last.std()
    tq = 1
    st = S.streams(w.wid, 3)
    qn, qr = S.queries(w, st, batch=len(lens), tq=tq)
    case = dict(base=base, cap=cap, codes=codes_g, sz=sz_g, kr=kr, qn=qn, qr=qr, lens=np.asarray(lens, np.int32))
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    out, lse = run_mla(layer, case, tq, True, scale)
    check_mla(layer, case, tq, True, scale, out, lse)


def offset_cache(rng, n, r, group, d_r):
    """Random INT2 cache whose groups sit far from zero: zeros of magnitude
    8..60 (either sign), scales 1e-3..2e-2, so |zero| / scale is 400..60000
    and the fp16 rounding of z_hat exceeds the code step."""
    codes = rng.integers(0, 256, size=(n, r // 4), dtype=np.uint8)
    scale = np.exp(rng.uniform(np.log(1e-3), np.log(2e-2), size=(n, r // group)))
    zero = rng.choice([-1.0, 1.0], size=(n, r // group)) * rng.uniform(8.0, 60.0, size=(n, r // group))
    sz = np.stack([scale, zero], axis=-1).astype(np.float16)
    return codes, sz, S.rope_keys(rng, n, d_r)


@pytest.mark.parametrize("variant", [2, 1])
@pytest.mark.parametrize("heads", [128, 16])
def test_decode_far_from_zero_groups(heads, variant):
    w = S.WORKLOADS[1].with_(num_heads=heads)
    C.say(f"far-from-zero groups H={heads} variant={variant}")
    layer = C.Layer(w)
    lens = [1000, 333]
    case = C.random_decode_case(w, lens, 1, seed=29)
    case["codes"], case["sz"], case["kr"] = offset_cache(np.random.default_rng(29), case["cap"], w.kv_lora_rank,
                                                         w.group_size, w.qk_rope_head_dim)
    # softer scores: the latent part of a score grows with |zero|
    scale = 0.05 * O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    M.mla_set_decode_variant(variant)
    out, lse = run_mla(layer, case, 1, True, scale)
    check_mla(layer, case, 1, True, scale, out, lse)


# ---------------------------------------------------------------------------
# fp16 operand range
# ---------------------------------------------------------------------------

FP16_MAX = 65504.0
TARGET = 40000.0  # scaled query operand magnitude aimed at (0.61 of the fp16 maximum)


@pytest.mark.parametrize("variant", [2, 1])
def test_decode_large_rope_query(variant):
    """q_rope channel 0 scaled so q_rope * scale * log2(e) is ~40000; the
    rope keys' channel 0 small (|k| <= 2e-4), so its score term stays a few
    log2 units."""
    w = S.WORKLOADS[1].with_(num_heads=32)
    C.say(f"large rope query variant={variant}")
    layer = C.Layer(w)
    case = C.random_decode_case(w, [700, 1500], 1, seed=37)
    scale = O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    rng = np.random.default_rng(37)
    qr = case["qr"].copy()
    qr[..., 0] = S.to_bf16_values(TARGET / (scale * LOG2E) * rng.choice([-1.0, 1.0], size=qr.shape[:-1]))
    case["qr"] = qr
    kr = case["kr"].copy()
    kr[:, 0] = S.to_bf16_values(rng.uniform(-2e-4, 2e-4, size=kr.shape[0]))
    case["kr"] = kr
    peak = np.max(np.abs(qr[..., 0])) * scale * LOG2E
    C.say(f"  max |q_rope * scale * log2 e| = {peak:.0f}")
    assert 0.5 * FP16_MAX < peak < FP16_MAX
    M.mla_set_decode_variant(variant)
    out, lse = run_mla(layer, case, 1, True, scale)
    check_mla(layer, case, 1, True, scale, out, lse)


@pytest.mark.parametrize("variant", [2, 1])
def test_decode_large_absorbed_query(variant):
    """q~ * scale * log2(e) ~ 40000 in one latent channel per head, with
    q_nope itself inside the fp16 range (the absorb runs on fp16 MFMA
    operands): q_nope[a] = c sign(W~_UK[h][a][j*]) for the channel j* where
    sum_a |W~_UK[h][a][j]| is largest, at twice the default softmax scale.
    The cache's z_hat is small (zero 0, scale 1e-4) in the groups holding
    those channels and 0 elsewhere, so the scores stay finite and moderate."""
    w = S.WORKLOADS[1].with_(num_heads=32)
    C.say(f"large absorbed query variant={variant}")
    layer = C.Layer(w)
    case = C.random_decode_case(w, [900, 400], 1, seed=41)
    scale = 2.0 * O.default_softmax_scale(w.qk_nope_head_dim, w.qk_rope_head_dim)
    wk = O.fold_weights(layer.w_uk, layer.R_apply)            # [H, d_n, r]
    col = np.sum(np.abs(wk), axis=1)                          # [H, r]
    jstar = np.argmax(col, axis=1)
    c = float(S.to_bf16_values(np.array([TARGET / (scale * LOG2E * np.min(col.max(axis=1)))]))[0])
    assert c < FP16_MAX
    qn = np.zeros_like(case["qn"])
    for h in range(w.num_heads):
        qn[:, :, h, :] = c * np.sign(wk[h, :, jstar[h]])
    case["qn"] = qn
    n, r, G = case["cap"], w.kv_lora_rank, w.group_size
    sz = np.zeros((n, r // G, 2), dtype=np.float16)
    sz[:, np.unique(jstar // G), 0] = np.float16(1e-4)   # other groups: z_hat = 0
    case["sz"] = sz
    qt = np.einsum("hnr,thn->thr", wk, qn[0].astype(np.float64)) * scale * LOG2E
    peak = float(np.max(np.abs(qt)))
    C.say(f"  max |q~ * scale * log2 e| = {peak:.0f} (|q_nope| = {c:.0f})")
    assert 0.5 * FP16_MAX < peak < FP16_MAX
    M.mla_set_decode_variant(variant)
    out, lse = run_mla(layer, case, 1, True, scale)
    check_mla(layer, case, 1, True, scale, out, lse)
