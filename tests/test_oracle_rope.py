"""Pins of the oracle's rope-key variant (4-bit groups of 16 rope dims,
fp16 scale and zero, the latent quantiser without clipping).

The pages name two designs for the rope part and describe neither, so the
quantiser is a reading: it is pinned here against brute force, the textbook
min-max form, hand-worked entry bytes and closed-form sizes.
"""
import json
import os

import numpy as np

from oracle import mla_oracle as O
from workloads import synth as S

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _keys(seed, n, d):
    rng = np.random.default_rng(seed)
    return S.to_bf16_values(rng.standard_normal((n, d)) * rng.uniform(0.05, 3.0, size=(n, 1)))


def test_rope_codes_are_the_nearest_level():
    """Every dim's code is the nearest of the 16 levels zero + k scale."""
    x = _keys(1, 80, 64)
    q = O.quantize_rope_key(x)
    for t in range(x.shape[0]):
        for g in range(4):
            s = float(np.float32(q["scale_h"][t, g]))
            z = float(np.float32(q["zero_h"][t, g]))
            lv = np.array([z + k * s for k in range(16)])
            for j in range(16 * g, 16 * g + 16):
                xv = float(x[t, j])
                d = np.abs(xv - lv)
                k = int(q["codes"][t, j])
                if lv[0] <= xv <= lv[15]:
                    assert d[k] <= d.min() + 1e-6 * max(1.0, abs(xv))
                    assert d[k] <= s / 2 * (1 + 1e-5) + 1e-12
                else:
                    assert k == (0 if xv < lv[0] else 15)


def test_rope_quantiser_is_textbook_minmax():
    """No clipping: zero = group min, scale = (max - min) / 15 (one fp16 ulp);
    the group min gets code 0 and the max code 15 (or 14 at the fp16 edge)."""
    x = _keys(2, 300, 64)
    q = O.quantize_rope_key(x)
    xg = x.reshape(300, 4, 16).astype(np.float64)
    mn, mx = xg.min(-1), xg.max(-1)
    ulp = lambda a: np.abs(np.spacing(a.astype(np.float16)).astype(np.float64))
    ws, wz = ((mx - mn) / 15).astype(np.float16), mn.astype(np.float16)
    assert np.all(np.abs(q["scale_h"].astype(np.float64) - ws) <= ulp(ws))
    assert np.all(np.abs(q["zero_h"].astype(np.float64) - wz) <= ulp(wz))
    cg = q["codes"].reshape(300, 4, 16)
    assert np.all(np.take_along_axis(cg, xg.argmin(-1)[..., None], -1) == 0)
    assert np.all(np.take_along_axis(cg, xg.argmax(-1)[..., None], -1) >= 14)


def test_rope_constant_group_and_half_ties():
    x = np.full((1, 16), -0.75, dtype=F32)
    q = O.quantize_rope_key(x)
    assert q["scale_h"][0, 0] == 0 and np.all(q["codes"] == 0)
    # a group spanning 0..15 exactly: scale 1, zero 0, u = k + 1/2 rounds to even
    x = np.array([[0.0, 15.0, 0.5, 1.5, 2.5, 13.5, 14.5, 7.0, 8.0, 3.0, 4.0, 5.0, 6.0, 9.0, 10.0, 11.0]],
                 dtype=F32)
    q = O.quantize_rope_key(x)
    assert float(q["scale_h"][0, 0]) == 1.0 and float(q["zero_h"][0, 0]) == 0.0
    assert q["codes"][0].tolist() == [0, 15, 0, 2, 2, 14, 14, 7, 8, 3, 4, 5, 6, 9, 10, 11]


def test_rope_entry_golden_bytes_and_roundtrip():
    with open(os.path.join(GOLDEN, "rope_pack_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        codes = np.array([c["codes"]], dtype=np.uint8)
        sh = np.array([c["scale"]], dtype=np.float16)
        zh = np.array([c["zero"]], dtype=np.float16)
        e = O.pack_rope_entry(codes, sh, zh)
        assert e[0].tolist() == c["bytes"]
        c2, s2, z2 = O.unpack_rope_entry(e, codes.shape[1], c["group"])
        assert np.array_equal(c2, codes) and np.array_equal(s2, sh) and np.array_equal(z2, zh)
    x = _keys(3, 50, 64)
    q = O.quantize_rope_key(x)
    e = O.pack_rope_entry(q["codes"], q["scale_h"], q["zero_h"])
    assert e.shape == (50, O.rope_entry_bytes(64)) and O.rope_entry_bytes(64) == 48
    c2, s2, z2 = O.unpack_rope_entry(e, 64)
    assert np.array_equal(c2, q["codes"])
    assert np.array_equal(s2.view(np.uint16), q["scale_h"].view(np.uint16))
    assert np.array_equal(z2.view(np.uint16), q["zero_h"].view(np.uint16))


def test_rope_dequantised_error_bound():
    x = _keys(4, 200, 64)
    q = O.quantize_rope_key(x)
    xh = O.dequantize_rope(q["codes"], q["scale_h"], q["zero_h"])
    step = np.repeat(q["scale_h"].astype(np.float64), 16, axis=1)
    # the fp16 zero can sit up to half an fp16 ulp from the group min
    slack = np.repeat(np.abs(np.spacing(q["zero_h"])).astype(np.float64), 16, axis=1)
    assert np.all(np.abs(xh - x) <= step / 2 * (1 + 1e-4) + slack)


def test_rope_entry_cuts_cache_bytes():
    """DeepSeek-V3 shapes: 128 B codes + 64 B latent side info + 48 B rope
    entry = 240 B per token, against 320 B with the bf16 rope key."""
    assert O.int2_cache_bytes_per_token(512, 32, 64) == 320
    assert O.int2_cache_bytes_per_token(512, 32, 64, rope_bits=4) == 240
    assert O.int2_cache_bytes_per_token(512, 32, 64, 64, rope_bits=4) == 368


def test_rope_int4_score_error_below_the_latent_int2_error():
    """Directional, not a pin: on the DeepSeek-V3-shaped synthetic layer the
    score error the 4-bit rope key adds is well below the one the INT2
    latent already carries."""
    w = S.WORKLOADS[1].with_(num_heads=8)
    st = S.streams(w.wid)
    model = S.latent_model(w, st)
    c_cal = S.calib_latents(w, st, model)
    R, _, _ = O.calibrate_rotation(c_cal)
    Ra = O.rotation_apply(R)
    alpha, _ = O.fit_clip(c_cal, R, w.group_size)
    lat = model.sample(st["cache"], 512)
    kr = S.rope_keys(st["cache"], 512, w.qk_rope_head_dim)
    qn, qr = S.queries(w, st, batch=1, tq=1)
    w_uk, _ = S.weights(w, st)
    qz = O.quantize_cache(lat, Ra, alpha, w.group_size)
    zh = O.dequantize(qz["codes"], qz["scale_h"], qz["zero_h"], w.group_size)
    qrk = O.quantize_rope_key(kr)
    krh = O.dequantize_rope(qrk["codes"], qrk["scale_h"], qrk["zero_h"])
    q_lat = np.einsum("hnr,hn->hr", w_uk.astype(np.float64), qn[0, 0].astype(np.float64))  # [H, r]
    c_exact = lat.astype(np.float64)
    c_hat = O.unrotate(zh, Ra)
    lat_err = np.abs(q_lat @ (c_hat - c_exact).T).mean()
    rope_err = np.abs(qr[0, 0].astype(np.float64) @ (krh - kr).T).mean()
    assert rope_err < 0.5 * lat_err, (rope_err, lat_err)
