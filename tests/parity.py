"""Comparison rules between the HIP path and the oracle.

* 2-bit codes: bit-exact, except where the oracle's pre-rounding value u lies
  within BAND = 1e-5 of a quantisation boundary (k + 1/2, k = 0, 1, 2).
* fp16 scale / zero: exact, except a one-ulp difference where the oracle's
  fp32 value before rounding lies within 1e-5 of the midpoint between the two
  fp16 neighbours, relative to the largest magnitude the fp32 computation of
  that value starts from (the group's max |z|: scale and zero come from the
  group's max and min through differences that can cancel, so an fp32
  accumulation difference in z carries into them as an absolute error of
  that size); codes of such a group are judged against u recomputed by the
  oracle from the GPU's own (scale, zero).
* attention outputs: per output row (b, t, h),
  max |out - ref| / max |ref| <= 2e-3 with out in fp32;
  log-sum-exp: |lse - ref| <= 1e-3 max(1, |ref|).
"""
from __future__ import annotations

import numpy as np

from oracle import mla_oracle as O

BAND = 1e-5
OUT_RTOL = 2e-3
# lse: the folded weights W~ = W R_apply are stored in fp16 (one rounding,
# 2^-11 relative), which moves each score by ~1e-4 of its size; 1e-3 of
# max(1, |lse|) is that bound with margin, far below what a wrong mask, scale
# or missing term would produce (O(0.1 - 1)).
LSE_TOL = 1e-3


def _near_boundary(u):
    u = np.asarray(u, dtype=np.float64)
    d = np.min(np.abs(u[..., None] - np.array([0.5, 1.5, 2.5])), axis=-1)
    return d < BAND


def _f16_midpoint_ok(g16, o16, pre32, mag):
    """A one-ulp fp16 difference is excused iff the fp32 value before rounding
    sits within BAND of the midpoint of the two candidates, relative to mag
    (at least the midpoint's own magnitude)."""
    g = g16.astype(np.float64)
    o = o16.astype(np.float64)
    gb = g16.astype(np.float16).view(np.uint16).astype(np.int32)
    ob = o16.astype(np.float16).view(np.uint16).astype(np.int32)
    # neighbours in the fp16 encoding: same sign bit, magnitudes one apart
    one_ulp = ((gb & 0x8000) == (ob & 0x8000)) & (np.abs(gb - ob) == 1)
    mid = 0.5 * (g + o)
    ref_mag = np.maximum(np.maximum(np.abs(mid), np.asarray(mag, dtype=np.float64)), 1e-30)
    near = np.abs(pre32.astype(np.float64) - mid) <= BAND * ref_mag
    return one_ulp & near


def compare_append(gpu_packed, gpu_sz, ref: dict, group: int) -> dict:
    """gpu_packed [n, r/4] uint8, gpu_sz [n, r/G, 2] float16, ref from
    O.quantize_cache.  Returns statistics; ``violations`` must be 0."""
    r = gpu_packed.shape[1] * 4
    gc = O.unpack_codes(gpu_packed, r)
    gs, gz = gpu_sz[..., 0], gpu_sz[..., 1]
    os_, oz = ref["scale_h"], ref["zero_h"]
    s_diff = gs.view(np.uint16) != os_.view(np.uint16)
    z_diff = gz.view(np.uint16) != oz.view(np.uint16)
    n = gc.shape[0]
    gmag = np.max(np.abs(ref["z32"].astype(np.float64)).reshape(n, -1, group), axis=2)
    sz_bad = (s_diff & ~_f16_midpoint_ok(gs, os_, ref["scale32"], gmag)) | \
             (z_diff & ~_f16_midpoint_ok(gz, oz, ref["lo"], gmag))
    grp_diff = s_diff | z_diff
    # codes: where the side info differs (excused), judge against u from the
    # GPU's own side info; elsewhere against the oracle's u
    u_ref = ref["u"].copy()
    codes_ref = ref["codes"].copy()
    if grp_diff.any():
        c2, u2 = O.codes_from_params(ref["z32"], gs, gz, group)
        mask = np.repeat(grp_diff, group, axis=1)
        u_ref = np.where(mask, u2, u_ref)
        codes_ref = np.where(mask, c2, codes_ref)
    mism = gc != codes_ref
    excused = mism & _near_boundary(u_ref)
    viol = mism & ~excused
    bad = np.argwhere(sz_bad)[:5]
    sz_detail = [dict(tok=int(t), grp=int(g), scale=(float(gs[t, g]), float(os_[t, g]), float(ref["scale32"][t, g])),
                      zero=(float(gz[t, g]), float(oz[t, g]), float(ref["lo"][t, g]))) for t, g in bad]
    return dict(n=gc.size, code_mismatch=int(mism.sum()), excused=int(excused.sum()),
                violations=int(viol.sum()), sz_diff=int(grp_diff.sum()), sz_violations=int(sz_bad.sum()),
                viol_index=np.argwhere(viol)[:5].tolist(), sz_detail=sz_detail)


def row_rel_err(out, ref):
    """Per-row max|out - ref| / max|ref| over the last axis."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.maximum(den, 1e-300)


def compare_rope(gpu_entries, ref: dict, d_r: int) -> dict:
    """4-bit rope-key entries [n, d_r/2 + d_r/4] uint8 against
    O.quantize_rope_key: codes bit-exact outside the BAND around the
    boundaries k + 1/2 (k = 0..14); fp16 scale / zero by the side-info rule
    above (a one-ulp midpoint difference, codes then judged on the GPU's own
    scale and zero)."""
    group = O.ROPE_GROUP
    gc, gs, gz = O.unpack_rope_entry(gpu_entries, d_r)
    os_, oz = ref["scale_h"], ref["zero_h"]
    s_diff = gs.view(np.uint16) != os_.view(np.uint16)
    z_diff = gz.view(np.uint16) != oz.view(np.uint16)
    n = gc.shape[0]
    gmag = np.max(np.abs(ref["x32"].astype(np.float64)).reshape(n, -1, group), axis=2)
    sz_bad = (s_diff & ~_f16_midpoint_ok(gs, os_, ref["scale32"], gmag)) | \
             (z_diff & ~_f16_midpoint_ok(gz, oz, ref["lo"], gmag))
    grp_diff = s_diff | z_diff
    u_ref, codes_ref = ref["u"].copy(), ref["codes"].copy()
    if grp_diff.any():
        c2, u2 = O.codes_from_params(ref["x32"], gs, gz, group, levels=15)
        mask = np.repeat(grp_diff, group, axis=1)
        u_ref = np.where(mask, u2, u_ref)
        codes_ref = np.where(mask, c2, codes_ref)
    bounds = np.arange(15) + 0.5
    near = np.min(np.abs(u_ref.astype(np.float64)[..., None] - bounds), axis=-1) < BAND
    mism = gc != codes_ref
    viol = mism & ~near
    return dict(n=gc.size, code_mismatch=int(mism.sum()), excused=int((mism & near).sum()),
                violations=int(viol.sum()), sz_diff=int(grp_diff.sum()), sz_violations=int(sz_bad.sum()))
