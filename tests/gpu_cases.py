"""Shared set-up for the GPU parity tests: seeded layers and caches.

Inputs come from workloads.synth only; expected values come from the oracle
only.  Nothing here computes any step of the method.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import int2_quantized_absorbed_amd as M
from oracle import mla_oracle as O
from workloads import synth as S

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dims_of(w: S.Workload) -> M.Dims:
    return M.Dims(w.kv_lora_rank, w.qk_rope_head_dim, w.qk_nope_head_dim, w.v_head_dim, w.num_heads,
                  w.group_size, w.index_head_dim)


def t_bf16(x: np.ndarray) -> torch.Tensor:
    """Device bf16 tensor from float32 values that are exactly bf16."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def t_f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def latent_tensor(x: np.ndarray, dtype: str) -> torch.Tensor:
    return t_bf16(x) if dtype == "bf16" else t_f32(x)


class Layer:
    """One calibrated layer: oracle rotation and clip ratios (numpy) plus
    the same values on the device."""

    def __init__(self, w: S.Workload, seed_offset: int = 0, mean=None):
        """mean = (n_dirs, lo, hi): latents with a seeded non-zero mean of
        lo..hi standard deviations along n_dirs eigen-directions."""
        self.w = w
        self.dims = dims_of(w)
        self.st = S.streams(w.wid, seed_offset)
        self.model = S.latent_model(w, self.st)
        if mean is not None:
            self.model = self.model.with_mean(np.random.default_rng(977 + seed_offset), *mean)
        self.c_cal = S.calib_latents(w, self.st, self.model)
        self.R, self.eig, _ = O.calibrate_rotation(self.c_cal)
        self.R_apply = O.rotation_apply(self.R)
        self.alpha, _ = O.fit_clip(self.c_cal, self.R, w.group_size)
        self.w_uk, self.w_uv = S.weights(w, self.st)
        # device copies of the oracle's calibration artefacts
        self.R_d = t_f32(self.R)
        self.alpha_d = t_f32(self.alpha)
        self.Rt_d = M.mla_prepare_rotation(self.dims, self.R_d)
        self.w_uk_f, self.w_uv_f = M.mla_fold_absorb_weights(self.dims, t_bf16(self.w_uk), t_bf16(self.w_uv),
                                                             self.Rt_d)


def random_decode_case(w: S.Workload, lens, tq: int, seed: int, gap: int = 3):
    """A random INT2 cache (no quantiser involved) plus queries; numpy."""
    rng = np.random.default_rng(seed)
    base, cap = S.contiguous_layout(lens, gap)
    codes, sz, kr = S.random_cache(rng, cap, w.kv_lora_rank, w.group_size, w.qk_rope_head_dim)
    st = S.streams(w.wid, seed)
    qn, qr = S.queries(w, st, batch=len(lens), tq=tq)
    return dict(base=base, cap=cap, codes=codes, sz=sz, kr=kr, qn=qn, qr=qr, lens=np.asarray(lens, np.int32))


def upload_cache(dims: M.Dims, case: dict) -> M.Cache:
    c = M.Cache(dims, case["cap"], DEV)
    c.codes.copy_(torch.from_numpy(case["codes"]))
    c.scale_zero.copy_(torch.from_numpy(case["sz"]))
    c.k_rope.copy_(t_bf16(case["kr"]))
    return c


def oracle_decode(layer: Layer, case: dict, tq: int, causal: bool, scale: float, seqs=None):
    """Oracle out [B, tq, H, d_v], lse [B, tq, H] for the listed sequences."""
    w = layer.w
    r, G = w.kv_lora_rank, w.group_size
    B = len(case["lens"])
    seqs = range(B) if seqs is None else seqs
    out = {}
    for b in seqs:
        L = int(case["lens"][b])
        a = int(case["base"][b])
        sl = slice(a, a + L)
        codes = O.unpack_codes(case["codes"][sl], r)
        zh = O.dequantize(codes, case["sz"][sl, :, 0], case["sz"][sl, :, 1], G)
        o, l = O.rotated_attention(case["qn"][b], case["qr"][b], layer.w_uk, layer.w_uv, zh, case["kr"][sl],
                                   layer.R_apply, scale, causal=causal)
        out[b] = (o, l)
    return out


def random_rope_entries(rng, n: int, d_r: int):
    """Random 4-bit rope-key entries (no quantiser involved): codes uniform in
    0..15, fp16 scales in [1e-3, 0.5], zeros in [-2, 0.5], per group of 16.
    Returns (entries [n, d_r/2 + d_r/4] uint8, the dequantised keys fp64)."""
    g = d_r // O.ROPE_GROUP
    codes = rng.integers(0, 16, size=(n, d_r), dtype=np.uint8)
    scale = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), size=(n, g))).astype(np.float16)
    zero = rng.uniform(-2.0, 0.5, size=(n, g)).astype(np.float16)
    return O.pack_rope_entry(codes, scale, zero), O.dequantize_rope(codes, scale, zero)


def upload_cache_rope4(dims: M.Dims, case: dict, entries) -> M.Cache:
    """A cache with 4-bit rope-key entries (dims.rope_bits == 4)."""
    c = M.Cache(dims, case["cap"], DEV)
    c.codes.copy_(torch.from_numpy(case["codes"]))
    c.scale_zero.copy_(torch.from_numpy(case["sz"]))
    c.k_rope.copy_(torch.from_numpy(np.ascontiguousarray(entries)))
    return c
