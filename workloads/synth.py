"""Seeded synthetic inputs for INT2 rotated-latent MLA decode.

This module only draws inputs: it holds none of the method's arithmetic (no
rotation fitting, quantisation or attention).  Tests, the benchmark and the
smoke check take their inputs from here, so the HIP path and the CPU oracle
always see the same values.

Workloads (shapes of DeepSeek-V3-style and GLM-5.3-Flash-style MLA layers):

  id  heads  r    d_r d_n d_v  G   batch  context            Tq  notes
  0   4      64   16  32  32   16  1      256                1   fp32 latent
  1   128    512  64  128 128  32  32     4096               1
  2   128    512  64  128 128  32  8      U[16384, 32768]    1   "32k" decode
  3   128    512  64  128 128  32  4      131072             8   causal drafts,
                                                                 + 4x4096 append
  4   64     512  64  128 128  32  4      262144             1   + bf16 indexer key

Latent tokens are c = (xi * sqrt(eig)) Q^T with xi ~ N(0, I), Q a seeded Haar
orthogonal matrix and eig log-uniform in [lo, 1] (lo = 1e-3 for workload 0,
1e-4 otherwise; workloads 1-4 also multiply 4 seeded directions by 20).
Queries and rope keys are N(0, 1); W_UK and W_UV are N(0, 1/64) for
workload 0 and N(0, 1/512) otherwise.  bf16 values are produced by torch's
round-to-nearest-even conversion.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

try:  # torch is only needed for bf16 rounding and the GPU-side generator
    import torch
except Exception:  # pragma: no cover
    torch = None


@dataclass(frozen=True)
class Workload:
    wid: int
    num_heads: int
    kv_lora_rank: int
    qk_rope_head_dim: int
    qk_nope_head_dim: int
    v_head_dim: int
    group_size: int
    batch: int
    context: int
    context_min: int          # == context unless lengths vary
    tq: int
    latent_dtype: str         # "fp32" or "bf16"
    eig_lo: float
    n_outliers: int
    outlier_factor: float
    weight_var: float
    index_head_dim: int = 0
    causal: bool = True
    n_calib: int = 2048
    append_per_seq: int = 0   # prefill tokens appended per sequence
    name: str = ""
    extra: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    0: Workload(0, 4, 64, 16, 32, 32, 16, 1, 256, 256, 1, "fp32", 1e-3, 0, 1.0,
                1.0 / 64, name="tiny-mla-r64-h4-ctx256"),
    1: Workload(1, 128, 512, 64, 128, 128, 32, 32, 4096, 4096, 1, "bf16", 1e-4,
                4, 20.0, 1.0 / 512, name="dsv3-layer-b32-ctx4096"),
    2: Workload(2, 128, 512, 64, 128, 128, 32, 8, 32768, 16384, 1, "bf16",
                1e-4, 4, 20.0, 1.0 / 512, name="dsv3-layer-b8-ctx16k-32k"),
    3: Workload(3, 128, 512, 64, 128, 128, 32, 4, 131072, 131072, 8, "bf16",
                1e-4, 4, 20.0, 1.0 / 512, append_per_seq=4096,
                name="dsv3-layer-b4-ctx131072-tq8-causal"),
    4: Workload(4, 64, 512, 64, 128, 128, 32, 4, 262144, 262144, 1, "bf16",
                1e-4, 4, 20.0, 1.0 / 512, index_head_dim=64,
                name="glm53flash-latent-layer-b4-ctx262144"),
}

STREAMS = ("rotation", "spectrum", "outliers", "calib", "cache", "queries",
           "weights", "lengths")


def streams(wid: int, seed_offset: int = 0) -> dict:
    """Independent numpy PCG64 generators, one per input family."""
    ss = np.random.SeedSequence(1000 + wid + 7919 * seed_offset)
    return {name: np.random.Generator(np.random.PCG64(s))
            for name, s in zip(STREAMS, ss.spawn(len(STREAMS)))}


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 array of the bf16 values nearest to x (torch's RNE conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def haar_orthogonal(rng, r: int) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian, signs by diag(R)."""
    x = rng.standard_normal((r, r))
    q, rr = np.linalg.qr(x)
    return q * np.sign(np.diag(rr))[None, :]


def spectrum(w: Workload, st: dict) -> np.ndarray:
    r = w.kv_lora_rank
    eig = np.exp(st["spectrum"].uniform(np.log(w.eig_lo), 0.0, size=r))
    if w.n_outliers:
        idx = st["outliers"].choice(r, size=w.n_outliers, replace=False)
        eig[idx] *= w.outlier_factor
    return eig


@dataclass
class LatentModel:
    """The latent distribution of one layer: c = mu + (xi * sqrt(eig)) Q^T
    (mu = 0 unless a mean is given)."""
    q: np.ndarray
    eig: np.ndarray
    dtype: str
    mean: np.ndarray | None = None

    def sample(self, rng, n: int) -> np.ndarray:
        xi = rng.standard_normal((n, self.q.shape[0]))
        c = (xi * np.sqrt(self.eig)[None, :]) @ self.q.T
        if self.mean is not None:
            c = c + self.mean[None, :]
        c = c.astype(np.float32)
        return to_bf16_values(c) if self.dtype == "bf16" else c

    def with_mean(self, rng, n_dirs: int, lo: float, hi: float) -> "LatentModel":
        """The same spectrum with a non-zero mean: n_dirs seeded eigen-directions
        k of the spectrum get mean a_k sqrt(eig_k), a_k uniform in [lo, hi]."""
        idx = rng.choice(self.q.shape[0], size=n_dirs, replace=False)
        a = rng.uniform(lo, hi, size=n_dirs)
        mu = self.q[:, idx] @ (a * np.sqrt(self.eig[idx]))
        return LatentModel(self.q, self.eig, self.dtype, mu)


def latent_model(w: Workload, st: dict) -> LatentModel:
    return LatentModel(haar_orthogonal(st["rotation"], w.kv_lora_rank),
                       spectrum(w, st), w.latent_dtype)


def calib_latents(w: Workload, st: dict, model: LatentModel, n=None):
    return model.sample(st["calib"], w.n_calib if n is None else n)


def seq_lens(w: Workload, st: dict, batch=None) -> np.ndarray:
    b = w.batch if batch is None else batch
    if w.context_min == w.context:
        return np.full(b, w.context, dtype=np.int32)
    return st["lengths"].integers(w.context_min, w.context, size=b,
                                  endpoint=True).astype(np.int32)


def bf16_normal(rng, shape, std=1.0) -> np.ndarray:
    return to_bf16_values(rng.standard_normal(shape) * std)


def queries(w: Workload, st: dict, batch=None, tq=None):
    b = w.batch if batch is None else batch
    t = w.tq if tq is None else tq
    qn = bf16_normal(st["queries"], (b, t, w.num_heads, w.qk_nope_head_dim))
    qr = bf16_normal(st["queries"], (b, t, w.num_heads, w.qk_rope_head_dim))
    return qn, qr


def weights(w: Workload, st: dict):
    std = np.sqrt(w.weight_var)
    h, r = w.num_heads, w.kv_lora_rank
    w_uk = bf16_normal(st["weights"], (h, w.qk_nope_head_dim, r), std)
    w_uv = bf16_normal(st["weights"], (h, w.v_head_dim, r), std)
    return w_uk, w_uv


def rope_keys(rng, n: int, d: int) -> np.ndarray:
    return bf16_normal(rng, (n, d))


def contiguous_layout(lens, gap: int = 0):
    """Sequences placed one after another in one slot pool (optional gap)."""
    lens = np.asarray(lens, dtype=np.int64)
    base = np.zeros(len(lens), dtype=np.int64)
    if len(lens) > 1:
        base[1:] = np.cumsum(lens[:-1] + gap)
    capacity = int(base[-1] + lens[-1] + gap) if len(lens) else gap
    return base, capacity


def random_cache(rng, n: int, r: int, group: int, d_r: int):
    """A syntactically valid INT2 cache with random content (no quantiser).

    Packed codes are uniform random bytes; scales are positive fp16 values in
    [1e-3, 0.5], zeros fp16 in [-1, 0.2]; rope keys bf16 N(0, 1).  Used to test
    decode on its own, independent of the append path.
    """
    codes = rng.integers(0, 256, size=(n, r // 4), dtype=np.uint8)
    scale = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), size=(n, r // group)))
    zero = rng.uniform(-1.0, 0.2, size=(n, r // group))
    sz = np.stack([scale, zero], axis=-1).astype(np.float16)
    return codes, sz, rope_keys(rng, n, d_r)


# ---------------------------------------------------------------------------
# GPU-side generation for benchmark-size caches (same distributions, torch RNG)
# ---------------------------------------------------------------------------


def torch_latents(model: LatentModel, n: int, seed: int, device, chunk=1 << 17):
    """Draw n latent tokens on ``device`` in bf16/fp32 (torch Philox RNG)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    qt = torch.from_numpy(model.q.T.astype(np.float32)).to(device)
    sq = torch.from_numpy(np.sqrt(model.eig).astype(np.float32)).to(device)
    dt = torch.bfloat16 if model.dtype == "bf16" else torch.float32
    out = torch.empty((n, model.q.shape[0]), dtype=dt, device=device)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        xi = torch.randn((b - a, model.q.shape[0]), generator=g, device=device)
        out[a:b] = ((xi * sq) @ qt).to(dt)
    return out


def torch_normal_bf16(shape, seed: int, device, std=1.0):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device) * std).to(torch.bfloat16)
