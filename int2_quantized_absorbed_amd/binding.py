"""Thin ctypes binding of libmla (include/mla.h), same names as the C ABI.

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity and handed over as raw device pointers together with the
current HIP stream.  Every step of the method runs in the library's HIP
kernels; there is no fallback path.  If libmla.so is missing, importing the
library fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mla.h")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_NUMERIC, MLA_ERR_HIP = range(6)
MLA_DTYPE_BF16, MLA_DTYPE_FP32 = 0, 1


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status}: {message}")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kv_lora_rank", "qk_rope_head_dim", "qk_nope_head_dim", "v_head_dim",
        "num_heads", "group_size", "index_head_dim", "rope_bits")]


class mla_cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale_zero", ctypes.c_void_p),
                ("k_rope", ctypes.c_void_p), ("idx_key", ctypes.c_void_p),
                ("capacity", ctypes.c_int64)]


GQA_K_QUERY_COVARIANCE = 0   # K rotation: eigenvectors of the query covariance
GQA_K_QUERY_METRIC = 1       # K rotation: key covariance whitened by the query covariance


class gqa_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("head_dim", "num_q_heads", "num_kv_heads", "group_size", "k_rotation")]


class gqa_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scale_zero", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scale_zero", ctypes.c_void_p),
                ("capacity", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIGS = {
    "mla_calibrate_rotation": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, ctypes.c_int, ctypes.c_int64, _P, _P, _P]),
    "mla_calibrate_rotation_weighted": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, ctypes.c_int, ctypes.c_int64,
                                                      _P, _P, _P, _P, _P]),
    "mla_prepare_rotation": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, _P, _P]),
    "mla_fit_clip": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, ctypes.c_int, ctypes.c_int64, _P, _P,
                                    ctypes.c_int32, _P, _P, _P]),
    "mla_fold_absorb_weights": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, _P, _P, _P, _P, _P]),
    "mla_append_quant": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, ctypes.c_int, _P, _P, _P, ctypes.c_int64,
                                        _P, _P, ctypes.POINTER(mla_cache), _P]),
    "mla_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(mla_dims), ctypes.c_int32, ctypes.c_int32]),
    "mla_decode_absorbed": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, _P, _P, _P, ctypes.POINTER(mla_cache),
                                           _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                           _P, ctypes.c_size_t, _P, _P, _P]),
    "mla_decode_noalloc_max_workspace": (ctypes.c_size_t, []),
    "mla_decode_absorbed_noalloc": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, _P, _P, _P,
                                                   ctypes.POINTER(mla_cache), _P, _P, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P, _P]),
    "mla_decode_step": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, ctypes.c_int, _P, _P, _P, ctypes.c_int64,
                                       _P, _P, _P, _P, _P, _P, ctypes.POINTER(mla_cache), _P, _P, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, ctypes.c_size_t, _P, _P,
                                       _P]),
    "mla_index_topk_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(mla_dims), ctypes.c_int32, ctypes.c_int64]),
    "mla_index_topk": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, ctypes.POINTER(mla_cache), _P, _P,
                                      ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t, _P, _P, _P]),
    "mla_decode_sparse": (ctypes.c_int, [ctypes.POINTER(mla_dims), _P, _P, _P, _P, ctypes.POINTER(mla_cache),
                                         _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                         _P, ctypes.c_size_t, _P, _P, _P]),
    "gqa_calibrate": (ctypes.c_int, [ctypes.POINTER(gqa_dims), _P, _P, _P, ctypes.c_int64, ctypes.c_float,
                                     _P, _P, _P, _P, _P]),
    "gqa_prepare_rotation": (ctypes.c_int, [ctypes.POINTER(gqa_dims), _P, _P, _P]),
    "gqa_fit_clip": (ctypes.c_int, [ctypes.POINTER(gqa_dims), _P, ctypes.c_int64, _P, _P, ctypes.c_int32, _P, _P]),
    "gqa_append_quant": (ctypes.c_int, [ctypes.POINTER(gqa_dims), _P, _P, _P, ctypes.c_int64, _P, _P, _P, _P,
                                        ctypes.POINTER(gqa_cache), _P]),
    "gqa_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(gqa_dims), ctypes.c_int32, ctypes.c_int32]),
    "gqa_decode": (ctypes.c_int, [ctypes.POINTER(gqa_dims), _P, ctypes.POINTER(gqa_cache), _P, _P, _P, _P,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P,
                                  ctypes.c_size_t, _P, _P, _P]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_abi_version": (ctypes.c_int32, []),
    "mla_set_decode_variant": (ctypes.c_int, [ctypes.c_int32]),
    "mla_timing_enable": (ctypes.c_int, [ctypes.c_int32]),
    "mla_timing_reset": (ctypes.c_int, []),
    "mla_timing_query": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


def lib():
    """Load libmla.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python -m int2_quantized_absorbed_amd.build_lib")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def header_functions() -> list:
    """Names of the functions include/mla.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:mla|gqa)_[a-z0-9_]+)\s*\(", text)))


def _check(st: int, where: str):
    if st != MLA_OK:
        msg = lib().mla_last_error().decode()
        raise MlaError(st, where, msg)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None, cuda=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MLA_DTYPE_FP32
    raise TypeError("latents must be bfloat16 or float32")


@dataclass(frozen=True)
class Dims:
    kv_lora_rank: int
    qk_rope_head_dim: int
    qk_nope_head_dim: int
    v_head_dim: int
    num_heads: int
    group_size: int
    index_head_dim: int = 0
    rope_bits: int = 0   # 0: bf16 rope key in the cache; 4: the 4-bit rope-key entry

    def c(self) -> mla_dims:
        return mla_dims(self.kv_lora_rank, self.qk_rope_head_dim, self.qk_nope_head_dim, self.v_head_dim,
                        self.num_heads, self.group_size, self.index_head_dim, self.rope_bits)

    @property
    def rope_entry_bytes(self):
        """Cache bytes of one token's rope key."""
        d = self.qk_rope_head_dim
        return 2 * d if self.rope_bits == 0 else d // 2 + d // 4

    @property
    def r(self):
        return self.kv_lora_rank

    @property
    def n_groups(self):
        return self.kv_lora_rank // self.group_size


class Cache:
    """Device tensors of the INT2 latent cache (structure of arrays)."""

    def __init__(self, dims: Dims, capacity: int, device="cuda"):
        r, g = dims.kv_lora_rank, dims.group_size
        self.dims = dims
        self.capacity = int(capacity)
        self.codes = torch.zeros((capacity, r // 4), dtype=torch.uint8, device=device)
        self.scale_zero = torch.zeros((capacity, r // g, 2), dtype=torch.float16, device=device)
        if dims.rope_bits == 0:
            self.k_rope = torch.zeros((capacity, dims.qk_rope_head_dim), dtype=torch.bfloat16, device=device)
        else:  # the 4-bit rope-key entries, bytes
            self.k_rope = torch.zeros((capacity, dims.rope_entry_bytes), dtype=torch.uint8, device=device)
        self.idx_key = (torch.zeros((capacity, dims.index_head_dim), dtype=torch.bfloat16, device=device)
                        if dims.index_head_dim else None)

    def c(self) -> mla_cache:
        return mla_cache(self.codes.data_ptr(), self.scale_zero.data_ptr(), self.k_rope.data_ptr(),
                         self.idx_key.data_ptr() if self.idx_key is not None else 0, self.capacity)


@dataclass(frozen=True)
class GqaDims:
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    group_size: int
    k_rotation: int = GQA_K_QUERY_COVARIANCE   # or GQA_K_QUERY_METRIC (gqa_calibrate only)

    def c(self) -> gqa_dims:
        return gqa_dims(self.head_dim, self.num_q_heads, self.num_kv_heads, self.group_size, self.k_rotation)

    @property
    def n_groups(self):
        return self.head_dim // self.group_size


class GqaCache:
    """Device tensors of the INT2 K/V cache of a grouped-query layer:
    [H_kv, capacity, ...] per side (entry (h, slot) is row h * capacity + slot)."""

    def __init__(self, dims: GqaDims, capacity: int, device="cuda"):
        d, g, h = dims.head_dim, dims.group_size, dims.num_kv_heads
        self.dims = dims
        self.capacity = int(capacity)
        self.k_codes = torch.zeros((h, capacity, d // 4), dtype=torch.uint8, device=device)
        self.k_scale_zero = torch.zeros((h, capacity, d // g, 2), dtype=torch.float16, device=device)
        self.v_codes = torch.zeros((h, capacity, d // 4), dtype=torch.uint8, device=device)
        self.v_scale_zero = torch.zeros((h, capacity, d // g, 2), dtype=torch.float16, device=device)

    def c(self) -> gqa_cache:
        return gqa_cache(self.k_codes.data_ptr(), self.k_scale_zero.data_ptr(), self.v_codes.data_ptr(),
                         self.v_scale_zero.data_ptr(), self.capacity)


# ---------------------------------------------------------------------------
# the ABI, one function per C entry point
# ---------------------------------------------------------------------------

def mla_calibrate_rotation(dims: Dims, c_cal: torch.Tensor):
    """Returns (R [r, r] fp32 device tensor, eigenvalues float64 numpy [r])."""
    r = dims.kv_lora_rank
    _need(c_cal, "c_cal", (torch.bfloat16, torch.float32))
    if c_cal.dim() != 2 or c_cal.shape[1] != r:
        raise ValueError("c_cal must be [n_cal, kv_lora_rank]")
    R = torch.empty((r, r), dtype=torch.float32, device=c_cal.device)
    eig = np.empty(r, dtype=np.float64)
    d = dims.c()
    st = lib().mla_calibrate_rotation(ctypes.byref(d), _ptr(c_cal), _dtype_code(c_cal), c_cal.shape[0],
                                      _ptr(R), eig.ctypes.data_as(ctypes.c_void_p), _stream())
    _check(st, "mla_calibrate_rotation")
    return R, eig


def mla_calibrate_rotation_weighted(dims: Dims, c_cal: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor):
    """Up-projection-aware rotation.  w_uk [H, d_n, r] and w_uv [H, d_v, r] bf16
    (un-folded).  Returns (R [r, r] fp32 device tensor, eigenvalues float64 numpy [r])."""
    r, H = dims.kv_lora_rank, dims.num_heads
    _need(c_cal, "c_cal", (torch.bfloat16, torch.float32))
    if c_cal.dim() != 2 or c_cal.shape[1] != r:
        raise ValueError("c_cal must be [n_cal, kv_lora_rank]")
    _need(w_uk, "w_uk", torch.bfloat16, (H, dims.qk_nope_head_dim, r))
    _need(w_uv, "w_uv", torch.bfloat16, (H, dims.v_head_dim, r))
    R = torch.empty((r, r), dtype=torch.float32, device=c_cal.device)
    eig = np.empty(r, dtype=np.float64)
    d = dims.c()
    st = lib().mla_calibrate_rotation_weighted(ctypes.byref(d), _ptr(c_cal), _dtype_code(c_cal), c_cal.shape[0],
                                               _ptr(w_uk), _ptr(w_uv), _ptr(R),
                                               eig.ctypes.data_as(ctypes.c_void_p), _stream())
    _check(st, "mla_calibrate_rotation_weighted")
    return R, eig


def mla_prepare_rotation(dims: Dims, R: torch.Tensor) -> torch.Tensor:
    """R_apply_t [r, r] bf16 with R_apply_t[j, i] = bf16(R[i, j])."""
    r = dims.kv_lora_rank
    _need(R, "R", torch.float32, (r, r))
    out = torch.empty((r, r), dtype=torch.bfloat16, device=R.device)
    d = dims.c()
    _check(lib().mla_prepare_rotation(ctypes.byref(d), _ptr(R), _ptr(out), _stream()), "mla_prepare_rotation")
    return out


def mla_fit_clip(dims: Dims, c_cal: torch.Tensor, R_apply_t: torch.Tensor, grid):
    """Returns (alpha [r/G] fp32 device tensor, sse float64 numpy [r/G, len(grid)])."""
    r = dims.kv_lora_rank
    _need(c_cal, "c_cal", (torch.bfloat16, torch.float32))
    _need(R_apply_t, "R_apply_t", torch.bfloat16, (r, r))
    g = np.ascontiguousarray(np.asarray(grid, dtype=np.float32))
    alpha = torch.empty(dims.n_groups, dtype=torch.float32, device=c_cal.device)
    sse = np.empty((dims.n_groups, len(g)), dtype=np.float64)
    d = dims.c()
    st = lib().mla_fit_clip(ctypes.byref(d), _ptr(c_cal), _dtype_code(c_cal), c_cal.shape[0], _ptr(R_apply_t),
                            g.ctypes.data_as(ctypes.c_void_p), len(g), _ptr(alpha),
                            sse.ctypes.data_as(ctypes.c_void_p), _stream())
    _check(st, "mla_fit_clip")
    return alpha, sse


def mla_fold_absorb_weights(dims: Dims, w_uk: torch.Tensor, w_uv: torch.Tensor, R_apply_t: torch.Tensor):
    """Returns (w_uk_f [H, r, d_n] fp16 (transposed per head), w_uv_f [H, d_v, r] fp16)."""
    H, r = dims.num_heads, dims.kv_lora_rank
    _need(w_uk, "w_uk", torch.bfloat16, (H, dims.qk_nope_head_dim, r))
    _need(w_uv, "w_uv", torch.bfloat16, (H, dims.v_head_dim, r))
    _need(R_apply_t, "R_apply_t", torch.bfloat16, (r, r))
    uk = torch.empty((H, r, dims.qk_nope_head_dim), dtype=torch.float16, device=w_uk.device)
    uv = torch.empty(w_uv.shape, dtype=torch.float16, device=w_uv.device)
    d = dims.c()
    st = lib().mla_fold_absorb_weights(ctypes.byref(d), _ptr(w_uk), _ptr(w_uv), _ptr(R_apply_t), _ptr(uk),
                                       _ptr(uv), _stream())
    _check(st, "mla_fold_absorb_weights")
    return uk, uv


def mla_append_quant(dims: Dims, latent: torch.Tensor, k_rope: torch.Tensor, idx_key, slot_mapping: torch.Tensor,
                     R_apply_t: torch.Tensor, alpha: torch.Tensor, cache: Cache) -> None:
    r = dims.kv_lora_rank
    _need(latent, "latent", (torch.bfloat16, torch.float32))
    n = latent.shape[0]
    if latent.dim() != 2 or latent.shape[1] != r:
        raise ValueError("latent must be [n, kv_lora_rank]")
    _need(k_rope, "k_rope", torch.bfloat16, (n, dims.qk_rope_head_dim))
    if dims.index_head_dim:
        _need(idx_key, "idx_key", torch.bfloat16, (n, dims.index_head_dim))
    _need(slot_mapping, "slot_mapping", torch.int64, (n,))
    _need(R_apply_t, "R_apply_t", torch.bfloat16, (r, r))
    _need(alpha, "alpha", torch.float32, (dims.n_groups,))
    d, c = dims.c(), cache.c()
    st = lib().mla_append_quant(ctypes.byref(d), _ptr(latent), _dtype_code(latent), _ptr(k_rope), _ptr(idx_key),
                                _ptr(slot_mapping), n, _ptr(R_apply_t), _ptr(alpha), ctypes.byref(c), _stream())
    _check(st, "mla_append_quant")


def mla_decode_workspace_size(dims: Dims, batch: int, tq: int) -> int:
    d = dims.c()
    return int(lib().mla_decode_workspace_size(ctypes.byref(d), batch, tq))


def mla_decode_absorbed(dims: Dims, q_nope, q_rope, w_uk_f, w_uv_f, cache: Cache, seq_base, seq_len, tq: int,
                        causal: bool, softmax_scale: float, workspace=None, out=None, lse=None):
    """Returns (out [B, tq, H, d_v] fp32, lse [B, tq, H] fp32)."""
    H, r = dims.num_heads, dims.kv_lora_rank
    B = seq_len.shape[0]
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.bfloat16, (B, tq, H, dims.qk_nope_head_dim))
    _need(q_rope, "q_rope", torch.bfloat16, (B, tq, H, dims.qk_rope_head_dim))
    _need(w_uk_f, "w_uk_f", torch.float16, (H, r, dims.qk_nope_head_dim))
    _need(w_uv_f, "w_uv_f", torch.float16, (H, dims.v_head_dim, r))
    _need(seq_base, "seq_base", torch.int64, (B,))
    _need(seq_len, "seq_len", torch.int32, (B,))
    need = mla_decode_workspace_size(dims, B, tq)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, tq, H, dims.v_head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, tq, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, tq, H, dims.v_head_dim))
    _need(lse, "lse", torch.float32, (B, tq, H))
    d, c = dims.c(), cache.c()
    st = lib().mla_decode_absorbed(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk_f), _ptr(w_uv_f),
                                   ctypes.byref(c), _ptr(seq_base), _ptr(seq_len), B, tq, int(bool(causal)),
                                   float(softmax_scale), _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                                   _stream())
    _check(st, "mla_decode_absorbed")
    return out, lse


def mla_decode_noalloc_max_workspace() -> int:
    return int(lib().mla_decode_noalloc_max_workspace())


def mla_decode_absorbed_noalloc(dims: Dims, q_nope, q_rope, w_uk_f, w_uv_f, cache: Cache, seq_base, seq_len,
                                tq: int, causal: bool, softmax_scale: float, out, lse):
    """mla_decode_absorbed on the library's static scratch: the caller passes
    the outputs (out [B, tq, H, d_v] fp32, lse [B, tq, H] fp32)."""
    H, r = dims.num_heads, dims.kv_lora_rank
    B = seq_len.shape[0]
    _need(q_nope, "q_nope", torch.bfloat16, (B, tq, H, dims.qk_nope_head_dim))
    _need(q_rope, "q_rope", torch.bfloat16, (B, tq, H, dims.qk_rope_head_dim))
    _need(w_uk_f, "w_uk_f", torch.float16, (H, r, dims.qk_nope_head_dim))
    _need(w_uv_f, "w_uv_f", torch.float16, (H, dims.v_head_dim, r))
    _need(seq_base, "seq_base", torch.int64, (B,))
    _need(seq_len, "seq_len", torch.int32, (B,))
    _need(out, "out", torch.float32, (B, tq, H, dims.v_head_dim))
    _need(lse, "lse", torch.float32, (B, tq, H))
    d, c = dims.c(), cache.c()
    st = lib().mla_decode_absorbed_noalloc(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk_f),
                                           _ptr(w_uv_f), ctypes.byref(c), _ptr(seq_base), _ptr(seq_len), B, tq,
                                           int(bool(causal)), float(softmax_scale), _ptr(out), _ptr(lse),
                                           _stream())
    _check(st, "mla_decode_absorbed_noalloc")
    return out, lse


def mla_decode_step(dims: Dims, latent, k_rope, idx_key, slot_mapping, R_apply_t, alpha, q_nope, q_rope, w_uk_f,
                    w_uv_f, cache: Cache, seq_base, seq_len, tq: int, causal: bool, softmax_scale: float,
                    workspace=None, out=None, lse=None):
    """mla_append_quant of the step's new tokens, then mla_decode_absorbed over
    the cache that holds them, in one call; returns (out, lse)."""
    H, r = dims.num_heads, dims.kv_lora_rank
    B = seq_len.shape[0]
    dev = q_nope.device
    _need(latent, "latent", (torch.bfloat16, torch.float32))
    n = latent.shape[0]
    if latent.dim() != 2 or latent.shape[1] != r:
        raise ValueError("latent must be [n, kv_lora_rank]")
    _need(k_rope, "k_rope", torch.bfloat16, (n, dims.qk_rope_head_dim))
    if dims.index_head_dim:
        _need(idx_key, "idx_key", torch.bfloat16, (n, dims.index_head_dim))
    _need(slot_mapping, "slot_mapping", torch.int64, (n,))
    _need(R_apply_t, "R_apply_t", torch.bfloat16, (r, r))
    _need(alpha, "alpha", torch.float32, (dims.n_groups,))
    _need(q_nope, "q_nope", torch.bfloat16, (B, tq, H, dims.qk_nope_head_dim))
    _need(q_rope, "q_rope", torch.bfloat16, (B, tq, H, dims.qk_rope_head_dim))
    _need(w_uk_f, "w_uk_f", torch.float16, (H, r, dims.qk_nope_head_dim))
    _need(w_uv_f, "w_uv_f", torch.float16, (H, dims.v_head_dim, r))
    _need(seq_base, "seq_base", torch.int64, (B,))
    _need(seq_len, "seq_len", torch.int32, (B,))
    need = mla_decode_workspace_size(dims, B, tq)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, tq, H, dims.v_head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, tq, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, tq, H, dims.v_head_dim))
    _need(lse, "lse", torch.float32, (B, tq, H))
    d, c = dims.c(), cache.c()
    st = lib().mla_decode_step(ctypes.byref(d), _ptr(latent), _dtype_code(latent), _ptr(k_rope), _ptr(idx_key),
                               _ptr(slot_mapping), n, _ptr(R_apply_t), _ptr(alpha), _ptr(q_nope), _ptr(q_rope),
                               _ptr(w_uk_f), _ptr(w_uv_f), ctypes.byref(c), _ptr(seq_base), _ptr(seq_len), B, tq,
                               int(bool(causal)), float(softmax_scale), _ptr(workspace), workspace.numel(), _ptr(out),
                               _ptr(lse), _stream())
    _check(st, "mla_decode_step")
    return out, lse


def mla_index_topk_workspace_size(dims: Dims, batch: int, capacity: int) -> int:
    return int(lib().mla_index_topk_workspace_size(ctypes.byref(dims.c()), int(batch), int(capacity)))


def mla_index_topk(dims: Dims, q_idx, cache: Cache, seq_base, seq_len, top_k: int, workspace=None, sel=None,
                   n_sel=None):
    """Returns (sel [B, top_k] int32, n_sel [B] int32); see include/mla.h."""
    B = seq_len.shape[0]
    dev = seq_len.device
    _need(q_idx, "q_idx", torch.bfloat16, (B, dims.index_head_dim))
    _need(seq_base, "seq_base", torch.int64, (B,))
    _need(seq_len, "seq_len", torch.int32, (B,))
    need = mla_index_topk_workspace_size(dims, B, cache.capacity)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    if sel is None:
        sel = torch.zeros((B, top_k), dtype=torch.int32, device=dev)
    if n_sel is None:
        n_sel = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(sel, "sel", torch.int32, (B, top_k))
    _need(n_sel, "n_sel", torch.int32, (B,))
    d, c = dims.c(), cache.c()
    st = lib().mla_index_topk(ctypes.byref(d), _ptr(q_idx), ctypes.byref(c), _ptr(seq_base), _ptr(seq_len), B,
                              int(top_k), _ptr(workspace), workspace.numel(), _ptr(sel), _ptr(n_sel), _stream())
    _check(st, "mla_index_topk")
    return sel, n_sel


def mla_decode_sparse(dims: Dims, q_nope, q_rope, w_uk_f, w_uv_f, cache: Cache, seq_base, sel, n_sel,
                      softmax_scale: float, workspace=None, out=None, lse=None):
    """Returns (out [B, 1, H, d_v] fp32, lse [B, 1, H] fp32) over the selected tokens."""
    H, r = dims.num_heads, dims.kv_lora_rank
    B, top_k = sel.shape
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.bfloat16, (B, 1, H, dims.qk_nope_head_dim))
    _need(q_rope, "q_rope", torch.bfloat16, (B, 1, H, dims.qk_rope_head_dim))
    _need(w_uk_f, "w_uk_f", torch.float16, (H, r, dims.qk_nope_head_dim))
    _need(w_uv_f, "w_uv_f", torch.float16, (H, dims.v_head_dim, r))
    _need(seq_base, "seq_base", torch.int64, (B,))
    _need(sel, "sel", torch.int32, (B, top_k))
    _need(n_sel, "n_sel", torch.int32, (B,))
    need = mla_decode_workspace_size(dims, B, 1)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, 1, H, dims.v_head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, 1, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, 1, H, dims.v_head_dim))
    _need(lse, "lse", torch.float32, (B, 1, H))
    d, c = dims.c(), cache.c()
    st = lib().mla_decode_sparse(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk_f), _ptr(w_uv_f),
                                 ctypes.byref(c), _ptr(seq_base), _ptr(sel), _ptr(n_sel), B, int(top_k),
                                 float(softmax_scale), _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                                 _stream())
    _check(st, "mla_decode_sparse")
    return out, lse


def mla_set_decode_variant(variant: int) -> None:
    _check(lib().mla_set_decode_variant(int(variant)), "mla_set_decode_variant")


def mla_timing_enable(enable: bool) -> None:
    _check(lib().mla_timing_enable(int(bool(enable))), "mla_timing_enable")


def mla_timing_reset() -> None:
    _check(lib().mla_timing_reset(), "mla_timing_reset")


def mla_timing_query(kernel: str):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().mla_timing_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)), "mla_timing_query")
    return ms.value, n.value


def mla_last_error() -> str:
    return lib().mla_last_error().decode()


def mla_status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def mla_abi_version() -> int:
    return int(lib().mla_abi_version())


# ---------------------------------------------------------------------------
# grouped-query (OSCAR full-attention) layers
# ---------------------------------------------------------------------------

def gqa_calibrate(dims: GqaDims, q_cal, k_cal, v_cal, softmax_scale: float):
    """q_cal [H_q, n, d], k_cal/v_cal [H_kv, n, d] bf16 -> (R_k, R_v [H_kv, d, d] fp32 device,
    eig_k, eig_v float64 numpy [H_kv, d])."""
    d, hq, hkv = dims.head_dim, dims.num_q_heads, dims.num_kv_heads
    n = q_cal.shape[1] if q_cal.dim() == 3 else -1
    _need(q_cal, "q_cal", torch.bfloat16, (hq, n, d))
    _need(k_cal, "k_cal", torch.bfloat16, (hkv, n, d))
    _need(v_cal, "v_cal", torch.bfloat16, (hkv, n, d))
    rk = torch.empty((hkv, d, d), dtype=torch.float32, device=q_cal.device)
    rv = torch.empty_like(rk)
    ek = np.empty((hkv, d), dtype=np.float64)
    ev = np.empty((hkv, d), dtype=np.float64)
    g = dims.c()
    st = lib().gqa_calibrate(ctypes.byref(g), _ptr(q_cal), _ptr(k_cal), _ptr(v_cal), n, float(softmax_scale),
                             _ptr(rk), _ptr(rv), ek.ctypes.data_as(ctypes.c_void_p),
                             ev.ctypes.data_as(ctypes.c_void_p), _stream())
    _check(st, "gqa_calibrate")
    return rk, rv, ek, ev


def gqa_prepare_rotation(dims: GqaDims, R: torch.Tensor) -> torch.Tensor:
    """R [H_kv, d, d] fp32 -> R_apply_t [H_kv, d, d] bf16, R_apply_t[h, j, i] = bf16(R[h, i, j])."""
    d, hkv = dims.head_dim, dims.num_kv_heads
    _need(R, "R", torch.float32, (hkv, d, d))
    out = torch.empty((hkv, d, d), dtype=torch.bfloat16, device=R.device)
    g = dims.c()
    _check(lib().gqa_prepare_rotation(ctypes.byref(g), _ptr(R), _ptr(out), _stream()), "gqa_prepare_rotation")
    return out


def gqa_fit_clip(dims: GqaDims, x_cal, R_apply_t, grid):
    """x_cal [H_kv, n, d] bf16 (keys or values) -> alpha [H_kv, d/G] fp32 device."""
    d, hkv = dims.head_dim, dims.num_kv_heads
    n = x_cal.shape[1] if x_cal.dim() == 3 else -1
    _need(x_cal, "x_cal", torch.bfloat16, (hkv, n, d))
    _need(R_apply_t, "R_apply_t", torch.bfloat16, (hkv, d, d))
    gr = np.ascontiguousarray(np.asarray(grid, dtype=np.float32))
    alpha = torch.empty((hkv, dims.n_groups), dtype=torch.float32, device=x_cal.device)
    g = dims.c()
    st = lib().gqa_fit_clip(ctypes.byref(g), _ptr(x_cal), n, _ptr(R_apply_t), gr.ctypes.data_as(ctypes.c_void_p),
                            len(gr), _ptr(alpha), _stream())
    _check(st, "gqa_fit_clip")
    return alpha


def gqa_append_quant(dims: GqaDims, k, v, slot_mapping, rk_apply_t, rv_apply_t, alpha_k, alpha_v,
                     cache: GqaCache) -> None:
    """k, v [n, H_kv, d] bf16; slot_mapping [n] int64."""
    d, hkv = dims.head_dim, dims.num_kv_heads
    n = k.shape[0]
    _need(k, "k", torch.bfloat16, (n, hkv, d))
    _need(v, "v", torch.bfloat16, (n, hkv, d))
    _need(slot_mapping, "slot_mapping", torch.int64, (n,))
    for t, name in ((rk_apply_t, "rk_apply_t"), (rv_apply_t, "rv_apply_t")):
        _need(t, name, torch.bfloat16, (hkv, d, d))
    for t, name in ((alpha_k, "alpha_k"), (alpha_v, "alpha_v")):
        _need(t, name, torch.float32, (hkv, dims.n_groups))
    g, c = dims.c(), cache.c()
    st = lib().gqa_append_quant(ctypes.byref(g), _ptr(k), _ptr(v), _ptr(slot_mapping), n, _ptr(rk_apply_t),
                                _ptr(rv_apply_t), _ptr(alpha_k), _ptr(alpha_v), ctypes.byref(c), _stream())
    _check(st, "gqa_append_quant")


def gqa_decode_workspace_size(dims: GqaDims, batch: int, tq: int) -> int:
    g = dims.c()
    return int(lib().gqa_decode_workspace_size(ctypes.byref(g), int(batch), int(tq)))


def gqa_decode(dims: GqaDims, q, cache: GqaCache, rk_apply_t, rv_apply_t, seq_base, seq_len, tq: int,
               causal: bool, softmax_scale: float, workspace=None, out=None, lse=None):
    """q [B, tq, H_q, d] bf16 -> (out [B, tq, H_q, d] fp32, lse [B, tq, H_q] fp32)."""
    d, hq, hkv = dims.head_dim, dims.num_q_heads, dims.num_kv_heads
    B = seq_len.shape[0]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, tq, hq, d))
    for t, name in ((rk_apply_t, "rk_apply_t"), (rv_apply_t, "rv_apply_t")):
        _need(t, name, torch.bfloat16, (hkv, d, d))
    _need(seq_base, "seq_base", torch.int64, (B,))
    _need(seq_len, "seq_len", torch.int32, (B,))
    need = gqa_decode_workspace_size(dims, B, tq)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, tq, hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, tq, hq), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, tq, hq, d))
    _need(lse, "lse", torch.float32, (B, tq, hq))
    g, c = dims.c(), cache.c()
    st = lib().gqa_decode(ctypes.byref(g), _ptr(q), ctypes.byref(c), _ptr(rk_apply_t), _ptr(rv_apply_t),
                          _ptr(seq_base), _ptr(seq_len), B, tq, int(bool(causal)), float(softmax_scale),
                          _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream())
    _check(st, "gqa_decode")
    return out, lse
