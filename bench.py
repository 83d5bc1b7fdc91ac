#!/usr/bin/env python3
"""Benchmark: one decode step of an INT2 rotated-latent MLA layer on one GPU.

A step is one pass of the whole hot path over one batch: quantise-on-append
of the step's new tokens (B x Tq latents rotated, clipped, INT2-packed into
their cache slots) followed by the absorbed split-K decode over the whole
cache (plan, query absorb, split-K attention, combine, up-projection).

Default workload: DeepSeek-V3-shaped layer, 128 heads, kv_lora_rank 512,
rope 64, batch 8, per-sequence context drawn uniformly in [16384, 32768]
("32k"), one query per sequence, INT2 groups of 32 + bf16 rope key.  Inputs
are seeded and synthetic (no dataset, no trained weights) and resident in
HBM before timing starts.  The cache is laid out in 8 separate copies used
in turn so the 256 MB Infinity Cache cannot serve a step from the previous
one.

Prints one JSON line (rank 0 only; one GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_MFMA_F16_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "splitk_decode_traffic.json")
KERNEL_SOURCES = ["int2_quantized_absorbed_amd/csrc/splitk.hip",
                  "int2_quantized_absorbed_amd/csrc/splitk_tile.hpp",
                  "int2_quantized_absorbed_amd/csrc/kernels.hpp",
                  "int2_quantized_absorbed_amd/csrc/common.hpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4])
    ap.add_argument("--copies", type=int, default=8, help="cache copies used in turn")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gqa", action="store_true",
                    help="skip the grouped-query (OSCAR full-attention) decode measurement")
    ap.add_argument("--no-sparse", action="store_true",
                    help="skip the sparse (indexer top-k) decode measurement")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (for scaling the HBM "
                         "byte counters of a profiler run) and exit")
    return ap.parse_args()


def copy_probe(mib: int) -> None:
    """A plain device-to-device copy of known size: a profiler's FETCH_SIZE /
    WRITE_SIZE for it should read mib MiB each per dispatch."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "dispatches": 3}))


def algorithmic_flops(w, lens) -> float:
    """Score + PV multiply-adds of the split-K kernel: per visible (token,
    query row) pair 2 * (2 r + d_r) flops, summed over heads."""
    r, dr, H, tq = w.kv_lora_rank, w.qk_rope_head_dim, w.num_heads, w.tq
    pairs = 0
    for L in lens:
        for t in range(tq):
            pairs += (L - tq + t + 1) if w.causal else L
    return 2.0 * H * (2 * r + dr) * pairs


def append_bytes_per_token(w) -> int:
    """Quantise-on-append traffic per token: bf16 latent, rope (and indexer)
    key and slot read; codes, fp16 scale/zero and the keys written."""
    keys = 2 * (w.qk_rope_head_dim + w.index_head_dim)
    return 2 * w.kv_lora_rank + keys + 8 + w.kv_lora_rank // 4 + 4 * (w.kv_lora_rank // w.group_size) + keys


def cache_bytes_per_token(w) -> int:
    return w.kv_lora_rank // 4 + 4 * (w.kv_lora_rank // w.group_size) + 2 * w.qk_rope_head_dim


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); this path is built and "
              "measured on one MI355X; sharding over GPUs is not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import int2_quantized_absorbed_amd as M
    from workloads import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = S.WORKLOADS[args.workload]
    st = S.streams(w.wid)
    d = M.Dims(w.kv_lora_rank, w.qk_rope_head_dim, w.qk_nope_head_dim, w.v_head_dim, w.num_heads,
               w.group_size, w.index_head_dim)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(torch.bfloat16)

    # ---- layer set-up through the library (untimed) ----
    model = S.latent_model(w, st)
    c_cal = S.calib_latents(w, st, model)
    c_cal_d = bf(c_cal)
    w_uk, w_uv = S.weights(w, st)
    # calibration (synchronous calls, timed on the host clock: set-up, not
    # part of the step)
    t = time.perf_counter()
    R, _ = M.mla_calibrate_rotation(d, c_cal_d)
    t_rot = time.perf_counter() - t
    t = time.perf_counter()
    M.mla_calibrate_rotation_weighted(d, c_cal_d, bf(w_uk), bf(w_uv))
    t_rotw = time.perf_counter() - t
    Rt = M.mla_prepare_rotation(d, R)
    grid = [1.0 - 0.05 * k for k in range(11)]
    torch.cuda.synchronize()
    t = time.perf_counter()
    alpha, _ = M.mla_fit_clip(d, c_cal_d, Rt, grid)
    t_clip = time.perf_counter() - t
    calibration = {"calib_tokens": int(c_cal.shape[0]), "rotation_ms": round(t_rot * 1e3, 2),
                   "rotation_weighted_ms": round(t_rotw * 1e3, 2), "fit_clip_ms": round(t_clip * 1e3, 2)}
    uk_f, uv_f = M.mla_fold_absorb_weights(d, bf(w_uk), bf(w_uv), Rt)

    lens = S.seq_lens(w, st)
    base, cap = S.contiguous_layout(lens)
    B, tq = len(lens), w.tq
    lat = S.torch_latents(model, cap, seed=1000 + w.wid, device=dev)
    kr = S.torch_normal_bf16((cap, w.qk_rope_head_dim), 2000 + w.wid, dev)
    idx = S.torch_normal_bf16((cap, w.index_head_dim), 3000 + w.wid, dev) if w.index_head_dim else None
    slots_all = torch.arange(cap, dtype=torch.int64, device=dev)
    caches = []
    for _ in range(args.copies):
        c = M.Cache(d, cap, dev)
        M.mla_append_quant(d, lat, kr, idx, slots_all, Rt, alpha, c)
        caches.append(c)
    # the step's new tokens: the last tq positions of every sequence
    step_slots = torch.tensor([int(base[b]) + int(lens[b]) - tq + t for b in range(B) for t in range(tq)],
                              dtype=torch.int64, device=dev)
    step_lat = lat[step_slots].contiguous()
    step_kr = kr[step_slots].contiguous()
    step_idx = idx[step_slots].contiguous() if idx is not None else None
    qn = S.torch_normal_bf16((B, tq, w.num_heads, w.qk_nope_head_dim), 4000 + w.wid, dev)
    qr = S.torch_normal_bf16((B, tq, w.num_heads, w.qk_rope_head_dim), 5000 + w.wid, dev)
    seq_base = torch.from_numpy(base).to(dev)
    seq_len = torch.from_numpy(lens).to(dev)
    ws = torch.empty(M.mla_decode_workspace_size(d, B, tq), dtype=torch.uint8, device=dev)
    out = torch.empty((B, tq, w.num_heads, w.v_head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((B, tq, w.num_heads), dtype=torch.float32, device=dev)
    scale = 1.0 / float(np.sqrt(w.qk_nope_head_dim + w.qk_rope_head_dim))
    del lat

    def step(k):
        # one decode step: the new tokens are quantised into the cache, then
        # every query attends over it (one call; the small append runs in
        # the query-absorb launch)
        c = caches[k % len(caches)]
        M.mla_decode_step(d, step_lat, step_kr, step_idx, step_slots, Rt, alpha, qn, qr, uk_f, uv_f, c, seq_base,
                          seq_len, tq, w.causal, scale, ws, out, lse)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t) * 1e3 / args.steps

    # second timed pass with the library's HIP events around every kernel
    # (recorded on the launch stream) for per-kernel durations
    M.mla_timing_enable(True)
    M.mla_timing_reset()
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    kernels = {}
    for name in ("append_quant", "append_absorb_q", "decode_plan", "absorb_q", "splitk_decode", "combine", "up_proj",
                 "combine_up_proj"):
        ms, n = M.mla_timing_query(name)
        if n:
            kernels[name] = round(ms / n * 1e3, 3)
    M.mla_timing_enable(False)

    # prefill-sized append (4 sequences x 4096 tokens of the 131k-context
    # workload, same layer shape) into a separate cache, timed with events
    n_pre = 4 * 4096
    pre_lat = S.torch_latents(model, n_pre, seed=6000 + w.wid, device=dev)
    pre_kr = S.torch_normal_bf16((n_pre, w.qk_rope_head_dim), 7000 + w.wid, dev)
    pre_idx = S.torch_normal_bf16((n_pre, w.index_head_dim), 8000 + w.wid, dev) if w.index_head_dim else None
    pre_slots = torch.arange(n_pre, dtype=torch.int64, device=dev)
    pre_cache = M.Cache(d, n_pre, dev)
    for _ in range(3):
        M.mla_append_quant(d, pre_lat, pre_kr, pre_idx, pre_slots, Rt, alpha, pre_cache)
    # 20 appends back to back between two events on the launch stream (the
    # library launches on torch's current stream), so host launch latency
    # does not enter the per-append time
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(20):
        M.mla_append_quant(d, pre_lat, pre_kr, pre_idx, pre_slots, Rt, alpha, pre_cache)
    ev1.record()
    torch.cuda.synchronize()
    pre_us = ev0.elapsed_time(ev1) / 20 * 1e3
    pre_bytes = n_pre * append_bytes_per_token(w)
    pre_flops = 2.0 * n_pre * w.kv_lora_rank * w.kv_lora_rank
    append_prefill = {
        "tokens": n_pre, "us": round(pre_us, 3), "algorithmic_bytes": pre_bytes,
        "GB/s": round(pre_bytes / (pre_us * 1e-6) / 1e9, 1),
        "hbm_frac": round(pre_bytes / (pre_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "mfma_frac": round(pre_flops / (pre_us * 1e-6) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
    }
    del pre_lat, pre_kr, pre_idx, pre_cache

    total_tokens = int(np.sum(lens))
    bpt = cache_bytes_per_token(w)
    cache_bytes = total_tokens * bpt
    value = cache_bytes / (ms_per_step * 1e-3) / 1e9
    flops = algorithmic_flops(w, lens)
    split_us = kernels.get("splitk_decode")
    achieved = flops / (split_us * 1e-6) / 1e12 if split_us else None
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("workload") == w.name:
            traffic = tr.get("bytes_per_launch")
    roofline = {
        "kernel": "splitk_decode",
        "bound": "mfma",
        "achieved": round(achieved, 2) if achieved else None,
        "peak": PEAK_MFMA_F16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4) if achieved else None,
        "traffic": traffic,
        "algorithmic_flops_per_launch": flops,
        "algorithmic_bytes_per_launch": cache_bytes,
        "hbm_frac_of_cache_stream": round(cache_bytes / (split_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if split_us else None,
    }

    result = {
        "metric": "INT2-latent MLA decode: cache GB/s vs HBM peak; query-tokens/s at 32k ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2 codes + fp16 scale/zero, bf16 rope; fp16 MFMA with fp32 accumulation",
        "data": "synthetic (seeded latents from a log-uniform spectrum, random-init bf16 weights)",
        "config": {
            "workload": w.name, "batch": B, "context_tokens": total_tokens, "context_min": int(lens.min()),
            "context_max": int(lens.max()), "tq": tq, "heads": w.num_heads, "kv_lora_rank": w.kv_lora_rank,
            "qk_rope_head_dim": w.qk_rope_head_dim, "group_size": w.group_size, "cache_bytes_per_token": bpt,
            "cache_copies": len(caches),
        },
        "query_tokens_per_s": round(B * tq / (ms_per_step * 1e-3), 1),
        "hbm_frac_step": round(value / PEAK_HBM_GBS, 4),
        "kernel_us": kernels,
        "append_prefill": append_prefill,
        "calibration": calibration,
        "roofline": roofline,
    }

    if not args.no_sparse:
        del caches
        torch.cuda.empty_cache()
        result["sparse_decode"] = sparse_bench(M, S, dev, args)

    if not args.no_gqa:
        if args.no_sparse:
            del caches
        torch.cuda.empty_cache()
        result["gqa_decode"] = gqa_bench(M, S, dev, args)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, st, c_cal, lat_seed=1000 + w.wid, lens=lens, base=base,
                                              model=model, w_uk=w_uk, w_uv=w_uv, qn=qn, qr=qr, kr=kr,
                                              out=out, budget=args.cpu_seconds, scale=scale)
    print(json.dumps(result))


def sparse_bench(M, S, dev, args):
    """Sparse decode through the indexer key on the GLM-5.3-Flash-like layer
    (64 heads, 64-dim indexer key), 4 sequences of 262,144 tokens, top-2048
    selection per sequence: index scores + exact top-k, then absorbed decode
    over the selected tokens; the dense decode of the same cache for context."""
    import torch
    w = S.WORKLOADS[4]
    st = S.streams(w.wid)
    d = M.Dims(w.kv_lora_rank, w.qk_rope_head_dim, w.qk_nope_head_dim, w.v_head_dim, w.num_heads,
               w.group_size, w.index_head_dim)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(torch.bfloat16)
    model = S.latent_model(w, st)
    c_cal_d = bf(S.calib_latents(w, st, model))
    w_uk, w_uv = S.weights(w, st)
    R, _ = M.mla_calibrate_rotation(d, c_cal_d)
    Rt = M.mla_prepare_rotation(d, R)
    alpha, _ = M.mla_fit_clip(d, c_cal_d, Rt, [1.0 - 0.05 * k for k in range(11)])
    uk_f, uv_f = M.mla_fold_absorb_weights(d, bf(w_uk), bf(w_uv), Rt)
    lens = S.seq_lens(w, st)
    base, cap = S.contiguous_layout(lens)
    B = len(lens)
    cache = M.Cache(d, cap, dev)
    for a in range(0, cap, 1 << 18):  # append in pieces to bound the latent buffer
        n = min(1 << 18, cap - a)
        lat = S.torch_latents(model, n, seed=1000 + w.wid + a, device=dev)
        kr = S.torch_normal_bf16((n, w.qk_rope_head_dim), 2000 + w.wid + a, dev)
        idx = S.torch_normal_bf16((n, w.index_head_dim), 3000 + w.wid + a, dev)
        M.mla_append_quant(d, lat, kr, idx, torch.arange(a, a + n, dtype=torch.int64, device=dev), Rt, alpha,
                           cache)
        del lat, kr, idx
    top_k = 2048
    q_idx = S.torch_normal_bf16((B, w.index_head_dim), 9000 + w.wid, dev)
    qn = S.torch_normal_bf16((B, 1, w.num_heads, w.qk_nope_head_dim), 4000 + w.wid, dev)
    qr = S.torch_normal_bf16((B, 1, w.num_heads, w.qk_rope_head_dim), 5000 + w.wid, dev)
    seq_base = torch.from_numpy(base).to(dev)
    seq_len = torch.from_numpy(lens).to(dev)
    ws_i = torch.empty(M.mla_index_topk_workspace_size(d, B, cap), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(M.mla_decode_workspace_size(d, B, 1), dtype=torch.uint8, device=dev)
    sel = torch.zeros((B, top_k), dtype=torch.int32, device=dev)
    n_sel = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, 1, w.num_heads, w.v_head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((B, 1, w.num_heads), dtype=torch.float32, device=dev)
    scale = 1.0 / float(np.sqrt(w.qk_nope_head_dim + w.qk_rope_head_dim))

    def step():
        M.mla_index_topk(d, q_idx, cache, seq_base, seq_len, top_k, ws_i, sel, n_sel)
        M.mla_decode_sparse(d, qn, qr, uk_f, uv_f, cache, seq_base, sel, n_sel, scale, ws_d, out, lse)

    def dense():
        M.mla_decode_absorbed(d, qn, qr, uk_f, uv_f, cache, seq_base, seq_len, 1, False, scale, ws_d, out, lse)

    n = max(args.steps // 2, 10)
    timings = {}
    for name, fn in (("sparse", step), ("dense", dense)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        timings[name] = (time.perf_counter() - t) * 1e3 / n
    M.mla_timing_enable(True)
    M.mla_timing_reset()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    k_us = {}
    for name in ("index_score", "index_select", "absorb_q", "splitk_decode", "combine", "up_proj", "combine_up_proj"):
        ms, cnt = M.mla_timing_query(name)
        if cnt:
            k_us[name] = round(ms / cnt * 1e3, 3)
    M.mla_timing_enable(False)
    tokens = int(np.sum(lens))
    score_bytes = tokens * (2 * w.index_head_dim + 4)   # read the index key, write one fp32 score
    sc_us = k_us.get("index_score")
    return {
        "workload": "glm53flash-layer-b4-ctx256k-top2048", "batch": B, "context_tokens": tokens,
        "heads": w.num_heads, "index_head_dim": w.index_head_dim, "top_k": top_k,
        "ms_per_step": round(timings["sparse"], 5),
        "query_tokens_per_s": round(B / (timings["sparse"] * 1e-3), 1),
        "dense_ms_per_step": round(timings["dense"], 5),
        "kernel_us": k_us,
        "index_score_roofline": {
            "bound": "hbm", "achieved": round(score_bytes / (sc_us * 1e-6) / 1e9, 1) if sc_us else None,
            "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(score_bytes / (sc_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if sc_us else None,
            "algorithmic_bytes_per_launch": score_bytes},
    }


def gqa_bench(M, S, dev, args):
    """OSCAR on a grouped-query layer: 32 query heads, 8 KV heads, head dim
    128, INT2 groups of 32, the 16k-32k context draw of the main measurement
    (8 sequences).  Calibration from 2048 synthetic tokens (anisotropic
    channels), K/V appended through gqa_append_quant, then decode steps of one
    query token per sequence."""
    import torch
    hq, hkv, hd, grp = 32, 8, 128, 32
    gd = M.GqaDims(hd, hq, hkv, grp)
    w2 = S.WORKLOADS[2]
    lens = S.seq_lens(w2, S.streams(w2.wid))
    base, cap = S.contiguous_layout(lens)
    B = len(lens)
    n_cal = 2048

    def aniso(shape, seed):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        ax = torch.exp(torch.empty(shape[-1], device=dev).uniform_(np.log(0.1), np.log(3.0), generator=g))
        return (torch.randn(shape, generator=g, device=dev) * ax).to(torch.bfloat16)

    q_cal, k_cal, v_cal = aniso((hq, n_cal, hd), 11), aniso((hkv, n_cal, hd), 12), aniso((hkv, n_cal, hd), 13)
    scale = float(np.float32(1.0 / np.sqrt(hd)))
    torch.cuda.synchronize()
    t = time.perf_counter()
    rk, rv, _, _ = M.gqa_calibrate(gd, q_cal, k_cal, v_cal, scale)
    calib_ms = (time.perf_counter() - t) * 1e3
    rk_t, rv_t = M.gqa_prepare_rotation(gd, rk), M.gqa_prepare_rotation(gd, rv)
    grid = [1.0 - 0.05 * k for k in range(11)]
    alpha_k, alpha_v = M.gqa_fit_clip(gd, k_cal, rk_t, grid), M.gqa_fit_clip(gd, v_cal, rv_t, grid)
    cache = M.GqaCache(gd, cap, dev)
    piece = 1 << 16
    for a in range(0, cap, piece):
        n = min(piece, cap - a)
        kn, vn = aniso((n, hkv, hd), 20000 + a), aniso((n, hkv, hd), 30000 + a)
        M.gqa_append_quant(gd, kn, vn, torch.arange(a, a + n, dtype=torch.int64, device=dev), rk_t, rv_t,
                           alpha_k, alpha_v, cache)
        del kn, vn
    q = S.torch_normal_bf16((B, 1, hq, hd), 40000, dev)
    seq_base, seq_len = torch.from_numpy(base).to(dev), torch.from_numpy(lens).to(dev)
    ws = torch.empty(M.gqa_decode_workspace_size(gd, B, 1), dtype=torch.uint8, device=dev)
    out = torch.empty((B, 1, hq, hd), dtype=torch.float32, device=dev)
    lse = torch.empty((B, 1, hq), dtype=torch.float32, device=dev)

    def step():
        M.gqa_decode(gd, q, cache, rk_t, rv_t, seq_base, seq_len, 1, True, scale, ws, out, lse)

    n = max(args.steps // 2, 10)
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / n
    M.mla_timing_enable(True)
    M.mla_timing_reset()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    k_us = {}
    for name in ("gqa_rotate_q", "decode_plan", "splitk_decode", "combine", "gqa_merge_unrotate"):
        c_ms, cnt = M.mla_timing_query(name)
        if cnt:
            k_us[name] = round(c_ms / cnt * 1e3, 3)
    M.mla_timing_enable(False)
    tokens = int(np.sum(lens))
    entry = 2 * (hd // 4 + (hd // grp) * 4)          # K and V: codes + fp16 scale/zero per token and KV head
    cache_bytes = tokens * hkv * entry
    sk_us = k_us.get("splitk_decode")
    return {
        "workload": "gqa-layer-h32-kv8-d128-b8-ctx16k-32k", "batch": B, "context_tokens": tokens,
        "q_heads": hq, "kv_heads": hkv, "head_dim": hd, "group_size": grp,
        "cache_bytes_per_token": hkv * entry,
        "ms_per_step": round(ms, 5),
        "GB/s": round(cache_bytes / (ms * 1e-3) / 1e9, 1),
        "query_tokens_per_s": round(B / (ms * 1e-3), 1),
        "kernel_us": k_us,
        "calibration_ms": round(calib_ms, 1),
        "splitk_roofline": {
            "bound": "hbm", "achieved": round(cache_bytes / (sk_us * 1e-6) / 1e9, 1) if sk_us else None,
            "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(cache_bytes / (sk_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if sk_us else None,
            "algorithmic_bytes_per_launch": cache_bytes},
    }


def cpu_baseline(w, st, c_cal, lat_seed, lens, base, model, w_uk, w_uv, qn, qr, kr, out, budget, scale):
    """The oracle (unchanged) on the host cores: quantise-on-append and
    absorbed decode of whole sequences of the same workload, sequence by
    sequence until the time budget is used.  Also reports the oracle-vs-GPU
    difference on those sequences (the benchmarked configuration)."""
    import torch
    from oracle import mla_oracle as O
    from workloads import synth as S

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = None
    cores = len(os.sched_getaffinity(0))
    # oracle calibration of the same layer (not timed: set-up)
    R, _, _ = O.calibrate_rotation(c_cal)
    alpha, _ = O.fit_clip(c_cal, R, w.group_size)
    Ra = O.rotation_apply(R)
    # the cache latents of the sampled sequences (regenerated: same seed)
    lat = S.torch_latents(model, int(base[-1] + lens[-1]), seed=lat_seed, device="cuda:0")
    qn_h = qn.float().cpu().numpy()
    qr_h = qr.float().cpu().numpy()
    out_h = out.cpu().numpy()
    done_tokens, t_used, worst = 0, 0.0, 0.0
    seqs = []
    for b in range(len(lens)):
        if t_used >= budget:
            break
        a, L = int(base[b]), int(lens[b])
        c = lat[a:a + L].float().cpu().numpy()
        k = kr[a:a + L].float().cpu().numpy()
        t0 = time.perf_counter()
        q = O.quantize_cache(c, Ra, alpha, w.group_size)
        zh = O.dequantize(q["codes"], q["scale_h"], q["zero_h"], w.group_size)
        ref, _ = O.rotated_attention(qn_h[b], qr_h[b], w_uk, w_uv, zh, k, Ra, scale, causal=w.causal)
        t_used += time.perf_counter() - t0
        done_tokens += L
        seqs.append(b)
        err = np.max(np.abs(out_h[b] - ref), axis=-1) / np.max(np.abs(ref), axis=-1)
        worst = max(worst, float(err.max()))
    bpt = cache_bytes_per_token(w)
    return {
        "value": round(done_tokens * bpt / t_used / 1e9, 4),
        "unit": "GB/s",
        "cores": threads if threads else cores,
        "cores_available": cores,
        "kind": "oracle",
        "sample": f"sequences {seqs} of the same workload ({done_tokens} cached tokens, all "
                  f"{w.num_heads} heads): quantise-on-append + absorbed decode, fp64 numpy; "
                  f"{t_used:.1f} s",
        "seconds": round(t_used, 2),
        "gpu_vs_oracle_worst_row_rel_err": worst,
    }


if __name__ == "__main__":
    main()
