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
HBM before timing starts.  Every measurement uses enough copies of its
cache (or of its input batches) in turn that the 256 MB Infinity Cache
cannot serve a call from the previous one.

Besides the headline line (value = cache GB/s of the step, the split-K
roofline, per-kernel HIP-event times, the oracle on the host cores), the
same JSON line carries: the prefill append of 4 x 4096 tokens; the same
decode at a 16-head share (HBM-bound); the same decode with the 4-bit rope
key; the 32 x 4096 and 4 x 131072 (8 causal drafts) workloads; the sparse
(indexer top-k) step and the dense decode on the 4 x 262144-token layer;
the grouped-query (OSCAR full-attention) step.  --only restricts the extras.

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
    ap.add_argument("--only", default="",
                    help="comma list of the extra measurements to run (append, h16, rope4, workloads, sparse, "
                         "gqa); default all")
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


def cache_bytes_per_token(w, rope_bits=0) -> int:
    """Bytes of one token the decode reads: codes, fp16 scale/zero and the
    rope key (bf16, or the 4-bit entry); the indexer key is not read."""
    d_r = w.qk_rope_head_dim
    rope = 2 * d_r if rope_bits == 0 else d_r // 2 + d_r // 4
    return w.kv_lora_rank // 4 + 4 * (w.kv_lora_rank // w.group_size) + rope


MALL_BYTES = 256 << 20   # MI355X Infinity Cache: rotate more bytes than this between timed calls


def copies_for(bytes_per_copy: int, at_least: int = 1) -> int:
    """Enough copies that the bytes touched in turn exceed the Infinity Cache."""
    return max(at_least, int(np.ceil(1.25 * MALL_BYTES / max(bytes_per_copy, 1))))


def time_calls(fn, n: int, warmup: int):
    """Wall time per call over n back-to-back calls (host clock, synchronised)."""
    import torch
    for k in range(warmup):
        fn(k)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for k in range(n):
        fn(k)
    torch.cuda.synchronize()
    return (time.perf_counter() - t) * 1e3 / n


def kernel_times(M, fn, n: int, names) -> dict:
    """Mean per-launch HIP-event time of each named kernel over n calls."""
    import torch
    M.mla_timing_enable(True)
    M.mla_timing_reset()
    torch.cuda.synchronize()
    for k in range(n):
        fn(k)
    torch.cuda.synchronize()
    out = {}
    for name in names:
        ms, cnt = M.mla_timing_query(name)
        if cnt:
            out[name] = round(ms / cnt * 1e3, 3)
    M.mla_timing_enable(False)
    return out


DECODE_KERNELS = ("append_quant", "append_rope", "append_absorb_q", "decode_plan", "absorb_q", "splitk_decode",
                  "combine", "up_proj", "combine_up_proj")


PIECE = 1 << 18  # cache tokens generated per piece (bounds the latent buffer)


def cache_piece(S, w, model, a, n, dev):
    """The seeded cache inputs of slots [a, a + n) of workload w (a piece
    start): latents, rope keys, indexer keys or None."""
    lat = S.torch_latents(model, n, seed=1000 + w.wid + a, device=dev)
    kr = S.torch_normal_bf16((n, w.qk_rope_head_dim), 2000 + w.wid + a, dev)
    idx = S.torch_normal_bf16((n, w.index_head_dim), 3000 + w.wid + a, dev) if w.index_head_dim else None
    return lat, kr, idx


def cache_pieces(S, w, model, cap, dev):
    """The cache inputs piece by piece: (first slot, count, latents, rope, indexer keys)."""
    for a in range(0, cap, PIECE):
        n = min(PIECE, cap - a)
        yield (a, n) + cache_piece(S, w, model, a, n, dev)


class Layer:
    """One MLA layer calibrated and folded through the library (untimed set-up)."""

    def __init__(self, M, S, dev, w, rope_bits=0, time_calibration=False):
        import torch
        self.w = w
        st = S.streams(w.wid)
        self.st = st
        self.d = M.Dims(w.kv_lora_rank, w.qk_rope_head_dim, w.qk_nope_head_dim, w.v_head_dim, w.num_heads,
                        w.group_size, w.index_head_dim, rope_bits)
        bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(torch.bfloat16)
        self.model = S.latent_model(w, st)
        self.c_cal = S.calib_latents(w, st, self.model)
        c_cal_d = bf(self.c_cal)
        self.w_uk, self.w_uv = S.weights(w, st)
        t = time.perf_counter()
        R, _ = M.mla_calibrate_rotation(self.d, c_cal_d)
        t_rot = time.perf_counter() - t
        self.calibration = None
        if time_calibration:
            t = time.perf_counter()
            M.mla_calibrate_rotation_weighted(self.d, c_cal_d, bf(self.w_uk), bf(self.w_uv))
            t_rotw = time.perf_counter() - t
        self.Rt = M.mla_prepare_rotation(self.d, R)
        torch.cuda.synchronize()
        t = time.perf_counter()
        self.alpha, _ = M.mla_fit_clip(self.d, c_cal_d, self.Rt, [1.0 - 0.05 * k for k in range(11)])
        t_clip = time.perf_counter() - t
        if time_calibration:
            self.calibration = {"calib_tokens": int(self.c_cal.shape[0]), "rotation_ms": round(t_rot * 1e3, 2),
                                "rotation_weighted_ms": round(t_rotw * 1e3, 2), "fit_clip_ms": round(t_clip * 1e3, 2)}
        self.uk_f, self.uv_f = M.mla_fold_absorb_weights(self.d, bf(self.w_uk), bf(self.w_uv), self.Rt)


def decode_step_bench(M, S, dev, w, steps, warmup, min_copies=1, rope_bits=0, keep=False, label=None,
                      time_calibration=False):
    """One decode step of workload w, timed: mla_decode_step appends the
    step's new tokens (the last tq positions of every sequence) and decodes
    every query over its whole cache.  The cache is laid out in enough copies,
    used in turn, that no step finds its bytes in the Infinity Cache."""
    import torch
    layer = Layer(M, S, dev, w, rope_bits, time_calibration)
    d = layer.d
    lens = S.seq_lens(w, layer.st)
    base, cap = S.contiguous_layout(lens)
    B, tq = len(lens), w.tq
    bpt = cache_bytes_per_token(w, rope_bits)
    n_copies = copies_for(cap * bpt, min_copies)
    first = M.Cache(d, cap, dev)
    # the step's new tokens: the last tq positions of every sequence, with the
    # inputs the cache holds there (each step rewrites the same entries)
    step_slots = torch.tensor([int(base[b]) + int(lens[b]) - tq + t for b in range(B) for t in range(tq)],
                              dtype=torch.int64, device=dev)
    n_new = len(step_slots)
    step_lat = torch.empty((n_new, w.kv_lora_rank), dtype=torch.bfloat16, device=dev)
    step_kr = torch.empty((n_new, w.qk_rope_head_dim), dtype=torch.bfloat16, device=dev)
    step_idx = torch.empty((n_new, w.index_head_dim), dtype=torch.bfloat16, device=dev) if w.index_head_dim else None
    for a, n, lat, kr, idx in cache_pieces(S, w, layer.model, cap, dev):
        M.mla_append_quant(d, lat, kr, idx, torch.arange(a, a + n, dtype=torch.int64, device=dev), layer.Rt,
                           layer.alpha, first)
        inside = (step_slots >= a) & (step_slots < a + n)
        step_lat[inside] = lat[step_slots[inside] - a]
        step_kr[inside] = kr[step_slots[inside] - a]
        if idx is not None:
            step_idx[inside] = idx[step_slots[inside] - a]
        del lat, kr, idx
    caches = [first]
    for _ in range(n_copies - 1):
        c = M.Cache(d, cap, dev)
        for name in ("codes", "scale_zero", "k_rope", "idx_key"):
            if getattr(c, name) is not None:
                getattr(c, name).copy_(getattr(first, name))
        caches.append(c)
    qn = S.torch_normal_bf16((B, tq, w.num_heads, w.qk_nope_head_dim), 4000 + w.wid, dev)
    qr = S.torch_normal_bf16((B, tq, w.num_heads, w.qk_rope_head_dim), 5000 + w.wid, dev)
    seq_base, seq_len = torch.from_numpy(base).to(dev), torch.from_numpy(lens).to(dev)
    ws = torch.empty(M.mla_decode_workspace_size(d, B, tq), dtype=torch.uint8, device=dev)
    out = torch.empty((B, tq, w.num_heads, w.v_head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((B, tq, w.num_heads), dtype=torch.float32, device=dev)
    scale = 1.0 / float(np.sqrt(w.qk_nope_head_dim + w.qk_rope_head_dim))

    def step(k):
        M.mla_decode_step(d, step_lat, step_kr, step_idx, step_slots, layer.Rt, layer.alpha, qn, qr, layer.uk_f,
                          layer.uv_f, caches[k % len(caches)], seq_base, seq_len, tq, w.causal, scale, ws, out, lse)

    ms = time_calls(step, steps, warmup)
    kus = kernel_times(M, step, steps, DECODE_KERNELS)
    tokens = int(np.sum(lens))
    cache_bytes = tokens * bpt
    flops = algorithmic_flops(w, lens)
    sk = kus.get("splitk_decode")
    ai = flops / cache_bytes
    bound = "mfma" if ai > PEAK_MFMA_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    if bound == "mfma":
        ach = flops / (sk * 1e-6) / 1e12 if sk else None
        roof = {"bound": "mfma", "achieved": ach and round(ach, 2), "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach and round(ach / PEAK_MFMA_F16_TFLOPS, 4)}
    else:
        ach = cache_bytes / (sk * 1e-6) / 1e9 if sk else None
        roof = {"bound": "hbm", "achieved": ach and round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach and round(ach / PEAK_HBM_GBS, 4)}
    roof.update({"kernel": "splitk_decode", "algorithmic_flops_per_launch": flops,
                 "algorithmic_bytes_per_launch": cache_bytes, "flop_per_byte": round(ai, 1),
                 "hbm_frac_of_cache_stream": round(cache_bytes / (sk * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if sk else None})
    res = {
        "workload": label or w.name, "batch": B, "tq": tq, "heads": w.num_heads, "context_tokens": tokens,
        "context_min": int(lens.min()), "context_max": int(lens.max()), "rope_bits": rope_bits,
        "cache_bytes_per_token": bpt, "cache_copies": len(caches), "ms_per_step": round(ms, 5),
        "cache_GB/s": round(cache_bytes / (ms * 1e-3) / 1e9, 2),
        "query_tokens_per_s": round(B * tq / (ms * 1e-3), 1), "kernel_us": kus, "splitk_roofline": roof,
    }
    if keep:
        res["_ctx"] = dict(layer=layer, lens=lens, base=base, qn=qn, qr=qr, out=out, scale=scale,
                           calibration=layer.calibration)
    del caches, first
    return res


def append_prefill_bench(M, S, dev, w, reps=40):
    """Quantise-on-append of a 4 x 4096-token bf16 prefill (the 131k-context
    workload's append, same layer shape).  Enough distinct input batches and
    target caches are used in turn (more bytes than the Infinity Cache holds)
    that no call finds its inputs or outputs there; the calls run back to back
    between two events on the launch stream."""
    import torch
    layer = Layer(M, S, dev, w)
    d = layer.d
    n_pre = 4 * 4096
    per_call = n_pre * append_bytes_per_token(w)
    n_sets = copies_for(per_call, 2)
    sets = []
    for k in range(n_sets):
        lat = S.torch_latents(layer.model, n_pre, seed=6000 + 31 * k, device=dev)
        kr = S.torch_normal_bf16((n_pre, w.qk_rope_head_dim), 7000 + 31 * k, dev)
        idx = S.torch_normal_bf16((n_pre, w.index_head_dim), 8000 + 31 * k, dev) if w.index_head_dim else None
        slots = torch.arange(n_pre, dtype=torch.int64, device=dev)
        sets.append((lat, kr, idx, slots, M.Cache(d, n_pre, dev)))

    def call(k):
        lat, kr, idx, slots, cache = sets[k % n_sets]
        M.mla_append_quant(d, lat, kr, idx, slots, layer.Rt, layer.alpha, cache)

    for k in range(2 * n_sets):
        call(k)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for k in range(reps):
        call(k)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) / reps * 1e3
    kus = kernel_times(M, call, reps, ("append_quant",))
    flops = 2.0 * n_pre * w.kv_lora_rank * w.kv_lora_rank
    return {
        "tokens": n_pre, "input_sets_in_turn": n_sets, "us": round(us, 3), "kernel_us": kus,
        "algorithmic_bytes": per_call, "GB/s": round(per_call / (us * 1e-6) / 1e9, 1),
        "hbm_frac": round(per_call / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "mfma_frac": round(flops / (us * 1e-6) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
    }


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the decode path runs on a "
              "single MI355X and does not shard over GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    import int2_quantized_absorbed_amd as M
    from workloads import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    parts = set(args.only.split(",")) if args.only else None
    want = lambda name: parts is None or name in parts
    w = S.WORKLOADS[args.workload]

    head = decode_step_bench(M, S, dev, w, args.steps, args.warmup, min_copies=args.copies, keep=True,
                             time_calibration=True)
    ctx = head.pop("_ctx")
    roof = dict(head["splitk_roofline"])
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("workload") == w.name:
            traffic = tr.get("bytes_per_launch")
    roof["traffic"] = traffic
    ms = head["ms_per_step"]
    result = {
        "metric": "INT2-latent MLA decode: cache GB/s vs HBM peak; query-tokens/s at 32k ctx",
        "value": head["cache_GB/s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2 codes + fp16 scale/zero, bf16 rope; fp16 MFMA with fp32 accumulation",
        "data": "synthetic (seeded latents from a log-uniform spectrum, random-init bf16 weights)",
        "config": {
            "workload": w.name, "batch": head["batch"], "context_tokens": head["context_tokens"],
            "context_min": head["context_min"], "context_max": head["context_max"], "tq": head["tq"],
            "heads": w.num_heads, "kv_lora_rank": w.kv_lora_rank, "qk_rope_head_dim": w.qk_rope_head_dim,
            "group_size": w.group_size, "cache_bytes_per_token": head["cache_bytes_per_token"],
            "cache_copies": head["cache_copies"],
        },
        "query_tokens_per_s": head["query_tokens_per_s"],
        "hbm_frac_step": round(head["cache_GB/s"] / PEAK_HBM_GBS, 4),
        "kernel_us": head["kernel_us"],
        "calibration": ctx["calibration"],
        "roofline": roof,
    }
    n_extra = max(args.steps // 3, 20)
    if want("append"):
        result["append_prefill"] = append_prefill_bench(M, S, dev, S.WORKLOADS[3])
    if want("h16"):
        # one GPU's share of the 128 heads under 8-way head parallelism (the
        # latent cache is replicated): the HBM-bound shape of the same decode
        result["decode_h16"] = decode_step_bench(M, S, dev, w.with_(num_heads=16), n_extra, 5,
                                                 label=w.name + "-h16")
    if want("rope4"):
        result["rope_int4"] = decode_step_bench(M, S, dev, w, n_extra, 5, rope_bits=4, label=w.name + "-rope4")
    if want("workloads"):
        for wid in (1, 3):
            if wid != args.workload:
                result[f"workload_{wid}"] = decode_step_bench(M, S, dev, S.WORKLOADS[wid], n_extra, 5)
        torch.cuda.empty_cache()
    if want("sparse"):
        torch.cuda.empty_cache()
        result["sparse_decode"] = sparse_bench(M, S, dev, args)
    if want("gqa"):
        torch.cuda.empty_cache()
        result["gqa_decode"] = gqa_bench(M, S, dev, args)
    if not args.no_cpu_baseline:
        lay = ctx["layer"]
        result["cpu_baseline"] = cpu_baseline(w, lay.st, lay.c_cal, lens=ctx["lens"], base=ctx["base"],
                                              model=lay.model, w_uk=lay.w_uk, w_uv=lay.w_uv, qn=ctx["qn"],
                                              qr=ctx["qr"], out=ctx["out"], budget=args.cpu_seconds,
                                              scale=ctx["scale"])
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

    # the index keys (the bytes the selection streams) exceed the Infinity
    # Cache once copies are used in turn
    caches = [cache] + [M.Cache(d, cap, dev) for _ in range(copies_for(cap * 2 * w.index_head_dim, 2) - 1)]
    for c in caches[1:]:
        for name in ("codes", "scale_zero", "k_rope", "idx_key"):
            getattr(c, name).copy_(getattr(cache, name))

    def step(k):
        c = caches[k % len(caches)]
        M.mla_index_topk(d, q_idx, c, seq_base, seq_len, top_k, ws_i, sel, n_sel)
        M.mla_decode_sparse(d, qn, qr, uk_f, uv_f, c, seq_base, sel, n_sel, scale, ws_d, out, lse)

    def dense(k):
        M.mla_decode_absorbed(d, qn, qr, uk_f, uv_f, caches[k % len(caches)], seq_base, seq_len, 1, False, scale,
                              ws_d, out, lse)

    n = max(args.steps // 2, 10)
    timings = {name: time_calls(fn, n, 5) for name, fn in (("sparse", step), ("dense", dense))}
    k_us = kernel_times(M, step, n, ("index_score", "index_select", "absorb_q", "splitk_decode", "combine",
                                     "up_proj", "combine_up_proj"))
    dk_us = kernel_times(M, dense, n, ("absorb_q", "splitk_decode", "combine_up_proj"))
    tokens = int(np.sum(lens))
    score_bytes = tokens * (2 * w.index_head_dim + 4)   # read the index key, write one fp32 score
    sc_us = k_us.get("index_score")
    dense_flops = algorithmic_flops(w, lens)
    dsk = dk_us.get("splitk_decode")
    return {
        "workload": "glm53flash-layer-b4-ctx256k-top2048", "batch": B, "context_tokens": tokens,
        "heads": w.num_heads, "index_head_dim": w.index_head_dim, "top_k": top_k,
        "ms_per_step": round(timings["sparse"], 5),
        "query_tokens_per_s": round(B / (timings["sparse"] * 1e-3), 1),
        "dense_ms_per_step": round(timings["dense"], 5),
        "dense_kernel_us": dk_us,
        "dense_splitk_roofline": {
            "bound": "mfma", "achieved": round(dense_flops / (dsk * 1e-6) / 1e12, 2) if dsk else None,
            "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(dense_flops / (dsk * 1e-6) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4) if dsk else None,
            "hbm_frac_of_cache_stream": round(tokens * cache_bytes_per_token(w) / (dsk * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            if dsk else None},
        "cache_copies": len(caches),
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

    tokens = int(np.sum(lens))
    entry = 2 * (hd // 4 + (hd // grp) * 4)          # K and V: codes + fp16 scale/zero per token and KV head
    cache_bytes = tokens * hkv * entry
    caches = [cache] + [M.GqaCache(gd, cap, dev) for _ in range(copies_for(cap * hkv * entry, 2) - 1)]
    for c in caches[1:]:
        for name in ("k_codes", "k_scale_zero", "v_codes", "v_scale_zero"):
            getattr(c, name).copy_(getattr(cache, name))

    def step(k):
        M.gqa_decode(gd, q, caches[k % len(caches)], rk_t, rv_t, seq_base, seq_len, 1, True, scale, ws, out, lse)

    n = max(args.steps // 2, 10)
    ms = time_calls(step, n, 5)
    k_us = kernel_times(M, step, n, ("gqa_rotate_q", "decode_plan", "splitk_decode", "combine", "gqa_merge_unrotate"))
    sk_us = k_us.get("splitk_decode")
    return {
        "workload": "gqa-layer-h32-kv8-d128-b8-ctx16k-32k", "batch": B, "context_tokens": tokens,
        "q_heads": hq, "kv_heads": hkv, "head_dim": hd, "group_size": grp,
        "cache_bytes_per_token": hkv * entry,
        "cache_copies": len(caches),
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


def cpu_baseline(w, st, c_cal, lens, base, model, w_uk, w_uv, qn, qr, out, budget, scale):
    """The oracle (unchanged) on the host cores: quantise-on-append and
    absorbed decode of whole sequences of the same workload, sequence by
    sequence until the time budget is used, the append timed on its own too.
    Also reports the oracle-vs-GPU difference on those sequences (the
    benchmarked configuration)."""
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
    cap = int(base[-1] + lens[-1])
    qn_h = qn.float().cpu().numpy()
    qr_h = qr.float().cpu().numpy()
    out_h = out.cpu().numpy()
    done_tokens, t_used, t_append, worst = 0, 0.0, 0.0, 0.0
    seqs = []
    pieces = {}
    for b in range(len(lens)):
        if t_used >= budget:
            break
        a0, L = int(base[b]), int(lens[b])
        # the sequence's cache inputs, regenerated from their seeds
        lat_parts, kr_parts = [], []
        for pa in range((a0 // PIECE) * PIECE, a0 + L, PIECE):
            if pa not in pieces:
                pieces.clear()
                lat, kr, _ = cache_piece(S, w, model, pa, min(PIECE, cap - pa), "cuda:0")
                pieces[pa] = (lat.float().cpu().numpy(), kr.float().cpu().numpy())
            lo, hi = max(a0, pa), min(a0 + L, pa + PIECE)
            lat_parts.append(pieces[pa][0][lo - pa:hi - pa])
            kr_parts.append(pieces[pa][1][lo - pa:hi - pa])
        c, k = np.concatenate(lat_parts), np.concatenate(kr_parts)
        t0 = time.perf_counter()
        q = O.quantize_cache(c, Ra, alpha, w.group_size)
        t1 = time.perf_counter()
        zh = O.dequantize(q["codes"], q["scale_h"], q["zero_h"], w.group_size)
        ref, _ = O.rotated_attention(qn_h[b], qr_h[b], w_uk, w_uv, zh, k, Ra, scale, causal=w.causal)
        t_used += time.perf_counter() - t0
        t_append += t1 - t0
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
        "append_us_per_token": round(t_append / max(done_tokens, 1) * 1e6, 3),
        "decode_ms_per_query_token": round((t_used - t_append) / max(len(seqs) * w.tq, 1) * 1e3, 1),
        "gpu_vs_oracle_worst_row_rel_err": worst,
    }


if __name__ == "__main__":
    main()
