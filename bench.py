#!/usr/bin/env python3
"""Benchmark of the transform-coded KV cache hot path on one MI355X.

One step = prefill-encode of the whole context of a Llama-3.1-8B-shaped attention layer
(8 KV heads, 32 query heads, head_dim 128, 131072 tokens, bf16 K/V, 2.75 bits/element)
followed by one decode-attention step over the packed cache.  Inputs are seeded synthetic
tensors (synth/) resident in HBM before timing starts; the codebook comes from the
library's own host calibration on synthetic calibration data.

Prints one JSON line.  `value` is the decode-attention effective HBM bandwidth
(algorithmic bytes / time); encode tokens/s, both kernels' roofline figures and the CPU
oracle baseline ride along.  The device's 256 MB last-level cache is flushed (512 MB
streaming write, untimed) before every timed encode and decode.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "quantized_attention_klt_amd", "csrc")
DECODE_PMC = (os.path.join(PROFILES, "decode_kernel_llama128k_pmc.txt"), os.path.join(CSRC, "decode.hip"))
ENCODE_PMC = (os.path.join(PROFILES, "encode_kernel_llama128k_pmc.txt"), os.path.join(CSRC, "encode.hip"))
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "decode-attn effective HBM GB/s (% of peak) + encode tokens/s, 128k ctx, 2.75 b/elem"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


VQ_TRAIN, VQ_ITERS = 8192, 20  # key codebook training draws and Lloyd rounds


def vq_keys(w) -> bool:
    """Workloads whose keys are vector-quantized (one byte per group of 4 coefficients)."""
    return "vq" in w.name


def build_inputs(wname: str, ctx: int):
    import synth
    import quantized_attention_klt_amd as q
    w = synth.WORKLOADS[wname]
    t0 = time.perf_counter()
    stats = []
    hms = []
    for h in range(w.n_kv):
        hm = synth.head_model(w, 0, h)
        hms.append(hm)
        K, V, Q = synth.calibration_samples(w, hm, 0, h)
        stats.append(q.stats_from_samples(K, V, Q))
    t1 = time.perf_counter()
    if vq_keys(w):
        cb = q.calibrate(stats, w.d, 1, w.n_kv, w.group, w.avg_bits, joint=False, key_quantizer="vq",
                         vq_normals=synth.vq_normals(w, 0, VQ_TRAIN), vq_iters=VQ_ITERS)
    else:
        cb = q.calibrate(stats, w.d, 1, w.n_kv, w.group, w.avg_bits)
    t2 = time.perf_counter()
    log(f"calibration: stats {t1 - t0:.2f}s, calibrate {t2 - t1:.2f}s")
    kb = np.zeros((1, ctx, w.n_kv, w.d), np.uint16)
    vb = np.zeros_like(kb)
    for h, hm in enumerate(hms):
        K, V = synth.cache_kv(w, hm, 0, 0, h, ctx)
        kb[0, :, h] = synth.to_bf16_bits(K)
        vb[0, :, h] = synth.to_bf16_bits(V)
    qb = synth.to_bf16_bits(synth.decode_queries(w, hms, 0, 0))[None]
    log(f"inputs generated ({time.perf_counter() - t2:.1f}s)")
    return w, cb, kb, vb, qb, t2 - t0


def source_hash(path: str) -> str:
    """Hash of a kernel source's code: line comments and blank lines are dropped and
    whitespace runs collapsed, so that only a change of the code itself invalidates the
    counters taken on it."""
    lines = []
    with open(path, encoding="utf-8") as f:
        for line in f:
            code = " ".join(line.split("//", 1)[0].split())
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def measured_traffic(summary: str, source: str):
    """HBM bytes per launch of a kernel from its committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy of known size), or None when the summary is missing
    or was taken from another revision of the kernel source."""
    try:
        fields = dict(l.split(":", 1) for l in open(summary) if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("source_sha256_16") != source_hash(source):
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(wname: str, n_tokens: int = 16384):
    """Oracle (numpy, float64) on one kv-head and n_tokens tokens: encode and decode rates."""
    import oracle
    import synth
    w = synth.WORKLOADS[wname]
    hm = synth.head_model(w, 0, 0)
    K, V, Q = synth.calibration_samples(w, hm, 0, 0)
    if vq_keys(w):
        cb = oracle.build_head_codebook(oracle.head_stats(K, V, Q), w.avg_bits, joint=False,
                                        key_quantizer="vq", vq_normals=synth.vq_normals(w, 0, VQ_TRAIN),
                                        vq_iters=VQ_ITERS)
    else:
        # the oracle encodes the library's packed layout: key records in whole 32-bit words
        cb = oracle.build_head_codebook(oracle.head_stats(K, V, Q), w.avg_bits, key_align=32)
    Kc, Vc = synth.cache_kv(w, hm, 0, 0, 0, n_tokens)
    kf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Kc))
    vf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Vc))
    q = synth.bf16_bits_to_f64(synth.to_bf16_bits(synth.decode_queries(w, [hm], 0, 0)))
    t0 = time.perf_counter()
    cache, _, _ = oracle.encode_cache(kf, vf, cb)
    t1 = time.perf_counter()
    oracle.decode_attention(cache, cb, q, n_tokens)
    t2 = time.perf_counter()
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    tb = oracle.tile_bytes(oracle.key_record_bits(cb), cb.bV)
    dec_bytes = n_tokens * tb / 64
    return {
        "value": dec_bytes / (t2 - t1) / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
        "sample": f"one kv-head of the workload, {n_tokens} tokens: oracle encode then oracle decode of one "
                  f"4-query-head group; decode rate = packed bytes / decode time",
        "encode_tokens_per_s": n_tokens / (t1 - t0),
        "encode_s": t1 - t0, "decode_s": t2 - t1,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--ctx", type=int, default=0, help="override context length")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path has no multi-GPU "
              "component (it would shard by kv-head, by sequence, or by context with an all-gather of "
              "the split partials).", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_attention_klt_amd as q
    q.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    import synth
    w0 = synth.WORKLOADS[args.workload]
    ctx = args.ctx or w0.ctx
    w, cb, kb, vb, qb, calib_s = build_inputs(args.workload, ctx)
    dev = torch.device("cuda:0")
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device=dev)
    cb.upload(blob)
    cache_t = torch.zeros(cb.cache_bytes(1, 1, ctx), dtype=torch.uint8, device=dev)
    cache = q.make_cache(cache_t, 1, 1, ctx)
    K = torch.from_numpy(kb.view(np.int16)).to(dev)
    V = torch.from_numpy(vb.view(np.int16)).to(dev)
    Qd = torch.from_numpy(qb.view(np.int16)).to(dev)
    out = torch.empty((1, w.n_q, w.d), dtype=torch.float32, device=dev)
    ws = torch.zeros(cb.decode_workspace_bytes(1, ctx), dtype=torch.uint8, device=dev)
    ids = torch.zeros(1, dtype=torch.int32, device=dev)
    lens = torch.full((1,), ctx, dtype=torch.int64, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    del kb, vb

    def encode():
        q.encode(cb, blob, cache, 0, [0], [0], ctx, K, V)

    def decode():
        q.decode_attention(cb, blob, cache, 0, ids, lens, ctx, Qd, out, ws)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        q.flush_write(flush)
        encode()
        q.flush_write(flush)
        decode()
    torch.cuda.synchronize()
    # timed region: the whole step, events around the encode and the decode call
    t0 = time.perf_counter()
    for i in range(args.steps):
        q.flush_write(flush)
        ev[i][0].record()
        encode()
        ev[i][1].record()
        q.flush_write(flush)
        ev[i][2].record()
        decode()
        ev[i][3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    # second timed region, same steps: device events around the split-decode kernel alone
    # (kept out of the first region: markers between kernels stretch the call they sit in)
    q.profile_begin(args.steps)
    for i in range(args.steps):
        q.flush_write(flush)
        decode()
    torch.cuda.synchronize()
    kern_ms = q.profile_end(args.steps)
    if args.copy_probe_mb:
        a = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mb} MiB read + written")

    tb = cb.tile_bytes
    n_tiles = (ctx + 63) // 64
    cache_bytes = w.n_kv * n_tiles * tb
    vq = vq_keys(w)
    # vector-quantized keys: the codebooks (n_g x 256 words of 4 fp32) are side information too
    books = w.n_kv * (w.d * w.avg_bits // 8) * 256 * 4 * 4 if vq else 0
    side = 2 * w.n_kv * w.d * w.d * 4 + w.n_q * w.d * 2 + w.n_q * w.d * 4 + books
    dec_bytes = int(cache_bytes + side)
    # the split-decode kernel alone: the packed cache, U_K (or T_K^-1), the codebooks, the bf16 queries
    kern_bytes = int(cache_bytes + w.n_kv * w.d * w.d * 4 + w.n_q * w.d * 2 + books)
    kern_s = float(kern_ms.mean()) / 1e3
    kern_gbs = kern_bytes / kern_s / 1e9
    enc_bytes = 2 * ctx * w.n_kv * w.d * 2 + cache_bytes
    dec_s = dec_ms.mean() / 1e3
    enc_s = enc_ms.mean() / 1e3
    dec_gbs = dec_bytes / dec_s / 1e9
    enc_gbs = enc_bytes / enc_s / 1e9
    enc_flops = 2 * 2 * ctx * w.n_kv * w.d * w.d  # K and V projections, algorithmic
    res = {
        "metric": METRIC,
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float((enc_ms + dec_ms).mean()), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f32",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b-attention-layer" + ("-vq-keys" if vq else ""),
                   "kv_heads": w.n_kv, "q_heads": w.n_q,
                   "head_dim": w.d, "ctx": ctx, "batch": 1, "bits_per_element": w.avg_bits,
                   "step": "prefill-encode of ctx tokens + one decode-attention step"},
        "decode_ms": round(float(dec_ms.mean()), 4),
        "decode_bytes": dec_bytes,
        "decode_ms_min": round(float(dec_ms.min()), 4),
        "decode_frac_of_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "encode_ms": round(float(enc_ms.mean()), 4),
        "encode_tokens_per_s": round(ctx / enc_s, 1),
        "encode_gbs": round(enc_gbs, 2),
        "compression_ratio": round(16.0 / w.avg_bits, 4),
        "calibration_s": round(calib_s, 3),
        "wall_s_timed_region": round(wall, 3),
        "roofline": {"kernel": ("vq_decode_kernel (split decode over vector-quantized keys)" if vq else
                                "decode_kernel (split decode: scores, online softmax, value sums)"),
                     "bound": "hbm",
                     "achieved": round(kern_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if vq else measured_traffic(*DECODE_PMC),
                     "algorithmic_bytes": kern_bytes, "kernel_ms": round(kern_s * 1e3, 4),
                     "source_sha256_16": source_hash(DECODE_PMC[1])},
        "roofline_encode": {"kernel": "encode", "bound": "hbm", "achieved": round(enc_gbs, 2),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(enc_gbs / HBM_PEAK_GBS, 4),
                            "mfma_tflops": round(enc_flops / enc_s / 1e12, 2),
                            "mfma_frac": round(enc_flops / enc_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                            "traffic": None if vq else measured_traffic(*ENCODE_PMC),
                            "algorithmic_bytes": enc_bytes,
                            "source_sha256_16": source_hash(ENCODE_PMC[1])},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
