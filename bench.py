#!/usr/bin/env python3
"""Benchmark of the transform-coded KV cache hot path on one MI355X.

Default workload (the headline): a Llama-3.1-8B-shaped attention layer (8 KV heads, 32
query heads, head_dim 128) at 131072 cached tokens and 2.75 bits/element.  One step =
prefill-encode of the whole context + one decode-attention step over the packed cache.
The codebook comes from the library's own host calibration on seeded synthetic
calibration data.

Other workloads (--workload):
  llama_32k      the same layer at 32768 tokens;
  qwen_128k      a Qwen-2.5-7B-shaped model, all 28 layers (4 KV / 28 query heads) at
                 131072 tokens: one decode step across the layers (28 calls in a HIP graph);
  llama_batch    Llama geometry, 32 layers x 32 sequences x 8192 tokens: one batched decode
                 step (32 calls in a HIP graph);
  llama_loop     one Llama layer, 65536 cached tokens, 1024 generation steps at 2.0 b/e, each
                 appending one token per kv-head and attending over the grown cache
                 (aatc_decode_attention_append);
  llama_vq_128k  the headline layer with vector-quantized keys at 2.0 b/e.

Inputs are resident in HBM before timing starts.  The device's 256 MB last-level cache
is flushed (512 MB streaming write, untimed) before every timed encode and decode.
Prints one JSON line: `value` is the decode-attention effective HBM bandwidth
(algorithmic bytes / time of the decode call(s)); the decode kernel's roofline (with the
read rate of the library's streaming probe on the same bytes), the encoder's, and the CPU
oracle baseline ride along.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

import synth

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "quantized_attention_klt_amd", "csrc")
DECODE_PMC = (os.path.join(PROFILES, "decode_kernel_llama128k_pmc.txt"), os.path.join(CSRC, "decode.hip"))
ENCODE_PMC = (os.path.join(PROFILES, "encode_kernel_llama128k_pmc.txt"), os.path.join(CSRC, "encode.hip"))
VQ_DECODE_PMC = (os.path.join(PROFILES, "vq_decode_kernel_llama128k_pmc.txt"), os.path.join(CSRC, "decode.hip"))
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "decode-attn effective HBM GB/s (% of peak) + encode tokens/s, 128k ctx, 2.75 b/elem"
FLUSH_BYTES = 512 << 20

WORKLOAD_LABELS = {
    "llama_128k": "llama3.1-8b-shaped attention layer, 131072 tokens, 2.75 b/e",
    "llama_32k": "llama3.1-8b-shaped attention layer, 32768 tokens, 2.75 b/e",
    "qwen_128k": "qwen2.5-7b-shaped model, 28 layers, 131072 tokens, 2.75 b/e",
    "llama_batch": "llama3.1-8b geometry, 32 layers x 32 sequences x 8192 tokens, 2.75 b/e",
    "llama_loop": "llama3.1-8b-shaped layer, 65536 -> 66560 tokens, 1024 append+decode steps, 2.0 b/e",
    "llama_vq_128k": "llama3.1-8b-shaped attention layer, 131072 tokens, vector-quantized keys, 2.0 b/e",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


VQ_TRAIN, VQ_ITERS = 8192, 20  # key codebook training draws and Lloyd rounds


def vq_keys(w) -> bool:
    """Workloads whose keys are vector-quantized (one byte per group of 4 coefficients)."""
    return "vq" in w.name


def path_dtype(w) -> str:
    """The arithmetic the decode path computes in: int8 MFMA digit products with fp32
    combination for scalar keys; fp32 score tables and fp16 value MFMAs for VQ keys."""
    return "f32+f16" if vq_keys(w) else "i8+f32"


def calibrate(w, q, n_layers: int):
    """Library host calibration of every (layer, kv-head) of the workload."""
    t0 = time.perf_counter()
    stats, hms = [], []
    for layer in range(n_layers):
        for h in range(w.n_kv):
            hm = synth.head_model(w, layer, h)
            hms.append(hm)
            K, V, Q = synth.calibration_samples(w, hm, layer, h)
            stats.append(q.stats_from_samples(K, V, Q))
    t1 = time.perf_counter()
    if vq_keys(w):
        cb = q.calibrate(stats, w.d, n_layers, w.n_kv, w.group, w.avg_bits, joint=False, key_quantizer="vq",
                         vq_normals=synth.vq_normals(w, 0, VQ_TRAIN), vq_iters=VQ_ITERS)
    else:
        cb = q.calibrate(stats, w.d, n_layers, w.n_kv, w.group, w.avg_bits)
    t2 = time.perf_counter()
    log(f"calibration of {len(stats)} heads: stats {t1 - t0:.2f}s, calibrate {t2 - t1:.2f}s")
    return cb, hms, t2 - t0


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


def profiled_us(summary: str, kernel: str):
    """Average duration (us) of the kernel whose name starts with `kernel` in a committed
    rocprofv3 --stats summary (profiles/*_kstats.txt), or None."""
    try:
        for line in open(summary):
            if not line.startswith("#") and kernel in line.split("(")[0]:
                return float(line.split()[-3])
    except (OSError, ValueError, IndexError):
        pass
    return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wname: str, n_tokens: int = 16384):
    """Oracle (numpy, float64) on a bounded sample: one kv-head of the workload's first
    layer, n_tokens tokens - oracle encode then oracle decode of its query-head group."""
    import oracle
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
    rate = dec_bytes / (t2 - t1) / 1e9
    full = w.n_layers * w.n_seqs * w.n_kv * w.ctx * tb / 64
    return {
        "value": rate, "unit": "GB/s", "cores": int(cores), "cpu_model": cpu_model(), "kind": "oracle",
        "sample": f"one kv-head of the first layer, {n_tokens} tokens: oracle encode, then oracle decode of its "
                  f"{w.group}-query-head group; decode rate = packed bytes / decode time",
        "scale_up": f"the rate is per byte and the same for every (layer, sequence, kv-head); at it the whole "
                    f"workload's {full / 1e6:.0f} MB of packed cache would take {full / rate / 1e9:.1f} s per decode step",
        "encode_tokens_per_s": n_tokens / (t1 - t0),
        "encode_s": t1 - t0, "decode_s": t2 - t1,
    }


class Timer:
    """Device events on torch's current stream around a region."""

    def __init__(self, torch, n):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]

    def start(self, i):
        self.ev[i][0].record()

    def stop(self, i):
        self.ev[i][1].record()

    def ms(self):
        return np.array([a.elapsed_time(b) for a, b in self.ev])


def probe_rates(torch, q, dev, nbytes: int, tile_bytes: int, cache_t, flush, reps: int):
    """Read rate (GB/s, median over reps, LLC flushed before each) of the library's
    streaming probe: plain loads of nbytes, and the decode kernel's tile stream over the
    cache buffer."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    res = {}
    for name, mode, buf, n in (("plain", 0, src, nbytes), ("tiles", 1, cache_t, cache_t.numel())):
        tm = Timer(torch, reps)
        for i in range(reps + 2):
            q.flush_write(flush)
            if i >= 2:
                tm.start(i - 2)
            q.read_probe(buf, mode, sink, tile_bytes=tile_bytes, nbytes=n)
            if i >= 2:
                tm.stop(i - 2)
        torch.cuda.synchronize()
        ms = float(np.median(tm.ms()))
        nb = n if mode == 0 else (n // tile_bytes) * tile_bytes
        res[name] = {"ms": ms, "gbs": nb / (ms * 1e6), "bytes": nb}
    del src
    return res


# ---------------------------------------------------------------------------- one layer
def run_layer(args, w, ctx, torch, q, dev):
    cb, hms, calib_s = calibrate(w, q, 1)
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device=dev)
    cb.upload(blob)
    cache_t = torch.zeros(cb.cache_bytes(1, 1, ctx), dtype=torch.uint8, device=dev)
    cache = q.make_cache(cache_t, 1, 1, ctx)
    kb = np.zeros((1, ctx, w.n_kv, w.d), np.uint16)
    vb = np.zeros_like(kb)
    for h, hm in enumerate(hms):
        K, V = synth.cache_kv(w, hm, 0, 0, h, ctx)
        kb[0, :, h] = synth.to_bf16_bits(K)
        vb[0, :, h] = synth.to_bf16_bits(V)
    qb = synth.to_bf16_bits(synth.decode_queries(w, hms, 0, 0))[None]
    K = torch.from_numpy(kb.view(np.int16)).to(dev)
    V = torch.from_numpy(vb.view(np.int16)).to(dev)
    Qd = torch.from_numpy(qb.view(np.int16)).to(dev)
    del kb, vb
    out = torch.empty((1, w.n_q, w.d), dtype=torch.float32, device=dev)
    ws = torch.zeros(cb.decode_workspace_bytes(1, ctx), dtype=torch.uint8, device=dev)
    ids = torch.zeros(1, dtype=torch.int32, device=dev)
    lens = torch.full((1,), ctx, dtype=torch.int64, device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def encode():
        q.encode(cb, blob, cache, 0, [0], [0], ctx, K, V)

    def decode():
        q.decode_attention(cb, blob, cache, 0, ids, lens, ctx, Qd, out, ws)

    for _ in range(args.warmup):
        q.flush_write(flush)
        encode()
        q.flush_write(flush)
        decode()
    torch.cuda.synchronize()
    te, td = Timer(torch, args.steps), Timer(torch, args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        q.flush_write(flush)
        te.start(i)
        encode()
        te.stop(i)
        q.flush_write(flush)
        td.start(i)
        decode()
        td.stop(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms, dec_ms = te.ms(), td.ms()
    # second pass, same steps: library events around the split-decode kernel alone
    q.profile_begin(args.steps)
    for i in range(args.steps):
        q.flush_write(flush)
        decode()
    torch.cuda.synchronize()
    kern_ms = q.profile_end(args.steps)

    tb = cb.tile_bytes
    cache_bytes = w.n_kv * ((ctx + 63) // 64) * tb
    vq = vq_keys(w)
    books = w.n_kv * (w.d * w.avg_bits // 8) * 256 * 4 * 4 if vq else 0  # VQ codebooks: side information
    side = 2 * w.n_kv * w.d * w.d * 4 + w.n_q * w.d * 2 + w.n_q * w.d * 4 + books
    dec_bytes = int(cache_bytes + side)
    # the split-decode kernel alone (the merge kernel that follows it reads U_V and writes
    # out): the packed cache, U_K (or T_K^-1), the VQ codebooks, the bf16 queries
    kern_bytes = int(cache_bytes + w.n_kv * w.d * w.d * 4 + w.n_q * w.d * 2 + books)
    probe = probe_rates(torch, q, dev, kern_bytes, tb, cache_t, flush, max(5, args.steps // 2)) if not vq else None
    if args.copy_probe_mb:
        a = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mb} MiB read + written")
    kern_s = float(kern_ms.mean()) / 1e3
    kern_gbs = kern_bytes / kern_s / 1e9
    enc_bytes = 2 * ctx * w.n_kv * w.d * 2 + cache_bytes
    dec_s = dec_ms.mean() / 1e3
    enc_s = enc_ms.mean() / 1e3
    dec_gbs = dec_bytes / dec_s / 1e9
    enc_gbs = enc_bytes / enc_s / 1e9
    enc_flops = 2 * 2 * ctx * w.n_kv * w.d * w.d  # K and V projections, algorithmic
    roof = {"kernel": ("vq_decode_kernel (split decode over vector-quantized keys)" if vq else
                       "decode_kernel (split decode: query transform, scores, online softmax, value sums)"),
            "bound": "hbm", "achieved": round(kern_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(*(VQ_DECODE_PMC if vq else DECODE_PMC)),
            "algorithmic_bytes": kern_bytes, "kernel_ms": round(kern_s * 1e3, 4),
            "source_sha256_16": source_hash(DECODE_PMC[1])}
    ks = os.path.join(PROFILES, "vq_path_kernels_llama128k_kstats.txt" if vq else "path_kernels_llama128k_kstats.txt")
    if w.name in ("llama_128k", "llama_vq_128k") and ctx == w.ctx:
        k_us = profiled_us(ks, "void vq_decode_kernel<" if vq else "void decode_kernel<")
        m_us = profiled_us(ks, "void merge_kernel<")
        if k_us:
            roof.update({"rocprof_summary": os.path.relpath(ks, ROOT), "rocprof_kernel_us": k_us,
                         "rocprof_merge_us": m_us, "rocprof_frac": round(kern_bytes / (k_us * 1e3) / HBM_PEAK_GBS, 4)})
    if probe:
        roof.update({"probe_gbs": round(probe["plain"]["gbs"], 2), "frac_of_probe": round(kern_gbs / probe["plain"]["gbs"], 4),
                     "probe_tile_stream_gbs": round(probe["tiles"]["gbs"], 2),
                     "probe": "library read probe (aatc_read_probe) by the same events, LLC flushed: mode 0 = plain "
                              "16-byte loads of the kernel's algorithmic bytes, mode 1 = this cache's tiles streamed "
                              "into LDS like the decode kernel"})
    return {
        "value": round(dec_gbs, 2),
        "steps": args.steps,
        "ms_per_step": round(float((enc_ms + dec_ms).mean()), 4),
        "config": {"workload": WORKLOAD_LABELS.get(w.name, w.name), "kv_heads": w.n_kv, "q_heads": w.n_q,
                   "head_dim": w.d, "ctx": ctx, "batch": 1, "layers": 1, "bits_per_element": w.avg_bits,
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
        "roofline": roof,
        "roofline_encode": {"kernel": "encode", "bound": "hbm", "achieved": round(enc_gbs, 2),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(enc_gbs / HBM_PEAK_GBS, 4),
                            "mfma_tflops": round(enc_flops / enc_s / 1e12, 2),
                            "mfma_frac": round(enc_flops / enc_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                            "traffic": None if vq else measured_traffic(*ENCODE_PMC),
                            "algorithmic_bytes": enc_bytes,
                            "source_sha256_16": source_hash(ENCODE_PMC[1])},
    }


# ------------------------------------------------------------------- several layers
def run_layers(args, w, torch, q, dev):
    """A decode step across every layer of the workload (one call per layer, captured in a
    HIP graph), over caches prefilled by aatc_encode from seeded device draws."""
    L, S, ctx = w.n_layers, w.n_seqs, w.ctx
    cb, hms, calib_s = calibrate(w, q, L)
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device=dev)
    cb.upload(blob)
    cache_t = torch.zeros(cb.cache_bytes(L, S, ctx), dtype=torch.uint8, device=dev)
    cache = q.make_cache(cache_t, L, S, ctx)
    t0 = time.perf_counter()
    enc_ms = []
    for layer in range(L):
        K = torch.empty((S, ctx, w.n_kv, w.d), dtype=torch.int16, device=dev)
        V = torch.empty_like(K)
        for s in range(S):
            for h in range(w.n_kv):
                k, v = synth.device_kv(torch, hms[layer * w.n_kv + h], ctx,
                                       synth.seed_of(w.cfg, layer, s, h, synth.ST_CACHE_KV), dev)
                K[s, :, h] = k
                V[s, :, h] = v
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        q.encode(cb, blob, cache, layer, list(range(S)), [0] * S, ctx, K, V)
        e1.record()
        torch.cuda.synchronize()
        enc_ms.append(e0.elapsed_time(e1))
        del K, V
    log(f"prefill of {L} layers x {S} sequences x {ctx} tokens ({time.perf_counter() - t0:.1f}s)")
    Qd = torch.stack([torch.stack([torch.cat([synth.device_queries(torch, hms[layer * w.n_kv + h], w.group,
                                                                   synth.seed_of(w.cfg, layer, s, h, synth.ST_DECODE_Q),
                                                                   dev)[0]
                                              for h in range(w.n_kv)]) for s in range(S)]) for layer in range(L)])
    out = torch.empty((L, S, w.n_q, w.d), dtype=torch.float32, device=dev)
    ws = torch.zeros(cb.decode_workspace_bytes(S, ctx), dtype=torch.uint8, device=dev)
    ids = torch.arange(S, dtype=torch.int32, device=dev)
    lens = torch.full((S,), ctx, dtype=torch.int64, device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def step():
        for layer in range(L):
            q.decode_attention(cb, blob, cache, layer, ids, lens, ctx, Qd[layer], out[layer], ws)

    side_stream = torch.cuda.Stream()
    side_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side_stream):
        step()
    torch.cuda.current_stream().wait_stream(side_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        q.flush_write(flush)
        g.replay()
    torch.cuda.synchronize()
    tg, te = Timer(torch, args.steps), Timer(torch, args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        q.flush_write(flush)
        tg.start(i)
        g.replay()
        tg.stop(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(args.steps):  # the same step launched eagerly
        q.flush_write(flush)
        te.start(i)
        step()
        te.stop(i)
    torch.cuda.synchronize()
    # the same layers' queries decoded by one batched-layers call (one launch per run of
    # layers that share a decode variant), for callers that hold every layer's queries
    wsl = torch.zeros(cb.decode_layers_workspace_bytes(0, L, S, ctx), dtype=torch.uint8, device=dev)
    outl = torch.empty_like(out)

    def step_layers():
        q.decode_attention_layers(cb, blob, cache, 0, L, ids, lens, ctx, Qd, outl, wsl)

    for _ in range(args.warmup):
        q.flush_write(flush)
        step_layers()
    tl = Timer(torch, args.steps)
    for i in range(args.steps):
        q.flush_write(flush)
        tl.start(i)
        step_layers()
        tl.stop(i)
    torch.cuda.synchronize()
    gms, ems, lms = tg.ms(), te.ms(), tl.ms()
    tb = cb.tile_bytes
    cache_bytes = L * S * w.n_kv * ((ctx + 63) // 64) * tb
    side = L * (2 * w.n_kv * w.d * w.d * 4 + S * (w.n_q * w.d * 2 + w.n_q * w.d * 4))
    dec_bytes = int(cache_bytes + side)
    gbs = dec_bytes / (gms.mean() / 1e3) / 1e9
    return {
        "value": round(gbs, 2),
        "steps": args.steps,
        "ms_per_step": round(float(gms.mean()), 4),
        "config": {"workload": WORKLOAD_LABELS.get(w.name, w.name), "kv_heads": w.n_kv, "q_heads": w.n_q,
                   "head_dim": w.d, "ctx": ctx, "batch": S, "layers": L, "bits_per_element": w.avg_bits,
                   "step": f"one decode step across {L} layers ({L} calls replayed as a HIP graph)"},
        "decode_ms": round(float(gms.mean()), 4),
        "decode_ms_p50": round(float(np.median(gms)), 4),
        "decode_ms_min": round(float(gms.min()), 4),
        "decode_ms_eager": round(float(ems.mean()), 4),
        "decode_ms_batched_layers": round(float(lms.mean()), 4),
        "decode_gbs_batched_layers": round(dec_bytes / (lms.mean() / 1e3) / 1e9, 2),
        "batched_layers": (f"the {L} layers' queries decoded by one aatc_decode_attention_layers call (a launch per "
                           "run of layers sharing a decode variant); a model's step runs its layers one after "
                           "another, which value and decode_ms measure"),
        "decode_bytes": dec_bytes,
        "decode_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "encode_ms_per_layer": round(float(np.mean(enc_ms)), 4),
        "encode_tokens_per_s": round(S * ctx / (np.mean(enc_ms) / 1e3), 1),
        "compression_ratio": round(16.0 / w.avg_bits, 4),
        "calibration_s": round(calib_s, 3),
        "wall_s_timed_region": round(wall, 3),
        "roofline": {"kernel": "decode_kernel per layer (one launch each)", "bound": "hbm",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": dec_bytes,
                     "kernel_ms": round(float(gms.mean()), 4), "source_sha256_16": source_hash(DECODE_PMC[1])},
    }


# ------------------------------------------------------------------- generation loop
def run_loop(args, w, torch, q, dev):
    """Prefill, then n generation steps: each appends one new K/V token per kv-head and
    decodes over the grown cache in one launch (aatc_decode_attention_append)."""
    l0, n = w.ctx, args.loop_steps
    cb, hms, calib_s = calibrate(w, q, 1)
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device=dev)
    cb.upload(blob)
    cap = l0 + n
    cache_t = torch.zeros(cb.cache_bytes(1, 1, cap), dtype=torch.uint8, device=dev)
    cache = q.make_cache(cache_t, 1, 1, cap)
    K = torch.empty((1, l0, w.n_kv, w.d), dtype=torch.int16, device=dev)
    V = torch.empty_like(K)
    for h in range(w.n_kv):
        k, v = synth.device_kv(torch, hms[h], l0, synth.seed_of(w.cfg, 0, 0, h, synth.ST_CACHE_KV), dev)
        K[0, :, h] = k
        V[0, :, h] = v
    q.encode(cb, blob, cache, 0, [0], [0], l0, K, V)
    del K, V
    # per-step draws: one K/V token per kv-head and the queries (stream 9 of the recipe)
    kn = torch.empty((n, 1, w.n_kv, w.d), dtype=torch.int16, device=dev)
    vn = torch.empty_like(kn)
    qn = torch.empty((n, 1, w.n_q, w.d), dtype=torch.int16, device=dev)
    for h in range(w.n_kv):
        k, v = synth.device_kv(torch, hms[h], n, synth.seed_of(w.cfg, 0, 0, h, synth.ST_STEP), dev)
        kn[:, 0, h] = k
        vn[:, 0, h] = v
        qn[:, 0, h * w.group:(h + 1) * w.group] = synth.device_queries(
            torch, hms[h], w.group, synth.seed_of(w.cfg, 0, 0, h, synth.ST_DECODE_Q), dev, n)
    lens_all = torch.arange(l0, l0 + n, dtype=torch.int64, device=dev)  # tokens cached before step i
    out = torch.empty((n, 1, w.n_q, w.d), dtype=torch.float32, device=dev)
    ws = torch.zeros(cb.decode_workspace_bytes(1, cap), dtype=torch.uint8, device=dev)
    ids = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    pristine = cache_t.clone()

    def step(i):
        q.decode_attention_append(cb, blob, cache, 0, ids, lens_all[i:i + 1], cap, kn[i], vn[i], qn[i], out[i], ws)

    # warm-up steps (first-call costs), then the cache back to its prefilled state
    for i in range(min(args.warmup, n)):
        q.flush_write(flush)
        step(i)
    cache_t.copy_(pristine)
    torch.cuda.synchronize()
    # (a) every step eagerly, the LLC flushed before each (as in a model whose other layers
    # evict this layer's cache between steps): per-step latency distribution
    tm = Timer(torch, n)
    for i in range(n):
        q.flush_write(flush)
        tm.start(i)
        step(i)
        tm.stop(i)
    torch.cuda.synchronize()
    ms = tm.ms()
    # (b) the whole loop back to back as one HIP graph (the single layer's cache stays in
    # the LLC between steps)
    cache_t.copy_(pristine)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step(i)
    cache_t.copy_(pristine)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_ms = e0.elapsed_time(e1)
    tb = cb.tile_bytes
    mean_len = l0 + (n + 1) / 2.0
    step_bytes = int(w.n_kv * mean_len / 64 * tb + 2 * w.n_kv * w.d * w.d * 4 + w.n_q * w.d * 6)
    gbs = step_bytes / (ms.mean() / 1e3) / 1e9
    return {
        "value": round(gbs, 2),
        "steps": n,
        "ms_per_step": round(float(ms.mean()), 4),
        "config": {"workload": WORKLOAD_LABELS.get(w.name, w.name), "kv_heads": w.n_kv, "q_heads": w.n_q,
                   "head_dim": w.d, "ctx": l0, "batch": 1, "layers": 1, "bits_per_element": w.avg_bits,
                   "step": "append one K/V token per kv-head + decode over the grown cache (one launch)"},
        "step_ms_mean": round(float(ms.mean()), 5),
        "step_ms_p50": round(float(np.percentile(ms, 50)), 5),
        "step_ms_p99": round(float(np.percentile(ms, 99)), 5),
        "step_ms_graph_back_to_back": round(graph_ms / n, 5),
        "loop_ms_graph": round(graph_ms, 3),
        "step_bytes_mean": step_bytes,
        "decode_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "compression_ratio": round(16.0 / w.avg_bits, 4),
        "calibration_s": round(calib_s, 3),
        "wall_s_timed_region": round(wall, 3),
        "roofline": {"kernel": "decode_kernel, append mode (one launch per step)", "bound": "hbm",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": step_bytes,
                     "kernel_ms": round(float(ms.mean()), 5), "source_sha256_16": source_hash(DECODE_PMC[1])},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--ctx", type=int, default=0, help="override context length (one-layer workloads)")
    ap.add_argument("--loop-steps", type=int, default=1024, help="generation steps of llama_loop")
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
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if w.name == "llama_loop":
        res = run_loop(args, w, torch, q, dev)
    elif w.n_layers > 1 or w.n_seqs > 1:
        res = run_layers(args, w, torch, q, dev)
    else:
        res = run_layer(args, w, args.ctx or w.ctx, torch, q, dev)
    line = {"metric": METRIC, "value": res.pop("value"), "unit": "GB/s", "n_gpus": 1, "steps": res.pop("steps"),
            "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": path_dtype(w), "data": "synthetic",
            "config": res.pop("config")}
    line.update(res)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
