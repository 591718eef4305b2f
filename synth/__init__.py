"""Seeded synthetic K/V/Q generators shared by the oracle, the tests and the bench.

This module only draws random numbers.  It holds none of the transform-coding
arithmetic (no statistics, no transform, no allocation, no quantizer, no
layout), so that the oracle and the HIP path can both take their inputs from
it without sharing any of the method.

The workloads stand in for the evaluation data of the AATC pages (Llama-3.1-8B
and Qwen-2.5-7B attention caches at 32k-128k context; "KV Cache Compression
Through the Lens of Transform Coding", abstract, and the blog's benchmark
section).  Neither those models nor their datasets are used: every tensor here
is a seeded Gaussian draw with the models' attention geometry.

Seeding: every draw comes from
``numpy.random.default_rng(SeedSequence([S0, cfg, layer, seq, head, stream]))``
so that any slice of a workload can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

S0 = 20260817

# stream ids
ST_K_BASIS = 0
ST_V_BASIS = 1
ST_EXPONENT = 2
ST_KEY_MEAN = 3
ST_OUTLIERS = 4
ST_CALIB_KV = 5
ST_CACHE_KV = 6
ST_CALIB_Q = 7
ST_DECODE_Q = 8
ST_STEP = 9
ST_VQ_TRAIN = 10  # standard normal training draws of the key codebooks
ST_Q_BASIS = 16  # + query head index


def rng_for(cfg: int, layer: int, seq: int, head: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([S0, cfg, layer, seq, head, stream]))


def haar_orthogonal(d: int, rng: np.random.Generator) -> np.ndarray:
    """Haar-distributed orthogonal matrix (QR of a Gaussian, signs fixed by diag(R))."""
    z = rng.standard_normal((d, d))
    q, r = np.linalg.qr(z)
    return q * np.sign(np.diag(r))[None, :]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bfloat16 (round to nearest even); returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    u = (np.asarray(b, dtype=np.uint32) << 16).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


@dataclass
class HeadModel:
    """Generative model of one (layer, kv-head): Gaussian K and V with given basis/spectrum."""
    d: int
    UK: np.ndarray
    lamK: np.ndarray
    muK: np.ndarray
    UV: np.ndarray
    lamV: np.ndarray
    muV: np.ndarray
    outK: np.ndarray  # native channels scaled x10 (may be empty)
    outV: np.ndarray
    # query heads of the group: basis and spectrum (already scaled to logit std 2)
    UQ: List[np.ndarray] = field(default_factory=list)
    lamQ: List[np.ndarray] = field(default_factory=list)


@dataclass
class Workload:
    name: str
    cfg: int
    d: int
    n_kv: int
    n_q: int
    n_layers: int
    n_seqs: int
    ctx: int
    avg_bits: float
    n_calib: int
    n_calib_q: int  # calibration queries per query head
    dtype: str  # 'fp32' or 'bf16'

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


WORKLOADS: Dict[str, Workload] = {
    # 1 layer, 1 KV head, 4 query heads, head_dim 64, 512 cached tokens, 3.0 bits/element
    "tiny": Workload("tiny", 1, 64, 1, 4, 1, 1, 512, 3.0, 2048, 256, "fp32"),
    # Llama-3.1-8B-shaped layer, 32k context, 2.75 bits/element
    "llama_32k": Workload("llama_32k", 2, 128, 8, 32, 1, 1, 32768, 2.75, 8192, 256, "bf16"),
    # the same layer at 128k context
    "llama_128k": Workload("llama_128k", 2, 128, 8, 32, 1, 1, 131072, 2.75, 8192, 256, "bf16"),
    # Qwen-2.5-7B-shaped, 28 layers, 128k context
    "qwen_128k": Workload("qwen_128k", 3, 128, 4, 28, 28, 1, 131072, 2.75, 8192, 256, "bf16"),
    # Llama geometry, 32 layers x 32 sequences x 8k tokens
    "llama_batch": Workload("llama_batch", 4, 128, 8, 32, 32, 32, 8192, 2.75, 8192, 256, "bf16"),
    # Llama geometry, one layer, 64k cached tokens, append loop at 2.0 bits/element
    "llama_loop": Workload("llama_loop", 5, 128, 8, 32, 1, 1, 65536, 2.0, 8192, 256, "bf16"),
    # limits of the decode path (the Llama recipe, own seeds): the largest query group
    # (16 heads per kv-head) at d = 64 and 3.0 bits/element, and at d = 128 and 6.0
    "edge_g16": Workload("edge_g16", 6, 64, 2, 32, 1, 1, 1024, 3.0, 2048, 64, "bf16"),
    "edge_rate": Workload("edge_rate", 7, 128, 1, 16, 1, 1, 1024, 6.0, 4096, 32, "bf16"),
    # the largest rate: 8 bits on every channel (d = 64, 8 KiB tiles)
    "edge_max": Workload("edge_max", 13, 64, 1, 4, 1, 1, 512, 8.0, 2048, 32, "bf16"),
    # vector-quantized keys at 2.0 bits/element (one byte per group of 4 coefficients):
    # a small head, and the Llama layer at 128k context
    "vq_tiny": Workload("vq_tiny", 8, 64, 1, 4, 1, 1, 512, 2.0, 2048, 256, "bf16"),
    # ... at 1.0 bit/element: 8 groups code the 32 coefficients of largest weight
    "vq_low": Workload("vq_low", 10, 64, 1, 4, 1, 1, 512, 1.0, 2048, 256, "bf16"),
    "llama_vq_128k": Workload("llama_vq_128k", 9, 128, 8, 32, 1, 1, 131072, 2.0, 8192, 256, "bf16"),
    # vector-quantized keys with 7 query heads per kv-head (the Qwen group, d = 128) and
    # with 2 (d = 64): group sizes the other vector-quantized workloads do not reach
    "vq_g7": Workload("vq_g7", 11, 128, 2, 14, 1, 1, 4096, 2.0, 4096, 64, "bf16"),
    "vq_g2": Workload("vq_g2", 12, 64, 2, 4, 1, 1, 4096, 2.0, 2048, 64, "bf16"),
}


def _query_spectrum(w: Workload) -> np.ndarray:
    j = np.arange(w.d, dtype=np.float64)
    if w.cfg == 1:
        return 2.0 ** (-j / 16.0)
    return 1.0 / (j + 1.0)


def head_model(w: Workload, layer: int, head: int) -> HeadModel:
    """Per-(layer, kv-head) generative model for workload ``w``."""
    d = w.d
    cfg = 2 if w.cfg in (2, 4, 5) else w.cfg  # configs 4 and 5 reuse the 32k-layer distribution
    UK = haar_orthogonal(d, rng_for(cfg, layer, 0, head, ST_K_BASIS))
    UV = haar_orthogonal(d, rng_for(cfg, layer, 0, head, ST_V_BASIS))
    j = np.arange(d, dtype=np.float64)
    outK = np.zeros(0, dtype=np.int64)
    outV = np.zeros(0, dtype=np.int64)
    if w.cfg == 1:
        lamK = 2.0 ** (-j / 8.0)
        lamV = lamK.copy()
        muK = np.zeros(d)
        ro = rng_for(cfg, layer, 0, head, ST_OUTLIERS)
        outK = np.sort(ro.choice(d, 2, replace=False))
        outV = np.sort(ro.choice(d, 2, replace=False))
    else:
        if w.cfg == 3:
            a = rng_for(cfg, layer, 0, 0, ST_EXPONENT).uniform(1.0, 2.0)
        else:
            a = 1.5
        lamK = (j + 1.0) ** (-a)
        lamV = lamK.copy()
        muK = rng_for(cfg, layer, 0, head, ST_KEY_MEAN).standard_normal(d)
    muV = np.zeros(d)
    hm = HeadModel(d, UK, lamK, muK, UV, lamV, muV, outK, outV)
    # queries of the G heads in this group: own basis, decaying spectrum, scaled to logit std 2
    lq = _query_spectrum(w)
    SigK = (UK * lamK[None, :]) @ UK.T
    if outK.size:
        s = np.ones(d)
        s[outK] = 10.0
        SigK = SigK * s[:, None] * s[None, :]
    for g in range(w.group):
        qh = head * w.group + g
        UQ = haar_orthogonal(d, rng_for(cfg, layer, 0, ST_Q_BASIS + qh, ST_Q_BASIS))
        SigQ = (UQ * lq[None, :]) @ UQ.T
        scale2 = 4.0 * d / float(np.trace(SigQ @ SigK))
        hm.UQ.append(UQ)
        hm.lamQ.append(lq * scale2)
    return hm


def _draw(U: np.ndarray, lam: np.ndarray, mu: np.ndarray, out: np.ndarray, n: int,
          rng: np.random.Generator) -> np.ndarray:
    z = rng.standard_normal((n, U.shape[0]))
    x = (z * np.sqrt(lam)[None, :]) @ U.T + mu[None, :]
    if out.size:
        x[:, out] *= 10.0
    return x


def draw_kv(hm: HeadModel, n: int, rng: np.random.Generator):
    """n K and V vectors (float64) from the head model."""
    K = _draw(hm.UK, hm.lamK, hm.muK, hm.outK, n, rng)
    V = _draw(hm.UV, hm.lamV, hm.muV, hm.outV, n, rng)
    return K, V


def draw_q(hm: HeadModel, g: int, n: int, rng: np.random.Generator) -> np.ndarray:
    """n queries (float64) for query head g of the group."""
    return _draw(hm.UQ[g], hm.lamQ[g], np.zeros(hm.d), np.zeros(0, dtype=np.int64), n, rng)


def vq_normals(w: Workload, layer: int, n: int) -> np.ndarray:
    """[n, 4] standard normal draws that train the key codebooks of one layer."""
    return rng_for(w.cfg, layer, 0, 0, ST_VQ_TRAIN).standard_normal((n, 4))


def calibration_samples(w: Workload, hm: HeadModel, layer: int, head: int):
    """Calibration K, V [n_calib x d] and pooled queries [G*n_calib_q x d], float64."""
    K, V = draw_kv(hm, w.n_calib, rng_for(w.cfg, layer, 0, head, ST_CALIB_KV))
    rq = rng_for(w.cfg, layer, 0, head, ST_CALIB_Q)
    Q = np.concatenate([draw_q(hm, g, w.n_calib_q, rq) for g in range(w.group)], axis=0)
    return K, V, Q


def cache_kv(w: Workload, hm: HeadModel, layer: int, seq: int, head: int, n: int,
             start: int = 0):
    """Cached K/V for tokens [start, start+n) of one (layer, seq, head), float64 before rounding.

    Tokens are drawn in fixed blocks of 4096 so that any token range can be
    regenerated without drawing the whole context.
    """
    blk = 4096
    out_k, out_v = [], []
    b0, b1 = start // blk, (start + n + blk - 1) // blk
    for b in range(b0, b1):
        r = np.random.default_rng(np.random.SeedSequence([S0, w.cfg, layer, seq, head, ST_CACHE_KV, b]))
        K, V = draw_kv(hm, blk, r)
        out_k.append(K)
        out_v.append(V)
    K = np.concatenate(out_k)[start - b0 * blk:start - b0 * blk + n]
    V = np.concatenate(out_v)[start - b0 * blk:start - b0 * blk + n]
    return K, V


def decode_queries(w: Workload, hms: List[HeadModel], layer: int, seq: int, step: int = 0) -> np.ndarray:
    """One decode step's queries for all query heads: [H_q x d] float64."""
    qs = []
    for h, hm in enumerate(hms):
        r = np.random.default_rng(np.random.SeedSequence([S0, w.cfg, layer, seq, h, ST_DECODE_Q, step]))
        for g in range(w.group):
            qs.append(draw_q(hm, g, 1, r)[0])
    return np.stack(qs)


def as_cache_dtype(w: Workload, x: np.ndarray):
    """Values as stored at the cache boundary: (bf16 bits, float64 values of those bits)."""
    bits = to_bf16_bits(x)
    return bits, bf16_bits_to_f64(bits)


# ------------------------------------------------------------------ device-side draws
# Large workloads are drawn on the GPU with torch's device generator: the same recipe
# as draw_kv / draw_q (x = mu + U diag(sqrt(lambda)) z, outlier channels x10), another
# random stream.  Seeds come from seed_of, so any (layer, seq, head, stream) slice can be
# drawn again on its own.

def seed_of(*parts) -> int:
    """63-bit torch generator seed for the slice named by parts (cfg, layer, seq, head, stream, ...)."""
    return int(np.random.SeedSequence([S0, *parts]).generate_state(1, np.uint64)[0] >> 1)


def device_kv(torch, hm: HeadModel, n: int, seed: int, dev):
    """n seeded K and V rows of one (layer, kv-head) on device dev: bf16 bit patterns as
    int16 tensors [n, d] (the z draws are fp32; the product rounds once to bf16)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    out = []
    for U, lam, mu, ch in ((hm.UK, hm.lamK, hm.muK, hm.outK), (hm.UV, hm.lamV, hm.muV, hm.outV)):
        z = torch.randn((n, hm.d), generator=gen, device=dev, dtype=torch.float32)
        A = torch.from_numpy((U * np.sqrt(lam)[None, :]).T.astype(np.float32)).to(dev)
        x = z @ A + torch.from_numpy(mu.astype(np.float32)).to(dev)
        if ch.size:
            x[:, torch.from_numpy(ch).to(dev)] *= 10.0
        out.append(x.to(torch.bfloat16).view(torch.int16))
    return out


def device_queries(torch, hm: HeadModel, group: int, seed: int, dev, n: int = 1):
    """n decode steps' queries of the group's query heads on device dev: bf16 bit patterns
    as int16 [n, group, d]."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    qs = []
    for g in range(group):
        z = torch.randn((n, hm.d), generator=gen, device=dev, dtype=torch.float32)
        A = torch.from_numpy((hm.UQ[g] * np.sqrt(hm.lamQ[g])[None, :]).T.astype(np.float32)).to(dev)
        qs.append(z @ A)
    return torch.stack(qs, dim=1).to(torch.bfloat16).view(torch.int16)
