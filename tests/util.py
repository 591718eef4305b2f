"""Test helpers: oracle-built cases for the GPU parity tests."""
from __future__ import annotations

import numpy as np

import oracle
import synth

# The library's packed layout keeps a token's key record in whole 32-bit words, so every
# codebook the GPU path is fed is calibrated with that storage constraint named.
LAYOUT_KEY_ALIGN = 32


class Case:
    """Oracle codebooks and synthetic K/V/Q for n_kv heads of one layer of workload w."""

    def __init__(self, wname: str, ctx: int, n_seqs: int = 1, n_kv: int | None = None, layer: int = 0,
                 n_calib_q: int | None = None, lens=None, step: int = 0, key_transform: str = "klt",
                 key_quantizer: str = "scalar", vq_train: int = 1024, vq_iters: int = 8):
        w = synth.WORKLOADS[wname]
        self.w = w
        self.d = w.d
        self.n_kv = n_kv or w.n_kv
        self.group = w.group
        self.n_q = self.n_kv * self.group
        self.layer = layer
        self.ctx = ctx
        self.n_seqs = n_seqs
        self.lens = list(lens) if lens is not None else [ctx] * n_seqs
        self.hms = [synth.head_model(w, layer, h) for h in range(self.n_kv)]
        self.cbs = []
        for h, hm in enumerate(self.hms):
            K, V, Q = synth.calibration_samples(w, hm, layer, h)
            if n_calib_q is not None:
                Q = Q.reshape(w.group, -1, w.d)[:, :n_calib_q].reshape(-1, w.d)
            if key_quantizer == "vq":
                self.cbs.append(oracle.build_head_codebook(
                    oracle.head_stats(K, V, Q), w.avg_bits, joint=False, key_transform=key_transform,
                    key_quantizer="vq", vq_normals=synth.vq_normals(w, layer, vq_train), vq_iters=vq_iters))
            else:
                self.cbs.append(oracle.build_head_codebook(oracle.head_stats(K, V, Q), w.avg_bits,
                                                           key_transform=key_transform,
                                                           key_align=LAYOUT_KEY_ALIGN))
        # cached K/V: bf16 bits [n_seqs, ctx, n_kv, d] and their float64 values
        self.k_bits = np.zeros((n_seqs, ctx, self.n_kv, w.d), np.uint16)
        self.v_bits = np.zeros_like(self.k_bits)
        for s in range(n_seqs):
            for h, hm in enumerate(self.hms):
                K, V = synth.cache_kv(w, hm, layer, s, h, ctx)
                self.k_bits[s, :, h] = synth.to_bf16_bits(K)
                self.v_bits[s, :, h] = synth.to_bf16_bits(V)
        self.q = np.stack([synth.decode_queries(w, self.hms, layer, s, step) for s in range(n_seqs)])
        self.q_bits = synth.to_bf16_bits(self.q)

    # values as float64
    def kf(self, s, h):
        return synth.bf16_bits_to_f64(self.k_bits[s, :, h])

    def vf(self, s, h):
        return synth.bf16_bits_to_f64(self.v_bits[s, :, h])

    def qf(self):
        return synth.bf16_bits_to_f64(self.q_bits)

    @property
    def tile_bytes(self):
        return oracle.tile_bytes(oracle.key_record_bits(self.cbs[0]), self.cbs[0].bV)

    def n_tiles(self, max_tokens=None):
        return ((max_tokens or self.ctx) + 63) // 64

    def oracle_cache(self, max_tokens=None):
        """Whole-layer packed cache [n_seqs, n_kv, n_tiles * tile_bytes] from the oracle."""
        nt = self.n_tiles(max_tokens)
        out = np.zeros((self.n_seqs, self.n_kv, nt * self.tile_bytes), np.uint8)
        codes = {}
        for s in range(self.n_seqs):
            for h in range(self.n_kv):
                b, cK, cV = oracle.encode_cache(self.kf(s, h), self.vf(s, h), self.cbs[h], nt)
                out[s, h] = b
                codes[(s, h)] = (cK, cV)
        return out, codes

    def oracle_decode(self, cache_bytes, lens=None):
        lens = lens or self.lens
        out = np.zeros((self.n_seqs, self.n_q, self.d))
        qf = self.qf()
        for s in range(self.n_seqs):
            for h in range(self.n_kv):
                g0 = h * self.group
                out[s, g0:g0 + self.group] = oracle.decode_attention(cache_bytes[s, h], self.cbs[h],
                                                                     qf[s, g0:g0 + self.group], lens[s])
        return out

    def codebook_arrays(self):
        cbs = self.cbs
        out = dict(UK=np.stack([c.UK for c in cbs]), UV=np.stack([c.UV for c in cbs]),
                   muK=np.stack([c.muK for c in cbs]), muV=np.stack([c.muV for c in cbs]),
                   bK=np.stack([c.bK for c in cbs]), bV=np.stack([c.bV for c in cbs]),
                   stepK=np.stack([c.stepK for c in cbs]), stepV=np.stack([c.stepV for c in cbs]))
        if cbs[0].vq is not None:  # vector-quantized keys
            out["vq"] = dict(groups=np.stack([c.vq.groups for c in cbs]),
                             scale32=np.stack([c.vq.scale32 for c in cbs]),
                             cent32=np.stack([c.vq.cent32 for c in cbs]))
        return out

    def coeffs(self, s):
        """Oracle fp32 KLT coefficients [ctx, n_kv, 2, d] of sequence s."""
        out = np.zeros((self.ctx, self.n_kv, 2, self.d), np.float32)
        for h, cb in enumerate(self.cbs):
            out[:, h, 0] = oracle.transform_coeffs(self.kf(s, h), cb.muK, cb.UK)
            out[:, h, 1] = oracle.transform_coeffs(self.vf(s, h), cb.muV, cb.UV)
        return out


def normwise_rel_err(o, ref):
    """max over (seq, head) of max_j |o - ref| / max_j |ref|."""
    o = np.asarray(o, np.float64).reshape(-1, o.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    return float((np.abs(o - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())


# ------------------------------------------------------------ end-to-end code flips
# The GPU encoder computes u = t + 2^(b-1) - 1/2 in fp32 from bf16 x: the bases scaled by the
# fp32 reciprocal step, W = fp32(U / step), held as two bf16 parts (hi + lo, which leaves
# |W - hi - lo| <= 2^-18 |W|), three (above 6.5 bits/element) or in fp32, and the
# accumulators starting at
# 2^(b-1) - 1/2 - mu W.  Its t then differs from the exact t = c * inv32 by at most
#     E = (2^-17 + (d + 4) 2^-24) S inv32 + (d + 4) 2^-24 (2^(b-1) + 1) + 4 2^-24 |t|,
#     S = sum_i (|x_i| + |mu_i|) |U_ij|
# (split and scaling roundings of W, fp32 accumulation over d terms and the start value,
# with margin), and the oracle's fp32 t (c rounded once, then the product) by at most
# 2 2^-24 |t|.  Codes are floor(t) + 2^(b-1) (the GPU rounds u to nearest, which is the same
# away from integers t), so the two codes can differ only where the exact t lies within E
# of an integer: every flipped code is checked for that.
_U24 = 2.0 ** -24


def edge_ratio(x64, mu, U, inv32, bits, idx):
    """max over (token, channel) pairs idx [n, 2] of (distance of the exact t from the
    nearest integer) / E; a flip outside the rounding window gives a ratio above 1."""
    if len(idx) == 0:
        return 0.0
    rows, ch = idx[:, 0], idx[:, 1]
    X = np.asarray(x64, np.float64)[rows] - mu[None, :]
    Uc = np.asarray(U, np.float64)[:, ch].T  # [n, d]
    inv = inv32[ch].astype(np.float64)
    t = (X * Uc).sum(axis=1) * inv
    S = ((np.abs(np.asarray(x64, np.float64)[rows]) + np.abs(mu)[None, :]) * np.abs(Uc)).sum(axis=1)
    d = Uc.shape[1]
    half = 2.0 ** (np.asarray(bits)[ch] - 1)
    bound = (2.0 ** -17 + (d + 4) * _U24) * S * inv + (d + 4) * _U24 * (half + 1) + 4 * _U24 * np.abs(t)
    return float((np.abs(t - np.round(t)) / bound).max())


def code_flips(got_bytes, cb, n_tokens, K64, V64, first=0):
    """Codes of the GPU's packed bytes for tokens [first, n_tokens) against the oracle's
    codes of the same bf16 rows (K64, V64 hold exactly those rows).  Scalar-coded
    channels only (vector-quantized keys are compared by their own near-tie test).
    Returns (flips, coded pairs, worst level difference, worst edge ratio)."""
    gK, gV = oracle.unpack_cache(got_bytes, oracle.key_record_bits(cb), cb.bV, n_tokens)
    flips = total = worst = 0
    edge = 0.0
    for which, g, x64, U, mu, bits in (("K", gK, K64, cb.UK, cb.muK, cb.bK), ("V", gV, V64, cb.UV, cb.muV, cb.bV)):
        if which == "K" and cb.vq is not None:
            continue
        g = g[first:]
        r = oracle.quantize(oracle.transform_coeffs(x64, mu, U), cb.inv_step(which), bits)
        m = np.broadcast_to(bits > 0, g.shape)
        dlt = np.abs(g.astype(np.int64) - r.astype(np.int64))
        bad = (dlt > 0) & m
        flips += int(bad.sum())
        total += int(m.sum())
        worst = max(worst, int(dlt[m].max(initial=0)))
        edge = max(edge, edge_ratio(x64, mu, U, cb.inv_step(which), bits, np.argwhere(bad)))
    return flips, total, worst, edge


def library_head_codebook(cb, i: int):
    """The library's calibrated codebook of head i (layer-major) as an oracle codebook, so
    that the oracle decodes the bytes the library's parameters produced."""
    h = cb.head(i)
    return oracle.HeadCodebook(d=cb.d, UK=h["UK"], UV=h["UV"], lamK=h["lamK"], lamV=h["lamV"], muK=h["muK"],
                               muV=h["muV"], xK=h["xK"], xV=h["xV"], bK=h["bK"], bV=h["bV"], stepK=h["stepK"],
                               stepV=h["stepV"], theta=h["theta"])
