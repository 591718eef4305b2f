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
