"""Oracle attention over a transform-coded cache, and the distortion theorem's terms.
Test infrastructure only.
"""
from __future__ import annotations

import math

import numpy as np

from .codec import dequantize, key_record_bits, reconstruct, unpack_cache
from .vq import vq_dequantize


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """o = softmax(q K^T / sqrt(d)) V in float64 (p2 "Formal Attention Distortion Model").
    q may be [d] or [m, d]."""
    q = np.atleast_2d(np.asarray(q, np.float64))
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = q @ K.T / math.sqrt(K.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ V


def decoded_kv(cache: np.ndarray, cb, n_tokens: int):
    """The keys and values a packed cache stands for, first n_tokens tokens: unpack,
    dequantize, inverse transform.  -> (K_hat, V_hat) [n_tokens, d] float64."""
    cK, cV = unpack_cache(cache, key_record_bits(cb), cb.bV, n_tokens)
    if cb.vq is not None:
        chatK = vq_dequantize(cK, cb.vq.groups, cb.vq.scale32, cb.vq.cent32, cb.d)
    else:
        chatK = dequantize(cK, cb.bK, cb.stepK)
    Khat = cb.muK[None, :] + chatK @ cb.UKinv  # c = (k - mu) T  =>  k = mu + c T^{-1}
    Vhat = reconstruct(dequantize(cV, cb.bV, cb.stepV), cb.muV, cb.UV)
    return Khat, Vhat


def decode_attention(cache: np.ndarray, cb, q_heads: np.ndarray, n_tokens: int) -> np.ndarray:
    """Attention of the query heads of one kv-head group over the first n_tokens of a
    packed cache: the decoded keys and values, then plain attention (every cached token
    is attended; no mask).  q_heads [G, d] -> out [G, d] float64."""
    Khat, Vhat = decoded_kv(cache, cb, n_tokens)
    return attention(q_heads, Khat, Vhat)


def predicted_distortion(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                         sigK2: np.ndarray, sigV2: np.ndarray):
    """(D_K, D_V) of p2 "Theorem: Additive Error Decomposition" for white errors of
    per-(token, channel) variances sigK2, sigV2 [L, d]:
    D_V = sum_i A_i^2 sum_j sigV2_ij,
    D_K = (1/d) sum_j q_j^2 sum_i A_i^2 ||v_i - o||^2 sigK2_ij."""
    q = np.asarray(q, np.float64)
    d = q.size
    s = K @ q / math.sqrt(d)
    s -= s.max()
    A = np.exp(s)
    A /= A.sum()
    o = A @ V
    resid = ((V - o[None, :]) ** 2).sum(axis=1)
    DV = float((A ** 2 * sigV2.sum(axis=1)).sum())
    DK = float(((A ** 2 * resid)[:, None] * sigK2 * (q ** 2)[None, :]).sum() / d)
    return DK, DV


def monte_carlo_distortion(q: np.ndarray, K: np.ndarray, V: np.ndarray, sigK: np.ndarray,
                           sigV: np.ndarray, trials: int, rng: np.random.Generator):
    """Empirical E||o - o_hat||^2 with independent zero-mean Gaussian errors of std
    sigK / sigV [L, d] added to keys only, values only, and both (common random
    numbers).  Returns dict of means and standard errors."""
    o = attention(q, K, V)[0]
    res = {"K": [], "V": [], "KV": []}
    for _ in range(trials):
        EK = rng.standard_normal(K.shape) * sigK
        EV = rng.standard_normal(V.shape) * sigV
        oK = attention(q, K + EK, V)[0]
        oV = attention(q, K, V + EV)[0]
        oKV = attention(q, K + EK, V + EV)[0]
        res["K"].append(((oK - o) ** 2).sum())
        res["V"].append(((oV - o) ** 2).sum())
        res["KV"].append(((oKV - o) ** 2).sum())
    out = {}
    for k, v in res.items():
        v = np.asarray(v)
        out[k] = (float(v.mean()), float(v.std(ddof=1) / math.sqrt(v.size)))
    cross = np.asarray(res["KV"]) - np.asarray(res["K"]) - np.asarray(res["V"])
    out["cross"] = (float(cross.mean()), float(cross.std(ddof=1) / math.sqrt(cross.size)))
    return out
