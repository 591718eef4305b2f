"""Pins of the oracle's attention-optimal key transform (nova_key_transform) and of the
general key transform in the oracle's codec ("Spend Bits Where Queries Look", abstract: a
non-orthogonal transform from calibration statistics under which the attention-aware
distortion becomes the MSE of the transform coefficients).

The pins check what the transform must do, by sampling rather than by restating it:
- isotropic queries reduce it to the KLT (a scaled orthogonal transform);
- coefficient errors cost their squared norm under the query moment M_Q (the generalized
  Parseval relation), measured by Monte Carlo; the KLT does not have that property;
- the coefficients of the calibration keys are uncorrelated;
- at the same bit budget its codebook gives smaller attention errors than the KLT's.
"""
import numpy as np
import pytest

import oracle
import synth
from util import LAYOUT_KEY_ALIGN


def _tiny_stats(head=0):
    w = synth.WORKLOADS["tiny"]
    hm = synth.head_model(w, 0, head)
    K, V, Q = synth.calibration_samples(w, hm, 0, head)
    return w, hm, K, oracle.head_stats(K, V, Q)


def test_isotropic_queries_give_the_klt():
    w, hm, K, st = _tiny_stats()
    c = 3.7
    lam, U = oracle.klt(st["SigK"])
    mu, T, Tinv = oracle.nova_key_transform(st["SigK"], c * np.eye(w.d))
    s = np.sqrt(c * (1.0 + oracle.calib.NOVA_RIDGE))
    np.testing.assert_allclose(T / s, U, atol=1e-9)
    np.testing.assert_allclose(mu, s * s * lam, rtol=1e-9, atol=1e-12 * lam.max())
    np.testing.assert_allclose(T @ Tinv, np.eye(w.d), atol=1e-9)


def test_coefficient_errors_cost_their_squared_norm():
    """e = eps T^{-1} for independent coefficient errors eps of variances s^2: the
    attention-aware cost E[e M_Q e^T] equals sum s^2 (Monte Carlo, 4 standard errors);
    for the KLT the same errors cost sum s^2 (U^T M_Q U)_jj, which is not sum s^2."""
    w, hm, K, st = _tiny_stats()
    d = w.d
    rng = np.random.default_rng(11)
    s2 = rng.uniform(0.2, 2.0, d) ** 2
    n = 40000
    eps = rng.standard_normal((n, d)) * np.sqrt(s2)[None, :]
    _, T, Tinv = oracle.nova_key_transform(st["SigK"], st["MQ"])
    e = eps @ Tinv
    cost = np.einsum("ni,ij,nj->n", e, st["MQ"], e)
    se = cost.std() / np.sqrt(n)
    ridge = oracle.calib.NOVA_RIDGE * np.trace(st["MQ"]) / d  # the ridge shifts the identity a little
    assert abs(cost.mean() - s2.sum()) < 4 * se + ridge * s2.sum() * 10
    _, U = oracle.klt(st["SigK"])
    eu = eps @ U.T
    cost_u = np.einsum("ni,ij,nj->n", eu, st["MQ"], eu).mean()
    assert abs(cost_u - s2.sum()) > 10 * se


def test_coefficients_are_uncorrelated():
    w, hm, K, st = _tiny_stats()
    mu, T, Tinv = oracle.nova_key_transform(st["SigK"], st["MQ"])
    C = (np.asarray(K, np.float64) - st["muK"][None, :]) @ T
    cov = C.T @ C / C.shape[0]
    off = cov - np.diag(np.diag(cov))
    assert np.abs(off).max() < 1e-9 * np.abs(np.diag(cov)).max()
    np.testing.assert_allclose(np.diag(cov), mu, rtol=1e-9, atol=1e-12 * mu.max())
    assert np.all(np.diff(mu) <= 0)


def test_general_key_transform_reconstruction():
    """decode_attention over a packed cache = attention over keys rebuilt as
    mu + c_hat T^{-1}, with T^{-1} from a general matrix inverse."""
    w, hm, K, st = _tiny_stats()
    cb = oracle.build_head_codebook(st, w.avg_bits, key_transform="nova", key_align=LAYOUT_KEY_ALIGN)
    L = 200
    Kc, Vc = synth.cache_kv(w, hm, 0, 0, 0, L)
    kf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Kc))
    vf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Vc))
    cache, cK, cV = oracle.encode_cache(kf, vf, cb)
    q = synth.bf16_bits_to_f64(synth.to_bf16_bits(synth.decode_queries(w, [hm], 0, 0)))[:w.group]
    Kh = cb.muK[None, :] + oracle.dequantize(cK, cb.bK, cb.stepK) @ np.linalg.inv(cb.UK)
    Vh = cb.muV[None, :] + oracle.dequantize(cV, cb.bV, cb.stepV) @ cb.UV.T
    np.testing.assert_allclose(oracle.decode_attention(cache, cb, q, L), oracle.attention(q, Kh, Vh), rtol=1e-9,
                               atol=1e-12)


@pytest.mark.parametrize("head", [0])
def test_smaller_attention_error_than_the_klt(head):
    """The method's claim on the tiny workload: at the same bits per token, keys coded in
    the attention-optimal basis give a smaller mean squared attention error over fresh
    decode queries than keys coded in the KLT basis (measured: about 25 % smaller)."""
    w, hm, K, st = _tiny_stats(head)
    L = 512
    Kc, Vc = synth.cache_kv(w, hm, 0, 0, head, L)
    kf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Kc))
    vf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Vc))
    qs = np.concatenate([synth.bf16_bits_to_f64(synth.to_bf16_bits(synth.decode_queries(w, [hm], 0, 0, step=s)))
                         [:w.group] for s in range(64)])
    exact = oracle.attention(qs, kf, vf)
    err = {}
    for kt in ("klt", "nova"):
        cb = oracle.build_head_codebook(st, w.avg_bits, key_transform=kt, key_align=LAYOUT_KEY_ALIGN)
        cache, _, _ = oracle.encode_cache(kf, vf, cb)
        err[kt] = ((oracle.decode_attention(cache, cb, qs, L) - exact) ** 2).sum(1).mean()
    assert err["nova"] < 0.9 * err["klt"], err
