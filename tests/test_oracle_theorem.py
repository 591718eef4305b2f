"""Monte Carlo check of the additive distortion decomposition (p2 "Theorem: Additive
Error Decomposition"; p1 abstract): under white zero-mean errors the expected
attention distortion is D_K + D_V, with no key/value cross term at second order."""
import numpy as np
import pytest

import oracle
import synth


def _setup(L=48):
    w = synth.WORKLOADS["tiny"]
    hm = synth.head_model(w, 0, 0)
    K, V = synth.cache_kv(w, hm, 0, 0, 0, L)
    q = synth.decode_queries(w, [hm], 0, 0)[0]
    return q, K, V


def test_value_term_is_exact():
    q, K, V = _setup()
    sig = 0.05 * np.ones_like(V)
    DK, DV = oracle.predicted_distortion(q, K, V, np.zeros_like(K), sig ** 2)
    mc = oracle.monte_carlo_distortion(q, K, V, np.zeros_like(K), sig, 4000, np.random.default_rng(0))
    m, se = mc["V"]
    assert abs(m - DV) < 4 * se
    assert mc["K"][0] == 0.0


@pytest.mark.parametrize("eps", [1e-2, 3e-3])
def test_key_term_and_additivity(eps):
    q, K, V = _setup()
    sK = eps * K.std(0)[None, :] * np.ones_like(K)
    sV = eps * V.std(0)[None, :] * np.ones_like(V)
    DK, DV = oracle.predicted_distortion(q, K, V, sK ** 2, sV ** 2)
    mc = oracle.monte_carlo_distortion(q, K, V, sK, sV, 6000, np.random.default_rng(1))
    mK, seK = mc["K"]
    assert abs(mK - DK) < 4 * seK + 0.05 * DK
    m, se = mc["KV"]
    assert abs(m - (DK + DV)) < 4 * se + 0.05 * DK
    c, sec = mc["cross"]
    assert abs(c) < 4 * sec + 1e-3 * (DK + DV)


def test_key_term_error_shrinks_with_noise():
    """The relative gap between the first-order D_K and Monte Carlo shrinks as eps -> 0."""
    q, K, V = _setup()
    gaps = []
    for eps in (3e-1, 3e-2):
        sK = eps * K.std(0)[None, :] * np.ones_like(K)
        DK, _ = oracle.predicted_distortion(q, K, V, sK ** 2, np.zeros_like(V))
        mc = oracle.monte_carlo_distortion(q, K, V, sK, np.zeros_like(V), 3000, np.random.default_rng(2))
        gaps.append(abs(mc["K"][0] / DK - 1))
    assert gaps[1] < gaps[0]


def test_theorem_in_klt_domain_with_quantizer_noise():
    """Uniform quantization-like noise of variance step^2/12 in the KLT domain, mapped
    back to native channels, is predicted by the KLT-domain weights."""
    w = synth.WORKLOADS["tiny"]
    hm = synth.head_model(w, 0, 0)
    st = oracle.head_stats(*synth.calibration_samples(w, hm, 0, 0))
    cb = oracle.build_head_codebook(st, 6.0)
    q, K, V = _setup()
    L, d = K.shape
    rng = np.random.default_rng(3)
    sk2 = cb.stepK.astype(np.float64) ** 2 / 12
    sv2 = cb.stepV.astype(np.float64) ** 2 / 12
    # native-domain per-channel variances of U e' with independent e'_j
    natK = (cb.UK ** 2) @ sk2
    natV = (cb.UV ** 2) @ sv2
    DK_nat, DV = oracle.predicted_distortion(q, K, V, np.tile(natK, (L, 1)), np.tile(natV, (L, 1)))
    # KLT-domain key term: (1/d) sum_j q'_j^2 sk2_j sum_i A_i^2 ||v_i - o||^2
    s = K @ q / np.sqrt(d)
    A = np.exp(s - s.max())
    A /= A.sum()
    o = A @ V
    g = (A ** 2 * ((V - o) ** 2).sum(1)).sum()
    DK_klt = ((cb.UK.T @ q) ** 2 * sk2).sum() * g / d
    tot = []
    o0 = oracle.attention(q, K, V)[0]
    for _ in range(3000):
        eK = (rng.uniform(-0.5, 0.5, (L, d)) * cb.stepK.astype(np.float64)) @ cb.UK.T
        eV = (rng.uniform(-0.5, 0.5, (L, d)) * cb.stepV.astype(np.float64)) @ cb.UV.T
        tot.append(((oracle.attention(q, K + eK, V + eV)[0] - o0) ** 2).sum())
    tot = np.array(tot)
    se = tot.std(ddof=1) / np.sqrt(tot.size)
    assert abs(tot.mean() - (DK_klt + DV)) < 4 * se + 0.05 * (DK_klt + DV)
    # the off-diagonal native-domain covariance is not captured by natK; the KLT-domain
    # expression is the exact first-order one and is what the allocation uses
    assert DK_klt > 0 and DK_nat > 0


def _calibration_head(nq=64):
    """Tiny workload, head 0: calibration keys/values and 64 calibration queries per query
    head, their statistics, both KLTs and the channel weights from channel_weights."""
    w = synth.WORKLOADS["tiny"]
    hm = synth.head_model(w, 0, 0)
    K, V, Q = synth.calibration_samples(w, hm, 0, 0)
    Q = Q.reshape(w.group, -1, w.d)[:, :nq].reshape(-1, w.d)
    st = oracle.head_stats(K, V, Q)
    lamK, UK = oracle.klt(st["SigK"])
    lamV, UV = oracle.klt(st["SigV"])
    xK, xV = oracle.channel_weights(st, UK, lamK, UV, lamV)
    return K, V, Q, st, lamK, UK, lamV, UV, xK, xV


def _mean_distortion(Q, K, V, eK, eV, trials, rng):
    """Monte Carlo over independent draws: per trial, the mean over the calibration queries
    of ||o - o_hat||^2 with KLT-domain errors eK(rng), eV(rng) added to every token."""
    o0 = oracle.attention(Q, K, V)
    D = np.array([((oracle.attention(Q, K + eK(rng), V + eV(rng)) - o0) ** 2).sum(1).mean()
                  for _ in range(trials)])
    return D.mean(), D.std(ddof=1) / np.sqrt(trials)


def test_channel_weights_predict_mean_distortion_over_calibration_queries():
    """p2 "Theorem: Additive Error Decomposition" averaged over the calibration queries:
    with KLT-domain errors of variance s_j^2 on every token, the mean over those queries of
    E||o - o_hat||^2 is sum_j s_j^2 x_j / lambda_j with the weights of channel_weights -
    to first order for keys, exactly for values.  The key weights must be the query average
    of the product g(q) q q^T: the same check with M_Q = mean(g) mean(q q^T) misses by many
    standard errors, so this pin tells the two readings apart."""
    K, V, Q, st, lamK, UK, lamV, UV, xK, xV = _calibration_head()
    n, d = K.shape
    eps = 0.01
    zero = lambda rng: 0.0
    rng = np.random.default_rng(11)
    # keys: every channel at eps^2 lambda_j, and a random subset of channels at one variance
    sub = rng.choice(d, 6, replace=False)
    for var in (eps ** 2 * lamK, np.where(np.isin(np.arange(d), sub), 0.05 * eps ** 2 * lamK[0], 0.0)):
        sd = np.sqrt(var)
        m, se = _mean_distortion(Q, K, V, lambda r: (r.standard_normal((n, d)) * sd) @ UK.T, zero, 100, rng)
        pred = float((var * xK / lamK).sum())
        assert abs(m - pred) < 4 * se + 0.01 * pred, (m, se, pred)
    # the product of expectations would predict a different distortion
    o, A = None, None
    s = Q @ K.T / np.sqrt(d)
    A = np.exp(s - s.max(1, keepdims=True))
    A /= A.sum(1, keepdims=True)
    o = A @ V
    g = np.einsum("qi,qi->q", A * A, ((V[None, :, :] - o[:, None, :]) ** 2).sum(2))
    mut = dict(st, MQ=g.mean() * (Q.T @ Q) / Q.shape[0])
    xKm, _ = oracle.channel_weights(mut, UK, lamK, UV, lamV)
    var = eps ** 2 * lamK
    m, se = _mean_distortion(Q, K, V, lambda r: (r.standard_normal((n, d)) * np.sqrt(var)) @ UK.T, zero, 100,
                             np.random.default_rng(12))
    assert abs(m - float((var * xKm / lamK).sum())) > 8 * se
    # values: the value term is quadratic in the errors, so the prediction is exact
    varV = eps ** 2 * lamV
    m, se = _mean_distortion(Q, K, V, zero, lambda r: (r.standard_normal((n, d)) * np.sqrt(varV)) @ UV.T, 100,
                             np.random.default_rng(13))
    assert abs(m - float((varV * xV / lamV).sum())) < 4 * se
