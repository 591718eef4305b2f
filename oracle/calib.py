"""Oracle calibration: statistics, KLT, attention-aware weights, reverse water-filling,
integer bit allocation and the scalar quantizer's step sizes.  Test infrastructure only.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------------------
# statistics
# ----------------------------------------------------------------------------------------
def head_stats(K: np.ndarray, V: np.ndarray, Q: np.ndarray) -> dict:
    """Calibration statistics of one (layer, kv-head).

    p2 "Decorrelation via the KLT": the channel covariances of calibration keys and
    values.  Reading: centred, normalised by 1/N (the listing centres; the formula
    does not; a key mean is part of the synthetic workloads).

    p2 "Theorem: Additive Error Decomposition": key errors are weighted by the
    query's channel energy times sum_i A_i^2 ||v_i - o||^2, value errors by
    sum_i A_i^2.  Reading: the expectation over calibration queries of the product,
    M_Q = mean_q g(q) q q^T with g(q) = sum_i A_i^2 ||v_i - o(q)||^2, and
    gamma_V = mean_q sum_i A_i^2, with A = softmax(q k_i / sqrt(d)) over the
    calibration tokens (non-causal, raw keys).
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Q = np.asarray(Q, np.float64)
    n, d = K.shape
    muK = K.mean(axis=0)
    muV = V.mean(axis=0)
    Kc = K - muK
    Vc = V - muV
    SigK = Kc.T @ Kc / n
    SigV = Vc.T @ Vc / n

    MQ = np.zeros((d, d))
    gam = 0.0
    vnorm2 = np.einsum("ij,ij->i", V, V)
    for s in range(0, Q.shape[0], 256):
        q = Q[s:s + 256]
        logits = q @ K.T / math.sqrt(d)
        logits -= logits.max(axis=1, keepdims=True)
        A = np.exp(logits)
        A /= A.sum(axis=1, keepdims=True)
        o = A @ V
        A2 = A * A
        # sum_i A_i^2 ||v_i - o||^2 expanded: sum A^2|v|^2 - 2 o.(sum A^2 v) + |o|^2 sum A^2
        sA2 = A2.sum(axis=1)
        g = A2 @ vnorm2 - 2.0 * np.einsum("qd,qd->q", o, A2 @ V) + np.einsum("qd,qd->q", o, o) * sA2
        MQ += (q * g[:, None]).T @ q
        gam += sA2.sum()
    nq = Q.shape[0]
    return {"muK": muK, "muV": muV, "SigK": SigK, "SigV": SigV,
            "MQ": MQ / nq, "gammaV": gam / nq, "n": n, "nq": nq, "d": d}


# ----------------------------------------------------------------------------------------
# KLT
# ----------------------------------------------------------------------------------------
def klt(Sigma: np.ndarray):
    """Eigendecomposition Sigma = U diag(lam) U^T (p2 "Decorrelation via the KLT").

    Reading for the freedom the pages leave: eigenvalues in descending order, and
    each eigenvector's largest-magnitude entry made positive (lowest row on ties).
    """
    lam, U = np.linalg.eigh(np.asarray(Sigma, np.float64))
    lam = lam[::-1].copy()
    U = U[:, ::-1].copy()
    for j in range(U.shape[1]):
        col = U[:, j]
        i = int(np.argmax(np.abs(col)))  # first index of the maximum
        if col[i] < 0:
            U[:, j] = -col
    lam = np.maximum(lam, 0.0)
    return lam, U


# ----------------------------------------------------------------------------------------
# attention-optimal (non-orthogonal) key transform
# ----------------------------------------------------------------------------------------
NOVA_RIDGE = 1e-6  # M_Q + ridge * (tr M_Q / d) I: the transform needs an invertible M_Q


def nova_key_transform(SigK: np.ndarray, MQ: np.ndarray, ridge: float = NOVA_RIDGE):
    """Key transform under which the attention-aware key distortion is plain MSE of the
    coefficients ("Spend Bits Where Queries Look", abstract: a non-orthogonal optimal
    transform from calibration statistics; a generalized Parseval relation turns
    attention distortion into transform-domain MSE).

    Reading (the pages give no formula): a key error e costs (first order, p2 "Theorem")
    e^T M_Q e.  With coefficients c = (k - mu) T, an error eps in c is e = eps T^{-1}, and
    e^T M_Q e = eps (T^{-1} M_Q T^{-T}) eps^T, which is |eps|^2 for every T = M_Q^{1/2} R with
    R orthogonal.  Among those, R = the eigenvectors of M_Q^{1/2} Sigma_K M_Q^{1/2} also
    decorrelates the coefficients (variances mu = its eigenvalues), which is what the
    per-channel quantizer and the water-filling assume.  M_Q gets a small ridge so that
    it is invertible (queries need not span every direction).

    Returns (mu descending, T, T^{-1}); R follows the KLT's order and sign rule."""
    MQ = np.asarray(MQ, np.float64)
    d = MQ.shape[0]
    Mr = 0.5 * (MQ + MQ.T) + ridge * (np.trace(MQ) / d) * np.eye(d)
    w, V = np.linalg.eigh(Mr)
    if not np.all(w > 0):
        raise ValueError("M_Q is not positive definite after the ridge")
    Mh = (V * np.sqrt(w)[None, :]) @ V.T
    Mih = (V / np.sqrt(w)[None, :]) @ V.T
    mu, R = klt(Mh @ np.asarray(SigK, np.float64) @ Mh)
    return mu, Mh @ R, R.T @ Mih


# ----------------------------------------------------------------------------------------
# attention-aware channel weights
# ----------------------------------------------------------------------------------------
def key_weights_general(MQ: np.ndarray, var: np.ndarray, Tinv: np.ndarray) -> np.ndarray:
    """x_j = var_j (T^{-1} M_Q T^{-T})_jj / d for a general key transform T (coefficient
    errors eps map to key errors eps T^{-1}); the KLT's weights are the case T = U_K."""
    d = MQ.shape[0]
    w = np.einsum("ji,ik,jk->j", Tinv, np.asarray(MQ, np.float64), Tinv) / d
    return np.maximum(np.asarray(var, np.float64) * w, 0.0)


def channel_weights(stats: dict, UK: np.ndarray, lamK: np.ndarray, UV: np.ndarray,
                    lamV: np.ndarray):
    """Per-channel distortion scale x_j = w_j * lambda_j in the KLT domain.

    p2 "Theorem": D_K = (1/d) sum_j q_j^2 sum_i A_i^2 ||v_i - o||^2 sigma_K,ij^2 and
    D_V = sum_i A_i^2 sum_j sigma_V,ij^2.  A key error e = U_K e' gives q.e = (U_K^T q).e',
    so in the KLT domain key channel j is weighted by (U_K^T M_Q U_K)_jj / d; an
    orthogonal U_V leaves value errors' norm unchanged, so value channels share gamma_V.
    With a coding distortion proportional to lambda_j (rate-distortion of a Gaussian),
    the weighted distortion of channel j is x_j * 4^(-b_j).
    """
    d = UK.shape[0]
    wK = np.einsum("ij,ik,kj->j", UK, stats["MQ"], UK) / d
    xK = np.maximum(lamK * wK, 0.0)
    xV = np.maximum(lamV * stats["gammaV"], 0.0)
    return xK, xV


# ----------------------------------------------------------------------------------------
# reverse water-filling
# ----------------------------------------------------------------------------------------
def waterfill_theta(x: np.ndarray, total_bits: float, max_bits: int = 8):
    """Continuous reverse water-filling (p2 "Optimal Bit Allocation via Reverse Water-Filling").

    R_j = max(0, 1/2 log2(x_j / theta)), capped at max_bits, with theta chosen so that
    sum_j R_j = total_bits.  Bisection on log(theta).  Returns (theta, R).
    """
    x = np.asarray(x, np.float64)
    pos = x[x > 0]
    if total_bits <= 0 or pos.size == 0:
        return float("inf"), np.zeros_like(x)
    if total_bits >= max_bits * pos.size:
        return 0.0, np.where(x > 0, float(max_bits), 0.0)

    def rate(log_theta):
        r = np.zeros_like(x)
        m = x > 0
        r[m] = 0.5 * (np.log2(x[m]) - log_theta / math.log(2.0))
        return np.clip(r, 0.0, max_bits)

    lo = math.log(pos.min()) - 2.0 * max_bits * math.log(2.0) - 1.0  # every channel capped
    hi = math.log(pos.max())  # every channel at zero
    for _ in range(400):
        mid = 0.5 * (lo + hi)
        if rate(mid).sum() > total_bits:
            lo = mid
        else:
            hi = mid
        if hi - lo < 1e-15 * max(1.0, abs(mid)):
            break
    lt = 0.5 * (lo + hi)
    return math.exp(lt), rate(lt)


def _greedy(groups, budget: int, max_bits: int):
    """The `budget` largest marginal gains x_j 4^(-k), k < max_bits, over the channels of
    `groups` [(group id, x)]; ties: lower group id, then lower channel, then lower k.
    Returns {group id: bits}."""
    cand = []
    for gi, x in groups:
        for j in range(x.size):
            for k in range(max_bits):
                cand.append((-(x[j] * 4.0 ** (-k)), gi, j, k))
    cand.sort()
    bits = {gi: np.zeros(x.size, np.int64) for gi, x in groups}
    for c in cand[:budget]:
        bits[c[1]][c[2]] += 1
    return bits


def _cost(x, b):
    return float(sum(xi * 4.0 ** (-int(bi)) for xi, bi in zip(x.tolist(), b.tolist())))


def allocate_bits(xK: np.ndarray, xV: np.ndarray, total_bits: int, max_bits: int = 8,
                  joint: bool = True, key_align: int = 1):
    """Integer bits per channel under an exact budget (reading of p2's water-filling
    "rounded to integers under the budget").

    Distortion model: channel j at b bits costs x_j 4^(-b).  The marginal gain of the
    (k+1)-th bit is proportional to x_j 4^(-k); taking the largest gains (k < max_bits)
    gives the exact-budget optimum of the separable convex problem (ties: keys before
    values, then lower channel index, then lower k).

    key_align = 1 (the default) is the method itself: one budget over all channels.
    key_align > 1 is a storage constraint named by the caller (a layout holding key
    records in whole words of key_align bits): the keys' total must be a multiple of it,
    and the result is the optimum over such splits - for every admissible key budget B_K
    the key and value sub-problems are solved exactly and the split of least total cost
    is taken (ties: the smaller B_K).  joint=False gives keys and values total_bits/2
    each.
    """
    xK = np.asarray(xK, np.float64)
    xV = np.asarray(xV, np.float64)
    d = xK.size
    if not joint:
        if total_bits % 2 or (total_bits // 2) % key_align:
            raise ValueError("separate budgets need total_bits/2 a multiple of key_align")
        return (_greedy([(0, xK)], total_bits // 2, max_bits)[0],
                _greedy([(1, xV)], total_bits // 2, max_bits)[1])
    assert 0 <= total_bits <= 2 * d * max_bits
    if key_align == 1:
        b = _greedy([(0, xK), (1, xV)], int(total_bits), max_bits)
        return b[0], b[1]
    best = None
    for bk_total in range(0, min(total_bits, d * max_bits) + 1, key_align):
        bv_total = total_bits - bk_total
        if bv_total > d * max_bits:
            continue
        bK = _greedy([(0, xK)], bk_total, max_bits)[0]
        bV = _greedy([(1, xV)], bv_total, max_bits)[1]
        cost = _cost(xK, bK) + _cost(xV, bV)
        if best is None or cost < best[0]:
            best = (cost, bK, bV)
    if best is None:
        raise ValueError("no admissible key/value split of the budget")
    return best[1], best[2]


# ----------------------------------------------------------------------------------------
# scalar quantizer design
# ----------------------------------------------------------------------------------------
def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi) if math.isfinite(x) else 0.0


def _Phi(x):
    if x == math.inf:
        return 1.0
    if x == -math.inf:
        return 0.0
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def uniform_quantizer_mse(step: float, levels: int) -> float:
    """MSE of a unit Gaussian through the midrise uniform quantizer with ``levels`` cells
    of width ``step`` centred on 0; the two outer cells extend to infinity.

    For a cell [a, b] with reconstruction r: int (x-r)^2 phi = [Phi] + [a phi(a) - b phi(b)]
    - 2 r [phi(a) - phi(b)] + r^2 [Phi], exact Gaussian integrals.
    """
    half = levels // 2
    total = 0.0
    for k in range(-half, half):
        a = -math.inf if k == -half else k * step
        b = math.inf if k == half - 1 else (k + 1) * step
        r = (k + 0.5) * step
        P = _Phi(b) - _Phi(a)
        m1 = _phi(a) - _phi(b)
        aphi = 0.0 if not math.isfinite(a) else a * _phi(a)
        bphi = 0.0 if not math.isfinite(b) else b * _phi(b)
        m2 = P + aphi - bphi
        total += m2 - 2.0 * r * m1 + r * r * P
    return total


def _mse_slope(step: float, levels: int) -> float:
    """Half the derivative of uniform_quantizer_mse with respect to the step.

    Moving a cell boundary changes nothing to first order (both neighbouring
    reconstructions sit half a step away), so only the reconstruction points move:
    d/dstep MSE = 2 sum_k (k+1/2) [(k+1/2) step P_k - M1_k] over the cells k.
    """
    half = levels // 2
    total = 0.0
    for k in range(-half, half):
        a = -math.inf if k == -half else k * step
        b = math.inf if k == half - 1 else (k + 1) * step
        c = k + 0.5
        total += c * (c * step * (_Phi(b) - _Phi(a)) - (_phi(a) - _phi(b)))
    return total


def optimal_step(bits: int) -> float:
    """Step of the MSE-optimal 2^bits-level midrise uniform quantizer for a unit Gaussian
    (reading: the static per-channel quantizer; steps scale with sqrt(lambda), the
    "whitening" of p1 Methodology).  Bisection on the sign of dMSE/dstep, which is
    negative below the optimum and positive above it."""
    levels = 1 << bits
    lo, hi = 1e-4, 4.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _mse_slope(mid, levels) < 0.0:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 4e-16 * hi:
            break
    return 0.5 * (lo + hi)


# ----------------------------------------------------------------------------------------
# codebook of one head
# ----------------------------------------------------------------------------------------
@dataclass
class VQKeys:
    groups: np.ndarray   # int [n_groups, 4] key channels per group
    scale32: np.ndarray  # float32 [d]: s_j = sqrt(w_j)
    cent: np.ndarray     # float64 [n_groups, 256, 4] Lloyd codebooks (weighted domain)

    @property
    def cent32(self):
        return self.cent.astype(np.float32)

    @property
    def record_bits(self):
        """Pseudo-channel widths of the key record: one byte per group."""
        return np.full(len(self.groups), 8, np.int64)


@dataclass
class HeadCodebook:
    d: int
    UK: np.ndarray      # float64 [d, d], columns = KLT basis (descending eigenvalues)
    UV: np.ndarray
    lamK: np.ndarray
    lamV: np.ndarray
    muK: np.ndarray     # float64 [d]
    muV: np.ndarray
    xK: np.ndarray
    xV: np.ndarray
    bK: np.ndarray      # int [d]
    bV: np.ndarray
    stepK: np.ndarray   # float32 [d] (0 where b = 0)
    stepV: np.ndarray
    theta: float
    UKinv: np.ndarray = None  # float64 [d, d]: key reconstruction (k_hat = mu + c_hat UKinv); U_K^T for the KLT
    vq: "VQKeys" = None       # vector-quantized keys (bK all zero then), else None

    def __post_init__(self):
        if self.UKinv is None:
            self.UKinv = self.UK.T.copy()

    @property
    def UK32(self):
        return self.UK.astype(np.float32)

    @property
    def UV32(self):
        return self.UV.astype(np.float32)

    def inv_step(self, which: str) -> np.ndarray:
        s = self.stepK if which == "K" else self.stepV
        out = np.zeros(s.shape, np.float32)
        m = s > 0
        out[m] = (1.0 / s[m].astype(np.float64)).astype(np.float32)
        return out


_STEP_CACHE: dict = {}


def step_table(max_bits: int = 8) -> np.ndarray:
    """Optimal unit-variance steps for b = 0..max_bits (entry 0 unused)."""
    if max_bits not in _STEP_CACHE:
        _STEP_CACHE[max_bits] = np.array([0.0] + [optimal_step(b) for b in range(1, max_bits + 1)])
    return _STEP_CACHE[max_bits]


def build_head_codebook(stats: dict, avg_bits: float, max_bits: int = 8,
                        joint: bool = True, key_transform: str = "klt",
                        key_quantizer: str = "scalar", vq_normals: np.ndarray | None = None,
                        vq_iters: int = 20, key_align: int = 1) -> HeadCodebook:
    """Calibrate one head: KLT of both covariances (or, for the keys, the attention-optimal
    transform of nova_key_transform), weights, exact-budget integer bits with total
    2 d avg_bits (a multiple of 8), and fp32 steps step_b * sqrt(coefficient variance).

    The bits are the exact-budget optimum of p2's water-filling over all 2d channels
    (key_align = 1).  key_align > 1 is a storage constraint that the caller names: a
    packed layout that keeps each token's key record in whole words of key_align bits
    can only hold key totals that are multiples of it, and allocate_bits then returns
    the best allocation among those (its cost over the unconstrained optimum is pinned by
    the tests).

    key_quantizer "vq" (NOVA-KV abstract; readings in oracle.vq): separate budgets of
    d avg_bits bits for keys and values; the key bits go to d avg_bits / 8 groups of four
    coefficients with one 256-word Lloyd codebook each (so avg_bits <= 2 and d avg_bits a
    multiple of 32: whole groups of four one-byte indices), trained on vq_normals; the
    values keep the scalar quantizer."""
    d = stats["d"]
    total = 2.0 * d * avg_bits
    B = int(round(total))
    if abs(total - B) > 1e-9 or B % 8:
        raise ValueError("2*d*avg_bits must be a whole number of bytes (the packed records "
                         "are byte strings)")
    lamV, UV = klt(stats["SigV"])
    if key_transform == "klt":
        lamK, UK = klt(stats["SigK"])
        UKinv = UK.T.copy()
        xK, xV = channel_weights(stats, UK, lamK, UV, lamV)
    elif key_transform == "nova":
        lamK, UK, UKinv = nova_key_transform(stats["SigK"], stats["MQ"])
        xK = key_weights_general(stats["MQ"], lamK, UKinv)
        xV = np.maximum(lamV * stats["gammaV"], 0.0)
    else:
        raise ValueError(f"unknown key transform {key_transform!r}")
    theta, _ = waterfill_theta(np.concatenate([xK, xV]), B, max_bits)
    vq = None
    if key_quantizer == "vq":
        if joint:
            raise ValueError("vector-quantized keys take separate key and value budgets")
        BK = B // 2
        if BK % 32 or 4 * (BK // 8) > d:
            raise ValueError("vector-quantized keys need d*avg_bits a multiple of 32 and "
                             "avg_bits <= 2")
        from .vq import equal_volume_groups, group_codebooks, vq_scales
        _, bV = allocate_bits(xK, xV, B, max_bits, False)
        bK = np.zeros(d, np.int64)
        groups = equal_volume_groups(xK, BK // 8)
        w = np.where(lamK > 0, xK / np.where(lamK > 0, lamK, 1.0), 0.0)
        vq = VQKeys(groups, vq_scales(w), group_codebooks(xK, groups, vq_normals, vq_iters))
    elif key_quantizer == "scalar":
        bK, bV = allocate_bits(xK, xV, B, max_bits, joint, key_align=key_align)
    else:
        raise ValueError(f"unknown key quantizer {key_quantizer!r}")
    st = step_table(max_bits)
    stepK = np.where(bK > 0, st[bK] * np.sqrt(lamK), 0.0).astype(np.float32)
    stepV = np.where(bV > 0, st[bV] * np.sqrt(lamV), 0.0).astype(np.float32)
    return HeadCodebook(d, UK, UV, lamK, lamV, stats["muK"].copy(), stats["muV"].copy(),
                        xK, xV, bK, bV, stepK, stepV, theta, UKinv, vq)
