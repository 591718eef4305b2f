"""Oracle vector quantization of the key coefficients: equal-volume grouping and one
fixed-size codebook per group.  Test infrastructure only.

Source: "Spend Bits Where Queries Look: KV Cache Vector Quantization with
Attention-Preserving Transforms" (NOVA-KV), abstract.  The abstract fixes three things:
MSE-optimal vector quantizers applied to the transformed key coefficients; a fixed bit
count per token (equal-size codebooks); and coefficients grouped into partitions of equal
volume, under which equal-size codebooks reach the variable-rate optimum of the
high-resolution model.  Everything else is a reading, stated where it is taken:

* Weighted domain.  The attention-aware key distortion is sum_j w_j E[e_j^2] over the
  coefficient errors e_j, with w_j the key weight per unit variance (the theorem's key
  term after the transform: x_j = lambda_j w_j).  The quantizer works on u_j = s_j c_j with
  s_j = sqrt(w_j), where that distortion is plain MSE and u_j has variance x_j.
* Groups.  VQ_DIM = 4 coefficients per group and VQ_SIZE = 256 codewords (one byte per
  group, 2 bits per coded coefficient).  The 4 n_g largest weights x_j are coded (ties:
  lower index); the others reconstruct to the mean.
* Equal volume.  The high-resolution distortion of a group of dimension m coded with
  2^b codewords scales as (prod_j x_j)^(1/m) 2^(-2b/m); with equal b for every group the
  total equals the variable-rate optimum exactly when every group has the same
  prod_j x_j (its volume).  Groups are formed greedily, as in largest-first bin
  balancing: with a_j = log(x_j / x_min) >= 0 (x_min the smallest coded weight; the shift
  adds the same amount to every full group), coefficients in order of decreasing x_j
  each join the unfilled group with the smallest sum of a so far (ties: lower group
  index).
* Codebooks.  Lloyd's algorithm (nearest codeword, then centroid of each cell; a cell
  left empty keeps its codeword) on the group's Gaussian model N(0, diag(x_g)): training
  samples are caller-supplied standard normal draws scaled by sqrt(x_j) (the draws are an
  input so that every implementation trains on the same points), initial codewords the
  first VQ_SIZE samples, a fixed number of iterations.
* Encoding arithmetic (fp32, decides the integer index): u_k = fp32(c_k * s_k) with
  fp32 s_k = fp32(sqrt(w_k)); t_k = u_k - z_k; distance (t_0 t_0 + t_1 t_1) + (t_2 t_2 +
  t_3 t_3), every operation rounded to fp32 (no fused multiply-add); the lowest index
  attains the minimum.
* Record.  The key record is n_g bytes, byte g = index of group g: the scalar layout
  with n_g pseudo-channels of 8 bits (codec.fields puts pseudo-channel g in byte g).
"""
from __future__ import annotations

import numpy as np

VQ_DIM = 4
VQ_SIZE = 256


def coded_key_channels(x: np.ndarray, n_groups: int) -> np.ndarray:
    """The VQ_DIM * n_groups channels of largest weight (ties: lower index), ascending."""
    x = np.asarray(x, np.float64)
    n = VQ_DIM * n_groups
    if n > x.size:
        raise ValueError("more coded coefficients than channels")
    order = sorted(range(x.size), key=lambda j: (-x[j], j))
    return np.array(sorted(order[:n]), np.int64)


def equal_volume_groups(x: np.ndarray, n_groups: int) -> np.ndarray:
    """[n_groups, VQ_DIM] channel indices (rows ascending) of the greedy equal-volume
    partition of the coded channels (module docstring, "Equal volume")."""
    x = np.asarray(x, np.float64)
    chans = coded_key_channels(x, n_groups)
    if np.any(x[chans] <= 0):
        raise ValueError("a coded key coefficient has zero weight")
    a = np.log(x[chans] / x[chans].min())
    shifted = dict(zip(chans.tolist(), a.tolist()))
    load = np.zeros(n_groups)
    members = [[] for _ in range(n_groups)]
    for j in sorted(chans.tolist(), key=lambda j: (-x[j], j)):
        open_g = [g for g in range(n_groups) if len(members[g]) < VQ_DIM]
        g = min(open_g, key=lambda g: (load[g], g))
        members[g].append(j)
        load[g] += shifted[j]
    return np.array([sorted(m) for m in members], np.int64)


def group_log_volumes(x: np.ndarray, groups: np.ndarray) -> np.ndarray:
    """sum_{j in g} log x_j per group."""
    return np.log(np.asarray(x, np.float64))[np.asarray(groups)].sum(axis=1)


def nearest(samples: np.ndarray, code: np.ndarray) -> np.ndarray:
    """Index of the nearest codeword (squared Euclidean distance, fp64; lowest index on
    ties) for each sample row."""
    d2 = ((samples[:, None, :] - code[None, :, :]) ** 2).sum(axis=2)
    return np.argmin(d2, axis=1)


def lloyd(samples: np.ndarray, init: np.ndarray, iters: int) -> np.ndarray:
    """Lloyd's algorithm in fp64: `iters` rounds of (assign every sample to its nearest
    codeword; move each codeword to the mean of its cell, an empty cell keeping its
    codeword).  Returns the codebook [K, m]."""
    y = np.asarray(samples, np.float64)
    code = np.array(init, np.float64, copy=True)
    for _ in range(iters):
        a = nearest(y, code)
        for k in range(code.shape[0]):
            cell = y[a == k]
            if cell.shape[0]:
                code[k] = cell.sum(axis=0) / cell.shape[0]
    return code


def group_codebooks(x: np.ndarray, groups: np.ndarray, normals: np.ndarray,
                    iters: int) -> np.ndarray:
    """One Lloyd codebook per group on samples normals * sqrt(x_g) (module docstring,
    "Codebooks"); normals [n, VQ_DIM] standard normal draws, n >= VQ_SIZE.
    Returns [n_groups, VQ_SIZE, VQ_DIM] float64."""
    z = np.asarray(normals, np.float64)
    if z.ndim != 2 or z.shape[1] != VQ_DIM or z.shape[0] < VQ_SIZE:
        raise ValueError("need at least VQ_SIZE training draws of dimension VQ_DIM")
    out = np.zeros((len(groups), VQ_SIZE, VQ_DIM))
    for g, chans in enumerate(groups):
        y = z * np.sqrt(np.asarray(x, np.float64)[chans])[None, :]
        out[g] = lloyd(y, y[:VQ_SIZE], iters)
    return out


def vq_scales(w: np.ndarray) -> np.ndarray:
    """fp32 s_j = sqrt(w_j) (the weighted domain of the module docstring)."""
    return np.sqrt(np.maximum(np.asarray(w, np.float64), 0.0)).astype(np.float32)


def vq_encode(c32: np.ndarray, groups: np.ndarray, scale32: np.ndarray,
              cent32: np.ndarray) -> np.ndarray:
    """Indices [n, n_groups] of fp32 key coefficients c32 [n, d] (module docstring,
    "Encoding arithmetic").  numpy float32 operations round each result once, as the
    definition requires."""
    c32 = np.asarray(c32, np.float32)
    if not np.all(np.isfinite(c32)):
        raise ValueError("non-finite coefficient")
    s = np.asarray(scale32, np.float32)
    out = np.zeros((c32.shape[0], len(groups)), np.int64)
    for g, chans in enumerate(groups):
        u = (c32[:, chans] * s[chans][None, :]).astype(np.float32)        # [n, 4]
        t = (u[:, None, :] - np.asarray(cent32[g], np.float32)[None, :, :]).astype(np.float32)
        sq = (t * t).astype(np.float32)
        e = ((sq[..., 0] + sq[..., 1]).astype(np.float32)
             + (sq[..., 2] + sq[..., 3]).astype(np.float32)).astype(np.float32)
        out[:, g] = np.argmin(e, axis=1)
    return out


def vq_dequantize(idx: np.ndarray, groups: np.ndarray, scale32: np.ndarray,
                  cent32: np.ndarray, d: int) -> np.ndarray:
    """Reconstructed coefficients c_hat [n, d] (fp64): c_hat_j = z_j / s_j for the
    codeword z of j's group, 0 for uncoded channels."""
    idx = np.asarray(idx, np.int64)
    s = np.asarray(scale32, np.float64)
    out = np.zeros((idx.shape[0], d))
    for g, chans in enumerate(groups):
        z = np.asarray(cent32[g], np.float64)[idx[:, g]]                   # [n, 4]
        out[:, chans] = z / s[chans][None, :]
    return out
