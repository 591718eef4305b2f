"""Oracle transform coding: projection, scalar quantizer, packed tile layout, unpack and
dequantization.  Test infrastructure only.

Packed layout (ours; the pages fix only a fixed per-token bit count, p3 abstract):

* The cache of one (layer, sequence, kv-head) is a run of tiles of 64 token slots.
  A tile is 8*B bytes, B = B_K + B_V = sum of all channel widths of the head; B_K is a
  multiple of 32 and B_V a multiple of 8.
* A token's key record (B_K bits) and value record (B_V bits) are byte strings.  The
  coded channels of a record are placed as byte-aligned fields, a field never crossing a
  byte boundary (``fields``):
    1. channels with b > 0, widest first (ties: lower channel index first), each go whole
       into the lowest-index byte with at least b free bits, at that byte's lowest free
       bit;
    2. channels that found no such byte are then cut, in the same order, into pieces that
       fill free bits byte by byte from the lowest byte: each piece takes min(free bits,
       bits left) of the code, lowest code bits first;
    3. the bytes are renumbered by decreasing field count (ties: lower byte first).
  A field (channel j, width w, shift e, byte q, position p) holds code bits [e, e+w) of
  channel j at bits [p, p+w) of record byte q.
* K block (first 8*B_K bytes): record byte q of slot s is byte 4*(64*(q//4) + s) + q%4
  (record word r = bytes 4r..4r+3 of slot s is block word 64r + s).
* V block (next 8*B_V bytes): record byte q of slot s is byte 64*q + s.
* Every record byte of a written slot (keys and values) is stored with its most
  significant bit inverted (XOR 0x80): masking one field of a stored byte and reading it
  as a two's-complement int8 then gives field * 2^p when the field stays below bit 7,
  and that value minus 128 when it ends at bit 7.
* Slots not yet written are zero.
"""
from __future__ import annotations

import numpy as np

TILE = 64


def fields(bits: np.ndarray):
    """Byte-aligned fields of one record: [(chan, width, shift, byte, pos)] sorted by
    (byte, pos); the placement rule is the one in the module docstring."""
    b = [int(x) for x in np.asarray(bits).tolist()]
    R = sum(b)
    if R % 8:
        raise ValueError("record bits must be a whole number of bytes")
    nbytes = R // 8
    free = [8] * nbytes
    out, left = [], []
    for j in sorted((j for j in range(len(b)) if b[j] > 0), key=lambda j: (-b[j], j)):
        q = next((q for q in range(nbytes) if free[q] >= b[j]), None)
        if q is None:
            left.append(j)
            continue
        out.append((j, b[j], 0, q, 8 - free[q]))
        free[q] -= b[j]
    for j in left:
        e = 0
        for q in range(nbytes):
            if e == b[j]:
                break
            w = min(free[q], b[j] - e)
            if w:
                out.append((j, w, e, q, 8 - free[q]))
                free[q] -= w
                e += w
    count = [0] * nbytes
    for f in out:
        count[f[3]] += 1
    rank = {q: i for i, q in enumerate(sorted(range(nbytes), key=lambda q: (-count[q], q)))}
    return sorted(((j, w, e, rank[q], p) for (j, w, e, q, p) in out), key=lambda f: (f[3], f[4]))


def record_bits(bits: np.ndarray) -> int:
    return int(np.asarray(bits).sum())


def tile_bytes(bK: np.ndarray, bV: np.ndarray) -> int:
    return 8 * (record_bits(bK) + record_bits(bV))


def transform_coeffs(x: np.ndarray, mu: np.ndarray, U: np.ndarray) -> np.ndarray:
    """KLT coefficients c = (x - mu) U (p2 "Decorrelation via the KLT": K' = K U_K),
    in float64, returned rounded to float32."""
    return ((np.asarray(x, np.float64) - mu[None, :]) @ U).astype(np.float32)


def quantize(c32: np.ndarray, inv_step32: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """Midrise uniform scalar quantizer with 2^b levels (reading of p2's listing, which
    quantizes each rotated channel at its allotted width).  fp32 arithmetic:
    t = c * (1/step) rounded once; code = clamp(floor(t) + 2^(b-1), 0, 2^b - 1).
    Channels with b = 0 get code 0 and are not stored."""
    c32 = np.asarray(c32, np.float32)
    if not np.all(np.isfinite(c32)):
        raise ValueError("non-finite coefficient")
    t = (c32 * np.asarray(inv_step32, np.float32)[None, :]).astype(np.float32)
    k = np.floor(t).astype(np.int64)
    b = np.asarray(bits, np.int64)[None, :]
    half = np.where(b > 0, 1 << np.maximum(b - 1, 0), 0)
    code = np.clip(k + half, 0, (1 << b) - 1)
    return np.where(b > 0, code, 0).astype(np.int64)


def dequantize(codes: np.ndarray, bits: np.ndarray, step32: np.ndarray) -> np.ndarray:
    """Reconstruction point (code - 2^(b-1) + 1/2) * step; zero for b = 0 (float64)."""
    b = np.asarray(bits, np.int64)[None, :]
    half = np.where(b > 0, 1 << np.maximum(b - 1, 0), 0)
    val = (codes - half + 0.5) * np.asarray(step32, np.float64)[None, :]
    return np.where(b > 0, val, 0.0)


def reconstruct(chat: np.ndarray, mu: np.ndarray, U: np.ndarray) -> np.ndarray:
    """Inverse transform x_hat = mu + c_hat U^T (the listing's K_hat = deq U_K^T)."""
    return mu[None, :] + chat @ np.asarray(U, np.float64).T


def _check_bits(bK, bV):
    BK, BV = record_bits(bK), record_bits(bV)
    if BK % 32:
        raise ValueError("key bits per token must be a multiple of 32")
    if BV % 8:
        raise ValueError("value bits per token must be a multiple of 8")
    return BK, BV


def _records(codes: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """[n, R/8] record bytes (before the bit-7 inversion) of codes [n, d]."""
    rec = np.zeros((codes.shape[0], record_bits(bits) // 8), np.int64)
    for (j, w, e, q, p) in fields(bits):
        rec[:, q] |= ((codes[:, j] >> e) & ((1 << w) - 1)) << p
    return rec


def _byte_offsets(n: int, BK: int, BV: int):
    """Cache byte offsets of record byte q of tokens 0..n-1: ([n, BK/8], [n, BV/8])."""
    tok = np.arange(n)
    tile, slot = tok // TILE, tok % TILE
    tbytes = 8 * (BK + BV)
    qk = np.arange(BK // 8)[None, :]
    qv = np.arange(BV // 8)[None, :]
    offK = tile[:, None] * tbytes + 4 * (64 * (qk // 4) + slot[:, None]) + qk % 4
    offV = tile[:, None] * tbytes + 8 * BK + 64 * qv + slot[:, None]
    return offK, offV


def pack_cache(codesK: np.ndarray, codesV: np.ndarray, bK: np.ndarray, bV: np.ndarray,
               n_tiles: int | None = None) -> np.ndarray:
    """Pack codes of tokens 0..n-1 (KLT channel order) into tiles; returns uint8 bytes."""
    n = codesK.shape[0]
    BK, BV = _check_bits(bK, bV)
    if n_tiles is None:
        n_tiles = (n + TILE - 1) // TILE
    out = np.zeros(n_tiles * 8 * (BK + BV), np.uint8)
    offK, offV = _byte_offsets(n, BK, BV)
    out[offK] = (_records(np.asarray(codesK, np.int64), bK) ^ 0x80).astype(np.uint8)
    out[offV] = (_records(np.asarray(codesV, np.int64), bV) ^ 0x80).astype(np.uint8)
    return out


def unpack_cache(cache: np.ndarray, bK: np.ndarray, bV: np.ndarray, n: int):
    """Inverse of pack_cache for the first n token slots: (codesK, codesV) [n, d]."""
    BK, BV = _check_bits(bK, bV)
    raw = np.asarray(cache, np.uint8)
    offK, offV = _byte_offsets(n, BK, BV)
    out = []
    for bits, off in ((bK, offK), (bV, offV)):
        rec = raw[off].astype(np.int64) ^ 0x80
        c = np.zeros((n, len(bits)), np.int64)
        for (j, w, e, q, p) in fields(bits):
            c[:, j] |= ((rec[:, q] >> p) & ((1 << w) - 1)) << e
        out.append(c)
    return out[0], out[1]


def key_record_bits(cb) -> np.ndarray:
    """Field widths of the key record: the channel bits, or one 8-bit pseudo-channel per
    group for vector-quantized keys (byte g = index of group g)."""
    return cb.vq.record_bits if cb.vq is not None else cb.bK


def encode_cache(K: np.ndarray, V: np.ndarray, cb, n_tiles: int | None = None):
    """Whole encoder for one (layer, seq, head): transform, quantize, pack.
    Returns (cache bytes, codesK, codesV); codesK holds the group indices [n, n_groups]
    for vector-quantized keys."""
    cKf = transform_coeffs(K, cb.muK, cb.UK)
    cVf = transform_coeffs(V, cb.muV, cb.UV)
    if cb.vq is not None:
        from .vq import vq_encode
        codesK = vq_encode(cKf, cb.vq.groups, cb.vq.scale32, cb.vq.cent32)
    else:
        codesK = quantize(cKf, cb.inv_step("K"), cb.bK)
    codesV = quantize(cVf, cb.inv_step("V"), cb.bV)
    return pack_cache(codesK, codesV, key_record_bits(cb), cb.bV, n_tiles), codesK, codesV
