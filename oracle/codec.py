"""Oracle transform coding: projection, scalar quantizer, packed tile layout, unpack and
dequantization.  Test infrastructure only.

Packed layout (ours; the pages fix only a fixed per-token bit count, p3 abstract):

* The cache of one (layer, sequence, kv-head) is a run of tiles of 64 token slots.
  A tile is 8*B bytes, B = B_K + B_V = sum of all channel widths of the head.
* Each channel of width b > 0 is split into "pieces" of width 4, 2 or 1: as many 4-bit
  pieces as fit (from the most significant bit), then a 2-bit and/or a 1-bit piece
  (b = 8 -> 4+4, 7 -> 4+2+1, 6 -> 4+2, 5 -> 4+1, 3 -> 2+1).  The piece of width w with
  shift e holds code bits [e, e+w).  Pieces are ordered by width (4, 2, 1), then by KLT
  channel index, then by shift (high first).  O_p is the sum of the widths of the pieces
  before p (so O_p is a multiple of w_p).
* Bit n of a block is bit n%8 of byte n//8 (little endian).
* K block (first 8*B_K bytes; B_K is a multiple of 32): each token slot s has a record
  of B_K bits, piece p at record bits [O_p, O_p + w_p).  Record word r (bits
  [32r, 32r+32)) of slot s is word 64*r + s of the K block.
* V block (next 8*B_V bytes): piece p owns a slab of 64*w_p bits starting at bit
  64*O_p.  Slab word r (32 bits) holds token slots r*(32/w) + k, k < 32/w, with slot
  k's field at word bits [8*(k%4) + w*(k//4), +w).
* Every byte of a written slot's key record is stored with its most significant bit
  inverted (XOR 0x80): an extraction that masks one field per byte then reads, as a
  two's-complement int8, field * 2^(bit position) when the field stays below bit 7 and
  that value minus 128 when it ends at bit 7 -- a constant per byte position that a
  reader can correct for.
* Slots not yet written are zero (all of their bytes, key records included).
"""
from __future__ import annotations

import numpy as np

TILE = 64


def _split(b: int):
    """Power-of-two pieces of a b-bit code, most significant first: as many 4-bit pieces as
    fit, then a 2-bit and/or a 1-bit piece.  Returns [(width, shift)]."""
    out, rem = [], b
    for w in (4, 4, 2, 1):
        if rem >= w:
            rem -= w
            out.append((w, rem))
    return out


def pieces(bits: np.ndarray):
    """Pieces of a head's K or V channels: list of (channel, width, shift), ordered by width
    (4, 2, 1), then channel, then shift (high first)."""
    out = []
    blist = np.asarray(bits).tolist()
    for w in (4, 2, 1):
        for j, b in enumerate(blist):
            for (pw, e) in _split(b):
                if pw == w:
                    out.append((j, w, e))
    return out


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


def _field_bits(values: np.ndarray, w: int) -> np.ndarray:
    """[n] ints -> [n, w] bits, least significant first."""
    return ((values[:, None] >> np.arange(w)[None, :]) & 1).astype(np.uint8)


def pack_cache(codesK: np.ndarray, codesV: np.ndarray, bK: np.ndarray, bV: np.ndarray,
               n_tiles: int | None = None) -> np.ndarray:
    """Pack codes of tokens 0..n-1 (KLT channel order) into tiles; returns uint8 bytes."""
    n = codesK.shape[0]
    BK, BV = record_bits(bK), record_bits(bV)
    if BK % 32:
        raise ValueError("key bits per token must be a multiple of 32")
    if n_tiles is None:
        n_tiles = (n + TILE - 1) // TILE
    kbits = 64 * BK
    tbits = 64 * (BK + BV)
    bitarr = np.zeros(n_tiles * tbits, np.uint8)
    tok = np.arange(n)
    tile = tok // TILE
    slot = tok % TILE
    off = 0
    for (j, w, e) in pieces(bK):
        vals = (codesK[:, j] >> e) & ((1 << w) - 1)
        rbit = off + np.arange(w)[None, :]
        pos = tile[:, None] * tbits + 32 * ((rbit // 32) * 64 + slot[:, None]) + rbit % 32
        bitarr[pos] = _field_bits(vals, w)
        off += w
    off = 0
    for (j, w, e) in pieces(bV):
        vals = (codesV[:, j] >> e) & ((1 << w) - 1)
        per_word = 32 // w
        r = slot // per_word
        k = slot % per_word
        inword = 8 * (k % 4) + w * (k // 4)
        base = tile * tbits + kbits + 64 * off + 32 * r + inword
        pos = base[:, None] + np.arange(w)[None, :]
        bitarr[pos] = _field_bits(vals, w)
        off += w
    out = np.packbits(bitarr, bitorder="little")
    _flip_key_bytes(out, n, BK, 8 * (BK + BV))
    return out


def _flip_key_bytes(buf: np.ndarray, n: int, BK: int, tbytes: int) -> None:
    """Invert bit 7 of every byte of the key records of token slots 0..n-1, in place."""
    tok = np.arange(n)
    tile, slot = tok // TILE, tok % TILE
    for r in range(BK // 32):
        byte0 = tile * tbytes + 4 * (64 * r + slot)
        for k in range(4):
            buf[byte0 + k] ^= np.uint8(0x80)


def unpack_cache(cache: np.ndarray, bK: np.ndarray, bV: np.ndarray, n: int):
    """Inverse of pack_cache for the first n token slots: (codesK, codesV) [n, d]."""
    d = len(bK)
    BK, BV = record_bits(bK), record_bits(bV)
    kbits = 64 * BK
    tbits = 64 * (BK + BV)
    n_tiles = (n + TILE - 1) // TILE
    raw = np.array(np.asarray(cache, np.uint8)[: n_tiles * tbits // 8])
    _flip_key_bytes(raw, n, BK, tbits // 8)
    bitarr = np.unpackbits(raw, bitorder="little")
    tok = np.arange(n)
    tile = tok // TILE
    slot = tok % TILE
    cK = np.zeros((n, d), np.int64)
    cV = np.zeros((n, len(bV)), np.int64)
    off = 0
    for (j, w, e) in pieces(bK):
        rbit = off + np.arange(w)[None, :]
        pos = tile[:, None] * tbits + 32 * ((rbit // 32) * 64 + slot[:, None]) + rbit % 32
        weights = (1 << np.arange(w))[None, :]
        cK[:, j] += ((bitarr[pos].astype(np.int64) * weights).sum(axis=1)) << e
        off += w
    off = 0
    for (j, w, e) in pieces(bV):
        per_word = 32 // w
        r = slot // per_word
        k = slot % per_word
        inword = 8 * (k % 4) + w * (k // 4)
        base = tile * tbits + kbits + 64 * off + 32 * r + inword
        pos = base[:, None] + np.arange(w)[None, :]
        weights = (1 << np.arange(w))[None, :]
        cV[:, j] += ((bitarr[pos].astype(np.int64) * weights).sum(axis=1)) << e
        off += w
    return cK, cV


def encode_cache(K: np.ndarray, V: np.ndarray, cb, n_tiles: int | None = None):
    """Whole encoder for one (layer, seq, head): transform, quantize, pack.
    Returns (cache bytes, codesK, codesV)."""
    cKf = transform_coeffs(K, cb.muK, cb.UK)
    cVf = transform_coeffs(V, cb.muV, cb.UV)
    codesK = quantize(cKf, cb.inv_step("K"), cb.bK)
    codesV = quantize(cVf, cb.inv_step("V"), cb.bV)
    return pack_cache(codesK, codesV, cb.bK, cb.bV, n_tiles), codesK, codesV
