"""Pins of the oracle's quantizer, layout and attention (no GPU)."""
import math

import numpy as np
import pytest

import oracle
import synth


# ---------------------------------------------------------------- quantizer
def test_reconstruction_points_round_trip():
    bits = np.array([1, 2, 3, 5, 8, 0])
    step = np.array([0.9, 0.5, 0.25, 0.1, 0.01, 0.0], np.float32)
    inv = np.where(step > 0, 1.0 / np.maximum(step, 1e-30), 0).astype(np.float32)
    rows = []
    for c in range(256):
        rows.append([min(c, (1 << b) - 1) if b else 0 for b in bits])
    codes = np.array(rows)
    chat = oracle.dequantize(codes, bits, step).astype(np.float32)
    back = oracle.quantize(chat, inv, bits)
    assert np.array_equal(back, codes)


def test_quantizer_special_values():
    bits = np.array([1, 3, 8])
    inv = np.array([2.0, 4.0, 100.0], np.float32)
    z = oracle.quantize(np.zeros((1, 3), np.float32), inv, bits)
    assert z.tolist() == [[1, 4, 128]]
    big = oracle.quantize(np.array([[1e6, 1e6, 1e6], [-1e6, -1e6, -1e6]], np.float32), inv, bits)
    assert big.tolist() == [[1, 7, 255], [0, 0, 0]]
    # cell boundaries belong to the upper cell
    b = oracle.quantize(np.array([[0.5, 0.25, 0.01]], np.float32), inv, bits)
    assert b.tolist() == [[1, 5, 129]]
    with pytest.raises(ValueError):
        oracle.quantize(np.array([[np.nan, 0, 0]], np.float32), inv, bits)


# ---------------------------------------------------------------- layout
def _pack_bit_by_bit(codesK, codesV, bK, bV):
    """Independent writer of the layout: one bit at a time with Python ints."""
    BK, BV = int(sum(bK)), int(sum(bV))
    n = len(codesK)
    n_tiles = (n + 63) // 64
    tile_bits = 64 * (BK + BV)
    buf = [0] * (n_tiles * tile_bits // 8)

    def put(bit_index, v):
        if v:
            buf[bit_index // 8] |= 1 << (bit_index % 8)

    def plist(bits):
        # widths 4, 2, 1; a channel's pieces taken greedily from its top bit
        per = {}
        for j in range(len(bits)):
            rem, lst = bits[j], []
            while rem >= 4:
                rem -= 4
                lst.append((4, rem))
            if rem >= 2:
                rem -= 2
                lst.append((2, rem))
            if rem == 1:
                lst.append((1, 0))
            per[j] = lst
        out = []
        for w in (4, 2, 1):
            for j in range(len(bits)):
                for (pw, e) in per[j]:
                    if pw == w:
                        out.append((j, w, e))
        return out

    for t in range(n):
        tile, s = divmod(t, 64)
        base = tile * tile_bits
        off = 0
        for (j, w, e) in plist(bK):
            val = (codesK[t][j] >> e) & ((1 << w) - 1)
            for i in range(w):
                rb = off + i  # record bit; record word r of slot s is block word 64 r + s
                put(base + 32 * (64 * (rb // 32) + s) + rb % 32, (val >> i) & 1)
            off += w
        off = 0
        for (j, w, e) in plist(bV):
            val = (codesV[t][j] >> e) & ((1 << w) - 1)
            per = 32 // w
            r, k = divmod(s, per)
            pos = 64 * BK + 64 * off + 32 * r + 8 * (k % 4) + w * (k // 4)
            for i in range(w):
                put(base + pos + i, (val >> i) & 1)
            off += w
    # the key-record bytes of written slots are stored with bit 7 inverted
    for t in range(n):
        tile, s = divmod(t, 64)
        for r in range(BK // 32):
            for k in range(4):
                buf[tile * tile_bits // 8 + 4 * (64 * r + s) + k] ^= 0x80
    return np.array(buf, np.uint8)


@pytest.mark.parametrize("n", [1, 63, 64, 70, 130])
def test_pack_matches_bit_by_bit_writer(n):
    rng = np.random.default_rng(n)
    bK = np.array([8, 0, 7, 3, 1, 2, 5, 6, 4, 8, 7, 5, 8])  # 64 bits: two record words
    bV = np.array([1, 2, 0, 4, 8, 3, 7, 5, 6])
    cK = np.stack([rng.integers(0, 1 << b, n) if b else np.zeros(n, int) for b in bK], 1)
    cV = np.stack([rng.integers(0, 1 << b, n) if b else np.zeros(n, int) for b in bV], 1)
    got = oracle.pack_cache(cK, cV, bK, bV)
    ref = _pack_bit_by_bit(cK.tolist(), cV.tolist(), bK.tolist(), bV.tolist())
    assert got.nbytes == ((n + 63) // 64) * oracle.tile_bytes(bK, bV)
    assert np.array_equal(got, ref)
    uK, uV = oracle.unpack_cache(got, bK, bV, n)
    assert np.array_equal(uK, cK) and np.array_equal(uV, cV)


def test_tile_size_and_zero_padding():
    bK = np.array([8, 8, 8, 8])  # 32 bits: one record word of eight nibbles
    bV = np.array([1, 2])
    assert oracle.tile_bytes(bK, bV) == 8 * 35
    cK = np.array([[0x12, 0x34, 0x56, 0x78], [0x9A, 0, 0, 0]])
    cV = np.array([[1, 3], [0, 2]])
    t = oracle.pack_cache(cK, cV, bK, bV)
    k = t[:256].copy()
    k[:8] ^= 0x80  # the two written slots' key records are stored with bit 7 inverted
    # slot 0's record word = block word 0: nibbles hi/lo of each code in channel order
    assert k[0:4].tolist() == [0x21, 0x43, 0x65, 0x87]
    # slot 1's record word = block word 1
    assert k[4:8].tolist() == [0xA9, 0, 0, 0]
    assert k[8:256].sum() == 0
    # V block at byte 256 (not inverted): (ch1 w2) slab first: slot0 = 3 at bits 0..1,
    # slot1 = 2 at bits 8..9; (ch0 w1) slab at bit 64*2: slot0 = 1 at bit 0
    assert t[256] == 0b11 and t[257] == 0b10 and t[256 + 16] == 1
    assert int(t[256:].astype(np.int64).sum()) == 3 + 2 + 1
    assert int(k.astype(np.int64).sum()) == 0x21 + 0x43 + 0x65 + 0x87 + 0xA9


def test_two_word_records_are_word_major():
    bK = np.array([8] * 8)  # 64 bits: record words 0 and 1
    cK = np.zeros((3, 8), np.int64)
    cK[2, 4] = 0xFF  # slot 2, channel 4 -> record word 1, low byte
    t = oracle.pack_cache(cK, np.zeros((3, 1), np.int64), bK, np.array([2]))
    w = t[:64 * 2 * 4].view(np.uint32).copy()
    for r in range(2):
        w[64 * r:64 * r + 3] ^= np.uint32(0x80808080)  # written slots 0..2: bit 7 inverted
    assert w[64 * 1 + 2] == 0xFF and int(w.sum()) == 0xFF


def test_eight_bit_code_is_two_nibbles():
    bK = np.array([8, 8, 8, 8])
    bV = np.array([2, 1])
    assert oracle.pieces(bK)[:2] == [(0, 4, 4), (0, 4, 0)]
    t = oracle.pack_cache(np.array([[0xA5, 0, 0, 0]]), np.array([[2, 1]]), bK, bV)
    # record: high nibble 0xA at bits 0..3, low nibble 0x5 at bits 4..7 (stored with bit 7
    # inverted)
    assert t[0] == 0x5A ^ 0x80


def test_masked_key_fields_read_as_signed_bytes():
    """With bit 7 of key bytes inverted, masking one field of a byte and reading the byte as
    int8 gives field * 2^p, minus 128 exactly when the field ends at bit 7."""
    rng = np.random.default_rng(7)
    bK = np.array([8, 7, 6, 5, 3, 2, 1, 4, 4, 8, 1, 2, 1, 3, 5, 4])  # 64 bits
    n = 64
    cK = np.stack([rng.integers(0, 1 << b, n) for b in bK], 1)
    t = oracle.pack_cache(cK, np.zeros((n, 1), np.int64), bK, np.array([2]))
    words = t[:64 * 2 * 4].view(np.uint32).reshape(2, 64)  # [record word][slot]
    off = 0
    for (j, w, e) in oracle.pieces(bK):
        r, bit = divmod(off, 32)
        byte, p = divmod(bit, 8)
        field = (cK[:, j] >> e) & ((1 << w) - 1)
        mask = ((1 << w) - 1) << p
        raw = (words[r] >> np.uint32(8 * byte)) & np.uint32(0xFF)
        got = (raw & np.uint32(mask)).astype(np.uint8).view(np.int8).astype(np.int64)
        want = field * (1 << p) - (128 if p + w == 8 else 0)
        assert np.array_equal(got, want), (j, w, e, p)
        off += w


def test_key_bits_must_fill_words():
    with pytest.raises(ValueError):
        oracle.pack_cache(np.zeros((1, 2), np.int64), np.zeros((1, 1), np.int64), np.array([3, 2]), np.array([1]))


# ---------------------------------------------------------------- attention
def test_attention_brute_force():
    rng = np.random.default_rng(7)
    L, d = 6, 4
    q = rng.standard_normal(d)
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    s = [sum(q[j] * K[i][j] for j in range(d)) / math.sqrt(d) for i in range(L)]
    z = sum(math.exp(x) for x in s)
    ref = [sum(math.exp(s[i]) / z * V[i][j] for i in range(L)) for j in range(d)]
    assert np.allclose(oracle.attention(q, K, V)[0], ref, rtol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    d = 8
    V = rng.standard_normal((1, d))
    assert np.allclose(oracle.attention(rng.standard_normal(d), rng.standard_normal((1, d)), V)[0], V[0])
    K = np.tile(rng.standard_normal(d), (5, 1))
    V = rng.standard_normal((5, d))
    assert np.allclose(oracle.attention(rng.standard_normal(d), K, V)[0], V.mean(0), rtol=1e-13)


def test_decode_attention_equals_dequantized_attention():
    w = synth.WORKLOADS["tiny"]
    hm = synth.head_model(w, 0, 0)
    st = oracle.head_stats(*synth.calibration_samples(w, hm, 0, 0))
    cb = oracle.build_head_codebook(st, w.avg_bits)
    K, V = synth.cache_kv(w, hm, 0, 0, 0, 100)
    cache, cK, cV = oracle.encode_cache(K, V, cb)
    q = synth.decode_queries(w, [hm], 0, 0)
    o = oracle.decode_attention(cache, cb, q, 100)
    # dequantize each coefficient by hand and rebuild with U
    Kh = np.zeros_like(K)
    Vh = np.zeros_like(V)
    for t in range(100):
        ck = np.array([(cK[t, j] - 2 ** (cb.bK[j] - 1) + 0.5) * float(cb.stepK[j]) if cb.bK[j] else 0.0
                       for j in range(w.d)])
        cv = np.array([(cV[t, j] - 2 ** (cb.bV[j] - 1) + 0.5) * float(cb.stepV[j]) if cb.bV[j] else 0.0
                       for j in range(w.d)])
        Kh[t] = cb.muK + cb.UK @ ck
        Vh[t] = cb.muV + cb.UV @ cv
    assert np.allclose(o, oracle.attention(q, Kh, Vh), rtol=1e-12, atol=1e-14)
    # the coded cache stays close to the exact attention
    ex = oracle.attention(q, K, V)
    assert np.abs(o - ex).max() / np.abs(ex).max() < 0.2


def test_reconstruction_error_within_half_step():
    w = synth.WORKLOADS["tiny"]
    hm = synth.head_model(w, 0, 0)
    st = oracle.head_stats(*synth.calibration_samples(w, hm, 0, 0))
    cb = oracle.build_head_codebook(st, w.avg_bits)
    K, V = synth.cache_kv(w, hm, 0, 0, 0, 256)
    c = oracle.transform_coeffs(K, cb.muK, cb.UK)
    codes = oracle.quantize(c, cb.inv_step("K"), cb.bK)
    ch = oracle.dequantize(codes, cb.bK, cb.stepK)
    half = (1 << np.maximum(cb.bK - 1, 0)) * cb.stepK.astype(np.float64)
    inside = (np.abs(c) < half[None, :] * 0.999) & (cb.bK[None, :] > 0)
    err = np.abs(ch - c)[inside]
    assert np.all(err <= 0.5 * np.broadcast_to(cb.stepK, c.shape)[inside] * (1 + 1e-6))


def test_compression_arithmetic():
    for rbar, d, ratio in ((2.75, 128, 16 / 2.75), (2.0, 128, 8.0), (3.0, 64, 16 / 3.0)):
        B = int(2 * d * rbar)
        assert abs(2 * d * 16 / B - ratio) < 1e-12
