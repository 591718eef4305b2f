"""Pins of the oracle's quantizer, layout and attention (no GPU)."""
import math

import numpy as np
import pytest

import oracle
import synth
from util import LAYOUT_KEY_ALIGN


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
def _place_by_bits(bits):
    """Independent statement of the field placement: each record byte is a list of 8 bit
    owners (chan, code bit) filled from bit 0; returns {(byte, pos): (chan, width, shift)}
    with bytes renumbered by decreasing field count."""
    nbytes = sum(bits) // 8
    owner = [[None] * 8 for _ in range(nbytes)]

    def free(q):
        return owner[q].count(None)

    def put(q, j, e, w):
        p = 8 - free(q)
        for i in range(w):
            owner[q][p + i] = (j, e + i)

    order = sorted([j for j in range(len(bits)) if bits[j]], key=lambda j: (-bits[j], j))
    left = []
    for j in order:
        for q in range(nbytes):
            if free(q) >= bits[j]:
                put(q, j, 0, bits[j])
                break
        else:
            left.append(j)
    for j in left:
        done = 0
        for q in range(nbytes):
            take = min(free(q), bits[j] - done)
            if take > 0:
                put(q, j, done, take)
                done += take
    # runs of one channel's consecutive code bits inside a byte are the fields
    per_byte = []
    for q in range(nbytes):
        runs, p = {}, 0
        while p < 8:
            j, e = owner[q][p]
            w = 1
            while p + w < 8 and owner[q][p + w] == (j, e + w):
                w += 1
            runs[p] = (j, w, e)
            p += w
        per_byte.append(runs)
    new_order = sorted(range(nbytes), key=lambda q: (-len(per_byte[q]), q))
    return {(i, p): f for i, q in enumerate(new_order) for p, f in per_byte[q].items()}


def _pack_bit_by_bit(codesK, codesV, bK, bV):
    """Independent writer of the layout: one bit at a time with Python ints."""
    BK, BV = int(sum(bK)), int(sum(bV))
    n = len(codesK)
    n_tiles = (n + 63) // 64
    tbytes = 8 * (BK + BV)
    buf = [0] * (n_tiles * tbytes)
    for t in range(n):
        tile, s = divmod(t, 64)
        for codes, bits, is_key in ((codesK, bK, True), (codesV, bV, False)):
            rec = [0] * (sum(bits) // 8)
            for (q, p), (j, w, e) in _place_by_bits(list(bits)).items():
                for i in range(w):
                    if (codes[t][j] >> (e + i)) & 1:
                        rec[q] |= 1 << (p + i)
            for q, byte in enumerate(rec):
                if is_key:  # record word q // 4 of slot s is block word 64 (q // 4) + s
                    at = tile * tbytes + 4 * (64 * (q // 4) + s) + q % 4
                else:  # record byte q of slot s is value-block byte 64 q + s
                    at = tile * tbytes + 8 * BK + 64 * q + s
                buf[at] = byte ^ 0x80  # written bytes carry bit 7 inverted
    return np.array(buf, np.uint8)


def test_field_placement_worked_examples():
    # 16 bits: five 3-bit channels and a 1-bit one.  ch0, ch1 fill byte 0 to 6 bits and
    # ch2, ch3 byte 1; ch4 fits nowhere; ch5 takes byte 0 bit 6; ch4 is then cut into
    # its bit 0 at byte 0 bit 7 and its bits 1..2 at byte 1 bits 6..7.
    assert oracle.fields(np.array([3, 3, 3, 3, 3, 1])) == [
        (0, 3, 0, 0, 0), (1, 3, 0, 0, 3), (5, 1, 0, 0, 6), (4, 1, 0, 0, 7),
        (2, 3, 0, 1, 0), (3, 3, 0, 1, 3), (4, 2, 1, 1, 6)]
    # an 8-bit channel fills byte 0; the four 2-bit channels fill byte 1, which has more
    # fields and is renumbered first
    assert oracle.fields(np.array([8, 2, 2, 2, 2])) == [
        (1, 2, 0, 0, 0), (2, 2, 0, 0, 2), (3, 2, 0, 0, 4), (4, 2, 0, 0, 6), (0, 8, 0, 1, 0)]
    # uncoded channels take no field
    assert oracle.fields(np.array([0, 4, 0, 4])) == [(1, 4, 0, 0, 0), (3, 4, 0, 0, 4)]


@pytest.mark.parametrize("seed", range(40))
def test_field_placement_invariants(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([8, 64, 128]))
    bits = rng.integers(0, 9, d)
    while bits.sum() % 8:  # whole bytes: drop bits from random coded channels
        bits[rng.choice(np.flatnonzero(bits))] -= 1
    f = oracle.fields(bits)
    nbytes = int(bits.sum()) // 8
    used = np.zeros((nbytes, 8), int)
    cover = {j: np.zeros(int(bits[j]), int) for j in range(d)}
    for (j, w, e, q, p) in f:
        assert w >= 1 and 0 <= p and p + w <= 8 and 0 <= q < nbytes
        used[q, p:p + w] += 1
        cover[j][e:e + w] += 1
    assert (used == 1).all()  # every record bit belongs to exactly one field
    assert all((c == 1).all() for c in cover.values())  # every code bit stored once
    counts = np.bincount([x[3] for x in f], minlength=nbytes)
    assert (np.diff(counts) <= 0).all()  # bytes ordered by decreasing field count
    assert f == sorted(f, key=lambda x: (x[3], x[4]))
    # the same placement from the bit-owner statement
    assert {(q, p): (j, w, e) for (j, w, e, q, p) in f} == _place_by_bits(bits.tolist())


@pytest.mark.parametrize("n", [1, 63, 64, 70, 130])
def test_pack_matches_bit_by_bit_writer(n):
    rng = np.random.default_rng(n)
    bK = np.array([8, 0, 7, 3, 1, 2, 5, 6, 4, 8, 7, 5, 8])  # 64 bits: two record words
    bV = np.array([1, 2, 0, 4, 8, 3, 7, 5, 6, 3, 1])  # 40 bits
    cK = np.stack([rng.integers(0, 1 << b, n) if b else np.zeros(n, int) for b in bK], 1)
    cV = np.stack([rng.integers(0, 1 << b, n) if b else np.zeros(n, int) for b in bV], 1)
    got = oracle.pack_cache(cK, cV, bK, bV)
    ref = _pack_bit_by_bit(cK.tolist(), cV.tolist(), bK.tolist(), bV.tolist())
    assert got.nbytes == ((n + 63) // 64) * oracle.tile_bytes(bK, bV)
    assert np.array_equal(got, ref)
    uK, uV = oracle.unpack_cache(got, bK, bV, n)
    assert np.array_equal(uK, cK) and np.array_equal(uV, cV)


def test_tile_size_and_zero_padding():
    bK = np.array([8, 8, 8, 8])  # one record word, channel q in byte q
    bV = np.array([4, 2, 2])     # one byte: ch0 bits 0..3, ch1 bits 4..5, ch2 bits 6..7
    assert oracle.tile_bytes(bK, bV) == 8 * 40
    cK = np.array([[0x12, 0x34, 0x56, 0x78], [0x9A, 0, 0, 0]])
    cV = np.array([[5, 1, 3], [0, 2, 0]])
    t = oracle.pack_cache(cK, cV, bK, bV)
    assert t.nbytes == 320
    # slot 0's key record = block word 0, slot 1's = block word 1 (bit 7 inverted)
    assert t[0:8].tolist() == [0x92, 0xB4, 0xD6, 0xF8, 0x1A, 0x80, 0x80, 0x80]
    assert t[8:256].sum() == 0
    # value block at byte 256, record byte 0 of slot s at 256 + s:
    # slot 0: 5 | 1 << 4 | 3 << 6 = 0xD5, slot 1: 2 << 4 = 0x20 (bit 7 inverted)
    assert t[256:258].tolist() == [0x55, 0xA0] and t[258:].sum() == 0


def test_two_word_records_are_word_major():
    bK = np.array([8] * 8)  # 64 bits: record words 0 and 1, channel q in byte q
    cK = np.zeros((3, 8), np.int64)
    cK[2, 4] = 0xFF  # slot 2, channel 4 -> record word 1, low byte
    t = oracle.pack_cache(cK, np.zeros((3, 1), np.int64), bK, np.array([8]))
    w = t[:64 * 2 * 4].view(np.uint32).copy()
    for r in range(2):
        w[64 * r:64 * r + 3] ^= np.uint32(0x80808080)  # written slots 0..2: bit 7 inverted
    assert w[64 * 1 + 2] == 0xFF and int(w.sum()) == 0xFF


def test_value_records_are_byte_major():
    bK = np.array([8, 8, 8, 8])
    bV = np.array([8, 8, 8])  # record bytes 0..2 = channels 0..2
    cV = np.zeros((70, 3), np.int64)
    cV[66, 1] = 0x7F  # tile 1, slot 2, record byte 1 -> value-block byte 64 + 2
    t = oracle.pack_cache(np.zeros((70, 4), np.int64), cV, bK, bV)
    tb = oracle.tile_bytes(bK, bV)
    vb = t[tb + 256: tb + 256 + 192].reshape(3, 64)  # tile 1: [record byte][slot]
    want = np.zeros((3, 64), np.uint8)
    want[:, :6] = 0x80  # slots 0..5 are written: zero codes stored with bit 7 inverted
    want[1, 2] = 0x7F ^ 0x80
    assert np.array_equal(vb, want)


def test_masked_fields_read_as_signed_bytes():
    """With bit 7 inverted, masking one field of a stored byte and reading the byte as
    int8 gives field * 2^p, minus 128 exactly when the field ends at bit 7."""
    rng = np.random.default_rng(7)
    bK = np.array([8, 7, 6, 5, 3, 2, 1, 4, 4, 8, 1, 2, 1, 3, 5, 4])  # 64 bits
    bV = np.array([3, 3, 3, 3, 3, 1, 6, 2])  # 24 bits
    n = 64
    cK = np.stack([rng.integers(0, 1 << b, n) for b in bK], 1)
    cV = np.stack([rng.integers(0, 1 << b, n) for b in bV], 1)
    t = oracle.pack_cache(cK, cV, bK, bV)
    kwords = t[:64 * 2 * 4].view(np.uint32).reshape(2, 64)  # [record word][slot]
    vbytes = t[512:512 + 64 * 3].reshape(3, 64)             # [record byte][slot]
    for codes, bits, raw_of in ((cK, bK, lambda q: (kwords[q // 4] >> np.uint32(8 * (q % 4))) & np.uint32(0xFF)),
                                (cV, bV, lambda q: vbytes[q].astype(np.uint32))):
        for (j, w, e, q, p) in oracle.fields(bits):
            field = (codes[:, j] >> e) & ((1 << w) - 1)
            got = (raw_of(q) & np.uint32(((1 << w) - 1) << p)).astype(np.uint8).view(np.int8).astype(np.int64)
            assert np.array_equal(got, field * (1 << p) - (128 if p + w == 8 else 0)), (j, w, e, q, p)


def test_record_bits_must_be_whole_words_and_bytes():
    with pytest.raises(ValueError):  # 5 key bits
        oracle.pack_cache(np.zeros((1, 2), np.int64), np.zeros((1, 1), np.int64), np.array([3, 2]), np.array([8]))
    with pytest.raises(ValueError):  # 4 value bits
        oracle.pack_cache(np.zeros((1, 4), np.int64), np.zeros((1, 1), np.int64), np.array([8, 8, 8, 8]),
                          np.array([4]))


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
    cb = oracle.build_head_codebook(st, w.avg_bits, key_align=LAYOUT_KEY_ALIGN)
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
    cb = oracle.build_head_codebook(st, w.avg_bits, key_align=LAYOUT_KEY_ALIGN)
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
