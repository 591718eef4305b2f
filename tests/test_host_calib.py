"""Host calibration of the library against the oracle (no GPU)."""
import os

import numpy as np
import pytest

import oracle
import quantized_attention_klt_amd as q
import synth
from util import LAYOUT_KEY_ALIGN


def _samples(wname, head=0, layer=0):
    w = synth.WORKLOADS[wname]
    hm = synth.head_model(w, layer, head)
    K, V, Q = synth.calibration_samples(w, hm, layer, head)
    return w, K.astype(np.float32), V.astype(np.float32), Q.astype(np.float32)


@pytest.mark.parametrize("wname", ["tiny", "llama_32k"])
def test_stats_match_oracle(wname):
    w, K, V, Q = _samples(wname)
    if wname != "tiny":
        K, V, Q = K[:2048], V[:2048], Q[:256]
    lib = q.stats_from_samples(K, V, Q)
    ref = oracle.head_stats(K.astype(np.float64), V.astype(np.float64), Q.astype(np.float64))
    for k in ("muK", "muV", "SigK", "SigV", "MQ"):
        scale = np.abs(ref[k]).max()
        assert np.abs(lib[k] - ref[k]).max() <= 1e-11 * scale, k
    assert abs(lib["gammaV"] - ref["gammaV"]) <= 1e-12 * ref["gammaV"]


@pytest.mark.parametrize("wname,joint", [("tiny", True), ("llama_32k", True), ("llama_32k", False)])
def test_calibrate_matches_oracle(wname, joint):
    w, K, V, Q = _samples(wname, head=1 if w_name_has_heads(wname) else 0)
    st = oracle.head_stats(K.astype(np.float64), V.astype(np.float64), Q.astype(np.float64))
    cb = q.calibrate([st], w.d, 1, 1, w.group, w.avg_bits, joint=joint)
    ref = oracle.build_head_codebook(st, w.avg_bits, joint=joint, key_align=LAYOUT_KEY_ALIGN)
    h = cb.head(0)
    lm = ref.lamK.max()
    assert np.abs(h["lamK"] - ref.lamK).max() <= 1e-10 * lm
    assert np.abs(h["lamV"] - ref.lamV).max() <= 1e-10 * ref.lamV.max()
    # U agrees where eigenvalues are well separated (the sign rule fixes the sign)
    for U, Ur, lam in ((h["UK"], ref.UK, ref.lamK), (h["UV"], ref.UV, ref.lamV)):
        gap = np.minimum(np.r_[np.inf, -np.diff(lam)], np.r_[-np.diff(lam), np.inf])
        sep = gap > 1e-6 * lam.max()
        assert np.abs(U[:, sep] - Ur[:, sep]).max() < 1e-7
        assert np.abs(U.T @ U - np.eye(w.d)).max() < 1e-12
    assert np.array_equal(h["bK"], ref.bK) and np.array_equal(h["bV"], ref.bV)
    assert h["bK"].sum() + h["bV"].sum() == int(2 * w.d * w.avg_bits)
    assert np.allclose(h["stepK"], ref.stepK, rtol=1e-6) and np.allclose(h["stepV"], ref.stepV, rtol=1e-6)
    assert abs(h["theta"] / ref.theta - 1) < 1e-9
    assert np.allclose(h["xK"], ref.xK, rtol=1e-9) and np.allclose(h["xV"], ref.xV, rtol=1e-9)
    assert cb.total_bits == int(2 * w.d * w.avg_bits) and cb.tile_bytes == 8 * cb.total_bits


@pytest.mark.parametrize("wname", ["tiny", "llama_32k"])
def test_calibrate_attention_optimal_keys_matches_oracle(wname):
    """key_transform = attention-optimal: the library's non-orthogonal key basis,
    coefficient variances, weights, bits and steps against the oracle's."""
    w, K, V, Q = _samples(wname)
    st = oracle.head_stats(K.astype(np.float64), V.astype(np.float64), Q.astype(np.float64))
    cb = q.calibrate([st], w.d, 1, 1, w.group, w.avg_bits, key_transform="nova")
    ref = oracle.build_head_codebook(st, w.avg_bits, key_transform="nova", key_align=LAYOUT_KEY_ALIGN)
    h = cb.head(0)
    assert np.abs(h["lamK"] - ref.lamK).max() <= 1e-10 * ref.lamK.max()
    gap = np.minimum(np.r_[np.inf, -np.diff(ref.lamK)], np.r_[-np.diff(ref.lamK), np.inf])
    sep = gap > 1e-6 * ref.lamK.max()
    assert np.abs(h["UK"][:, sep] - ref.UK[:, sep]).max() < 1e-7 * np.abs(ref.UK).max()
    assert np.abs(h["UK"].T @ h["UK"] - np.eye(w.d)).max() > 1e-3  # not orthogonal
    assert np.array_equal(h["bK"], ref.bK) and np.array_equal(h["bV"], ref.bV)
    assert np.allclose(h["stepK"], ref.stepK, rtol=1e-6) and np.allclose(h["stepV"], ref.stepV, rtol=1e-6)
    assert np.allclose(h["xK"], ref.xK, rtol=1e-9) and np.allclose(h["xV"], ref.xV, rtol=1e-9)


def test_codebook_rejects_singular_key_basis():
    w, ref = _oracle_codebook()
    T = ref.UK.copy()
    T[:, 1] = T[:, 0]
    with pytest.raises(q.AatcError):
        q.codebook_create(ref.d, 1, 1, 4, T[None], ref.UV[None], ref.muK[None], ref.muV[None], ref.bK[None],
                          ref.bV[None], ref.stepK[None], ref.stepV[None])


def w_name_has_heads(wname):
    return synth.WORKLOADS[wname].n_kv > 1


def _oracle_codebook(wname="tiny"):
    w, K, V, Q = _samples(wname)
    st = oracle.head_stats(K.astype(np.float64), V.astype(np.float64), Q.astype(np.float64))
    return w, oracle.build_head_codebook(st, w.avg_bits, key_align=LAYOUT_KEY_ALIGN)


def test_codebook_create_and_persist(tmp_path):
    w, ref = _oracle_codebook()
    cb = q.codebook_create(w.d, 1, 1, w.group, ref.UK[None], ref.UV[None], ref.muK[None], ref.muV[None],
                           ref.bK[None], ref.bV[None], ref.stepK[None], ref.stepV[None])
    assert cb.total_bits == 384
    path = str(tmp_path / "cb.bin")
    cb.save(path)
    cb2 = q.codebook_load(path)
    a, b = cb.head(0), cb2.head(0)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    # a flipped byte is caught by the checksum
    raw = bytearray(open(path, "rb").read())
    raw[100] ^= 1
    open(path, "wb").write(bytes(raw))
    with pytest.raises(q.AatcError) as e:
        q.codebook_load(path)
    assert e.value.status == -10
    with pytest.raises(q.AatcError) as e:
        q.codebook_load(str(tmp_path / "missing.bin"))
    assert e.value.status == -9


def test_error_paths():
    w, ref = _oracle_codebook()
    st = oracle.head_stats(*[x.astype(np.float64) for x in _samples("tiny")[1:]])
    for avg in (2.7, 324 / 128):  # 2*d*avg_bits not an integer; an integer, not a multiple of 8
        with pytest.raises(q.AatcError) as e:
            q.calibrate([st], 64, 1, 1, 4, avg)
        assert e.value.status == -3
    with pytest.raises(q.AatcError) as e:
        q.calibrate([st], 96, 1, 1, 4, 3.0)
    assert e.value.status == -1
    with pytest.raises(q.AatcError) as e:  # eigensolver sweep limit
        q.calibrate([st], 64, 1, 1, 4, 3.0, max_sweeps=1)
    assert e.value.status == -5
    bad = dict(st)
    bad["SigK"] = st["SigK"].copy()
    bad["SigK"][0, 0] = np.nan
    with pytest.raises(q.AatcError) as e:
        q.calibrate([bad], 64, 1, 1, 4, 3.0)
    assert e.value.status == -4
    bK = ref.bK.copy()
    bK[0] += 1  # total bits now odd and different
    with pytest.raises(q.AatcError) as e:
        q.codebook_create(64, 1, 1, 4, ref.UK[None], ref.UV[None], ref.muK[None], ref.muV[None], bK[None],
                          ref.bV[None], ref.stepK[None], ref.stepV[None])
    assert e.value.status == -3
    with pytest.raises(q.AatcError) as e:
        q.stats_from_samples(np.zeros((1, 64)), np.zeros((1, 64)), np.zeros((1, 64)))
    assert e.value.status == -1


def test_multi_head_codebook_geometry():
    w = synth.WORKLOADS["tiny"]
    stats = []
    for layer in range(2):
        for h in range(2):
            hm = synth.head_model(w, layer, h)
            K, V, Q = synth.calibration_samples(w, hm, layer, h)
            stats.append(oracle.head_stats(K, V, Q[:64]))
    cb = q.calibrate(stats, 64, 2, 2, 4, 3.0)
    assert cb.n_layers == 2 and cb.n_kv == 2 and cb.n_heads == 4
    assert cb.cache_bytes(2, 3, 100) == 2 * 3 * 2 * 2 * 3072
    assert cb.device_bytes() > 0


def test_batched_layers_workspace_and_argument_errors():
    """The batched-layers decode's workspace query runs its plans on the host: a layer range
    inside the codebook gives a positive size at least that of the largest per-layer call's
    share, a range outside it or an empty one is INVALID_ARG, and a codebook with
    vector-quantized keys is UNSUPPORTED."""
    w = synth.WORKLOADS["tiny"]
    stats = []
    for layer in range(2):
        for h in range(2):
            hm = synth.head_model(w, layer, h)
            K, V, Q = synth.calibration_samples(w, hm, layer, h)
            stats.append(oracle.head_stats(K, V, Q[:64]))
    cb = q.calibrate(stats, 64, 2, 2, 4, 3.0)
    both = cb.decode_layers_workspace_bytes(0, 2, 3, 100)
    assert both > 0 and cb.decode_layers_workspace_bytes(1, 1, 3, 100) > 0
    for args in ((0, 3, 3, 100), (2, 1, 3, 100), (-1, 1, 3, 100), (0, 0, 3, 100), (0, 2, 0, 100), (0, 2, 3, 0)):
        with pytest.raises(q.AatcError) as e:
            cb.decode_layers_workspace_bytes(*args)
        assert e.value.status == -1  # AATC_ERR_INVALID_ARG
    wv, K, V, Q = _samples("vq_tiny")
    st = oracle.head_stats(K.astype(np.float64), V.astype(np.float64), Q.astype(np.float64))
    cbv = q.calibrate([st], wv.d, 1, 1, wv.group, wv.avg_bits, joint=False, key_quantizer="vq",
                      vq_normals=synth.vq_normals(wv, 0, 512))
    with pytest.raises(q.AatcError) as e:
        cbv.decode_layers_workspace_bytes(0, 1, 1, 512)
    assert e.value.status == -2  # AATC_ERR_UNSUPPORTED


def test_record_fields_match_the_oracle_placement():
    """The library's field placement (what the encoder and decoder use) equals the
    oracle's, for calibrated heads and for random bit vectors."""
    w, ref = _oracle_codebook()
    for seed in range(30):
        rng = np.random.default_rng(100 + seed)
        d = 64 if seed % 2 else 128
        bK = rng.integers(0, 9, d)
        bV = rng.integers(0, 9, d)
        while bK.sum() % 32:
            bK[rng.choice(np.flatnonzero(bK))] -= 1
        while (bK.sum() + bV.sum()) % 8:
            bV[rng.choice(np.flatnonzero(bV))] -= 1
        U = np.eye(d)[None]
        mu = np.zeros((1, d))
        step = lambda b: np.where(b > 0, 0.1, 0.0).astype(np.float32)[None]
        cb = q.codebook_create(d, 1, 1, 1, U, U, mu, mu, bK[None].astype(np.int32), bV[None].astype(np.int32),
                               step(bK), step(bV))
        assert cb.fields(0, 0) == oracle.fields(bK)
        assert cb.fields(0, 1) == oracle.fields(bV)
    cbl = q.codebook_create(ref.d, 1, 1, 4, ref.UK[None], ref.UV[None], ref.muK[None], ref.muV[None],
                            ref.bK[None].astype(np.int32), ref.bV[None].astype(np.int32), ref.stepK[None],
                            ref.stepV[None])
    assert cbl.fields(0, 0) == oracle.fields(ref.bK) and cbl.fields(0, 1) == oracle.fields(ref.bV)


@pytest.mark.parametrize("key_transform", ["klt", "nova"])
def test_calibrate_vector_quantized_keys_matches_oracle(key_transform):
    """key_quantizer = vq: the library's groups, weighted-domain scales, Lloyd codebooks and
    value bits against the oracle's (same statistics, same training draws)."""
    w, K, V, Q = _samples("vq_tiny")
    st = oracle.head_stats(K.astype(np.float64), V.astype(np.float64), Q.astype(np.float64))
    normals = synth.vq_normals(w, 0, 1024)
    cb = q.calibrate([st], w.d, 1, 1, w.group, w.avg_bits, joint=False, key_transform=key_transform,
                     key_quantizer="vq", vq_normals=normals, vq_iters=6)
    ref = oracle.build_head_codebook(st, w.avg_bits, joint=False, key_transform=key_transform,
                                     key_quantizer="vq", vq_normals=normals, vq_iters=6)
    got = cb.vq(0)
    assert got is not None and got["groups"].shape == (w.d * w.avg_bits // 8, 4)
    np.testing.assert_array_equal(got["groups"], ref.vq.groups)
    np.testing.assert_allclose(got["scale32"], ref.vq.scale32, rtol=2e-7)
    np.testing.assert_allclose(got["cent32"], ref.vq.cent32, rtol=1e-5, atol=1e-6 * np.abs(ref.vq.cent).max())
    h = cb.head(0)
    assert not h["bK"].any() and np.array_equal(h["bV"], ref.bV)
    assert cb.total_bits == 2 * int(w.d * w.avg_bits)
    with pytest.raises(q.AatcError):
        cb.save("/dev/null")


def test_vector_quantized_keys_error_paths():
    w, K, V, Q = _samples("vq_tiny")
    st = oracle.head_stats(K.astype(np.float64), V.astype(np.float64), Q.astype(np.float64))
    normals = synth.vq_normals(w, 0, 512)
    for kw in (dict(joint=True, vq_normals=normals), dict(joint=False, vq_normals=None),
               dict(joint=False, vq_normals=normals[:100])):
        with pytest.raises(q.AatcError):
            q.calibrate([st], w.d, 1, 1, w.group, w.avg_bits, key_quantizer="vq", **kw)
    with pytest.raises(q.AatcError):  # more than 2 bits per key element
        q.calibrate([st], w.d, 1, 1, w.group, 3.0, joint=False, key_quantizer="vq", vq_normals=normals)
    ref = oracle.build_head_codebook(st, w.avg_bits, joint=False, key_quantizer="vq", vq_normals=normals,
                                     vq_iters=2)
    args = (w.d, 1, 1, w.group, ref.UK[None], ref.UV[None], ref.muK[None], ref.muV[None])
    good = (ref.vq.groups[None], ref.vq.scale32[None], ref.vq.cent32[None], ref.bV[None], ref.stepV[None])
    cb = q.codebook_create_vq(*args, *good)
    np.testing.assert_array_equal(cb.vq(0)["groups"], ref.vq.groups)
    np.testing.assert_array_equal(cb.vq(0)["cent32"], ref.vq.cent32)
    dup = ref.vq.groups.copy()
    dup[1, 0] = dup[0, 0]
    bad_scale = ref.vq.scale32.copy()
    bad_scale[ref.vq.groups[0, 0]] = 0.0
    bad_cent = ref.vq.cent32.copy()
    bad_cent[0, 0, 0] = np.nan
    for g, sc, ce in ((dup, good[1][0], good[2][0]), (good[0][0], bad_scale, good[2][0]),
                      (good[0][0], good[1][0], bad_cent), (good[0][0][:3], good[1][0], good[2][0][:3])):
        with pytest.raises(q.AatcError):
            q.codebook_create_vq(*args, g[None], sc[None], ce[None], ref.bV[None], ref.stepV[None])


def test_decode_rate_limit_is_reported_before_launch():
    """At d = 128 the decode supports up to 7.5 bits/element: 8 bits on every channel makes
    16 KiB tiles whose ring and operand scratch need more LDS than a CU holds, and the plan
    (computed on the host, before anything is enqueued) says so with UNSUPPORTED.  At d = 64
    the same rate is supported."""
    for d, rate, ok in ((128, 7.5, True), (128, 8.0, False), (64, 8.0, True)):
        w = synth.Workload("limit", 13, d, 1, 4, 1, 1, 512, rate, 2048, 16, "bf16")
        hm = synth.head_model(w, 0, 0)
        K, V, Q = synth.calibration_samples(w, hm, 0, 0)
        ref = oracle.build_head_codebook(oracle.head_stats(K, V, Q), rate, key_align=LAYOUT_KEY_ALIGN)
        cb = q.codebook_create(d, 1, 1, 4, ref.UK[None], ref.UV[None], ref.muK[None], ref.muV[None], ref.bK[None],
                               ref.bV[None], ref.stepK[None], ref.stepV[None])
        if ok:
            assert cb.decode_workspace_bytes(1, 512) > 0
        else:
            with pytest.raises(q.AatcError) as e:
                cb.decode_workspace_bytes(1, 512)
            assert e.value.status == -2  # AATC_ERR_UNSUPPORTED
