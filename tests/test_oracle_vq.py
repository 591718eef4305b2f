"""Pins of the oracle's vector quantization of key coefficients (oracle.vq) against
textbook values, closed forms and brute force."""
import math

import numpy as np
import pytest

import oracle
from oracle import vq


# Max (1960), "Quantizing for minimum distortion", table of optimum non-uniform quantizers
# for a unit-variance Gaussian: positive output levels and mean squared error.
MAX_1960 = {
    2: ([0.7980], 0.3634),
    4: ([0.4528, 1.510], 0.1175),
}


@pytest.mark.parametrize("K", [2, 4])
def test_lloyd_reproduces_max_gaussian_quantizers(K):
    rng = np.random.default_rng(1960 + K)
    y = rng.standard_normal((200_000, 1))
    code = np.sort(vq.lloyd(y, y[:K], 150)[:, 0])
    levels, mse = MAX_1960[K]
    np.testing.assert_allclose(code[K // 2:], levels, atol=0.012)
    np.testing.assert_allclose(code[:K // 2], -np.array(levels[::-1]), atol=0.012)
    a = vq.nearest(y, code[:, None])
    assert abs(float(((y[:, 0] - code[a]) ** 2).mean()) - mse) < 0.03 * mse


def test_lloyd_two_levels_closed_form():
    """Two cells of a symmetric density split at 0; each level is E[|X|] = sqrt(2/pi)."""
    rng = np.random.default_rng(7)
    y = rng.standard_normal((400_000, 1))
    code = np.sort(vq.lloyd(y, np.array([[-0.1], [0.3]]), 30)[:, 0])
    np.testing.assert_allclose(code, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=5e-3)


def test_lloyd_reaches_a_fixed_point():
    """After convergence every codeword is the mean of its cell and every sample sits in
    the cell of its nearest codeword (the two Lloyd conditions)."""
    rng = np.random.default_rng(3)
    y = rng.standard_normal((3000, 4)) * np.array([2.0, 1.0, 0.5, 0.25])
    code = vq.lloyd(y, y[:16], 300)
    a = vq.nearest(y, code)
    for k in range(16):
        cell = y[a == k]
        assert cell.shape[0] > 0
        np.testing.assert_allclose(code[k], cell.mean(axis=0), atol=1e-12)
    again = vq.lloyd(y, code, 1)
    np.testing.assert_array_equal(again, code)


def test_lloyd_empty_cell_keeps_its_codeword():
    y = np.array([[0.0], [0.1], [1.0], [1.1]])
    code = vq.lloyd(y, np.array([[0.0], [1.0], [50.0]]), 3)
    np.testing.assert_allclose(code[:, 0], [0.05, 1.05, 50.0])


def test_vq_beats_scalar_and_respects_the_shannon_bound():
    """A 256-word codebook on 4-D unit Gaussians (2 bits per dimension) does better than
    the best scalar 4-level quantizer (Max: 0.1175) and worse than the rate-distortion
    bound 2^-4 = 0.0625."""
    rng = np.random.default_rng(11)
    normals = rng.standard_normal((16384, 4))
    cb = oracle.group_codebooks(np.ones(4), np.array([[0, 1, 2, 3]]), normals, 25)[0]
    test = rng.standard_normal((20000, 4))
    mse = float(((test - cb[vq.nearest(test, cb)]) ** 2).mean())
    assert 0.0625 < mse < 0.1175 * 0.95, mse


def test_group_codebook_scales_with_the_weights():
    """The training points of a group are the draws scaled by sqrt(x_j): for weights that
    are a common multiple c of the unit ones the codebook is sqrt(c) times the unit one."""
    rng = np.random.default_rng(5)
    normals = rng.standard_normal((2048, 4))
    g = np.array([[0, 1, 2, 3]])
    a = oracle.group_codebooks(np.ones(4), g, normals, 8)
    b = oracle.group_codebooks(np.full(4, 9.0), g, normals, 8)
    np.testing.assert_allclose(b, 3.0 * a, rtol=1e-12, atol=1e-12)


def test_coded_channels_are_the_largest_weights():
    x = np.array([5.0, 1.0, 3.0, 3.0, 0.5, 9.0, 2.0, 3.0])
    np.testing.assert_array_equal(vq.coded_key_channels(x, 1), [0, 2, 3, 5])
    with pytest.raises(ValueError):
        vq.coded_key_channels(x, 3)


def test_equal_volume_groups_exact_partition():
    """Weights 2^3, 2^2, 2^1, 2^0 repeated: the equal-volume partition puts one of each in
    every group, and the greedy rule finds it."""
    n_g = 8
    x = np.tile(2.0 ** np.array([3, 2, 1, 0]), n_g)
    groups = oracle.equal_volume_groups(x, n_g)
    assert sorted(groups.ravel().tolist()) == list(range(4 * n_g))
    lv = oracle.group_log_volumes(x, groups)
    np.testing.assert_allclose(lv, lv[0], atol=1e-12)
    for row in groups:
        assert sorted((x[row]).tolist()) == [1.0, 2.0, 4.0, 8.0]


def _highres_ratio(x, groups, bits_per_group=8):
    """High-resolution distortion of equal-size codebooks over the groups divided by the
    variable-rate optimum with the same total bits (both up to the same constant)."""
    m = groups.shape[1]
    fixed = sum(m * np.exp(np.log(x[g]).mean()) * 2.0 ** (-2 * bits_per_group / m) for g in groups)
    n = groups.size
    allx = x[groups.ravel()]
    opt = n * np.exp(np.log(allx).mean()) * 2.0 ** (-2 * bits_per_group * len(groups) / n)
    return fixed / opt


def test_equal_volume_groups_reach_the_variable_rate_optimum():
    """Closed form: equal-size codebooks match the variable-rate optimum iff the group
    volumes are equal (AM-GM); on a decaying spectrum the greedy grouping comes within
    0.5 % of it, where grouping consecutive coefficients loses a factor of several."""
    n_g = 32
    x = np.arange(1, 129, dtype=np.float64) ** -1.5
    groups = oracle.equal_volume_groups(x, n_g)
    assert sorted(groups.ravel().tolist()) == list(range(128))
    assert all(len(set(r)) == 4 for r in groups)
    good = _highres_ratio(x, groups)
    naive = _highres_ratio(x, np.arange(128).reshape(n_g, 4))
    assert 1.0 - 1e-12 <= good < 1.005, good
    assert naive > 3.0, naive


def test_equal_volume_groups_brute_force_tiny():
    """d = 8 in two groups of four: the greedy partition's volume spread is within the
    largest single log-weight gap of the best of all 35 partitions, and the two largest
    weights open different groups."""
    import itertools
    rng = np.random.default_rng(2)
    for _ in range(20):
        x = np.exp(rng.normal(size=8) * 2)
        groups = oracle.equal_volume_groups(x, 2)
        lv = oracle.group_log_volumes(x, groups)
        spread = abs(lv[0] - lv[1])
        best = min(abs(np.log(x[list(a)]).sum() - np.log(x[[j for j in range(8) if j not in a]]).sum())
                   for a in itertools.combinations(range(8), 4))
        lx = np.sort(np.log(x))
        assert spread <= best + (lx[-1] - lx[0]) + 1e-12
        top2 = np.argsort(-x)[:2]
        assert not any(top2[0] in r and top2[1] in r for r in groups.tolist())


def test_vq_encode_is_the_nearest_codeword():
    """fp32 index = fp64 nearest codeword of u = c s, except on near-ties (relative
    distance gap below 1e-5)."""
    rng = np.random.default_rng(9)
    d, n_g = 16, 2
    groups = np.array([[0, 3, 5, 9], [1, 2, 12, 15]])
    scale = rng.uniform(0.5, 2.0, d).astype(np.float32)
    cent = rng.standard_normal((n_g, 256, 4))
    c = rng.standard_normal((4000, d)).astype(np.float32) * 1.5
    idx = oracle.vq_encode(c, groups, scale, cent.astype(np.float32))
    for g in range(n_g):
        u = c[:, groups[g]].astype(np.float64) * scale[groups[g]].astype(np.float64)
        d2 = ((u[:, None, :] - cent[g].astype(np.float32).astype(np.float64)[None]) ** 2).sum(-1)
        ref = d2.argmin(1)
        bad = idx[:, g] != ref
        gap = (d2[np.arange(len(u)), idx[:, g]] - d2[np.arange(len(u)), ref]) / d2[np.arange(len(u)), ref]
        assert np.all(gap[bad] < 1e-5)
        assert bad.mean() < 1e-3


def test_vq_round_trip_of_codewords():
    """A coefficient vector at a codeword (c = z / s) encodes to that codeword's index,
    and dequantizes to it."""
    rng = np.random.default_rng(4)
    d = 8
    groups = np.array([[0, 2, 4, 6], [1, 3, 5, 7]])
    scale = rng.uniform(0.5, 2.0, d).astype(np.float32)
    cent = rng.standard_normal((2, 256, 4)).astype(np.float32)
    pick = rng.integers(0, 256, (50, 2))
    c = np.zeros((50, d))
    for g in range(2):
        c[:, groups[g]] = cent[g][pick[:, g]] / scale[groups[g]].astype(np.float64)
    idx = oracle.vq_encode(c.astype(np.float32), groups, scale, cent)
    np.testing.assert_array_equal(idx, pick)
    chat = oracle.vq_dequantize(idx, groups, scale, cent, d)
    np.testing.assert_allclose(chat, c, rtol=1e-6, atol=1e-7)


def test_vq_special_cases():
    groups = np.array([[0, 1, 2, 3]])
    cent = np.zeros((1, 256, 4), np.float32)
    cent[0, :, 0] = np.arange(256)              # codewords on one axis, all other equal
    scale = np.ones(4, np.float32)
    c = np.array([[300.0, 0, 0, 0], [-5.0, 0, 0, 0], [7.5, 0, 0, 0]], np.float32)
    np.testing.assert_array_equal(oracle.vq_encode(c, groups, scale, cent)[:, 0], [255, 0, 7])
    cent[0, 3] = cent[0, 9]                     # duplicate codewords: the lower index wins
    c = cent[0, 9][None, :].astype(np.float32)
    assert oracle.vq_encode(c, groups, scale, cent)[0, 0] == 3
    with pytest.raises(ValueError):
        oracle.vq_encode(np.array([[np.nan, 0, 0, 0]], np.float32), groups, scale, cent)


def test_vq_record_pack_round_trip():
    """Key records of n_g one-byte pseudo-channels: byte g holds group g's index."""
    rng = np.random.default_rng(6)
    n_g = 8
    bits = np.full(n_g, 8)
    f = oracle.fields(bits)
    assert [(j, w, e, q, p) for (j, w, e, q, p) in f] == [(g, 8, 0, g, 0) for g in range(n_g)]
    idx = rng.integers(0, 256, (130, n_g))
    bV = np.array([2] * 16)
    cv = rng.integers(0, 4, (130, 16))
    cache = oracle.pack_cache(idx, cv, bits, bV)
    a, b = oracle.unpack_cache(cache, bits, bV, 130)
    np.testing.assert_array_equal(a, idx)
    np.testing.assert_array_equal(b, cv)
    # slot 5 of tile 0: record byte g sits at 4 (64 (g // 4) + 5) + g % 4, bit 7 inverted
    for g in range(n_g):
        assert cache[4 * (64 * (g // 4) + 5) + g % 4] == (idx[5, g] ^ 0x80)


def test_vq_keys_reduce_attention_error():
    """The abstract's claim at 2 bits per element, on the oracle: with the attention-optimal
    key transform, vector-quantized keys give a clearly smaller attention error than the
    scalar quantizer at the same bits, and that pair is the best of the four.  (The codebooks
    need enough training draws: with 4 draws per codeword they overfit and lose to the
    scalar quantizer.)"""
    import synth
    w = synth.WORKLOADS["vq_tiny"]
    err = {}
    for kt in ("klt", "nova"):
        for kq in ("scalar", "vq"):
            e = []
            for layer in range(2):
                hm = synth.head_model(w, layer, 0)
                K, V, Q = synth.calibration_samples(w, hm, layer, 0)
                cb = oracle.build_head_codebook(oracle.head_stats(K, V, Q), w.avg_bits, joint=False,
                                                key_transform=kt, key_quantizer=kq,
                                                vq_normals=synth.vq_normals(w, layer, 2048), vq_iters=15)
                Kc, Vc = synth.cache_kv(w, hm, layer, 0, 0, 512)
                kf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Kc))
                vf = synth.bf16_bits_to_f64(synth.to_bf16_bits(Vc))
                q = synth.decode_queries(w, [hm], layer, 0)
                cache, _, _ = oracle.encode_cache(kf, vf, cb)
                o = oracle.decode_attention(cache, cb, q, 512)
                e.append(((o - oracle.attention(q, kf, vf)) ** 2).sum(axis=1).mean())
            err[(kt, kq)] = float(np.mean(e))
    assert err[("nova", "vq")] < 0.8 * err[("nova", "scalar")], err
    assert err[("nova", "vq")] == min(err.values()), err
