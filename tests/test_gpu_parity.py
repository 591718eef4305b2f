"""GPU parity of the HIP path (through the C ABI) against the oracle.

Bars: packed bytes bit-exact when the encoder is fed the oracle's fp32 coefficients;
end-to-end codes differ on at most 1e-4 of coded (token, channel) pairs and by one level;
decode attention within 2e-3 normwise relative error (max over sequences and query heads
of max_j |o - o_ref| / max_j |o_ref|) of the oracle run on the same packed bytes.
"""
import numpy as np
import pytest

import oracle
from util import Case, code_flips, normwise_rel_err

pytestmark = pytest.mark.gpu

FLIP_BAR = 1e-4
ATTN_BAR = 2e-3
# GPU encode + GPU decode against oracle encode + oracle decode: the two caches differ by
# the code flips the encode bar allows (one level at rounding boundaries), so the decode
# bar does not apply; each flip moves one coefficient by one step, a small relative change
# of the (small) attention output.  Bound used for the composition: 1e-2.
END_TO_END_BAR = 1e-2


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _device_codebook(q, torch, case):
    a = case.codebook_arrays()
    if "vq" in a:
        v = a["vq"]
        cb = q.codebook_create_vq(case.d, 1, case.n_kv, case.group, a["UK"], a["UV"], a["muK"], a["muV"],
                                  v["groups"], v["scale32"], v["cent32"], a["bV"], a["stepV"])
    else:
        cb = q.codebook_create(case.d, 1, case.n_kv, case.group, a["UK"], a["UV"], a["muK"], a["muV"], a["bK"],
                               a["bV"], a["stepK"], a["stepV"])
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device="cuda")
    cb.upload(blob)
    return cb, blob


def _new_cache(q, torch, cb, n_seqs, max_tokens):
    t = torch.zeros(cb.cache_bytes(1, n_seqs, max_tokens), dtype=torch.uint8, device="cuda")
    return t, q.make_cache(t, 1, n_seqs, max_tokens)


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("wname,ctx,chunks", [
    ("tiny", 512, [512]),
    ("tiny", 130, [37, 1, 60, 32]),
    ("llama_32k", 200, [200]),
    ("llama_32k", 300, [64, 100, 136]),
])
def test_encode_coeffs_bit_exact(lib, torch, wname, ctx, chunks):
    _log(f"encode_coeffs {wname} ctx={ctx} chunks={chunks}")
    case = Case(wname, ctx, n_calib_q=64)
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, ctx)
    coeffs = torch.from_numpy(case.coeffs(0)).cuda()
    pos = 0
    for n in chunks:
        lib.encode_coeffs(cb, blob, cache, 0, 0, pos, n, coeffs[pos:pos + n])
        pos += n
    torch.cuda.synchronize()
    got = ct.cpu().numpy().reshape(case.n_kv, -1)
    ref, _ = case.oracle_cache()
    assert np.array_equal(got, ref[0])


@pytest.mark.parametrize("wname,ctx,chunks", [
    ("tiny", 512, [512]),
    ("llama_32k", 1000, [1000]),
    ("llama_32k", 333, [1, 127, 205]),
])
def test_encode_end_to_end_flips(lib, torch, wname, ctx, chunks):
    _log(f"encode {wname} ctx={ctx} chunks={chunks}")
    case = Case(wname, ctx, n_calib_q=64)
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, ctx)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    pos = 0
    for n in chunks:
        lib.encode(cb, blob, cache, 0, [0], [pos], n, K[:, pos:pos + n].contiguous(), V[:, pos:pos + n].contiguous())
        pos += n
    torch.cuda.synchronize()
    got = ct.cpu().numpy().reshape(case.n_kv, -1)
    flips = total = worst = 0
    edge = 0.0
    for h, c in enumerate(case.cbs):
        f, t, wst, e = code_flips(got[h], c, ctx, case.kf(0, h), case.vf(0, h))
        flips, total, worst, edge = flips + f, total + t, max(worst, wst), max(edge, e)
    _log(f"  flips {flips}/{total}, worst edge ratio {edge:.3g}")
    assert worst <= 1
    assert edge <= 1.0  # every flipped code sits within the fp32 rounding window of a cell edge
    assert flips <= FLIP_BAR * total


def test_encode_is_deterministic(lib, torch):
    case = Case("llama_32k", 256, n_calib_q=32)
    cb, blob = _device_codebook(lib, torch, case)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    outs = []
    for _ in range(2):
        ct, cache = _new_cache(lib, torch, cb, 1, 256)
        lib.encode(cb, blob, cache, 0, [0], [0], 256, K, V)
        torch.cuda.synchronize()
        outs.append(ct.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def _decode(lib, torch, case, cache_host, lens, max_tokens):
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, case.n_seqs, max_tokens)
    ct.copy_(torch.from_numpy(cache_host.reshape(-1)))
    ids = torch.arange(case.n_seqs, dtype=torch.int32, device="cuda")
    ln = torch.tensor(lens, dtype=torch.int64, device="cuda")
    qd = torch.from_numpy(case.q_bits.view(np.int16)).cuda()
    out = torch.full((case.n_seqs, case.n_q, case.d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(case.n_seqs, max(lens)),), dtype=torch.uint8, device="cuda")
    lib.decode_attention(cb, blob, cache, 0, ids, ln, max(lens), qd, out, ws)
    torch.cuda.synchronize()
    first = out.cpu().numpy()
    # the call leaves the workspace ready: a second call on it gives the same bits
    out.fill_(float("nan"))
    lib.decode_attention(cb, blob, cache, 0, ids, ln, max(lens), qd, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(first, out.cpu().numpy(), equal_nan=True)
    return first


@pytest.mark.parametrize("wname,ctx,n_seqs,lens", [
    ("tiny", 512, 1, [512]),
    ("tiny", 512, 1, [1]),
    ("tiny", 512, 1, [65]),
    ("tiny", 512, 3, [512, 1, 300]),
    ("llama_32k", 1000, 1, [1000]),
    ("llama_32k", 16400, 1, [16400]),
    ("llama_32k", 32768, 1, [32768]),
    ("llama_batch", 700, 3, [700, 64, 129]),
    ("qwen_128k", 2000, 1, [2000]),
])
def test_decode_parity(lib, torch, wname, ctx, n_seqs, lens):
    _log(f"decode {wname} ctx={ctx} lens={lens}")
    case = Case(wname, ctx, n_seqs=n_seqs, n_calib_q=64, lens=lens)
    cache_host, _ = case.oracle_cache()
    got = _decode(lib, torch, case, cache_host, lens, ctx)
    ref = case.oracle_decode(cache_host, lens)
    err = normwise_rel_err(got, ref)
    _log(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_BAR


def test_encode_then_decode_end_to_end(lib, torch):
    """GPU encode followed by GPU decode, against the oracle's own encode and decode."""
    case = Case("llama_32k", 4096, n_calib_q=64)
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, 4096)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    lib.encode(cb, blob, cache, 0, [0], [0], 4096, K, V)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ln = torch.full((1,), 4096, dtype=torch.int64, device="cuda")
    qd = torch.from_numpy(case.q_bits.view(np.int16)).cuda()
    out = torch.empty((1, case.n_q, case.d), dtype=torch.float32, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(1, 4096),), dtype=torch.uint8, device="cuda")
    lib.decode_attention(cb, blob, cache, 0, ids, ln, 4096, qd, out, ws)
    torch.cuda.synchronize()
    ref_cache, _ = case.oracle_cache()
    ref = case.oracle_decode(ref_cache)
    err = normwise_rel_err(out.cpu().numpy(), ref)
    _log(f"  end-to-end rel err {err:.3e}")
    assert err <= END_TO_END_BAR


def test_decode_workspace_reuse_across_shapes(lib, torch):
    """One workspace serves calls of different batch and length in a row."""
    case = Case("llama_batch", 3000, n_seqs=3, n_calib_q=32, lens=[3000, 64, 1290])
    cache_host, _ = case.oracle_cache()
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, case.n_seqs, 3000)
    ct.copy_(torch.from_numpy(cache_host.reshape(-1)))
    qd = torch.from_numpy(case.q_bits.view(np.int16)).cuda()
    ws = torch.zeros((cb.decode_workspace_bytes(3, 3000),), dtype=torch.uint8, device="cuda")
    shapes = [([0, 1, 2], [3000, 64, 1290], 3000), ([2], [1290], 1290), ([1, 0], [64, 700], 700),
              ([0, 1, 2], [3000, 64, 1290], 3000)]
    outs = []
    for ids_l, lens_l, mx in shapes:
        ids = torch.tensor(ids_l, dtype=torch.int32, device="cuda")
        ln = torch.tensor(lens_l, dtype=torch.int64, device="cuda")
        q_sel = qd[torch.tensor(ids_l, device="cuda")].contiguous()
        out = torch.full((len(ids_l), case.n_q, case.d), float("nan"), dtype=torch.float32, device="cuda")
        lib.decode_attention(cb, blob, cache, 0, ids, ln, mx, q_sel, out, ws)
        fresh_ws = torch.zeros((cb.decode_workspace_bytes(len(ids_l), mx),), dtype=torch.uint8, device="cuda")
        fresh = torch.full_like(out, float("nan"))
        lib.decode_attention(cb, blob, cache, 0, ids, ln, mx, q_sel, fresh, fresh_ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), fresh.cpu().numpy())
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[3])


def test_decode_argument_errors(lib, torch):
    case = Case("tiny", 128, n_calib_q=16)
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, 128)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ln = torch.full((1,), 128, dtype=torch.int64, device="cuda")
    qd = torch.zeros((1, case.n_q, case.d), dtype=torch.int16, device="cuda")
    out = torch.empty((1, case.n_q, case.d), dtype=torch.float32, device="cuda")
    ws = torch.empty((cb.decode_workspace_bytes(1, 128),), dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.AatcError) as e:
        lib.decode_attention(cb, blob, cache, 0, ids, ln, 129, qd, out, ws)
    assert e.value.status == -6
    small = torch.empty((16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.AatcError) as e:
        lib.decode_attention(cb, blob, cache, 0, ids, ln, 128, qd, out, small)
    assert e.value.status == -7
    K = torch.zeros((1, 10, 1, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(lib.AatcError) as e:
        lib.encode(cb, blob, cache, 0, [0], [120], 10, K, K)
    assert e.value.status == -6
    # the batched-layers call: layers outside the codebook, max_len beyond the cache and a
    # short workspace are refused before anything is launched (out keeps its contents)
    out.fill_(7.0)
    wsl = torch.zeros((cb.decode_layers_workspace_bytes(0, 1, 1, 128),), dtype=torch.uint8, device="cuda")
    for l0, nl, status in ((0, 2, -1), (1, 1, -1), (-1, 1, -1), (0, 0, -1)):
        with pytest.raises(lib.AatcError) as e:
            lib.decode_attention_layers(cb, blob, cache, l0, nl, ids, ln, 128, qd, out, wsl)
        assert e.value.status == status
    with pytest.raises(lib.AatcError) as e:
        lib.decode_attention_layers(cb, blob, cache, 0, 1, ids, ln, 129, qd, out, wsl)
    assert e.value.status == -6
    with pytest.raises(lib.AatcError) as e:
        lib.decode_attention_layers(cb, blob, cache, 0, 1, ids, ln, 128, qd, out, small)
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # and a valid one-layer batch equals aatc_decode_attention (same plan, same bits)
    ws.zero_()
    wsl.zero_()
    g = torch.Generator(device="cuda").manual_seed(11)
    qd.copy_(torch.randn(qd.shape, generator=g, device="cuda").to(torch.bfloat16).view(torch.int16))
    ref = torch.empty_like(out)
    lib.decode_attention(cb, blob, cache, 0, ids, ln, 128, qd, ref, ws)
    lib.decode_attention_layers(cb, blob, cache, 0, 1, ids, ln, 128, qd, out, wsl)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


# ---- attention-optimal (non-orthogonal) key transform: the encoder projects keys with T,
# the decode transforms queries with T^{-1} (computed by the library); same bars.
@pytest.mark.parametrize("wname,ctx", [("tiny", 512), ("llama_32k", 3000)])
def test_decode_parity_attention_optimal_keys(lib, torch, wname, ctx):
    _log(f"decode (attention-optimal keys) {wname} ctx={ctx}")
    case = Case(wname, ctx, n_calib_q=64, key_transform="nova")
    cache_host, _ = case.oracle_cache()
    got = _decode(lib, torch, case, cache_host, case.lens, ctx)
    err = normwise_rel_err(got, case.oracle_decode(cache_host))
    _log(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_BAR


@pytest.mark.parametrize("wname,ctx", [("tiny", 512), ("llama_32k", 1000)])
def test_encode_flips_attention_optimal_keys(lib, torch, wname, ctx):
    _log(f"encode (attention-optimal keys) {wname} ctx={ctx}")
    case = Case(wname, ctx, n_calib_q=64, key_transform="nova")
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, ctx)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    lib.encode(cb, blob, cache, 0, [0], [0], ctx, K, V)
    torch.cuda.synchronize()
    got = ct.cpu().numpy().reshape(case.n_kv, -1)
    _, codes = case.oracle_cache()
    flips, total, worst = 0, 0, 0
    for h, c in enumerate(case.cbs):
        gK, gV = oracle.unpack_cache(got[h], c.bK, c.bV, ctx)
        rK, rV = codes[(0, h)]
        for g, r, b in ((gK, rK, c.bK), (gV, rV, c.bV)):
            m = np.broadcast_to(b > 0, g.shape)
            dlt = np.abs(g - r)[m]
            flips += int((dlt > 0).sum())
            total += int(m.sum())
            worst = max(worst, int(dlt.max()))
    _log(f"  flips {flips}/{total}")
    assert worst <= 1
    assert flips <= FLIP_BAR * total
