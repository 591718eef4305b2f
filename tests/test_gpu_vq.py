"""GPU parity of vector-quantized keys (equal-volume groups, one 256-word codebook per
group): the encoder's index bytes bit-exact on the oracle's coefficients and within the
flip bar end to end; decode attention within 2e-3 of the oracle on the GPU's own bytes."""
import numpy as np
import pytest

import oracle
from test_gpu_parity import ATTN_BAR, FLIP_BAR, _decode, _device_codebook, _new_cache
from util import Case, code_flips, normwise_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _log(msg):
    print(msg, flush=True)


def _encode_bf16(lib, torch, case, chunks=None):
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, case.n_seqs, case.ctx)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    pos = 0
    for n in chunks or [case.ctx]:
        lib.encode(cb, blob, cache, 0, list(range(case.n_seqs)), [pos] * case.n_seqs, n,
                   K[:, pos:pos + n].contiguous(), V[:, pos:pos + n].contiguous())
        pos += n
    torch.cuda.synchronize()
    return ct.cpu().numpy().reshape(case.n_seqs, case.n_kv, -1)


@pytest.mark.parametrize("wname,ctx,n_kv,chunks", [
    ("vq_tiny", 512, None, [512]),
    ("vq_tiny", 512, None, [1, 63, 200, 248]),
    ("vq_low", 300, None, [300]),
    ("llama_vq_128k", 333, 2, [1, 127, 205]),
    ("vq_g7", 700, None, [700]),
    ("vq_g2", 300, None, [100, 200]),
])
def test_vq_encode_coeffs_bit_exact(lib, torch, wname, ctx, n_kv, chunks):
    _log(f"vq encode_coeffs {wname} ctx={ctx} chunks={chunks}")
    case = Case(wname, ctx, n_kv=n_kv, n_calib_q=64, key_quantizer="vq")
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


@pytest.mark.parametrize("wname,ctx,n_kv,chunks", [
    ("vq_tiny", 512, None, [512]),
    ("llama_vq_128k", 1000, 2, [1000]),
    ("llama_vq_128k", 333, 2, [1, 127, 205]),
    ("vq_g7", 1000, None, [1000]),
    ("vq_g2", 1000, None, [1000]),
])
def test_vq_encode_end_to_end(lib, torch, wname, ctx, n_kv, chunks):
    """Index bytes and value codes of the bf16 encoder: at most FLIP_BAR of them differ from
    the oracle's, and a differing index is a near-tie of the fp64 coefficients."""
    _log(f"vq encode {wname} ctx={ctx} chunks={chunks}")
    case = Case(wname, ctx, n_kv=n_kv, n_calib_q=64, key_quantizer="vq")
    got = _encode_bf16(lib, torch, case, chunks)[0]
    _, codes = case.oracle_cache()
    diffs, total = 0, 0
    for h, c in enumerate(case.cbs):
        gK, gV = oracle.unpack_cache(got[h], oracle.key_record_bits(c), c.bV, ctx)
        rK, _ = codes[(0, h)]
        bad = np.argwhere(gK != rK)
        diffs += len(bad)
        total += rK.size
        c64 = (case.kf(0, h) - c.muK[None, :]) @ c.UK
        for t, g in bad:
            u = c64[t, c.vq.groups[g]] * c.vq.scale32[c.vq.groups[g]].astype(np.float64)
            z = c.vq.cent32[g].astype(np.float64)
            e_got = ((u - z[gK[t, g]]) ** 2).sum()
            e_ref = ((u - z[rK[t, g]]) ** 2).sum()
            assert abs(e_got - e_ref) <= 1e-4 * max(e_ref, 1e-12), (t, g, e_got, e_ref)
        f, t, wst, edge = code_flips(got[h], c, ctx, case.kf(0, h), case.vf(0, h))  # value codes
        assert wst <= 1
        assert edge <= 1.0, f"kv-head {h}: a flipped value code lies {edge:.3g} windows from a cell edge"
        diffs += f
        total += t
    _log(f"  {diffs} of {total} codes differ")
    assert diffs <= FLIP_BAR * total


@pytest.mark.parametrize("wname,ctx,n_kv,n_seqs,lens", [
    ("vq_tiny", 512, None, 1, [512]),
    ("vq_tiny", 512, None, 1, [1]),
    ("vq_tiny", 512, None, 1, [65]),
    ("vq_tiny", 512, None, 3, [512, 1, 300]),
    ("vq_low", 512, None, 3, [512, 77, 300]),
    ("llama_vq_128k", 1000, 2, 1, [1000]),
    ("llama_vq_128k", 4096, 2, 2, [4096, 2049]),
    ("vq_g7", 4096, None, 2, [4096, 1001]),  # 7 query heads per kv-head: chunks of 4 and 3
    ("vq_g2", 2048, None, 3, [2048, 64, 130]),
])
def test_vq_decode_parity(lib, torch, wname, ctx, n_kv, n_seqs, lens):
    _log(f"vq decode {wname} ctx={ctx} lens={lens}")
    case = Case(wname, ctx, n_kv=n_kv, n_seqs=n_seqs, lens=lens, n_calib_q=64, key_quantizer="vq")
    cache_host, _ = case.oracle_cache()
    got = _decode(lib, torch, case, cache_host, case.lens, ctx)
    err = normwise_rel_err(got, case.oracle_decode(cache_host))
    _log(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_BAR


def test_vq_decode_full_layer_128k(lib, torch):
    """The Llama-shaped layer at 131072 tokens and 2.0 bits/element with vector-quantized
    keys, in the launch configuration the benchmark times: bf16 encode of all 8 kv-heads,
    one decode; the oracle decodes two sampled kv-heads from the GPU's bytes."""
    ctx = 131072
    _log(f"vq full layer ctx={ctx}")
    case = Case("llama_vq_128k", ctx, n_calib_q=32, key_quantizer="vq", vq_iters=4)
    got_cache = _encode_bf16(lib, torch, case)
    out = _decode(lib, torch, case, got_cache, case.lens, ctx)
    qf = case.qf()
    G = case.group
    for h in (0, 5):
        ref = oracle.decode_attention(got_cache[0, h], case.cbs[h], qf[0, h * G:(h + 1) * G], ctx)
        err = normwise_rel_err(out[0, h * G:(h + 1) * G], ref)
        _log(f"  kv-head {h}: rel err {err:.3e}")
        assert err <= ATTN_BAR


def test_vq_append_is_refused(lib, torch):
    case = Case("vq_tiny", 64, n_calib_q=32, key_quantizer="vq")
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, 128)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ln = torch.full((1,), 64, dtype=torch.int64, device="cuda")
    kn = torch.zeros((1, 1, case.d), dtype=torch.int16, device="cuda")
    qd = torch.zeros((1, case.n_q, case.d), dtype=torch.int16, device="cuda")
    out = torch.zeros((1, case.n_q, case.d), dtype=torch.float32, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(1, 65),), dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.AatcError):
        lib.decode_attention_append(cb, blob, cache, 0, ids, ln, 65, kn, kn, qd, out, ws)
