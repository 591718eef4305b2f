"""GPU parity at the shapes of the remaining workloads (through the C ABI):

- the 128k-token Llama-shaped layer in the launch configuration the benchmark times
  (all 8 kv-heads on the GPU; the oracle decodes two sampled kv-heads from the GPU's own
  bytes, and checks the codes of one kv-head end to end);
- the 2.0 bits/element decode loop: prefill, then per step append one token per kv-head
  and decode over the grown cache;
- a two-layer cache (layer indexing of codebook and cache);
- a wide serving batch (32 ragged sequences: few workgroups per kv-head).

Bars as in the other parity tests: attention within 2e-3 normwise relative error of the
oracle on the same bytes; end-to-end codes differ on at most 1e-4 of coded pairs, by one
level, each within the fp32 rounding window of a cell edge.
"""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import _decode, _device_codebook, _new_cache
from util import Case, code_flips, normwise_rel_err

pytestmark = pytest.mark.gpu

ATTN_BAR = 2e-3
FLIP_BAR = 1e-4


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _log(msg):
    print(msg, flush=True)


def _flips(got_bytes, case, h, n_tokens, K64, V64):
    """(flips, coded pairs, worst level difference) of kv-head h's codes against the
    oracle's; every flipped code must lie in the fp32 rounding window of a cell edge."""
    flips, total, worst, edge = code_flips(got_bytes, case.cbs[h], n_tokens, K64, V64)
    assert edge <= 1.0, f"kv-head {h}: a flipped code lies {edge:.3g} windows from a cell edge"
    return flips, total, worst


def test_full_llama_128k_layer(lib, torch):
    ctx = 131072
    _log(f"llama_128k full layer, {ctx} tokens")
    case = Case("llama_128k", ctx, n_calib_q=64)
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, ctx)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    lib.encode(cb, blob, cache, 0, [0], [0], ctx, K, V)
    del K, V
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ln = torch.full((1,), ctx, dtype=torch.int64, device="cuda")
    qd = torch.from_numpy(case.q_bits.view(np.int16)).cuda()
    out = torch.full((1, case.n_q, case.d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(1, ctx),), dtype=torch.uint8, device="cuda")
    lib.decode_attention(cb, blob, cache, 0, ids, ln, ctx, qd, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    cache_bytes = ct.cpu().numpy().reshape(case.n_kv, -1)
    qf = case.qf()
    G = case.group
    for h in (0, 5):
        ref = oracle.decode_attention(cache_bytes[h], case.cbs[h], qf[0, h * G:(h + 1) * G], ctx)
        err = normwise_rel_err(got[:, h * G:(h + 1) * G], ref[None])
        _log(f"  kv-head {h}: rel err {err:.3e}")
        assert err <= ATTN_BAR
    flips, total, worst = _flips(cache_bytes[0], case, 0, ctx, case.kf(0, 0), case.vf(0, 0))
    _log(f"  kv-head 0 codes: {flips} flips of {total}")
    assert worst <= 1
    assert flips <= FLIP_BAR * total


def test_decode_loop_append_then_decode(lib, torch):
    """Decode-loop workload at 2.0 bits/element: prefill, then steps of one appended token
    per kv-head (its own fresh draw) followed by a decode over the grown cache."""
    L0, steps = 3000, 5
    case = Case("llama_loop", L0 + steps, n_calib_q=64)
    _log(f"llama_loop: prefill {L0}, {steps} append+decode steps")
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, L0 + steps)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    lib.encode(cb, blob, cache, 0, [0], [0], L0, K[:, :L0].contiguous(), V[:, :L0].contiguous())
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(1, L0 + steps),), dtype=torch.uint8, device="cuda")
    G = case.group
    for s in range(steps):
        L = L0 + s
        lib.encode(cb, blob, cache, 0, [0], [L], 1, K[:, L:L + 1].contiguous(), V[:, L:L + 1].contiguous())
        q_bits = synth.to_bf16_bits(synth.decode_queries(case.w, case.hms, case.layer, 0, step=s + 1))
        qf = synth.bf16_bits_to_f64(q_bits)
        qd = torch.from_numpy(q_bits.view(np.int16)[None]).cuda()
        ln = torch.full((1,), L + 1, dtype=torch.int64, device="cuda")
        out = torch.full((1, case.n_q, case.d), float("nan"), dtype=torch.float32, device="cuda")
        lib.decode_attention(cb, blob, cache, 0, ids, ln, L + 1, qd, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        cache_bytes = ct.cpu().numpy().reshape(case.n_kv, -1)
        ref = np.stack([oracle.decode_attention(cache_bytes[h], case.cbs[h], qf[h * G:(h + 1) * G], L + 1)
                        for h in range(case.n_kv)]).reshape(1, case.n_q, case.d)
        err = normwise_rel_err(got, ref)
        _log(f"  step {s}: {L + 1} tokens, rel err {err:.3e}")
        assert np.all(np.isfinite(got))
        assert err <= ATTN_BAR
    cache_bytes = ct.cpu().numpy().reshape(case.n_kv, -1)
    flips = total = worst = 0
    for h in range(case.n_kv):
        f, t, wst = _flips(cache_bytes[h], case, h, L0 + steps, case.kf(0, h), case.vf(0, h))
        flips, total, worst = flips + f, total + t, max(worst, wst)
    _log(f"  codes: {flips} flips of {total}")
    assert worst <= 1
    assert flips <= FLIP_BAR * total


def test_decode_second_layer(lib, torch):
    """Two-layer codebook and cache (Qwen-shaped layers, G = 7): each layer decodes with its
    own codebook from its own part of the cache."""
    ctx = 1500
    cases = [Case("qwen_128k", ctx, n_calib_q=32, layer=layer) for layer in (0, 1)]
    c0 = cases[0]
    arrs = [c.codebook_arrays() for c in cases]
    a = {k: np.concatenate([x[k] for x in arrs]) for k in arrs[0]}
    cb = lib.codebook_create(c0.d, 2, c0.n_kv, c0.group, a["UK"], a["UV"], a["muK"], a["muV"], a["bK"], a["bV"],
                             a["stepK"], a["stepV"])
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device="cuda")
    cb.upload(blob)
    hosts = [c.oracle_cache()[0] for c in cases]
    assert hosts[0].shape == hosts[1].shape
    ct = torch.zeros(cb.cache_bytes(2, 1, ctx), dtype=torch.uint8, device="cuda")
    ct.copy_(torch.from_numpy(np.concatenate([h.reshape(-1) for h in hosts])))
    cache = lib.make_cache(ct, 2, 1, ctx)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ln = torch.full((1,), ctx, dtype=torch.int64, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(1, ctx),), dtype=torch.uint8, device="cuda")
    for layer in (1, 0):
        c = cases[layer]
        qd = torch.from_numpy(c.q_bits.view(np.int16)).cuda()
        out = torch.full((1, c.n_q, c.d), float("nan"), dtype=torch.float32, device="cuda")
        lib.decode_attention(cb, blob, cache, layer, ids, ln, ctx, qd, out, ws)
        torch.cuda.synchronize()
        err = normwise_rel_err(out.cpu().numpy(), c.oracle_decode(hosts[layer]))
        _log(f"  layer {layer}: rel err {err:.3e}")
        assert err <= ATTN_BAR


def test_decode_wide_batch(lib, torch):
    """32 sequences of ragged lengths (1 to 300 tokens) in one call."""
    rng = np.random.default_rng(7)
    lens = [1, 64, 65, 300] + [int(x) for x in rng.integers(1, 301, 28)]
    case = Case("llama_batch", 300, n_seqs=32, n_calib_q=32, lens=lens)
    _log(f"llama_batch: 32 sequences, lengths {min(lens)}..{max(lens)}")
    cache_host, _ = case.oracle_cache()
    got = _decode(lib, torch, case, cache_host, lens, 300)
    err = normwise_rel_err(got, case.oracle_decode(cache_host, lens))
    _log(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_BAR


@pytest.mark.parametrize("wname,n_seqs,l0,steps", [("tiny", 2, (126, 63), 4), ("llama_loop", 1, (3000,), 4),
                                                    ("edge_max", 1, (127,), 3)])
def test_fused_append_decode_loop(lib, torch, wname, n_seqs, l0, steps):
    """Generation loop through aatc_decode_attention_append: per step one new token per
    (sequence, kv-head) is coded and attended in the same launch.  The cache bytes equal
    those of aatc_encode appending the same tokens (bit-exact), and every step's output
    is within the decode bar of the oracle on the GPU's own bytes (tile boundaries and
    ragged sequences included; 8 bits on every channel takes the three-term encoder basis)."""
    ctx = max(l0) + steps
    case = Case(wname, ctx, n_seqs=n_seqs, n_calib_q=64)
    _log(f"{wname}: fused append+decode, {n_seqs} sequences from {l0}, {steps} steps")
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, n_seqs, ctx)
    rt, rcache = _new_cache(lib, torch, cb, n_seqs, ctx)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    for s in range(n_seqs):  # prefill both caches with the encoder
        for c in (cache, rcache):
            lib.encode(cb, blob, c, 0, [s], [0], l0[s], K[s:s + 1, :l0[s]].contiguous(), V[s:s + 1, :l0[s]].contiguous())
    ids = torch.arange(n_seqs, dtype=torch.int32, device="cuda")
    lens = torch.tensor(l0, dtype=torch.int64, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(n_seqs, ctx),), dtype=torch.uint8, device="cuda")
    G = case.group
    for st in range(steps):
        pos = [l + st for l in l0]
        kn = torch.stack([K[s, pos[s]] for s in range(n_seqs)]).contiguous()  # [n_seqs, n_kv, d]
        vn = torch.stack([V[s, pos[s]] for s in range(n_seqs)]).contiguous()
        q_bits = np.stack([synth.to_bf16_bits(synth.decode_queries(case.w, case.hms, case.layer, s, step=st + 1))
                           for s in range(n_seqs)])
        qd = torch.from_numpy(q_bits.view(np.int16)).cuda()
        out = torch.full((n_seqs, case.n_q, case.d), float("nan"), dtype=torch.float32, device="cuda")
        lib.decode_attention_append(cb, blob, cache, 0, ids, lens, ctx, kn, vn, qd, out, ws)
        for s in range(n_seqs):
            lib.encode(cb, blob, rcache, 0, [s], [pos[s]], 1, K[s:s + 1, pos[s]:pos[s] + 1].contiguous(),
                       V[s:s + 1, pos[s]:pos[s] + 1].contiguous())
        lens += 1
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        bytes_ = ct.cpu().numpy().reshape(n_seqs, case.n_kv, -1)
        assert np.array_equal(bytes_, rt.cpu().numpy().reshape(n_seqs, case.n_kv, -1)), f"step {st}: cache bytes"
        qf = synth.bf16_bits_to_f64(q_bits)
        ref = np.stack([np.stack([oracle.decode_attention(bytes_[s, h], case.cbs[h], qf[s, h * G:(h + 1) * G],
                                                          pos[s] + 1) for h in range(case.n_kv)]).reshape(case.n_q, case.d)
                        for s in range(n_seqs)])
        err = normwise_rel_err(got, ref)
        _log(f"  step {st}: lengths {[p + 1 for p in pos]}, rel err {err:.3e}")
        assert np.all(np.isfinite(got))
        assert err <= ATTN_BAR


@pytest.mark.parametrize("wname,ctx,lens", [("edge_g16", 700, [700, 65]), ("edge_rate", 300, [300]),
                                            ("edge_max", 300, [300, 1])])
def test_decode_and_encode_at_the_limits(lib, torch, wname, ctx, lens):
    """16 query heads per kv-head (the probability operands in buffers of their own when the
    key block is smaller, d = 64 at 3.0 b/e), a high rate (d = 128 at 6.0 b/e: the widest
    score and value schedules) and the largest (8 bits on every channel at d = 64, a 1-token
    sequence beside a 300-token one): decode within the bar of the oracle on the same bytes,
    end-to-end codes within the flip bar."""
    case = Case(wname, ctx, n_seqs=len(lens), n_calib_q=32, lens=lens)
    _log(f"{wname}: G={case.group}, d={case.d}, lengths {lens}")
    cache_host, _ = case.oracle_cache()
    got = _decode(lib, torch, case, cache_host, lens, ctx)
    err = normwise_rel_err(got, case.oracle_decode(cache_host, lens))
    _log(f"  decode rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_BAR
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, ctx)
    K = torch.from_numpy(case.k_bits[:1].view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits[:1].view(np.int16)).cuda()
    lib.encode(cb, blob, cache, 0, [0], [0], ctx, K, V)
    torch.cuda.synchronize()
    got_b = ct.cpu().numpy().reshape(case.n_kv, -1)
    flips = total = worst = 0
    for h in range(case.n_kv):
        f, t, wst = _flips(got_b[h], case, h, ctx, case.kf(0, h), case.vf(0, h))
        flips, total, worst = flips + f, total + t, max(worst, wst)
    _log(f"  codes: {flips} flips of {total}")
    assert worst <= 1
    assert flips <= FLIP_BAR * total
