"""GPU parity at the full sizes of the multi-layer, batch and generation-loop workloads, in
the launch configurations the benchmark times, through the library's own calibration
(host statistics -> calibrate -> upload -> aatc_encode -> decode):

- Qwen-2.5-7B-shaped cache, 28 layers x 131072 tokens (4 kv-heads of 7 query heads);
- Llama-shaped serving batch, 32 layers x 32 sequences x 8192 tokens;
- generation loop at 2.0 bits/element: 65536 prefilled tokens, then 1024 steps of
  aatc_decode_attention_append.

Checks: the library's bit allocation of sampled heads is the oracle's (bit-exact; steps
within 1e-6); a decode step over every layer replayed as a HIP graph is bit-identical to
the same calls made eagerly; on sampled slices the attention is within 2e-3 normwise
relative error of the oracle decoding the GPU's own bytes with the library's parameters,
and the end-to-end codes differ from the oracle's on at most 1e-4 of coded pairs, by one
level, each inside the fp32 rounding window of a cell edge.  Inputs are seeded device
draws (synth.device_kv / device_queries); the oracle side draws the same slices again.
"""
from concurrent.futures import ThreadPoolExecutor
import time

import numpy as np
import pytest

import oracle
import synth
from util import LAYOUT_KEY_ALIGN, code_flips, library_head_codebook, normwise_rel_err

pytestmark = pytest.mark.gpu

ATTN_BAR = 2e-3
FLIP_BAR = 1e-4
# batched-layers call against one call per layer: the same arithmetic per (layer, sequence,
# kv-head) with the tiles split among another number of workgroups.  The probabilities are
# fixed-point integers relative to each wave's reference maximum, so another split rounds
# them differently; over diffuse attention on zero-mean values that noise reaches a few
# 1e-4 of the output (observed 5e-4 on the Qwen-shaped model), within the oracle bar that
# both outputs are held to.  The whole outputs are compared at that bar, and both are
# checked against the oracle on the (layer, sequence, kv-head) where they differ most.
BATCH_BAR = ATTN_BAR
DEV = "cuda"


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _log(msg):
    print(msg, flush=True)


def _library_codebook(q, w, n_layers):
    """Library statistics and calibration of every (layer, kv-head), heads in parallel threads."""
    keys = [(layer, h) for layer in range(n_layers) for h in range(w.n_kv)]
    hms = [synth.head_model(w, layer, h) for layer, h in keys]

    def stats(i):
        layer, h = keys[i]
        K, V, Q = synth.calibration_samples(w, hms[i], layer, h)
        return q.stats_from_samples(K, V, Q)

    with ThreadPoolExecutor(8) as ex:
        st = list(ex.map(stats, range(len(keys))))
    return q.calibrate(st, w.d, n_layers, w.n_kv, w.group, w.avg_bits), hms


def _check_calibration(cb, w, hms, heads):
    """The library's allocation and steps of the sampled heads against the oracle's
    calibration of the same samples."""
    for layer, h in heads:
        i = layer * w.n_kv + h
        K, V, Q = synth.calibration_samples(w, hms[i], layer, h)
        ref = oracle.build_head_codebook(oracle.head_stats(K, V, Q), w.avg_bits, key_align=LAYOUT_KEY_ALIGN)
        got = cb.head(i)
        assert np.array_equal(got["bK"], ref.bK) and np.array_equal(got["bV"], ref.bV), (layer, h)
        assert np.allclose(got["stepK"], ref.stepK, rtol=1e-6) and np.allclose(got["stepV"], ref.stepV, rtol=1e-6)
    _log(f"  calibration of heads {heads}: bits identical to the oracle's")


def _prefill(torch, q, cb, blob, cache, w, hms, n_layers, n_seqs, ctx):
    for layer in range(n_layers):
        K = torch.empty((n_seqs, ctx, w.n_kv, w.d), dtype=torch.int16, device=DEV)
        V = torch.empty_like(K)
        for s in range(n_seqs):
            for h in range(w.n_kv):
                k, v = synth.device_kv(torch, hms[layer * w.n_kv + h], ctx,
                                       synth.seed_of(w.cfg, layer, s, h, synth.ST_CACHE_KV), DEV)
                K[s, :, h] = k
                V[s, :, h] = v
        q.encode(cb, blob, cache, layer, list(range(n_seqs)), [0] * n_seqs, ctx, K, V)
        del K, V


def _queries(torch, w, hms, layer, s):
    return torch.cat([synth.device_queries(torch, hms[layer * w.n_kv + h], w.group,
                                           synth.seed_of(w.cfg, layer, s, h, synth.ST_DECODE_Q), DEV)[0]
                      for h in range(w.n_kv)])


def _bits_of(t):
    return t.cpu().numpy().view(np.uint16)


def _layers_step(torch, q, w, n_layers, n_seqs, ctx):
    """Calibrate, prefill every layer, then one decode step over all layers as a HIP graph
    and eagerly, and once more as one batched-layers call; returns what the slice checks
    need (the per-layer and the batched outputs)."""
    t0 = time.perf_counter()
    cb, hms = _library_codebook(q, w, n_layers)
    _log(f"  library calibration of {len(hms)} heads: {time.perf_counter() - t0:.1f}s")
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device=DEV)
    cb.upload(blob)
    cache_t = torch.zeros(cb.cache_bytes(n_layers, n_seqs, ctx), dtype=torch.uint8, device=DEV)
    cache = q.make_cache(cache_t, n_layers, n_seqs, ctx)
    t0 = time.perf_counter()
    _prefill(torch, q, cb, blob, cache, w, hms, n_layers, n_seqs, ctx)
    torch.cuda.synchronize()
    _log(f"  prefill of {n_layers} layers x {n_seqs} sequences x {ctx} tokens: {time.perf_counter() - t0:.1f}s")
    Qd = torch.stack([torch.stack([_queries(torch, w, hms, layer, s) for s in range(n_seqs)])
                      for layer in range(n_layers)])
    out = torch.full((n_layers, n_seqs, w.n_q, w.d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(cb.decode_workspace_bytes(n_seqs, ctx), dtype=torch.uint8, device=DEV)
    ids = torch.arange(n_seqs, dtype=torch.int32, device=DEV)
    lens = torch.full((n_seqs,), ctx, dtype=torch.int64, device=DEV)

    def step():
        for layer in range(n_layers):
            q.decode_attention(cb, blob, cache, layer, ids, lens, ctx, Qd[layer], out[layer], ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    out.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "graph replay differs from the eager calls"
    _log(f"  decode step over {n_layers} layers: graph replays bit-identical to the eager calls")
    # all layers in one batched call (one launch per run of layers sharing a decode variant):
    # another split of the tiles, so the same attention up to the rounding of the merge
    wsl = torch.zeros(cb.decode_layers_workspace_bytes(0, n_layers, n_seqs, ctx), dtype=torch.uint8, device=DEV)
    outl = torch.full_like(out, float("nan"))
    q.decode_attention_layers(cb, blob, cache, 0, n_layers, ids, lens, ctx, Qd, outl, wsl)
    torch.cuda.synchronize()
    a, b = outl.double(), eager.double()
    assert bool(torch.isfinite(a).all()), "batched-layers call left non-finite outputs"
    G = w.group
    rel = ((a - b).reshape(n_layers, n_seqs, w.n_kv, G * w.d).norm(dim=-1) /
           b.reshape(n_layers, n_seqs, w.n_kv, G * w.d).norm(dim=-1))
    diff = rel.max().item()
    worst = np.unravel_index(int(rel.argmax().item()), tuple(rel.shape))
    _log(f"  batched-layers call: largest normwise difference to the per-layer calls {diff:.2e} "
         f"at (layer, seq, kv-head) {tuple(int(x) for x in worst)}")
    assert diff <= BATCH_BAR
    return cb, hms, cache_t, (out.cpu().numpy(), outl.cpu().numpy()), tuple(int(x) for x in worst)


def _check_slice(torch, cb, w, hms, cache_t, out, n_seqs, ctx, layer, s, h):
    i = layer * w.n_kv + h
    ocb = library_head_codebook(cb, i)
    nt = (ctx + 63) // 64
    span = nt * cb.tile_bytes
    off = ((layer * n_seqs + s) * w.n_kv + h) * span
    got_bytes = cache_t[off:off + span].cpu().numpy()
    k, v = synth.device_kv(torch, hms[i], ctx, synth.seed_of(w.cfg, layer, s, h, synth.ST_CACHE_KV), DEV)
    K64, V64 = synth.bf16_bits_to_f64(_bits_of(k)), synth.bf16_bits_to_f64(_bits_of(v))
    del k, v
    qf = synth.bf16_bits_to_f64(_bits_of(_queries(torch, w, hms, layer, s)))
    G = w.group
    ref = oracle.decode_attention(got_bytes, ocb, qf[h * G:(h + 1) * G], ctx)
    err = 0.0
    for o in out:  # the per-layer calls' output and the batched call's
        assert np.all(np.isfinite(o[layer, s, h * G:(h + 1) * G]))
        err = max(err, normwise_rel_err(o[layer, s, h * G:(h + 1) * G], ref))
    flips, total, worst, edge = code_flips(got_bytes, ocb, ctx, K64, V64)
    _log(f"  (layer {layer}, seq {s}, kv-head {h}): rel err {err:.3e}, {flips} flips of {total}, "
         f"edge ratio {edge:.3g}")
    assert err <= ATTN_BAR
    assert worst <= 1 and edge <= 1.0
    assert flips <= FLIP_BAR * total


def test_qwen_28_layers_131072_tokens(lib, torch):
    w = synth.WORKLOADS["qwen_128k"]
    L, S, ctx = w.n_layers, 1, w.ctx
    _log(f"qwen_128k: {L} layers x {ctx} tokens, {w.n_kv} kv-heads, G={w.group}")
    cb, hms, cache_t, out, worst = _layers_step(torch, lib, w, L, S, ctx)
    _check_calibration(cb, w, hms, [(0, 0), (13, 2), (27, 3)])
    for layer, s, h in ((0, 0, 0), (13, 0, 2), (27, 0, 3), worst):
        _check_slice(torch, cb, w, hms, cache_t, out, S, ctx, layer, s, h)


def test_llama_batch_32_layers_32_sequences_8192_tokens(lib, torch):
    w = synth.WORKLOADS["llama_batch"]
    L, S, ctx = w.n_layers, w.n_seqs, w.ctx
    _log(f"llama_batch: {L} layers x {S} sequences x {ctx} tokens")
    cb, hms, cache_t, out, worst = _layers_step(torch, lib, w, L, S, ctx)
    _check_calibration(cb, w, hms, [(0, 0), (31, 7)])
    for layer, s, h in ((0, 0, 0), (9, 31, 5), (22, 4, 2), (31, 17, 7), worst):
        _check_slice(torch, cb, w, hms, cache_t, out, S, ctx, layer, s, h)


def test_generation_loop_1024_steps(lib, torch):
    w = synth.WORKLOADS["llama_loop"]
    l0, n = w.ctx, 1024
    cap = l0 + n
    _log(f"llama_loop: {l0} prefilled tokens, {n} append+decode steps")
    cb, hms = _library_codebook(lib, w, 1)
    _check_calibration(cb, w, hms, [(0, 0), (0, 5)])
    blob = torch.empty(cb.device_bytes(), dtype=torch.uint8, device=DEV)
    cb.upload(blob)
    cache_t = torch.zeros(cb.cache_bytes(1, 1, cap), dtype=torch.uint8, device=DEV)
    cache = lib.make_cache(cache_t, 1, 1, cap)
    _prefill(torch, lib, cb, blob, cache, w, hms, 1, 1, l0)
    kn = torch.empty((n, 1, w.n_kv, w.d), dtype=torch.int16, device=DEV)
    vn = torch.empty_like(kn)
    qn = torch.empty((n, 1, w.n_q, w.d), dtype=torch.int16, device=DEV)
    for h in range(w.n_kv):
        k, v = synth.device_kv(torch, hms[h], n, synth.seed_of(w.cfg, 0, 0, h, synth.ST_STEP), DEV)
        kn[:, 0, h] = k
        vn[:, 0, h] = v
        qn[:, 0, h * w.group:(h + 1) * w.group] = synth.device_queries(
            torch, hms[h], w.group, synth.seed_of(w.cfg, 0, 0, h, synth.ST_DECODE_Q), DEV, n)
    torch.cuda.synchronize()
    pristine = cache_t.clone()
    lens_all = torch.arange(l0, cap, dtype=torch.int64, device=DEV)
    out = torch.full((n, 1, w.n_q, w.d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(cb.decode_workspace_bytes(1, cap), dtype=torch.uint8, device=DEV)
    ids = torch.zeros(1, dtype=torch.int32, device=DEV)

    def step(i):
        lib.decode_attention_append(cb, blob, cache, 0, ids, lens_all[i:i + 1], cap, kn[i], vn[i], qn[i], out[i], ws)

    for i in range(n):  # eagerly, as the benchmark's per-step timing runs it
        step(i)
    torch.cuda.synchronize()
    eager_out, eager_cache = out.clone(), cache_t.clone()
    # the cache bytes equal those of aatc_encode appending the same tokens in one call
    ref_t = pristine.clone()
    rcache = lib.make_cache(ref_t, 1, 1, cap)
    lib.encode(cb, blob, rcache, 0, [0], [l0], n, kn[:, 0].unsqueeze(0).contiguous(), vn[:, 0].unsqueeze(0).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(eager_cache, ref_t), "appended bytes differ from aatc_encode's"
    # the whole loop as one HIP graph: bit-identical outputs and cache
    cache_t.copy_(pristine)
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step(i)
    cache_t.copy_(pristine)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager_out) and torch.equal(cache_t, eager_cache), "graph loop differs from eager"
    _log("  eager loop == graph loop == aatc_encode bytes")
    got = eager_out.cpu().numpy()
    assert np.all(np.isfinite(got))
    span = ((cap + 63) // 64) * cb.tile_bytes
    final = eager_cache.cpu().numpy().reshape(w.n_kv, span)
    qf = synth.bf16_bits_to_f64(_bits_of(qn))  # [n, 1, n_q, d]
    kf = synth.bf16_bits_to_f64(_bits_of(kn))
    vf = synth.bf16_bits_to_f64(_bits_of(vn))
    steps = [0, 1, 62, 63, 64, 127, 511, 1022, 1023]
    G = w.group
    worst_err = 0.0
    flips = total = 0
    for h in range(w.n_kv):
        ocb = library_head_codebook(cb, h)
        Khat, Vhat = oracle.decoded_kv(final[h], ocb, cap)
        for i in steps:
            ref = oracle.attention(qf[i, 0, h * G:(h + 1) * G], Khat[:l0 + i + 1], Vhat[:l0 + i + 1])
            err = normwise_rel_err(got[i, 0, h * G:(h + 1) * G], ref)
            worst_err = max(worst_err, err)
            assert err <= ATTN_BAR, (h, i, err)
        f, t, wst, edge = code_flips(final[h], ocb, cap, kf[:, 0, h], vf[:, 0, h], first=l0)
        assert wst <= 1 and edge <= 1.0, (h, wst, edge)
        flips, total = flips + f, total + t
    _log(f"  steps {steps}, every kv-head: worst rel err {worst_err:.3e}; appended codes: {flips} flips of {total}")
    assert flips <= FLIP_BAR * total
    for h in (0, 7):  # prefill codes of two kv-heads
        k, v = synth.device_kv(torch, hms[h], l0, synth.seed_of(w.cfg, 0, 0, h, synth.ST_CACHE_KV), DEV)
        f, t, wst, edge = code_flips(final[h], library_head_codebook(cb, h), l0,
                                     synth.bf16_bits_to_f64(_bits_of(k)), synth.bf16_bits_to_f64(_bits_of(v)))
        _log(f"  kv-head {h} prefill codes: {f} flips of {t}, edge ratio {edge:.3g}")
        assert wst <= 1 and edge <= 1.0
        assert f <= FLIP_BAR * t
