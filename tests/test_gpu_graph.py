"""The decode calls inside a HIP graph (torch.cuda.CUDAGraph over the caller's stream):
every launch argument is a device pointer or a host scalar fixed at capture, sequence
lengths are read on the device, and nothing is allocated, copied or cleared by the
library, so a captured step replays correctly.  Each replay is compared bit for bit with
the same step run eagerly, with eager work between the replays."""
import numpy as np
import pytest

import synth
from test_gpu_parity import _device_codebook, _new_cache
from util import Case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _log(msg):
    print(msg, flush=True)


def test_decode_replays_match_eager(lib, torch):
    ctx = 2000
    case = Case("llama_32k", ctx, n_calib_q=32)
    _log("graph: plain decode, 3 replays")
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, ctx)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    lib.encode(cb, blob, cache, 0, [0], [0], ctx, K, V)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens = torch.full((1,), ctx, dtype=torch.int64, device="cuda")
    qd = torch.empty((1, case.n_q, case.d), dtype=torch.int16, device="cuda")
    out_g = torch.empty((1, case.n_q, case.d), dtype=torch.float32, device="cuda")
    ws_g = torch.zeros((cb.decode_workspace_bytes(1, ctx),), dtype=torch.uint8, device="cuda")
    ws_e = torch.zeros_like(ws_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.decode_attention(cb, blob, cache, 0, ids, lens, ctx, qd, out_g, ws_g)
    for rep in range(3):
        q_bits = synth.to_bf16_bits(synth.decode_queries(case.w, case.hms, 0, 0, step=rep + 1))[None]
        qd.copy_(torch.from_numpy(q_bits.view(np.int16)))
        out_g.fill_(float("nan"))
        g.replay()
        out_e = torch.full_like(out_g, float("nan"))
        lib.decode_attention(cb, blob, cache, 0, ids, lens, ctx, qd, out_e, ws_e)  # eager, between replays
        torch.cuda.synchronize()
        assert np.array_equal(out_g.cpu().numpy(), out_e.cpu().numpy()), f"replay {rep}"


def test_append_decode_replays_match_eager(lib, torch):
    l0, steps = 1000, 4
    ctx = l0 + steps
    case = Case("llama_loop", ctx, n_calib_q=32)
    _log(f"graph: fused append + decode + length update, {steps} replays")
    cb, blob = _device_codebook(lib, torch, case)
    ct_g, cache_g = _new_cache(lib, torch, cb, 1, ctx)
    ct_e, cache_e = _new_cache(lib, torch, cb, 1, ctx)
    K = torch.from_numpy(case.k_bits.view(np.int16)).cuda()
    V = torch.from_numpy(case.v_bits.view(np.int16)).cuda()
    for c in (cache_g, cache_e):
        lib.encode(cb, blob, c, 0, [0], [0], l0, K[:, :l0].contiguous(), V[:, :l0].contiguous())
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens_g = torch.full((1,), l0, dtype=torch.int64, device="cuda")
    lens_e = torch.full((1,), l0, dtype=torch.int64, device="cuda")
    kn = torch.empty((1, case.n_kv, case.d), dtype=torch.int16, device="cuda")
    vn = torch.empty_like(kn)
    qd = torch.empty((1, case.n_q, case.d), dtype=torch.int16, device="cuda")
    out_g = torch.empty((1, case.n_q, case.d), dtype=torch.float32, device="cuda")
    ws_g = torch.zeros((cb.decode_workspace_bytes(1, ctx),), dtype=torch.uint8, device="cuda")
    ws_e = torch.zeros_like(ws_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.decode_attention_append(cb, blob, cache_g, 0, ids, lens_g, ctx, kn, vn, qd, out_g, ws_g)
        lens_g.add_(1)
    for st in range(steps):
        pos = l0 + st
        kn.copy_(K[0, pos].unsqueeze(0))
        vn.copy_(V[0, pos].unsqueeze(0))
        q_bits = synth.to_bf16_bits(synth.decode_queries(case.w, case.hms, 0, 0, step=st + 1))[None]
        qd.copy_(torch.from_numpy(q_bits.view(np.int16)))
        out_g.fill_(float("nan"))
        g.replay()
        out_e = torch.full_like(out_g, float("nan"))
        lib.decode_attention_append(cb, blob, cache_e, 0, ids, lens_e, ctx, kn, vn, qd, out_e, ws_e)
        lens_e.add_(1)
        torch.cuda.synchronize()
        assert int(lens_g.item()) == pos + 1
        assert np.array_equal(out_g.cpu().numpy(), out_e.cpu().numpy()), f"replay {st}: output"
        assert np.array_equal(ct_g.cpu().numpy(), ct_e.cpu().numpy()), f"replay {st}: cache bytes"
