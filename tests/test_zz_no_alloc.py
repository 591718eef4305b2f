"""aatc_decode_attention_static (partials in the library's own device array, no
allocation) against aatc_decode_attention with a caller workspace: two calls in a row on
the same GPU, the second with a smaller input, each through the C ABI and bit for bit
equal to the workspace entry point (the same kernels run on the same inputs), and within
the decode bar of the oracle run on the same cache bytes.  The first call's plan merges in
a separate kernel, the second's in the decode kernel's last workgroup (the arrival counters
the static array keeps must be back at zero after the first)."""
import numpy as np
import pytest

from test_gpu_parity import _device_codebook, _new_cache
from util import Case, normwise_rel_err

pytestmark = pytest.mark.gpu

ATTN_BAR = 2e-3


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _log(msg):
    print(msg, flush=True)


def _call(lib, torch, case, cb, blob, cache, ids_l, lens_l, mx):
    ids = torch.tensor(ids_l, dtype=torch.int32, device="cuda")
    ln = torch.tensor(lens_l, dtype=torch.int64, device="cuda")
    qd = torch.from_numpy(case.q_bits.view(np.int16)).cuda()[torch.tensor(ids_l, device="cuda")].contiguous()
    ref = torch.full((len(ids_l), case.n_q, case.d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros((cb.decode_workspace_bytes(len(ids_l), mx),), dtype=torch.uint8, device="cuda")
    lib.decode_attention(cb, blob, cache, 0, ids, ln, mx, qd, ref, ws)
    got = torch.full_like(ref, float("nan"))
    lib.decode_attention_static(cb, blob, cache, 0, ids, ln, mx, qd, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_static_scratch_matches_workspace_entry_point(lib, torch):
    # call 1: 8 kv-heads x 13000 tokens -> 17 workgroups per kv-head, 36 KB of partials each
    # (separate merge kernel); call 2: 300 tokens -> one workgroup per kv-head (merged in
    # the decode kernel, which counts arrivals in the scratch array)
    n_seqs, ctx = 2, 13000
    case = Case("llama_32k", ctx, n_seqs=n_seqs, n_calib_q=32, lens=[13000, 300])
    cb, blob = _device_codebook(lib, torch, case)
    cache_host, _ = case.oracle_cache()
    ct, cache = _new_cache(lib, torch, cb, n_seqs, ctx)
    ct.copy_(torch.from_numpy(cache_host.reshape(-1)))
    _log("static scratch: call 1, one sequence of 13000 tokens (separate merge kernel)")
    got, ref = _call(lib, torch, case, cb, blob, cache, [0], [13000], 13000)
    assert np.array_equal(got, ref)
    oracle_out = case.oracle_decode(cache_host)
    assert normwise_rel_err(got, oracle_out[[0]]) <= ATTN_BAR
    _log("static scratch: call 2, one sequence of 300 tokens (merge in the decode kernel)")
    got, ref = _call(lib, torch, case, cb, blob, cache, [1], [300], 300)
    assert np.array_equal(got, ref)
    assert normwise_rel_err(got, oracle_out[[1]]) <= ATTN_BAR
    _log("static scratch: call 3, the first call again")
    got, ref = _call(lib, torch, case, cb, blob, cache, [0], [13000], 13000)
    assert np.array_equal(got, ref)


def test_static_scratch_rejects_calls_beyond_its_size(lib, torch):
    case = Case("tiny", 128, n_calib_q=16)
    cb, blob = _device_codebook(lib, torch, case)
    ct, cache = _new_cache(lib, torch, cb, 1, 128)
    ids = torch.zeros(60000, dtype=torch.int32, device="cuda")
    ln = torch.full((60000,), 128, dtype=torch.int64, device="cuda")
    qd = torch.zeros((60000, case.n_q, case.d), dtype=torch.int16, device="cuda")
    out = torch.empty((60000, case.n_q, case.d), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.AatcError) as e:
        lib.decode_attention_static(cb, blob, cache, 0, ids, ln, 128, qd, out)
    assert e.value.status == -6
