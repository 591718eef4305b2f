"""Python binding of libaatc (transform-coded KV cache for MI355X).

Argument marshalling only: every computation runs in the library (host calibration in
C++, encode/decode in gfx950 HIP kernels).  PyTorch supplies device memory and streams.
The names follow the C ABI in include/aatc.h.  Loading fails loudly if the library has
not been built (python -m quantized_attention_klt_amd.build).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libaatc.so")

OK = 0
ERRORS = {
    -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "BUDGET", -4: "STATS", -5: "NO_CONVERGENCE",
    -6: "CAPACITY", -7: "WORKSPACE", -8: "HIP", -9: "IO", -10: "VERSION",
}


class AatcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"aatc error {status} ({ERRORS.get(status, '?')}): {msg}")
        self.status = status


class HeadStats(C.Structure):
    _fields_ = [("mu_k", C.POINTER(C.c_double)), ("mu_v", C.POINTER(C.c_double)),
                ("sigma_k", C.POINTER(C.c_double)), ("sigma_v", C.POINTER(C.c_double)),
                ("m_q", C.POINTER(C.c_double)), ("gamma_v", C.c_double)]


class CalibParams(C.Structure):
    _fields_ = [("avg_bits", C.c_double), ("max_bits", C.c_int32), ("joint", C.c_int32),
                ("max_sweeps", C.c_int32), ("key_transform", C.c_int32), ("key_quantizer", C.c_int32),
                ("vq_iters", C.c_int32), ("vq_normals", C.c_void_p), ("vq_n_train", C.c_int64)]


class Cache(C.Structure):
    _fields_ = [("data", C.c_void_p), ("n_layers", C.c_int32), ("n_seqs", C.c_int32),
                ("max_tokens", C.c_int64)]


EXPORTS = [
    "aatc_version", "aatc_layout_version", "aatc_status_string", "aatc_last_error",
    "aatc_stats_from_samples", "aatc_calibrate", "aatc_codebook_create", "aatc_codebook_create_vq",
    "aatc_codebook_vq", "aatc_codebook_info",
    "aatc_codebook_head", "aatc_codebook_fields", "aatc_codebook_save", "aatc_codebook_load", "aatc_codebook_free",
    "aatc_codebook_device_bytes", "aatc_codebook_upload", "aatc_cache_bytes", "aatc_encode",
    "aatc_encode_coeffs", "aatc_decode_workspace_bytes", "aatc_decode_attention",
    "aatc_decode_layers_workspace_bytes", "aatc_decode_attention_layers",
    "aatc_decode_attention_append", "aatc_decode_attention_static", "aatc_flush_write", "aatc_read_probe",
    "aatc_profile_begin", "aatc_profile_end",
]

_lib = None


def load() -> C.CDLL:
    """Load libaatc.so (after torch if importable, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_attention_klt_amd.build`")
    try:
        import torch  # noqa: F401
    except Exception:
        pass
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    i32, i64, dbl = C.c_int32, C.c_int64, C.c_double
    pd = C.POINTER(C.c_double)
    sig = {
        "aatc_version": ([], C.c_int),
        "aatc_layout_version": ([], C.c_int),
        "aatc_status_string": ([C.c_int], C.c_char_p),
        "aatc_last_error": ([], C.c_char_p),
        "aatc_stats_from_samples": ([i32, P, P, i64, P, i64, P, P, P, P, P, P], C.c_int),
        "aatc_calibrate": ([i32, i32, i32, i32, C.POINTER(HeadStats), C.POINTER(CalibParams),
                            C.POINTER(P)], C.c_int),
        "aatc_codebook_create": ([i32, i32, i32, i32, P, P, P, P, P, P, P, P, C.POINTER(P)], C.c_int),
        "aatc_codebook_create_vq": ([i32, i32, i32, i32, P, P, P, P, i32, P, P, P, P, P, C.POINTER(P)], C.c_int),
        "aatc_codebook_vq": ([P, i32, P, P, P, P], C.c_int),
        "aatc_codebook_info": ([P, P, P, P, P, P, P], C.c_int),
        "aatc_codebook_head": ([P, i32] + [P] * 13, C.c_int),
        "aatc_codebook_fields": ([P, i32, i32, P, P], C.c_int),
        "aatc_codebook_save": ([P, C.c_char_p], C.c_int),
        "aatc_codebook_load": ([C.c_char_p, C.POINTER(P)], C.c_int),
        "aatc_codebook_free": ([P], None),
        "aatc_codebook_device_bytes": ([P, C.POINTER(C.c_size_t)], C.c_int),
        "aatc_codebook_upload": ([P, P, C.c_size_t, P], C.c_int),
        "aatc_cache_bytes": ([P, i32, i32, i64, C.POINTER(C.c_size_t)], C.c_int),
        "aatc_encode": ([P, P, C.POINTER(Cache), i32, i32, P, P, i64, P, P, P], C.c_int),
        "aatc_encode_coeffs": ([P, P, C.POINTER(Cache), i32, i32, i64, i64, P, P], C.c_int),
        "aatc_decode_workspace_bytes": ([P, i32, i64, C.POINTER(C.c_size_t)], C.c_int),
        "aatc_decode_layers_workspace_bytes": ([P, i32, i32, i32, i64, C.POINTER(C.c_size_t)], C.c_int),
        "aatc_decode_attention_layers": ([P, P, C.POINTER(Cache), i32, i32, i32, P, P, i64, P, P, P, C.c_size_t, P],
                                         C.c_int),
        "aatc_decode_attention": ([P, P, C.POINTER(Cache), i32, i32, P, P, i64, P, P, P, C.c_size_t, P],
                                  C.c_int),
        "aatc_decode_attention_append": ([P, P, C.POINTER(Cache), i32, i32, P, P, i64, P, P, P, P, P, C.c_size_t, P],
                                         C.c_int),
        "aatc_decode_attention_static": ([P, P, C.POINTER(Cache), i32, i32, P, P, i64, P, P, P], C.c_int),
        "aatc_flush_write": ([P, C.c_size_t, P], C.c_int),
        "aatc_read_probe": ([P, C.c_size_t, i32, i32, P, P], C.c_int),
        "aatc_profile_begin": ([i32], C.c_int),
        "aatc_profile_end": ([C.POINTER(C.c_float), C.POINTER(i32)], C.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(rc: int):
    if rc != OK:
        raise AatcError(rc, load().aatc_last_error().decode())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _dev(t) -> Optional[int]:
    """Device pointer of a torch tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def version() -> int:
    return load().aatc_version()


def layout_version() -> int:
    return load().aatc_layout_version()


def status_string(status: int) -> str:
    return load().aatc_status_string(status).decode()


# ------------------------------------------------------------------------------ host calibration
def stats_from_samples(K: np.ndarray, V: np.ndarray, Q: np.ndarray) -> dict:
    """aatc_stats_from_samples on float32 host arrays K, V [n, d], Q [nq, d]."""
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    Q = np.ascontiguousarray(Q, np.float32)
    n, d = K.shape
    out = {k: np.zeros(d) for k in ("muK", "muV")}
    for k in ("SigK", "SigV", "MQ"):
        out[k] = np.zeros((d, d))
    g = np.zeros(1)
    _check(load().aatc_stats_from_samples(d, _ptr(K), _ptr(V), n, _ptr(Q), Q.shape[0], _ptr(out["muK"]),
                                          _ptr(out["muV"]), _ptr(out["SigK"]), _ptr(out["SigV"]),
                                          _ptr(out["MQ"]), _ptr(g)))
    out["gammaV"] = float(g[0])
    out["d"] = d
    return out


class Codebook:
    """Owner of an aatc_codebook* (freed on garbage collection)."""

    def __init__(self, handle: int):
        self.handle = C.c_void_p(handle)
        d, nl, nkv, grp, tb, tby = (C.c_int32() for _ in range(6))
        _check(load().aatc_codebook_info(self.handle, C.byref(d), C.byref(nl), C.byref(nkv), C.byref(grp),
                                         C.byref(tb), C.byref(tby)))
        self.d, self.n_layers, self.n_kv, self.group = d.value, nl.value, nkv.value, grp.value
        self.total_bits, self.tile_bytes = tb.value, tby.value

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.aatc_codebook_free(self.handle)
            self.handle = None

    @property
    def n_heads(self):
        return self.n_layers * self.n_kv

    def head(self, h: int) -> dict:
        d = self.d
        r = {k: np.zeros((d, d)) for k in ("UK", "UV")}
        for k in ("lamK", "lamV", "muK", "muV", "xK", "xV"):
            r[k] = np.zeros(d)
        r["bK"] = np.zeros(d, np.int32)
        r["bV"] = np.zeros(d, np.int32)
        r["stepK"] = np.zeros(d, np.float32)
        r["stepV"] = np.zeros(d, np.float32)
        th = np.zeros(1)
        _check(load().aatc_codebook_head(self.handle, h, _ptr(r["UK"]), _ptr(r["UV"]), _ptr(r["lamK"]),
                                         _ptr(r["lamV"]), _ptr(r["muK"]), _ptr(r["muV"]), _ptr(r["xK"]),
                                         _ptr(r["xV"]), _ptr(r["bK"]), _ptr(r["bV"]), _ptr(r["stepK"]),
                                         _ptr(r["stepV"]), _ptr(th)))
        r["theta"] = float(th[0])
        return r

    def vq(self, h: int):
        """Vector-quantized keys of head h: None for scalar keys, else dict(groups [n_g, 4],
        scale32 [d], cent32 [n_g, 256, 4])."""
        n = C.c_int32()
        _check(load().aatc_codebook_vq(self.handle, h, C.byref(n), None, None, None))
        if n.value == 0:
            return None
        ch = np.zeros((n.value, 4), np.int32)
        sc = np.zeros(self.d, np.float32)
        ce = np.zeros((n.value, 256, 4), np.float32)
        _check(load().aatc_codebook_vq(self.handle, h, C.byref(n), _ptr(ch), _ptr(sc), _ptr(ce)))
        return dict(groups=ch.astype(np.int64), scale32=sc, cent32=ce)

    def fields(self, h: int, which: int) -> list:
        """Record fields of head h (which: 0 keys, 1 values) as (chan, width, shift, byte, pos)."""
        n = C.c_int32(0)
        buf = np.zeros(384, np.uint32)
        _check(load().aatc_codebook_fields(self.handle, h, which, _ptr(buf), C.byref(n)))
        return [(int(x) & 0xFF, (int(x) >> 8) & 0xF, (int(x) >> 12) & 0xF, int(x) >> 20, (int(x) >> 16) & 0xF)
                for x in buf[:n.value]]

    def save(self, path: str):
        _check(load().aatc_codebook_save(self.handle, path.encode()))

    def device_bytes(self) -> int:
        n = C.c_size_t()
        _check(load().aatc_codebook_device_bytes(self.handle, C.byref(n)))
        return n.value

    def upload(self, d_blob, stream=None):
        _check(load().aatc_codebook_upload(self.handle, _dev(d_blob), d_blob.numel() * d_blob.element_size(),
                                           _stream(stream)))

    def cache_bytes(self, n_layers: int, n_seqs: int, max_tokens: int) -> int:
        n = C.c_size_t()
        _check(load().aatc_cache_bytes(self.handle, n_layers, n_seqs, max_tokens, C.byref(n)))
        return n.value

    def decode_layers_workspace_bytes(self, layer0: int, n_layers: int, n_seqs: int, max_len: int) -> int:
        n = C.c_size_t()
        _check(load().aatc_decode_layers_workspace_bytes(self.handle, layer0, n_layers, n_seqs, max_len, C.byref(n)))
        return n.value

    def decode_workspace_bytes(self, n_seqs: int, max_len: int) -> int:
        n = C.c_size_t()
        _check(load().aatc_decode_workspace_bytes(self.handle, n_seqs, max_len, C.byref(n)))
        return n.value


def calibrate(stats: Sequence[dict], d: int, n_layers: int, n_kv: int, group: int, avg_bits: float,
              max_bits: int = 8, joint: bool = True, max_sweeps: int = 0, key_transform: str = "klt",
              key_quantizer: str = "scalar", vq_normals=None, vq_iters: int = 0) -> Codebook:
    """aatc_calibrate over per-head statistics dicts (muK, muV, SigK, SigV, MQ, gammaV);
    key_transform "klt" (orthogonal) or "nova" (attention-optimal, non-orthogonal);
    key_quantizer "scalar" or "vq" (vq_normals: [n, 4] standard normal training draws)."""
    kt = {"klt": 0, "nova": 1}.get(key_transform)
    if kt is None:
        raise ValueError(f"unknown key transform {key_transform!r}")
    kq = {"scalar": 0, "vq": 1}.get(key_quantizer)
    if kq is None:
        raise ValueError(f"unknown key quantizer {key_quantizer!r}")
    normals = None if vq_normals is None else np.ascontiguousarray(vq_normals, np.float64).reshape(-1, 4)
    keep = []
    arr = (HeadStats * len(stats))()
    for i, s in enumerate(stats):
        a = [np.ascontiguousarray(s[k], np.float64) for k in ("muK", "muV", "SigK", "SigV", "MQ")]
        keep.append(a)
        pd = C.POINTER(C.c_double)
        arr[i] = HeadStats(*(x.ctypes.data_as(pd) for x in a), float(s["gammaV"]))
    p = CalibParams(avg_bits, max_bits, 1 if joint else 0, max_sweeps, kt, kq, vq_iters,
                    None if normals is None else normals.ctypes.data, 0 if normals is None else normals.shape[0])
    out = C.c_void_p()
    _check(load().aatc_calibrate(d, n_layers, n_kv, group, arr, C.byref(p), C.byref(out)))
    return Codebook(out.value)


def codebook_create(d: int, n_layers: int, n_kv: int, group: int, UK, UV, muK, muV, bK, bV, stepK,
                    stepV) -> Codebook:
    """aatc_codebook_create from per-head arrays stacked along the first axis."""
    a = [np.ascontiguousarray(x, np.float64) for x in (UK, UV, muK, muV)]
    b = [np.ascontiguousarray(x, np.int32) for x in (bK, bV)]
    s = [np.ascontiguousarray(x, np.float32) for x in (stepK, stepV)]
    out = C.c_void_p()
    _check(load().aatc_codebook_create(d, n_layers, n_kv, group, *(_ptr(x) for x in a), *(_ptr(x) for x in b),
                                       *(_ptr(x) for x in s), C.byref(out)))
    return Codebook(out.value)


def codebook_create_vq(d: int, n_layers: int, n_kv: int, group: int, UK, UV, muK, muV, vq_chan,
                       vq_scale, vq_cent, bV, stepV) -> Codebook:
    """aatc_codebook_create_vq from per-head arrays stacked along the first axis:
    vq_chan [heads, n_groups, 4], vq_scale [heads, d], vq_cent [heads, n_groups, 256, 4]."""
    a = [np.ascontiguousarray(x, np.float64) for x in (UK, UV, muK, muV)]
    ch = np.ascontiguousarray(vq_chan, np.int32)
    sc = np.ascontiguousarray(vq_scale, np.float32)
    ce = np.ascontiguousarray(vq_cent, np.float32)
    bv = np.ascontiguousarray(bV, np.int32)
    sv = np.ascontiguousarray(stepV, np.float32)
    out = C.c_void_p()
    _check(load().aatc_codebook_create_vq(d, n_layers, n_kv, group, *(_ptr(x) for x in a), ch.shape[-2],
                                          _ptr(ch), _ptr(sc), _ptr(ce), _ptr(bv), _ptr(sv), C.byref(out)))
    return Codebook(out.value)


def codebook_load(path: str) -> Codebook:
    out = C.c_void_p()
    _check(load().aatc_codebook_load(path.encode(), C.byref(out)))
    return Codebook(out.value)


# ------------------------------------------------------------------------------ device calls
def make_cache(data, n_layers: int, n_seqs: int, max_tokens: int) -> Cache:
    return Cache(_dev(data), n_layers, n_seqs, max_tokens)


def encode(cb: Codebook, d_blob, cache: Cache, layer: int, seq_ids: Sequence[int],
           start_pos: Sequence[int], n_tokens: int, K, V, stream=None):
    """aatc_encode: K, V device bf16 tensors [n_seqs, n_tokens, n_kv, d] (as int16/bfloat16)."""
    ids = np.ascontiguousarray(seq_ids, np.int32)
    st = np.ascontiguousarray(start_pos, np.int64)
    _check(load().aatc_encode(cb.handle, _dev(d_blob), C.byref(cache), layer, ids.size, _ptr(ids), _ptr(st),
                              n_tokens, _dev(K), _dev(V), _stream(stream)))


def encode_coeffs(cb: Codebook, d_blob, cache: Cache, layer: int, seq: int, start_pos: int, n_tokens: int,
                  coeffs, stream=None):
    """aatc_encode_coeffs: coeffs device float32 [n_tokens, n_kv, 2, d]."""
    _check(load().aatc_encode_coeffs(cb.handle, _dev(d_blob), C.byref(cache), layer, seq, start_pos, n_tokens,
                                     _dev(coeffs), _stream(stream)))


def decode_attention(cb: Codebook, d_blob, cache: Cache, layer: int, seq_ids, seq_lens, max_len: int, q, out,
                     workspace, stream=None):
    """aatc_decode_attention: seq_ids int32 / seq_lens int64 device tensors, q bf16 device
    [n_seqs, H_q, d], out float32 device [n_seqs, H_q, d]."""
    _check(load().aatc_decode_attention(cb.handle, _dev(d_blob), C.byref(cache), layer, seq_ids.numel(),
                                        _dev(seq_ids), _dev(seq_lens), max_len, _dev(q), _dev(out),
                                        _dev(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream)))


def decode_attention_layers(cb: Codebook, d_blob, cache: Cache, layer0: int, n_layers: int, seq_ids, seq_lens,
                            max_len: int, q, out, workspace, stream=None):
    """aatc_decode_attention_layers: layers [layer0, layer0 + n_layers) at once; q bf16 device
    [n_layers, n_seqs, H_q, d], out float32 device of the same shape."""
    _check(load().aatc_decode_attention_layers(cb.handle, _dev(d_blob), C.byref(cache), layer0, n_layers,
                                               seq_ids.numel(), _dev(seq_ids), _dev(seq_lens), max_len, _dev(q),
                                               _dev(out), _dev(workspace), workspace.numel() * workspace.element_size(),
                                               _stream(stream)))


def decode_attention_append(cb: Codebook, d_blob, cache: Cache, layer: int, seq_ids, seq_lens, max_len: int, k_new,
                            v_new, q, out, workspace, stream=None):
    """aatc_decode_attention_append: k_new, v_new bf16 device [n_seqs, n_kv, d] are written
    at slot seq_lens[s] (the tokens cached before the call) and attended to together with
    the cached tokens; the caller advances seq_lens afterwards."""
    _check(load().aatc_decode_attention_append(cb.handle, _dev(d_blob), C.byref(cache), layer, seq_ids.numel(),
                                               _dev(seq_ids), _dev(seq_lens), max_len, _dev(k_new), _dev(v_new),
                                               _dev(q), _dev(out), _dev(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_attention_static(cb: Codebook, d_blob, cache: Cache, layer: int, seq_ids, seq_lens, max_len: int, q,
                            out, stream=None):
    """aatc_decode_attention_static: as decode_attention, with the partials in the library's
    own device array instead of a caller workspace (no allocation anywhere in the call)."""
    _check(load().aatc_decode_attention_static(cb.handle, _dev(d_blob), C.byref(cache), layer, seq_ids.numel(),
                                               _dev(seq_ids), _dev(seq_lens), max_len, _dev(q), _dev(out),
                                               _stream(stream)))


def flush_write(buf, stream=None):
    _check(load().aatc_flush_write(_dev(buf), buf.numel() * buf.element_size(), _stream(stream)))


def read_probe(src, mode: int, sink, tile_bytes: int = 0, nbytes: int | None = None, stream=None):
    """aatc_read_probe: stream `nbytes` (default: all) of device tensor src; mode 0 register
    loads, mode 1 tiles of tile_bytes into LDS like the decode kernel."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(load().aatc_read_probe(_dev(src), n, mode, tile_bytes, _dev(sink), _stream(stream)))


def profile_begin(n: int):
    """aatc_profile_begin: time the split-decode kernel of the next n decode calls."""
    _check(load().aatc_profile_begin(n))


def profile_end(n: int) -> np.ndarray:
    """aatc_profile_end: the recorded kernel durations (ms) of the calls since profile_begin(n)."""
    ms = np.zeros(n, np.float32)
    got = C.c_int32(0)
    _check(load().aatc_profile_end(ms.ctypes.data_as(C.POINTER(C.c_float)), C.byref(got)))
    return ms[:got.value].copy()
