"""The rounding-window check the GPU flip tests apply (util.edge_ratio), pinned on the CPU:
codes from a different but legitimate fp32 evaluation (the bf16 encoder's: bases scaled by
the reciprocal step and split into bf16 hi + lo, fp32 products and sums in BLAS order, the
offset 2^(b-1) - 1/2 - mu W as the start value, the result clamped and rounded to nearest)
differ from the oracle's codes only inside the window, while a code moved by one level at
a random coded position falls outside it."""
import numpy as np

import oracle
import synth
from util import Case, edge_ratio


def _bf16(x):
    return synth.bf16_bits_to_f64(synth.to_bf16_bits(x)).astype(np.float32)


def _folded_codes(x64, mu, U, inv, bits):
    W = (U * inv.astype(np.float64)[None, :]).astype(np.float32)
    hi = _bf16(W)
    lo = _bf16(W - hi)
    Wd = hi.astype(np.float64) + lo.astype(np.float64)
    half = np.where(bits > 0, 2.0 ** (bits - 1), 0.0)
    start = np.where(bits > 0, half - 0.5 - mu @ Wd, 0.0).astype(np.float32)
    x32 = x64.astype(np.float32)
    u = (x32 @ hi + x32 @ lo) + start[None, :]
    cmax = (2.0 ** bits - 1).astype(np.float32)
    return np.rint(np.clip(u, 0.0, cmax[None, :])).astype(np.int64)  # nearest, ties to even


def test_fp32_evaluation_flips_lie_in_the_window_and_planted_flips_do_not():
    case = Case("llama_32k", 32768, n_kv=1, n_calib_q=64)
    cb = case.cbs[0]
    flips = 0
    for which, x64, U, mu, bits in (("K", case.kf(0, 0), cb.UK, cb.muK, cb.bK),
                                    ("V", case.vf(0, 0), cb.UV, cb.muV, cb.bV)):
        inv = cb.inv_step(which)
        ref = oracle.quantize(oracle.transform_coeffs(x64, mu, U), inv, bits).astype(np.int64)
        alt = _folded_codes(x64, mu, U, inv, bits)
        m = np.broadcast_to(bits > 0, alt.shape)
        bad = np.argwhere((alt != ref) & m)
        assert np.abs(alt - ref)[m].max() <= 1
        assert edge_ratio(x64, mu, U, inv, bits, bad) <= 1.0
        flips += len(bad)
        # planted: one level off at random coded positions
        rng = np.random.default_rng(11)
        coded = np.argwhere(m)
        pick = coded[rng.choice(len(coded), 200, replace=False)]
        outside = sum(edge_ratio(x64, mu, U, inv, bits, p[None]) > 1.0 for p in pick)
        assert outside >= 190, outside
    assert flips > 0  # the alternative evaluation does flip codes, so the window is exercised
