"""CPU oracle for Attention-Aware Transform Coding (AATC) of KV caches.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  The library never calls it, and it
shares no code with the library (no kernels, headers, helpers or tables); both
take their inputs from the separate seeded generators in ``synth``.

Everything is plain numpy in float64 unless a step fixes another precision
(the fp32 quantizer arithmetic, whose rounding decides integer codes).  Each
function cites the passage of the AATC pages it follows:

* p1 = "KV Cache Compression Through the Lens of Transform Coding" (arxivlens
  summary page): abstract, Methodology, Limitations.
* p2 = "Attention-Aware Transform Coding Guide: KV Compression" (blog):
  sections "Formal Attention Distortion Model", "Theorem: Additive Error
  Decomposition", "Decorrelation via the Karhunen-Loeve Transform (KLT)",
  "Optimal Bit Allocation via Reverse Water-Filling", and its code listing
  (taken as a description only).
* p3 = "Spend Bits Where Queries Look" (NOVA-KV) abstract: fixed per-token
  bit count, bandwidth-bound decoding, and a non-orthogonal key transform under which
  attention distortion becomes transform-domain MSE (nova_key_transform); vector
  quantization of the key coefficients with equal-volume groups and equal-size
  codebooks (oracle.vq).

Readings taken where the pages are silent, garbled or contradict each other
are stated in the docstring of the function that takes them.  Parity status:
every public function is pinned by a CPU test against closed forms, brute
force or textbook values (tests/test_oracle_*.py); the packed layout is ours
and is pinned by an independent bit-by-bit implementation in the tests.
"""
from .calib import (  # noqa: F401
    head_stats, klt, channel_weights, waterfill_theta, allocate_bits,
    uniform_quantizer_mse, optimal_step, build_head_codebook, HeadCodebook,
    nova_key_transform, key_weights_general,
)
from .codec import (  # noqa: F401
    fields, quantize, transform_coeffs, pack_cache, unpack_cache, dequantize,
    reconstruct, tile_bytes, record_bits, encode_cache, key_record_bits,
)
from .vq import (  # noqa: F401
    VQ_DIM, VQ_SIZE, coded_key_channels, equal_volume_groups, group_log_volumes, lloyd,
    group_codebooks, vq_scales, vq_encode, vq_dequantize,
)
from .attention import (  # noqa: F401
    attention, decoded_kv, decode_attention, predicted_distortion, monte_carlo_distortion,
)
