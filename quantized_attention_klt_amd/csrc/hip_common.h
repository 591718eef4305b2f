// Helpers shared by the HIP translation units: error macro, cache geometry checks and small
// device utilities.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "aatc_internal.h"

#define HIP_TRY(expr)                                                                                     \
    do {                                                                                                  \
        hipError_t e_ = (expr);                                                                           \
        if (e_ != hipSuccess) return aatc::set_error(AATC_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

namespace aatc {

inline int64_t n_tiles_of(int64_t max_tokens) { return (max_tokens + kTile - 1) / kTile; }

inline int check_cache(const aatc_codebook* cb, const aatc_cache* cache, int layer) {
    if (!cache || !cache->data) return set_error(AATC_ERR_INVALID_ARG, "null cache");
    if (layer < 0 || layer >= cb->n_layers || layer >= cache->n_layers)
        return set_error(AATC_ERR_INVALID_ARG, "layer %d out of range", layer);
    if (cache->n_seqs < 1 || cache->max_tokens < 1) return set_error(AATC_ERR_INVALID_ARG, "empty cache geometry");
    if (((uintptr_t)cache->data) & 15) return set_error(AATC_ERR_INVALID_ARG, "cache pointer not 16-byte aligned");
    return AATC_OK;
}

__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// The scalar quantizer of every encode path: t = c * inv (one fp32 rounding),
// code = clamp(floor(t) + 2^(b-1), 0, 2^b - 1) (b >= 1).
__device__ __forceinline__ uint32_t quantize(float c, float inv, int b) {
    const float v = floorf(__fmul_rn(c, inv)) + (float)(1 << (b - 1));
    return (uint32_t)__builtin_amdgcn_fmed3f(v, 0.0f, (float)((1 << b) - 1));
}

}  // namespace aatc
