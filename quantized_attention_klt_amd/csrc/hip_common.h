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

// The quantizer of the bf16 encode paths, on the projection u = t + 2^(b-1) - 1/2 (the
// encoder bases carry the factor 1/step and the start value the offset): u clamped to
// [0, cmax = 2^b - 1], rounded to the nearest integer (ties to even) and written into byte
// `byte` of acc (v_cvt_pk_u8_f32).  Equal to clamp(floor(t) + 2^(b-1), 0, 2^b - 1) except
// where t + 2^(b-1) is an odd integer: on a cell edge, where the fp32 projection's own
// rounding decides the code anyway.
__device__ __forceinline__ uint32_t code_byte(float u, float cmax, uint32_t byte, uint32_t acc) {
    return __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(u, 0.0f, cmax), byte, acc);
}

// Nearest codeword of the weighted key coefficients (u0, u1, u2, u3) among cent[0..255]
// (one group of vector-quantized keys): t_k = u_k - z_k, distance (t0 t0 + t1 t1) +
// (t2 t2 + t3 t3), each operation rounded to fp32 (contraction off), lowest index on ties.
__device__ __forceinline__ uint32_t vq_nearest(const float (*__restrict__ cent)[kVqDim], float u0, float u1, float u2,
                                               float u3) {
#pragma clang fp contract(off)
    float best = __builtin_inff();
    uint32_t bi = 0;
    for (int i = 0; i < kVqSize; ++i) {
        const float4 z = *(const float4*)cent[i];
        const float t0 = u0 - z.x, t1 = u1 - z.y, t2 = u2 - z.z, t3 = u3 - z.w;
        const float e = (t0 * t0 + t1 * t1) + (t2 * t2 + t3 * t3);
        if (e < best) {
            best = e;
            bi = (uint32_t)i;
        }
    }
    return bi;
}

}  // namespace aatc
