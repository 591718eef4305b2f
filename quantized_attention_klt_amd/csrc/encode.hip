// HIP encoder (gfx950) of the transform-coded KV cache and the device side of the C ABI
// for codebook upload, cache sizing, encode (projection + quantize + bit-pack) and the
// cache-flush helper.
//
// Pages: "Attention-Aware Transform Coding Guide" (KLT section: K' = K U_K; listing's
// compress step: rotate, quantize per channel, dequantize and rotate back); "Spend Bits
// Where Queries Look" abstract (fixed per-token bit count; decoding reads the cache at
// every step and is bandwidth-bound).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "hip_common.h"

using aatc::bf16f;
using aatc::check_cache;
using aatc::DevHead;
using aatc::kTile;
using aatc::n_tiles_of;
using aatc::set_error;

namespace {

constexpr int kMaxSeqPerLaunch = 64;

struct SeqArgs {
    int32_t n;
    int32_t seq[kMaxSeqPerLaunch];
    int64_t start[kMaxSeqPerLaunch];
};

// quantizer: t = c * inv (one fp32 rounding), code = clamp(floor(t) + 2^(b-1), 0, 2^b - 1)
__device__ __forceinline__ uint32_t quantize(float c, float inv, int b) {
    float t = __fmul_rn(c, inv);
    float v = floorf(t) + (float)(1 << (b - 1));
    v = fminf(fmaxf(v, 0.0f), (float)((1 << b) - 1));
    return (uint32_t)v;
}

// Bytes of tile word i that belong to slots in [s0, s1): a key-block word (i < nkw) is
// one slot's (slot i % 64); a value-block word holds slots 4 (i % 16) + b in byte b.
__device__ __forceinline__ uint32_t written_mask(int i, int nkw, int s0, int s1) {
    if (i < nkw) {
        const int s = i & 63;
        return s >= s0 && s < s1 ? 0xFFFFFFFFu : 0u;
    }
    const int sb = 4 * ((i - nkw) & 15);
    uint32_t m = 0u;
    for (int b = 0; b < 4; ++b)
        if (sb + b >= s0 && sb + b < s1) m |= 0xFFu << (8 * b);
    return m;
}

// ------------------------------------------------------------------------------------
// encode: one workgroup per (tile, kv-head, sequence).  Coefficients either come in
// (FROM_COEFFS) or are computed as c = x (U_hi + U_lo) - bias in fp32.
// ------------------------------------------------------------------------------------
template <bool FROM_COEFFS>
__global__ __launch_bounds__(256) void encode_kernel(const DevHead* __restrict__ blob, uint8_t* __restrict__ cache,
                                                     int n_layers_seqs_base, int layer, int n_kv, int64_t n_tiles_cap,
                                                     int tile_bytes, SeqArgs sa, int64_t n_tokens,
                                                     const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                     const float* __restrict__ coeffs, int n_seqs_cache) {
    extern __shared__ uint32_t smem[];
    const int h = blockIdx.y;
    const int zi = blockIdx.z;
    const DevHead& H = blob[layer * n_kv + h];
    const int d = H.d, BK = H.BK;
    const int64_t start = sa.start[zi];
    const int64_t first_tile = start / kTile;
    const int64_t tile = first_tile + blockIdx.x;
    // slots of this tile written by this call
    const int64_t tok0 = tile * kTile;
    const int s0 = (int)std::max<int64_t>(start - tok0, 0);
    const int s1 = (int)std::min<int64_t>(start + n_tokens - tok0, kTile);
    uint32_t* words = smem;
    uint8_t* codes = (uint8_t*)(smem + tile_bytes / 4);  // [64][2][d] codes of this tile
    const int nw = tile_bytes / 4;
    const int seq = sa.seq[zi];
    uint8_t* tp = cache + ((((int64_t)layer * n_seqs_cache + seq) * n_kv + h) * n_tiles_cap + tile) * (int64_t)tile_bytes;
    uint32_t* tw = (uint32_t*)tp;
    // The records of the slots written here are rebuilt from zero (their stored bytes carry
    // bit 7 inverted): key-block word i belongs to slot i % 64; value-block word i holds
    // byte plane (i / 16), slots 4 (i % 16) .. 4 (i % 16) + 3.
    const int nkw = 2 * BK;  // 64 slots * BK / 32 words
    for (int i = threadIdx.x; i < nw; i += blockDim.x) words[i] = tw[i] & ~written_mask(i, nkw, s0, s1);
    // codes of the slots being written
    for (int i = threadIdx.x; i < (s1 - s0) * 2 * d; i += blockDim.x) {
        int s = s0 + i / (2 * d);
        int r = i % (2 * d);
        int kv = r / d, j = r % d;
        int64_t t = tok0 + s - start;  // token index in this call's input
        float c;
        if (FROM_COEFFS) {
            c = coeffs[((t * n_kv + h) * 2 + kv) * d + j];
        } else {
            const uint16_t* x = (kv ? V : K) + ((int64_t)zi * n_tokens + t) * n_kv * d + (int64_t)h * d;
            const uint16_t* hi = (kv ? H.UVt_hi : H.UKt_hi) + j * d;
            const uint16_t* lo = (kv ? H.UVt_lo : H.UKt_lo) + j * d;
            float acc = 0.0f;
            for (int ii = 0; ii < d; ++ii) acc = fmaf(bf16f(x[ii]), bf16f(hi[ii]) + bf16f(lo[ii]), acc);
            c = acc - (kv ? H.biasV[j] : H.biasK[j]);
        }
        int b = kv ? H.bitsV[j] : H.bitsK[j];
        codes[(s * 2 + kv) * d + j] = b ? (uint8_t)quantize(c, kv ? H.invV[j] : H.invK[j], b) : 0;
    }
    __syncthreads();
    // pack: one (slot, field) per thread iteration; fields never cross a byte
    const int nfK = H.nfK, nfV = H.nfV;
    const int nf = nfK + nfV;
    for (int i = threadIdx.x; i < (s1 - s0) * nf; i += blockDim.x) {
        const int s = s0 + i / nf;
        const int f = i % nf;
        const bool isK = f < nfK;
        const uint32_t fw = isK ? H.fieldK[f] : H.fieldV[f - nfK];
        const int chan = fw & 0xff, w = (fw >> 8) & 0xf, e = (fw >> 12) & 0xf, pos = (fw >> 16) & 0xf;
        const uint32_t q = fw >> 20;
        const uint32_t code = codes[(s * 2 + (isK ? 0 : 1)) * d + chan];
        const uint32_t val = (code >> e) & ((1u << w) - 1u);
        // key record word q/4 of slot s is block word 64 (q/4) + s; value record byte q of
        // slot s is value-block byte 64 q + s
        const uint32_t byte = isK ? 4u * (64u * (q >> 2) + (uint32_t)s) + (q & 3u) : 8u * BK + 64u * q + (uint32_t)s;
        atomicOr(&words[byte >> 2], val << (8u * (byte & 3u) + (uint32_t)pos));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nw; i += blockDim.x) tw[i] = words[i] ^ (written_mask(i, nkw, s0, s1) & 0x80808080u);
}

__global__ void flush_kernel(uint4* p, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = make_uint4((uint32_t)i, 0u, 0u, 0u);
}

}  // namespace

// ======================================================================================
// C ABI: device side
// ======================================================================================
extern "C" int aatc_codebook_device_bytes(const aatc_codebook* cb, size_t* bytes) {
    if (!cb || !bytes) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    *bytes = cb->blob.size() * sizeof(DevHead);
    return AATC_OK;
}

extern "C" int aatc_codebook_upload(const aatc_codebook* cb, void* d_blob, size_t bytes, void* stream) {
    if (!cb || !d_blob) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    size_t need = cb->blob.size() * sizeof(DevHead);
    if (bytes < need) return set_error(AATC_ERR_WORKSPACE, "blob buffer has %zu bytes, needs %zu", bytes, need);
    if (((uintptr_t)d_blob) & 255) return set_error(AATC_ERR_INVALID_ARG, "blob pointer must be 256-byte aligned");
    HIP_TRY(hipMemcpyAsync(d_blob, cb->blob.data(), need, hipMemcpyHostToDevice, (hipStream_t)stream));
    return AATC_OK;
}

extern "C" int aatc_cache_bytes(const aatc_codebook* cb, int32_t n_layers, int32_t n_seqs, int64_t max_tokens,
                                size_t* bytes) {
    if (!cb || !bytes) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n_layers < 1 || n_layers > cb->n_layers || n_seqs < 1 || max_tokens < 1)
        return set_error(AATC_ERR_INVALID_ARG, "bad cache geometry");
    *bytes = (size_t)n_layers * n_seqs * cb->n_kv * n_tiles_of(max_tokens) * (size_t)(8 * cb->total_bits);
    return AATC_OK;
}

static int encode_common(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache, int32_t layer,
                         int32_t n_seqs, const int32_t* seq_ids, const int64_t* start_pos, int64_t n_tokens,
                         const uint16_t* K, const uint16_t* V, const float* coeffs, void* stream) {
    if (!cb || !d_blob) return set_error(AATC_ERR_INVALID_ARG, "null codebook or blob");
    int rc = check_cache(cb, cache, layer);
    if (rc) return rc;
    if (n_seqs < 1 || !seq_ids || !start_pos) return set_error(AATC_ERR_INVALID_ARG, "need n_seqs >= 1 and host seq arrays");
    if (n_tokens < 0) return set_error(AATC_ERR_INVALID_ARG, "negative n_tokens");
    if (!coeffs && (!K || !V)) return set_error(AATC_ERR_INVALID_ARG, "null K/V");
    for (int s = 0; s < n_seqs; ++s) {
        if (seq_ids[s] < 0 || seq_ids[s] >= cache->n_seqs) return set_error(AATC_ERR_INVALID_ARG, "seq id %d out of range", seq_ids[s]);
        if (start_pos[s] < 0 || start_pos[s] + n_tokens > cache->max_tokens)
            return set_error(AATC_ERR_CAPACITY, "sequence %d: slots [%lld, %lld) exceed capacity %lld", seq_ids[s],
                             (long long)start_pos[s], (long long)(start_pos[s] + n_tokens), (long long)cache->max_tokens);
    }
    if (n_tokens == 0) return AATC_OK;
    const int tile_bytes = 8 * cb->total_bits;
    const int d = cb->d;
    const size_t shmem = (size_t)tile_bytes + (size_t)kTile * 2 * d;
    const int64_t ncap = n_tiles_of(cache->max_tokens);
    const DevHead* blob = (const DevHead*)d_blob;
    for (int s0 = 0; s0 < n_seqs;) {
        int nz = std::min(kMaxSeqPerLaunch, n_seqs - s0);
        // sequences sharing a launch must touch the same number of tiles
        SeqArgs sa;
        std::memset(&sa, 0, sizeof sa);
        int64_t ntiles = -1;
        int used = 0;
        for (int i = 0; i < nz; ++i) {
            int64_t st = start_pos[s0 + i];
            int64_t nt = (st + n_tokens - 1) / kTile - st / kTile + 1;
            if (ntiles >= 0 && nt != ntiles) break;
            ntiles = nt;
            sa.seq[i] = seq_ids[s0 + i];
            sa.start[i] = st;
            ++used;
        }
        sa.n = used;
        dim3 grid((unsigned)ntiles, (unsigned)cb->n_kv, (unsigned)used);
        const uint16_t* Kz = K ? K + (size_t)s0 * n_tokens * cb->n_kv * d : nullptr;
        const uint16_t* Vz = V ? V + (size_t)s0 * n_tokens * cb->n_kv * d : nullptr;
        if (coeffs)
            hipLaunchKernelGGL(encode_kernel<true>, grid, dim3(256), shmem, (hipStream_t)stream, blob,
                               (uint8_t*)cache->data, 0, layer, cb->n_kv, ncap, tile_bytes, sa, n_tokens, Kz, Vz, coeffs,
                               cache->n_seqs);
        else
            hipLaunchKernelGGL(encode_kernel<false>, grid, dim3(256), shmem, (hipStream_t)stream, blob,
                               (uint8_t*)cache->data, 0, layer, cb->n_kv, ncap, tile_bytes, sa, n_tokens, Kz, Vz, nullptr,
                               cache->n_seqs);
        HIP_TRY(hipGetLastError());
        s0 += used;
    }
    return AATC_OK;
}

extern "C" int aatc_encode(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache, int32_t layer,
                           int32_t n_seqs, const int32_t* seq_ids, const int64_t* start_pos, int64_t n_tokens,
                           const uint16_t* K, const uint16_t* V, void* stream) {
    return encode_common(cb, d_blob, cache, layer, n_seqs, seq_ids, start_pos, n_tokens, K, V, nullptr, stream);
}

extern "C" int aatc_encode_coeffs(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache, int32_t layer,
                                  int32_t seq, int64_t start_pos, int64_t n_tokens, const float* coeffs, void* stream) {
    if (!coeffs) return set_error(AATC_ERR_INVALID_ARG, "null coefficients");
    return encode_common(cb, d_blob, cache, layer, 1, &seq, &start_pos, n_tokens, nullptr, nullptr, coeffs, stream);
}

extern "C" int aatc_flush_write(void* d_buf, size_t bytes, void* stream) {
    if (!d_buf) return set_error(AATC_ERR_INVALID_ARG, "null buffer");
    size_t n = bytes / sizeof(uint4);
    if (n == 0) return AATC_OK;
    hipLaunchKernelGGL(flush_kernel, dim3(2048), dim3(256), 0, (hipStream_t)stream, (uint4*)d_buf, n);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}
