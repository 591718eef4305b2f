// HIP kernels (gfx950) of the transform-coded KV cache and the device side of the C ABI:
// codebook upload, encode (projection + quantize + bit-pack), query transform,
// split-context decode attention over the packed cache, split combine + inverse transform.
//
// Pages: "Attention-Aware Transform Coding Guide" (KLT section: K' = K U_K; listing's
// compress step: rotate, quantize per channel, dequantize and rotate back); "Spend Bits
// Where Queries Look" abstract (fixed per-token bit count; decoding reads the cache at
// every step and is bandwidth-bound).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "aatc_internal.h"

using aatc::DevHead;
using aatc::kTile;
using aatc::set_error;

#define HIP_TRY(expr)                                                                              \
    do {                                                                                           \
        hipError_t e_ = (expr);                                                                    \
        if (e_ != hipSuccess) return set_error(AATC_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

namespace {

constexpr int kMaxSeqPerLaunch = 64;
constexpr float kLog2e = 1.4426950408889634f;

struct SeqArgs {
    int32_t n;
    int32_t seq[kMaxSeqPerLaunch];
    int64_t start[kMaxSeqPerLaunch];
};

__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// quantizer: t = c * inv (one fp32 rounding), code = clamp(floor(t) + 2^(b-1), 0, 2^b - 1)
__device__ __forceinline__ uint32_t quantize(float c, float inv, int b) {
    float t = __fmul_rn(c, inv);
    float v = floorf(t) + (float)(1 << (b - 1));
    v = fminf(fmaxf(v, 0.0f), (float)((1 << b) - 1));
    return (uint32_t)v;
}

// OR a field of `w` bits (w <= 8) at bit position `pos` of an LDS word array.
__device__ __forceinline__ void lds_put(uint32_t* words, uint32_t pos, uint32_t val, int w) {
    uint32_t wi = pos >> 5, sh = pos & 31;
    atomicOr(&words[wi], val << sh);
    if (sh + w > 32) atomicOr(&words[wi + 1], val >> (32 - sh));
}

__device__ __forceinline__ uint32_t lds_get(const uint32_t* words, uint32_t pos, int w) {
    uint32_t wi = pos >> 5, sh = pos & 31;
    uint64_t two = (uint64_t)words[wi] | ((sh + w > 32) ? ((uint64_t)words[wi + 1] << 32) : 0ull);
    return (uint32_t)(two >> sh) & ((1u << w) - 1u);
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
    for (int i = threadIdx.x; i < nw; i += blockDim.x) words[i] = tw[i];
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
            const uint16_t* hi = kv ? H.UVhi : H.UKhi;
            const uint16_t* lo = kv ? H.UVlo : H.UKlo;
            float acc = 0.0f;
            for (int ii = 0; ii < d; ++ii) acc = fmaf(bf16f(x[ii]), bf16f(hi[ii * d + j]) + bf16f(lo[ii * d + j]), acc);
            c = acc - (kv ? H.biasV[j] : H.biasK[j]);
        }
        int b = kv ? H.bitsV[j] : H.bitsK[j];
        codes[(s * 2 + kv) * d + j] = b ? (uint8_t)quantize(c, kv ? H.invV[j] : H.invK[j], b) : 0;
    }
    __syncthreads();
    // quantize + pack: one (slot, piece) per thread iteration
    const int nKp = H.nKp, nVp = H.nVp;
    const int np = nKp + nVp;
    for (int i = threadIdx.x; i < (s1 - s0) * np; i += blockDim.x) {
        int s = s0 + i / np;
        int p = i % np;
        bool isK = p < nKp;
        int pw = isK ? H.pieceK[p] : H.pieceV[p - nKp];
        int chan = pw & 0xff, w = (pw >> 8) & 0xf, e = (pw >> 12) & 0xf, off = pw >> 16;
        uint32_t code = codes[(s * 2 + (isK ? 0 : 1)) * d + chan];
        uint32_t val = (code >> e) & ((1u << w) - 1u);
        uint32_t pos;
        if (isK) {
            pos = (uint32_t)s * BK + off;
        } else {
            int per = 32 / w, r = s / per, k = s % per;
            pos = 64u * BK + 64u * off + 32u * r + 8u * (k & 3) + (uint32_t)w * (k >> 2);
        }
        lds_put(words, pos, val, w);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nw; i += blockDim.x) tw[i] = words[i];
}

// ------------------------------------------------------------------------------------
// query transform: q'' = (U_K^T q) * step_K * log2(e) / sqrt(d), KLT channel order
// ------------------------------------------------------------------------------------
__global__ void qtransform_kernel(const DevHead* __restrict__ blob, int layer, int n_kv, int group,
                                  const uint16_t* __restrict__ q, float* __restrict__ qpp) {
    const int hq = blockIdx.x, z = blockIdx.y, j = threadIdx.x;
    const int nq = n_kv * group;
    const DevHead& H = blob[layer * n_kv + hq / group];
    const int d = H.d;
    const uint16_t* qv = q + ((int64_t)z * nq + hq) * d;
    float acc = 0.0f;
    for (int i = 0; i < d; ++i) acc = fmaf(H.UK[i * d + j], bf16f(qv[i]), acc);
    float scale = kLog2e / sqrtf((float)d);
    qpp[((int64_t)z * nq + hq) * d + j] = H.bitsK[j] ? acc * H.stepK[j] * scale : 0.0f;
}

// ------------------------------------------------------------------------------------
// split decode: one workgroup per (split, kv-head, sequence); scores and value sums in
// the code domain, online softmax in base 2.  Partials: m, l, acc[d] per query head.
// ------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void decode_split_kernel(const DevHead* __restrict__ blob, const uint8_t* __restrict__ cache,
                                                           int layer, int n_kv, int group, int n_seqs_cache,
                                                           int64_t n_tiles_cap, int tile_bytes, int tiles_per_split,
                                                           const int32_t* __restrict__ seq_ids,
                                                           const int64_t* __restrict__ seq_lens,
                                                           const float* __restrict__ qpp, float* __restrict__ part,
                                                           int n_split, int64_t max_len) {
    extern __shared__ uint32_t smem[];
    const int split = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
    const DevHead& H = blob[layer * n_kv + h];
    const int d = H.d, BK = H.BK, nKp = H.nKp, nVp = H.nVp;
    const int G = group, nq = n_kv * group;
    // device-side arguments are clamped so that a bad length or id cannot read outside
    // the cache (such a sequence produces an empty or truncated result instead)
    const int seq = seq_ids[z];
    int64_t len = std::min<int64_t>(std::min<int64_t>(seq_lens[z], max_len), n_tiles_cap * kTile);
    if (seq < 0 || seq >= n_seqs_cache) len = 0;
    const int64_t n_tiles = (len + kTile - 1) / kTile;
    const int64_t t0 = (int64_t)split * tiles_per_split;
    const int64_t t1 = std::min<int64_t>(t0 + tiles_per_split, n_tiles);

    uint32_t* words = smem;                              // tile_bytes/4
    float* qs = (float*)(smem + tile_bytes / 4);         // [G][d]
    float* pr = qs + G * d;                              // [G][64] probabilities
    float* accP = pr + G * kTile;                        // [G][nVp]
    float* stat = accP + G * nVp;                        // m[G], l[G], alpha[G]
    const int nw = tile_bytes / 4;

    for (int i = threadIdx.x; i < G * d; i += blockDim.x)
        qs[i] = qpp[((int64_t)z * nq + h * G + i / d) * d + (i % d)];
    for (int i = threadIdx.x; i < G * nVp; i += blockDim.x) accP[i] = 0.0f;
    if (threadIdx.x < G) {
        stat[threadIdx.x] = -INFINITY;
        stat[G + threadIdx.x] = 0.0f;
    }
    const uint8_t* base = cache + (((int64_t)layer * n_seqs_cache + seq) * n_kv + h) * n_tiles_cap * (int64_t)tile_bytes;
    for (int64_t t = t0; t < t1; ++t) {
        __syncthreads();
        const uint32_t* tw = (const uint32_t*)(base + t * (int64_t)tile_bytes);
        for (int i = threadIdx.x; i < nw; i += blockDim.x) words[i] = tw[i];
        __syncthreads();
        const int valid = (int)std::min<int64_t>(kTile, len - t * kTile);
        // scores
        for (int i = threadIdx.x; i < G * kTile; i += blockDim.x) {
            int g = i / kTile, s = i % kTile;
            float sc = -INFINITY;
            if (s < valid) {
                sc = 0.0f;
                for (int p = 0; p < nKp; ++p) {
                    int pw = H.pieceK[p];
                    int chan = pw & 0xff, w = (pw >> 8) & 0xf, e = (pw >> 12) & 0xf, off = pw >> 16;
                    uint32_t v = lds_get(words, (uint32_t)s * BK + off, w);
                    sc = fmaf(qs[g * d + chan] * (float)(1 << e), (float)v, sc);
                }
            }
            pr[i] = sc;
        }
        __syncthreads();
        // online softmax: one thread per query head (G <= 16, 64 tokens each)
        if (threadIdx.x < G) {
            int g = threadIdx.x;
            float mx = -INFINITY;
            for (int s = 0; s < kTile; ++s) mx = fmaxf(mx, pr[g * kTile + s]);
            float mold = stat[g];
            float mnew = fmaxf(mold, mx);
            float alpha = exp2f(mold - mnew);
            float sum = 0.0f;
            for (int s = 0; s < kTile; ++s) {
                float pv = exp2f(pr[g * kTile + s] - mnew);
                pr[g * kTile + s] = pv;
                sum += pv;
            }
            stat[g] = mnew;
            stat[G + g] = stat[G + g] * alpha + sum;
            stat[2 * G + g] = alpha;
        }
        __syncthreads();
        // value pieces
        for (int i = threadIdx.x; i < G * nVp; i += blockDim.x) {
            int g = i / nVp, p = i % nVp;
            int pw = H.pieceV[p];
            int w = (pw >> 8) & 0xf, off = pw >> 16;
            int per = 32 / w;
            float acc = 0.0f;
            for (int s = 0; s < valid; ++s) {
                int r = s / per, k = s % per;
                uint32_t pos = 64u * BK + 64u * off + 32u * r + 8u * (k & 3) + (uint32_t)w * (k >> 2);
                acc = fmaf(pr[g * kTile + s], (float)lds_get(words, pos, w), acc);
            }
            accP[i] = accP[i] * stat[2 * G + g] + acc;
        }
    }
    __syncthreads();
    // write partials: m, l, acc per channel (pieces summed with their weights)
    for (int i = threadIdx.x; i < G * (d + 2); i += blockDim.x) {
        int g = i / (d + 2), c = i % (d + 2);
        float v;
        if (c == 0) {
            v = stat[g];
        } else if (c == 1) {
            v = stat[G + g];
        } else {
            int j = c - 2;
            v = 0.0f;
            for (int p = 0; p < nVp; ++p) {
                int pw = H.pieceV[p];
                if ((pw & 0xff) == j) v += accP[g * nVp + p] * (float)(1 << ((pw >> 12) & 0xf));
            }
        }
        part[(((int64_t)z * nq + h * G + g) * n_split + split) * (d + 2) + c] = v;
    }
}

// combine splits, dequantize value coefficients, inverse transform, add the value mean
__global__ void decode_combine_kernel(const DevHead* __restrict__ blob, int layer, int n_kv, int group,
                                      const float* __restrict__ part, int n_split, float* __restrict__ out) {
    __shared__ float cbar[aatc::kMaxD];
    const int hq = blockIdx.x, z = blockIdx.y, j = threadIdx.x;
    const int nq = n_kv * group;
    const DevHead& H = blob[layer * n_kv + hq / group];
    const int d = H.d;
    const float* P = part + ((int64_t)z * nq + hq) * n_split * (d + 2);
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, P[s * (d + 2)]);
    float L = 0.0f, A = 0.0f;
    for (int s = 0; s < n_split; ++s) {
        float m = P[s * (d + 2)];
        if (m == -INFINITY) continue;
        float sc = exp2f(m - M);
        L += P[s * (d + 2) + 1] * sc;
        A += P[s * (d + 2) + 2 + j] * sc;
    }
    int b = H.bitsV[j];
    cbar[j] = b ? H.stepV[j] * (A / L - (float)(1 << (b - 1)) + 0.5f) : 0.0f;
    __syncthreads();
    float o = H.muV[j];
    for (int c = 0; c < d; ++c) o = fmaf(H.UV[j * d + c], cbar[c], o);
    out[((int64_t)z * nq + hq) * d + j] = o;
}

__global__ void flush_kernel(uint4* p, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = make_uint4((uint32_t)i, 0u, 0u, 0u);
}

// ------------------------------------------------------------------------------------
// host helpers
// ------------------------------------------------------------------------------------
int64_t n_tiles_of(int64_t max_tokens) { return (max_tokens + kTile - 1) / kTile; }

int decode_splits(const aatc_codebook* cb, int n_seqs, int64_t max_len) {
    int64_t tiles = std::max<int64_t>(1, n_tiles_of(max_len));
    int64_t want = (512 + (int64_t)n_seqs * cb->n_kv - 1) / ((int64_t)n_seqs * cb->n_kv);
    return (int)std::max<int64_t>(1, std::min<int64_t>(want, tiles));
}

int check_cache(const aatc_codebook* cb, const aatc_cache* cache, int layer) {
    if (!cache || !cache->data) return set_error(AATC_ERR_INVALID_ARG, "null cache");
    if (layer < 0 || layer >= cb->n_layers || layer >= cache->n_layers)
        return set_error(AATC_ERR_INVALID_ARG, "layer %d out of range", layer);
    if (cache->n_seqs < 1 || cache->max_tokens < 1) return set_error(AATC_ERR_INVALID_ARG, "empty cache geometry");
    if (((uintptr_t)cache->data) & 15) return set_error(AATC_ERR_INVALID_ARG, "cache pointer not 16-byte aligned");
    return AATC_OK;
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

extern "C" int aatc_decode_workspace_bytes(const aatc_codebook* cb, int32_t n_seqs, int64_t max_len, size_t* bytes) {
    if (!cb || !bytes) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n_seqs < 1 || max_len < 1) return set_error(AATC_ERR_INVALID_ARG, "need n_seqs >= 1 and max_len >= 1");
    const int S = decode_splits(cb, n_seqs, max_len);
    const size_t nq = (size_t)cb->n_kv * cb->group;
    *bytes = (size_t)n_seqs * nq * cb->d * sizeof(float) + (size_t)n_seqs * nq * S * (cb->d + 2) * sizeof(float) + 256;
    return AATC_OK;
}

extern "C" int aatc_decode_attention(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                     int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const int64_t* seq_lens,
                                     int64_t max_len, const uint16_t* q, float* out, void* workspace,
                                     size_t ws_bytes, void* stream) {
    if (!cb || !d_blob) return set_error(AATC_ERR_INVALID_ARG, "null codebook or blob");
    int rc = check_cache(cb, cache, layer);
    if (rc) return rc;
    if (n_seqs < 1 || n_seqs > cache->n_seqs || !seq_ids || !seq_lens || !q || !out || !workspace)
        return set_error(AATC_ERR_INVALID_ARG, "bad decode arguments");
    if (max_len < 1 || max_len > cache->max_tokens)
        return set_error(AATC_ERR_CAPACITY, "max_len %lld outside [1, %lld]", (long long)max_len, (long long)cache->max_tokens);
    size_t need = 0;
    aatc_decode_workspace_bytes(cb, n_seqs, max_len, &need);
    if (ws_bytes < need) return set_error(AATC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    if (cb->group > 16) return set_error(AATC_ERR_UNSUPPORTED, "group > 16");
    const int S = decode_splits(cb, n_seqs, max_len);
    const int64_t tiles = n_tiles_of(max_len);
    const int tps = (int)((tiles + S - 1) / S);
    const int d = cb->d, G = cb->group, nq = cb->n_kv * G;
    const int tile_bytes = 8 * cb->total_bits;
    float* qpp = (float*)workspace;
    float* part = qpp + (size_t)n_seqs * nq * d;
    const DevHead* blob = (const DevHead*)d_blob;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(qtransform_kernel, dim3(nq, n_seqs), dim3(d), 0, st, blob, layer, cb->n_kv, G, q, qpp);
    HIP_TRY(hipGetLastError());
    int max_nvp = 0;
    for (int h = 0; h < cb->n_kv; ++h) max_nvp = std::max(max_nvp, cb->blob[layer * cb->n_kv + h].nVp);
    size_t shmem = (size_t)tile_bytes + sizeof(float) * ((size_t)G * d + (size_t)G * kTile + (size_t)G * max_nvp + 3 * G);
    hipLaunchKernelGGL(decode_split_kernel, dim3(S, cb->n_kv, n_seqs), dim3(256), shmem, st, blob,
                       (const uint8_t*)cache->data, layer, cb->n_kv, G, cache->n_seqs, n_tiles_of(cache->max_tokens),
                       tile_bytes, tps, seq_ids, seq_lens, qpp, part, S, max_len);
    HIP_TRY(hipGetLastError());
    hipLaunchKernelGGL(decode_combine_kernel, dim3(nq, n_seqs), dim3(d), 0, st, blob, layer, cb->n_kv, G, part, S, out);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}

extern "C" int aatc_flush_write(void* d_buf, size_t bytes, void* stream) {
    if (!d_buf) return set_error(AATC_ERR_INVALID_ARG, "null buffer");
    size_t n = bytes / sizeof(uint4);
    if (n == 0) return AATC_OK;
    hipLaunchKernelGGL(flush_kernel, dim3(2048), dim3(256), 0, (hipStream_t)stream, (uint4*)d_buf, n);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}
