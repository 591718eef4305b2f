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
constexpr int kEncodeSlots = 768;  // resident encode workgroups the launch aims for

struct SeqArgs {
    int32_t n;
    int32_t seq[kMaxSeqPerLaunch];
    int64_t start[kMaxSeqPerLaunch];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// quantizer: t = c * inv (one fp32 rounding), code = clamp(floor(t) + 2^(b-1), 0, 2^b - 1)
__device__ __forceinline__ uint32_t quantize(float c, float inv, int b) {
    float t = __fmul_rn(c, inv);
    float v = floorf(t) + (float)(1 << (b - 1));
    v = fminf(fmaxf(v, 0.0f), (float)((1 << b) - 1));
    return (uint32_t)v;
}

// Field tables of one record (keys or values) staged in LDS: fields sorted by (byte, pos)
// (chan | width << 8 | shift << 12 | pos << 16 | byte << 20) and per record byte the first
// field index.
struct FieldTab {
    uint32_t field[aatc::kMaxFields];
    int16_t first[aatc::kMaxRecordBytes + 8];
};

__device__ void stage_fields(const DevHead& H, bool isV, FieldTab& ft, int tid, int nthreads) {
    const uint32_t* f = isV ? H.fieldV : H.fieldK;
    const int16_t* fb = isV ? H.fbyteV : H.fbyteK;
    const int nf = isV ? H.nfV : H.nfK;
    const int nb = (isV ? H.BV : H.BK) / 8;
    for (int i = tid; i < nf; i += nthreads) ft.field[i] = f[i];
    for (int i = tid; i <= nb; i += nthreads) ft.first[i] = fb[i];
}

// record byte q of the slot whose codes are codes[chan * 64] (one byte per code, stride 64)
__device__ __forceinline__ uint32_t record_byte(const FieldTab& ft, const uint8_t* codes, int q) {
    uint32_t byte = 0u;
    for (int f = ft.first[q]; f < ft.first[q + 1]; ++f) {
        const uint32_t fw = ft.field[f];
        const uint32_t chan = fw & 0xff, w = (fw >> 8) & 0xf, e = (fw >> 12) & 0xf, pos = (fw >> 16) & 0xf;
        byte |= (((uint32_t)codes[chan * 64] >> e) & ((1u << w) - 1u)) << pos;
    }
    return byte;
}

// Pack one block of a tile from its codes (LDS codes[chan][slot]) for the slots [s0, s1):
// the key block is word-major (word 64 r + s = record word r of slot s), the value block
// byte-major (word 16 q + u = record byte q of slots 4u .. 4u + 3).  Stored bytes carry bit
// 7 inverted; a value word shared with slots outside [s0, s1) keeps their stored bytes.
__device__ void pack_block(const FieldTab& ft, bool isV, int nbytes, const uint8_t* codes, uint32_t* dst, int s0,
                           int s1, int tid, int nthreads) {
    const int nwords = 16 * nbytes;  // 64 slots x nbytes / 4
    for (int i = tid; i < nwords; i += nthreads) {
        uint32_t word = 0u, keep = 0u;
        if (!isV) {
            const int r = i >> 6, s = i & 63;
            if (s < s0 || s >= s1) continue;
#pragma unroll
            for (int b = 0; b < 4; ++b) word |= record_byte(ft, codes + s, 4 * r + b) << (8 * b);
        } else {
            const int q = i >> 4, u = i & 15;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int s = 4 * u + b;
                if (s >= s0 && s < s1)
                    word |= record_byte(ft, codes + s, q) << (8 * b);
                else
                    keep |= 0xFFu << (8 * b);
            }
            if (keep == 0xFFFFFFFFu) continue;
        }
        word ^= 0x80808080u & ~keep;
        if (keep) word |= dst[i] & keep;
        dst[i] = word;
    }
}

__device__ __forceinline__ uint8_t* tile_ptr(uint8_t* cache, int layer, int n_seqs_cache, int seq, int n_kv, int h,
                                             int64_t n_tiles_cap, int64_t tile, int tile_bytes) {
    return cache + ((((int64_t)layer * n_seqs_cache + seq) * n_kv + h) * n_tiles_cap + tile) * (int64_t)tile_bytes;
}

// ------------------------------------------------------------------------------------
// encode from bf16 K, V (MFMA): a workgroup owns one (sequence, kv-head, keys | values)
// and the tiles bx, bx + gridDim.x, ... of the call.  c = x (U_hi + U_lo) - bias on
// v_mfma_f32_16x16x32_bf16: rows = tokens, columns = channels; wave w keeps the B operands
// (U^T hi / lo fragments) of its D / 4 channels in registers for all its tiles.  The 64-token
// x tile is staged in LDS with its 16-byte chunks XOR-swizzled by token, so that the 16
// rows an operand read touches fall in distinct banks.
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void encode_mfma_kernel(const DevHead* __restrict__ blob, uint8_t* __restrict__ cache,
                                                          int layer, int n_kv, int64_t n_tiles_cap, int tile_bytes,
                                                          SeqArgs sa, int64_t n_tokens, int64_t ntiles,
                                                          const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                          int n_seqs_cache) {
    constexpr int CH = D / 8;          // 16-byte chunks per token row
    constexpr int CBW = D / 64;        // 16-channel column blocks per wave
    constexpr int KS = D / 32;         // k-steps
    constexpr int XB = 64 * D * 2;     // bytes of one x tile
    constexpr int NLD = 64 * CH / 256;  // chunk loads per thread
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][XB];
    __shared__ __attribute__((aligned(16))) uint8_t codes[D * 64];
    __shared__ FieldTab ft;
    const int h = blockIdx.y >> 1, kv = blockIdx.y & 1, zi = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
    const DevHead& H = blob[layer * n_kv + h];
    const uint16_t* X = (kv ? V : K) + ((int64_t)zi * n_tokens * n_kv + h) * D;  // token t at X + t * n_kv * D
    const int64_t xstride = (int64_t)n_kv * D;
    const int64_t start = sa.start[zi];
    const int64_t first_tile = start / kTile;
    const int seq = sa.seq[zi];
    stage_fields(H, kv, ft, tid, 256);
    // B operands and quantizer constants of this lane's channels j = 16 (w CBW + cbw) + c
    bf16x8 bh[CBW][KS], bl[CBW][KS];
    float bias[CBW], inv[CBW];
    int bits[CBW];
    {
        const uint16_t* uh = kv ? H.UVt_hi : H.UKt_hi;
        const uint16_t* ul = kv ? H.UVt_lo : H.UKt_lo;
#pragma unroll
        for (int cbw = 0; cbw < CBW; ++cbw) {
            const int j = 16 * (w * CBW + cbw) + c;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bh[cbw][ks] = *(const bf16x8*)(uh + j * D + 32 * ks + 8 * g);
                bl[cbw][ks] = *(const bf16x8*)(ul + j * D + 32 * ks + 8 * g);
            }
            bias[cbw] = kv ? H.biasV[j] : H.biasK[j];
            inv[cbw] = kv ? H.invV[j] : H.invK[j];
            bits[cbw] = kv ? H.bitsV[j] : H.bitsK[j];
        }
    }
    const int nbytes = (kv ? H.BV : H.BK) / 8;
    const int boff = kv ? 8 * H.BK : 0;  // block offset in the tile
    // x tile of tile index k (chunk n of this thread: token t = ci / CH, chunk ci % CH);
    // slots outside the call's tokens read as zero
    auto load_x = [&](int64_t tile, u32x4 (&r)[NLD]) {
        const int64_t tok0 = tile * kTile;
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const int ci = tid + 256 * n, t = ci / CH, kc = ci % CH;
            const int64_t tt = tok0 + t - start;  // token index in this call's input
            r[n] = (tt >= 0 && tt < n_tokens) ? *(const u32x4*)(X + tt * xstride + 8 * kc) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_x = [&](int buf, const u32x4 (&r)[NLD]) {
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            const int ci = tid + 256 * n, t = ci / CH, kc = ci % CH;
            *(u32x4*)(&xs[buf][t * 2 * D + 16 * (kc ^ (t & (CH - 1)))]) = r[n];
        }
    };
    int64_t tile = blockIdx.x;
    u32x4 xr[NLD];
    if (tile < ntiles) {
        load_x(first_tile + tile, xr);
        store_x(0, xr);
    }
    __syncthreads();
    for (int k = 0; tile < ntiles; ++k, tile += gridDim.x) {
        const int buf = k & 1;
        const int64_t tile_n = tile + gridDim.x;
        if (tile_n < ntiles) load_x(first_tile + tile_n, xr);  // next tile, in flight during the MFMAs
        f32x4 acc[CBW][4];
#pragma unroll
        for (int cbw = 0; cbw < CBW; ++cbw)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[cbw][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int t = 16 * tb + c;  // A row: token
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 av = *(const bf16x8*)(&xs[buf][t * 2 * D + 16 * ((4 * ks + g) ^ (t & (CH - 1)))]);
#pragma unroll
                for (int cbw = 0; cbw < CBW; ++cbw) {
                    acc[cbw][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[cbw][ks], acc[cbw][tb], 0, 0, 0);
                    acc[cbw][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[cbw][ks], acc[cbw][tb], 0, 0, 0);
                }
            }
        }
        // codes of tokens 16 tb + 4 g + e, channel 16 (w CBW + cbw) + c -> codes[j][token]
#pragma unroll
        for (int cbw = 0; cbw < CBW; ++cbw) {
            const int j = 16 * (w * CBW + cbw) + c;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                uint32_t wv = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t code = bits[cbw] ? quantize(acc[cbw][tb][e] - bias[cbw], inv[cbw], bits[cbw]) : 0u;
                    wv |= code << (8 * e);
                }
                *(uint32_t*)(&codes[j * 64 + 16 * tb + 4 * g]) = wv;
            }
        }
        __syncthreads();
        const int64_t tok0 = (first_tile + tile) * kTile;
        const int s0 = (int)max(start - tok0, (int64_t)0);
        const int s1 = (int)min(start + n_tokens - tok0, (int64_t)kTile);
        uint8_t* tp = tile_ptr(cache, layer, n_seqs_cache, seq, n_kv, h, n_tiles_cap, first_tile + tile, tile_bytes);
        pack_block(ft, kv, nbytes, codes, (uint32_t*)(tp + boff), s0, s1, tid, 256);
        if (tile_n < ntiles) store_x(buf ^ 1, xr);
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------
// encode given KLT coefficients: one workgroup per (tile, kv-head, sequence); codes of
// both blocks in LDS, then both blocks packed.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void encode_coeffs_kernel(const DevHead* __restrict__ blob,
                                                            uint8_t* __restrict__ cache, int layer, int n_kv,
                                                            int64_t n_tiles_cap, int tile_bytes, SeqArgs sa,
                                                            int64_t n_tokens, const float* __restrict__ coeffs,
                                                            int n_seqs_cache) {
    __shared__ __attribute__((aligned(16))) uint8_t codes[2][aatc::kMaxD * 64];
    __shared__ FieldTab ft[2];
    const int h = blockIdx.y, zi = blockIdx.z;
    const DevHead& H = blob[layer * n_kv + h];
    const int d = H.d;
    const int64_t start = sa.start[zi];
    const int64_t tile = start / kTile + blockIdx.x;
    const int64_t tok0 = tile * kTile;
    const int s0 = (int)std::max<int64_t>(start - tok0, 0);
    const int s1 = (int)std::min<int64_t>(start + n_tokens - tok0, kTile);
    stage_fields(H, false, ft[0], threadIdx.x, blockDim.x);
    stage_fields(H, true, ft[1], threadIdx.x, blockDim.x);
    for (int i = threadIdx.x; i < (s1 - s0) * 2 * d; i += blockDim.x) {
        const int s = s0 + i / (2 * d), r = i % (2 * d), kv = r / d, j = r % d;
        const int64_t t = tok0 + s - start;  // token index in this call's input
        const float cf = coeffs[((t * n_kv + h) * 2 + kv) * d + j];
        const int b = kv ? H.bitsV[j] : H.bitsK[j];
        codes[kv][j * 64 + s] = b ? (uint8_t)quantize(cf, kv ? H.invV[j] : H.invK[j], b) : 0;
    }
    __syncthreads();
    uint8_t* tp = tile_ptr(cache, layer, n_seqs_cache, sa.seq[zi], n_kv, h, n_tiles_cap, tile, tile_bytes);
    pack_block(ft[0], false, H.BK / 8, codes[0], (uint32_t*)tp, s0, s1, threadIdx.x, blockDim.x);
    pack_block(ft[1], true, H.BV / 8, codes[1], (uint32_t*)(tp + 8 * H.BK), s0, s1, threadIdx.x, blockDim.x);
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
        const uint16_t* Kz = K ? K + (size_t)s0 * n_tokens * cb->n_kv * d : nullptr;
        const uint16_t* Vz = V ? V + (size_t)s0 * n_tokens * cb->n_kv * d : nullptr;
        if (coeffs) {
            hipLaunchKernelGGL(encode_coeffs_kernel, dim3((unsigned)ntiles, (unsigned)cb->n_kv, (unsigned)used), dim3(256),
                               0, (hipStream_t)stream, blob, (uint8_t*)cache->data, layer, cb->n_kv, ncap, tile_bytes, sa,
                               n_tokens, coeffs, cache->n_seqs);
        } else {
            // workgroups per (sequence, kv-head, keys | values): fill the resident slots
            const int64_t units = (int64_t)used * cb->n_kv * 2;
            const unsigned wx = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ntiles, kEncodeSlots / units));
            const dim3 grid(wx, (unsigned)(2 * cb->n_kv), (unsigned)used);
            if (d == 64)
                hipLaunchKernelGGL(encode_mfma_kernel<64>, grid, dim3(256), 0, (hipStream_t)stream, blob,
                                   (uint8_t*)cache->data, layer, cb->n_kv, ncap, tile_bytes, sa, n_tokens, ntiles, Kz, Vz,
                                   cache->n_seqs);
            else
                hipLaunchKernelGGL(encode_mfma_kernel<128>, grid, dim3(256), 0, (hipStream_t)stream, blob,
                                   (uint8_t*)cache->data, layer, cb->n_kv, ncap, tile_bytes, sa, n_tokens, ntiles, Kz, Vz,
                                   cache->n_seqs);
        }
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
