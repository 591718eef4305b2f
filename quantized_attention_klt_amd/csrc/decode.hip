// Split-context decode attention over the packed cache (gfx950).
//
// Pages: "Attention-Aware Transform Coding Guide" ("Formal Attention Distortion Model":
// o = softmax(q K^T / sqrt(d)) V; KLT section K' = K U_K, so q.k = (U_K^T q).(U_K^T k) and
// keys are scored in the transform domain and never reconstructed; values are
// inverse-transformed once per query head); "Spend Bits Where Queries Look" abstract
// (decoding reads the whole cache every step and is bandwidth-bound).
//
// Three kernels, all on the caller's stream:
//   qprep   : q' = U_K^T q per query head, scaled by the key steps (and log2 e / sqrt d),
//             split into three int8 digits and laid out as the A operands of the score
//             MFMAs of each kv-head (the slot order follows the key unpack schedule).
//   decode  : workgroups of 4 waves; each wave streams a run of 64-token tiles through LDS
//             (direct global->LDS loads, double-buffered), unpacks key pieces with SWAR
//             shift/mask into int8 operands and runs v_mfma_i32_16x16x64_i8 for the scores,
//             keeps an online softmax (base 2) with a lazily rescaled reference maximum,
//             turns probabilities into three int8 digits and accumulates P x value-piece
//             codes with the same MFMA into int32.  Waves of a workgroup merge their
//             (max, sum, accumulator) partials in LDS.
//   combine : log-sum-exp merge of the workgroup partials, dequantisation of the value
//             coefficients, inverse transform U_V and the value mean.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "hip_common.h"

using aatc::check_cache;
using aatc::DevHead;
using aatc::kTile;
using aatc::n_tiles_of;
using aatc::set_error;

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kTargetWaves = 2048;   // waves per launch (8 per CU on 256 CUs)
constexpr float kHeadroom = 2.0f;    // log2 headroom added to the reference max at a rescale
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kM4 = 0x0F0F0F0Fu, kM2 = 0x03030303u, kM1 = 0x01010101u;

struct DecodeArgs {
    int layer, n_kv, G, n_seqs_cache;
    int64_t n_tiles_cap;
    int64_t max_len;
    int tile_bytes, tpw, wg_per_head, nqb_max;
    // LDS carve-up (bytes)
    int off_qsc, off_kdw, off_vslab, off_wave, wave_bytes, buf_bytes;
};

// 32 bits of an LDS word array starting at an arbitrary bit position
__device__ __forceinline__ uint32_t bits32(const uint32_t* w, uint32_t bit) {
    uint32_t i = bit >> 5;
    return __builtin_amdgcn_alignbit(w[i + 1], w[i], bit & 31);
}

// order this wave's earlier LDS writes before its later LDS reads
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float reduce16_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    return v;
}

__device__ __forceinline__ float reduce16_sum(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

// Stream one tile (bytes, a multiple of 16) from global memory into LDS, 16 bytes per lane
// per instruction (LDS address = base + 16 * lane).
__device__ __forceinline__ void load_tile(const uint8_t* src, uint8_t* lds, int bytes, int lane) {
    for (int off = 0; off < bytes; off += 1024) {
        int o = off + 16 * lane;
        if (o < bytes)
            __builtin_amdgcn_global_load_lds((const void*)(src + o),
                                             (__attribute__((address_space(3))) void*)(lds + off), 16, 0, 0);
    }
}

// ---------------------------------------------------------------------------------------
// query preparation: int8 digits of q'' in the A-operand layout of the score MFMAs
// ---------------------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(256) void qprep_kernel(const DevHead* __restrict__ blob, int layer, int n_kv, int G,
                                                    int nqb_max, const uint16_t* __restrict__ q,
                                                    int8_t* __restrict__ qa_out, float* __restrict__ qsc_out) {
    __shared__ float qpp[16][aatc::kMaxD];
    __shared__ float scale[16];
    const int h = blockIdx.x, z = blockIdx.y, tid = threadIdx.x;
    const DevHead& H = blob[layer * n_kv + h];
    const int d = H.d, nq = n_kv * G;
    const float qs = kLog2e / sqrtf((float)d);
    for (int i = tid; i < G * d; i += blockDim.x) {
        int g = i / d, j = i % d;
        const uint16_t* qv = q + ((int64_t)z * nq + h * G + g) * d;
        float acc = 0.0f;
        for (int ii = 0; ii < d; ++ii) acc = fmaf(H.UK[ii * d + j], aatc::bf16f(qv[ii]), acc);
        qpp[g][j] = H.bitsK[j] ? acc * H.stepK[j] * qs : 0.0f;
    }
    __syncthreads();
    if (tid < G) {
        float mx = 0.0f;
        for (int j = 0; j < d; ++j) {
            int b = H.bitsK[j];
            if (!b) continue;
            int top = b >= 4 ? b - 4 : (b >= 2 ? b - 2 : 0);  // shift of the channel's top piece
            mx = fmaxf(mx, fabsf(qpp[tid][j]) * (float)(1 << top));
        }
        scale[tid] = mx > 0.0f ? mx / 127.0f : 1.0f;
    }
    __syncthreads();
    const int nqb = H.nqb[0] + H.nqb[1] + H.nqb[2];
    int8_t* qa = qa_out + ((int64_t)z * n_kv + h) * nqb_max * RB * 1024;
    for (int i = tid; i < nqb * RB * 1024; i += blockDim.x) {
        int b = i & 15, lane = (i >> 4) & 63, rb = (i >> 10) % RB, qb = (i >> 10) / RB;
        int r = 16 * rb + (lane & 15), g = lane >> 4;
        int val = 0;
        if (r < 3 * G) {
            int k = r / G, hh = r % G;
            int m = H.kq_map[qb][g][b];
            if (m >= 0) {
                float x = qpp[hh][m & 255] * (float)(1 << (m >> 8)) / scale[hh];
                float d0 = rintf(x);
                float r1 = (x - d0) * 254.0f;
                float d1 = rintf(r1);
                float r2 = (r1 - d1) * 254.0f;
                float d2 = rintf(r2);
                val = (int)(k == 0 ? d0 : (k == 1 ? d1 : d2));
            }
        }
        qa[i] = (int8_t)val;
    }
    float* qsc = qsc_out + ((int64_t)z * n_kv + h) * RB * 16;
    for (int r = tid; r < RB * 16; r += blockDim.x)
        qsc[r] = r < 3 * G ? scale[r % G] * (r / G == 0 ? 1.0f : (r / G == 1 ? 1.0f / 254.0f : 1.0f / 64516.0f)) : 0.0f;
}

// ---------------------------------------------------------------------------------------
// split decode
// ---------------------------------------------------------------------------------------
template <int RB, int NVB, int NCH>
__global__ __launch_bounds__(256) void decode_kernel(const DevHead* __restrict__ blob, const uint8_t* __restrict__ cache,
                                                     DecodeArgs a, const int32_t* __restrict__ seq_ids,
                                                     const int64_t* __restrict__ seq_lens,
                                                     const int8_t* __restrict__ qa_all, const float* __restrict__ qsc_all,
                                                     float* __restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int wgi = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c = lane & 15;
    const DevHead& H = blob[a.layer * a.n_kv + h];
    const int G = a.G, d = H.d, BK = H.BK, TB = a.tile_bytes;
    const int nqb4 = H.nqb[0], nqb2 = H.nqb[1], nqb = H.nqb[0] + H.nqb[1] + H.nqb[2];
    const int nvb4 = H.nvb[0], nvb2 = H.nvb[1], nvb = H.nvb[0] + H.nvb[1] + H.nvb[2];
    const int R3 = 3 * G;

    int8_t* qa_lds = (int8_t*)smem;
    float* qsc_lds = (float*)(smem + a.off_qsc);
    int16_t* kdw_lds = (int16_t*)(smem + a.off_kdw);
    int16_t* vslab_lds = (int16_t*)(smem + a.off_vslab);
    uint8_t* wbase = smem + a.off_wave + wave * a.wave_bytes;
    uint8_t* buf[2] = {wbase, wbase + a.buf_bytes};
    float* sc = (float*)(wbase + 2 * a.buf_bytes);       // [RB*16][64] scores (log2 units)
    uint8_t* P = (uint8_t*)(sc + RB * 16 * 64);           // [RB*16][64] probability digits
    float* alpha_lds = (float*)(P + RB * 16 * 64);        // [16] per-head rescale factors

    // ---- sequence geometry (device arguments clamped: no read outside the cache)
    const int seq = seq_ids[z];
    int64_t len = min(min(seq_lens[z], a.max_len), a.n_tiles_cap * kTile);
    if (seq < 0 || seq >= a.n_seqs_cache) len = 0;
    const int64_t n_tiles = (len + kTile - 1) / kTile;
    const int64_t t_begin = ((int64_t)wgi * kWaves + wave) * a.tpw;
    const int64_t t_end = min(t_begin + a.tpw, n_tiles);
    const uint8_t* tiles = cache + (((int64_t)a.layer * a.n_seqs_cache + seq) * a.n_kv + h) * a.n_tiles_cap * TB;
    if (t_begin < t_end) load_tile(tiles + t_begin * TB, buf[0], TB, lane);

    // ---- stage per-(seq, head) operands and tables
    {
        const uint4* src = (const uint4*)(qa_all + ((int64_t)z * a.n_kv + h) * a.nqb_max * RB * 1024);
        uint4* dst = (uint4*)qa_lds;
        for (int i = tid; i < nqb * RB * 64; i += 256) dst[i] = src[i];
        const float* qs = qsc_all + ((int64_t)z * a.n_kv + h) * RB * 16;
        for (int i = tid; i < RB * 16; i += 256) qsc_lds[i] = qs[i];
        for (int i = tid; i < nqb * 8; i += 256) kdw_lds[i] = (&H.kq_dw[0][0][0])[i];
        for (int i = tid; i < nvb * 16; i += 256) vslab_lds[i] = (&H.vb_slab[0][0])[i];
        uint32_t* Pw = (uint32_t*)P;
        for (int i = lane; i < RB * 16 * 16; i += 64) Pw[i] = 0u;
    }
    __syncthreads();

    v4i acc_i[RB][NVB];
    v4f acc_f[RB][NVB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb) {
            acc_i[rb][cb] = v4i{0, 0, 0, 0};
            acc_f[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    float mref[NCH], lsum[NCH];
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) mref[cc] = -INFINITY, lsum[cc] = 0.0f;
    // digit scale of each accumulator row this lane holds (row = 16 rb + 4 g + v)
    float dsc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            int r = 16 * rb + 4 * g + v, k = r / G;
            dsc[rb][v] = r < R3 ? (k == 0 ? 1.0f / 127.0f : (k == 1 ? 1.0f / (127.0f * 254.0f) : 1.0f / (127.0f * 64516.0f)))
                                : 0.0f;
        }

    for (int64_t t = t_begin; t < t_end; ++t) {
        const int cur = (int)((t - t_begin) & 1);
        __builtin_amdgcn_s_waitcnt(0);  // tile t is in LDS
        if (t + 1 < t_end) load_tile(tiles + (t + 1) * TB, buf[cur ^ 1], TB, lane);
        const uint32_t* kw = (const uint32_t*)buf[cur];
        const uint32_t* vw = (const uint32_t*)(buf[cur] + 8 * BK);
        const int valid = (int)min((int64_t)kTile, len - t * kTile);

        // ---------------- scores: S[head-digit row][token] = sum_slots qdigit * key piece
        v4i S[4][RB];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) S[blk][rb] = v4i{0, 0, 0, 0};
        for (int qb = 0; qb < nqb; ++qb) {
            v4i A[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) A[rb] = *(const v4i*)(qa_lds + ((qb * RB + rb) * 64 + lane) * 16);
            const uint32_t o0 = 32u * (uint32_t)kdw_lds[(qb * 4 + g) * 2];
            const uint32_t o1 = 32u * (uint32_t)kdw_lds[(qb * 4 + g) * 2 + 1];
            const int mode = qb < nqb4 ? 0 : (qb < nqb4 + nqb2 ? 1 : 2);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const uint32_t rec = (uint32_t)(16 * blk + c) * (uint32_t)BK;
                const uint32_t x0 = bits32(kw, rec + o0);
                v4i B;
                if (mode == 0) {
                    const uint32_t x1 = bits32(kw, rec + o1);
                    B = v4i{(int)(x0 & kM4), (int)((x0 >> 4) & kM4), (int)(x1 & kM4), (int)((x1 >> 4) & kM4)};
                } else if (mode == 1) {
                    B = v4i{(int)(x0 & kM2), (int)((x0 >> 2) & kM2), (int)((x0 >> 4) & kM2), (int)((x0 >> 6) & kM2)};
                } else {
                    const uint32_t y = x0 >> (4 * (g & 1));
                    B = v4i{(int)(y & kM1), (int)((y >> 1) & kM1), (int)((y >> 2) & kM1), (int)((y >> 3) & kM1)};
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) S[blk][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[rb], B, S[blk][rb], 0, 0, 0);
            }
        }
        // scaled scores to LDS: sc[row][token]
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int r = 16 * rb + 4 * g + v;
                    if (r < R3) sc[r * 64 + 16 * blk + c] = (float)S[blk][rb][v] * qsc_lds[r];
                }
        wave_lds_fence();

        // ---------------- online softmax: lane handles head 4cc+g, tokens 4c..4c+3
        v4f s4[NCH];
        float tmax[NCH];
        bool need = false;
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
            tmax[cc] = -INFINITY;
            s4[cc] = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            {
                const int hh = 4 * cc + g;
                if (hh < G) {
                    v4f s = *(const v4f*)(sc + hh * 64 + 4 * c);
                    s += *(const v4f*)(sc + (G + hh) * 64 + 4 * c);
                    s += *(const v4f*)(sc + (2 * G + hh) * 64 + 4 * c);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * c + i >= valid) s[i] = -INFINITY;
                    s4[cc] = s;
                    tmax[cc] = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
                }
                tmax[cc] = reduce16_max(tmax[cc]);
                need |= tmax[cc] > mref[cc];
            }
        }
        if (__any(need)) {
            // raise the reference of the heads whose tile max passed it; fold the int
            // accumulators (relative to the old reference) into the float ones and rescale
#pragma unroll
            for (int cc = 0; cc < NCH; ++cc) {
                {
                    const int hh = 4 * cc + g;
                    float nref = tmax[cc] > mref[cc] ? tmax[cc] + kHeadroom : mref[cc];
                    float al = hh < G ? exp2f(mref[cc] - nref) : 1.0f;
                    lsum[cc] *= al;
                    mref[cc] = nref;
                    if (c == 0 && hh < G) alpha_lds[hh] = al;
                }
            }
            wave_lds_fence();
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                float al[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int r = 16 * rb + 4 * g + v;
                    al[v] = r < R3 ? alpha_lds[r % G] : 0.0f;
                }
#pragma unroll
                for (int cb = 0; cb < NVB; ++cb) {
                    if (cb < nvb) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc_f[rb][cb][v] = (acc_f[rb][cb][v] + (float)acc_i[rb][cb][v] * dsc[rb][v]) * al[v];
                        acc_i[rb][cb] = v4i{0, 0, 0, 0};
                    }
                }
            }
        }
        // probabilities as three int8 digits: p*127 = d0 + d1/254 + d2/254^2
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
            const int hh = 4 * cc + g;
            if (hh < G) {
                uint32_t w0 = 0, w1 = 0, w2 = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float p = exp2f(s4[cc][i] - mref[cc]);
                    lsum[cc] += p;
                    float x = p * 127.0f;
                    float d0 = rintf(x);
                    float r1 = (x - d0) * 254.0f;
                    float d1 = rintf(r1);
                    float d2 = rintf((r1 - d1) * 254.0f);
                    w0 |= ((uint32_t)(int)d0 & 255u) << (8 * i);
                    w1 |= ((uint32_t)(int)d1 & 255u) << (8 * i);
                    w2 |= ((uint32_t)(int)d2 & 255u) << (8 * i);
                }
                *(uint32_t*)(P + hh * 64 + 4 * c) = w0;
                *(uint32_t*)(P + (G + hh) * 64 + 4 * c) = w1;
                *(uint32_t*)(P + (2 * G + hh) * 64 + 4 * c) = w2;
            }
        }
        wave_lds_fence();

        // ---------------- values: acc[head-digit row][piece] += P digits x value pieces
        v4i Ap[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) Ap[rb] = *(const v4i*)(P + (16 * rb + c) * 64 + 16 * g);
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb) {
            if (cb < nvb) {
                const uint32_t* sw = vw + vslab_lds[cb * 16 + c];
                v4i B;
                if (cb < nvb4) {
                    const uint32_t x0 = sw[2 * g], x1 = sw[2 * g + 1];
                    B = v4i{(int)(x0 & kM4), (int)((x0 >> 4) & kM4), (int)(x1 & kM4), (int)((x1 >> 4) & kM4)};
                } else if (cb < nvb4 + nvb2) {
                    const uint32_t x = sw[g];
                    B = v4i{(int)(x & kM2), (int)((x >> 2) & kM2), (int)((x >> 4) & kM2), (int)((x >> 6) & kM2)};
                } else {
                    const uint32_t y = sw[g >> 1] >> (4 * (g & 1));
                    B = v4i{(int)(y & kM1), (int)((y >> 1) & kM1), (int)((y >> 2) & kM1), (int)((y >> 3) & kM1)};
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc_i[rb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ap[rb], B, acc_i[rb][cb], 0, 0, 0);
            }
        }
    }

    // ---------------- epilogue: fold the int accumulators, reduce digits and pieces
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb)
            if (cb < nvb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc_f[rb][cb][v] += (float)acc_i[rb][cb][v] * dsc[rb][v];
    const int ncol = 16 * nvb;
    float* accg = (float*)wbase;                       // [3G][ncol]
    float* wp = accg + R3 * ncol;                      // [G][d+2] this wave's partial
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb)
            if (cb < nvb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int r = 16 * rb + 4 * g + v;
                    if (r < R3) accg[r * ncol + 16 * cb + c] = acc_f[rb][cb][v];
                }
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
        {
            float ls = reduce16_sum(lsum[cc]);
            const int hh = 4 * cc + g;
            if (c == 0 && hh < G) {
                wp[hh * (d + 2)] = mref[cc];
                wp[hh * (d + 2) + 1] = ls;
            }
        }
    }
    wave_lds_fence();
    for (int i = lane; i < G * d; i += 64) {
        const int hh = i / d, j = i % d;
        float s = 0.0f;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int e = H.chan_cols[j][t];
            if (e < 0) break;
            const int col = e & 0xfff;
            const float wgt = (float)(1 << (e >> 12));
            s += wgt * (accg[hh * ncol + col] + accg[(G + hh) * ncol + col] + accg[(2 * G + hh) * ncol + col]);
        }
        wp[hh * (d + 2) + 2 + j] = s;
    }
    __syncthreads();
    // merge the workgroup's waves
    float* out = part + (((int64_t)z * a.n_kv + h) * a.wg_per_head + wgi) * G * (d + 2);
    for (int i = tid; i < G * (d + 2); i += 256) {
        const int hh = i / (d + 2), col = i % (d + 2);
        float M = -INFINITY;
        for (int w = 0; w < kWaves; ++w)
            M = fmaxf(M, ((const float*)(smem + a.off_wave + w * a.wave_bytes))[R3 * ncol + hh * (d + 2)]);
        float v;
        if (col == 0) {
            v = M;
        } else {
            v = 0.0f;
            for (int w = 0; w < kWaves; ++w) {
                const float* pw = (const float*)(smem + a.off_wave + w * a.wave_bytes) + R3 * ncol + hh * (d + 2);
                if (pw[0] != -INFINITY) v += pw[col] * exp2f(pw[0] - M);
            }
        }
        out[i] = v;
    }
}

// merge the workgroup partials of one (sequence, query head); dequantise and inverse-transform
__global__ void combine_kernel(const DevHead* __restrict__ blob, int layer, int n_kv, int G, int wg_per_head,
                               const float* __restrict__ part, float* __restrict__ out) {
    __shared__ float cbar[aatc::kMaxD];
    __shared__ float red[2];
    const int hq = blockIdx.x, z = blockIdx.y, j = threadIdx.x;
    const int kv = hq / G, gg = hq % G;
    const DevHead& H = blob[layer * n_kv + kv];
    const int d = H.d;
    const float* P = part + ((int64_t)z * n_kv + kv) * wg_per_head * G * (d + 2) + gg * (d + 2);
    const int stride = G * (d + 2);
    if (j == 0) {
        float M = -INFINITY;
        for (int s = 0; s < wg_per_head; ++s) M = fmaxf(M, P[s * stride]);
        float L = 0.0f;
        for (int s = 0; s < wg_per_head; ++s) {
            float m = P[s * stride];
            if (m != -INFINITY) L += P[s * stride + 1] * exp2f(m - M);
        }
        red[0] = M;
        red[1] = L;
    }
    __syncthreads();
    const float M = red[0], L = red[1];
    float A = 0.0f;
    for (int s = 0; s < wg_per_head; ++s) {
        float m = P[s * stride];
        if (m != -INFINITY) A += P[s * stride + 2 + j] * exp2f(m - M);
    }
    const int b = H.bitsV[j];
    cbar[j] = b ? H.stepV[j] * (A / L - (float)(1 << (b - 1)) + 0.5f) : 0.0f;
    __syncthreads();
    float o = H.muV[j];
    for (int cidx = 0; cidx < d; ++cidx) o = fmaf(H.UV[j * d + cidx], cbar[cidx], o);
    out[((int64_t)z * n_kv * G + hq) * d + j] = o;
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
struct Plan {
    int RB, NVB, NCH, nqb_max, nvb_max, tpw, wg_per_head;
    size_t qa_bytes, qsc_bytes, part_bytes;
    DecodeArgs args;
    size_t lds;
};

int make_plan(const aatc_codebook* cb, int layer, int n_seqs, int64_t max_len, Plan& p) {
    const int G = cb->group, d = cb->d;
    p.RB = (3 * G + 15) / 16;
    p.nqb_max = 0;
    p.nvb_max = 0;
    for (int h = 0; h < cb->n_kv; ++h) {
        const DevHead& D = cb->blob[(size_t)layer * cb->n_kv + h];
        p.nqb_max = std::max(p.nqb_max, D.nqb[0] + D.nqb[1] + D.nqb[2]);
        p.nvb_max = std::max(p.nvb_max, D.nvb[0] + D.nvb[1] + D.nvb[2]);
    }
    static const int kNvbChoices[] = {8, 12, 16, 24, 32};
    p.NVB = 32;
    for (int v : kNvbChoices)
        if (p.nvb_max <= v) {
            p.NVB = v;
            break;
        }
    p.NCH = (G + 3) / 4;
    if (p.RB > 3) return set_error(AATC_ERR_UNSUPPORTED, "query group of %d heads exceeds 16", G);
    if (p.RB > 1 && p.NVB > 16)
        return set_error(AATC_ERR_UNSUPPORTED, "%d value column blocks with a group of %d query heads", p.nvb_max, G);
    const int64_t tiles = n_tiles_of(max_len);
    const int64_t total = tiles * cb->n_kv * (int64_t)n_seqs;
    p.tpw = (int)std::max<int64_t>(1, (total + kTargetWaves - 1) / kTargetWaves);
    const int64_t waves_per_head = (tiles + p.tpw - 1) / p.tpw;
    p.wg_per_head = (int)((waves_per_head + kWaves - 1) / kWaves);
    p.qa_bytes = (size_t)n_seqs * cb->n_kv * p.nqb_max * p.RB * 1024;
    p.qsc_bytes = (size_t)n_seqs * cb->n_kv * p.RB * 16 * sizeof(float);
    p.part_bytes = (size_t)n_seqs * cb->n_kv * p.wg_per_head * G * (d + 2) * sizeof(float);
    DecodeArgs& a = p.args;
    a.G = G;
    a.tile_bytes = 8 * cb->total_bits;
    a.tpw = p.tpw;
    a.wg_per_head = p.wg_per_head;
    a.nqb_max = p.nqb_max;
    auto al16 = [](size_t x) { return (int)((x + 15) & ~(size_t)15); };
    a.off_qsc = al16((size_t)p.nqb_max * p.RB * 1024);
    a.off_kdw = al16(a.off_qsc + p.RB * 16 * sizeof(float));
    a.off_vslab = al16(a.off_kdw + (size_t)p.nqb_max * 8 * sizeof(int16_t));
    a.off_wave = al16(a.off_vslab + (size_t)p.nvb_max * 16 * sizeof(int16_t));
    a.buf_bytes = al16(a.tile_bytes + 16);
    size_t stream_part = 2 * (size_t)a.buf_bytes + p.RB * 16 * 64 * sizeof(float) + p.RB * 16 * 64 + 16 * sizeof(float);
    size_t epi_part = (size_t)3 * G * 16 * p.nvb_max * sizeof(float) + (size_t)G * (d + 2) * sizeof(float);
    a.wave_bytes = al16(std::max(stream_part, epi_part));
    p.lds = (size_t)a.off_wave + kWaves * (size_t)a.wave_bytes;
    if (p.lds > 160 * 1024) return set_error(AATC_ERR_UNSUPPORTED, "decode needs %zu bytes of LDS per workgroup", p.lds);
    return AATC_OK;
}

template <int RB, int NVB, int NCH>
int launch_decode(const Plan& p, dim3 grid, hipStream_t st, const DevHead* blob, const uint8_t* cache,
                  const int32_t* ids, const int64_t* lens, const int8_t* qa, const float* qsc, float* part) {
    static bool attr_set = false;
    if (!attr_set) {
        HIP_TRY(hipFuncSetAttribute((const void*)decode_kernel<RB, NVB, NCH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    160 * 1024));
        attr_set = true;
    }
    hipLaunchKernelGGL((decode_kernel<RB, NVB, NCH>), grid, dim3(256), p.lds, st, blob, cache, p.args, ids, lens, qa, qsc,
                       part);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}

template <int RB>
void launch_qprep(const Plan& p, int layer, int n_kv, int G, int n_seqs, hipStream_t st, const DevHead* blob,
                  const uint16_t* q, int8_t* qa, float* qsc) {
    hipLaunchKernelGGL(qprep_kernel<RB>, dim3(n_kv, n_seqs), dim3(256), 0, st, blob, layer, n_kv, G, p.nqb_max, q, qa,
                       qsc);
}

}  // namespace

extern "C" int aatc_decode_workspace_bytes(const aatc_codebook* cb, int32_t n_seqs, int64_t max_len, size_t* bytes) {
    if (!cb || !bytes) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n_seqs < 1 || max_len < 1) return set_error(AATC_ERR_INVALID_ARG, "need n_seqs >= 1 and max_len >= 1");
    size_t worst = 0;
    for (int layer = 0; layer < cb->n_layers; ++layer) {
        Plan p;
        int rc = make_plan(cb, layer, n_seqs, max_len, p);
        if (rc) return rc;
        worst = std::max(worst, ((p.qa_bytes + 255) & ~(size_t)255) + ((p.qsc_bytes + 255) & ~(size_t)255) + p.part_bytes);
    }
    *bytes = worst;
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
        return set_error(AATC_ERR_CAPACITY, "max_len %lld outside [1, %lld]", (long long)max_len,
                         (long long)cache->max_tokens);
    if (((uintptr_t)workspace) & 255) return set_error(AATC_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    Plan p;
    rc = make_plan(cb, layer, n_seqs, max_len, p);
    if (rc) return rc;
    const size_t qa_al = (p.qa_bytes + 255) & ~(size_t)255, qsc_al = (p.qsc_bytes + 255) & ~(size_t)255;
    if (ws_bytes < qa_al + qsc_al + p.part_bytes)
        return set_error(AATC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, qa_al + qsc_al + p.part_bytes);
    int8_t* qa = (int8_t*)workspace;
    float* qsc = (float*)((uint8_t*)workspace + qa_al);
    float* part = (float*)((uint8_t*)workspace + qa_al + qsc_al);
    DecodeArgs& a = p.args;
    a.layer = layer;
    a.n_kv = cb->n_kv;
    a.n_seqs_cache = cache->n_seqs;
    a.n_tiles_cap = n_tiles_of(cache->max_tokens);
    a.max_len = max_len;
    const DevHead* blob = (const DevHead*)d_blob;
    hipStream_t st = (hipStream_t)stream;
    const int G = cb->group;
    if (p.RB == 1)
        launch_qprep<1>(p, layer, cb->n_kv, G, n_seqs, st, blob, q, qa, qsc);
    else if (p.RB == 2)
        launch_qprep<2>(p, layer, cb->n_kv, G, n_seqs, st, blob, q, qa, qsc);
    else
        launch_qprep<3>(p, layer, cb->n_kv, G, n_seqs, st, blob, q, qa, qsc);
    HIP_TRY(hipGetLastError());
    dim3 grid(p.wg_per_head, cb->n_kv, n_seqs);
    const uint8_t* c = (const uint8_t*)cache->data;
#define AATC_DECODE_CASE(rb, nvb, nch)                                                       \
    if (p.RB == rb && p.NVB == nvb && p.NCH == nch)                                          \
        rc = launch_decode<rb, nvb, nch>(p, grid, st, blob, c, seq_ids, seq_lens, qa, qsc, part); \
    else
    AATC_DECODE_CASE(1, 8, 1)
    AATC_DECODE_CASE(1, 12, 1)
    AATC_DECODE_CASE(1, 16, 1)
    AATC_DECODE_CASE(1, 24, 1)
    AATC_DECODE_CASE(1, 32, 1)
    AATC_DECODE_CASE(1, 8, 2)
    AATC_DECODE_CASE(1, 12, 2)
    AATC_DECODE_CASE(1, 16, 2)
    AATC_DECODE_CASE(2, 8, 2)
    AATC_DECODE_CASE(2, 12, 2)
    AATC_DECODE_CASE(2, 16, 2)
    AATC_DECODE_CASE(2, 8, 3)
    AATC_DECODE_CASE(2, 12, 3)
    AATC_DECODE_CASE(2, 16, 3)
    AATC_DECODE_CASE(3, 8, 4)
    AATC_DECODE_CASE(3, 12, 4)
    AATC_DECODE_CASE(3, 16, 4)
    rc = set_error(AATC_ERR_UNSUPPORTED, "no decode variant for %d query-head rows and %d value blocks", 3 * G,
                   p.nvb_max);
#undef AATC_DECODE_CASE
    if (rc) return rc;
    hipLaunchKernelGGL(combine_kernel, dim3(cb->n_kv * G, n_seqs), dim3(cb->d), 0, st, blob, layer, cb->n_kv, G,
                       p.wg_per_head, part, out);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}
