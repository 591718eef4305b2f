// Split-context decode attention over the packed cache (gfx950).
//
// Pages: "Attention-Aware Transform Coding Guide" ("Formal Attention Distortion Model":
// o = softmax(q K^T / sqrt(d)) V; KLT section K' = K U_K, so q.k = (U_K^T q).(U_K^T k) and
// keys are scored in the transform domain and never reconstructed; values are
// inverse-transformed once per query head); "Spend Bits Where Queries Look" abstract
// (decoding reads the whole cache every step and is bandwidth-bound).
//
// Two kernels, both on the caller's stream:
//   qprep   : q' = U_K^T q per query head, scaled by the key steps (and log2 e / sqrt d),
//             split into three int8 digits and laid out as the A operands of the score
//             MFMAs of each kv-head (slot order = the key unpack schedule); clears the
//             completion counters used by the decode kernel.
//   decode  : a workgroup of 4 waves streams a run of 64-token tiles of one (sequence,
//             kv-head) through LDS (direct global->LDS loads, double-buffered) and works on
//             each tile cooperatively:
//               scores  - wave w takes tokens 16w..16w+15: key pieces are unpacked with
//                         SWAR shift/mask into int8 operands of v_mfma_i32_16x16x64_i8;
//                         MFMA rows are 4*head + digit, so a lane holds the three digit
//                         rows of one head and combines them in registers;
//               softmax - per-head tile maxima meet in LDS; every wave keeps the same
//                         online reference maximum (base 2, raised lazily with headroom);
//                         probabilities become three int8 digits in LDS;
//               values  - wave w takes value column blocks w, w+4, ... over all 64 tokens
//                         and accumulates P x pieces in int32 with the same MFMA.
//             Each wave holds a quarter of the value accumulators, which keeps registers
//             low enough for four waves per SIMD.  The workgroup writes one partial
//             (max, sum, accumulator); the last workgroup of each (sequence, kv-head)
//             merges them, dequantises the value coefficients and applies U_V and mu_V.
// Inner loops are branch-free straight-line code (compile-time bounds NQB score operand
// blocks and NVB value column blocks; the unpack mode of a block is a uniform select).
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kTargetGroups = 1024;  // workgroups per launch (4 per CU on 256 CUs)
constexpr float kHeadroom = 2.0f;    // log2 headroom added to the reference max at a rescale
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kM4 = 0x0F0F0F0Fu, kM2 = 0x03030303u, kM1 = 0x01010101u;
constexpr float kDig1 = 1.0f / 254.0f, kDig2 = 1.0f / 64516.0f;

struct DecodeArgs {
    int layer, n_kv, G, n_seqs_cache;
    int64_t n_tiles_cap;
    int64_t max_len;
    int tile_bytes, tpg, wg_per_head, nqb_max;
    // LDS carve-up (bytes)
    int off_qsc, off_ccol, off_buf, buf_bytes, off_P, off_tm;
};

// order this wave's earlier LDS writes before its later LDS reads
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// all of this wave's memory operations (incl. global->LDS tile loads) have completed
__device__ __forceinline__ void wait_all() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// max / sum over the 16 lanes of a DPP row (every lane gets the result)
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));      // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));      // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));     // row_half_mirror
    return fmaxf(x, dpp<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}

// Stream one tile (bytes, a multiple of 16) from global memory into LDS with the whole
// workgroup: wave w moves the 1 KiB chunks w, w+4, ... (16 bytes per lane per instruction;
// LDS address = chunk base + 16 * lane).
__device__ __forceinline__ void load_tile(const uint8_t* src, LDS_AS uint8_t* lds, int bytes, int wave, int lane) {
    for (int off = 1024 * wave; off < bytes; off += 1024 * kWaves) {
        const int o = off + 16 * lane;
        if (o < bytes) __builtin_amdgcn_global_load_lds((const void*)(src + o), (LDS_AS void*)(lds + off), 16, 0, 0);
    }
}

// Four int8 operand words from packed pieces.  m4 / m2 select the 4-bit / 2-bit modes
// (uniform), otherwise 1-bit: 4-bit takes the nibbles of x0 then x1, 2-bit the crumbs of
// x0, 1-bit bits 0..3 of each byte of x0 >> pre.
__device__ __forceinline__ v4i unpack(uint32_t x0, uint32_t x1, bool m4, bool m2, uint32_t pre) {
    const uint32_t base = (m4 || m2) ? x0 : (x0 >> pre);
    const uint32_t hi = m4 ? x1 : base;
    const uint32_t M = m4 ? kM4 : (m2 ? kM2 : kM1);
    const uint32_t s1 = m4 ? 4u : (m2 ? 2u : 1u), s2 = m4 ? 0u : (m2 ? 4u : 2u), s3 = m4 ? 4u : (m2 ? 6u : 3u);
    return v4i{(int)(base & M), (int)((base >> s1) & M), (int)((hi >> s2) & M), (int)((hi >> s3) & M)};
}


// ---------------------------------------------------------------------------------------
// query preparation: int8 digits of q'' in the A-operand layout of the score MFMAs
// (row 16 rb + 4 h' + k holds digit k of query head 4 rb + h' of the group)
// ---------------------------------------------------------------------------------------
template <int RB, int D>
__global__ __launch_bounds__(256) void qprep_kernel(const DevHead* __restrict__ blob, int layer, int n_kv, int G,
                                                    int nqb_max, const uint16_t* __restrict__ q,
                                                    int8_t* __restrict__ qa_out, float* __restrict__ qsc_out,
                                                    uint32_t* __restrict__ counters) {
    constexpr int PARTS = 256 / D;     // row slices of U_K per column
    constexpr int ROWS = D / PARTS;    // rows per slice
    __shared__ float qf[16][D];
    __shared__ float part_s[PARTS][16][D];
    __shared__ int smax[16];
    __shared__ int16_t kmap[aatc::kMaxQB * 64];
    const int h = blockIdx.x, z = blockIdx.y, tid = threadIdx.x;
    const DevHead& H = blob[layer * n_kv + h];
    const int nq = n_kv * G;
    const int nqb = H.nqb[0] + H.nqb[1] + H.nqb[2];
    // every global read is issued up front so that a cold codebook costs one latency
    const int j = tid % D, part = tid / D;
    float u[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) u[r] = H.UK[(part * ROWS + r) * D + j];
    const int b = H.bitsK[j];
    const float st = H.stepK[j];
    for (int i = tid; i < nqb * 64; i += 256) kmap[i] = (&H.kq_map[0][0][0])[i];
    if (tid == 0) counters[z * n_kv + h] = 0u;
    const uint16_t* qg = q + ((int64_t)z * nq + h * G) * D;
    for (int i = tid; i < G * D; i += 256) qf[i / D][i % D] = aatc::bf16f(qg[i]);
    if (tid < 16) smax[tid] = 0;
    __syncthreads();
    // q' = U_K^T q: thread (j, part) sums its slice of rows, slices meet in LDS
    for (int g = 0; g < G; ++g) {
        float a = 0.0f;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) a = fmaf(u[r], qf[g][part * ROWS + r], a);
        part_s[part][g][j] = a;
    }
    __syncthreads();
    const float qs = kLog2e / sqrtf((float)D);
    const int top = b >= 4 ? b - 4 : (b >= 2 ? b - 2 : 0);  // shift of the channel's top piece
    for (int g = part; g < G; g += PARTS) {
        float a = 0.0f;
#pragma unroll
        for (int pp = 0; pp < PARTS; ++pp) a += part_s[pp][g][j];
        const float v = b ? a * st * qs : 0.0f;
        qf[g][j] = v;  // q'' (qf is free again)
        atomicMax(&smax[g], __float_as_int(fabsf(v) * (float)(1 << top)));
    }
    __syncthreads();
    int8_t* qa = qa_out + ((int64_t)z * n_kv + h) * nqb_max * RB * 1024;
    for (int i = tid; i < nqb_max * RB * 1024; i += 256) {
        const int bb = i & 15, lane = (i >> 4) & 63, rb = (i >> 10) % RB, qb = (i >> 10) / RB;
        const int row = lane & 15, g = lane >> 4;
        const int hh = 4 * rb + (row >> 2), k = row & 3;
        int val = 0;
        if (qb < nqb && hh < G && k < 3) {
            const int m = kmap[(qb * 4 + g) * 16 + bb];
            if (m >= 0) {
                const float mx = __int_as_float(smax[hh]);
                const float x = mx > 0.0f ? qf[hh][m & 255] * (float)(1 << (m >> 8)) * (127.0f / mx) : 0.0f;
                const float d0 = rintf(x);
                const float r1 = (x - d0) * 254.0f;
                const float d1 = rintf(r1);
                const float d2 = rintf((r1 - d1) * 254.0f);
                val = (int)(k == 0 ? d0 : (k == 1 ? d1 : d2));
            }
        }
        qa[i] = (int8_t)val;
    }
    float* qsc = qsc_out + ((int64_t)z * n_kv + h) * RB * 16;
    for (int r = tid; r < RB * 16; r += 256) {
        const int hh = r >> 2, k = r & 3;
        float v = 0.0f;
        if (hh < G && k < 3) {
            const float mx = __int_as_float(smax[hh]);
            v = (mx / 127.0f) * (k == 0 ? 1.0f : (k == 1 ? kDig1 : kDig2));
        }
        qsc[r] = v;
    }
}

// ---------------------------------------------------------------------------------------
// split decode (+ the final merge by the last workgroup of each (sequence, kv-head))
// ---------------------------------------------------------------------------------------
// waves per SIMD the register budget is sized for: four for the common shapes (one row
// block, up to 16 value column blocks), fewer where more accumulators are live
constexpr int waves_for(int rb, int nqb, int nvb) { return rb * nvb <= 16 && nqb <= 8 ? 4 : (rb * nvb <= 24 ? 3 : 2); }

template <int RB, int NQB, int NVB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_for(RB, NQB, NVB)))) void decode_kernel(
    const DevHead* __restrict__ blob, const uint8_t* __restrict__ cache, DecodeArgs a,
    const int32_t* __restrict__ seq_ids, const int64_t* __restrict__ seq_lens, const int8_t* __restrict__ qa_all,
    const float* __restrict__ qsc_all, float* __restrict__ part, uint32_t* __restrict__ counters,
    float* __restrict__ out) {
    constexpr int NVW = NVB / kWaves;  // value column blocks per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    LDS_AS uint8_t* sm = (LDS_AS uint8_t*)smem_generic;
    const int wgi = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c = lane & 15;
    const DevHead& H = blob[a.layer * a.n_kv + h];
    const int G = a.G, d = H.d, TB = a.tile_bytes;
    const int WK = H.BK >> 5;  // key record words per token
    const int nqb4 = H.nqb[0], nqb2 = H.nqb[1], nqb = H.nqb[0] + H.nqb[1] + H.nqb[2];
    const int nvb4 = H.nvb[0], nvb2 = H.nvb[1], nvb = H.nvb[0] + H.nvb[1] + H.nvb[2];

    LDS_AS int8_t* qa_lds = (LDS_AS int8_t*)sm;                  // [NQB][RB][64 lanes][16]
    LDS_AS float* qsc_lds = (LDS_AS float*)(sm + a.off_qsc);     // [RB*4 heads][4 digits]
    LDS_AS int16_t* ccol_lds = (LDS_AS int16_t*)(sm + a.off_ccol);
    LDS_AS uint8_t* buf0 = sm + a.off_buf;                       // two tile buffers
    LDS_AS uint8_t* P = sm + a.off_P;                            // [RB*16 rows][64 tokens] digits
    LDS_AS float* tm = (LDS_AS float*)(sm + a.off_tm);           // [4 waves][RB*4 heads] maxima

    // ---- sequence geometry (device arguments clamped: no read outside the cache)
    const int seq = seq_ids[z];
    int64_t len = min(min(seq_lens[z], a.max_len), a.n_tiles_cap * kTile);
    if (seq < 0 || seq >= a.n_seqs_cache) len = 0;
    const int64_t n_tiles = (len + kTile - 1) / kTile;
    const int64_t t_begin = (int64_t)wgi * a.tpg;
    const int64_t t_end = min(t_begin + a.tpg, n_tiles);
    const uint8_t* tiles = cache + (((int64_t)a.layer * a.n_seqs_cache + seq) * a.n_kv + h) * a.n_tiles_cap * TB;
    if (t_begin < t_end) load_tile(tiles + t_begin * TB, buf0, TB, w, lane);

    // ---- per-lane schedule constants (registers) and staged operands (LDS)
    uint32_t kofs[NQB];  // key record words (o0 | o1 << 16) of this lane group for each score block
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
        kofs[qb] = qb < nqb ? (uint32_t)H.kq_dw[qb][g][0] | ((uint32_t)H.kq_dw[qb][g][1] << 16) : 0u;
    uint32_t vofs[NVW];  // first word of this lane's value slab in this wave's column blocks
#pragma unroll
    for (int j = 0; j < NVW; ++j) {
        const int cb = w + kWaves * j;
        vofs[j] = cb < nvb ? (uint32_t)H.vb_slab[cb][c] : 0u;
    }
    {
        const u32x4* src = (const u32x4*)(qa_all + ((int64_t)z * a.n_kv + h) * a.nqb_max * RB * 1024);
        LDS_AS u32x4* dst = (LDS_AS u32x4*)qa_lds;
        for (int i = tid; i < NQB * RB * 64; i += 256)
            dst[i] = i < nqb * RB * 64 ? src[i] : u32x4{0u, 0u, 0u, 0u};
        const float* qs = qsc_all + ((int64_t)z * a.n_kv + h) * RB * 16;
        for (int i = tid; i < RB * 16; i += 256) qsc_lds[i] = qs[i];
        for (int i = tid; i < d * 4; i += 256) ccol_lds[i] = (&H.chan_cols[0][0])[i];
        LDS_AS uint32_t* Pw = (LDS_AS uint32_t*)P;
        for (int i = tid; i < RB * 16 * 16; i += 256) Pw[i] = 0u;
    }
    __syncthreads();

    const int tok = 16 * w + c;  // this lane's token inside the tile (scores, softmax)
    float qs[RB][3];
    bool hv[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        hv[rb] = 4 * rb + g < G;
#pragma unroll
        for (int k = 0; k < 3; ++k) qs[rb][k] = qsc_lds[(4 * rb + g) * 4 + k];
    }
    const uint32_t vwi4 = 2 * g, vwi2 = g, vwi1 = g >> 1, pre1 = 4 * (g & 1);

    v4i acc_i[RB][NVW];
    float acc_f[RB][NVW][3];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
            acc_i[rb][j] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < 3; ++k) acc_f[rb][j][k] = 0.0f;
        }
    float mref[RB], lsum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mref[rb] = -INFINITY, lsum[rb] = 0.0f;

    for (int64_t t = t_begin; t < t_end; ++t) {
        LDS_AS uint8_t* cur = buf0 + (((t - t_begin) & 1) ? a.buf_bytes : 0);
        LDS_AS uint8_t* nxt = buf0 + (((t - t_begin) & 1) ? 0 : a.buf_bytes);
        wait_all();
        __syncthreads();  // tile t resident; every wave is done with tile t-1 (buffers, P, tm)
        if (t + 1 < t_end) load_tile(tiles + (t + 1) * TB, nxt, TB, w, lane);
        const LDS_AS uint32_t* kw = (const LDS_AS uint32_t*)cur + tok;  // record word r at kw[64 r]
        const LDS_AS uint32_t* vw = (const LDS_AS uint32_t*)cur + 64 * WK;
        const int valid = (int)min((int64_t)kTile, len - t * kTile);

        // ---------------- scores of this wave's 16 tokens: S[4 head + digit][token]
        v4i S[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) S[rb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const bool m4 = qb < nqb4, m2 = !m4 && qb < nqb4 + nqb2;
            const v4i B = unpack(kw[64 * (kofs[qb] & 0xFFFFu)], kw[64 * (kofs[qb] >> 16)], m4, m2, pre1);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const v4i A = *(const LDS_AS v4i*)(qa_lds + ((qb * RB + rb) * 64 + lane) * 16);
                S[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, S[rb], 0, 0, 0);
            }
        }
        // lane (g, c): head 4rb+g, token 16w+c; per-wave head maxima to LDS
        float s[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float v = (float)S[rb][0] * qs[rb][0] + (float)S[rb][1] * qs[rb][1] + (float)S[rb][2] * qs[rb][2];
            s[rb] = (hv[rb] && tok < valid) ? v : -INFINITY;
            const float mx = row16_max(s[rb]);
            if (c == 0) tm[w * RB * 4 + 4 * rb + g] = mx;
        }
        __syncthreads();  // per-wave maxima visible

        // ---------------- online softmax (all waves keep the same reference maxima)
        float tmax[RB];
        bool need = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float mx = tm[4 * rb + g];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) mx = fmaxf(mx, tm[ww * RB * 4 + 4 * rb + g]);
            tmax[rb] = mx;
            need |= mx > mref[rb];
        }
        if (__any(need)) {
            // raise the reference of heads whose tile max passed it; fold the int
            // accumulators (relative to the old reference) into the float ones and rescale
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float nref = tmax[rb] > mref[rb] ? tmax[rb] + kHeadroom : mref[rb];
                const float al = hv[rb] ? exp2f(mref[rb] - nref) : 0.0f;
                lsum[rb] *= al;
                mref[rb] = nref;
#pragma unroll
                for (int j = 0; j < NVW; ++j) {
                    acc_f[rb][j][0] = (acc_f[rb][j][0] + (float)acc_i[rb][j][0] * (1.0f / 127.0f)) * al;
                    acc_f[rb][j][1] = (acc_f[rb][j][1] + (float)acc_i[rb][j][1] * (kDig1 / 127.0f)) * al;
                    acc_f[rb][j][2] = (acc_f[rb][j][2] + (float)acc_i[rb][j][2] * (kDig2 / 127.0f)) * al;
                    acc_i[rb][j] = v4i{0, 0, 0, 0};
                }
            }
        }
        // probabilities as three int8 digits (p*127 = d0 + d1/254 + d2/254^2) into
        // P[4 head + digit][token], the value MFMA's A operand
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float p = hv[rb] ? exp2f(s[rb] - mref[rb]) : 0.0f;
            lsum[rb] += p;
            const float x = p * 127.0f;
            const float d0 = rintf(x);
            const float r1 = (x - d0) * 254.0f;
            const float d1 = rintf(r1);
            const float d2 = rintf((r1 - d1) * 254.0f);
            LDS_AS int8_t* pp = (LDS_AS int8_t*)(P + (16 * rb + 4 * g) * 64 + tok);
            pp[0] = (int8_t)(int)d0;
            pp[64] = (int8_t)(int)d1;
            pp[128] = (int8_t)(int)d2;
        }
        __syncthreads();  // all 64 tokens' digits in P

        // ---------------- values: this wave's column blocks over all 64 tokens
        v4i Ap[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) Ap[rb] = *(const LDS_AS v4i*)(P + (16 * rb + c) * 64 + 16 * g);
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
            const int cb = w + kWaves * j;
            const bool m4 = cb < nvb4, m2 = !m4 && cb < nvb4 + nvb2;
            const uint32_t wi = vofs[j] + (m4 ? vwi4 : (m2 ? vwi2 : vwi1));
            const v4i B = unpack(vw[wi], vw[wi + 1], m4, m2, pre1);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc_i[rb][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ap[rb], B, acc_i[rb][j], 0, 0, 0);
        }
    }

    // ---------------- epilogue: fold, reduce digits and pieces, one partial per workgroup
    wait_all();
    __syncthreads();  // tile buffers free
    const int ncol = 16 * nvb;
    LDS_AS float* accg = (LDS_AS float*)buf0;          // [RB*4 heads][ncol]
    LDS_AS float* lsw = accg + RB * 4 * ncol;          // [4 waves][RB*4 heads]
    LDS_AS float* wp = lsw + kWaves * RB * 4;          // [G][d+2]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float ls = row16_sum(lsum[rb]);
        if (c == 0) lsw[w * RB * 4 + 4 * rb + g] = ls;
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
            const int cb = w + kWaves * j;
            if (cb < nvb)
                accg[(4 * rb + g) * ncol + 16 * cb + c] =
                    acc_f[rb][j][0] + (float)acc_i[rb][j][0] * (1.0f / 127.0f) + acc_f[rb][j][1] +
                    (float)acc_i[rb][j][1] * (kDig1 / 127.0f) + acc_f[rb][j][2] +
                    (float)acc_i[rb][j][2] * (kDig2 / 127.0f);
        }
        if (w == 0 && c == 0 && hv[rb]) wp[(4 * rb + g) * (d + 2)] = mref[rb];
    }
    __syncthreads();
    float* pout = part + (((int64_t)z * a.n_kv + h) * a.wg_per_head + wgi) * G * (d + 2);
    for (int i = tid; i < G * (d + 2); i += 256) {
        const int hh = i / (d + 2), col = i % (d + 2);
        float v;
        if (col == 0) {
            v = wp[hh * (d + 2)];
        } else if (col == 1) {
            v = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) v += lsw[ww * RB * 4 + hh];
        } else {
            const int jj = col - 2;
            v = 0.0f;
#pragma unroll
            for (int tt = 0; tt < 3; ++tt) {
                const int e = ccol_lds[jj * 4 + tt];
                if (e >= 0) v += (float)(1 << (e >> 12)) * accg[hh * ncol + (e & 0xfff)];
            }
        }
        pout[i] = v;
    }

    // ---------------- the last workgroup of this (sequence, kv-head) merges all partials,
    // dequantises the value coefficients and applies the inverse transform
    __threadfence();
    __syncthreads();
    __shared__ int is_last;
    if (tid == 0) is_last = atomicAdd(&counters[z * a.n_kv + h], 1u) == (uint32_t)(a.wg_per_head - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    const int W = a.wg_per_head;
    const float* ph = part + ((int64_t)z * a.n_kv + h) * W * G * (d + 2);
    LDS_AS float* wgt = (LDS_AS float*)sm;  // [G][W] maxima, then merge weights
    LDS_AS float* lw = wgt + G * W;         // [G][W] sums
    LDS_AS float* Ls = lw + G * W;          // [G]
    LDS_AS float* cbar = Ls + G;            // [G][d]
    for (int i = tid; i < G * W; i += 256) {
        const float* src = ph + ((i % W) * G + i / W) * (d + 2);
        wgt[i] = src[0];
        lw[i] = src[1];
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int s2 = 0; s2 < W; ++s2) M = fmaxf(M, wgt[tid * W + s2]);
        float L = 0.0f;
        for (int s2 = 0; s2 < W; ++s2) {
            const float m = wgt[tid * W + s2];
            const float wt = m == -INFINITY ? 0.0f : exp2f(m - M);
            wgt[tid * W + s2] = wt;
            L += wt * lw[tid * W + s2];
        }
        Ls[tid] = L;
    }
    __syncthreads();
    for (int i = tid; i < G * d; i += 256) {
        const int hh = i / d, jj = i % d;
        float A = 0.0f;
#pragma unroll 8
        for (int s2 = 0; s2 < W; ++s2) A += wgt[hh * W + s2] * ph[(s2 * G + hh) * (d + 2) + 2 + jj];
        const int bv = H.bitsV[jj];
        cbar[i] = bv ? H.stepV[jj] * (A / Ls[hh] - (float)(1 << (bv - 1)) + 0.5f) : 0.0f;
    }
    __syncthreads();
    for (int i = tid; i < G * d; i += 256) {
        const int hh = i / d, ii = i % d;
        float o = H.muV[ii];
#pragma unroll 8
        for (int jj = 0; jj < d; ++jj) o = fmaf(H.UVt[jj * d + ii], cbar[hh * d + jj], o);
        out[((int64_t)z * a.n_kv * G + h * G + hh) * d + ii] = o;
    }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
struct Variant {
    int rb, nqb, nvb;
};
// compile-time (row blocks, score operand blocks, value column blocks) bounds available;
// value column blocks are a multiple of 4 (a quarter per wave)
constexpr Variant kVariants[] = {{1, 4, 8},  {1, 6, 12},  {1, 8, 16},  {1, 12, 24}, {1, 12, 32},
                                 {2, 6, 12}, {2, 8, 16},  {2, 12, 24}, {2, 12, 32}, {3, 6, 12},
                                 {3, 8, 16}, {3, 12, 24}, {3, 12, 32}, {4, 6, 12}, {4, 8, 16},
                                 {4, 12, 24}, {4, 12, 32}};

struct Plan {
    Variant v;
    int nqb_max, nvb_max, tpg, wg_per_head;
    size_t qa_bytes, qsc_bytes, part_bytes, cnt_bytes;
    DecodeArgs args;
    size_t lds;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

int make_plan(const aatc_codebook* cb, int layer, int n_seqs, int64_t max_len, Plan& p) {
    const int G = cb->group, d = cb->d;
    const int RB = (G + 3) / 4;
    p.nqb_max = 0;
    p.nvb_max = 0;
    for (int h = 0; h < cb->n_kv; ++h) {
        const DevHead& D = cb->blob[(size_t)layer * cb->n_kv + h];
        p.nqb_max = std::max(p.nqb_max, D.nqb[0] + D.nqb[1] + D.nqb[2]);
        p.nvb_max = std::max(p.nvb_max, D.nvb[0] + D.nvb[1] + D.nvb[2]);
    }
    bool found = false;
    for (const Variant& v : kVariants)
        if (v.rb == RB && v.nqb >= p.nqb_max && v.nvb >= p.nvb_max) {
            p.v = v;
            found = true;
            break;
        }
    if (!found)
        return set_error(AATC_ERR_UNSUPPORTED, "no decode variant for %d query heads, %d score and %d value blocks", G,
                         p.nqb_max, p.nvb_max);
    const int64_t tiles = n_tiles_of(max_len);
    const int64_t total = tiles * cb->n_kv * (int64_t)n_seqs;
    p.tpg = (int)std::max<int64_t>(1, (total + kTargetGroups - 1) / kTargetGroups);
    p.wg_per_head = (int)((tiles + p.tpg - 1) / p.tpg);
    p.qa_bytes = (size_t)n_seqs * cb->n_kv * p.nqb_max * RB * 1024;
    p.qsc_bytes = (size_t)n_seqs * cb->n_kv * RB * 16 * sizeof(float);
    p.part_bytes = (size_t)n_seqs * cb->n_kv * p.wg_per_head * G * (d + 2) * sizeof(float);
    p.cnt_bytes = (size_t)n_seqs * cb->n_kv * sizeof(uint32_t);
    DecodeArgs& a = p.args;
    a.G = G;
    a.tile_bytes = 8 * cb->total_bits;
    a.tpg = p.tpg;
    a.wg_per_head = p.wg_per_head;
    a.nqb_max = p.nqb_max;
    auto al16 = [](size_t x) { return (int)((x + 15) & ~(size_t)15); };
    a.off_qsc = al16((size_t)p.v.nqb * RB * 1024);
    a.off_ccol = al16(a.off_qsc + RB * 16 * sizeof(float));
    a.off_buf = al16(a.off_ccol + (size_t)d * 4 * sizeof(int16_t));
    a.buf_bytes = al16(a.tile_bytes + 16);
    // the epilogue reuses the tile buffers
    const size_t epi = ((size_t)RB * 4 * 16 * p.nvb_max + kWaves * RB * 4 + (size_t)G * (d + 2)) * sizeof(float);
    const size_t bufs = std::max(2 * (size_t)a.buf_bytes, epi);
    a.off_P = al16(a.off_buf + bufs);
    a.off_tm = al16(a.off_P + (size_t)RB * 16 * 64);
    const size_t merge = ((size_t)2 * G * p.wg_per_head + G + (size_t)G * d) * sizeof(float);
    p.lds = std::max((size_t)a.off_tm + kWaves * RB * 4 * sizeof(float), merge);
    if (p.lds > 160 * 1024 - 256)
        return set_error(AATC_ERR_UNSUPPORTED, "decode needs %zu bytes of LDS per workgroup", p.lds);
    return AATC_OK;
}

template <int RB, int NQB, int NVB>
int launch_decode(const Plan& p, dim3 grid, hipStream_t st, const DevHead* blob, const uint8_t* cache,
                  const int32_t* ids, const int64_t* lens, const int8_t* qa, const float* qsc, float* part,
                  uint32_t* counters, float* out) {
    static size_t attr_lds = 0;  // dynamic LDS limit already granted to this instantiation
    if (p.lds > attr_lds) {
        HIP_TRY(hipFuncSetAttribute((const void*)decode_kernel<RB, NQB, NVB>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds));
        attr_lds = p.lds;
    }
    hipLaunchKernelGGL((decode_kernel<RB, NQB, NVB>), grid, dim3(256), p.lds, st, blob, cache, p.args, ids, lens, qa,
                       qsc, part, counters, out);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}

template <int RB>
void launch_qprep(const Plan& p, int d, int layer, int n_kv, int G, int n_seqs, hipStream_t st, const DevHead* blob,
                  const uint16_t* q, int8_t* qa, float* qsc, uint32_t* counters) {
    if (d == 64)
        hipLaunchKernelGGL((qprep_kernel<RB, 64>), dim3(n_kv, n_seqs), dim3(256), 0, st, blob, layer, n_kv, G,
                           p.nqb_max, q, qa, qsc, counters);
    else
        hipLaunchKernelGGL((qprep_kernel<RB, 128>), dim3(n_kv, n_seqs), dim3(256), 0, st, blob, layer, n_kv, G,
                           p.nqb_max, q, qa, qsc, counters);
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
        worst = std::max(worst, al256(p.qa_bytes) + al256(p.qsc_bytes) + al256(p.part_bytes) + p.cnt_bytes);
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
    const size_t need = al256(p.qa_bytes) + al256(p.qsc_bytes) + al256(p.part_bytes) + p.cnt_bytes;
    if (ws_bytes < need) return set_error(AATC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    uint8_t* wsp = (uint8_t*)workspace;
    int8_t* qa = (int8_t*)wsp;
    float* qsc = (float*)(wsp + al256(p.qa_bytes));
    float* part = (float*)(wsp + al256(p.qa_bytes) + al256(p.qsc_bytes));
    uint32_t* counters = (uint32_t*)(wsp + al256(p.qa_bytes) + al256(p.qsc_bytes) + al256(p.part_bytes));
    DecodeArgs& a = p.args;
    a.layer = layer;
    a.n_kv = cb->n_kv;
    a.n_seqs_cache = cache->n_seqs;
    a.n_tiles_cap = n_tiles_of(cache->max_tokens);
    a.max_len = max_len;
    const DevHead* blob = (const DevHead*)d_blob;
    hipStream_t st = (hipStream_t)stream;
    const int G = cb->group;
    switch (p.v.rb) {
        case 1: launch_qprep<1>(p, cb->d, layer, cb->n_kv, G, n_seqs, st, blob, q, qa, qsc, counters); break;
        case 2: launch_qprep<2>(p, cb->d, layer, cb->n_kv, G, n_seqs, st, blob, q, qa, qsc, counters); break;
        case 3: launch_qprep<3>(p, cb->d, layer, cb->n_kv, G, n_seqs, st, blob, q, qa, qsc, counters); break;
        default: launch_qprep<4>(p, cb->d, layer, cb->n_kv, G, n_seqs, st, blob, q, qa, qsc, counters); break;
    }
    HIP_TRY(hipGetLastError());
    dim3 grid(p.wg_per_head, cb->n_kv, n_seqs);
    const uint8_t* c = (const uint8_t*)cache->data;
#define AATC_DECODE_CASE(rb_, nqb_, nvb_)                                                                     \
    if (p.v.rb == rb_ && p.v.nqb == nqb_ && p.v.nvb == nvb_)                                                  \
        return launch_decode<rb_, nqb_, nvb_>(p, grid, st, blob, c, seq_ids, seq_lens, qa, qsc, part, counters, out);
    AATC_DECODE_CASE(1, 4, 8)
    AATC_DECODE_CASE(1, 6, 12)
    AATC_DECODE_CASE(1, 8, 16)
    AATC_DECODE_CASE(1, 12, 24)
    AATC_DECODE_CASE(1, 12, 32)
    AATC_DECODE_CASE(2, 6, 12)
    AATC_DECODE_CASE(2, 8, 16)
    AATC_DECODE_CASE(2, 12, 24)
    AATC_DECODE_CASE(2, 12, 32)
    AATC_DECODE_CASE(3, 6, 12)
    AATC_DECODE_CASE(3, 8, 16)
    AATC_DECODE_CASE(3, 12, 24)
    AATC_DECODE_CASE(3, 12, 32)
    AATC_DECODE_CASE(4, 6, 12)
    AATC_DECODE_CASE(4, 8, 16)
    AATC_DECODE_CASE(4, 12, 24)
    AATC_DECODE_CASE(4, 12, 32)
#undef AATC_DECODE_CASE
    return set_error(AATC_ERR_UNSUPPORTED, "decode variant missing");
}
