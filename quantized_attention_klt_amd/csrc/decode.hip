// Split-context decode attention over the packed cache (gfx950).
//
// Pages: "Attention-Aware Transform Coding Guide" ("Formal Attention Distortion Model":
// o = softmax(q K^T / sqrt(d)) V; KLT section K' = K U_K, so q.k = (U_K^T q).(U_K^T k) and
// keys are scored in the transform domain and never reconstructed; values are
// inverse-transformed once per query head); "Spend Bits Where Queries Look" abstract
// (decoding reads the whole cache every step and is bandwidth-bound).
//
// Two kernels on the caller's stream:
//   qprep  - one workgroup per (sequence, kv-head) forms q' = U_K^T q for its query
//            heads, scales it by the key steps (and log2 e / sqrt d) and splits it into
//            three int8 digits laid out as the A operands of the score MFMAs (one byte per
//            key field, weighted by the field's code shift over its bit position).
//   decode - a workgroup of 4 waves owns a run of 64-token tiles of one (sequence,
//            kv-head); wave w takes tiles w, w+4, ... of the run and streams them through
//            a private ring of LDS buffers (direct global->LDS loads, counted waits, no
//            workgroup barriers in the loop).  Per tile:
//     scores  - v_mfma_i32_16x16x64_i8 with rows 4*head + digit and one column per token:
//               a B dword is a key-record word ANDed with a mask that keeps one field per
//               byte; with bit 7 of stored bytes inverted such a byte reads as
//               field * 2^pos (- 128 when the field ends at bit 7), the 2^pos is divided
//               out of the query digits and the -128 is the accumulator's start value;
//     softmax - online, base 2, reference max raised lazily with headroom; probabilities
//               p * 127 * 2^16 are rounded to integers whose bytes are three int8 digits
//               (base 256), written over the tile's key block as the next A operand;
//     values  - the same MFMA with one column per value field: the B operand of a column
//               is 16 bytes of its record byte's plane (16 tokens) ANDed with the field
//               mask.  Column weights 2^(shift - pos) and the -128 of top fields (fixed
//               by the exact integer row sums of the probability digits) are applied once
//               at the end.
//   merge   - each workgroup writes one partial (max, sum, value-coefficient accumulator per
//             query head) with device-coherent stores; the last workgroup of each group of
//             partials merges them and applies U_V to its result, and the last group merger
//             of each (sequence, kv-head) combines the group results into the output.
//             Arrival counters wrap to zero on the last arrival (atomic increment modulo
//             the member count), so a zeroed workspace stays ready for the next call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

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
constexpr int kMergeGroup = 16;      // partials per first-level merge
// Arrival counters occupy a fixed table at the start of the workspace, whatever the call's
// shape, so counters a call leaves at zero are never overwritten by another call's partials.
constexpr int kCounterSlots = 32768;
constexpr size_t kCounterBytes = kCounterSlots * sizeof(uint32_t);
constexpr float kHeadroom = 2.0f;    // log2 headroom added to the reference max at a rescale
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kQ1 = 1.0f / 254.0f, kQ2 = 1.0f / 64516.0f;  // query digit weights (base 254)
constexpr float kP1 = 1.0f / 256.0f, kP2 = 1.0f / 65536.0f;  // probability digit weights (base 256)
constexpr float kPScale = 127.0f * 65536.0f;                  // p -> integer of three digits
constexpr int kQscStride = 80;  // floats per (sequence, kv-head) in the query-scale buffer

struct DecodeArgs {
    int layer, n_kv, G, n_seqs_cache;
    int64_t n_tiles_cap;
    int64_t max_len;
    int tile_bytes, tpg, wg_per_head, n_grp;
    // LDS carve-up (bytes): per wave a ring of nbw tile buffers
    int nbw, buf_bytes, wave_bytes, off_ksched, off_flag;
};

// LDS-only workgroup barrier: this wave's LDS operations are complete, then s_barrier.
// (Global->LDS tile loads in flight are not waited for; their waits are explicit.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait until at most n of this wave's vector memory operations are outstanding (n is
// clamped to 15, which only waits longer)
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
#define AATC_W(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        AATC_W(0) AATC_W(1) AATC_W(2) AATC_W(3) AATC_W(4) AATC_W(5) AATC_W(6) AATC_W(7)
        AATC_W(8) AATC_W(9) AATC_W(10) AATC_W(11) AATC_W(12) AATC_W(13) AATC_W(14)
#undef AATC_W
        default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    }
}

// data exchanged between workgroups: device-scope loads and stores (coherent across the
// per-XCD L2 caches without a cache writeback)
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Stream one tile (bytes, a multiple of 16) from global memory into LDS with one wave:
// 1 KiB per instruction, 16 bytes per lane (LDS address = chunk base + 16 * lane).  The
// loads carry the non-temporal hint (cache policy bit 1): the cache is read once per step,
// and with the default policy these direct-to-LDS loads stream at about half the rate.
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ void load_tile(const uint8_t* src, LDS_AS uint8_t* lds, int bytes, int lane) {
    for (int off = 0; off < bytes; off += 1024) {
        const int o = off + 16 * lane;
        if (o < bytes)
            __builtin_amdgcn_global_load_lds((const void*)(src + o), (LDS_AS void*)(lds + off), 16, 0, kStreamPolicy);
    }
}

// all of this wave's memory operations (incl. global->LDS tile loads) have completed
__device__ __forceinline__ void wait_all() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// three base-254 digits of x: x = d0 + d1 / 254 + d2 / 254^2 (+ rounding); each fits int8
// when |x| <= 127
__device__ __forceinline__ void digits254(float x, float& d0, float& d1, float& d2) {
    d0 = rintf(x);
    const float r1 = (x - d0) * 254.0f;
    d1 = rintf(r1);
    d2 = rintf((r1 - d1) * 254.0f);
}

// an int32 accumulator triple (digit rows of weight 1, 1/256, 1/65536) as one float
__device__ __forceinline__ float combine256(int a0, int a1, int a2) {
    return (float)a0 + (float)a1 * kP1 + (float)a2 * kP2;
}
// ... and back: x = d0 + d1 / 256 + d2 / 65536 (+ rounding of the last digit)
__device__ __forceinline__ void split256(float x, int& a0, int& a1, int& a2) {
    const float d0 = rintf(x);
    const float r1 = (x - d0) * 256.0f;
    const float d1 = rintf(r1);
    a0 = (int)d0;
    a1 = (int)d1;
    a2 = (int)rintf((r1 - d1) * 256.0f);
}

// Merge n partials (reference max m, sum l, coefficient accumulator x[d] per query head,
// stored at src[(s * G + hh) * (D + 2) + {0, 1, 2 + jj}]) into the running (M, L, A) of
// this thread's columns i = tid + 256 k (head i / D, coefficient i % D), CH partials per
// round with every load of a round in flight at once.
template <int D, int CPT, int CH>
__device__ __forceinline__ void merge_cols(const float* src, int n, int G, int tid, float (&M)[CPT], float (&L)[CPT],
                                           float (&A)[CPT]) {
    constexpr int ld = D + 2;
#pragma unroll
    for (int k = 0; k < CPT; ++k) M[k] = -INFINITY, L[k] = 0.0f, A[k] = 0.0f;
    for (int s0 = 0; s0 < n; s0 += CH) {
        float m[CPT][CH], l[CPT][CH], x[CPT][CH];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int i = tid + 256 * k, hh = min(i / D, G - 1), jj = i % D;
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const float* p = src + (min(s0 + e, n - 1) * G + hh) * ld;
                m[k][e] = ld_dev(p);
                l[k][e] = ld_dev(p + 1);
                x[k][e] = ld_dev(p + 2 + jj);
            }
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float mx = M[k];
#pragma unroll
            for (int e = 0; e < CH; ++e)
                if (s0 + e < n) mx = fmaxf(mx, m[k][e]);
            const float f = M[k] == -INFINITY ? 0.0f : exp2f(M[k] - mx);
            L[k] *= f;
            A[k] *= f;
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const float wgt = (s0 + e < n && m[k][e] != -INFINITY) ? exp2f(m[k][e] - mx) : 0.0f;
                L[k] = fmaf(wgt, l[k][e], L[k]);
                A[k] = fmaf(wgt, x[k][e], A[k]);
            }
            M[k] = mx;
        }
    }
}

// ---------------------------------------------------------------------------------------
// query preparation, one workgroup per (sequence, kv-head): q'' = (U_K^T q) * step_K *
// log2(e) / sqrt(d) for the G query heads; key field (chan, shift, pos) of score slot k
// gets q''[chan] * 2^shift / 2^pos, scaled per head so that the largest slot is 127 and
// split into three int8 digits; written as the A operands of the score MFMAs
// ([m][rb][lane][16] bytes; lane row = 4 head + digit).  Also per head the digit scale
// and per operand row 128 x the digits of slots whose field ends at bit 7.  Every global
// read is issued in one batch so that a cold codebook costs one latency.
// ---------------------------------------------------------------------------------------
template <int RB, int NQM, int D>
__global__ __launch_bounds__(256) void qprep_kernel(const DevHead* __restrict__ blob, int layer, int n_kv, int G,
                                                    const uint16_t* __restrict__ q, uint32_t* __restrict__ qa_out,
                                                    float* __restrict__ qscale_out) {
    constexpr int PARTS = 256 / D;           // row slices of U_K per column
    constexpr int ROWS = D / PARTS;          // rows per slice
    constexpr int QPT = 16 * D / 256;        // query elements per thread (<= 16 heads)
    constexpr int KPT = (NQM * 64 + 255) / 256;
    typedef float f4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) float qf[16 * D];
    __shared__ float ps[PARTS * 16 * D];
    __shared__ int smax[16];
    __shared__ uint16_t kmap[KPT * 256];
    __shared__ int corr[64];  // per operand row: sum of the digits in inverted-bit-7 slots
    const int h = blockIdx.x, z = blockIdx.y, tid = threadIdx.x;
    const DevHead& H = blob[layer * n_kv + h];
    const int64_t zh = (int64_t)z * n_kv + h;
    const int j = tid % D, pt = __builtin_amdgcn_readfirstlane(tid / D);
    const float* ub = H.UK + pt * ROWS * D + j;
    float u[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) u[r] = ub[r * D];
    const int bj = H.bitsK[j];
    const float stj = H.stepK[j];
    const int nqm = H.nqm;
    const uint16_t* qg = q + zh * G * D;
    uint16_t qv[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) qv[k] = qg[min(tid + 256 * k, G * D - 1)];
    uint16_t km[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) km[k] = (&H.kq_slot[0][0][0])[tid + 256 * k];
#pragma unroll
    for (int k = 0; k < QPT; ++k)
        if (tid + 256 * k < G * D) qf[tid + 256 * k] = aatc::bf16f(qv[k]);
#pragma unroll
    for (int k = 0; k < KPT; ++k) kmap[tid + 256 * k] = km[k];
    if (tid < 16) smax[tid] = 0;
    if (tid < 64) corr[tid] = 0;
    __syncthreads();
    // q' = U_K^T q: thread (j, pt) sums its slice of rows, slices meet in LDS
    for (int hh = 0; hh < G; ++hh) {
        const f4* q4 = (const f4*)(qf + hh * D + pt * ROWS);
        float acc = 0.0f;
#pragma unroll
        for (int r4 = 0; r4 < ROWS / 4; ++r4) {
            const f4 x = q4[r4];
            acc = fmaf(u[4 * r4], x[0], acc);
            acc = fmaf(u[4 * r4 + 1], x[1], acc);
            acc = fmaf(u[4 * r4 + 2], x[2], acc);
            acc = fmaf(u[4 * r4 + 3], x[3], acc);
        }
        ps[(pt * 16 + hh) * D + j] = acc;
    }
    __syncthreads();
    const float qscale = kLog2e / sqrtf((float)D);
    for (int hh = pt; hh < G; hh += PARTS) {
        float acc = 0.0f;
#pragma unroll
        for (int p2 = 0; p2 < PARTS; ++p2) acc += ps[(p2 * 16 + hh) * D + j];
        qf[hh * D + j] = bj ? acc * stj * qscale : 0.0f;
    }
    __syncthreads();
    // per head: the largest slot value |q''[chan]| 2^shift / 2^pos (wave maxima, then one
    // LDS max per wave)
    for (int hh = 0; hh < G; ++hh) {
        float mag = 0.0f;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int i = tid + 256 * k;
            const uint32_t sl = kmap[i];
            if (i < NQM * 64 && sl != 0xFFFFu)
                mag = fmaxf(mag, fabsf(qf[hh * D + (sl & 255)]) * (float)(1 << ((sl >> 8) & 7)) *
                                     (1.0f / (float)(1 << ((sl >> 11) & 7))));
        }
        mag = row16_max(mag);
        mag = fmaxf(mag, __shfl_xor(mag, 16));
        mag = fmaxf(mag, __shfl_xor(mag, 32));
        if ((tid & 63) == 0) atomicMax(&smax[hh], __float_as_int(mag));
    }
    __syncthreads();
    // operand word i: bytes 4i..4i+3 of [m][rb][lane][16]; byte 4i'+b of lane group g holds
    // the slot kq_slot[m][g][4i'+b]: q''[chan] 2^shift / 2^pos (the field is read at bit pos)
    uint32_t* qa = qa_out + zh * NQM * RB * 256;
    for (int i = tid; i < NQM * RB * 256; i += 256) {
        const int bb = (i & 3) * 4, ln = (i >> 2) & 63, rb = (i >> 8) % RB, m = (i >> 8) / RB;
        const int row = ln & 15, gg = ln >> 4;
        const int hh = 4 * rb + (row >> 2), k = row & 3;
        uint32_t word = 0u;
        int flipped = 0;
        if (m < nqm && hh < G && k < 3) {
            const float mx = __int_as_float(smax[hh]);
            const float sc = mx > 0.0f ? 127.0f / mx : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t sl = kmap[(m * 4 + gg) * 16 + bb + e];
                if (sl != 0xFFFFu) {
                    const int chan = sl & 255, sh = (sl >> 8) & 7, pos = (sl >> 11) & 7;
                    float d0, d1, d2;
                    digits254(qf[hh * D + chan] * (float)(1 << sh) * (1.0f / (float)(1 << pos)) * sc, d0, d1, d2);
                    const int dv = (int)(k == 0 ? d0 : (k == 1 ? d1 : d2));
                    word |= ((uint32_t)dv & 0xFFu) << (8 * e);
                    if (sl & 0x4000u) flipped += dv;
                }
            }
        }
        if (flipped) atomicAdd(&corr[rb * 16 + row], flipped);
        qa[i] = word;
    }
    __syncthreads();
    // [0, 16): per-head digit scale; [16, 16 + 64): per operand row the accumulator's start
    // value, 128 x the digits that multiply inverted-bit-7 bytes
    float* qsc = qscale_out + zh * kQscStride;
    if (tid < 16) qsc[tid] = tid < G ? __int_as_float(smax[tid]) * (1.0f / 127.0f) : 0.0f;
    if (tid < 64) ((int*)qsc)[16 + tid] = 128 * corr[tid];
}

// Registers per lane grow with the row blocks and value column blocks; the waves per SIMD
// the allocation is sized for (the LDS plan matches it).
constexpr int vgpr_estimate(int rb, int nqm, int nvb) { return rb * nvb * 4 + nqm * rb * 4 + 2 * nvb + rb * 20 + 56; }
constexpr int waves_for(int rb, int nqm, int nvb) {
    return vgpr_estimate(rb, nqm, nvb) <= 128 ? 4 : (vgpr_estimate(rb, nqm, nvb) <= 168 ? 3 : 2);
}

template <int RB, int NQM, int NVB, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_for(RB, NQM, NVB)))) void decode_kernel(
    const DevHead* __restrict__ blob, const uint8_t* __restrict__ cache, DecodeArgs a,
    const int32_t* __restrict__ seq_ids, const int64_t* __restrict__ seq_lens, const uint8_t* __restrict__ qa_all,
    const float* __restrict__ qscale, float* __restrict__ part1, float* __restrict__ part2,
    uint32_t* __restrict__ cnt1, uint32_t* __restrict__ cnt2, float* __restrict__ out) {
    constexpr int PARTS = 256 / D;  // row slices of a d x d matrix per column
    constexpr int ROWS = D / PARTS;  // rows per slice
    constexpr int PST = 64;          // bytes per row of the probability operand (64 tokens)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    LDS_AS uint8_t* sm = (LDS_AS uint8_t*)smem_generic;
    const int wgi = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, c = lane & 15;
    const DevHead& H = blob[a.layer * a.n_kv + h];
    const int G = a.G, TB = a.tile_bytes, BB = a.buf_bytes;
    const int nvb = H.nvb;
    const int64_t zh = (int64_t)z * a.n_kv + h;

    // this wave's LDS: a ring of tile buffers; the probability operand [RB*16 rows][64
    // tokens] overwrites the key block of the current tile once its scores are done
    LDS_AS uint8_t* ring = sm + w * a.wave_bytes;
    LDS_AS int* flag = (LDS_AS int*)(sm + a.off_flag);

    // ---- sequence geometry (device arguments clamped: no read outside the cache)
    const int seq = seq_ids[z];
    int64_t len = min(min(seq_lens[z], a.max_len), a.n_tiles_cap * kTile);
    if (seq < 0 || seq >= a.n_seqs_cache) len = 0;
    const int64_t n_tiles = (len + kTile - 1) / kTile;
    const int64_t t_begin = (int64_t)wgi * a.tpg;
    const int64_t t_end = min(t_begin + a.tpg, n_tiles);
    const uint8_t* tiles = cache + (((int64_t)a.layer * a.n_seqs_cache + seq) * a.n_kv + h) * a.n_tiles_cap * TB;

    // ---- prologue: one batch of reads, waited for before the first tile load
    v4i Aq[NQM][RB];  // score A operands (query digits), resident for the whole loop
    {
        const v4i* src = (const v4i*)(qa_all + zh * NQM * RB * 1024);
#pragma unroll
        for (int m = 0; m < NQM; ++m)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) Aq[m][rb] = src[(m * RB + rb) * 64 + lane];
    }
    // key dwords per (MFMA, lane group): LDS byte offset of the record word in the tile and
    // the field mask, staged once in LDS ([m][g] -> 4 offsets then 4 masks) and read per tile
    LDS_AS u32x4* ksched = (LDS_AS u32x4*)(sm + a.off_ksched);
    for (int i = tid; i < NQM * 4 * 8; i += 256) {
        const int m = i >> 5, gg = (i >> 3) & 3, e = i & 7;
        ((LDS_AS uint32_t*)ksched)[i] =
            e < 4 ? 256u * (uint32_t)H.kq_word[m][gg][e] : H.kq_mask[m][gg][e - 4];
    }
    // value columns of this lane (column c of each block): tile byte offset of the lane's
    // 16 tokens in its record byte's plane, and the field mask repeated in every byte
    uint32_t voff[NVB], vmask[NVB];
#pragma unroll
    for (int cb = 0; cb < NVB; ++cb) {
        voff[cb] = 8u * (uint32_t)H.BK + (uint32_t)H.vb_plane[cb][c] + 16u * (uint32_t)g;
        vmask[cb] = 0x01010101u * (uint32_t)H.vb_mask[cb][c];
    }
    float qs[RB][3];  // digit scales of this lane's query head
    v4i sinit[RB];    // score accumulator start: the inverted-bit-7 correction of each row
    {
        const float* qsc = qscale + zh * kQscStride;
        const int* qci = (const int*)qsc + 16;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float mx = qsc[4 * rb + g];
            qs[rb][0] = mx;
            qs[rb][1] = mx * kQ1;
            qs[rb][2] = mx * kQ2;
            sinit[rb] = v4i{qci[16 * rb + 4 * g], qci[16 * rb + 4 * g + 1], qci[16 * rb + 4 * g + 2], 0};
        }
    }
    // the operands have arrived before any tile load: inside the loop the only vector
    // memory operations are this wave's tile loads
#pragma unroll
    for (int m = 0; m < NQM; ++m)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) asm volatile("" ::"v"(Aq[m][rb]));
    lds_barrier();  // the key schedule table is staged
#pragma unroll
    for (int cb = 0; cb < NVB; ++cb) asm volatile("" ::"v"(voff[cb]), "v"(vmask[cb]));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) asm volatile("" ::"v"(qs[rb][0]), "v"(sinit[rb]));

    // int32 sums of P digits x value bytes, relative to the reference max mref, and the
    // digit sums of this lane's probabilities (the row sums that undo the -128 of top
    // fields).  A rescale combines the three digit sums, scales by 2^(old - new) and
    // splits the result into digits again: the error is a float rounding of the sum.
    v4i acc_i[RB][NVB];
    int ones[RB][3];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb) acc_i[rb][cb] = v4i{0, 0, 0, 0};
        ones[rb][0] = ones[rb][1] = ones[rb][2] = 0;
    }
    float mref[RB], lsum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mref[rb] = -INFINITY, lsum[rb] = 0.0f;

    // ---- tiles t_begin + w, t_begin + w + 4, ...: a ring of NBW buffers per wave keeps up
    // to NBW - 1 of them in flight; the wave waits on its own load count
    const int NBW = a.nbw;
    const int nl = (TB + 1023) >> 10;  // load instructions per tile
    int64_t t = t_begin + w;
    for (int k = 0; k < NBW - 1 && t + kWaves * k < t_end; ++k)
        load_tile(tiles + (t + kWaves * k) * TB, ring + k * BB, TB, lane);
    int slot = 0;
    for (; t < t_end; t += kWaves) {
        // tile t has landed once only the later tiles' loads may be outstanding; this wave's
        // LDS reads of the slot refilled next are done
        wait_vm(nl * (int)min((int64_t)NBW - 2, (t_end - 1 - t) / kWaves));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int64_t tn = t + (int64_t)kWaves * (NBW - 1);
        if (tn < t_end) load_tile(tiles + tn * TB, ring + (slot == 0 ? NBW - 1 : slot - 1) * BB, TB, lane);
        LDS_AS uint8_t* curb = ring + slot * BB;
        slot = slot + 1 == NBW ? 0 : slot + 1;
        const int valid = (int)min((int64_t)kTile, len - t * kTile);

        // ---------------- scores: token group tg, lane (g, c) -> token 4c + tg.  One 16-byte
        // read gives a record word of the lane's four tokens; each operand dword keeps one
        // field per byte (a mask), so no shifts.
        v4i S[4][RB];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) S[tg][rb] = sinit[rb];
        const LDS_AS uint8_t* kbase = curb + 16 * c;  // record word 0 of tokens 4c..4c+3
#pragma unroll
        for (int m = 0; m < NQM; ++m) {
            const u32x4 koff = ksched[(m * 4 + g) * 2], kmask = ksched[(m * 4 + g) * 2 + 1];
            u32x4 x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = *(const LDS_AS u32x4*)(kbase + koff[i]);
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                const v4i B = v4i{(int)(x[0][tg] & kmask[0]), (int)(x[1][tg] & kmask[1]), (int)(x[2][tg] & kmask[2]),
                                  (int)(x[3][tg] & kmask[3])};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    S[tg][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aq[m][rb], B, S[tg][rb], 0, 0, 0);
            }
        }
        // lane (g, c) holds head 4rb+g, tokens 4c..4c+3, digit rows 0..2 (rows of heads
        // >= G have zero operands and stay harmless)
        float s[RB][4], tmx[RB];
        bool need = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float mx = -INFINITY;
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                s[rb][tg] = (float)S[tg][rb][0] * qs[rb][0] + (float)S[tg][rb][1] * qs[rb][1] +
                            (float)S[tg][rb][2] * qs[rb][2];
                if (valid < kTile) s[rb][tg] = 4 * c + tg < valid ? s[rb][tg] : -INFINITY;
                mx = fmaxf(mx, s[rb][tg]);
            }
            tmx[rb] = row16_max(mx);
            if (tmx[rb] > mref[rb]) need = true;
        }
        if (__any(need)) {
            // raise the reference of heads whose tile max passed it and rescale their sums
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float nref = tmx[rb] > mref[rb] ? tmx[rb] + kHeadroom : mref[rb];
                const float al = exp2f(mref[rb] - nref);
                lsum[rb] *= al;
                mref[rb] = nref;
#pragma unroll
                for (int cb = 0; cb < NVB; ++cb) {
                    int d0, d1, d2;
                    split256(combine256(acc_i[rb][cb][0], acc_i[rb][cb][1], acc_i[rb][cb][2]) * al, d0, d1, d2);
                    acc_i[rb][cb] = v4i{d0, d1, d2, 0};
                }
                split256(combine256(ones[rb][0], ones[rb][1], ones[rb][2]) * al, ones[rb][0], ones[rb][1], ones[rb][2]);
            }
        }
        // probabilities: N = round(p * 127 * 2^16) < 2^23; the bytes of N + 0x8080 with
        // bit 7 of the two low bytes inverted are its base-256 digits (top digit 0..127, the
        // others -128..127).  P[16 rb + 4 head + digit][token] over the tile's key block
        // (wave-private; the key words of this tile were all read above).
        LDS_AS uint8_t* P = curb;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            uint32_t Mv[4];
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                const float p = __builtin_amdgcn_exp2f(s[rb][tg] - mref[rb]);
                lsum[rb] += p;
                Mv[tg] = (uint32_t)fmaf(p, kPScale, 32896.5f);  // truncation: round(p 127 2^16) + 0x8080
            }
            const uint32_t t01 = __builtin_amdgcn_perm(Mv[1], Mv[0], 0x05010400u);  // b0 b0' b1 b1'
            const uint32_t t23 = __builtin_amdgcn_perm(Mv[3], Mv[2], 0x05010400u);
            const uint32_t u01 = __builtin_amdgcn_perm(Mv[1], Mv[0], 0x0C0C0602u);  // b2 b2'
            const uint32_t u23 = __builtin_amdgcn_perm(Mv[3], Mv[2], 0x0C0C0602u);
            const uint32_t w2 = __builtin_amdgcn_perm(u23, u01, 0x05040100u);                // top digits
            const uint32_t w1 = __builtin_amdgcn_perm(t23, t01, 0x07060302u) ^ 0x80808080u;  // middle
            const uint32_t w0 = __builtin_amdgcn_perm(t23, t01, 0x05040100u) ^ 0x80808080u;  // low
            ones[rb][0] = __builtin_amdgcn_sdot4((int)w2, 0x01010101, ones[rb][0], false);
            ones[rb][1] = __builtin_amdgcn_sdot4((int)w1, 0x01010101, ones[rb][1], false);
            ones[rb][2] = __builtin_amdgcn_sdot4((int)w0, 0x01010101, ones[rb][2], false);
            LDS_AS uint32_t* pw = (LDS_AS uint32_t*)(P + (16 * rb + 4 * g) * PST + 4 * c);
            pw[0] = w2;
            pw[PST / 4] = w1;
            pw[2 * PST / 4] = w0;
            pw[3 * PST / 4] = 0u;  // digit row 3 multiplies nothing
        }
        asm volatile("" ::: "memory");  // the operand reads below follow this wave's writes
        v4i Ap[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) Ap[rb] = *(const LDS_AS v4i*)(P + (16 * rb + c) * PST + 16 * g);

        // ---------------- values: column c of block cb = one field; its B operand is the
        // lane's 16 tokens of the field's byte plane under the field mask
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb) {
            const u32x4 x = *(const LDS_AS u32x4*)(curb + voff[cb]);
            const v4i B = v4i{(int)(x[0] & vmask[cb]), (int)(x[1] & vmask[cb]), (int)(x[2] & vmask[cb]),
                              (int)(x[3] & vmask[cb])};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc_i[rb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ap[rb], B, acc_i[rb][cb], 0, 0, 0);
        }
    }

    // ---------------- epilogue: the four waves' results meet in LDS (ring reused).  Per
    // wave and head: reference max, sum, the probability digit sum (x 2^16 / 127 = 2^16 sum
    // of p), and per value column the accumulator / 127 (= sum of p x stored byte).
    wait_all();
    lds_barrier();
    const int ld = D + 2;
    const int ncol = 16 * NVB;
    LDS_AS float* wm = (LDS_AS float*)sm;                 // [4 waves][RB*4 heads] reference maxima
    LDS_AS float* wl = wm + kWaves * RB * 4;              // [4 waves][RB*4 heads] sums
    LDS_AS float* wo = wl + kWaves * RB * 4;              // [4 waves][RB*4 heads] 128 x digit sums / 127
    LDS_AS float* wa = wo + kWaves * RB * 4;              // [4 waves][RB*4 heads][ncol] columns
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float ls = row16_sum(lsum[rb]);
        const float os = row16_sum(combine256(ones[rb][0], ones[rb][1], ones[rb][2]));
        if (c == 0) {
            wm[w * RB * 4 + 4 * rb + g] = mref[rb];
            wl[w * RB * 4 + 4 * rb + g] = ls;
            wo[w * RB * 4 + 4 * rb + g] = os * (128.0f / 127.0f);
        }
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb)
            if (cb < nvb)
                wa[(w * RB * 4 + 4 * rb + g) * ncol + 16 * cb + c] =
                    combine256(acc_i[rb][cb][0], acc_i[rb][cb][1], acc_i[rb][cb][2]) * (1.0f / 127.0f);
    }
    lds_barrier();
    const int W = a.wg_per_head, NG = a.n_grp;
    const int grp_size = (W + NG - 1) / NG;
    const int grp = wgi / grp_size;
    float* pout = part1 + (zh * W + wgi) * G * ld;
    for (int i = tid; i < G * ld; i += 256) {
        const int hh = i / ld, col = i - hh * ld;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, wm[ww * RB * 4 + hh]);
        float e[kWaves];
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float m = wm[ww * RB * 4 + hh];
            e[ww] = m == -INFINITY ? 0.0f : exp2f(m - M);
        }
        float v;
        if (col == 0) {
            v = M;
        } else if (col == 1) {
            v = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) v += e[ww] * wl[ww * RB * 4 + hh];
        } else {
            // channel jj: its fields' columns, each (column + 128 flip sum p) 2^(shift - pos)
            const int jj = col - 2;
            v = 0.0f;
            for (int f = H.vch_first[jj]; f < H.vch_first[jj + 1]; ++f) {
                const uint32_t en = H.vch_col[f];
                const int cc = en & 511;
                const float sc = __builtin_amdgcn_ldexpf(1.0f, (int)((en >> 9) & 15) - 8);
                const bool top = (en >> 13) & 1;
                float x = 0.0f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww)
                    x += e[ww] * (wa[(ww * RB * 4 + hh) * ncol + cc] + (top ? wo[ww * RB * 4 + hh] : 0.0f));
                v = fmaf(sc, x, v);
            }
        }
        st_dev(pout + i, v);
    }
    wait_vm(0);     // this wave's partial stores have completed
    lds_barrier();  // ... and every wave's
    const int members1 = min(grp_size, W - grp * grp_size);
    if (tid == 0) *flag = atomicInc(cnt1 + zh * NG + grp, (uint32_t)members1 - 1u) == (uint32_t)members1 - 1u;
    lds_barrier();
    if (!*flag) return;

    // ---------------- merges.  Each group merger combines its group in the coefficient
    // domain and applies the inverse transform to its own (unnormalised) result,
    // y = U_V (step * A); the last of them combines the y's: o = obias + Y / L.
    const int ii = tid % D, pt = __builtin_amdgcn_readfirstlane(tid / D);  // (column, row slice)
    const float* vb = H.UVt + pt * ROWS * D + ii;  // UVt[j * d + i] = U_V[i][j]
    float uv[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) uv[r] = vb[r * D];
    // thread columns: i = tid + 256 k -> query head i / D, coefficient i % D
    constexpr int CPT = RB * 4 * D / 256;
    constexpr int CH = RB == 1 ? 8 : 4;  // partials per merge round
    float M[CPT], L[CPT], A[CPT];
    merge_cols<D, CPT, CH>(part1 + (zh * W + grp * grp_size) * G * ld, members1, G, tid, M, L, A);
    LDS_AS float* cbar = (LDS_AS float*)sm;  // [G][D] step * A
    LDS_AS float* red = cbar + G * D;        // [PARTS][G][D]
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int i = tid + 256 * k, hh = i / D, jj = i - hh * D;
        if (hh < G) cbar[i] = H.bitsV[jj] ? H.stepV[jj] * A[k] : 0.0f;
    }
    lds_barrier();
    for (int hh = 0; hh < G; ++hh) {
        float o = 0.0f;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) o = fmaf(uv[r], cbar[hh * D + pt * ROWS + r], o);
        red[(pt * G + hh) * D + ii] = o;
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int i = tid + 256 * k, hh = i / D, i2 = i - hh * D;
        float y = 0.0f;
        if (hh < G) {
#pragma unroll
            for (int p2 = 0; p2 < PARTS; ++p2) y += red[(p2 * G + hh) * D + i2];
        }
        A[k] = y;
    }
    if (NG > 1) {
        float* gout = part2 + (zh * NG + grp) * G * ld;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int i = tid + 256 * k, hh = i / D, jj = i - hh * D;
            if (hh < G) {
                st_dev(gout + hh * ld + 2 + jj, A[k]);
                if (jj == 0) {
                    st_dev(gout + hh * ld, M[k]);
                    st_dev(gout + hh * ld + 1, L[k]);
                }
            }
        }
        wait_vm(0);
        lds_barrier();
        if (tid == 0) *flag = atomicInc(cnt2 + zh, (uint32_t)NG - 1u) == (uint32_t)NG - 1u;
        lds_barrier();
        if (!*flag) return;
        merge_cols<D, CPT, CH>(part2 + zh * NG * G * ld, NG, G, tid, M, L, A);
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int i = tid + 256 * k, hh = i / D, i2 = i - hh * D;
        if (hh < G) out[(zh * G + hh) * D + i2] = L[k] > 0.0f ? H.obias[i2] + A[k] / L[k] : H.muV[i2];
    }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
struct Variant {
    int rb, nqm, nvb;
};
// compile-time (row blocks, score operand blocks, value column blocks) bounds available;
// (the operand blocks of a head must fit the bounds; unused blocks multiply zero)
constexpr Variant kVariants[] = {{1, 2, 4},  {1, 2, 8},  {1, 3, 8},  {1, 3, 10}, {1, 4, 12}, {1, 6, 16},
                                 {1, 8, 24}, {1, 16, 24}, {2, 2, 8},  {2, 3, 10}, {2, 4, 12}, {2, 8, 24},
                                 {2, 16, 24}, {3, 4, 12}, {3, 16, 24}, {4, 4, 12}, {4, 16, 24}};

struct Plan {
    Variant v;
    int nqm_max, nvb_max, tpg, wg_per_head, n_grp, wgs_per_cu;
    size_t qa_bytes, qsc_bytes, part1_bytes, part2_bytes;
    int64_t n_counters;
    DecodeArgs args;
    size_t lds;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }

int make_plan(const aatc_codebook* cb, int layer, int n_seqs, int64_t max_len, Plan& p) {
    const int G = cb->group, d = cb->d;
    const int RB = (G + 3) / 4;
    const int PARTS = 256 / d;
    p.nqm_max = 0;
    p.nvb_max = 0;
    for (int h = 0; h < cb->n_kv; ++h) {
        const DevHead& D = cb->blob[(size_t)layer * cb->n_kv + h];
        p.nqm_max = std::max(p.nqm_max, D.nqm);
        p.nvb_max = std::max(p.nvb_max, D.nvb);
    }
    bool found = false;
    for (const Variant& v : kVariants)
        if (v.rb == RB && v.nqm >= p.nqm_max && v.nvb >= p.nvb_max) {
            p.v = v;
            found = true;
            break;
        }
    if (!found)
        return set_error(AATC_ERR_UNSUPPORTED, "no decode variant for %d query heads, %d score MFMAs and %d value blocks", G,
                         p.nqm_max, p.nvb_max);
    const int64_t tiles = n_tiles_of(max_len);
    const int64_t total = tiles * cb->n_kv * (int64_t)n_seqs;
    // one wave per tile at a time: aim for every wave slot of the chip busy
    const int64_t target = 256 * (int64_t)waves_for(p.v.rb, p.v.nqm, p.v.nvb) * kWaves;
    p.tpg = (int)std::max<int64_t>(kWaves, (total + target - 1) / target * kWaves);
    p.wg_per_head = (int)((tiles + p.tpg - 1) / p.tpg);
    p.n_grp = (p.wg_per_head + kMergeGroup - 1) / kMergeGroup;
    const size_t ld = (size_t)d + 2;
    p.qa_bytes = (size_t)n_seqs * cb->n_kv * p.v.nqm * RB * 1024;
    p.qsc_bytes = (size_t)n_seqs * cb->n_kv * kQscStride * sizeof(float);
    p.part1_bytes = (size_t)n_seqs * cb->n_kv * p.wg_per_head * G * ld * sizeof(float);
    p.part2_bytes = (size_t)n_seqs * cb->n_kv * p.n_grp * G * ld * sizeof(float);
    p.n_counters = (int64_t)n_seqs * cb->n_kv * (p.n_grp + 1);
    if (p.n_counters > kCounterSlots)
        return set_error(AATC_ERR_CAPACITY, "%d sequences x %d kv-heads need %lld arrival counters (at most %d); split the batch",
                         n_seqs, cb->n_kv, (long long)p.n_counters, kCounterSlots);
    DecodeArgs& a = p.args;
    a.G = G;
    a.tile_bytes = 8 * cb->total_bits;
    a.tpg = p.tpg;
    a.wg_per_head = p.wg_per_head;
    a.n_grp = p.n_grp;
    a.buf_bytes = (int)al16(a.tile_bytes);
    // the probability operand (RB KiB) overwrites the tile's key block (8 B_K bytes)
    int bk_min = 1 << 30;
    for (int h = 0; h < cb->n_kv; ++h) bk_min = std::min(bk_min, cb->blob[(size_t)layer * cb->n_kv + h].BK);
    if (RB * 1024 > 8 * bk_min)
        return set_error(AATC_ERR_UNSUPPORTED, "%d key bits per token are too few for %d query heads", bk_min, G);
    // the epilogue and the merges reuse the buffers
    const size_t epi = ((size_t)3 * kWaves * RB * 4 + (size_t)kWaves * RB * 4 * 16 * p.v.nvb) * sizeof(float);
    const size_t mrg = ((size_t)G * d + (size_t)PARTS * G * d) * sizeof(float);
    // ring depth: the deepest that the workgroups resident per CU (set by registers) leave
    // room for, between 2 and 4 buffers per wave
    const int wgs = waves_for(p.v.rb, p.v.nqm, p.v.nvb);
    const size_t budget = (size_t)(160 * 1024) / wgs - 64 - (size_t)p.v.nqm * 128;
    a.nbw = 2;
    while (a.nbw < 4 && (size_t)kWaves * (a.nbw + 1) * a.buf_bytes <= budget) ++a.nbw;
    a.wave_bytes = a.nbw * a.buf_bytes;
    a.off_ksched = (int)al16(std::max({(size_t)kWaves * a.wave_bytes, epi, mrg}));
    a.off_flag = a.off_ksched + p.v.nqm * 4 * 8 * 4;
    p.lds = a.off_flag + 16;
    p.wgs_per_cu = std::min<int>(wgs, (int)((160 * 1024) / p.lds));
    if (p.lds > 160 * 1024 - 256)
        return set_error(AATC_ERR_UNSUPPORTED, "decode needs %zu bytes of LDS per workgroup", p.lds);
    return AATC_OK;
}

// Measurement hook (aatc_profile_begin / aatc_profile_end): event pairs recorded around
// the split-decode kernel of the next calls.
struct Profile {
    std::mutex mu;
    bool active = false;
    std::vector<hipEvent_t> ev;  // 2 per call slot
    int used = 0;
};
Profile& profile() {
    static Profile p;
    return p;
}

// the event pair for this call, or nulls when not profiling (or out of slots)
void profile_slot(hipEvent_t& a, hipEvent_t& b) {
    Profile& P = profile();
    std::lock_guard<std::mutex> lk(P.mu);
    a = b = nullptr;
    if (!P.active || 2 * (P.used + 1) > (int)P.ev.size()) return;
    a = P.ev[2 * P.used];
    b = P.ev[2 * P.used + 1];
    ++P.used;
}

template <int RB, int NQM, int NVB, int D>
int launch_decode(const Plan& p, int n_seqs, hipStream_t st, const DevHead* blob, const uint8_t* cache,
                  const int32_t* ids, const int64_t* lens, const uint16_t* q, uint8_t* qa, float* qsc, float* part1,
                  float* part2, uint32_t* cnt1, uint32_t* cnt2, float* out) {
    const DecodeArgs& a = p.args;
    hipLaunchKernelGGL((qprep_kernel<RB, NQM, D>), dim3(a.n_kv, n_seqs), dim3(256), 0, st, blob, a.layer, a.n_kv, a.G,
                       q, (uint32_t*)qa, qsc);
    HIP_TRY(hipGetLastError());
    if (p.lds > 64 * 1024)
        HIP_TRY(hipFuncSetAttribute((const void*)decode_kernel<RB, NQM, NVB, D>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds));
    hipEvent_t e0, e1;
    profile_slot(e0, e1);
    if (e0) HIP_TRY(hipEventRecord(e0, st));
    hipLaunchKernelGGL((decode_kernel<RB, NQM, NVB, D>), dim3(p.wg_per_head, a.n_kv, n_seqs), dim3(256), p.lds, st,
                       blob, cache, a, ids, lens, qa, qsc, part1, part2, cnt1, cnt2, out);
    HIP_TRY(hipGetLastError());
    if (e1) HIP_TRY(hipEventRecord(e1, st));
    return AATC_OK;
}

}  // namespace

extern "C" int aatc_profile_begin(int32_t n) {
    if (n < 1) return set_error(AATC_ERR_INVALID_ARG, "need n >= 1");
    Profile& P = profile();
    std::lock_guard<std::mutex> lk(P.mu);
    if (P.active) return set_error(AATC_ERR_INVALID_ARG, "profiling already active");
    P.ev.assign(2 * (size_t)n, nullptr);
    for (auto& e : P.ev) {
        hipError_t rc = hipEventCreate(&e);
        if (rc != hipSuccess) {
            for (auto& f : P.ev)
                if (f) (void)hipEventDestroy(f);
            P.ev.clear();
            return set_error(AATC_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(rc));
        }
    }
    P.used = 0;
    P.active = true;
    return AATC_OK;
}

extern "C" int aatc_profile_end(float* ms, int32_t* n_out) {
    if (!ms || !n_out) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    Profile& P = profile();
    std::lock_guard<std::mutex> lk(P.mu);
    if (!P.active) return set_error(AATC_ERR_INVALID_ARG, "profiling not active");
    int rc = AATC_OK;
    for (int i = 0; i < P.used && rc == AATC_OK; ++i) {
        hipError_t e = hipEventSynchronize(P.ev[2 * i + 1]);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], P.ev[2 * i], P.ev[2 * i + 1]);
        if (e != hipSuccess) rc = set_error(AATC_ERR_HIP, "profile events: %s", hipGetErrorString(e));
    }
    *n_out = P.used;
    for (auto& e : P.ev) (void)hipEventDestroy(e);
    P.ev.clear();
    P.used = 0;
    P.active = false;
    return rc;
}

extern "C" int aatc_decode_workspace_bytes(const aatc_codebook* cb, int32_t n_seqs, int64_t max_len, size_t* bytes) {
    if (!cb || !bytes) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n_seqs < 1 || max_len < 1) return set_error(AATC_ERR_INVALID_ARG, "need n_seqs >= 1 and max_len >= 1");
    size_t worst = 0;
    for (int layer = 0; layer < cb->n_layers; ++layer) {
        Plan p;
        int rc = make_plan(cb, layer, n_seqs, max_len, p);
        if (rc) return rc;
        worst = std::max(worst, kCounterBytes + al256(p.qa_bytes) + al256(p.qsc_bytes) + al256(p.part1_bytes) +
                                    p.part2_bytes);
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
    const size_t need =
        kCounterBytes + al256(p.qa_bytes) + al256(p.qsc_bytes) + al256(p.part1_bytes) + p.part2_bytes;
    if (ws_bytes < need) return set_error(AATC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    uint8_t* wsp = (uint8_t*)workspace;
    uint32_t* cnt1 = (uint32_t*)wsp;  // [n_seqs][n_kv][n_grp] group arrivals
    uint32_t* cnt2 = cnt1 + (size_t)n_seqs * cb->n_kv * p.n_grp;  // [n_seqs][n_kv] group-merger arrivals
    uint8_t* qa = wsp + kCounterBytes;  // [n_seqs][n_kv][NQM][RB][64][16] score operands
    float* qsc = (float*)(qa + al256(p.qa_bytes));  // [n_seqs][n_kv][80] digit scales, accumulator starts
    float* part1 = (float*)((uint8_t*)qsc + al256(p.qsc_bytes));
    float* part2 = (float*)((uint8_t*)part1 + al256(p.part1_bytes));
    DecodeArgs& a = p.args;
    a.layer = layer;
    a.n_kv = cb->n_kv;
    a.n_seqs_cache = cache->n_seqs;
    a.n_tiles_cap = n_tiles_of(cache->max_tokens);
    a.max_len = max_len;
    const DevHead* blob = (const DevHead*)d_blob;
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* c = (const uint8_t*)cache->data;
#define AATC_DECODE_CASE(rb_, nqm_, nvb_)                                                                         \
    if (p.v.rb == rb_ && p.v.nqm == nqm_ && p.v.nvb == nvb_)                                                      \
        return cb->d == 64 ? launch_decode<rb_, nqm_, nvb_, 64>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, qa,  \
                                                                qsc, part1, part2, cnt1, cnt2, out)                \
                           : launch_decode<rb_, nqm_, nvb_, 128>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, qa, \
                                                                 qsc, part1, part2, cnt1, cnt2, out);
    AATC_DECODE_CASE(1, 2, 4)
    AATC_DECODE_CASE(1, 2, 8)
    AATC_DECODE_CASE(1, 3, 8)
    AATC_DECODE_CASE(1, 3, 10)
    AATC_DECODE_CASE(1, 4, 12)
    AATC_DECODE_CASE(1, 6, 16)
    AATC_DECODE_CASE(1, 8, 24)
    AATC_DECODE_CASE(1, 16, 24)
    AATC_DECODE_CASE(2, 2, 8)
    AATC_DECODE_CASE(2, 3, 10)
    AATC_DECODE_CASE(2, 4, 12)
    AATC_DECODE_CASE(2, 8, 24)
    AATC_DECODE_CASE(2, 16, 24)
    AATC_DECODE_CASE(3, 4, 12)
    AATC_DECODE_CASE(3, 16, 24)
    AATC_DECODE_CASE(4, 4, 12)
    AATC_DECODE_CASE(4, 16, 24)
#undef AATC_DECODE_CASE
    return set_error(AATC_ERR_UNSUPPORTED, "decode variant missing");
}
