// Split-context decode attention over the packed cache (gfx950).
//
// Pages: "Attention-Aware Transform Coding Guide" ("Formal Attention Distortion Model":
// o = softmax(q K^T / sqrt(d)) V; KLT section K' = K U_K); "Spend Bits Where Queries Look"
// abstract (decoding reads the whole cache every step and is bandwidth-bound; a
// non-orthogonal key transform).  Key coefficients are c = (k - mu) T_K (T_K = U_K for the
// KLT), so q.k = (T_K^{-1} q).c + q.mu: keys are scored in the transform domain and never
// reconstructed (the q.mu term is the same for every token); values are inverse-transformed
// once per query head.
//
// Two kernels on the caller's stream.
//   decode - W workgroups (one per CU, 8 or 12 waves) share the 64-token tiles of one
//            (sequence, kv-head).
//     prologue - every workgroup forms q' = T_K^{-1} q for the kv-head's query heads on bf16
//                MFMAs (the matrix is read from the device cache), scales it by the key
//                steps (and log2 e / sqrt d) and builds the score operands: per key field a
//                query weight (the field's code shift over its bit position), scaled per
//                head so the largest is 127 and split into three int8 digits laid out as
//                MFMA A operands, plus per head the digit scales and the accumulator's start
//                value; the first tiles stream meanwhile;
//     tiles    - workgroup i takes an even share of the tiles, its waves every NW-th of
//                those, streamed through private rings of LDS buffers (direct buffer loads
//                into LDS, counted waits, no workgroup barriers in the loop).  Per tile:
//       scores  - v_mfma_i32_16x16x64_i8 with rows 4*head + digit and one column per token:
//                 a B dword is a key-record word ANDed with a mask that keeps one field per
//                 byte; with bit 7 of stored bytes inverted such a byte reads as
//                 field * 2^pos (- 128 when the field ends at bit 7), the 2^pos is divided
//                 out of the query digits and the -128 is the accumulator's start value;
//       softmax - online, base 2, reference max raised lazily with headroom; probabilities
//                 p * 127 * 2^16 are rounded to integers whose bytes are three int8 digits
//                 (base 256), written over the tile's key block as the next A operand;
//       values  - the same MFMA with one column per value field: the B operand of a column
//                 is 16 bytes of its record byte's plane (16 tokens) ANDed with the field
//                 mask;
//     epilogue - the waves meet in LDS; the workgroup writes one partial per query head:
//                reference max, sum of p, sum of p x (128 for fields ending at bit 7), and
//                per value column sum of p x stored byte.
//   merge  - one workgroup per (sequence, kv-head, query head, 32 output channels) combines
//            the W partials, turns columns into value coefficients (weight 2^(shift - pos),
//            plus the 128 for fields ending at bit 7), and writes its slice of
//            o = obias + U_V (step * A) / L.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <mutex>
#include <vector>

#include "hip_common.h"

using aatc::check_cache;
using aatc::DevHead;
using aatc::kTile;
using aatc::kVqSize;
using aatc::bf16f;
using aatc::n_tiles_of;
using aatc::code_byte;
using aatc::set_error;

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kMergeThreads = 256;  // threads per merge workgroup
constexpr float kHeadroom = 2.0f;    // log2 headroom added to the reference max at a rescale
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kQ1 = 1.0f / 254.0f, kQ2 = 1.0f / 64516.0f;  // query digit weights (base 254)
constexpr float kP1 = 1.0f / 256.0f, kP2 = 1.0f / 65536.0f;  // probability digit weights (base 256)
constexpr float kPScale = 127.0f * 65536.0f;                  // p -> integer of three digits
constexpr int kPartHead = 4;  // partial entries before the columns: max, sum, top-field sum, pad

// the load instructions of one cache tile (stream_tile)
struct TileLoads {
    int n16, r4, r2, r1;
};

struct DecodeArgs {
    int layer, n_kv, G, n_seqs_cache;
    int64_t n_tiles_cap;
    int64_t max_len;
    int tile_bytes, wg_per_head, part_ld;
    // append mode: one new token per (sequence, kv-head) - keys, values [n_seqs][n_kv][d]
    // bf16 - is written at slot seq_lens[s] and attended to (null: plain decode)
    const uint16_t* k_new;
    const uint16_t* v_new;
    TileLoads tl;  // the load instructions of one tile
    // LDS carve-up (bytes): slot k of wave w's ring at (k * 4 + w) * buf_bytes; the
    // prologue's scratch at off_scratch, beside the ring (early = nbw: every slot streams
    // from the start) or in its last nbw - early slots
    int nbw, buf_bytes, early, off_scratch, off_ksched, off_rec, off_sync;
    int off_pbuf;  // per-wave probability operands [NW][RB KiB] when the key block is smaller, else -1
    int fused;  // the last workgroup of each (sequence, kv-head) merges (no merge launch)
    // sequences per layer: grid index z covers layer a.layer + z / n_seqs_call, sequence slot
    // z mod n_seqs_call (one layer per launch unless layers are batched)
    int n_seqs_call;
};

// LDS-only workgroup barrier: this wave's LDS operations are complete, then s_barrier.
// (Global->LDS tile loads in flight are not waited for; their waits are explicit.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS add written as an instruction of its own: the compiler makes every LDS atomic wait for
// all direct-to-LDS copies in flight (vmcnt(0)), which would stall the tile stream.  LDS
// operations complete in order; the LDS-only barrier waits for them.
__device__ __forceinline__ void lds_add_async(LDS_AS int* p, int v) {
    asm volatile("ds_add_u32 %0, %1" ::"v"(p), "v"(v) : "memory");
}

// LDS OR as an instruction of its own (see lds_add_async)
__device__ __forceinline__ void lds_or_async(LDS_AS uint32_t* p, uint32_t v) {
    asm volatile("ds_or_b32 %0, %1" ::"v"(p), "v"(v) : "memory");
}

// LDS-counter meeting of a subset of the workgroup's waves (the others carry on): this wave's
// LDS operations complete, lane 0 adds one arrival, then the wave waits until `target`
// arrivals have been counted.  LDS operations complete in order, so data written before an
// arrival is visible to every wave that has seen the count.
__device__ __forceinline__ void q_wait(LDS_AS int* ctr, int target) {
    while (*(volatile LDS_AS int*)ctr < target) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void q_sync(LDS_AS int* ctr, int target, int lane) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) lds_add_async(ctr, 1);
    while (*(volatile LDS_AS int*)ctr < target) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}

// Scalar loads of a head's record sizes (DevHead::BK, BV at byte offset 4), a sequence id and a
// sequence length, waited for inside the same statement on the scalar counter only.
__device__ __forceinline__ void load_head_and_sequence(const DevHead* hp, const int32_t* idp, const int64_t* lenp,
                                                       int& BK, int& BV, int& seq, int64_t& len) {
    static_assert(offsetof(DevHead, BK) == 4 && offsetof(DevHead, BV) == 8, "record sizes at bytes 4..11");
    uint64_t kv, ln;
    uint32_t sq;
    asm volatile(
        "s_load_dwordx2 %0, %3, 0x4\n\t"
        "s_load_dword %1, %4, 0x0\n\t"
        "s_load_dwordx2 %2, %5, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(kv), "=&s"(sq), "=&s"(ln)
        : "s"(hp), "s"(idp), "s"(lenp));
    BK = (int)(uint32_t)kv;
    BV = (int)(uint32_t)(kv >> 32);
    seq = (int)sq;
    len = (int64_t)ln;
}

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
__device__ __forceinline__ float wave_max(float x) {
    x = row16_max(x);
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Stream one tile (bytes, a multiple of 16) from global memory into LDS with one wave:
// 1 KiB per instruction, 16 bytes per lane (LDS address = chunk base + 16 * lane).  The
// loads carry the non-temporal hint (cache policy bit 1): the cache is read once per step,
// and with the default policy these direct-to-LDS loads stream at about half the rate.
constexpr int kStreamPolicy = 2;
template <int POLICY>
__device__ __forceinline__ void load_tile_p(const uint8_t* src, LDS_AS uint8_t* lds, int bytes, int lane) {
    for (int off = 0; off < bytes; off += 1024) {
        const int o = off + 16 * lane;
        if (o < bytes) __builtin_amdgcn_global_load_lds((const void*)(src + o), (LDS_AS void*)(lds + off), 16, 0, POLICY);
    }
}
__device__ __forceinline__ void load_tile(const uint8_t* src, LDS_AS uint8_t* lds, int bytes, int lane, int policy) {
    if (policy == kStreamPolicy)
        load_tile_p<kStreamPolicy>(src, lds, bytes, lane);
    else
        load_tile_p<0>(src, lds, bytes, lane);
}

// Stream one cache tile (64 token slots of B bits: 64 x B / 8 bytes, so every lane's share is
// whole bytes) with all lanes active: n16 loads of 16 bytes per lane (1 KiB each), then the
// lane share's remainder in 4-, 2- and 1-byte loads (r4, r2, r1 of them).  Buffer loads
// over the (sequence, kv-head)'s tile range: the tile's offset is a scalar, the lane's a
// fixed register, so a load costs no vector instruction (and a read past the range returns
// zeros instead of faulting).
__device__ __forceinline__ void stream_tile(__amdgpu_buffer_rsrc_t rs, uint32_t off, LDS_AS uint8_t* lds,
                                            const TileLoads& tl, int lane) {
    for (int k = 0; k < tl.n16; ++k, off += 1024)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lds + 1024 * k), 16, 16 * lane, off, 0, kStreamPolicy);
    LDS_AS uint8_t* l = lds + 1024 * tl.n16;
    for (int k = 0; k < tl.r4; ++k, off += 256, l += 256)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)l, 4, 4 * lane, off, 0, kStreamPolicy);
    if (tl.r2) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)l, 2, 2 * lane, off, 0, kStreamPolicy);
        off += 128;
        l += 128;
    }
    if (tl.r1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)l, 1, lane, off, 0, kStreamPolicy);
}

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

// Registers per lane grow with the row blocks and value column blocks.  One row block with
// at most 3 score operand blocks and 8 value column blocks fits 168 VGPRs (three waves per
// SIMD) without spills; the rest take two waves (256 VGPRs).  A spill reloaded in the tile
// loop would wait for every tile load in flight.  The LDS plan matches the wave count.
// The key schedule (per score MFMA: four record-word offsets and four masks of this lane's
// group) stays in registers when it is small.
constexpr bool ksched_in_regs(int nqm) { return nqm <= 2; }
constexpr int waves_for(int rb, int nqm, int nvb) { return rb == 1 && nqm <= 3 && nvb <= 8 ? 3 : 2; }
// A decode workgroup fills one CU at that occupancy: 4 SIMDs x waves_for waves.
constexpr int wg_waves(int rb, int nqm, int nvb) { return 4 * waves_for(rb, nqm, nvb); }
// the epilogue combines the waves' results for at most two row blocks at a time
constexpr int epilogue_row_blocks(int rb) { return rb < 2 ? rb : 2; }

// bytes of the score operands in LDS: the A operands [NQM][RB][64 lanes] (16 bytes each),
// then per (row block, head) a 32-byte lane record (three float digit scales, three int
// score start values, two zero words)
constexpr int operand_bytes(int rb, int nqm) { return nqm * rb * 1024 + rb * 4 * 32; }
// bytes of the decode prologue's LDS scratch: the operands, the value columns [NVB][16],
// the slot descriptors [NQM][4][16], q'' [4 RB][D], block maxima [D / 16][16], bit-7 digit
// sums [RB][16]
constexpr int kMaxRecord = 2 * aatc::kMaxD;  // bytes of a token's two records at 8 bits per element
constexpr int scratch_bytes(int rb, int nqm, int nvb, int d) {
    return operand_bytes(rb, nqm) + nvb * 64 + nqm * 128 + 16 * rb * d + 4 * d + 64 * rb;
}

// Append mode: the codes of one token for column block cb of 2 D / 16 (key blocks, then
// value blocks), OR-ed into its records staged in LDS (key record bytes, then value record
// bytes).  The projection runs on the encoder's MFMAs with the same operands, start value
// and order (hi, lo and, for three-term bases, mid per k-step), and the same quantizer, so
// the codes equal those the encoder writes for the token.  Lane (0, c) holds the token's coefficient of channel
// 16 (cb mod D / 16) + c (MFMA row 0; the other rows are zero).
template <int D>
__device__ __forceinline__ void append_block(const DevHead& H, const uint16_t* xk, const uint16_t* xv, int cb,
                                             LDS_AS uint32_t* rec, int g, int c) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    constexpr int NB = D / 16, KS = D / 32;
    const bool isV = cb >= NB;
    const int j = 16 * (isV ? cb - NB : cb) + c;
    const uint16_t* uh = isV ? H.EVt_hi : H.EKt_hi;
    const uint16_t* ul = isV ? H.EVt_lo : H.EKt_lo;
    const uint16_t* um = isV ? H.EVt_mid : H.EKt_mid;
    const bool t3 = H.enc_terms == 3;
    const uint16_t* x = isV ? xv : xk;
    bf16x8 bh[KS], bl[KS], bm[KS], av[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bh[ks] = *(const bf16x8*)(uh + j * D + 32 * ks + 8 * g);
        bl[ks] = *(const bf16x8*)(ul + j * D + 32 * ks + 8 * g);
        bm[ks] = *(const bf16x8*)(um + j * D + 32 * ks + 8 * g);
        const bf16x8 xa = *(const bf16x8*)(x + 32 * ks + 8 * g);
        av[ks] = c == 0 ? xa : bf16x8{};
    }
    const float st = isV ? H.estartV[j] : H.estartK[j];
    const int bits = isV ? H.bitsV[j] : H.bitsK[j];
    const uint32_t* pc = isV ? H.cpieceV : H.cpieceK;
    const int16_t* cf = isV ? H.cfirstV : H.cfirstK;
    const int p0 = cf[j], p1 = cf[j + 1];
    const int base = isV ? H.BK / 8 : 0;  // record byte of the value record's byte 0
    f4 acc = f4{st, st, st, st};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks], bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks], bl[ks], acc, 0, 0, 0);
        if (t3) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks], bm[ks], acc, 0, 0, 0);
    }
    if (g == 0 && bits > 0) {
        const uint32_t code = code_byte(acc[0], (float)((1 << bits) - 1), 0, 0u);
        for (int p = p0; p < p1; ++p) {  // piece = byte | pos << 8 | width << 12 | shift << 16
            const uint32_t pcv = pc[p];
            const int rb = base + (int)(pcv & 0xff), pos = (pcv >> 8) & 7, wd = (pcv >> 12) & 15, sh = (pcv >> 16) & 15;
            const uint32_t v = ((code >> sh) & ((1u << wd) - 1u)) << pos;
            lds_or_async(rec + (rb >> 2), v << (8 * (rb & 3)));
        }
    }
}

// The new token's codes of the column blocks cb = w0, w0 + STEP, ... (NBW of them) of one
// wave, with append_block's arithmetic and order, but the memory accesses of all the blocks
// batched into two rounds instead of two per block: (1) every block's channel start value,
// bits and piece range, the token's key and value rows and the first half of the blocks'
// operands, (2) every block's first field pieces (a channel has at most kPrePieces; more are
// read one by one) and the second half's operands.  Under the tile stream of the other
// workgroups a round trip to memory takes over a microsecond, so the owner workgroup's
// prologue would otherwise be the last to finish.
constexpr int kPrePieces = 3;
template <int D, int NBW, int STEP>
__device__ __forceinline__ void append_blocks(const DevHead& H, const uint16_t* xk, const uint16_t* xv, int w0,
                                              LDS_AS uint32_t* rec, int g, int c) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    constexpr int NB = D / 16, KS = D / 32, HALF = (NBW + 1) / 2;
    const bool t3 = H.enc_terms == 3;
    int jb[NBW], bits[NBW], p0[NBW], p1[NBW];
    float st[NBW];
    bool isv[NBW];
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
        const int cb = w0 + STEP * k;
        isv[k] = cb >= NB;
        const int j = 16 * (isv[k] ? cb - NB : cb) + c;
        jb[k] = j;
        st[k] = isv[k] ? H.estartV[j] : H.estartK[j];
        bits[k] = isv[k] ? H.bitsV[j] : H.bitsK[j];
        const int16_t* cf = isv[k] ? H.cfirstV : H.cfirstK;
        p0[k] = cf[j];
        p1[k] = cf[j + 1];
    }
    bf16x8 xr[2][KS];  // the token's key and value rows (MFMA row 0; the other rows are zero)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 xa = *(const bf16x8*)(xk + 32 * ks + 8 * g);
        const bf16x8 xb = *(const bf16x8*)(xv + 32 * ks + 8 * g);
        xr[0][ks] = c == 0 ? xa : bf16x8{};
        xr[1][ks] = c == 0 ? xb : bf16x8{};
    }
    auto operands = [&](int k, bf16x8 (&bh)[KS], bf16x8 (&bl)[KS], bf16x8 (&bm)[KS]) {
        const uint16_t* uh = isv[k] ? H.EVt_hi : H.EKt_hi;
        const uint16_t* ul = isv[k] ? H.EVt_lo : H.EKt_lo;
        const uint16_t* um = isv[k] ? H.EVt_mid : H.EKt_mid;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bh[ks] = *(const bf16x8*)(uh + jb[k] * D + 32 * ks + 8 * g);
            bl[ks] = *(const bf16x8*)(ul + jb[k] * D + 32 * ks + 8 * g);
            bm[ks] = t3 ? *(const bf16x8*)(um + jb[k] * D + 32 * ks + 8 * g) : bf16x8{};
        }
    };
    auto project = [&](int k, const bf16x8 (&bh)[KS], const bf16x8 (&bl)[KS], const bf16x8 (&bm)[KS]) {
        f4 acc = f4{st[k], st[k], st[k], st[k]};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[isv[k]][ks], bh[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[isv[k]][ks], bl[ks], acc, 0, 0, 0);
            if (t3) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[isv[k]][ks], bm[ks], acc, 0, 0, 0);
        }
        return acc[0];
    };
    float u[NBW];
    {
        bf16x8 bh[HALF][KS], bl[HALF][KS], bm[HALF][KS];
#pragma unroll
        for (int k = 0; k < HALF; ++k) operands(k, bh[k], bl[k], bm[k]);
#pragma unroll
        for (int k = 0; k < HALF; ++k) u[k] = project(k, bh[k], bl[k], bm[k]);
    }
    uint32_t pcs[NBW][kPrePieces];
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
        const uint32_t* pc = isv[k] ? H.cpieceV : H.cpieceK;
#pragma unroll
        for (int e = 0; e < kPrePieces; ++e) pcs[k][e] = p0[k] + e < p1[k] ? pc[p0[k] + e] : 0u;
    }
    if constexpr (NBW > HALF) {
        bf16x8 bh[NBW - HALF][KS], bl[NBW - HALF][KS], bm[NBW - HALF][KS];
#pragma unroll
        for (int k = HALF; k < NBW; ++k) operands(k, bh[k - HALF], bl[k - HALF], bm[k - HALF]);
#pragma unroll
        for (int k = HALF; k < NBW; ++k) u[k] = project(k, bh[k - HALF], bl[k - HALF], bm[k - HALF]);
    }
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
        if (g == 0 && bits[k] > 0) {
            const uint32_t code = code_byte(u[k], (float)((1 << bits[k]) - 1), 0, 0u);
            const uint32_t* pc = isv[k] ? H.cpieceV : H.cpieceK;
            const int base = isv[k] ? H.BK / 8 : 0;  // record byte of the value record's byte 0
            for (int p = p0[k]; p < p1[k]; ++p) {  // piece = byte | pos << 8 | width << 12 | shift << 16
                uint32_t pcv = 0u;
#pragma unroll
                for (int e = 0; e < kPrePieces; ++e)
                    if (p == p0[k] + e) pcv = pcs[k][e];
                if (p >= p0[k] + kPrePieces) pcv = pc[p];
                const int rb = base + (int)(pcv & 0xff), pos = (pcv >> 8) & 7, wd = (pcv >> 12) & 15, sh = (pcv >> 16) & 15;
                const uint32_t v = ((code >> sh) & ((1u << wd) - 1u)) << pos;
                lds_or_async(rec + (rb >> 2), v << (8 * (rb & 3)));
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// The merge done by the last workgroup of a (sequence, kv-head) to finish the split decode
// (one launch for the whole call).  Its arithmetic is merge_kernel's (softmax merge of the W
// partials, value coefficients from the columns, o = obias + U_V (step * A) / L) for the G
// query heads of the kv-head at once.  Every global read is issued in one round: the partial
// maxima, the partial rows (thread (c4, s) holds float4 c4 of partials s, s + S, ...), the
// columns of U_V^T that thread (i, js) multiplies (rows js JR .. js JR + JR - 1 of column i)
// and the channel tables; then reductions in LDS.
// ---------------------------------------------------------------------------------------
constexpr int kFuseMaxW = 64;       // partials per (sequence, kv-head) the last workgroup merges
// ... and their bytes: one CU reads them all, so a large merge (the 128k Llama layer: 32
// partials x 4 heads, 68 KB; the Qwen layer: 64 x 7, 236 KB) is faster as the separate
// merge kernel spread over many CUs, despite its launch (measured: 5.3 vs 5.2 us and 10 vs
// 5 us); small merges (one workgroup per sequence in a batch) are fused
constexpr int kFuseMaxBytes = 32 * 1024;
constexpr int kFuseMaxPairs = 256;  // (sequence, kv-head) pairs per fused call: one counter each
constexpr int kFuseRows = 8;        // partial rows per thread and round
constexpr size_t kCounterBytes = 4 * kFuseMaxPairs;  // the workspace's first bytes: arrival counters

// LDS bytes of merge_last (beside nothing else: the ring is free by then)
__host__ __device__ constexpr int merge_lds_bytes(int G, int PL, int D, int NT) {
    return 4 * kFuseMaxW * 16 + 16 * NT + 4 * G * PL + 4 * G * D + 4 * (D / 8) * G * D;
}
constexpr int kCoherentLoad = 16;  // buffer-load cache policy sc1: coherent across the device's caches

template <int D, int NVB, int NT>
__device__ __forceinline__ void merge_last(const DevHead& H, const float* __restrict__ P, int W, int G, float* __restrict__ out,
                           LDS_AS uint8_t* sm, int tid) {
    constexpr int PL = kPartHead + 16 * NVB;
    constexpr int JR = 8, JS = D / JR;  // row slices of U_V^T in the product (JS x D/4 threads)
    static_assert(NT % D == 0 && JS * (D / 4) <= NT, "merge thread layout");
    const int PW = G * PL;  // floats per partial
    const int C4 = PW / 4, S = NT / C4;
    const int c4 = tid % C4, sl = tid / C4;
    const bool rowt = sl < S;
    LDS_AS float* ew = (LDS_AS float*)sm;                     // [W][G] weights 2^(m - M)
    LDS_AS f4* red = (LDS_AS f4*)(ew + kFuseMaxW * 16);       // [S][C4] slice sums
    LDS_AS float* colv = (LDS_AS float*)(red + NT);           // [G][PL] merged rows
    LDS_AS float* cbar = colv + G * PL;                       // [G][D] step * A / L
    LDS_AS float* red2 = cbar + G * D;                        // [JS][G][D] product slices (16-byte aligned)
    // ---- every global read of the merge.  The partials were written by other workgroups,
    // possibly on other XCDs, with device-coherent stores; they are read with device-coherent
    // loads (cache policy sc1), which need no cache invalidation.
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc((void*)P, (short)0, W * PW * 4, 0x00020000);
    f4 X[kFuseRows];
#pragma unroll
    for (int k = 0; k < kFuseRows; ++k) {
        const int w = sl + S * k;
        X[k] = rowt && w < W ? __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          prs, 4 * (w * PW + 4 * c4), 0, kCoherentLoad))
                             : f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int i = tid % D;                             // channel i (value coefficient, output)
    const int i4 = tid % (D / 4), js = tid / (D / 4);  // product: outputs 4 i4 .. 4 i4 + 3 of row slice js
    f4 U[JR];
    if (js < JS) {
#pragma unroll
        for (int r = 0; r < JR; ++r) U[r] = *(const f4*)&H.UVt[(js * JR + r) * D + 4 * i4];
    }
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    const u16x8 fl = *(const u16x8*)&H.vch[i][0];  // channel i's field columns
    // (both loaded and selected after the first barrier: a branch on bitsV here would wait
    // for every load issued before it)
    const int bv = H.bitsV[i];
    const float sv = H.stepV[i];
    const float ob = H.obias[i], mu = H.muV[i];
    // per head (one wave each) the partial maxima, the largest one and each partial's weight
    const int wv = tid >> 6, ln = tid & 63;
    for (int hh = wv; hh < G; hh += NT / 64) {
        const float m = ln < W ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                               prs, 4 * (ln * PW + hh * PL), 0, kCoherentLoad))
                               : -INFINITY;
        const float M = wave_max(m);
        if (ln < W) ew[ln * G + hh] = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    }
    __syncthreads();
    // ---- merged rows: sum over partials of weight x row
    if (rowt) {
        const int hh = (4 * c4) / PL;
        f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int w0 = 0;; w0 += S * kFuseRows) {
#pragma unroll
            for (int k = 0; k < kFuseRows; ++k) {
                const int w = w0 + sl + S * k;
                if (w < W) acc += ew[w * G + hh] * X[k];
            }
            if (w0 + S * kFuseRows >= W) break;
#pragma unroll
            for (int k = 0; k < kFuseRows; ++k) {  // the next round (partials beyond 8 S)
                const int w = w0 + S * kFuseRows + sl + S * k;
                X[k] = w < W ? *(const f4*)(P + (int64_t)w * PW + 4 * c4) : f4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        red[sl * C4 + c4] = acc;
    }
    __syncthreads();
    for (int k = tid; k < C4; k += NT) {
        f4 v = f4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s2 = 0; s2 < S; ++s2) v += red[s2 * C4 + k];
        ((LDS_AS f4*)colv)[k] = v;
    }
    __syncthreads();
    // ---- value coefficients, dequantisation step and 1 / L (thread: channel i of heads hh)
    for (int k = tid; k < G * D; k += NT) {
        const int hh = k / D;
        const LDS_AS float* cv = colv + hh * PL;
        const float L = cv[1], O = cv[2];
        float A = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t en = fl[e];
            if (en != 0xFFFFu) {
                const float v = cv[kPartHead + (en & 511)] + (((en >> 13) & 1) ? O : 0.0f);
                A = fmaf(__builtin_amdgcn_ldexpf(1.0f, (int)((en >> 9) & 15) - 8), v, A);
            }
        }
        cbar[hh * D + i] = L > 0.0f && bv ? sv * A / L : 0.0f;
    }
    __syncthreads();
    // ---- o = obias + U_V cbar: row slices meet in LDS
    if (js < JS) {
        for (int hh = 0; hh < G; ++hh) {
            f4 y = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < JR; ++r) y += cbar[hh * D + js * JR + r] * U[r];
            *(LDS_AS f4*)&red2[(js * G + hh) * D + 4 * i4] = y;
        }
    }
    __syncthreads();
    for (int k = tid; k < G * D; k += NT) {
        const int hh = k / D;
        float y = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < JS; ++s2) y += red2[(s2 * G + hh) * D + i];
        out[k] = colv[hh * PL + 1] > 0.0f ? ob + y : mu;
    }
}

template <int RB, int NQM, int NVB, int D>
__global__ __launch_bounds__(64 * wg_waves(RB, NQM, NVB))
__attribute__((amdgpu_waves_per_eu(waves_for(RB, NQM, NVB)))) void decode_kernel(
    const DevHead* __restrict__ blob, uint8_t* __restrict__ cache, DecodeArgs a,
    const int32_t* __restrict__ seq_ids, const int64_t* __restrict__ seq_lens, const uint16_t* __restrict__ q,
    float* __restrict__ part, int* __restrict__ ctrs, float* __restrict__ out) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    constexpr int PST = 64;          // bytes per row of the probability operand (64 tokens)
    constexpr int GM = 4 * RB;       // query heads the operands have room for
    constexpr int NW = wg_waves(RB, NQM, NVB);  // waves per workgroup
    constexpr int RBP = epilogue_row_blocks(RB);  // row blocks per epilogue pass
    constexpr int GP = 4 * RBP;                   // query heads per epilogue pass
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    LDS_AS uint8_t* sm = (LDS_AS uint8_t*)smem_generic;
    const int wgi = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, c = lane & 15;
    const int zl = z / a.n_seqs_call, zs = z - zl * a.n_seqs_call;  // layer offset, sequence slot
    const int layer = a.layer + zl;
    const DevHead& H = blob[layer * a.n_kv + h];
    const int G = a.G, TB = a.tile_bytes, BB = a.buf_bytes;
    const int64_t zh = (int64_t)z * a.n_kv + h;
    // every pointer argument in scalar registers at once: the argument loads then form one
    // batch instead of a second round trip inside a branch
    asm volatile("" ::"s"(blob), "s"(cache), "s"(seq_ids), "s"(seq_lens), "s"(q), "s"(part), "s"(ctrs), "s"(out));
    constexpr int NB = D / 16;         // 16-channel blocks of q'
    constexpr int KS = D / 32;         // k-steps over the input dimension
    constexpr int QW = 4;              // q-waves (see the prologue below)
    constexpr int BPW = NB / QW;       // channel blocks per q-wave
    static_assert(NB % QW == 0 && QW >= 3 && QW < NW, "whole blocks per q-wave; the first three copy the tables");
    const bool qwave = w < QW;
    // The q-waves request their matrix rows, query heads, key steps and slot weights first:
    // the addresses come from the arguments alone, so these requests are in flight while the
    // scalar loads below (codebook fields, sequence ids and lengths) make their round trip.
    bf16x8 ah[BPW][KS], al[BPW][KS], bq[KS];
    f4 stv[BPW], fmv[BPW];
    if (qwave) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int j = 16 * (w * BPW + b) + c;  // A row: channel j
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                ah[b][ks] = *(const bf16x8*)(H.QKt_hi + j * D + 32 * ks + 8 * g);
                al[b][ks] = *(const bf16x8*)(H.QKt_lo + j * D + 32 * ks + 8 * g);
            }
            stv[b] = *(const f4*)(H.stepK + 16 * (w * BPW + b) + 4 * g);
            fmv[b] = *(const f4*)(H.kq_fmax + 16 * (w * BPW + b) + 4 * g);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)  // B column: query head c of the group (clamped; zeroed below)
            bq[ks] = *(const bf16x8*)(q + ((int64_t)zh * G + min(c, G - 1)) * D + 32 * ks + 8 * g);
    }

    // The record sizes of the head and this sequence's id and length, as scalar loads issued
    // after the q-waves' requests and waited for on the scalar counter only (those requests
    // stay in flight); the compiler would make them vector loads here, whose wait would also
    // wait for the matrix rows.  They are read before any copy is issued: a vector load after
    // the copies would make the compiler wait for every copy in flight.
    int hBK, hBV, seq;
    int64_t len0;  // tokens cached before this call
    load_head_and_sequence(&H, seq_ids + zs, seq_lens + zs, hBK, hBV, seq, len0);
    const uint32_t vblock = 8u * (uint32_t)hBK;
    const int nkw = hBK / 32, nvr = hBV / 8;  // a token's key record words, value record bytes
    asm volatile("" ::"s"(vblock), "s"(nkw), "s"(nvr));
    // ---- sequence geometry (device arguments clamped: no read outside the cache)
    int64_t len = min(min(len0 + (a.k_new ? 1 : 0), a.max_len), a.n_tiles_cap * kTile);
    if (seq < 0 || seq >= a.n_seqs_cache) len = 0;
    const int n_tiles = (int)((len + kTile - 1) / kTile);  // < 2^31 / 64: the host bounds the range
    uint8_t* tiles = cache + (((int64_t)layer * a.n_seqs_cache + seq) * a.n_kv + h) * a.n_tiles_cap * TB;
    // append mode: the new token's slot, when it lies within the attended range
    const bool app = a.k_new && len0 >= 0 && len0 < len;
    const int64_t t_app = app ? len0 / kTile : -1;
    const int s_app = (int)(len0 & (kTile - 1));
    // buffer resource over this (sequence, kv-head)'s tiles (the host keeps the range below 2^31 bytes)
    const __amdgpu_buffer_rsrc_t trs =
        __builtin_amdgcn_make_buffer_rsrc((void*)tiles, (short)0, (int)(a.n_tiles_cap * TB), 0x00020000);
    // workgroup wgi takes the tiles [t_begin, t_end) of an even split (the first n_tiles mod W
    // workgroups one more; 32-bit arithmetic), and its wave w the tiles t_begin + w + NW k:
    // the waves of a workgroup differ by at most one tile, and the waves with one more are
    // the first ones, which the SIMDs' oldest-first issue favours (measured: 0.5-1 us less
    // than giving the extra tiles to the last waves).  The assignment is static, so every
    // call sums in the same order and gives the same bits (a wave claiming tiles from an LDS
    // counter balanced the waves but not the workgroup's end, which its CU's share of the
    // bandwidth sets).  Ring slot k of this wave: ring + k * RS.
    const int tq = n_tiles / a.wg_per_head, tr = n_tiles - tq * a.wg_per_head;
    const int64_t t_begin = (int64_t)tq * wgi + min(wgi, tr);
    const int64_t t_end = t_begin + tq + (wgi < tr ? 1 : 0);
    const int64_t stride = NW;
    const int NBW = a.nbw;
    const TileLoads tl = a.tl;
    const int nl = tl.n16 + tl.r4 + tl.r2 + tl.r1;  // load instructions per tile
    LDS_AS uint8_t* ring = sm + w * BB;
    const int RS = NW * BB;  // bytes between a wave's ring slots
    int64_t t = t_begin + w;
    const bool owner = t_app >= t_begin && t_app < t_end;  // this workgroup codes the new token
    // ---- prologue.  The first QW waves (the "q-waves") form q' = T_K^{-1} q (T_K the key
    // basis; U_K^T for the KLT), BPW 16-channel blocks each: (1) register loads of their
    // blocks' rows (hi, lo), the query heads, the key steps and slot weights (at the top of
    // the kernel), and direct global->LDS copies of the slot descriptors, the key schedule
    // and the value columns (waves 0..2, one table each); (2) a workgroup barrier, so that these requests precede
    // every tile request of the workgroup and are not queued behind the tile stream;
    // (3) the blocks on bf16 MFMAs, q'' and per head each block's largest slot value into
    // LDS; (4) the score operands (three int8 digits per key field, laid out as MFMA A
    // operands) and per head the lane record (digit scales and the accumulator's start
    // value) - the q-waves meet each other through an LDS counter between these steps.  The
    // other waves (the "stream waves") issue their tile copies right after the barrier and
    // meet the q-waves only at the final barrier: a copy issue stalls while the memory
    // queues are full, and a stalled wave must not hold up the operands.  The q-waves issue
    // their own tiles after the prologue (the compiler cannot count copies of run-time size,
    // so a register load consumed after them would wait for all of them).
    constexpr int QB = operand_bytes(RB, NQM);
    LDS_AS uint8_t* scr = sm + a.off_scratch;                             // [QB] operands and records
    LDS_AS uint32_t* vcol = (LDS_AS uint32_t*)(scr + QB);                 // [NVB][16] value columns
    LDS_AS uint16_t* kslot = (LDS_AS uint16_t*)(scr + QB + NVB * 64);     // [NQM][4][16] slot descriptors
    LDS_AS float* qf = (LDS_AS float*)(scr + QB + NVB * 64 + NQM * 128);  // [GM][D] q''
    LDS_AS float* bmax = qf + GM * D;                                     // [NB][16] block maxima per head
    LDS_AS int* corr = (LDS_AS int*)(bmax + NB * 16);                     // [RB][16] digit sums of bit-7 slots
    LDS_AS uint32_t* rec = (LDS_AS uint32_t*)(sm + a.off_rec);            // [kMaxRecord] appended token's records
    LDS_AS u32x4* ksched = (LDS_AS u32x4*)(sm + a.off_ksched);            // [NQM][4][2]: offsets, masks
    LDS_AS int* qctr = (LDS_AS int*)(sm + a.off_sync);                    // arrivals of the q-waves

    if (w == 0) load_tile((const uint8_t*)&H.vb_col[0][0], (LDS_AS uint8_t*)vcol, NVB * 64, lane, 0);
    if (w == 1) load_tile((const uint8_t*)&H.kq_sched[0][0][0], (LDS_AS uint8_t*)ksched, NQM * 128, lane, 0);
    if (w == 2) load_tile((const uint8_t*)&H.kq_slot[0][0][0], (LDS_AS uint8_t*)kslot, NQM * 128, lane, 0);
    if (tid == 0) qctr[0] = qctr[2] = 0;
    if (owner && tid < kMaxRecord / 4) rec[tid] = 0u;
    lds_barrier();  // the q-waves' requests are issued; the counters and records are zero
    int issued = 0;  // tiles of this wave whose loads have been issued; tile number k uses ring slot k % NBW
    if (!qwave && !owner)
        for (; issued < a.early && t + stride * issued < t_end; ++issued)
            stream_tile(trs, (uint32_t)((t + stride * issued) * TB), ring + issued * RS, tl, lane);
    if (qwave) {
        if (tid < RB * 16) corr[tid] = 0;
        const float qscale = kLog2e / sqrtf((float)D);
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int blk = w * BPW + b;
            f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 bv = c < G ? bq[ks] : bf16x8{};  // heads past G: zero columns
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[b][ks], bv, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[b][ks], bv, acc, 0, 0, 0);
            }
            // lane (g, c): channels 16 blk + 4 g + e of head c
            f4 v;
            float mag = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = acc[e] * stv[b][e] * qscale;  // step_K is 0 for uncoded channels
                mag = fmaxf(mag, fabsf(v[e]) * fmv[b][e]);
            }
            if (c < GM) *(LDS_AS f4*)&qf[c * D + 16 * blk + 4 * g] = v;
            mag = fmaxf(mag, __shfl_xor(mag, 16));
            mag = fmaxf(mag, __shfl_xor(mag, 32));
            if (g == 0) bmax[blk * 16 + c] = mag;
        }
        wait_vm(0);  // the table copies have landed (these waves have no tile in flight yet)
        q_sync(qctr, QW, lane);
        // score operands: item (m, rb, lane group gg, dword iw, head hh4) forms the three digit
        // words of its four slots (rows 4 hh4 + 0..2 of operand [m][rb]; row 4 hh4 + 3 is zero)
        for (int i = tid; i < NQM * RB * 64; i += QW * 64) {
            const int hh4 = i & 3, iw = (i >> 2) & 3, gg = (i >> 4) & 3, rb = (i >> 6) % RB, m = (i >> 6) / RB;
            const int hh = 4 * rb + hh4;
            float mx = 0.0f;
#pragma unroll
            for (int bk = 0; bk < NB; ++bk) mx = fmaxf(mx, bmax[bk * 16 + hh]);
            const float sc = hh < G && mx > 0.0f ? 127.0f / mx : 0.0f;
            typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
            const u16x4 sls = *(const LDS_AS u16x4*)&kslot[(m * 4 + gg) * 16 + 4 * iw];
            uint32_t w0 = 0u, w1 = 0u, w2 = 0u;
            int f0 = 0, f1 = 0, f2 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t sl = sls[e];
                if (sl != 0xFFFFu) {  // slot = chan | shift << 8 | pos << 11 | ends-at-bit-7 << 14
                    const int sh = (int)((sl >> 8) & 7) - (int)((sl >> 11) & 7);
                    float d0, d1, d2;
                    digits254(qf[hh * D + (sl & 255)] * __builtin_amdgcn_ldexpf(sc, sh), d0, d1, d2);
                    w0 |= ((uint32_t)(int)d0 & 0xFFu) << (8 * e);
                    w1 |= ((uint32_t)(int)d1 & 0xFFu) << (8 * e);
                    w2 |= ((uint32_t)(int)d2 & 0xFFu) << (8 * e);
                    if (sl & 0x4000u) f0 += (int)d0, f1 += (int)d1, f2 += (int)d2;
                }
            }
            LDS_AS uint32_t* dst = (LDS_AS uint32_t*)(scr + ((m * RB + rb) * 64 + 16 * gg + 4 * hh4) * 16) + iw;
            dst[0] = w0;
            dst[4] = w1;
            dst[8] = w2;
            dst[12] = 0u;
            if (f0 | f1 | f2) {
                lds_add_async(&corr[rb * 16 + 4 * hh4], f0);
                lds_add_async(&corr[rb * 16 + 4 * hh4 + 1], f1);
                lds_add_async(&corr[rb * 16 + 4 * hh4 + 2], f2);
            }
        }
        q_sync(qctr, 2 * QW, lane);
        if (tid < RB * 4) {  // lane record of (row block, head): digit scales, 128 x bit-7 digit sums
            const int rb = tid >> 2, g4 = tid & 3, hh = 4 * rb + g4;
            float mx = 0.0f;
#pragma unroll
            for (int bk = 0; bk < NB; ++bk) mx = fmaxf(mx, bmax[bk * 16 + hh]);
            mx *= 1.0f / 127.0f;
            const LDS_AS int* cr = &corr[16 * rb + 4 * g4];
            LDS_AS u32x4* lr = (LDS_AS u32x4*)(scr + NQM * RB * 1024 + 32 * tid);
            lr[0] = u32x4{__float_as_uint(mx), __float_as_uint(mx * kQ1), __float_as_uint(mx * kQ2),
                          (uint32_t)(128 * cr[0])};
            lr[1] = u32x4{(uint32_t)(128 * cr[1]), (uint32_t)(128 * cr[2]), 0u, 0u};
        }
        q_sync(qctr, 3 * QW, lane);
    }
    constexpr int NSW = NW - QW;  // stream waves
    if (owner) {
        // (workgroup-uniform) the new token's codes, by the stream waves before they request
        // any tile: their loads then meet nearly empty memory queues (a coding block's two
        // dependent round trips take several microseconds each once every CU's ring is in
        // flight); every wave meets the complete records before its tile loop
        static_assert((2 * NB) % NSW == 0, "whole coding blocks per stream wave");
        if (!qwave) {
            const int64_t row = ((int64_t)z * a.n_kv + h) * D;
            append_blocks<D, 2 * NB / NSW, NSW>(H, a.k_new + row, a.v_new + row, w - QW, rec, g, c);
            q_sync(qctr + 2, NSW, lane);
            for (; issued < a.early && t + stride * issued < t_end; ++issued)
                stream_tile(trs, (uint32_t)((t + stride * issued) * TB), ring + issued * RS, tl, lane);
        } else {
            q_wait(qctr + 2, NSW);
        }
    }
    if (!qwave) q_wait(qctr, 3 * QW);  // the operands, records, tables and the appended token's records are in LDS
    uint32_t voff[NVB], vmask[NVB];  // value columns of this lane: tile offset of its plane slice, mask
#pragma unroll
    for (int cb = 0; cb < NVB; ++cb) {
        const uint32_t v = vcol[cb * 16 + c];
        voff[cb] = vblock + (v & 0xFFFFu) + 16u * (uint32_t)g;
        vmask[cb] = 0x01010101u * (v >> 16);
    }
    v4i Aq[NQM][RB];  // score A operands (query digits), resident for the whole loop
#pragma unroll
    for (int m = 0; m < NQM; ++m)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) Aq[m][rb] = ((const LDS_AS v4i*)scr)[(m * RB + rb) * 64 + lane];
    // key schedule of this lane group: tile offsets of the four record words of tokens
    // 4c..4c+3 (registers), or read per tile from LDS
    constexpr bool KREG = ksched_in_regs(NQM);
    constexpr int KR = KREG ? NQM : 1;
    u32x4 koffr[KR], kmaskr[KR];
    if constexpr (KREG) {
#pragma unroll
        for (int m = 0; m < NQM; ++m) {
            koffr[m] = ksched[(m * 4 + g) * 2] + (uint32_t)(16 * c);
            kmaskr[m] = ksched[(m * 4 + g) * 2 + 1];
        }
    }
    float qs[RB][3];  // digit scales of this lane's query head
    v4i sinit[RB];    // score accumulator start: 128 x the digits multiplying bit-7 fields
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const LDS_AS u32x4* lr = (const LDS_AS u32x4*)(scr + NQM * RB * 1024 + 32 * (4 * rb + g));
        const u32x4 r0 = lr[0], r1 = lr[1];
        // (through scalars: a bit cast of a vector element reads element 0 with this compiler)
        const uint32_t q0 = r0[0], q1 = r0[1], q2 = r0[2];
        qs[rb][0] = __uint_as_float(q0);
        qs[rb][1] = __uint_as_float(q1);
        qs[rb][2] = __uint_as_float(q2);
        sinit[rb] = v4i{(int)r0[3], (int)r1[0], (int)r1[1], 0};
    }
    // the operands are in registers and every prologue read has completed: inside the loop
    // the only vector memory operations are this wave's tile loads
#pragma unroll
    for (int m = 0; m < NQM; ++m)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) asm volatile("" ::"v"(Aq[m][rb]));
#pragma unroll
    for (int cb = 0; cb < NVB; ++cb) asm volatile("" ::"v"(voff[cb]), "v"(vmask[cb]));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) asm volatile("" ::"v"(qs[rb][0]), "v"(qs[rb][1]), "v"(qs[rb][2]), "v"(sinit[rb]));
    if constexpr (KREG) {
#pragma unroll
        for (int m = 0; m < NQM; ++m) asm volatile("" ::"v"(koffr[m]), "v"(kmaskr[m]));
    }
    for (; issued < a.early && t + stride * issued < t_end; ++issued)  // the q-waves' first slots
        stream_tile(trs, (uint32_t)((t + stride * issued) * TB), ring + issued * RS, tl, lane);
    if (a.early < NBW) {  // the scratch was in the ring's last slots: stream them now
        lds_barrier();
        for (; issued < NBW && t + stride * issued < t_end; ++issued)
            stream_tile(trs, (uint32_t)((t + stride * issued) * TB), ring + issued * RS, tl, lane);
    }

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

    // ---- this wave's tiles: the ring keeps up to NBW - 1 of them in flight; the wave
    // waits on its own load count
    int slot = 0;
    for (int done = 0; t < t_end; t += stride, ++done) {
        // tile t (this wave's tile number done) has landed once only the later tiles' loads
        // are outstanding
        wait_vm(nl * (issued - done - 1));
        LDS_AS uint8_t* curb = ring + slot * RS;
        if (owner && t == t_app) {  // the appended token's slot, whatever the copy read for it
            for (int r = lane; r < nkw; r += 64) ((LDS_AS uint32_t*)curb)[64 * r + s_app] = rec[r] ^ 0x80808080u;
            for (int q = lane; q < nvr; q += 64)
                curb[vblock + 64 * q + s_app] = (uint8_t)(((const LDS_AS uint8_t*)rec)[4 * nkw + q] ^ 0x80u);
            asm volatile("" ::: "memory");
        }
        const int valid = (int)min((int64_t)kTile, len - t * kTile);

        // ---------------- scores: token group tg, lane (g, c) -> token 4c + tg.  One 16-byte
        // read gives a record word of the lane's four tokens; each operand dword keeps one
        // field per byte (a mask), so no shifts.
        v4i S[4][RB];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) S[tg][rb] = sinit[rb];
#pragma unroll
        for (int m = 0; m < NQM; ++m) {
            const LDS_AS uint8_t* kbase = KREG ? curb : curb + 16 * c;  // record word 0 of tokens 4c..4c+3
            u32x4 koff, kmask;
            if constexpr (KREG) {
                koff = koffr[m];
                kmask = kmaskr[m];
            } else {
                koff = ksched[(m * 4 + g) * 2];
                kmask = ksched[(m * 4 + g) * 2 + 1];
            }
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
        float s[RB][4], lmx[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tg = 0; tg < 4; ++tg)
                s[rb][tg] = (float)S[tg][rb][0] * qs[rb][0] + (float)S[tg][rb][1] * qs[rb][1] +
                            (float)S[tg][rb][2] * qs[rb][2];
        if (valid < kTile) {  // the sequence's last tile: slots past its end score -inf
            asm volatile("");  // (a real branch: only one tile per sequence takes it)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int tg = 0; tg < 4; ++tg) s[rb][tg] = 4 * c + tg < valid ? s[rb][tg] : -INFINITY;
        }
        bool need = false;  // some score of this lane passed its head's reference max
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            lmx[rb] = fmaxf(fmaxf(s[rb][0], s[rb][1]), fmaxf(s[rb][2], s[rb][3]));
            need = need || lmx[rb] > mref[rb];
        }
        if (done == 0) {
            // the wave's first tile (it has a valid slot): the references start at its maxima,
            // the sums are still zero
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) mref[rb] = row16_max(lmx[rb]) + kHeadroom;
        } else if (__any(need)) {
            asm volatile("");  // (a real branch: rescales are rare)
            // raise the reference of heads whose tile max passed it and rescale their sums
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float tmx = row16_max(lmx[rb]);
                const float nref = tmx > mref[rb] ? tmx + kHeadroom : mref[rb];
                const float al = __builtin_amdgcn_exp2f(mref[rb] - nref);
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
        // (wave-private; the key words of this tile were all read above), or in a buffer of
        // the wave's own when the key block is smaller than the operand.
        LDS_AS uint8_t* P = a.off_pbuf < 0 ? curb : sm + a.off_pbuf + w * (RB * 1024);
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
        u32x4 xv[NVB];
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb) xv[cb] = *(const LDS_AS u32x4*)(curb + voff[cb]);
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb) {
            const u32x4 x = xv[cb];
            const v4i B = v4i{(int)(x[0] & vmask[cb]), (int)(x[1] & vmask[cb]), (int)(x[2] & vmask[cb]),
                              (int)(x[3] & vmask[cb])};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc_i[rb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ap[rb], B, acc_i[rb][cb], 0, 0, 0);
        }
        // the slot streams the tile NBW ahead once this wave's reads of it are done
        const int64_t tn = t + stride * NBW;
        if (tn < t_end) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stream_tile(trs, (uint32_t)(tn * TB), curb, tl, lane);
            ++issued;
        }
        slot = slot + 1 == NBW ? 0 : slot + 1;
    }

    // ---------------- epilogue: the waves' results meet in LDS (ring reused), laid out
    // like the partial: per wave and head [reference max, sum, 128 x probability digit sum
    // / 127, 0, columns: accumulator / 127 = sum of p x stored byte].  Per head the
    // workgroup's reference is the largest of the waves', each wave weighted by 2^(m - M).
    constexpr int PL = kPartHead + 16 * NVB;  // floats per partial and head
    wait_all();
    if (owner && w == NW - 1) {  // the new token's records into the cache (stored bytes: bit 7 inverted)
        uint8_t* tp = tiles + t_app * TB;
        for (int r = lane; r < nkw; r += 64) ((uint32_t*)tp)[64 * r + s_app] = rec[r] ^ 0x80808080u;
        for (int q = lane; q < nvr; q += 64)
            tp[vblock + 64 * q + s_app] = (uint8_t)(((const LDS_AS uint8_t*)rec)[4 * nkw + q] ^ 0x80u);
    }
    // (in passes of at most two row blocks - 8 query heads - to bound the LDS it takes)
    float* pout = part + (zh * a.wg_per_head + wgi) * G * PL;
    LDS_AS float* wx = (LDS_AS float*)sm;   // [NW waves][GP][PL]
#pragma unroll
    for (int r0 = 0; r0 < RB; r0 += RBP) {
        lds_barrier();  // (the previous pass's reads are done)
#pragma unroll
        for (int rb = r0; rb < r0 + RBP && rb < RB; ++rb) {
            LDS_AS float* o = wx + (w * GP + 4 * (rb - r0) + g) * PL;
            const float ls = row16_sum(lsum[rb]);
            const float os = row16_sum(combine256(ones[rb][0], ones[rb][1], ones[rb][2]));
            if (c == 0) {
                o[0] = mref[rb];
                o[1] = ls;
                o[2] = os * (128.0f / 127.0f);
                o[3] = 0.0f;
            }
#pragma unroll
            for (int cb = 0; cb < NVB; ++cb)
                o[kPartHead + 16 * cb + c] = combine256(acc_i[rb][cb][0], acc_i[rb][cb][1], acc_i[rb][cb][2]) * (1.0f / 127.0f);
        }
        lds_barrier();
        // every entry of the workgroup's partial: each thread forms its head's reference (the
        // waves' largest maximum) and the waves' weights itself (no serial pass, no barrier)
        const int h0 = 4 * r0, nh = min(GP, G - h0);  // this pass's query heads
        for (int i = tid; i < nh * PL; i += NW * 64) {
            const int hl = i / PL, col = i - hl * PL;
            float mw[NW], M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                mw[ww] = wx[(ww * GP + hl) * PL];
                M = fmaxf(M, mw[ww]);
            }
            float v = M;
            if (col > 0) {
                v = 0.0f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww)
                    v = fmaf(mw[ww] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[ww] - M),
                             wx[(ww * GP + hl) * PL + col], v);
            }
            if (a.fused)  // read by the last workgroup, possibly on another XCD
                __hip_atomic_store(pout + h0 * PL + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                pout[h0 * PL + i] = v;
        }
    }
    if (a.fused) {
        // publish this workgroup's partial and count it; the last of the W workgroups of this
        // (sequence, kv-head) merges them and writes the output, then resets the counter
        LDS_AS int* lastf = qctr + 1;
        // every thread's coherent partial stores have completed before the count
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(ctrs + zh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int last = old == a.wg_per_head - 1;
            if (last) __hip_atomic_store(ctrs + zh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *lastf = last;
        }
        __syncthreads();
        if (*lastf) {
            merge_last<D, NVB, NW * 64>(H, part + zh * a.wg_per_head * G * PL, a.wg_per_head, G, out + zh * G * D,
                                        sm, tid);
        }
    }
}

// ---------------------------------------------------------------------------------------
// merge: one workgroup of 256 threads per (sequence, kv-head, query head, slice of 32 output
// channels).  Softmax merge of the W partials (a partial row is [reference max m, sum of p,
// top-field sum, 0, columns]; column c = sum of p x stored byte of value field c, relative
// to m), then per channel j
//   A_j = sum over its fields of 2^(shift - pos) (column + [field ends at bit 7] top sum)
// (the stored byte of a field at bit pos is field 2^pos, minus 128 at the top of a byte)
// and the slice of o = obias + U_V (step * A / L).  The reads - the partial maxima, the
// partial rows (thread (q, s) holds float4 q of rows s, s + NS, ...), the slice's columns
// of U_V^T (thread (i4, js) holds float4 i4 of rows js JR .. js JR + JR - 1) and the
// channel tables - are issued together at the start, 16 bytes per lane where they can be.
// ---------------------------------------------------------------------------------------
static_assert(offsetof(DevHead, vch) % 16 == 0, "the merge loads a channel's field table as 16 bytes");
static_assert(offsetof(DevHead, UVt) % 16 == 0, "the merge loads U_V^T 16 bytes per lane");
static_assert(offsetof(DevHead, kq_slot) % 16 == 0 && offsetof(DevHead, kq_sched) % 16 == 0 &&
                  offsetof(DevHead, vb_col) % 16 == 0,
              "the decode prologue copies these tables 16 bytes per lane");
constexpr int kMergeSlice = 32;  // output channels per merge workgroup
constexpr int kMergeRows = 12;   // partial rows per thread and round (84 partials in one round)
constexpr int kMaxWG = 256;      // workgroups per (sequence, kv-head) at most (one per CU)
constexpr int kMaxPL = kPartHead + 16 * aatc::kMaxVB;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const DevHead* __restrict__ blob, int layer, int n_kv,
                                                              int G, int W, int PL, const float* __restrict__ part,
                                                              float* __restrict__ out, int n_seqs_call) {
    constexpr int NT = kMergeThreads, NWV = NT / 64;
    constexpr int NSL = D / kMergeSlice;  // slices
    constexpr int I4 = kMergeSlice / 4;   // float4 columns of the slice
    constexpr int JS = NT / I4;           // row slices of U_V^T
    constexpr int JR = D / JS;            // rows per row slice
    static_assert(D <= NT && JR * JS == D, "merge thread layout");
    __shared__ float pm[kMaxWG];                              // partial maxima
    __shared__ float wred[NWV];
    __shared__ f4 red[NT];                                    // slice sums
    __shared__ __attribute__((aligned(16))) float colv[kMaxPL];  // merged row
    __shared__ float cbar[D];                                 // step * A / L
    const int h = blockIdx.x / NSL, sl = blockIdx.x - h * NSL, z = blockIdx.y, hh = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t zh = (int64_t)z * n_kv + h;
    const DevHead& H = blob[(layer + z / n_seqs_call) * n_kv + h];  // (z: layer offset and sequence slot)
    const int64_t PS = (int64_t)G * PL;              // floats between partials
    const float* P = part + (zh * W * G + hh) * PL;  // partial w at P + w * PS
    const int PL4 = PL >> 2, NS = NT / PL4;
    const int q = tid % PL4, s = tid / PL4;
    // ---- every global read of the first round
    for (int w = tid; w < W; w += NT) pm[w] = P[w * PS];
    f4 X[kMergeRows];
#pragma unroll
    for (int k = 0; k < kMergeRows; ++k) {
        const int w = s + NS * k;
        X[k] = s < NS && w < W ? *(const f4*)(P + w * PS + 4 * q) : f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int i4 = tid % I4, js = tid / I4;
    f4 U[JR];
#pragma unroll
    for (int r = 0; r < JR; ++r) U[r] = *(const f4*)(H.UVt + (js * JR + r) * D + kMergeSlice * sl + 4 * i4);
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    const int jc = tid % D;  // channel tid (tid < D): its field columns
    const u16x8 fl = *(const u16x8*)&H.vch[jc][0];
    const float stv = H.bitsV[jc] ? H.stepV[jc] : 0.0f;
    const int io = kMergeSlice * sl + (tid & (kMergeSlice - 1));  // output channel (tid < kMergeSlice)
    const float ob = H.obias[io], mu = H.muV[io];
    __syncthreads();
    // ---- reference: the largest partial maximum
    float mx = -INFINITY;
    for (int w = tid; w < W; w += NT) mx = fmaxf(mx, pm[w]);
    mx = wave_max(mx);
    if (lane == 0) wred[wv] = mx;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NWV; ++k) M = fmaxf(M, wred[k]);
    // ---- merged row: sum over partials of 2^(m - M) x row, kMergeRows rows per thread a round
    f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int w0 = 0;; w0 += NS * kMergeRows) {
#pragma unroll
        for (int k = 0; k < kMergeRows; ++k) {
            const int w = w0 + s + NS * k;
            if (s < NS && w < W) {
                const float m = pm[w];
                const float e = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
                acc += e * X[k];
            }
        }
        if (w0 + NS * kMergeRows >= W) break;
#pragma unroll
        for (int k = 0; k < kMergeRows; ++k) {  // the next round (partials beyond 8 NS)
            const int w = w0 + NS * kMergeRows + s + NS * k;
            X[k] = s < NS && w < W ? *(const f4*)(P + w * PS + 4 * q) : f4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    red[tid] = acc;
    __syncthreads();
    if (tid < PL4) {
        f4 v = f4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s2 = 0; s2 < NS; ++s2) v += red[s2 * PL4 + tid];
        *(f4*)&colv[4 * tid] = v;
    }
    __syncthreads();
    const float L = colv[1], O = colv[2];
    // ---- value coefficients, dequantisation step and 1 / L (every channel)
    if (tid < D) {
        float A = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t en = fl[k];
            if (en != 0xFFFFu) {
                const float v = colv[kPartHead + (en & 511)] + (((en >> 13) & 1) ? O : 0.0f);
                A = fmaf(__builtin_amdgcn_ldexpf(1.0f, (int)((en >> 9) & 15) - 8), v, A);
            }
        }
        cbar[tid] = L > 0.0f ? stv * A / L : 0.0f;
    }
    __syncthreads();
    // ---- this slice of o = obias + U_V cbar: row slices meet in LDS
    f4 y = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < JR; ++r) y += cbar[js * JR + r] * U[r];
    red[tid] = y;
    __syncthreads();
    if (tid < kMergeSlice) {
        float o = 0.0f;
        for (int s2 = 0; s2 < JS; ++s2) o += red[s2 * I4 + (tid >> 2)][tid & 3];
        out[(zh * G + hh) * D + io] = L > 0.0f ? ob + o : mu;
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
                                 {1, 8, 24}, {1, 16, 24}, {2, 2, 8},  {2, 3, 8},  {2, 3, 10}, {2, 4, 12}, {2, 8, 24},
                                 {2, 16, 24}, {3, 4, 12}, {3, 16, 24}, {4, 4, 12}, {4, 16, 24}};

// ------------------------------------------------------------------------------------
// Split decode over vector-quantized keys ("Spend Bits Where Queries Look", abstract).
// Grid (workgroups per head x chunks of 4 query heads, kv-heads, sequences), one workgroup
// of kVqWaves waves per CU.  Prologue: q'' = (T_K^{-1} q) / s * log2(e) / sqrt(d) for the
// chunk's heads, then one score table per (head, group) in LDS: lut[m][g][i] =
// sum_k q''[chan(g, k)] z_gik over the group's 256 codewords, so that a token's score is
// the sum over groups of lut[m][g][index_g] (the dropped term q . mu_K is the same for every
// token).  Every wave owns whole tiles of the workgroup's share (t_begin + w, + kVqWaves,
// ...), read straight into registers (buffer loads over the (sequence, kv-head)'s range; the
// next tile's loads are in flight while one is computed): lane = token, its key record
// words, and per value block the 16 bytes (tokens 16 kk .. 16 kk + 15 of one field's byte
// plane) that its MFMA B operand needs.  Per tile a wave scores the chunk's heads (one table
// read per (head, group)), keeps per head the running max and sum (base 2) of p rounded to
// fp16, writes p to its own LDS rows, and accumulates the value columns on
// v_mfma_f32_16x16x16_f16: A = p of the heads over 16 tokens, B = the field's masked byte,
// as the fp16 number 1024 + byte (its bits 0x64 | byte, one v_perm per two values; a top
// field's byte with bit 7 restored).  The waves' results are combined in LDS into one
// partial per head in the split-decode layout [max, sum, 128 sum, 0, columns], the column
// of a field being sum p * (its stored bits as a signed byte): the offsets 1024 (and 128
// for top fields) times the sum are taken off.  merge_kernel finishes the call.
// ------------------------------------------------------------------------------------
constexpr int kVqWaves = 8;  // waves per workgroup (one workgroup per CU)
// value blocks per launch (all read ahead into registers): d / 16, the blocks of a record
// with one field per channel; a record with more takes one launch per d / 16 blocks
constexpr int vq_blocks(int d) { return d / 16; }

struct VqLds {
    int lut, pbuf, epi, total;
};

// LDS: the score tables [4][n_g][256] float, then per wave p [4][64] fp16 (the prologue's
// q'' [4][d] float in the same place); the epilogue reuses the start: per wave and head the
// max and sum, then the columns [kVqWaves][4][16 nvb] float
__host__ __device__ inline VqLds vq_lds(int n_g, int d, int nvb) {
    VqLds L;
    L.lut = 0;
    L.pbuf = 4 * n_g * kVqSize * 4;
    const int pb = kVqWaves * 4 * 64 * 2, qv = 4 * d * 4;
    L.epi = 2 * kVqWaves * 4 * 4;
    const int epi_end = L.epi + kVqWaves * 4 * 16 * nvb * 4;
    L.total = L.pbuf + (pb > qv ? pb : qv);
    if (epi_end > L.total) L.total = epi_end;
    return L;
}

// NG: the number of groups when fixed at compile time, 0 for any multiple of 4 at run time.
// vb0: the first value block of this launch (its columns and the maxima and sums go to the
// partials; launches for later blocks of the same call write the same maxima and sums).
template <int D, int NG>
__global__ __launch_bounds__(64 * kVqWaves) void vq_decode_kernel(const DevHead* __restrict__ blob,
                                                                  const uint8_t* __restrict__ cache, DecodeArgs a,
                                                                  const int32_t* __restrict__ seq_ids,
                                                                  const int64_t* __restrict__ seq_lens,
                                                                  const uint16_t* __restrict__ q,
                                                                  float* __restrict__ part, int vb0) {
    constexpr int NGW = (NG ? NG : aatc::kMaxVqGroups) / 4;  // key record words per token (at most)
    constexpr int NVB = vq_blocks(D);
    constexpr int NT = 64 * kVqWaves;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    extern __shared__ __attribute__((aligned(16))) uint8_t vsm_generic[];
    LDS_AS uint8_t* const sm = (LDS_AS uint8_t*)vsm_generic;
    const int n_chunks = (a.G + 3) / 4;
    const int wgi = blockIdx.x / n_chunks, chunk = blockIdx.x - wgi * n_chunks;
    const int h = blockIdx.y, z = blockIdx.z;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, kk = lane >> 4;
    const DevHead& H = blob[a.layer * a.n_kv + h];
    const int n_g = NG ? NG : H.vq_groups, nvb = max(0, min(NVB, H.nvb - vb0)), BK = H.BK;
    const int hh0 = 4 * chunk, GC = min(4, a.G - hh0);
    const int tbytes = a.tile_bytes;
    const VqLds L = vq_lds(n_g, D, nvb);
    LDS_AS float* const lut = (LDS_AS float*)(sm + L.lut);
    LDS_AS float* const qv = (LDS_AS float*)(sm + L.pbuf);
    LDS_AS _Float16* const pw = (LDS_AS _Float16*)(sm + L.pbuf) + w * 256;  // this wave's p [4][64]
    // sequence geometry (device arguments clamped: no read outside the cache)
    const int seq = seq_ids[z];
    int64_t len = max<int64_t>(0, min<int64_t>(min<int64_t>(seq_lens[z], a.max_len), a.n_tiles_cap * kTile));
    if (seq < 0 || seq >= a.n_seqs_cache) len = 0;
    const int64_t n_tiles = (len + kTile - 1) / kTile;
    const int64_t t_begin = n_tiles * wgi / a.wg_per_head, t_end = n_tiles * (wgi + 1) / a.wg_per_head;
    const uint8_t* const base =
        cache + (((int64_t)a.layer * a.n_seqs_cache + max(seq, 0)) * a.n_kv + h) * a.n_tiles_cap * (int64_t)tbytes;
    // buffer resource over this (sequence, kv-head)'s tiles (the host keeps the range below
    // 2^31 bytes); the offsets are per lane, so a read past the range returns zeros
    const __amdgpu_buffer_rsrc_t trs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(a.n_tiles_cap * tbytes), 0x00020000);
    // this lane's value operand bytes of block vb0 + r: tile offset, byte mask, top-field flag
    uint32_t voff[NVB], vmsk[NVB], vflp[NVB];
#pragma unroll
    for (int r = 0; r < NVB; ++r) {
        const uint32_t vc = r < nvb ? H.vb_col[vb0 + r][col] : 0u;
        const uint32_t m8 = (vc >> 16) & 0xFFu;
        voff[r] = 8 * BK + (vc & 0xFFFFu) + 16 * kk;
        vmsk[r] = m8 * 0x01010101u;
        vflp[r] = (m8 & 0x80u) ? 0x80808080u : 0u;
    }
    struct Tile {
        uint32_t kw[NGW];
        u32x4 vv[NVB];
    };
    // a tile's registers; every tile issues the same loads, and those of a tile past the
    // workgroup's share take an offset past the range (zeros, no memory traffic)
    auto load = [&](int64_t t, Tile& T) {
        const uint32_t tb = t < t_end ? (uint32_t)(t * tbytes) : 0x80000000u;
#pragma unroll
        for (int r = 0; r < NGW; ++r)
            if (NG || 4 * r < n_g)
                T.kw[r] = __builtin_amdgcn_raw_buffer_load_b32(trs, tb + 4 * (64 * r + lane), 0, 2);
#pragma unroll
        for (int r = 0; r < NVB; ++r)  // blocks past the record's read too (their offsets stay in the tile)
            T.vv[r] = __builtin_amdgcn_raw_buffer_load_b128(trs, tb + voff[r], 0, 2);
    };
    // ---- prologue: q' = T_K^{-1} q of the chunk's heads on bf16 MFMAs (wave w < D / 16: rows
    // 16 w .. 16 w + 15 of T_K^{-1} = hi + lo as A, the heads' q as the B columns), then
    // q'' = q' / s * log2(e) / sqrt(d) into LDS
    if (w < D / 16) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        const int j0 = 16 * w;
        const uint16_t* qr = q + (((int64_t)z * a.n_kv + h) * a.G + hh0 + min(col, GC - 1)) * D;
        f4 qa = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 ah = *(const bf16x8*)&H.QKt_hi[(j0 + col) * D + 32 * ks + 8 * kk];
            const bf16x8 al = *(const bf16x8*)&H.QKt_lo[(j0 + col) * D + 32 * ks + 8 * kk];
            const bf16x8 bq = col < GC ? *(const bf16x8*)&qr[32 * ks + 8 * kk] : bf16x8{};
            qa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bq, qa, 0, 0, 0);
            qa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bq, qa, 0, 0, 0);
        }
        if (col < 4) {  // lane (kk, head col): rows j0 + 4 kk + e
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 4 * kk + e;
                qv[col * D + j] = col < GC ? qa[e] * (H.vq_rscale[j] * (kLog2e / sqrtf((float)D))) : 0.0f;
            }
        }
    }
    lds_barrier();
    // tables, the four heads' entries of one (group, codeword) side by side (one 16-byte read
    // per group and token in the tile loop; entries of absent heads are zero).  Codeword
    // i = tid mod 256 of groups tid / 256, + NT / 256, ...: every load first
    LDS_AS f4* const lut4 = (LDS_AS f4*)lut;
    constexpr int GPT = (NG ? NG : aatc::kMaxVqGroups) / (NT / 256);  // groups per thread (at most)
    constexpr int GB = GPT > 8 ? GPT / 2 : GPT;                             // ... per batch of loads
    {
        const int i = tid & 255, g0 = tid >> 8;
        Tile T0;
#pragma unroll
        for (int u0 = 0; u0 < GPT; u0 += GB) {
            float4 zc[GB];
            uint32_t chw[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const int g = g0 + (u0 + u) * (NT / 256);
                if (NG || g < n_g) {
                    zc[u] = *(const float4*)H.vq_cent[g][i];
                    chw[u] = *(const uint32_t*)H.vq_chan[g];
                }
            }
            // the first tile's loads follow the first batch: in flight while the tables are built
            if (u0 == 0 && t_begin + w < t_end) load(t_begin + w, T0);
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const int g = g0 + (u0 + u) * (NT / 256);
                if (NG || g < n_g) {
                    const int c0 = chw[u] & 255, c1 = (chw[u] >> 8) & 255, c2 = (chw[u] >> 16) & 255,
                              c3 = chw[u] >> 24;
                    f4 e4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const LDS_AS float* qm = qv + m * D;
                        e4[m] = fmaf(qm[c3], zc[u].w, fmaf(qm[c2], zc[u].z, fmaf(qm[c1], zc[u].y, qm[c0] * zc[u].x)));
                    }
                    lut4[g * kVqSize + i] = e4;
                }
            }
        }
        lds_barrier();  // tables complete, q'' no longer read (the p rows take its place)
        // ---- this wave's tiles
        f4 acc[NVB];
#pragma unroll
        for (int r = 0; r < NVB; ++r) acc[r] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        // per head: the reference max (uniform; raised only when a score exceeds it) and this
        // lane's sum of p
        float m_run[4], l_lane[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            m_run[m] = -INFINITY;
            l_lane[m] = 0.0f;
            if (m >= GC) pw[m * 64 + lane] = (_Float16)0.0f;  // rows of absent heads stay zero
        }
        auto process = [&](const Tile& T, int64_t t) {
            const bool valid = t * kTile + lane < len;
            // scores of the chunk's heads
            float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            // the table base as a value the sums so far feed (a move in asm): reads of at most
            // two record words (8 groups) are in flight before their sums are formed, where
            // the compiler would otherwise hold all of them in registers
            uint32_t lb = (uint32_t)(uintptr_t)lut4;
#pragma unroll
            for (int r = 0; r < NGW; ++r) {
                if (!NG && 4 * r >= n_g) break;
                const uint32_t wd = T.kw[r] ^ 0x80808080u;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t ad = lb + 16u * ((4 * r + b) * kVqSize + ((wd >> (8 * b)) & 255u));
                    const f4 e4 = *(const LDS_AS f4*)(uintptr_t)ad;
#pragma unroll
                    for (int m = 0; m < 4; ++m) s[m] += e4[m];
                }
                if (r & 1)
                    asm volatile("v_mov_b32 %0, %1" : "=v"(lb) : "v"(lb), "v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]));
            }
            // online softmax per head (base 2): the reference max rises only when a score of
            // the tile exceeds it, rescaling the sums and the accumulators; p (fp16) into this
            // wave's rows
            f4 al4 = f4{1.0f, 1.0f, 1.0f, 1.0f};
            bool rescale = false;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m < GC) {
                    const float sv = valid ? s[m] : -INFINITY;
                    if (__builtin_amdgcn_ballot_w64(sv > m_run[m])) {
                        const float mn = wave_max(sv);
                        const float al = __builtin_amdgcn_exp2f(m_run[m] - mn);  // 0 while nothing is summed
                        l_lane[m] *= al;
                        al4[m] = al;
                        rescale = true;
                        m_run[m] = mn;
                    }
                    const float p = valid ? (float)(_Float16)__builtin_amdgcn_exp2f(sv - m_run[m]) : 0.0f;
                    l_lane[m] += p;
                    pw[m * 64 + lane] = (_Float16)p;
                }
            }
            // A operands: row = head (rows 4.. zero), k-slot e of MFMA i = token 16 kk + 4 i + e
            h4 A[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                A[i] = col < GC ? *(const LDS_AS h4*)&pw[col * 64 + 16 * kk + 4 * i] : h4{};
#pragma unroll
            for (int r = 0; r < NVB; ++r) {
                if (r >= nvb) break;
                if (rescale) acc[r] *= al4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t y = (T.vv[r][i] & vmsk[r]) ^ vflp[r];
                    // fp16 1024 + byte: high byte 0x64 over each data byte
                    const uint32_t lo2 = __builtin_amdgcn_perm(0x64646464u, y, 0x07010600u);
                    const uint32_t hi2 = __builtin_amdgcn_perm(0x64646464u, y, 0x07030602u);
                    const h4 B = __builtin_bit_cast(h4, (uint64_t)lo2 | ((uint64_t)hi2 << 32));
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x16f16(A[i], B, acc[r], 0, 0, 0);
                }
            }
        };
        // two register sets: the next tile's loads in flight while one is computed
        Tile T1;
        for (int64_t t = t_begin + w; t < t_end; t += 2 * kVqWaves) {
            load(t + kVqWaves, T1);
            process(T0, t);
            if (t + kVqWaves >= t_end) break;
            load(t + 2 * kVqWaves, T0);
            process(T1, t + kVqWaves);
        }
        float l_run[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) l_run[m] = m < GC ? wave_sum(l_lane[m]) : 0.0f;
        // ---- combine the waves: maxima and sums, then the columns
        lds_barrier();  // every wave is past its tiles (the tables are free)
        LDS_AS float* const em = (LDS_AS float*)(sm + L.epi) - 2 * kVqWaves * 4;  // [2][kVqWaves][4]
        LDS_AS float* const ec = (LDS_AS float*)(sm + L.epi);                      // [kVqWaves][4][16 nvb]
        if (lane < 4) {
            em[w * 4 + lane] = lane < GC ? m_run[lane] : -INFINITY;
            em[(kVqWaves + w) * 4 + lane] = lane < GC ? l_run[lane] : 0.0f;
        }
        if (kk == 0) {
#pragma unroll
            for (int r = 0; r < NVB; ++r) {
                if (r >= nvb) break;
                const float off = vflp[r] ? 1152.0f : 1024.0f;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (m < GC) ec[(w * 4 + m) * 16 * nvb + 16 * r + col] = acc[r][m] - off * l_run[m];
            }
        }
    }
    lds_barrier();
    LDS_AS float* const em = (LDS_AS float*)(sm + L.epi) - 2 * kVqWaves * 4;
    LDS_AS float* const ec = (LDS_AS float*)(sm + L.epi);
    const int64_t zh = (int64_t)z * a.n_kv + h;
    float* const P = part + ((zh * a.wg_per_head + wgi) * a.G + hh0) * a.part_ld;
    for (int i = tid; i < GC * (16 * nvb + 1); i += NT) {
        const int m = i / (16 * nvb + 1), c = i - m * (16 * nvb + 1);
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kVqWaves; ++v) M = fmaxf(M, em[v * 4 + m]);
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < kVqWaves; ++v) {
            const float mv = em[v * 4 + m];
            const float wt = mv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
            sum += wt * (c == 16 * nvb ? em[(kVqWaves + v) * 4 + m] : ec[(v * 4 + m) * 16 * nvb + c]);
        }
        if (c == 16 * nvb) {
            P[m * a.part_ld + 0] = M;
            P[m * a.part_ld + 1] = sum;
            P[m * a.part_ld + 2] = 128.0f * sum;
            P[m * a.part_ld + 3] = 0.0f;
        } else {
            P[m * a.part_ld + kPartHead + 16 * vb0 + c] = sum;
        }
    }
}

struct Plan {
    Variant v;
    int nqm_max, nvb_max, wg_per_head, wgs_per_cu, nw;
    size_t part_bytes;
    DecodeArgs args;
    size_t lds;
    bool vq = false;  // vector-quantized keys: vq_decode_kernel
};

size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// n_seqs: the launch's (layer, sequence) slots - n_layers consecutive layers from `layer`,
// n_seqs / n_layers sequences each
int make_plan(const aatc_codebook* cb, int layer, int n_seqs, int64_t max_len, Plan& p, int n_layers = 1) {
    const int G = cb->group, d = cb->d;
    const int RB = (G + 3) / 4;
    p.nqm_max = 0;
    p.nvb_max = 0;
    for (int l = layer; l < layer + n_layers; ++l)
        for (int h = 0; h < cb->n_kv; ++h) {
            const DevHead& D = cb->blob[(size_t)l * cb->n_kv + h];
            p.nqm_max = std::max(p.nqm_max, D.nqm);
            p.nvb_max = std::max(p.nvb_max, D.nvb);
        }
    p.args.n_seqs_call = n_seqs / n_layers;
    if (cb->heads[0].vq_groups) {  // vector-quantized keys
        DecodeArgs& a = p.args;
        p.vq = true;
        a.G = G;
        a.tile_bytes = 8 * cb->total_bits;
        const VqLds L = vq_lds(cb->heads[0].vq_groups, d, std::min(p.nvb_max, vq_blocks(d)));
        p.lds = (size_t)L.total;
        if (p.lds > 160 * 1024) return set_error(AATC_ERR_UNSUPPORTED, "decode needs %zu bytes of LDS", p.lds);
        p.wgs_per_cu = 1;
        p.nw = kVqWaves;
        const int64_t units = (int64_t)cb->n_kv * n_seqs * ((G + 3) / 4);
        const int64_t slots = 256 * (int64_t)p.wgs_per_cu;
        p.wg_per_head = (int)std::max<int64_t>(1, std::min<int64_t>({slots / units, n_tiles_of(max_len), kMaxWG}));
        a.wg_per_head = p.wg_per_head;
        a.part_ld = kPartHead + 16 * p.nvb_max;
        a.fused = 0;
        p.part_bytes = kCounterBytes + (size_t)n_seqs * cb->n_kv * p.wg_per_head * G * a.part_ld * sizeof(float);
        return AATC_OK;
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
    DecodeArgs& a = p.args;
    a.G = G;
    a.tile_bytes = 8 * cb->total_bits;
    {
        const int lane_bytes = cb->total_bits / 8;  // a multiple of 8 bits: whole bytes per lane
        a.tl.n16 = lane_bytes / 16;
        a.tl.r4 = (lane_bytes % 16) / 4;
        a.tl.r2 = (lane_bytes % 4) / 2;
        a.tl.r1 = lane_bytes % 2;
    }
    a.buf_bytes = (int)al16(a.tile_bytes);
    // the probability operand (RB KiB) overwrites the tile's key block (8 B_K bytes)
    int bk_min = 1 << 30;
    for (int h = 0; h < cb->n_kv; ++h) bk_min = std::min(bk_min, cb->blob[(size_t)layer * cb->n_kv + h].BK);
    const bool own_p = RB * 1024 > 8 * bk_min;  // the probability operand does not fit the key block
    // one workgroup of NW waves per CU; the epilogue reuses the ring
    const int NW = wg_waves(p.v.rb, p.v.nqm, p.v.nvb);
    p.nw = NW;
    const int GP = 4 * epilogue_row_blocks(RB);
    const size_t epi = (size_t)NW * GP * (kPartHead + 16 * p.v.nvb) * sizeof(float);
    const size_t scr = al16((size_t)scratch_bytes(RB, p.v.nqm, p.v.nvb, d));
    const size_t ksch = (size_t)p.v.nqm * 4 * 8 * 4;
    const size_t group = (size_t)NW * a.buf_bytes;  // one ring slot of every wave
    // ring depth: the deepest that the CU's LDS leaves room for beside the prologue's
    // scratch, between 2 and 4 buffers per wave (1 when two do not fit: the waves then
    // overlap each other's streams rather than their own)
    const size_t budget =
        (size_t)(160 * 1024) - ksch - 256 - kMaxRecord - 16 - 32 - (own_p ? (size_t)NW * RB * 1024 : 0);
    a.nbw = 2;
    while (a.nbw < 4 && (a.nbw + 1) * group + scr <= budget) ++a.nbw;
    if (2 * group > budget) a.nbw = 1;  // large tiles: one buffer per wave
    const size_t ring = a.nbw * group;
    size_t top;
    if (ring + scr <= budget) {  // the scratch beside the ring: every slot streams from the start
        a.early = a.nbw;
        a.off_scratch = (int)ring;
        top = ring + scr;
    } else {  // the scratch in the ring's last slots, streamed once the prologue is done
        const int k = (int)std::min<size_t>(a.nbw, (scr + group - 1) / group);
        a.early = a.nbw - k;
        a.off_scratch = (int)(a.early * group);
        top = std::max(ring, a.off_scratch + scr);
    }
    a.off_ksched = (int)al16(std::max(top, epi));
    a.off_rec = (int)al16(a.off_ksched + ksch);  // the appended token's records (outside ring and scratch)
    a.off_sync = a.off_rec + kMaxRecord;         // the q-waves' arrival counter
    p.lds = a.off_sync + 16;
    a.off_pbuf = -1;
    if (own_p) {
        a.off_pbuf = (int)al16(p.lds);
        p.lds = a.off_pbuf + (size_t)NW * RB * 1024;
    }
    p.wgs_per_cu = 1;
    if (p.lds > 160 * 1024 - 256)
        return set_error(AATC_ERR_UNSUPPORTED, "decode needs %zu bytes of LDS per workgroup", p.lds);
    // workgroups per (sequence, kv-head): every resident workgroup slot of the chip busy,
    // at least one tile per wave, at most what one merge round reads
    const int64_t pairs = (int64_t)cb->n_kv * n_seqs;
    const int64_t slots = 256 * (int64_t)p.wgs_per_cu;
    p.wg_per_head = (int)std::max<int64_t>(1, std::min<int64_t>({slots / pairs, (tiles + NW - 1) / NW, kMaxWG}));
    a.wg_per_head = p.wg_per_head;
    a.part_ld = kPartHead + 16 * p.v.nvb;
    // the workspace: kCounterBytes of arrival counters (zero between calls), then the partials
    p.part_bytes = kCounterBytes + (size_t)n_seqs * cb->n_kv * p.wg_per_head * G * a.part_ld * sizeof(float);
    // one launch when the last workgroup of a (sequence, kv-head) can merge: few enough
    // partials, one counter per pair, a partial row within one workgroup's threads, and the
    // merge's LDS below the arrival words
    a.fused = pairs <= kFuseMaxPairs && p.wg_per_head <= kFuseMaxW && G * a.part_ld / 4 <= 64 * NW &&
              (size_t)p.wg_per_head * G * a.part_ld * sizeof(float) <= kFuseMaxBytes &&
              merge_lds_bytes(G, a.part_ld, d, 64 * NW) <= a.off_sync;
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
int launch_decode(const Plan& p, int n_seqs, hipStream_t st, const DevHead* blob, uint8_t* cache,
                  const int32_t* ids, const int64_t* lens, const uint16_t* q, int* ctrs, float* part, float* out) {
    const DecodeArgs& a = p.args;
    if (p.lds > 64 * 1024)
        HIP_TRY(hipFuncSetAttribute((const void*)decode_kernel<RB, NQM, NVB, D>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds));
    hipEvent_t e0, e1;
    profile_slot(e0, e1);
    if (e0) HIP_TRY(hipEventRecord(e0, st));
    if (p.nw != wg_waves(RB, NQM, NVB)) return set_error(AATC_ERR_UNSUPPORTED, "decode plan and variant disagree");
    hipLaunchKernelGGL((decode_kernel<RB, NQM, NVB, D>), dim3(p.wg_per_head, a.n_kv, n_seqs), dim3(64 * p.nw), p.lds, st,
                       blob, cache, a, ids, lens, q, part, ctrs, out);
    HIP_TRY(hipGetLastError());
    if (e1) HIP_TRY(hipEventRecord(e1, st));
    if (!a.fused) {
        hipLaunchKernelGGL((merge_kernel<D>), dim3(a.n_kv * (D / kMergeSlice), n_seqs, a.G), dim3(kMergeThreads), 0, st,
                           blob, a.layer, a.n_kv, a.G, p.wg_per_head, a.part_ld, (const float*)part, out, a.n_seqs_call);
        HIP_TRY(hipGetLastError());
    }
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

template <int D, int NG>
int launch_vq_decode(const Plan& p, int n_seqs, hipStream_t st, const DevHead* blob, uint8_t* cache,
                     const int32_t* ids, const int64_t* lens, const uint16_t* q, float* part, float* out) {
    const DecodeArgs& a = p.args;
    if (p.lds > 64 * 1024)
        HIP_TRY(hipFuncSetAttribute((const void*)vq_decode_kernel<D, NG>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)p.lds));
    hipEvent_t e0, e1;
    profile_slot(e0, e1);
    if (e0) HIP_TRY(hipEventRecord(e0, st));
    for (int vb0 = 0; vb0 < p.nvb_max; vb0 += vq_blocks(D)) {
        hipLaunchKernelGGL((vq_decode_kernel<D, NG>), dim3(p.wg_per_head * ((a.G + 3) / 4), a.n_kv, n_seqs),
                           dim3(64 * kVqWaves), p.lds, st, blob, cache, a, ids, lens, q, part, vb0);
        HIP_TRY(hipGetLastError());
    }
    if (e1) HIP_TRY(hipEventRecord(e1, st));
    hipLaunchKernelGGL((merge_kernel<D>), dim3(a.n_kv * (D / kMergeSlice), n_seqs, a.G), dim3(kMergeThreads), 0, st,
                       blob, a.layer, a.n_kv, a.G, p.wg_per_head, a.part_ld, (const float*)part, out, a.n_seqs_call);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}

extern "C" int aatc_decode_workspace_bytes(const aatc_codebook* cb, int32_t n_seqs, int64_t max_len, size_t* bytes) {
    if (!cb || !bytes) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n_seqs < 1 || max_len < 1) return set_error(AATC_ERR_INVALID_ARG, "need n_seqs >= 1 and max_len >= 1");
    size_t worst = 0;
    for (int layer = 0; layer < cb->n_layers; ++layer) {
        Plan p;
        int rc = make_plan(cb, layer, n_seqs, max_len, p);
        if (rc) return rc;
        worst = std::max(worst, p.part_bytes);
    }
    *bytes = worst;
    return AATC_OK;
}

// Fill a plan's call arguments and launch it: n_slots (layer, sequence) slots of the plan's
// layers (p.args.n_seqs_call sequences per layer), partials and counters in workspace.
static int launch_plan(const aatc_codebook* cb, Plan& p, const aatc_cache* cache, int32_t layer, int n_slots,
                       int64_t max_len, const DevHead* blob, const int32_t* seq_ids, const int64_t* seq_lens,
                       const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q, float* out, void* workspace,
                       hipStream_t st) {
    int* ctrs = (int*)workspace;                                  // arrival counters
    float* part = (float*)((uint8_t*)workspace + kCounterBytes);  // [slots][n_kv][wg][G][part_ld]
    DecodeArgs& a = p.args;
    a.layer = layer;
    a.n_kv = cb->n_kv;
    a.n_seqs_cache = cache->n_seqs;
    a.n_tiles_cap = n_tiles_of(cache->max_tokens);
    if (a.n_tiles_cap * (int64_t)a.tile_bytes >= ((int64_t)1 << 31))
        return set_error(AATC_ERR_CAPACITY, "a (sequence, kv-head) cache range of %lld bytes (at most 2^31 - 1)",
                         (long long)(a.n_tiles_cap * a.tile_bytes));
    a.max_len = max_len;
    uint8_t* c = (uint8_t*)cache->data;
    a.k_new = k_new;
    a.v_new = v_new;
    const int n_seqs = n_slots;
    if (p.vq) {
        if (k_new) return set_error(AATC_ERR_UNSUPPORTED, "fused append with vector-quantized keys");
        const int ng = cb->heads[0].vq_groups;
        if (cb->d == 64)
            return ng == 16 ? launch_vq_decode<64, 16>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, part, out)
                            : launch_vq_decode<64, 0>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, part, out);
        return ng == 32 ? launch_vq_decode<128, 32>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, part, out)
               : ng == 16 ? launch_vq_decode<128, 16>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, part, out)
                          : launch_vq_decode<128, 0>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, part, out);
    }
#define AATC_DECODE_CASE(rb_, nqm_, nvb_)                                                                    \
    if (p.v.rb == rb_ && p.v.nqm == nqm_ && p.v.nvb == nvb_)                                                 \
        return cb->d == 64                                                                                   \
                   ? launch_decode<rb_, nqm_, nvb_, 64>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, ctrs, part, out) \
                   : launch_decode<rb_, nqm_, nvb_, 128>(p, n_seqs, st, blob, c, seq_ids, seq_lens, q, ctrs, part, out);
    AATC_DECODE_CASE(1, 2, 4)
    AATC_DECODE_CASE(1, 2, 8)
    AATC_DECODE_CASE(1, 3, 8)
    AATC_DECODE_CASE(1, 3, 10)
    AATC_DECODE_CASE(1, 4, 12)
    AATC_DECODE_CASE(1, 6, 16)
    AATC_DECODE_CASE(1, 8, 24)
    AATC_DECODE_CASE(1, 16, 24)
    AATC_DECODE_CASE(2, 2, 8)
    AATC_DECODE_CASE(2, 3, 8)
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

static int check_decode_args(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache, int32_t layer,
                             int32_t n_seqs, const int32_t* seq_ids, const int64_t* seq_lens, int64_t max_len,
                             const uint16_t* q, float* out, void* workspace) {
    if (!cb || !d_blob) return set_error(AATC_ERR_INVALID_ARG, "null codebook or blob");
    int rc = check_cache(cb, cache, layer);
    if (rc) return rc;
    if (n_seqs < 1 || n_seqs > cache->n_seqs || !seq_ids || !seq_lens || !q || !out || !workspace)
        return set_error(AATC_ERR_INVALID_ARG, "bad decode arguments");
    if (n_seqs > 65535) return set_error(AATC_ERR_CAPACITY, "at most 65535 sequences per call");
    if (max_len < 1 || max_len > cache->max_tokens)
        return set_error(AATC_ERR_CAPACITY, "max_len %lld outside [1, %lld]", (long long)max_len,
                         (long long)cache->max_tokens);
    if (((uintptr_t)workspace) & 255) return set_error(AATC_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return AATC_OK;
}

static int decode_impl(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache, int32_t layer,
                       int32_t n_seqs, const int32_t* seq_ids, const int64_t* seq_lens, int64_t max_len,
                       const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q, float* out, void* workspace,
                       size_t ws_bytes, void* stream) {
    int rc = check_decode_args(cb, d_blob, cache, layer, n_seqs, seq_ids, seq_lens, max_len, q, out, workspace);
    if (rc) return rc;
    Plan p;
    rc = make_plan(cb, layer, n_seqs, max_len, p);
    if (rc) return rc;
    if (ws_bytes < p.part_bytes)
        return set_error(AATC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, p.part_bytes);
    return launch_plan(cb, p, cache, layer, n_seqs, max_len, (const DevHead*)d_blob, seq_ids, seq_lens, k_new, v_new, q,
                       out, workspace, (hipStream_t)stream);
}

// Layers [layer0, layer0 + n_layers) in runs of consecutive layers that take the same decode
// variant (one launch per run, merge included): run r covers layers [first[r], first[r + 1]).
static int layer_runs(const aatc_codebook* cb, int layer0, int n_layers, int n_seqs, int64_t max_len,
                      std::vector<int>& first) {
    first.clear();
    Variant prev{0, 0, 0};
    for (int l = layer0; l < layer0 + n_layers; ++l) {
        Plan p;
        const int rc = make_plan(cb, l, n_seqs, max_len, p);
        if (rc) return rc;
        if (p.vq) return set_error(AATC_ERR_UNSUPPORTED, "batched layers with vector-quantized keys");
        if (l == layer0 || p.v.rb != prev.rb || p.v.nqm != prev.nqm || p.v.nvb != prev.nvb) first.push_back(l);
        prev = p.v;
    }
    first.push_back(layer0 + n_layers);
    return AATC_OK;
}

extern "C" int aatc_decode_attention(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                     int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const int64_t* seq_lens,
                                     int64_t max_len, const uint16_t* q, float* out, void* workspace,
                                     size_t ws_bytes, void* stream) {
    return decode_impl(cb, d_blob, cache, layer, n_seqs, seq_ids, seq_lens, max_len, nullptr, nullptr, q, out,
                       workspace, ws_bytes, stream);
}

extern "C" int aatc_decode_layers_workspace_bytes(const aatc_codebook* cb, int32_t layer0, int32_t n_layers,
                                                  int32_t n_seqs, int64_t max_len, size_t* bytes) {
    if (!cb || !bytes) return set_error(AATC_ERR_INVALID_ARG, "null pointer");
    if (n_seqs < 1 || max_len < 1 || n_layers < 1 || layer0 < 0 || layer0 + n_layers > cb->n_layers)
        return set_error(AATC_ERR_INVALID_ARG, "need n_seqs, max_len, n_layers >= 1 and layers within the codebook");
    std::vector<int> first;
    int rc = layer_runs(cb, layer0, n_layers, n_seqs, max_len, first);
    if (rc) return rc;
    size_t worst = 0;
    for (size_t r = 0; r + 1 < first.size(); ++r) {
        const int nl = first[r + 1] - first[r];
        Plan p;
        rc = make_plan(cb, first[r], nl * n_seqs, max_len, p, nl);
        if (rc) return rc;
        worst = std::max(worst, p.part_bytes);
    }
    *bytes = worst;
    return AATC_OK;
}

extern "C" int aatc_decode_attention_layers(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                            int32_t layer0, int32_t n_layers, int32_t n_seqs, const int32_t* seq_ids,
                                            const int64_t* seq_lens, int64_t max_len, const uint16_t* q, float* out,
                                            void* workspace, size_t ws_bytes, void* stream) {
    if (n_layers < 1 || layer0 < 0 || !cb || layer0 + n_layers > cb->n_layers)
        return set_error(AATC_ERR_INVALID_ARG, "layers [%d, %d) outside the codebook", layer0, layer0 + n_layers);
    for (int l = layer0; l < layer0 + n_layers; ++l) {
        const int rc = check_decode_args(cb, d_blob, cache, l, n_seqs, seq_ids, seq_lens, max_len, q, out, workspace);
        if (rc) return rc;
    }
    if ((int64_t)n_layers * n_seqs > 65535) return set_error(AATC_ERR_CAPACITY, "at most 65535 (layer, sequence) slots");
    std::vector<int> first;
    int rc = layer_runs(cb, layer0, n_layers, n_seqs, max_len, first);
    if (rc) return rc;
    std::vector<Plan> plans(first.size() - 1);
    for (size_t r = 0; r + 1 < first.size(); ++r) {  // every run checked before the first launch
        const int nl = first[r + 1] - first[r];
        rc = make_plan(cb, first[r], nl * n_seqs, max_len, plans[r], nl);
        if (rc) return rc;
        if (ws_bytes < plans[r].part_bytes)
            return set_error(AATC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, plans[r].part_bytes);
    }
    const size_t row = (size_t)cb->n_kv * cb->group * cb->d;  // q / out elements per (layer, sequence)
    for (size_t r = 0; r + 1 < first.size(); ++r) {
        const int nl = first[r + 1] - first[r];
        const size_t off = (size_t)(first[r] - layer0) * n_seqs * row;
        rc = launch_plan(cb, plans[r], cache, first[r], nl * n_seqs, max_len, (const DevHead*)d_blob, seq_ids, seq_lens,
                         nullptr, nullptr, q + off, out + off, workspace, (hipStream_t)stream);
        if (rc) return rc;
    }
    return AATC_OK;
}

// ---------------------------------------------------------------------------------------
// Decode without a caller-provided workspace: the partials and arrival counters live in a
// file-scope device array, one copy per GPU, for callers that cannot allocate device memory
// (code under graph capture, serving loops that forbid allocation).  Host code uses the
// array only through the address hipGetSymbolAddress returns for the current device (the
// array's name on the host is a stand-in, not a device address).  The arrival counters
// (the first bytes) are zero when the code object is loaded and every call leaves them at
// zero; the partials are overwritten by each call before they are read.  Calls that overlap
// in time on one GPU share the array and race.
// ---------------------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // per device: the device address of `scratch`, once looked up

// the current device's copy of the scratch array (looked up once per device)
static int static_scratch(void** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return set_error(AATC_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return set_error(AATC_ERR_HIP, "hipGetSymbolAddress returned a null address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return AATC_OK;
}

extern "C" int aatc_decode_attention_static(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                            int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                            const int64_t* seq_lens, int64_t max_len, const uint16_t* q, float* out,
                                            void* stream) {
    if (!cb) return set_error(AATC_ERR_INVALID_ARG, "null codebook");
    if (n_seqs < 1 || max_len < 1) return set_error(AATC_ERR_INVALID_ARG, "need n_seqs >= 1 and max_len >= 1");
    size_t need = 0;
    int rc = aatc_decode_workspace_bytes(cb, n_seqs, max_len, &need);
    if (rc) return rc;
    if (need > kStaticScratchBytes)
        return set_error(AATC_ERR_CAPACITY, "the call needs %zu bytes of partials, the static scratch holds %zu", need,
                         kStaticScratchBytes);
    void* ws = nullptr;
    rc = static_scratch(&ws);
    if (rc) return rc;
    return decode_impl(cb, d_blob, cache, layer, n_seqs, seq_ids, seq_lens, max_len, nullptr, nullptr, q, out, ws,
                       kStaticScratchBytes, stream);
}

extern "C" int aatc_decode_attention_append(const aatc_codebook* cb, const void* d_blob, const aatc_cache* cache,
                                            int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                            const int64_t* seq_lens, int64_t max_len, const uint16_t* k_new,
                                            const uint16_t* v_new, const uint16_t* q, float* out, void* workspace,
                                            size_t ws_bytes, void* stream) {
    if (!k_new || !v_new) return set_error(AATC_ERR_INVALID_ARG, "null new key or value");
    if ((((uintptr_t)k_new) | ((uintptr_t)v_new)) & 15)
        return set_error(AATC_ERR_INVALID_ARG, "new key and value rows must be 16-byte aligned");
    return decode_impl(cb, d_blob, cache, layer, n_seqs, seq_ids, seq_lens, max_len, k_new, v_new, q, out,
                       workspace, ws_bytes, stream);
}
