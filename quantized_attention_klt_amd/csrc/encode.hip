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
using aatc::code_byte;
using aatc::quantize;
using aatc::set_error;

namespace {

constexpr int kMaxSeqPerLaunch = 64;
constexpr int kCUs = 256;               // compute units of an MI355X
constexpr size_t kLdsPerCU = 160 * 1024;  // LDS bytes per compute unit (gfx950)

struct SeqArgs {
    int32_t n;
    int32_t seq[kMaxSeqPerLaunch];
    int64_t start[kMaxSeqPerLaunch];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))


// LDS-only workgroup barrier: this wave's LDS operations are complete, then s_barrier
// (vector memory operations in flight are not waited for; their waits are explicit)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait until at most n of this wave's vector memory operations are outstanding (they
// complete in issue order; n is clamped to 15, which only waits longer)
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

// A tile's block (keys or values) is assembled in LDS byte-major, every code's fields OR-ed
// into place: record byte q of slots 4u .. 4u + 3 is LDS word q * kStageRow + u.  The row
// stride of 18 words puts record byte q in bank group q mod 16, so codes of one instruction
// whose record bytes differ mod 16 hit distinct banks.  Then the block is copied out: the
// value block is byte-major in the tile as well; the key block is word-major (tile word
// 64 r + s = record word r of slot s), a 4 x 4 byte transpose of four staged rows.
constexpr int kStageRow = 18;
constexpr int kStageWords = aatc::kMaxRecordBytes * kStageRow;

// Fields of one record kind by channel, staged in LDS: channel j's fields (lowest code bits
// first) are piece[first[j] .. first[j + 1]), each byte | pos << 8 | width << 12 | shift << 16.
struct PieceTab {
    uint32_t piece[aatc::kMaxFields];
    int16_t first[aatc::kMaxD + 8];
};

__device__ void stage_pieces(const DevHead& H, bool isV, LDS_AS PieceTab* pt, int tid, int nthreads) {
    const uint32_t* p = isV ? H.cpieceV : H.cpieceK;
    const int16_t* f = isV ? H.cfirstV : H.cfirstK;
    const int np = isV ? H.nfV : H.nfK;
    for (int i = tid; i < np; i += nthreads) pt->piece[i] = p[i];
    for (int i = tid; i <= H.d; i += nthreads) pt->first[i] = f[i];
}

__device__ __forceinline__ void lds_or(LDS_AS uint32_t* p, uint32_t v) { (void)__atomic_fetch_or(p, v, __ATOMIC_RELAXED); }

// The same LDS OR written as an instruction of its own, at p + OFF bytes.  The compiler
// makes every LDS atomic wait for all direct-to-LDS copies in flight (vmcnt(0)), which would
// stall the tile stream; this one it does not see.  LDS operations complete in order, so its
// own LDS waits stay sufficient, and the workgroup barrier waits for all LDS operations.
template <int OFF>
__device__ __forceinline__ void lds_or_async(LDS_AS uint32_t* p, uint32_t v) {
    asm volatile("ds_or_b32 %0, %1 offset:%2" ::"v"(p), "v"(v), "i"(OFF) : "memory");
}

// every field of channel j's code of slot s, OR-ed into the staged block
__device__ __forceinline__ void scatter_code(LDS_AS uint32_t* stg, const LDS_AS PieceTab* pt, int j, int s, uint32_t code) {
    for (int p = pt->first[j]; p < pt->first[j + 1]; ++p) {
        const uint32_t pc = pt->piece[p];
        const int q = pc & 0xff, pos = (pc >> 8) & 7, wd = (pc >> 12) & 15, e = (pc >> 16) & 15;
        lds_or(stg + q * kStageRow + (s >> 2), ((code >> e) & ((1u << wd) - 1u)) << (8 * (s & 3) + pos));
    }
}

// Copy the staged block to the tile at dst for the slots [s0, s1) and clear the staging.
// One item = 16 tile bytes: key block, record word r of slots 4u .. 4u + 3 (from staged
// rows 4r .. 4r + 3); value block, record byte q of slots 16 v .. 16 v + 15 (staged row q).
// Stored bytes carry bit 7 inverted; a value word shared with slots outside [s0, s1) keeps
// their stored bytes (the staging holds codes of every slot of the tile, so the bytes of
// those slots are masked out).
template <bool ISV>
__device__ __forceinline__ void staged_item(LDS_AS uint32_t* stg, int it, uint32_t (&out)[4], int& word0) {
    if (!ISV) {
        const int r = it >> 4, u = it & 15;
        uint32_t W[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            W[b] = stg[(4 * r + b) * kStageRow + u];
            stg[(4 * r + b) * kStageRow + u] = 0u;
        }
        const uint32_t t0 = __builtin_amdgcn_perm(W[1], W[0], 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(W[3], W[2], 0x05010400u);
        const uint32_t t2 = __builtin_amdgcn_perm(W[1], W[0], 0x07030602u);
        const uint32_t t3 = __builtin_amdgcn_perm(W[3], W[2], 0x07030602u);
        out[0] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);  // slot 4u: bytes of rows 4r .. 4r + 3
        out[1] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
        out[2] = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
        out[3] = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
        word0 = 64 * r + 4 * u;
    } else {
        const int q = it >> 2, v = it & 3;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[k] = stg[q * kStageRow + 4 * v + k];
            stg[q * kStageRow + 4 * v + k] = 0u;
        }
        word0 = 16 * q + 4 * v;
    }
}

template <bool ISV>
__device__ void copy_out(LDS_AS uint32_t* stg, int nbytes, uint32_t* dst, int s0, int s1, int tid, int nthreads) {
    const int nitems = 4 * nbytes;  // 16 nbytes tile words, 4 per item
    if (s0 == 0 && s1 == kTile) {   // a whole tile: one 16-byte store per item
        for (int it = tid; it < nitems; it += nthreads) {
            uint32_t out[4];
            int word0;
            staged_item<ISV>(stg, it, out, word0);
            *(u32x4*)(dst + word0) =
                u32x4{out[0] ^ 0x80808080u, out[1] ^ 0x80808080u, out[2] ^ 0x80808080u, out[3] ^ 0x80808080u};
        }
        return;
    }
    for (int it = tid; it < nitems; it += nthreads) {
        uint32_t out[4];
        int word0;
        staged_item<ISV>(stg, it, out, word0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t keep = 0u;
            if (!ISV) {
                const int s = 4 * (it & 15) + k;
                if (s < s0 || s >= s1) keep = 0xFFFFFFFFu;
            } else {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int s = 16 * (it & 3) + 4 * k + b;
                    if (s < s0 || s >= s1) keep |= 0xFFu << (8 * b);
                }
            }
            if (keep != 0xFFFFFFFFu)
                dst[word0 + k] = ((out[k] ^ 0x80808080u) & ~keep) | (keep ? dst[word0 + k] & keep : 0u);
        }
    }
}

__device__ __forceinline__ uint8_t* tile_ptr(uint8_t* cache, int layer, int n_seqs_cache, int seq, int n_kv, int h,
                                             int64_t n_tiles_cap, int64_t tile, int tile_bytes) {
    return cache + ((((int64_t)layer * n_seqs_cache + seq) * n_kv + h) * n_tiles_cap + tile) * (int64_t)tile_bytes;
}

// The 64 token rows (D bf16 each) of tile index tl into LDS at xd by direct global->LDS
// copies: copy n of wave w fills the 64 chunk positions p = 64 (NLD w + n) + lane (token
// t = p / CH, position p % CH), and position p holds the token's chunk (p % CH) ^ (t mod CH)
// (the swizzle is in the source addresses), so that the 16 rows an MFMA operand read touches
// fall in distinct banks.  Slots outside the call's tokens copy the call's first token
// (their codes are never stored).  The copies carry the non-temporal hint: inputs are read
// once.  A tile whose 64 tokens all lie in the call is read by buffer loads: one resource per
// tile (scalar, based at its first token).  Copy n's token is t0 + n (64 / CH) and its chunk
// kc0 ^ ((n 64 / CH) mod CH) (t0 mod CH has no bits in common with n 64 / CH), so the lane's
// byte offset is xa + (xb ^ 16 K_n) plus a scalar n (64 / CH) token rows.
template <int D>
__device__ __forceinline__ void copy_x_rows(const uint16_t* __restrict__ X, int64_t xstride, int64_t start,
                                            int64_t n_tokens, int64_t tl, LDS_AS uint8_t* xd, int w, int lane) {
    constexpr int CH = D / 8, NLD = 64 * CH / 256;
    const int64_t tok0 = tl * kTile;
    if (tok0 >= start && tok0 + kTile <= start + n_tokens) {
        const int t0 = (64 * NLD * w + lane) / CH;
        const uint32_t xa = (uint32_t)(2 * t0 * xstride), xb = 16u * (uint32_t)((lane % CH) ^ (t0 & (CH - 1)));
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(X + (tok0 - start) * xstride), (short)0, (int)(2 * kTile * xstride), 0x00020000);
#pragma unroll
        for (int n = 0; n < NLD; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(xd + 1024 * (NLD * w + n)), 16,
                                                     xa + (xb ^ (16u * ((n * 64 / CH) & (CH - 1)))),
                                                     (int)(2 * n * (64 / CH) * xstride), 0, 2);
        return;
    }
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const int p = 64 * (NLD * w + n) + lane, t = p / CH, kc = (p % CH) ^ (t & (CH - 1));
        int64_t tt = tok0 + t - start;  // token index in this call's input
        tt = tt < 0 || tt >= n_tokens ? 0 : tt;
        __builtin_amdgcn_global_load_lds((const void*)(X + tt * xstride + 8 * kc),
                                         (LDS_AS void*)(xd + 1024 * (NLD * w + n)), 16, 0, 2);
    }
}

// ------------------------------------------------------------------------------------
// encode from bf16 K, V (MFMA): a workgroup owns one (sequence, kv-head, keys | values)
// and the tiles bx, bx + gridDim.x, ... of the call.  u = x (W_hi + W_lo) + start (W = U
// scaled by 1/step per channel, start = 2^(b-1) - 1/2 - mu W, so u = c/step + 2^(b-1) - 1/2)
// on v_mfma_f32_16x16x32_bf16: rows = tokens, columns = channels (in the encoder's channel
// order), accumulators starting at start; the code is u clamped and rounded (code_byte).
// Wave w keeps the B operands (W^T hi / lo
// fragments) of its D / 4 columns in registers for all its tiles.  The 64-token x tiles
// arrive by direct global->LDS copies into two buffers (the next tile streams while this
// one is computed), their 16-byte chunks XOR-swizzled by token so that the 16 rows an
// operand read touches fall in distinct banks.  Lane (g, c) quantizes tokens 16 tb + 4 g + e
// of its channel, packs the four codes of one tb into a word (they share a staged word) and
// ORs each field into the staged block with one LDS operation per field and four tokens.
// ------------------------------------------------------------------------------------
// x tiles per workgroup in LDS (all but one in flight).  Two: a third buffer lowers the
// residency to two workgroups per CU, and the kernel is bound by its MFMA and VALU work, not
// by the bytes in flight (the 128k Llama layer: 164 us with two buffers, 197 us with three,
// before the quantizer was folded into the projection).
constexpr int kEncodeRing = 2;

template <int D>
constexpr size_t encode_lds_bytes() { return kEncodeRing * 64 * D * 2 + 4 * kStageWords + sizeof(PieceTab); }

template <int D, bool isV, int NT3>
__device__ __forceinline__ void encode_mfma_body(const DevHead* __restrict__ blob, uint8_t* __restrict__ cache,
                                                 int layer, int n_kv, int64_t n_tiles_cap, int tile_bytes,
                                                 const SeqArgs& sa, int64_t n_tokens, int64_t ntiles,
                                                 const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                 int n_seqs_cache) {
    constexpr int CH = D / 8;          // 16-byte chunks per token row
    constexpr int CBW = D / 64;        // 16-channel column blocks per wave
    constexpr int KS = D / 32;         // k-steps
    constexpr int XB = 64 * D * 2;     // bytes of one x tile
    constexpr int NLD = 64 * CH / 256;  // chunk loads per thread
    constexpr int NB = kEncodeRing;
    // LDS (one dynamic array): NB x tiles, the staged block, the field table
    extern __shared__ __attribute__((aligned(16))) uint8_t esm_generic[];
    LDS_AS uint8_t* const esm = (LDS_AS uint8_t*)esm_generic;
    LDS_AS uint32_t* const stg = (LDS_AS uint32_t*)(esm + NB * XB);
    LDS_AS PieceTab* const pt = (LDS_AS PieceTab*)(esm + NB * XB + 4 * kStageWords);
    const int h = blockIdx.y >> 1, zi = blockIdx.z;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, c = lane & 15;
    const DevHead& H = blob[layer * n_kv + h];
    const uint16_t* X = (isV ? V : K) + ((int64_t)zi * n_tokens * n_kv + h) * D;  // token t at X + t * n_kv * D
    const int64_t xstride = (int64_t)n_kv * D;
    const int64_t start = sa.start[zi];
    const int64_t first_tile = start / kTile;
    const int seq = sa.seq[zi];
    stage_pieces(H, isV, pt, tid, 256);
    for (int i = tid; i < kStageWords; i += 256) stg[i] = 0u;
    // B operands and quantizer constants of this lane's columns 16 (w CBW + cbw) + c: channel
    // j = encoder order of that column (an uncoded channel has a zero column and no field)
    bf16x8 bh[CBW][KS], bl[CBW][KS];
    bf16x8 bm[NT3 == 3 ? CBW : 1][KS];  // third terms (three-term bases only)
    float ustart[CBW], cmax[CBW];
    int jj[CBW];
    {
        const uint16_t* uh = isV ? H.EVt_hi : H.EKt_hi;
        const uint16_t* ul = isV ? H.EVt_lo : H.EKt_lo;
        const uint8_t* perm = isV ? H.encpermV : H.encpermK;
#pragma unroll
        for (int cbw = 0; cbw < CBW; ++cbw) {
            const int j = perm[16 * (w * CBW + cbw) + c];
            jj[cbw] = j;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bh[cbw][ks] = *(const bf16x8*)(uh + j * D + 32 * ks + 8 * g);
                bl[cbw][ks] = *(const bf16x8*)(ul + j * D + 32 * ks + 8 * g);
                if constexpr (NT3 == 3) bm[cbw][ks] = *(const bf16x8*)((isV ? H.EVt_mid : H.EKt_mid) + j * D + 32 * ks + 8 * g);
            }
            ustart[cbw] = isV ? H.estartV[j] : H.estartK[j];
            cmax[cbw] = (float)((1 << (isV ? H.bitsV[j] : H.bitsK[j])) - 1);
        }
    }
    const int nbytes = (isV ? H.BV : H.BK) / 8;
    const int boff = isV ? 8 * H.BK : 0;  // block offset in the tile
    auto copy_x = [&](int64_t tl, LDS_AS uint8_t* xd) { copy_x_rows<D>(X, xstride, start, n_tokens, tl, xd, w, lane); };
    int64_t tile = blockIdx.x;
    // the first NB - 1 tiles stream during the set-up
#pragma unroll
    for (int m = 0; m < NB - 1; ++m)
        if (tile + (int64_t)m * gridDim.x < ntiles) copy_x(first_tile + tile + (int64_t)m * gridDim.x, esm + m * XB);
    lds_barrier();  // field table staged, staging clear
    // this lane's channels: their fields (usually one) are pt->piece[pf[cbw] .. pl[cbw]); the
    // first (code bits from 0) as registers: staged word of its record byte for this lane's
    // slots 4g .. 4g + 3, bit position, per-byte mask (0: no field)
    int pf[CBW], pl[CBW], pos0[CBW];
    LDS_AS uint32_t* base0[CBW];
    uint32_t mask0[CBW];
#pragma unroll
    for (int cbw = 0; cbw < CBW; ++cbw) {
        pf[cbw] = pt->first[jj[cbw]];
        pl[cbw] = pt->first[jj[cbw] + 1];
        const uint32_t pc = pt->piece[min(pf[cbw], aatc::kMaxFields - 1)];
        base0[cbw] = stg + (pc & 0xff) * kStageRow + g;
        pos0[cbw] = (pc >> 8) & 7;
        mask0[cbw] = pl[cbw] > pf[cbw] ? ((1u << ((pc >> 12) & 15)) - 1u) * 0x01010101u : 0u;
    }
    // this wave's copy-out stores per full tile: one 16-byte store per item round it takes part in
    const int n_items = 4 * nbytes;
    const int st_full = max(0, (n_items - 64 * w + 255) / 256);
    // stores issued by the copy-outs of the previous NB - 1 tiles, latest first (-1: not
    // counted; a partial tile's copy-out is a read-modify-write of run-time length)
    int st_prev[NB - 1];
#pragma unroll
    for (int m = 0; m < NB - 1; ++m) st_prev[m] = 0;
    // one tile: its x in ring slot `slot`; tile + (NB - 1) strides is copied into the slot
    // the previous tile used
    auto step = [&](int slot) {
        const LDS_AS uint8_t* xc = esm + slot * XB;
        // this tile's copies have landed: issued after them are the copies of the next
        // NB - 2 tiles (those that exist) and the copy-outs of the previous NB - 1 tiles;
        // then every wave's have, and every wave is past the previous tile
        int after = 0;
        bool counted = true;
#pragma unroll
        for (int m = 0; m < NB - 1; ++m) {
            counted = counted && st_prev[m] >= 0;
            after += st_prev[m];
        }
#pragma unroll
        for (int m = 1; m < NB - 1; ++m)
            if (tile + (int64_t)m * gridDim.x < ntiles) after += NLD;
        wait_vm(counted ? after : 0);
        lds_barrier();
        const int64_t tile_f = tile + (int64_t)(NB - 1) * gridDim.x;
        if (tile_f < ntiles)  // in flight during this tile and the next NB - 2
            copy_x(first_tile + tile_f, esm + (slot == 0 ? NB - 1 : slot - 1) * XB);
        f32x4 acc[CBW][4];
#pragma unroll
        for (int cbw = 0; cbw < CBW; ++cbw)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[cbw][tb] = f32x4{ustart[cbw], ustart[cbw], ustart[cbw], ustart[cbw]};
        // two token blocks at a time, per k-step: the hi products of their 2 CBW accumulators,
        // then the lo products, so that consecutive MFMAs are independent (each accumulator
        // still adds hi then lo per k-step; four blocks at once spill registers)
        constexpr int TBG = 2;
#pragma unroll
        for (int tg = 0; tg < 4; tg += TBG)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 av[TBG];
#pragma unroll
            for (int u = 0; u < TBG; ++u) {
                const int t = 16 * (tg + u) + c;  // A row: token
                av[u] = *(const LDS_AS bf16x8*)(xc + t * 2 * D + 16 * ((4 * ks + g) ^ (t & (CH - 1))));
            }
#pragma unroll
            for (int u = 0; u < TBG; ++u)
#pragma unroll
                for (int cbw = 0; cbw < CBW; ++cbw)
                    acc[cbw][tg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bh[cbw][ks], acc[cbw][tg + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < TBG; ++u)
#pragma unroll
                for (int cbw = 0; cbw < CBW; ++cbw)
                    acc[cbw][tg + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bl[cbw][ks], acc[cbw][tg + u], 0, 0, 0);
            if constexpr (NT3 == 3) {
#pragma unroll
                for (int u = 0; u < TBG; ++u)
#pragma unroll
                    for (int cbw = 0; cbw < CBW; ++cbw)
                        acc[cbw][tg + u] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bm[cbw][ks], acc[cbw][tg + u], 0, 0, 0);
            }
        }
        // codes of tokens 16 tb + 4 g + e: the four of one tb share staged word q * kStageRow +
        // 4 tb + g (byte e), so they are packed into one word and OR-ed with one operation per
        // field (the per-byte mask keeps a field's bits; later fields shift the code down)
#pragma unroll
        for (int cbw = 0; cbw < CBW; ++cbw) {
            uint32_t c4[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                uint32_t v = code_byte(acc[cbw][tb][0], cmax[cbw], 0, 0u);
                v = code_byte(acc[cbw][tb][1], cmax[cbw], 1, v);
                v = code_byte(acc[cbw][tb][2], cmax[cbw], 2, v);
                c4[tb] = code_byte(acc[cbw][tb][3], cmax[cbw], 3, v);
            }
            if (mask0[cbw]) {
                lds_or_async<0>(base0[cbw], (c4[0] & mask0[cbw]) << pos0[cbw]);
                lds_or_async<16>(base0[cbw], (c4[1] & mask0[cbw]) << pos0[cbw]);
                lds_or_async<32>(base0[cbw], (c4[2] & mask0[cbw]) << pos0[cbw]);
                lds_or_async<48>(base0[cbw], (c4[3] & mask0[cbw]) << pos0[cbw]);
            }
            for (int p = pf[cbw] + 1; p < pl[cbw]; ++p) {  // the rest of a split channel
                const uint32_t pc = pt->piece[p];
                LDS_AS uint32_t* base = stg + (pc & 0xff) * kStageRow + g;
                const int pos = (pc >> 8) & 7, e0 = (pc >> 16) & 15;
                const uint32_t mask = ((1u << ((pc >> 12) & 15)) - 1u) * 0x01010101u;
                lds_or_async<0>(base, ((c4[0] >> e0) & mask) << pos);
                lds_or_async<16>(base, ((c4[1] >> e0) & mask) << pos);
                lds_or_async<32>(base, ((c4[2] >> e0) & mask) << pos);
                lds_or_async<48>(base, ((c4[3] >> e0) & mask) << pos);
            }
        }
        lds_barrier();
        const int64_t tok0 = (first_tile + tile) * kTile;
        const int s0 = (int)max(start - tok0, (int64_t)0);
        const int s1 = (int)min(start + n_tokens - tok0, (int64_t)kTile);
        uint8_t* tp = tile_ptr(cache, layer, n_seqs_cache, seq, n_kv, h, n_tiles_cap, first_tile + tile, tile_bytes);
        copy_out<isV>(stg, nbytes, (uint32_t*)(tp + boff), s0, s1, tid, 256);
#pragma unroll
        for (int m = NB - 2; m > 0; --m) st_prev[m] = st_prev[m - 1];
        st_prev[0] = (s0 == 0 && s1 == kTile) ? st_full : -1;
        tile += gridDim.x;
    };
    for (int slot = 0; tile < ntiles; slot = slot + 1 == NB ? 0 : slot + 1) step(slot);
    wait_vm(0);
}

// NT3: basis terms (2, or 3 for rates above 6.5 bits/element, whose third operands take the
// registers of a third wave per SIMD)
template <int D, int NT3>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT3 == 3 ? 2 : 3))) void encode_mfma_kernel(
    const DevHead* __restrict__ blob, uint8_t* __restrict__ cache, int layer, int n_kv, int64_t n_tiles_cap,
    int tile_bytes, SeqArgs sa, int64_t n_tokens, int64_t ntiles, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int n_seqs_cache, int values_only) {
    if (values_only && !(blockIdx.y & 1)) return;  // keys are vector-quantized by vq_keys_kernel
    if (blockIdx.y & 1)
        encode_mfma_body<D, true, NT3>(blob, cache, layer, n_kv, n_tiles_cap, tile_bytes, sa, n_tokens, ntiles, K, V,
                                       n_seqs_cache);
    else
        encode_mfma_body<D, false, NT3>(blob, cache, layer, n_kv, n_tiles_cap, tile_bytes, sa, n_tokens, ntiles, K, V,
                                        n_seqs_cache);
}

// ------------------------------------------------------------------------------------
// encode given KLT coefficients: one workgroup per (tile, kv-head, sequence); the codes of
// both blocks are OR-ed into their staging, then both blocks are copied out.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void encode_coeffs_kernel(const DevHead* __restrict__ blob,
                                                            uint8_t* __restrict__ cache, int layer, int n_kv,
                                                            int64_t n_tiles_cap, int tile_bytes, SeqArgs sa,
                                                            int64_t n_tokens, const float* __restrict__ coeffs,
                                                            int n_seqs_cache) {
    __shared__ __attribute__((aligned(16))) uint32_t stg[2][kStageWords];
    __shared__ PieceTab pt[2];
    const int h = blockIdx.y, zi = blockIdx.z;
    const DevHead& H = blob[layer * n_kv + h];
    const int d = H.d, n_g = H.vq_groups;
    const int64_t start = sa.start[zi];
    const int64_t tile = start / kTile + blockIdx.x;
    const int64_t tok0 = tile * kTile;
    const int s0 = (int)std::max<int64_t>(start - tok0, 0);
    const int s1 = (int)std::min<int64_t>(start + n_tokens - tok0, kTile);
    LDS_AS PieceTab* const ptl = (LDS_AS PieceTab*)&pt[0];
    LDS_AS uint32_t* const sg0 = (LDS_AS uint32_t*)&stg[0][0];
    LDS_AS uint32_t* const sg1 = (LDS_AS uint32_t*)&stg[1][0];
    stage_pieces(H, false, ptl, threadIdx.x, blockDim.x);
    stage_pieces(H, true, ptl + 1, threadIdx.x, blockDim.x);
    for (int i = threadIdx.x; i < 2 * kStageWords; i += blockDim.x) stg[i / kStageWords][i % kStageWords] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < (s1 - s0) * 2 * d; i += blockDim.x) {
        const int s = s0 + i / (2 * d), r = i % (2 * d), kv = r / d, j = r % d;
        const int64_t t = tok0 + s - start;  // token index in this call's input
        const float cf = coeffs[((t * n_kv + h) * 2 + kv) * d + j];
        const int b = kv ? H.bitsV[j] : H.bitsK[j];
        if (b) scatter_code(kv ? sg1 : sg0, ptl + kv, j, s, quantize(cf, kv ? H.invV[j] : H.invK[j], b));
    }
    // vector-quantized keys: one index per (slot, group), record byte g
    for (int i = threadIdx.x; i < (s1 - s0) * n_g; i += blockDim.x) {
        const int s = s0 + i / n_g, g = i % n_g;
        const float* cf = coeffs + ((tok0 + s - start) * n_kv + h) * 2 * d;
        float u[aatc::kVqDim];
#pragma unroll
        for (int k = 0; k < aatc::kVqDim; ++k) {
            const int j = H.vq_chan[g][k];
            u[k] = __fmul_rn(cf[j], H.vq_scale[j]);
        }
        scatter_code(sg0, ptl, g, s, aatc::vq_nearest(H.vq_cent[g], u[0], u[1], u[2], u[3]));
    }
    __syncthreads();
    uint8_t* tp = tile_ptr(cache, layer, n_seqs_cache, sa.seq[zi], n_kv, h, n_tiles_cap, tile, tile_bytes);
    copy_out<false>(sg0, H.BK / 8, (uint32_t*)tp, s0, s1, threadIdx.x, blockDim.x);
    copy_out<true>(sg1, H.BV / 8, (uint32_t*)(tp + 8 * H.BK), s0, s1, threadIdx.x, blockDim.x);
}

// ------------------------------------------------------------------------------------
// vector-quantized keys from bf16 K ("Spend Bits Where Queries Look", abstract): one
// workgroup per (tile, kv-head, sequence).  The tile's centred rows x - mu_K go to LDS in
// fp32; coefficients c_j = sum_i (x - mu)_i U_K[i][j] by fp32 multiply-adds in i order
// (thread: channel j, every 256/D-th token), written back over the rows; then wave w takes
// the groups w, w + 4, ... with one token per lane: u_k = fp32(c_k s_k), the nearest of the
// group's 256 codewords (the host-side definition, bit for bit), OR-ed into the staged key
// block as record byte g.  The values of these tokens are coded by the MFMA encoder.
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void vq_keys_kernel(const DevHead* __restrict__ blob, uint8_t* __restrict__ cache,
                                                      int layer, int n_kv, int64_t n_tiles_cap, int tile_bytes,
                                                      SeqArgs sa, int64_t n_tokens, const uint16_t* __restrict__ K,
                                                      int n_seqs_cache) {
    constexpr int XS = D + 4;        // LDS row stride (floats)
    constexpr int TPH = 256 / D;     // token phases
    constexpr int NT = kTile / TPH;  // tokens per thread
    __shared__ __attribute__((aligned(16))) float xs[kTile * XS];
    __shared__ __attribute__((aligned(16))) uint32_t stg[kStageWords];
    __shared__ PieceTab pt;
    const int h = blockIdx.y, zi = blockIdx.z, tid = threadIdx.x;
    const DevHead& H = blob[layer * n_kv + h];
    const int n_g = H.vq_groups;
    const int64_t start = sa.start[zi];
    const int64_t tile = start / kTile + blockIdx.x;
    const int64_t tok0 = tile * kTile;
    const int s0 = (int)std::max<int64_t>(start - tok0, 0);
    const int s1 = (int)std::min<int64_t>(start + n_tokens - tok0, kTile);
    LDS_AS PieceTab* const ptl = (LDS_AS PieceTab*)&pt;
    LDS_AS uint32_t* const sg = (LDS_AS uint32_t*)&stg[0];
    stage_pieces(H, false, ptl, tid, 256);
    for (int i = tid; i < kStageWords; i += 256) stg[i] = 0u;
    const uint16_t* X = K + ((int64_t)zi * n_tokens * n_kv + h) * D;  // token t at X + t * n_kv * D
    for (int i = tid; i < kTile * D; i += 256) {
        const int s = i / D, c = i % D;
        xs[s * XS + c] = s >= s0 && s < s1 ? bf16f(X[(tok0 + s - start) * n_kv * D + c]) - H.muK[c] : 0.0f;
    }
    __syncthreads();
    const int j = tid % D, ph = tid / D;
    float acc[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = 0.0f;
    for (int i = 0; i < D; i += 4) {
        const float u0 = H.UK[(i + 0) * D + j], u1 = H.UK[(i + 1) * D + j];
        const float u2 = H.UK[(i + 2) * D + j], u3 = H.UK[(i + 3) * D + j];
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const float4 x = *(const float4*)&xs[(ph + TPH * k) * XS + i];
            acc[k] = fmaf(x.x, u0, acc[k]);
            acc[k] = fmaf(x.y, u1, acc[k]);
            acc[k] = fmaf(x.z, u2, acc[k]);
            acc[k] = fmaf(x.w, u3, acc[k]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NT; ++k) xs[(ph + TPH * k) * XS + j] = acc[k];
    __syncthreads();
    const int w = tid >> 6, s = tid & 63;
    for (int g = w; g < n_g; g += 4) {
        float u[aatc::kVqDim];
#pragma unroll
        for (int k = 0; k < aatc::kVqDim; ++k) {
            const int c = H.vq_chan[g][k];
            u[k] = __fmul_rn(xs[s * XS + c], H.vq_scale[c]);
        }
        const uint32_t idx = aatc::vq_nearest(H.vq_cent[g], u[0], u[1], u[2], u[3]);
        if (s >= s0 && s < s1) scatter_code(sg, ptl, g, s, idx);
    }
    __syncthreads();
    uint8_t* tp = tile_ptr(cache, layer, n_seqs_cache, sa.seq[zi], n_kv, h, n_tiles_cap, tile, tile_bytes);
    copy_out<false>(sg, H.BK / 8, (uint32_t*)tp, s0, s1, tid, 256);
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
            const int nt3 = aatc::enc_terms_for(cb->total_bits, d);
            const int64_t units = (int64_t)used * cb->n_kv * 2;
            const size_t lds = d == 64 ? encode_lds_bytes<64>() : encode_lds_bytes<128>();
            const int64_t slots = (int64_t)kCUs * std::min<size_t>(nt3 == 3 ? 2 : 3, kLdsPerCU / lds);  // waves_per_eu
            const unsigned wx = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ntiles, slots / units));
            const dim3 grid(wx, (unsigned)(2 * cb->n_kv), (unsigned)used);
            const int vq = cb->heads[0].vq_groups > 0;
            const dim3 kgrid((unsigned)ntiles, (unsigned)cb->n_kv, (unsigned)used);
            const void* kern = d == 64 ? (nt3 == 3 ? (const void*)encode_mfma_kernel<64, 3> : (const void*)encode_mfma_kernel<64, 2>)
                                       : (nt3 == 3 ? (const void*)encode_mfma_kernel<128, 3> : (const void*)encode_mfma_kernel<128, 2>);
            if (lds > 64 * 1024)
                HIP_TRY(hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
            uint8_t* cdata = (uint8_t*)cache->data;
#define AATC_ENCODE_LAUNCH(D_, T_)                                                                                 \
    hipLaunchKernelGGL((encode_mfma_kernel<D_, T_>), grid, dim3(256), lds, (hipStream_t)stream, blob, cdata, layer, \
                       cb->n_kv, ncap, tile_bytes, sa, n_tokens, ntiles, Kz, Vz, cache->n_seqs, vq)
            if (d == 64) {
                if (nt3 == 3)
                    AATC_ENCODE_LAUNCH(64, 3);
                else
                    AATC_ENCODE_LAUNCH(64, 2);
            } else {
                if (nt3 == 3)
                    AATC_ENCODE_LAUNCH(128, 3);
                else
                    AATC_ENCODE_LAUNCH(128, 2);
            }
#undef AATC_ENCODE_LAUNCH
            if (vq) {
                if (d == 64)
                    hipLaunchKernelGGL(vq_keys_kernel<64>, kgrid, dim3(256), 0, (hipStream_t)stream, blob, cdata, layer,
                                       cb->n_kv, ncap, tile_bytes, sa, n_tokens, Kz, cache->n_seqs);
                else
                    hipLaunchKernelGGL(vq_keys_kernel<128>, kgrid, dim3(256), 0, (hipStream_t)stream, blob, cdata, layer,
                                       cb->n_kv, ncap, tile_bytes, sa, n_tokens, Kz, cache->n_seqs);
            }
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
