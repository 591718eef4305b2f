// Read-bandwidth probe: the rate at which one launch can stream a buffer from HBM, measured
// the way the decode kernel is ("Spend Bits Where Queries Look", abstract: decoding reads the
// whole cache every step, so its speed is set by memory bandwidth).  Two forms:
//   mode 0 - plain register loads, 16 bytes per lane, eight in flight per lane (1024
//            workgroups of 256 threads, each a contiguous chunk, non-temporal hint);
//   mode 1 - the decode kernel's stream: tiles of tile_bytes bytes copied straight into LDS
//            (buffer loads, non-temporal hint), one 768-thread workgroup per CU taking an even
//            share of the tiles, its waves every 12th tile, two ring slots per wave.
// The loaded data is folded into a checksum that is stored only if it equals a value no
// real input produces, so the loads cannot be dropped and nothing is written.
#include <hip/hip_runtime.h>

#include "hip_common.h"

using aatc::set_error;

namespace {

#define LDS_AS __attribute__((address_space(3)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kNever = 0x9E3779B9u;  // checksum value that triggers the (never taken) store
constexpr int kRegBlocks = 1024, kRegThreads = 256, kRegUnroll = 8;
constexpr int kLdsWaves = 12, kLdsRing = 2, kLdsBlocks = 256;

__global__ __launch_bounds__(kRegThreads) void probe_reg_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                uint32_t* __restrict__ sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = blockIdx.x * per, b1 = min(n16, b0 + per);
    uint32_t acc = 0;
    for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)kRegThreads * kRegUnroll) {
        u32x4 v[kRegUnroll];
#pragma unroll
        for (int u = 0; u < kRegUnroll; ++u) {
            const size_t j = i + (size_t)u * kRegThreads;
            v[u] = j < b1 ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kRegUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == kNever) sink[0] = acc;
}

__device__ __forceinline__ void wait_vm_at_most(int n) {
    switch (n) {
#define AATC_W(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        AATC_W(0) AATC_W(1) AATC_W(2) AATC_W(3) AATC_W(4) AATC_W(5) AATC_W(6) AATC_W(7) AATC_W(8) AATC_W(9)
        AATC_W(10) AATC_W(11) AATC_W(12) AATC_W(13) AATC_W(14) AATC_W(15) AATC_W(16) AATC_W(17) AATC_W(18)
        AATC_W(19) AATC_W(20) AATC_W(21) AATC_W(22) AATC_W(23) AATC_W(24) AATC_W(25) AATC_W(26) AATC_W(27)
        AATC_W(28) AATC_W(29) AATC_W(30) AATC_W(31)
#undef AATC_W
        default: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    }
}

// tiles of TB bytes (a multiple of 64: n16 loads of 16 bytes per lane, then r4 of 4)
__global__ __launch_bounds__(64 * kLdsWaves) void probe_lds_kernel(const uint8_t* __restrict__ p, int64_t n_tiles,
                                                                   int TB, int n16, int r4,
                                                                   uint32_t* __restrict__ sink) {
    extern __shared__ __attribute__((aligned(16))) uint8_t probe_smem[];
    LDS_AS uint8_t* sm = (LDS_AS uint8_t*)probe_smem;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int BB = (TB + 15) & ~15;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)min<int64_t>(n_tiles * TB, 0x7FFFFFFF), 0x00020000);
    const int64_t t0 = n_tiles * blockIdx.x / gridDim.x, t1 = n_tiles * (blockIdx.x + 1) / gridDim.x;
    const int nl = n16 + r4;
    auto issue = [&](int64_t t, int slot) {
        LDS_AS uint8_t* l = sm + (slot * kLdsWaves + w) * BB;
        uint32_t off = (uint32_t)(t * TB);
        for (int k = 0; k < n16; ++k, off += 1024)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(l + 1024 * k), 16, 16 * lane, off, 0, 2);
        for (int k = 0; k < r4; ++k, off += 256)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(l + 1024 * n16 + 256 * k), 4, 4 * lane, off, 0,
                                                     2);
    };
    int issued = 0;
    int64_t t = t0 + w;
    for (; issued < kLdsRing && t + (int64_t)kLdsWaves * issued < t1; ++issued)
        issue(t + (int64_t)kLdsWaves * issued, issued);
    uint32_t acc = 0;
    int slot = 0;
    for (int done = 0; t < t1; t += kLdsWaves, ++done) {
        wait_vm_at_most(nl * (issued - done - 1));
        LDS_AS uint8_t* l = sm + (slot * kLdsWaves + w) * BB;
        acc ^= ((LDS_AS uint32_t*)l)[lane];
        const int64_t tn = t + (int64_t)kLdsWaves * kLdsRing;
        if (tn < t1) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue(tn, slot);
            ++issued;
        }
        slot = slot + 1 == kLdsRing ? 0 : slot + 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (acc == kNever) sink[0] = acc;
}

}  // namespace

extern "C" int aatc_read_probe(const void* d_src, size_t bytes, int32_t mode, int32_t tile_bytes, void* d_sink,
                               void* stream) {
    if (!d_src || !d_sink) return set_error(AATC_ERR_INVALID_ARG, "null buffer");
    if ((((uintptr_t)d_src) | ((uintptr_t)d_sink)) & 15)
        return set_error(AATC_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    if (mode == 0) {
        const size_t n16 = bytes / 16;
        if (n16 == 0) return AATC_OK;
        hipLaunchKernelGGL(probe_reg_kernel, dim3(kRegBlocks), dim3(kRegThreads), 0, st, (const u32x4*)d_src, n16,
                           (uint32_t*)d_sink);
        HIP_TRY(hipGetLastError());
        return AATC_OK;
    }
    if (mode != 1) return set_error(AATC_ERR_INVALID_ARG, "mode must be 0 (register loads) or 1 (tiles into LDS)");
    // two ring slots of 12 waves in 160 KiB of LDS; 4-byte remainder loads per lane
    if (tile_bytes < 256 || tile_bytes % 256 || tile_bytes > 6656)
        return set_error(AATC_ERR_INVALID_ARG, "tile_bytes must be a multiple of 256 in [256, 6656]");
    const int lane_bytes = tile_bytes / 64;
    const int n16 = lane_bytes / 16, r4 = (lane_bytes % 16) / 4;
    const int64_t n_tiles = (int64_t)(bytes / tile_bytes);
    if (n_tiles == 0) return AATC_OK;
    if (n_tiles * tile_bytes >= ((int64_t)1 << 31)) return set_error(AATC_ERR_CAPACITY, "at most 2^31 - 1 bytes");
    const int lds = kLdsRing * kLdsWaves * ((tile_bytes + 15) & ~15);
    HIP_TRY(hipFuncSetAttribute((const void*)probe_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    hipLaunchKernelGGL(probe_lds_kernel, dim3(kLdsBlocks), dim3(64 * kLdsWaves), lds, st, (const uint8_t*)d_src, n_tiles,
                       tile_bytes, n16, r4, (uint32_t*)d_sink);
    HIP_TRY(hipGetLastError());
    return AATC_OK;
}
