// stream_copy.hip -- a calibration copy for gfx950.
//
// A memory-bound kernel pays a DRAM read, a DRAM write and a launch (FlashRT
// "optimization details", the fused-ops overview).  This kernel pays exactly
// those and does no arithmetic, so its time at a byte count is the floor that
// the fused kernels moving the same bytes are measured against.  It streams
// with the same nontemporal 16-byte buffer loads and stores as they do.
//
// Block b (256 lanes) owns the 256 * C consecutive 16-byte chunks from
// b * 256 * C; lane t takes chunks t, t + 256, ... so every load instruction
// of a wave covers 1 KiB of consecutive bytes.  All C loads are issued before
// the first store; with SYNC the block also waits, at a barrier, until all
// its loads have landed before any wave stores, which keeps a block's reads
// and writes apart (faster at some sizes: 14.8 MB 3.58 -> 3.42 us, 29.6 MB
// 6.22 -> 5.77 us at eight chunks per lane).  The block's buffer resource
// ends at the copy's last byte: chunks past it read zeros and their stores
// are dropped by the hardware's range check, so the ragged last block needs
// no branch.

#include "mbt_device.hpp"
#include "mbt_launch.hpp"

namespace mbt {
namespace {

constexpr int kCopyLanes = 256;

template <int C, bool SYNC>
__global__ __launch_bounds__(kCopyLanes) void stream_copy(const char* __restrict__ src,
                                                          char* __restrict__ dst,
                                                          int64_t nbytes) {
    constexpr int64_t span = (int64_t)kCopyLanes * C * 16;
    const int64_t base = (int64_t)blockIdx.x * span;
    const int64_t left = nbytes - base;
    const uint32_t bytes = (uint32_t)(left < span ? left : span);
    const auto rs = buf_rsrc(const_cast<char*>(src) + base, bytes);
    const auto rd = buf_rsrc(dst + base, bytes);
    u32x4 v[C];
#pragma unroll
    for (int k = 0; k < C; ++k)
        v[k] = buf_ld16_nt(rs, (uint32_t)(k * kCopyLanes + (int)threadIdx.x) * 16u);
    if constexpr (SYNC) {
        // the barrier alone would only wait for the loads to be issued (a
        // workgroup fence waits for stores, not for loads into registers)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < C; ++k)
        buf_st16_nt(rd, (uint32_t)(k * kCopyLanes + (int)threadIdx.x) * 16u, v[k]);
}

template <int C>
hipError_t launch_c(const void* src, void* dst, int64_t nbytes, bool sync, hipStream_t s) {
    constexpr int64_t span = (int64_t)kCopyLanes * C * 16;
    const int64_t blocks = (nbytes + span - 1) / span;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (sync)
        hipLaunchKernelGGL((stream_copy<C, true>), dim3((uint32_t)blocks), dim3(kCopyLanes), 0,
                           s, (const char*)src, (char*)dst, nbytes);
    else
        hipLaunchKernelGGL((stream_copy<C, false>), dim3((uint32_t)blocks), dim3(kCopyLanes), 0,
                           s, (const char*)src, (char*)dst, nbytes);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t nbytes, int chunks,
                              bool block_sync, hipStream_t s) {
    if (nbytes <= 0) return hipSuccess;
    switch (chunks) {
    case 1: return launch_c<1>(src, dst, nbytes, block_sync, s);
    case 2: return launch_c<2>(src, dst, nbytes, block_sync, s);
    case 4: return launch_c<4>(src, dst, nbytes, block_sync, s);
    case 8: return launch_c<8>(src, dst, nbytes, block_sync, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mbt
