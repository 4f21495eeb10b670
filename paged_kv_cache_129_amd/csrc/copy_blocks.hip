// copy_blocks: the data half of copy-on-write.  Before a sequence writes into
// a block that other sequences still use, the block is copied to a fresh one
// and the write goes into the copy (KV 缓存与分页注意力 §08 共用，写时复制).
//
// The (src, dst) pairs are read from device memory, so a captured launch can
// be replayed with the pairs the host writes into the same buffer before each
// step; a pair with an id outside [0, num_blocks) (e.g. -1 padding) or with
// src == dst is skipped.  One workgroup copies a 4 KiB slice of one (pair,
// layer, K|V) block with 16-byte loads and stores; bytes move unchanged.
#include "kernels.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kSliceBytes = kThreads * 16;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyArgs a) {
    // blockIdx.x = pair * slices + slice; blockIdx.y = 2 * layer + (V ? 1 : 0)
    const int64_t pair = (int64_t)blockIdx.x / a.slices;
    const int64_t slice = (int64_t)blockIdx.x - pair * a.slices;
    const int layer = blockIdx.y >> 1;
    const int is_v = blockIdx.y & 1;
    const int64_t off = slice * kSliceBytes + threadIdx.x * 16;
    // both ids of the pair in one 8-byte load, the same for the whole workgroup
    const int2 pr = *reinterpret_cast<const int2*>(a.pairs + 2 * pair);
    const int src = __builtin_amdgcn_readfirstlane(pr.x);
    const int dst = __builtin_amdgcn_readfirstlane(pr.y);
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst) return;
    if (off >= a.block_bytes) return;
    char* pool = reinterpret_cast<char*>(is_v ? a.v[layer] : a.k[layer]);
    const Raw16 r = load16(pool + (int64_t)src * a.block_bytes + off);
    store16(pool + (int64_t)dst * a.block_bytes + off, r);
}

// swap_blocks: a preempted sequence's blocks moved between device pools and
// pools in pinned host memory (KV 缓存与分页注意力 §09 放不下的时候): block s of
// every source pool to block d of the matching destination pool, bytes
// unchanged.  One side is read or written across the host link.
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(SwapArgs a) {
    const int64_t pair = (int64_t)blockIdx.x / a.slices;
    const int64_t slice = (int64_t)blockIdx.x - pair * a.slices;
    const int pool = blockIdx.y;
    const int64_t off = slice * kSliceBytes + threadIdx.x * 16;
    const int2 pr = *reinterpret_cast<const int2*>(a.pairs + 2 * pair);
    const int src = __builtin_amdgcn_readfirstlane(pr.x);
    const int dst = __builtin_amdgcn_readfirstlane(pr.y);
    if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
    if (off >= a.block_bytes) return;
    const char* sp = reinterpret_cast<const char*>(a.src[pool]) + (int64_t)src * a.block_bytes + off;
    char* dp = reinterpret_cast<char*>(a.dst[pool]) + (int64_t)dst * a.block_bytes + off;
    store16(dp, load16(sp));
}

}  // namespace

hipError_t launch_swap_blocks(SwapArgs& a, hipStream_t stream) {
    a.slices = (int32_t)((a.block_bytes + kSliceBytes - 1) / kSliceBytes);
    const int64_t wgs = (int64_t)a.num_pairs * a.slices;
    if (wgs <= 0 || wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(swap_blocks_kernel, dim3((uint32_t)wgs, a.num_pools), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(CopyArgs& a, hipStream_t stream) {
    a.slices = (int32_t)((a.block_bytes + kSliceBytes - 1) / kSliceBytes);
    const int64_t wgs = (int64_t)a.num_pairs * a.slices;
    if (wgs <= 0 || wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)wgs, a.num_layers * 2), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace pa
