// copy_blocks: the data half of copy-on-write.  Before a sequence writes into
// a block that other sequences still use, the block is copied to a fresh one
// and the write goes into the copy (KV 缓存与分页注意力 §08 共用，写时复制).
//
// The (src, dst) pairs are read from device memory, so a captured launch can
// be replayed with the pairs the host writes into the same buffer before each
// step; a pair with an id outside [0, num_blocks) (e.g. -1 padding) or with
// src == dst is skipped.  One workgroup copies a 4 KiB slice of one (pair,
// layer, K|V) block with 16-byte loads and stores; bytes move unchanged.
#include <algorithm>

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

// stream_read: reads a buffer once with the 16-byte streaming loads the decode
// kernels use for K/V (consecutive lanes on consecutive pieces), one workgroup
// per CU, each on a contiguous span, each thread with kReadRing loads in
// flight, and folds every word into one XOR per workgroup so the loads cannot
// be dropped.  It measures the read rate those kernels' HBM rooflines are set
// against on the device at hand.  Measured over 2 GiB, one workgroup of 256
// threads per CU with eight loads per thread was the fastest launch shape
// (7.2 TB/s on one device, 6.5-6.7 TB/s on another); four loads per thread,
// more workgroups per CU, 512 or 1,024 threads or a grid stride were not faster.
constexpr int kReadRing = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* buf, int64_t pieces,
                                                               uint32_t* sink) {
    const int64_t per = (pieces + gridDim.x - 1) / gridDim.x;
    const int64_t base = min(pieces, (int64_t)blockIdx.x * per);
    const int64_t p1 = min(pieces, base + per);             // this workgroup's span ends here
    const int64_t p0 = base + threadIdx.x;                  // the thread's first piece
    // the same non-temporal 16-byte load as load16_stream, kept as a vector so that
    // the folds wait for each load in turn rather than for all eight; loads past the
    // span read the buffer's last piece again (in bounds) and are not folded
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    auto ld = [&](int64_t i) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(buf + min(i, pieces - 1) * 16));
    };
    uint32_t x = 0;
    u32x4 r[kReadRing];
#pragma unroll
    for (int k = 0; k < kReadRing; ++k) r[k] = ld(p0 + k * kThreads);
    for (int64_t i = p0; i < p1; i += kReadRing * kThreads) {
#pragma unroll
        for (int k = 0; k < kReadRing; ++k) {
            const uint32_t f = r[k][0] ^ r[k][1] ^ r[k][2] ^ r[k][3];
            x ^= (i + k * kThreads < p1) ? f : 0u;
            r[k] = ld(i + (k + kReadRing) * kThreads);
        }
    }
#pragma unroll
    for (int k = 0; k < kReadRing; ++k) x += r[k][0] & 0u;   // the last loads are used
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d, 64);
    __shared__ uint32_t wsum[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) y ^= wsum[w];
        sink[blockIdx.x] = y;
    }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t pieces = bytes / 16;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t grid = std::min<int64_t>({(int64_t)cus, (pieces + kThreads - 1) / kThreads,
                                            (int64_t)PA_STREAM_READ_SINK_WORDS});
    hipLaunchKernelGGL(stream_read_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const char*>(buf), pieces, sink);
    return hipGetLastError();
}

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
