// copy_blocks: the data half of copy-on-write.  Before a sequence writes into
// a block that other sequences still use, the block is copied to a fresh one
// and the write goes into the copy (KV 缓存与分页注意力 §08 共用，写时复制).
// One workgroup copies a 4 KiB slice of one (pair, layer, K|V) block with
// 16-byte loads and stores; bytes move unchanged.
#include "kernels.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kSliceBytes = kThreads * 16;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyArgs a) {
    const int pair = blockIdx.y;
    const int layer = blockIdx.z >> 1;
    const int is_v = blockIdx.z & 1;
    const int64_t off = (int64_t)blockIdx.x * kSliceBytes + threadIdx.x * 16;
    if (off >= a.block_bytes) return;
    char* pool = reinterpret_cast<char*>(is_v ? a.v[layer] : a.k[layer]);
    const Raw16 r = load16(pool + (int64_t)a.src[pair] * a.block_bytes + off);
    store16(pool + (int64_t)a.dst[pair] * a.block_bytes + off, r);
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
    const int64_t slices = (a.block_bytes + kSliceBytes - 1) / kSliceBytes;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)slices, a.num_pairs, a.num_layers * 2),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
