// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
// Arguments reaching these launchers have been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct WriteArgs {
    const void* k_new;
    const void* v_new;
    void* k_pool;
    void* v_pool;
    const int64_t* slot_mapping;
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t log2_bs;
    int64_t num_slots;          // num_blocks * block_size
    float k_inv_scale;          // fp32 1/k_scale (fp8 pools)
    float v_inv_scale;
};
hipError_t launch_kv_write(const WriteArgs& a, int src_dt, int kv_dt, hipStream_t stream);

constexpr int kCopyMaxLayers = 32;
constexpr int kCopyMaxPairs = 64;
struct CopyArgs {
    void* k[kCopyMaxLayers];
    void* v[kCopyMaxLayers];
    int32_t src[kCopyMaxPairs];
    int32_t dst[kCopyMaxPairs];
    int64_t block_bytes;        // one block of one pool, a multiple of 16
    int32_t num_layers;         // <= kCopyMaxLayers
    int32_t num_pairs;          // <= kCopyMaxPairs
};
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

struct DecodeArgs {
    const void* q;
    void* out;
    const void* k_pool;
    const void* v_pool;
    const int32_t* tables;
    const int32_t* ctx_lens;
    float* ws;                  // partials when num_parts > 1
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t max_blocks;
    int32_t ctx_cap;            // min(max_context_len, max_blocks * block_size)
    int32_t num_blocks;
    int32_t log2_bs;
    int32_t part_tokens;        // tokens per partition (>= ctx_cap for a single pass)
    int32_t num_parts;          // partitions per (sequence, head) in the launch grid
    float qk_scale;             // softmax scale * log2(e) * K dequant factor
    float out_scale;            // V dequant factor
};
hipError_t launch_decode(const DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                         hipStream_t stream);

// matrix-core kernel for grouped heads (decode_mfma.hip)
bool decode_mfma_supported(int q_dt, int kv_dt, int head_dim, int group);
hipError_t launch_decode_mfma(const DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                              hipStream_t stream);

// matrix-core kernel for large groups, G > 16 (decode_mqa.hip)
bool decode_mqa_supported(int q_dt, int kv_dt, int head_dim, int group);
hipError_t launch_decode_mqa(const DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                             hipStream_t stream);

}  // namespace pa
