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

// Sequences are scheduled in windows of kWindow (their metadata is staged in
// LDS).  The balanced schedule gives each worker (a wavefront or a workgroup)
// two partial-record slots and one range descriptor per window; a launch has
// at most balanced_workers_per_cu(group) workers per CU, so that the workspace
// can be sized before the kernel is chosen.
constexpr int kWindow = 1024;
constexpr int kDescWords = 6;
// 32 wavefronts per CU at most; the large-group kernel's workers are
// workgroups of at least two wavefronts
__host__ __device__ constexpr int balanced_workers_per_cu(int group) { return group > 16 ? 16 : 32; }

struct DecodeArgs {
    const void* q;
    void* out;
    const void* k_pool;
    const void* v_pool;
    const int32_t* tables;
    const int32_t* ctx_lens;
    float* ws;                  // partial records: m[nrec], l[nrec], o[nrec][head_dim]
    int64_t nrec;               // partial records in ws (set with the grid when balanced)
    int64_t* desc;              // balanced: 4 words per (window, workgroup) for the reduction
    int32_t units;              // work units per sequence: query heads or KV heads (set at launch)
    int32_t workers;            // workers of the attention launch (set at launch)
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t max_blocks;
    int32_t ctx_cap;            // min(max_context_len, max_blocks * block_size)
    int32_t num_blocks;
    int32_t log2_bs;
    int32_t part_tokens;        // tokens per partition (>= ctx_cap for a single pass);
                                // negative: balanced split
    int32_t num_parts;          // partitions per (sequence, head); 1 when balanced
    float qk_scale;             // softmax scale * log2(e) * K dequant factor
    float out_scale;            // V dequant factor
};

// compute units of the current device (cached per device)
int device_cus();
// Grid of an attention launch with `units` work units per sequence, whose
// workers are wavefronts (wave_workers) or workgroups; records the worker
// count (and, when balanced, the partial-record count) in `a`.
int64_t decode_grid(const void* kernel, int threads, int units, int wave_workers, DecodeArgs& a);
hipError_t launch_decode(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                         hipStream_t stream);

// matrix-core kernel for grouped heads (decode_mfma.hip)
bool decode_mfma_supported(int q_dt, int kv_dt, int head_dim, int group);
hipError_t launch_decode_mfma(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                              hipStream_t stream);

// matrix-core kernel for large groups, G > 16 (decode_mqa.hip)
bool decode_mqa_supported(int q_dt, int kv_dt, int head_dim, int group);
hipError_t launch_decode_mqa(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                             hipStream_t stream);

}  // namespace pa
