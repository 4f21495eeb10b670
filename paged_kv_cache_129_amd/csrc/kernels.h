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
    float* k_scales;            // int8 pools: scale pools [num_blocks][num_kv_heads][block_size]
    float* v_scales;
};
hipError_t launch_kv_write(const WriteArgs& a, int src_dt, int kv_dt, hipStream_t stream);

constexpr int kCopyMaxLayers = 32;        // layers per copy launch (pointers in the arguments)
struct CopyArgs {
    void* k[kCopyMaxLayers];
    void* v[kCopyMaxLayers];
    const int32_t* pairs;       // DEVICE int32 [num_pairs][2] = (src, dst)
    int64_t block_bytes;        // one block of one pool, a multiple of 16
    int32_t num_blocks;         // pairs with an id outside [0, num_blocks) are skipped
    int32_t num_layers;         // <= kCopyMaxLayers
    int32_t num_pairs;
    int32_t slices;             // 4 KiB slices per block (set at launch)
};
hipError_t launch_copy_blocks(CopyArgs& a, hipStream_t stream);

constexpr int kSwapMaxPools = 64;       // pools per swap launch (pointers in the arguments)
struct SwapArgs {
    void* dst[kSwapMaxPools];           // device-visible addresses (device or pinned host)
    const void* src[kSwapMaxPools];
    const int32_t* pairs;               // DEVICE int32 [num_pairs][2] = (src block, dst block)
    int64_t block_bytes;
    int32_t src_blocks, dst_blocks;     // ids outside these pool sizes are skipped
    int32_t num_pools;
    int32_t num_pairs;
    int32_t slices;                     // set at launch
};
hipError_t launch_swap_blocks(SwapArgs& a, hipStream_t stream);

// Sequences are scheduled in windows of kWindow (their metadata is staged in
// LDS).  The balanced schedule gives each worker (a wavefront) two
// partial-record slots and one range descriptor per window; a launch has at
// most kMaxWorkersPerCu workers per CU, so that the workspace can be sized
// before the launch.
constexpr int kWindow = 1024;
constexpr int kDescWords = 6;
// 32 wavefronts per CU at most, each a worker
constexpr int kMaxWorkersPerCu = 32;

// Matrix-core kernels.  Up to 16 query heads per KV head, a wavefront computes
// one 16-head tile of a KV head's query heads (decode_mfma.hip); larger groups
// (multi-query attention among them) take a workgroup per KV head, one
// wavefront per 16-head tile, sharing one load and conversion of K and V
// (decode_group.hip).  Either way a work unit is every query head of a KV head.
constexpr int kMaxGroup = 128;
// workers per CU of a launch at most: wavefronts (per-tile kernel), workgroups
// (group kernel)
constexpr int kMfmaMaxWorkersPerCu = 8;
constexpr int kGroupMaxWorkersPerCu = 4;

struct DecodeArgs {
    const void* q;
    void* out;
    const void* k_pool;
    const void* v_pool;
    const int32_t* tables;
    const int32_t* ctx_lens;
    const float* k_scales;      // int8 cache: one scale per (block, kv head, slot)
    const float* v_scales;
    float* ws;                  // partial records: m[nrec], l[nrec], o[nrec][head_dim]
    int64_t nrec;               // partial records in ws (set with the grid when balanced)
    int64_t rec_capacity;       // balanced: records ws can hold, or -1 (sized for any grid)
    int64_t* desc;              // balanced: kDescWords per (window, worker) for the reduction
    int32_t units;              // work units per sequence (set at launch): a unit is
                                // unit_heads query heads of KV head unit / units_per_kv,
                                // from head (unit % units_per_kv) * unit_heads of its group
    int32_t units_per_kv;
    int32_t unit_heads;
    int32_t workers;            // workers of the attention launch (set at launch)
    int32_t simds;              // SIMDs of the device (set at launch)
    int32_t seg_cost;           // balanced: tokens' worth of cost per segment (set at launch)
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
// Grid of an attention launch with `units` work units per sequence (unit_heads
// and units_per_kv already set), whose workers are wavefronts (wave_workers) or
// workgroups; records the worker count (and, when balanced, the partial-record
// count) in `a`.  Returns -1 when the balanced records would not fit
// a.rec_capacity (the launcher then returns hipErrorOutOfMemory unlaunched).
int64_t decode_grid(const void* kernel, int threads, int units, int wave_workers, DecodeArgs& a,
                    int max_workers_per_cu = kMaxWorkersPerCu);
hipError_t launch_decode(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                         hipStream_t stream);

// Multi-token (prefill / chunked prefill) attention, matrix-core kernel
// (prefill_mfma.hip).  Columns of a (sequence, KV head) item are the pairs
// (query row i, head hl of the KV head's group), column c = i * G + hl.
struct PrefillArgs {
    const void* q;              // [num_query_tokens][num_heads][head_dim]
    void* out;
    const void* k_pool;
    const void* v_pool;
    const int32_t* tables;      // [num_seqs][max_blocks]
    const int32_t* ctx_lens;    // [num_seqs], chunk included
    const int32_t* query_start; // [num_seqs + 1]
    int32_t num_seqs;
    int32_t num_tokens;         // rows of q / out
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t log2_bs;
    int32_t max_query_len;      // rows per sequence the launch covers
    int32_t col_blocks;         // column blocks per (sequence, KV head) (set at launch)
    float qk_scale;             // softmax scale * log2(e) * K dequant factor
    float out_scale;            // V dequant factor
};
bool prefill_supported(int q_dt, int kv_dt, int head_dim);
hipError_t launch_prefill(PrefillArgs& a, int q_dt, int kv_dt, int head_dim, hipStream_t stream);

// matrix-core kernel for grouped heads, 2 <= G <= 16 (decode_mfma.hip)
bool decode_mfma_supported(int q_dt, int kv_dt, int head_dim, int group);
hipError_t launch_decode_mfma(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                              hipStream_t stream);
// matrix-core kernel for large groups, 16 < G <= kMaxGroup (decode_group.hip)
bool decode_group_supported(int q_dt, int kv_dt, int head_dim, int group);
hipError_t launch_decode_group(DecodeArgs& a, int q_dt, int kv_dt, int head_dim,
                               hipStream_t stream);



}  // namespace pa
