// C-ABI entry points: argument validation (host, before anything is
// enqueued), then dispatch to the gfx950 kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>

#include "kernels.h"
#include "pa_device.h"
#include "pagedattn.h"

namespace {

bool valid_dtype(int32_t dt) { return dt >= PA_F32 && dt <= PA_INT8; }

int log2_exact(int32_t v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

thread_local char g_last_error[256] = "";

// Launch through `fn` after clearing any error an earlier, unrelated runtime
// call left behind, so that only this launch's own failure is reported.
template <typename F>
pa_status launch_checked(F&& fn) {
    (void)hipGetLastError();
    g_last_error[0] = 0;
    const hipError_t e = fn();
    if (e == hipSuccess) return PA_OK;
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return PA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t num_partitions(int32_t ctx_cap, int32_t partition_size) {
    if (partition_size <= 0 || ctx_cap <= 0) return 1;
    return ((int64_t)ctx_cap + partition_size - 1) / partition_size;
}

size_t partial_bytes(int64_t num_seqs, int64_t num_heads, int64_t head_dim, int64_t parts) {
    if (parts <= 1) return 0;
    const size_t b = (size_t)num_seqs * num_heads * parts * (size_t)(head_dim + 2) * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Balanced split: partial records for two slots per (window, worker) and the
// workers' range descriptors, for the most workers a launch can have on the
// current device: per CU, kMaxWorkersPerCu one-head workers (per-head kernel),
// or kMfmaMaxWorkersPerCu / kGroupMaxWorkersPerCu workers of unit_heads heads
// (matrix-core kernels, groups of up to / beyond 16), whichever needs more.
size_t balanced_record_bytes(int64_t num_seqs, int64_t unit_heads, int64_t head_dim) {
    const int64_t windows = (num_seqs + pa::kWindow - 1) / pa::kWindow;
    const int64_t per_cu = unit_heads > 16 ? pa::kGroupMaxWorkersPerCu : pa::kMfmaMaxWorkersPerCu;
    const int64_t slots_per_cu = std::max<int64_t>((int64_t)pa::kMaxWorkersPerCu, per_cu * unit_heads);
    const int64_t slots = (int64_t)pa::device_cus() * slots_per_cu;
    return round256((size_t)(windows * slots * 2) * (size_t)(head_dim + 2) * sizeof(float));
}
size_t balanced_desc_bytes(int64_t num_seqs) {
    const int64_t windows = (num_seqs + pa::kWindow - 1) / pa::kWindow;
    const int64_t workers = (int64_t)pa::device_cus() * pa::kMaxWorkersPerCu;
    return round256((size_t)(windows * workers) * pa::kDescWords * sizeof(int64_t));
}

// record slots per work unit: all G query heads of a KV head when a
// matrix-core kernel may run (2 <= G <= kMaxGroup), else one head (per-head
// kernel); an upper bound whichever kernel the data types select
int64_t unit_group(int32_t num_heads, int32_t num_kv_heads) {
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return 1;
    const int g = num_heads / num_kv_heads;
    return g >= 2 && g <= pa::kMaxGroup ? g : 1;
}

}  // namespace

extern "C" {

const char* pa_status_string(int32_t status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_OUT_OF_BLOCKS: return "Out of KV cache blocks";
        case PA_ERR_INDEX: return "index out of range";
        case PA_ERR_UNKNOWN_SEQ: return "unknown sequence id";
        case PA_ERR_REFCOUNT: return "reference count error";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_EXISTS: return "sequence id already exists";
        default: return "unknown status";
    }
}

const char* pa_version(void) { return "libpagedattn 0.1 gfx950"; }

const char* pa_last_error(void) { return g_last_error; }

int64_t pa_kv_bytes_per_token(int32_t num_kv_heads, int32_t head_dim, int32_t num_layers,
                              int32_t dtype) {
    if (num_kv_heads <= 0 || head_dim <= 0 || num_layers <= 0 || !valid_dtype(dtype)) return -1;
    const int64_t per_head = (int64_t)head_dim * pa::elem_bytes(dtype) +
                             (dtype == PA_INT8 ? (int64_t)sizeof(float) : 0);   // + the scale
    return 2 * (int64_t)num_kv_heads * num_layers * per_head;
}

pa_status pa_kv_cache_write(const void* k_new, const void* v_new, int32_t src_dtype,
                            void* k_pool, void* v_pool, int32_t kv_dtype,
                            const int64_t* slot_mapping, int32_t num_tokens,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float k_scale, float v_scale, void* stream) {
    if (!valid_dtype(src_dtype) || !valid_dtype(kv_dtype)) return PA_ERR_INVALID_ARG;
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    const int lbs = log2_exact(block_size);
    if (lbs < 0 || lbs > 8) return PA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
    if (src_dtype == PA_INT8 || kv_dtype == PA_INT8) return PA_ERR_UNSUPPORTED;   // scale pools
    const bool quantise = kv_dtype == PA_FP8_E4M3 && src_dtype != PA_FP8_E4M3;
    if (src_dtype != kv_dtype && !quantise) return PA_ERR_UNSUPPORTED;
    if (quantise && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) &&
                      v_scale > 0.0f))
        return PA_ERR_INVALID_ARG;
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_INVALID_ARG;
    pa::WriteArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.log2_bs = lbs;
    a.num_slots = (int64_t)num_blocks * block_size;
    a.k_inv_scale = quantise ? 1.0f / k_scale : 1.0f;     // IEEE fp32 division
    a.v_inv_scale = quantise ? 1.0f / v_scale : 1.0f;
    return launch_checked([&] { return pa::launch_kv_write(a, src_dtype, kv_dtype, as_stream(stream)); });
}

pa_status pa_kv_cache_write_int8(const void* k_new, const void* v_new, int32_t src_dtype,
                                 void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, void* stream) {
    if (src_dtype != PA_F32 && src_dtype != PA_F16 && src_dtype != PA_BF16)
        return valid_dtype(src_dtype) ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARG;
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    const int lbs = log2_exact(block_size);
    if (lbs < 0 || lbs > 8) return PA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_tokens * num_kv_heads > ((int64_t)1 << 33)) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scales || !v_scales || !slot_mapping)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (reinterpret_cast<uintptr_t>(k_scales) & 3u) || (reinterpret_cast<uintptr_t>(v_scales) & 3u))
        return PA_ERR_INVALID_ARG;
    pa::WriteArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.log2_bs = lbs;
    a.num_slots = (int64_t)num_blocks * block_size;
    return launch_checked([&] { return pa::launch_kv_write(a, src_dtype, PA_INT8, as_stream(stream)); });
}

size_t pa_paged_attention_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_context_len,
                                         int32_t partition_size) {
    if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || (partition_size < 0 && partition_size != PA_PARTITION_BALANCED))
        return 0;
    if (partition_size == PA_PARTITION_BALANCED)
        return balanced_record_bytes(num_seqs, unit_group(num_heads, num_kv_heads), head_dim) +
               balanced_desc_bytes(num_seqs);
    return partial_bytes(num_seqs, num_heads, head_dim,
                         num_partitions(max_context_len, partition_size));
}

}  // extern "C"

// Scratch of the allocation-free decode entry point (see scratch_ptr below).
static __device__ __attribute__((aligned(256))) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

// ---------------------------------------------------------------- static scratch
// The allocation-free decode entry point keeps its partial records and range
// descriptors here: a file-scope device array, one copy per GPU, alive until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in symbol); it asks the runtime for the array's
// address on each device once and uses that address.
constexpr size_t kScratchBytes = (size_t)PA_NOALLOC_SCRATCH_BYTES;

// Address of `scratch` on the current device (looked up once per device, with
// that device current), or NULL if the runtime cannot give it.
void* scratch_ptr() {
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> g(mu);
    auto it = ptrs.find(dev);
    if (it != ptrs.end()) return it->second;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        snprintf(g_last_error, sizeof(g_last_error), "hipGetSymbolAddress(scratch): %s",
                 hipGetErrorString(e));
        return nullptr;
    }
    ptrs.emplace(dev, p);
    return p;
}

pa_status decode_impl(void* out, const void* q, int32_t q_dtype,
                                    const void* k_pool, const void* v_pool, int32_t kv_dtype,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    float scale, float k_scale, float v_scale,
                                    const float* k_scales, const float* v_scales,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, bool use_scratch, void* stream) {
    if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype)) return PA_ERR_INVALID_ARG;
    // int8 caches come with their scale pools (pa_paged_attention_decode_int8) and only then
    if ((kv_dtype == PA_INT8) != (k_scales != nullptr)) return PA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
        (partition_size < 0 && partition_size != PA_PARTITION_BALANCED))
        return PA_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    const int lbs = log2_exact(block_size);
    if (lbs < 0 || lbs > 8) return PA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    if (q_dtype == PA_FP8_E4M3 || q_dtype == PA_INT8) return PA_ERR_UNSUPPORTED;
    if (kv_dtype != q_dtype && kv_dtype != PA_FP8_E4M3 && kv_dtype != PA_INT8)
        return PA_ERR_UNSUPPORTED;
    if (kv_dtype == PA_FP8_E4M3 && !(std::isfinite(k_scale) && k_scale > 0.0f &&
                                     std::isfinite(v_scale) && v_scale > 0.0f))
        return PA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_INVALID_ARG;
    if (kv_dtype == PA_INT8 && (!v_scales || (reinterpret_cast<uintptr_t>(k_scales) & 3u) ||
                                (reinterpret_cast<uintptr_t>(v_scales) & 3u)))
        return PA_ERR_INVALID_ARG;

    const int64_t cap64 = std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq << lbs);
    const int32_t ctx_cap = (int32_t)std::min<int64_t>(cap64, INT32_MAX);
    const bool balanced = partition_size == PA_PARTITION_BALANCED;
    const int64_t parts = balanced ? 1 : num_partitions(ctx_cap, partition_size);
    if ((int64_t)num_seqs * num_heads * parts >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    size_t rec_bytes =
        balanced ? balanced_record_bytes(num_seqs, unit_group(num_heads, num_kv_heads), head_dim)
                 : partial_bytes(num_seqs, num_heads, head_dim, parts);
    int64_t rec_capacity = -1;                            // records: sized for any grid
    if (use_scratch) {
        // the library's own per-device scratch: records from its start, the
        // balanced split's range descriptors at its end; the balanced records
        // are checked against what remains once the grid is known
        if (!rec_bytes && !balanced) {
            workspace = nullptr;
        } else {
            workspace = scratch_ptr();
            if (!workspace) return PA_ERR_HIP;
            const size_t desc_bytes = balanced ? balanced_desc_bytes(num_seqs) : 0;
            if (desc_bytes >= kScratchBytes || (!balanced && rec_bytes > kScratchBytes))
                return PA_ERR_WORKSPACE;
            if (balanced) {
                rec_bytes = kScratchBytes - desc_bytes;
                rec_capacity = (int64_t)(rec_bytes / ((size_t)(head_dim + 2) * sizeof(float)));
            }
        }
    } else {
        const size_t need = rec_bytes + (balanced ? balanced_desc_bytes(num_seqs) : 0);
        if (need > 0 && (!workspace || workspace_bytes < need ||
                         (reinterpret_cast<uintptr_t>(workspace) & 255u)))
            return PA_ERR_WORKSPACE;
    }

    pa::DecodeArgs a{};
    a.q = q;
    a.out = out;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.tables = block_tables;
    a.ctx_lens = context_lens;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.ws = reinterpret_cast<float*>(workspace);
    a.nrec = (int64_t)num_seqs * num_heads * parts;     // balanced: set with the grid
    a.rec_capacity = rec_capacity;
    a.desc = balanced ? reinterpret_cast<int64_t*>(reinterpret_cast<char*>(workspace) + rec_bytes)
                      : nullptr;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.ctx_cap = ctx_cap;
    a.num_blocks = num_blocks;
    a.log2_bs = lbs;
    a.num_parts = (int32_t)parts;
    a.part_tokens = balanced ? -1 : (parts > 1 ? partition_size : std::max<int32_t>(ctx_cap, 1));
    const float kfac = kv_dtype == PA_FP8_E4M3 ? k_scale * pa::dequant_factor(kv_dtype) : 1.0f;
    const float vfac = kv_dtype == PA_FP8_E4M3 ? v_scale * pa::dequant_factor(kv_dtype) : 1.0f;
    a.qk_scale = scale * pa::kLog2e * kfac;
    a.out_scale = vfac;
    const pa_status st = launch_checked(
        [&] { return pa::launch_decode(a, q_dtype, kv_dtype, head_dim, as_stream(stream)); });
    // the records of the chosen grid did not fit the scratch (nothing launched)
    if (st == PA_ERR_HIP && rec_capacity >= 0 && a.nrec > rec_capacity) return PA_ERR_WORKSPACE;
    return st;
}

}  // namespace

namespace pa {
// the streaming-read probe's launcher (copy_blocks.hip); not part of the decode path
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
}  // namespace pa

extern "C" {

pa_status pa_paged_attention_decode(void* out, const void* q, int32_t q_dtype,
                                    const void* k_pool, const void* v_pool, int32_t kv_dtype,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    float scale, float k_scale, float v_scale,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, scale, k_scale, v_scale, nullptr, nullptr,
                       partition_size, workspace, workspace_bytes, false, stream);
}

pa_status pa_paged_attention_decode_int8(void* out, const void* q, int32_t q_dtype,
                                         const void* k_pool, const void* v_pool,
                                         const float* k_scales, const float* v_scales,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         int32_t num_seqs, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t num_blocks, float scale,
                                         int32_t partition_size, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (!k_scales) return PA_ERR_INVALID_ARG;
    return decode_impl(out, q, q_dtype, k_pool, v_pool, PA_INT8, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, scale, 1.0f, 1.0f, k_scales, v_scales,
                       partition_size, workspace, workspace_bytes, false, stream);
}

pa_status pa_paged_attention_decode_noalloc(void* out, const void* q, int32_t q_dtype,
                                            const void* k_pool, const void* v_pool,
                                            int32_t kv_dtype, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t max_context_len,
                                            int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t num_blocks, float scale,
                                            float k_scale, float v_scale, int32_t partition_size,
                                            void* stream) {
    return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, scale, k_scale, v_scale, nullptr, nullptr,
                       partition_size, nullptr, 0, true, stream);
}

// device-visible address of a pool: device memory as is, pinned host memory
// (allocated or registered with HIP) through its device mapping; NULL for
// anything else, pageable host memory included, which a kernel must not touch
static void* device_view(const void* p) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeHost) return nullptr;
    return attr.devicePointer;
}

pa_status pa_swap_blocks(void* const* dst_pools, const void* const* src_pools, int32_t num_pools,
                         int64_t block_bytes, int32_t dst_num_blocks, int32_t src_num_blocks,
                         const int32_t* pairs, int32_t num_pairs, void* stream) {
    if (num_pools < 0 || num_pairs < 0 || block_bytes <= 0 || dst_num_blocks <= 0 ||
        src_num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
    if (num_pools == 0 || num_pairs == 0) return PA_OK;
    if (!dst_pools || !src_pools || !pairs || (reinterpret_cast<uintptr_t>(pairs) & 7u))
        return PA_ERR_INVALID_ARG;
    if ((block_bytes + 4095) / 4096 * (int64_t)num_pairs > INT32_MAX) return PA_ERR_UNSUPPORTED;
    for (int32_t p0 = 0; p0 < num_pools; p0 += pa::kSwapMaxPools) {
        pa::SwapArgs a{};
        a.pairs = pairs;
        a.block_bytes = block_bytes;
        a.src_blocks = src_num_blocks;
        a.dst_blocks = dst_num_blocks;
        a.num_pairs = num_pairs;
        a.num_pools = std::min(num_pools - p0, pa::kSwapMaxPools);
        for (int32_t l = 0; l < a.num_pools; ++l) {
            void* d = dst_pools[p0 + l] ? device_view(dst_pools[p0 + l]) : nullptr;
            const void* sv = src_pools[p0 + l] ? device_view(src_pools[p0 + l]) : nullptr;
            if (!d || !sv || !aligned16(d) || !aligned16(sv)) return PA_ERR_INVALID_ARG;
            a.dst[l] = d;
            a.src[l] = sv;
        }
        const pa_status st =
            launch_checked([&] { return pa::launch_swap_blocks(a, as_stream(stream)); });
        if (st != PA_OK) return st;
    }
    return PA_OK;
}

pa_status pa_paged_attention_prefill(void* out, const void* q, int32_t q_dtype,
                                     const void* k_pool, const void* v_pool, int32_t kv_dtype,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, const int32_t* query_start,
                                     int32_t num_seqs, int32_t num_query_tokens,
                                     int32_t max_query_len, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, float scale, void* stream) {
    if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype)) return PA_ERR_INVALID_ARG;
    if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || num_heads <= 0 ||
        num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    const int lbs = log2_exact(block_size);
    if (lbs < 0 || lbs > 8) return PA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    if (!pa::prefill_supported(q_dtype, kv_dtype, head_dim)) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_INVALID_ARG;
    pa::PrefillArgs a{};
    a.q = q;
    a.out = out;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.tables = block_tables;
    a.ctx_lens = context_lens;
    a.query_start = query_start;
    a.num_seqs = num_seqs;
    a.num_tokens = num_query_tokens;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.log2_bs = lbs;
    a.max_query_len = max_query_len;
    a.qk_scale = scale * pa::kLog2e;
    a.out_scale = 1.0f;
    return launch_checked(
        [&] { return pa::launch_prefill(a, q_dtype, kv_dtype, head_dim, as_stream(stream)); });
}

pa_status pa_copy_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                         int32_t kv_dtype, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, const int32_t* pairs,
                         int32_t num_pairs, void* stream) {
    if (!valid_dtype(kv_dtype) || num_layers < 0 || num_pairs < 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    const int lbs = log2_exact(block_size);
    if (lbs < 0 || lbs > 8) return PA_ERR_INVALID_ARG;
    const int64_t block_bytes =
        (int64_t)num_kv_heads * block_size * head_dim * pa::elem_bytes(kv_dtype);
    if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
    if (num_layers == 0 || num_pairs == 0) return PA_OK;
    if (!k_pools || !v_pools || !pairs || (reinterpret_cast<uintptr_t>(pairs) & 7u))
        return PA_ERR_INVALID_ARG;
    for (int32_t l = 0; l < num_layers; ++l)
        if (!k_pools[l] || !v_pools[l] || !aligned16(k_pools[l]) || !aligned16(v_pools[l]))
            return PA_ERR_INVALID_ARG;
    const int64_t slices = (block_bytes + 4095) / 4096;
    if ((int64_t)num_pairs * slices > INT32_MAX) return PA_ERR_UNSUPPORTED;

    for (int32_t l0 = 0; l0 < num_layers; l0 += pa::kCopyMaxLayers) {
        pa::CopyArgs a{};
        a.pairs = pairs;
        a.block_bytes = block_bytes;
        a.num_blocks = num_blocks;
        a.num_pairs = num_pairs;
        a.num_layers = std::min(num_layers - l0, pa::kCopyMaxLayers);
        for (int32_t l = 0; l < a.num_layers; ++l) {
            a.k[l] = k_pools[l0 + l];
            a.v[l] = v_pools[l0 + l];
        }
        const pa_status st =
            launch_checked([&] { return pa::launch_copy_blocks(a, as_stream(stream)); });
        if (st != PA_OK) return st;
    }
    return PA_OK;
}

// whether [p, p + bytes) lies inside one allocation HIP knows
static bool inside_allocation(const void* p, size_t bytes) {
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    return q >= b && bytes <= size && q - b <= size - bytes;
}

pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || !aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) || bytes == 0 ||
        bytes % 16 != 0 || bytes > (size_t)INT64_MAX)
        return PA_ERR_INVALID_ARG;
    if (!inside_allocation(buf, bytes) ||
        !inside_allocation(sink, sizeof(uint32_t) * PA_STREAM_READ_SINK_WORDS))
        return PA_ERR_INVALID_ARG;
    return launch_checked([&] {
        return pa::launch_stream_read(buf, (int64_t)bytes, sink, as_stream(stream));
    });
}

}  // extern "C"
