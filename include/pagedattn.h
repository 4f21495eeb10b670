/*
 * libpagedattn — decode-phase paged attention for AMD MI355X (gfx950).
 *
 * Each running sequence's single new query attends over its whole KV cache.
 * The cache lives in fixed-size blocks scattered through one physical pool
 * and is located through a per-sequence block table: logical block j of a
 * sequence is physical block table[j], blocks need not be adjacent, and the
 * attention walks the table block by block (KV 缓存与分页注意力 §06 像内存分页,
 * §07 块表; Paged Attention in LLMs, "Block Table").
 *
 * C ABI.  Every pointer argument is documented as HOST or DEVICE.  The
 * library never allocates, frees or retains device memory: the caller owns
 * every buffer (including the optional workspace, whose size is queried
 * first).  Device work is enqueued on the caller's `stream` (a hipStream_t
 * passed as void*, NULL = the default stream) and ordered only by it; the
 * functions return once the work is enqueued.  Argument errors are detected
 * on the host before anything is enqueued and leave every buffer untouched.
 * Faults inside kernels surface at the caller's next synchronisation.
 * The device entry points keep no device state between calls and may be
 * called from several host threads at once, on the same or different
 * streams. Calls that write the same buffers (pools, outputs or a
 * workspace) must be ordered by the caller. The host allocator below is
 * the exception: serialise the calls on each of its handles.
 *
 * KV pool layout (one pool for K and one for V, per layer), dense row-major:
 *     pool[num_blocks][num_kv_heads][block_size][head_dim]
 * so one (block, kv-head) tile is a contiguous block_size x head_dim array.
 * A token's cache slot is  slot = physical_block * block_size + offset.
 * q and out are dense [num_seqs][num_heads][head_dim]; new K/V are dense
 * [num_tokens][num_kv_heads][head_dim].  Query head h reads KV head
 * h / (num_heads / num_kv_heads) (grouped / multi-query attention, KV 缓存与
 * 分页注意力 §11 后来的做法).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_F32 = 0,
    PA_F16 = 1,
    PA_BF16 = 2,
    PA_FP8_E4M3 = 3,  /* OCP E4M3FN: bias 7, max 448, no inf, NaN = S.1111.111 */
    PA_INT8 = 4       /* group-wise int8 cache: codes in [-127, 127], one float32
                         scale per (token, KV head) in separate scale pools */
} pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1,   /* bad pointer, size, shape or range            */
    PA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (dtype pair, head_dim) */
    PA_ERR_OUT_OF_BLOCKS = -3, /* allocator: not enough free blocks; nothing changed */
    PA_ERR_INDEX = -4,         /* allocator: logical index / table size out of range */
    PA_ERR_UNKNOWN_SEQ = -5,   /* allocator: no such sequence id               */
    PA_ERR_REFCOUNT = -6,      /* allocator: reference count would go negative */
    PA_ERR_HIP = -7,           /* the HIP runtime refused a launch             */
    PA_ERR_WORKSPACE = -8,     /* workspace missing or too small               */
    PA_ERR_EXISTS = -9         /* allocator: sequence id already in use        */
} pa_status;

/* Static, NUL-terminated description of a status code (never NULL). */
const char* pa_status_string(int32_t status);

/* Library version string, e.g. "libpagedattn 0.1 gfx950". */
const char* pa_version(void);

/* Name and description of the HIP error behind the calling thread's last
 * PA_ERR_HIP (empty string if none).  Valid until the thread's next call. */
const char* pa_last_error(void);

/*
 * Per-token KV-cache bytes: 2 x (num_kv_heads x head_dim) x num_layers x
 * bytes-per-number — one key and one value per layer (KV 缓存与分页注意力
 * §03 一个词元 800 KB; KV Cache从原理到实战 §2.2 KV Cache的显存账); for
 * PA_INT8 each key and value head vector adds its 4-byte scale.
 * Returns -1 for a non-positive size or an unknown dtype.
 */
int64_t pa_kv_bytes_per_token(int32_t num_kv_heads, int32_t head_dim, int32_t num_layers,
                              int32_t dtype);

/*
 * kv_cache_write — store each new token's K and V once, at its slot.
 * One token's keys and values are computed once per step and then kept
 * (KV 缓存与分页注意力 §02 一次写一个词元); the slot comes from the
 * sequence's block table (§07).
 *
 *   k_new, v_new   DEVICE, dense [num_tokens][num_kv_heads][head_dim] of src_dtype
 *   k_pool, v_pool DEVICE, pool layout above, kv_dtype
 *   slot_mapping   DEVICE int64 [num_tokens]; slot of token i, -1 = skip.  Slots
 *                  outside [0, num_blocks*block_size) are skipped as well.  Two
 *                  tokens with the same slot in one call: undefined which wins.
 *   Dtype pairs: src == kv (bytes copied unchanged), or kv == PA_FP8_E4M3 with
 *   src in {F32, F16, BF16}: value x is stored as e4m3(float(x) * (1/scale))
 *   with 1/scale computed in fp32 on the host, saturating to +-448, rounding
 *   to nearest even, NaN kept as NaN (KV 缓存与分页注意力 §11: 8-bit floats,
 *   one byte per number).  k_scale/v_scale are ignored for non-fp8 pools and
 *   must be finite and > 0 for fp8.  PA_INT8 pools carry scale pools and are
 *   written by pa_kv_cache_write_int8 (PA_ERR_UNSUPPORTED here).
 *   num_tokens == 0 is a no-op.
 */
pa_status pa_kv_cache_write(const void* k_new, const void* v_new, int32_t src_dtype,
                            void* k_pool, void* v_pool, int32_t kv_dtype,
                            const int64_t* slot_mapping, int32_t num_tokens,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float k_scale, float v_scale, void* stream);

/*
 * kv_cache_write_int8 — the cache write into a group-wise int8 cache
 * (KV Cache从原理到实战 §5.2 量化: 8-bit integers with one scale per group of
 * numbers; here a group is one token's head vector, so every key and value
 * vector carries its own scale).  For each new token i with a valid slot and
 * each KV head g, separately for K and V, in float32:
 *     amax  = max_d |x[i][g][d]|,   scale = amax / 127 (correctly rounded)
 *     code  = x / scale rounded to nearest, ties to even, clamped to [-127, 127]
 *             (all codes 0 and scale 0 for an all-zero vector)
 * stored as pool[block][g][offset][d] = code and scales[block][g][offset] = scale;
 * the value a code stands for is code * scale.
 *
 *   k_new, v_new      DEVICE, dense [num_tokens][num_kv_heads][head_dim], src_dtype
 *                     in {F32, F16, BF16}; non-finite inputs give unspecified codes
 *   k_pool, v_pool    DEVICE int8 pools, pool layout above (16-byte aligned)
 *   k_scales, v_scales DEVICE float32 [num_blocks][num_kv_heads][block_size]
 *   slot_mapping      DEVICE int64 [num_tokens], as for pa_kv_cache_write
 * Copy-on-write and swapping of an int8 cache move its scale pools as well:
 * pass them to pa_copy_blocks as PA_F32 pools with head_dim 1.
 */
pa_status pa_kv_cache_write_int8(const void* k_new, const void* v_new, int32_t src_dtype,
                                 void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, void* stream);

/* partition_size value that selects the balanced split (see below) */
#define PA_PARTITION_BALANCED (-1)

/*
 * Workspace bytes needed by pa_paged_attention_decode with the same
 * arguments: 0 for a single pass (partition_size == 0) or when every
 * sequence fits one partition.  The balanced split's size depends on the
 * compute-unit count of the current device.  Returns 0 for invalid sizes.
 */
size_t pa_paged_attention_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_context_len,
                                         int32_t partition_size);

/*
 * paged_attention_decode — one decode step of attention over a paged cache.
 * For each sequence s and query head h, with n = context_lens[s] and
 * g = h / (num_heads / num_kv_heads):
 *     out[s][h] = sum_t softmax_t(scale * q[s][h] . K_s[t][g]) * V_s[t][g]
 * over tokens t < n, where K_s[t] is read from
 * k_pool[block_tables[s][t / block_size]][g][t % block_size] (the new query
 * dotted with every cached key gives the weights; the weighted sum of the
 * values is the output: KV Cache从原理到实战 §2.1; fetched block by block
 * through the table: KV 缓存与分页注意力 §07).  n == 0 gives zeros.
 *
 *   out            DEVICE [num_seqs][num_heads][head_dim], dtype = q_dtype
 *                  (rounded to nearest even from fp32 accumulators)
 *   q              DEVICE [num_seqs][num_heads][head_dim], q_dtype in {F32, F16, BF16}
 *   k_pool, v_pool DEVICE, pool layout above, kv_dtype.  Supported pairs:
 *                  kv == q, or kv == PA_FP8_E4M3 with q in {F32, F16, BF16}
 *                  (PA_INT8 pools: pa_paged_attention_decode_int8).
 *   block_tables   DEVICE int32 [num_seqs][max_blocks_per_seq]; entries past
 *                  ceil(n / block_size) are never read.  An entry outside
 *                  [0, num_blocks) makes its tokens count as absent (never read).
 *   context_lens   DEVICE int32 [num_seqs]; values are clamped to
 *                  [0, min(max_context_len, max_blocks_per_seq * block_size)].
 *   max_context_len  host-known upper bound of context_lens (sizes the launch).
 *   scale          softmax scale (1/sqrt(head_dim) for standard attention)
 *   k_scale, v_scale  fp8 per-tensor scales (value = e4m3 code value * scale);
 *                  ignored unless kv_dtype == PA_FP8_E4M3.
 *   partition_size 0: single pass, every (sequence, head) handled whole.
 *                  > 0: split-context — each sequence is cut into partitions
 *                  of that many tokens, each partition produces (max, sum,
 *                  output) partials in `workspace`, and a log-sum-exp
 *                  reduction kernel merges them.
 *                  PA_PARTITION_BALANCED: the batch's contexts (each with a
 *                  fixed per-item cost added), laid end to end, are cut into
 *                  one equal range per wavefront of a launch that fills the
 *                  GPU (a whole number per SIMD when the batch is small);
 *                  contexts cut by a range boundary are merged by the same
 *                  log-sum-exp reduction.
 *                  Every mode gives the single pass's result within rounding.
 *   workspace      DEVICE, >= pa_paged_attention_workspace_size(...) bytes,
 *                  256-byte aligned, no initial contents; may be NULL when
 *                  that size is 0.  Calls that share a workspace must be
 *                  ordered (one stream, or synchronised).
 * Limits: head_dim in {64, 128}; block_size a power of two in [1, 256];
 * num_heads % num_kv_heads == 0; num_seqs * num_heads * partitions < 2^31.
 */
pa_status pa_paged_attention_decode(void* out, const void* q, int32_t q_dtype,
                                    const void* k_pool, const void* v_pool, int32_t kv_dtype,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    float scale, float k_scale, float v_scale,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_int8 — pa_paged_attention_decode over an int8 cache
 * written by pa_kv_cache_write_int8: K_s[t][g] and V_s[t][g] are the codes
 * times their own scales, k_scales / v_scales [block][g][offset] (same layout
 * and scale pools as the write).  q_dtype in {F32, F16, BF16}; out in q_dtype.
 * Every other argument, the workspace (pa_paged_attention_workspace_size)
 * and the limits are as for pa_paged_attention_decode.  The scale is applied
 * to each token's dot product and to its softmax weight, so the codes are
 * never widened to another cache format.
 */
pa_status pa_paged_attention_decode_int8(void* out, const void* q, int32_t q_dtype,
                                         const void* k_pool, const void* v_pool,
                                         const float* k_scales, const float* v_scales,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         int32_t num_seqs, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t num_blocks, float scale,
                                         int32_t partition_size, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * paged_attention_prefill — multi-token attention over a paged cache: the
 * prompt phase, or one chunk of a chunked prefill.  The prompt phase handles
 * a whole prompt at once (KV 缓存与分页注意力 §02); it is compute-bound where
 * decode is bandwidth-bound, and a long prompt may be cut into chunks so that
 * its prefill does not hold up decoding (KV Cache从原理到实战 §2.3, §5.4).
 * Write the chunk's K/V with pa_kv_cache_write first (one slot per new
 * token), then call this: every token is read through the block table.
 *
 * For sequence s with n = context_lens[s] tokens (the chunk included) and the
 * q_len = query_start[s+1] - query_start[s] query rows query_start[s] + i,
 * row i sits at position p = n - q_len + i and, for each head h with
 * g = h / (num_heads / num_kv_heads):
 *     out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_s[t][g]) * V_s[t][g]
 * (causal over the new tokens; every earlier token is visible).  Rows with
 * p < 0 (a chunk longer than its context) give zeros.
 *
 *   out, q          DEVICE [num_query_tokens][num_heads][head_dim], q_dtype
 *   k_pool, v_pool  DEVICE, pool layout above; kv_dtype == q_dtype in {F16, BF16}
 *                   (other pairs: PA_ERR_UNSUPPORTED)
 *   block_tables    DEVICE int32 [num_seqs][max_blocks_per_seq]; an entry
 *                   outside [0, num_blocks) makes its tokens absent
 *   context_lens    DEVICE int32 [num_seqs], clamped to [0, max_blocks_per_seq * block_size]
 *   query_start     DEVICE int32 [num_seqs + 1], non-decreasing row offsets
 *                   (values are clamped to [0, num_query_tokens])
 *   max_query_len   host-known bound of every q_len (sizes the launch); rows of
 *                   a sequence beyond it are not written
 *   scale           softmax scale (1/sqrt(head_dim) for standard attention)
 * Limits: head_dim in {64, 128}; block_size a power of two in [1, 256];
 * num_heads % num_kv_heads == 0.  No workspace; nothing is allocated.
 */
pa_status pa_paged_attention_prefill(void* out, const void* q, int32_t q_dtype,
                                     const void* k_pool, const void* v_pool, int32_t kv_dtype,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, const int32_t* query_start,
                                     int32_t num_seqs, int32_t num_query_tokens,
                                     int32_t max_query_len, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, float scale, void* stream);

/* Size of the device scratch the allocation-free decode entry point uses
 * (one copy per GPU, held from the library's load until the process ends). */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * paged_attention_decode_noalloc — pa_paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, meaning and
 * result as pa_paged_attention_decode without the workspace: the split modes'
 * partial records and range descriptors go to a static device array of
 * PA_NOALLOC_SCRATCH_BYTES inside the library instead.  The call allocates
 * nothing (no hipMalloc, no allocating library routine); the scratch needs no
 * initial contents, and every call writes what it later reads.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams, or host threads without ordering) race and
 * give undefined outputs; order them.  A launch whose records exceed the
 * scratch returns PA_ERR_WORKSPACE with nothing enqueued (the balanced split
 * needs (head_dim + 2) * 4 bytes per record, two records per worker and head
 * of its unit; e.g. about 8.5 MB for 128 sequences of 64 query heads over 8
 * KV heads of 128); partition_size > 0 needs what
 * pa_paged_attention_workspace_size returns.  PA_ERR_HIP if the runtime
 * cannot give the scratch's address.
 */
pa_status pa_paged_attention_decode_noalloc(void* out, const void* q, int32_t q_dtype,
                                            const void* k_pool, const void* v_pool,
                                            int32_t kv_dtype, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t max_context_len,
                                            int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t num_blocks, float scale,
                                            float k_scale, float v_scale, int32_t partition_size,
                                            void* stream);

/*
 * copy_blocks — the data half of copy-on-write: for each pair (src, dst),
 * copy physical block src to dst, bit for bit, in the K and V pool of every
 * layer.  Before a sequence writes into a block it shares with others, the
 * block is copied and the write goes into the copy (KV 缓存与分页注意力
 * §08 共用，写时复制).  Issue it on the same stream before the cache write.
 *
 *   k_pools, v_pools  HOST arrays of num_layers DEVICE pool pointers (their
 *                     values are baked into the launches: a captured graph
 *                     keeps copying the same pools)
 *   pairs             DEVICE int32 [num_pairs][2] = (src, dst), 8-byte
 *                     aligned, e.g. the pairs pa_alloc_append_slots returned,
 *                     copied to the device.  The pairs are read by the kernel
 *                     when it runs, so one captured launch can be replayed
 *                     with new pairs written into the same buffer each step.
 *                     A pair with an id outside [0, num_blocks) — such as
 *                     -1 padding of a fixed-capacity buffer — or with
 *                     src == dst is skipped.  Destinations must be distinct
 *                     and no destination may also be a source in the same
 *                     call (the caller's contract, not checked: the copies
 *                     run concurrently, so a violation gives undefined bytes
 *                     in the blocks concerned).
 *   num_pairs         rows of `pairs` the launch covers (its capacity).
 *   num_pairs == 0 or num_layers == 0 is a no-op.
 */
pa_status pa_copy_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                         int32_t kv_dtype, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks,
                         const int32_t* pairs, int32_t num_pairs, void* stream);

/*
 * swap_blocks — move blocks between pools, e.g. a preempted sequence's blocks
 * from device pools to pools in pinned host memory and back when it resumes
 * (KV 缓存与分页注意力 §09 放不下的时候: when blocks run out, the latest
 * request gives up all of its blocks, which go to CPU memory and come back
 * later; the data moves unchanged).  For each pair (s, d) and each pool l:
 * block d of dst_pools[l] = block s of src_pools[l], bit for bit.
 *
 *   dst_pools, src_pools  HOST arrays of num_pools pool pointers; each is device
 *                     memory or pinned host memory known to HIP (hipHostMalloc,
 *                     torch pin_memory); memory HIP does not know (pageable)
 *                     gives PA_ERR_INVALID_ARG with nothing enqueued.  16-byte
 *                     aligned; src and dst must not overlap.
 *   block_bytes       bytes of one block of one pool (a multiple of 16), e.g.
 *                     num_kv_heads * block_size * head_dim * element bytes
 *   dst_num_blocks, src_num_blocks  pool sizes in blocks; pairs with ids
 *                     outside them (e.g. -1 padding) are skipped
 *   pairs             DEVICE int32 [num_pairs][2] = (src block, dst block), as
 *                     pa_alloc_swap_out / pa_alloc_swap_in return (copied to
 *                     the device); read when the kernel runs.  Destinations
 *                     must be distinct.
 * Issue the swap-out copy before any later write into the released device
 * blocks, and the swap-in copy before the sequence is read (same stream).
 */
pa_status pa_swap_blocks(void* const* dst_pools, const void* const* src_pools, int32_t num_pools,
                         int64_t block_bytes, int32_t dst_num_blocks, int32_t src_num_blocks,
                         const int32_t* pairs, int32_t num_pairs, void* stream);

/*
 * stream_read — a measurement aid, not part of the attention path: reads
 * `bytes` bytes of device memory once with the same 16-byte streaming
 * (non-temporal) loads, consecutive lanes on consecutive pieces, that the
 * decode kernels use for K and V, so that the rate their HBM rooflines are
 * compared with can be measured on the device at hand (time it with events on
 * `stream`).
 *
 *   buf    DEVICE memory, 16-byte aligned; bytes: a positive multiple of 16
 *   sink   DEVICE uint32 [PA_STREAM_READ_SINK_WORDS], caller-owned; the call
 *          writes the XOR of all of buf's 32-bit words, folded per workgroup,
 *          into its first words (the XOR of every sink word written equals the
 *          XOR of buf's words when the sink was zeroed first)
 *   stream hipStream_t (NULL: the default stream)
 * Errors: PA_ERR_INVALID_ARG for a null, misaligned or badly sized argument, or
 * when [buf, buf + bytes) or the sink does not lie inside one HIP allocation
 * (checked with hipMemGetAddressRange before anything is enqueued).
 */
#define PA_STREAM_READ_SINK_WORDS 4096
pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator: free list, per-block reference counts, block tables
 * and copy-on-write (KV 缓存与分页注意力 §07 块表, §08 共用，写时复制;
 * KV Cache从原理到实战 §6.2 加上分页管理).  Host memory only, no GPU calls;
 * one allocator serves every layer (block ids are shared by all layers).
 * Not thread-safe: serialise calls on one handle.  Every operation that
 * fails returns an error and leaves the allocator unchanged.
 * ---------------------------------------------------------------------- */
typedef struct pa_allocator pa_allocator;

/* free_order: HOST int32 [num_blocks] permutation of 0..num_blocks-1 giving the
 * initial free list (blocks are taken from its END), or NULL for 0..n-1. */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                          pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);

/* New sequence holding num_tokens tokens: takes ceil(num_tokens/block_size)
 * blocks, all or none (PA_ERR_OUT_OF_BLOCKS when short; PA_ERR_EXISTS for a
 * used id). */
pa_status pa_alloc_add_seq(pa_allocator* a, int64_t seq_id, int32_t num_tokens);

/* Parallel sample: child_id shares every block of parent_id (counts + 1). */
pa_status pa_alloc_fork(pa_allocator* a, int64_t parent_id, int64_t child_id);

/* One new token for each of n distinct sequences, in order.  A sequence
 * whose blocks are all full gets a fresh block; one whose partly filled last
 * block is still shared gets a copy (its count drops by one) and the pair
 * (old, new) is appended to cow_pairs_out; the last holder writes in place.
 *   seq_ids          HOST int64 [n]
 *   slot_mapping_out HOST int64 [n]: slot of each new token
 *   cow_pairs_out    HOST int32 [n][2] (at most n pairs), may be NULL only if
 *                    no copy is needed (else PA_ERR_INVALID_ARG, nothing done)
 *   num_pairs_out    HOST int32 (pairs written)
 * All or nothing: if the free list is short, nothing changes. */
pa_status pa_alloc_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n,
                                int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                                int32_t* num_pairs_out);

/* Finished sequence: every block's count drops by one; blocks reaching zero go
 * back to the free list in table order. */
pa_status pa_alloc_free_seq(pa_allocator* a, int64_t seq_id);

/* Swapping (KV 缓存与分页注意力 §09): a sequence's blocks all move or none do.
 * swap_out: the sequence leaves `dev` for `host` (an allocator over host
 * blocks of the same block size): it takes fresh host blocks in the same
 * logical order and releases its device blocks (a block another sequence
 * still shares stays with it, its count down by one).  pairs_out HOST int32
 * [max_pairs][2] receives one (device block, host block) copy per logical
 * block; PA_ERR_INDEX if max_pairs is smaller than the table, PA_ERR_OUT_OF_BLOCKS
 * if the host pool is short, and nothing changes on any error.
 * swap_in: the reverse, (host block, device block) pairs, fresh device blocks.
 * Prefix-cache tracking of a swapped sequence ends (its blocks come back
 * uncached). */
pa_status pa_alloc_swap_out(pa_allocator* dev, pa_allocator* host, int64_t seq_id,
                            int32_t* pairs_out, int32_t max_pairs, int32_t* num_pairs_out);
pa_status pa_alloc_swap_in(pa_allocator* dev, pa_allocator* host, int64_t seq_id,
                           int32_t* pairs_out, int32_t max_pairs, int32_t* num_pairs_out);

/* Block tables HOST int32 [n][max_blocks] (-1 padded) and context lengths HOST
 * int32 [n] of the given sequences.  PA_ERR_INDEX if a table is longer than
 * max_blocks.  context_lens_out may be NULL. */
pa_status pa_alloc_export(const pa_allocator* a, const int64_t* seq_ids, int32_t n,
                          int32_t* block_tables_out, int32_t max_blocks,
                          int32_t* context_lens_out);

/* Physical block of logical block `logical_idx` (PA_ERR_INDEX past the table;
 * KV Cache内存优化技术原理与PagedAttention分页注意力实现, the BlockTable sketch). */
pa_status pa_alloc_physical_block(const pa_allocator* a, int64_t seq_id, int32_t logical_idx,
                                  int32_t* block_out);

/* ---- prefix caching (KV 缓存与分页注意力 §11 后来的做法: every full block is
 * identified by its tokens and everything before them, and a new request with
 * the same beginning reuses the cached blocks; KV Cache从原理到实战 §4.2:
 * block-level matching, reference counts, LRU eviction that never takes a
 * block in use).  Identities are 64-bit hashes chained over the blocks,
 * checked on every hit against the block's tokens and its predecessor's
 * identity.  A block whose count reaches zero while its identity is held
 * stays cached (contents kept) in a least-recently-used list; fresh blocks
 * come from the free list first, then from the LRU end of that list (a
 * finished sequence's cached blocks enter it last block first).  Blocks of
 * sequences admitted without token ids are never cached. */

/* New sequence with known token ids (HOST int32 [num_tokens]): reuses the
 * longest run of leading full blocks whose identities are cached and takes
 * fresh blocks for the rest; its own new full blocks become findable.
 * num_cached_out (HOST, may be NULL): tokens already in the cache (a multiple
 * of block_size) — their keys and values need not be written again.  All or
 * nothing (PA_ERR_OUT_OF_BLOCKS when short; PA_ERR_EXISTS for a used id). */
pa_status pa_alloc_add_seq_tokens(pa_allocator* a, int64_t seq_id, const int32_t* tokens,
                                  int32_t num_tokens, int32_t* num_cached_out);

/* pa_alloc_append_slots with the new tokens' ids (HOST int32 [n]): a block
 * that its new token fills becomes findable by later sequences.  (A sequence
 * appended to without ids stops being tracked: its later blocks are not
 * cached.) */
pa_status pa_alloc_append_tokens(pa_allocator* a, const int64_t* seq_ids, const int32_t* token_ids,
                                 int32_t n, int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                                 int32_t* num_pairs_out);

/* Block accounting.  Utilisation of the KV memory in use (KV 缓存与分页注意力
 * §05, §07) is filled_slots / (used_blocks * block_size). */
typedef struct {
    int64_t num_blocks;
    int64_t free_blocks;        /* on the free list                               */
    int64_t evictable_blocks;   /* cached, unreferenced (reusable or evictable)   */
    int64_t used_blocks;        /* reference count > 0                            */
    int64_t cached_blocks;      /* identity held (in use or evictable)            */
    int64_t filled_slots;       /* token slots holding a token, each used block once */
    int64_t prefix_hit_blocks;  /* blocks reused by admissions so far             */
    int64_t evictions;          /* cached blocks taken back so far                */
} pa_alloc_counts;
pa_status pa_alloc_stats(const pa_allocator* a, pa_alloc_counts* out);
int32_t pa_alloc_num_evictable(const pa_allocator* a);              /* -1 if a is NULL */

int32_t pa_alloc_num_free(const pa_allocator* a);                   /* -1 if a is NULL */
int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block);   /* -1 if out of range */
int32_t pa_alloc_seq_len(const pa_allocator* a, int64_t seq_id);   /* -1 if unknown */
int32_t pa_alloc_num_seqs(const pa_allocator* a);                   /* -1 if a is NULL */

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
