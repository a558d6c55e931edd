/*
 * pa.h -- C ABI of libpagedattn.so, a paged KV-cache attention library for
 * AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [vllm]   "PagedAttention 在 vLLM 中的实现分析" (blog.chen3feng.top):
 *            §3.1 block table, §3.2 slot mapping, §3.3 KV cache layouts,
 *            §4.1 block pool, §5.4 CommonAttentionMetadata, §6.2 forward with
 *            flash_attn_varlen_func(block_table=..., causal=True), §6.3
 *            reshape_and_cache_flash, §7.3 V1/V2 kernels, §7.4 cache write.
 *   [k4i]    "Paged attention" post (k4i.top): block table, block manager,
 *            attention over non-contiguous blocks (online softmax), copy-on-write.
 *   [atb]    ATB PagedAttention + virtual memory article (2048ai.net):
 *            reference counting, copy-on-write.
 *   [packed] cann-recipes-infer Paged KV Cache + Packed Sequence notes
 *            (m.xxqk.cn): §2.3 packed sequences and their offsets.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are HIP device memory owned by the caller; the
 *     library never allocates, frees or keeps them.  Pointers marked (host)
 *     are host memory, read during the call only.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Device
 *     work is enqueued on it and the call returns without synchronising.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     failed check returns a status and enqueues nothing.  Device-resident
 *     metadata (block ids, slots, lengths) is NOT checked on the hot path:
 *     out-of-range values are undefined behaviour; pa_check_metadata checks
 *     them synchronously for tests and debugging.
 *   - Element types: PA_F32, PA_BF16, PA_F16.  K/V caches, keys, values and
 *     queries of one call share one type, except in the *_fp8 calls, whose
 *     caches are PA_FP8_E4M3.
 *   - Sizes are in elements unless the name says bytes.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1, /* a size, pointer or combination is invalid      */
  PA_ERR_UNSUPPORTED = 2,      /* valid, but not a shape/type this build handles */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_OUT_OF_BLOCKS = 4,    /* block pool: not enough free blocks (no change) */
  PA_ERR_HIP = 5,              /* a HIP runtime call or launch failed            */
  PA_ERR_METADATA = 6          /* pa_check_metadata found a violated precondition*/
} pa_status;

/* PA_FP8_E4M3: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; no infinities, largest finite 448, S.1111.111 = NaN), one
 * byte per element.  A cache element type only ([vllm] §6.3 kv_cache_dtype
 * with k_scale / v_scale, §8 FP8 KV-cache quantisation): it is written by
 * pa_reshape_and_cache_fp8 (or bit-copied by pa_reshape_and_cache /
 * pa_copy_blocks) and read by pa_decode_fp8 and pa_prefill_fp8; queries
 * and outputs stay 16-bit or fp32. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_F16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Cache layouts ([vllm] §3.3).  A block is contiguous in both. */
typedef enum {
  PA_LAYOUT_NHD = 0, /* [num_blocks, block_size, num_kv_heads, head_size]        */
  PA_LAYOUT_HND = 1  /* [num_blocks, num_kv_heads, block_size, head_size] (head-major) */
} pa_layout;

/* Human-readable name of a status code (static string). */
const char* pa_status_string(pa_status status);

/* Text of the last failure in the calling thread (static per-thread buffer). */
const char* pa_last_error(void);

/*
 * pa_reshape_and_cache -- scatter this step's new K/V rows into the block pool
 * ([vllm] §3.2, §6.3, §7.4).
 *
 * Row i of key/value ([num_kv_heads, head_size], contiguous; rows
 * `key_row_stride` / `value_row_stride` elements apart) is copied bit for bit
 * to slot s = slot_mapping[i] of the pool: block s / block_size, offset
 * s % block_size, laid out as `layout`.  A negative slot marks a padding row
 * and the row is skipped.  All other slots of the pool are left untouched.
 *   key, value          (device) [num_tokens, ...] rows of `dtype`
 *   key_cache, value_cache (device) pools of num_blocks blocks
 *   slot_mapping        (device) int64 [num_tokens]
 * Preconditions (not checked on the device): non-negative slots are distinct
 * and < num_blocks * block_size.  head_size * sizeof(dtype) must be a
 * multiple of 16 bytes and all pointers and row strides 16-byte aligned.
 * num_tokens == 0 is a no-op.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value,
                               int64_t key_row_stride, int64_t value_row_stride,
                               void* key_cache, void* value_cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_size,
                               int32_t block_size, int32_t num_blocks,
                               pa_dtype dtype, pa_layout layout, void* stream);

/*
 * pa_reshape_and_cache_fp8 -- the cache write into FP8 pools ([vllm] §6.3
 * reshape_and_cache_flash with kv_cache_dtype, k_scale and v_scale; §7.4 the
 * flash variant of the write kernel).
 *
 * As pa_reshape_and_cache, but every element x of a key (value) row is
 * stored as the E4M3 code of x / k_scale (x / v_scale): the quotient is
 * taken in fp32 (correctly rounded), clamped to [-448, 448] (infinities
 * too), then rounded to the nearest E4M3 value with ties to the even code;
 * NaN stays NaN (code 0x7F or 0xFF).  A code c later reads back as
 * value(c) * scale.
 *   key, value             (device) rows of src_dtype (PA_F32, PA_BF16, PA_F16)
 *   key_cache, value_cache (device) uint8 pools of num_blocks blocks
 *   k_scale, v_scale       positive, finite
 * head_size must be a multiple of 16; pointers and source row strides
 * 16-byte aligned.  Slot preconditions as in pa_reshape_and_cache.
 */
pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, pa_dtype src_dtype,
                                   int64_t key_row_stride, int64_t value_row_stride,
                                   void* key_cache, void* value_cache,
                                   const int64_t* slot_mapping, int32_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_size,
                                   int32_t block_size, int32_t num_blocks,
                                   pa_layout layout, float k_scale, float v_scale,
                                   void* stream);

/*
 * pa_copy_blocks -- whole-block copies of both pools (copy-on-write, [k4i]
 * copy-on-write step 2, [atb] copy-on-write section).
 *   block_pairs (device) int32 [num_pairs][2] = (source block, destination block)
 * Every destination must be distinct and no destination may be a source
 * (not checked on the device).  A pair naming a block outside
 * [0, num_blocks) is skipped (the kernel checks each pair before touching
 * either pool).  num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(void* key_cache, void* value_cache,
                         const int32_t* block_pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                         void* stream);

/*
 * pa_swap_blocks -- whole-block copies from one pair of pools to another,
 * e.g. a preempted sequence's blocks out to a host pool and back in later
 * ([k4i] "relation to continuous batching": when the pool runs out, the
 * scheduler may swap blocks to CPU memory).  For pair i, block
 * block_pairs[i][0] of each source pool is copied bit for bit to block
 * block_pairs[i][1] of the matching destination pool (K to K, V to V), in
 * pair order.
 *   src_key_cache, src_value_cache, dst_key_cache, dst_value_cache: device
 *       memory or pinned host memory (hipHostMalloc); the direction of each
 *       copy follows from the addresses
 *   block_pairs (host) int32 [num_pairs][2], read during the call
 *   block_bytes bytes of one block (block_size * num_kv_heads * head_size *
 *       element size)
 * The copies are enqueued on `stream` (asynchronous; with pinned host memory
 * they overlap other work).  Block ids are checked against src_num_blocks /
 * dst_num_blocks before anything is enqueued.  num_pairs == 0 is a no-op.
 */
pa_status pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                         void* dst_key_cache, void* dst_value_cache,
                         const int32_t* block_pairs, int32_t num_pairs,
                         int64_t block_bytes, int32_t src_num_blocks,
                         int32_t dst_num_blocks, void* stream);

/*
 * pa_decode -- one query token per sequence attends to its cached context
 * through its block table ([vllm] §3.1, §6.2, §7.2; [k4i] attention over
 * non-contiguous blocks).
 *
 * For sequence s, query head h, kv head g = h / (num_heads / num_kv_heads)
 * (contiguous GQA groups) and L = context_lens[s]:
 *   out[s,h,:] = softmax_t(scale * q[s,h,:] . K_t) V_t,  t = 0 .. L-1,
 * where K_t/V_t are read at block block_tables[s][t / block_size], offset
 * t % block_size of the pools.  L includes this step's token, which must
 * already be written (pa_reshape_and_cache).  L == 0 gives a zero row.
 *   out          (device) [num_seqs, num_heads, head_size] of out_dtype
 *                (PA_F32, or kv_dtype)
 *   query        (device) [num_seqs, num_heads, head_size] of kv_dtype
 *   block_tables (device) int32 [num_seqs, max_blocks_per_seq]; entries past
 *                ceil(L / block_size) are never read
 *   context_lens (device) int32 [num_seqs], each in [0, max_context_len] and
 *                <= max_blocks_per_seq * block_size
 *   partition_size  0  = one pass per (sequence, kv head) ("V1", [vllm] §7.3)
 *                   >0 = split-K over partitions of that many tokens, then a
 *                        reduce ("V2", [vllm] §7.3); a multiple of 16
 *                   -1 = chosen by the library from the shape
 *   workspace    (device) >= pa_decode_workspace_size(...) bytes when split-K
 *                is used (may be NULL for partition_size 0): the partials
 *                and, for the grouped kernels over more than 256
 *                sequences or with a partition size that is not a power of
 *                two, the partition kernel's dispatch list (largest
 *                partitions first); no content is needed on entry
 * Supported: head_size 64 or 128; num_heads / num_kv_heads in {1,2,4,8,16};
 * block_size a power of two in [1, 1024]; PA_LAYOUT_NHD or PA_LAYOUT_HND.
 * Results are bitwise deterministic for a fixed launch configuration and do
 * not depend on which physical blocks hold the context.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                int32_t head_size, int32_t max_context_len,
                                int32_t partition_size);

/*
 * Partition size for this decode shape (0 = single pass): 512 for the
 * per-head kernel (group size 1 or 2, or fp32), a larger power of two for
 * the grouped kernels (group size 4, 8 or 16 with bf16, f16 or
 * PA_FP8_E4M3 caches) while about four workgroups per compute unit remain.
 * total_context_len is the sum of context_lens when the caller knows it
 * (<= 0: unknown, num_seqs * max_context_len is assumed); partition_size -1
 * in the decode calls resolves with it unknown.  Never below 512, so a
 * workspace sized for partition_size -1 fits every value it returns.
 */
int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, pa_dtype kv_dtype,
                                 int32_t max_context_len,
                                 int64_t total_context_len);

pa_status pa_decode(void* out, pa_dtype out_dtype, const void* query,
                    const void* key_cache, const void* value_cache,
                    pa_dtype kv_dtype, pa_layout layout,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_size, int32_t block_size, int32_t num_blocks,
                    float scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * pa_decode_static_scratch -- pa_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  No workspace argument: split-K
 * partials, their (max, sum) records and the dispatch list live in a
 * library-owned array of PA_STATIC_SCRATCH_BYTES (96 MiB) on each GPU, held
 * from when the library's code is loaded on that GPU until the process
 * ends; the call allocates nothing.  Arguments, result, partition policy
 * and errors are those of pa_decode (16-bit and fp32 caches); additionally,
 * a shape whose split-K workspace at the resolved partition size
 * (pa_decode_workspace_size) exceeds PA_STATIC_SCRATCH_BYTES returns
 * PA_ERR_WORKSPACE_TOO_SMALL before any device call.  Every call on one GPU
 * uses that GPU's one array: calls ordered on one stream are safe, calls
 * that overlap in time on one GPU (other streams, other threads) race and
 * give undefined results.  Nothing needs clearing between calls: every byte
 * a call reads from the array it has written first.
 */
#define PA_STATIC_SCRATCH_BYTES (96u << 20)
pa_status pa_decode_static_scratch(void* out, pa_dtype out_dtype, const void* query,
                                   const void* key_cache, const void* value_cache,
                                   pa_dtype kv_dtype, pa_layout layout,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t num_blocks,
                                   float scale, int32_t partition_size, void* stream);

/*
 * pa_decode_fp8 -- pa_decode over FP8 (E4M3) pools written by
 * pa_reshape_and_cache_fp8: the cached key t reads back as K_t = value(code)
 * * k_scale and the value as V_t = value(code) * v_scale ([vllm] §6.3), so
 *   out[s,h,:] = softmax_t(scale * k_scale * q . value(K codes)) value(V codes) * v_scale.
 * The query is q_dtype (PA_BF16 or PA_F16); out_dtype is PA_F32 or q_dtype.
 * Every other argument, the workspace (pa_decode_workspace_size) and the
 * partition policy (pa_decode_auto_partition with kv_dtype PA_FP8_E4M3) are
 * as in pa_decode; head_size 64 or 128.
 */
pa_status pa_decode_fp8(void* out, pa_dtype out_dtype, const void* query, pa_dtype q_dtype,
                        const void* key_cache, const void* value_cache,
                        float k_scale, float v_scale, pa_layout layout,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t max_context_len,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_size, int32_t block_size, int32_t num_blocks,
                        float scale, int32_t partition_size, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * pa_decode_partitions_fp8 -- the partition half of pa_decode_fp8 with
 * partition_size > 0 (contract of pa_decode_partitions, with the scales and
 * query type of pa_decode_fp8; the partials already carry v_scale).
 * pa_decode_reduce finishes it: pa_decode_fp8 runs exactly these two.
 */
pa_status pa_decode_partitions_fp8(void* out, pa_dtype out_dtype, const void* query,
                                   pa_dtype q_dtype, const void* key_cache,
                                   const void* value_cache, float k_scale, float v_scale,
                                   pa_layout layout, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t num_blocks,
                                   float scale, int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * The two halves of split-K decode, for callers that schedule or time them
 * separately; pa_decode with partition_size > 0 runs exactly these two.
 *
 * pa_decode_partitions -- for every (sequence, query head, partition p) with
 * tokens t in [p * partition_size, min((p + 1) * partition_size, L)), writes
 * to `workspace` the partition's running max m_p (log2 units of
 * scale * q . K), the sum l_p of 2^(z_t - m_p) and the unnormalised output
 * sum_t 2^(z_t - m_p) V_t (fp32).  Partitions at or past L are not written.
 * Heads of sequences whose whole context is one partition (L <=
 * partition_size) get their final row written to `out` directly instead.
 * partition_size must be > 0 (PA_ERR_INVALID_ARGUMENT otherwise); other
 * arguments as in pa_decode.
 *
 * pa_decode_reduce -- merges the ceil(L / partition_size) partitions of every
 * (sequence, head) with L > partition_size using the log-sum-exp rule
 * ([vllm] §7.3 V2 reduce):
 *   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
 * and writes those rows of out; the other rows were written by the
 * partitions call.  The workspace, out, context_lens, max_context_len and
 * partition_size must be those of the partitions call.
 */
pa_status pa_decode_partitions(void* out, pa_dtype out_dtype, const void* query, const void* key_cache,
                               const void* value_cache, pa_dtype kv_dtype,
                               pa_layout layout, const int32_t* block_tables,
                               int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len,
                               int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size,
                               int32_t block_size, int32_t num_blocks, float scale,
                               int32_t partition_size, void* workspace,
                               size_t workspace_bytes, void* stream);

pa_status pa_decode_reduce(void* out, pa_dtype out_dtype,
                           const int32_t* context_lens, int32_t max_context_len,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_size, int32_t partition_size,
                           const void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade -- pa_decode for a batch whose sequences share their
 * first common_prefix_len tokens in the same physical blocks ([vllm] §6.4
 * cascade attention: the shared prefix is attended once, without a causal
 * mask, each sequence's own tokens separately, and the parts are merged with
 * the online-softmax rule of §7.3).
 *
 * Same result as pa_decode up to the order of fp32 sums (same arguments and
 * output; both equal the plain definition within the same bound, at any V
 * magnitude).  Additionally:
 *   common_prefix_len  tokens, a positive multiple of block_size, at most
 *                      every context_lens[s]; block_tables[s][0 ..
 *                      common_prefix_len / block_size - 1] must be the same
 *                      blocks for every s (row 0's are read; not checked on
 *                      the device -- pa_check_metadata checks it on request)
 *   partition_size     split of each sequence's own tokens [common_prefix_len,
 *                      L): > 0 (a multiple of 16), 0 = one partition for the
 *                      longest, -1 = chosen by the library
 *   workspace          (device, 16-byte aligned) >=
 *                      pa_decode_cascade_workspace_size(...) bytes; out must
 *                      be 16-byte aligned
 * The prefix pass runs on matrix cores: kv_dtype must be PA_BF16 or PA_F16
 * (PA_ERR_UNSUPPORTED otherwise).  Three launches on `stream`: the prefix
 * pass (all sequences' queries against the common blocks, in key
 * partitions), the partitions of each sequence's own tokens, and the reduce.
 */
size_t pa_decode_cascade_workspace_size(int32_t num_seqs, int32_t num_heads,
                                        int32_t head_size, int32_t max_context_len,
                                        int32_t common_prefix_len,
                                        int32_t partition_size);

pa_status pa_decode_cascade(void* out, pa_dtype out_dtype, const void* query,
                            const void* key_cache, const void* value_cache,
                            pa_dtype kv_dtype, pa_layout layout,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len,
                            int32_t common_prefix_len, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int32_t block_size, int32_t num_blocks, float scale,
                            int32_t partition_size, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade_fp8 -- pa_decode_cascade over FP8 (E4M3) pools, with the
 * query type, scales and read-back of pa_decode_fp8 ([vllm] §6.3, §6.4).
 * Same workspace (pa_decode_cascade_workspace_size) and preconditions.
 */
pa_status pa_decode_cascade_fp8(void* out, pa_dtype out_dtype, const void* query,
                                pa_dtype q_dtype, const void* key_cache,
                                const void* value_cache, float k_scale, float v_scale,
                                pa_layout layout, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, int32_t common_prefix_len,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t block_size, int32_t num_blocks,
                                float scale, int32_t partition_size, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * pa_prefill -- causal attention of packed query rows over the paged cache
 * ([vllm] §6.2 flash_attn_varlen_func with cu_seqlens_q = query_start_loc,
 * seqlen_k = seq_lens, block_table, causal = True; [packed] §2.3).
 *
 * Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1
 * (n rows, packed without padding); with L = context_lens[s] >= n, row j is
 * the token at position L - n + j and attends to positions 0 .. L - n + j
 * (causal mask aligned to the end of the context).  K/V of all L positions
 * must already be in the pool.
 *   out             (device) [num_tokens, num_heads, head_size] of out_dtype
 *                   (PA_F32, or kv_dtype)
 *   query           (device) [num_tokens, num_heads, head_size] of kv_dtype
 *   query_start_loc (device) int32 [num_seqs + 1], query_start_loc[0] = 0,
 *                   non-decreasing, query_start_loc[num_seqs] = num_tokens
 *   max_query_len   >= every n (host value)
 * out, query and both caches must be 16-byte aligned (PA_ERR_INVALID_ARGUMENT
 * otherwise).  Each probability enters the P.V product as two f16 terms
 * (hi = f16(p), lo = f16(p - hi): about 22 significant bits) and the
 * normaliser sums those same terms; V of any finite bf16 magnitude is
 * handled (values of 2^16 and more switch the workgroup to V scaled by a
 * power of two, its earlier sums rescaled exactly), infinities and NaN
 * propagate as in the plain definition.
 * Supported: kv_dtype PA_BF16 or PA_F16 (matrix cores), head_size 64 or 128,
 * num_heads / num_kv_heads in {1,2,4,8,16}, block_size a power of two.
 */
pa_status pa_prefill(void* out, pa_dtype out_dtype, const void* query,
                     const void* key_cache, const void* value_cache,
                     pa_dtype kv_dtype, pa_layout layout,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* query_start_loc, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                     int32_t max_context_len, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                     int32_t num_blocks, float scale, void* stream);

/*
 * pa_prefill_fp8 -- pa_prefill over FP8 (E4M3) pools written by
 * pa_reshape_and_cache_fp8 ([vllm] §6.2 with the §6.3 cache types): the
 * cached key t reads back as value(code) * k_scale and the value as
 * value(code) * v_scale.  The query is q_dtype (PA_BF16 or PA_F16); out_dtype
 * is PA_F32 or q_dtype; k_scale, v_scale positive and finite.  Every other
 * argument and precondition is as in pa_prefill.
 */
pa_status pa_prefill_fp8(void* out, pa_dtype out_dtype, const void* query, pa_dtype q_dtype,
                         const void* key_cache, const void* value_cache,
                         float k_scale, float v_scale, pa_layout layout,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* query_start_loc, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                         int32_t max_context_len, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                         int32_t num_blocks, float scale, void* stream);

/*
 * pa_check_metadata -- synchronous host-side check of the device metadata
 * the kernels trust ([vllm] §3.1 block table, §3.2 slot mapping, §5.4
 * CommonAttentionMetadata; §6.4 for the cascade's shared blocks).  For
 * tests and debugging: it synchronises `stream`, copies the arrays to the
 * host and reads nothing else.  Checks, each skipped when its pointer is
 * NULL:
 *   context_lens (device, int32 [num_seqs])
 *       0 <= context_lens[s] <= max_context_len (the bound the split-K grid,
 *       workspace and reduce are sized by), and, with block_tables,
 *       context_lens[s] <= max_blocks_per_seq * block_size;
 *   block_tables (device, int32 [num_seqs, max_blocks_per_seq])
 *       every entry a sequence reads (entries below ceil(context_lens[s] /
 *       block_size); every entry when context_lens is NULL) lies in
 *       [0, num_blocks);
 *   slot_mapping (device, int64 [num_tokens])
 *       non-negative slots are < num_blocks * block_size and distinct
 *       (negative slots are padding and always pass);
 *   common_prefix_len > 0 (the cascade's precondition; needs both
 *       block_tables and context_lens)
 *       a multiple of block_size, at most every context_lens[s], and
 *       block_tables[s][0 .. common_prefix_len / block_size - 1] equal to
 *       row 0's for every s.  0 skips this check.
 * Sizes must be non-negative, block_size and num_blocks positive
 * (PA_ERR_INVALID_ARGUMENT).  Returns PA_OK, or PA_ERR_METADATA with the
 * first violation (array, index, value) in pa_last_error().
 */
pa_status pa_check_metadata(const int32_t* block_tables,
                            const int32_t* context_lens,
                            const int64_t* slot_mapping, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            int32_t num_tokens, int32_t block_size, int32_t num_blocks,
                            int32_t common_prefix_len, void* stream);

/*
 * Measurement aid (not a step of the method): the practical HBM read
 * ceiling.  pa_stream_read_probe reads `bytes` (a positive multiple of 16)
 * of device memory at `buf` (16-byte aligned) exactly once, with the
 * 16-byte non-temporal loads the decode kernels use for K/V rows, and
 * writes one 32-bit XOR digest per workgroup to `sink` (device, uint32
 * [pa_stream_read_probe_sink_words()]) so that no load can be dropped.  One
 * launch on `stream`; timing it gives the read bandwidth that decode's
 * algorithmic bandwidth is compared with besides the published peak.
 */
int32_t pa_stream_read_probe_sink_words(void);
pa_status pa_stream_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * Block pool -- host-side block manager that hands out physical blocks and
 * builds block tables and slot mappings ([k4i] block manager, copy-on-write;
 * [vllm] §4.1 free queue; [atb] reference counting).  Host memory only; not
 * thread-safe (one pool per thread or external locking).
 *
 * Free blocks wait in a FIFO queue: allocation takes from the front, blocks
 * whose count drops to zero go to the back.  `free_order` (host, int32
 * [num_blocks], a permutation of 0..num_blocks-1; NULL = ascending) is the
 * initial queue.  Every operation is all-or-nothing: PA_ERR_OUT_OF_BLOCKS
 * leaves the pool unchanged.
 */
typedef struct pa_pool pa_pool;

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* free_order, pa_pool** out);
void pa_pool_destroy(pa_pool* pool);

/* New empty sequence; its id is written to *seq_id. */
pa_status pa_pool_add_seq(pa_pool* pool, int32_t* seq_id);

/* New sequence sharing every block of `parent` (each count + 1). */
pa_status pa_pool_fork(pa_pool* pool, int32_t parent, int32_t* child);

/*
 * Prefix cache ([k4i] #prefix-caching; [vllm] §4.2 allocation steps 1-5 and
 * §4.3 chained block hash).  New sequence holding a prompt of num_tokens
 * token ids (host int32): its full blocks are hashed in a chain
 * hash(parent hash, block's token ids, extra_key) and looked up from the
 * left; every cached block up to the first miss is reused (count + 1; a
 * block whose count was 0 leaves the free queue), the remaining blocks are
 * taken from the front of the free queue and the fresh full blocks are
 * registered (their K/V is the caller's to write, e.g. by prefill of the
 * uncached tokens).  *cached_tokens = reused blocks x block_size: the
 * caller skips attention/K-V computation for those positions.  extra_key
 * separates caches of different configurations (adapter, salt).  A block
 * freed to count 0 stays cached at the back of the queue; its entry is
 * dropped when the queue hands it out for new content (least recently
 * freed first).  Partial last blocks and blocks filled later by
 * pa_pool_append are not cached.  Hash matches are confirmed against the
 * stored token ids, so a collision is a miss.  All-or-nothing:
 * PA_ERR_OUT_OF_BLOCKS with no change when the queue is too short.
 */
pa_status pa_pool_add_seq_cached(pa_pool* pool, const int32_t* token_ids,
                                 int32_t num_tokens, uint64_t extra_key,
                                 int32_t* seq_id, int32_t* cached_tokens);
/* Number of blocks currently registered in the prefix cache. */
int32_t pa_pool_num_cached(const pa_pool* pool);

/*
 * Append n tokens to a sequence.  slots_out (host, int64 [n], may be NULL)
 * receives block * block_size + offset of each new position.  When the first
 * new token lands in a partly filled block shared with other sequences, the
 * block is copied first (copy-on-write): a free block is taken, the old
 * block's count drops by one and the table is repointed; the (source,
 * destination) pair is written to cow_pairs (host, int32 [cow_cap][2]) and
 * *n_cow counts the pairs (0 or 1).  The caller copies the pair's contents
 * (pa_copy_blocks) before writing the new tokens.  cow_cap < 1 with a copy
 * needed returns PA_ERR_INVALID_ARGUMENT with no change.
 */
pa_status pa_pool_append(pa_pool* pool, int32_t seq_id, int32_t n,
                         int64_t* slots_out, int32_t* cow_pairs,
                         int32_t cow_cap, int32_t* n_cow);

/* Release a sequence: every block's count drops by one; blocks at zero return
 * to the back of the free queue in table order. */
pa_status pa_pool_free_seq(pa_pool* pool, int32_t seq_id);

/* Copy a sequence's block table to out (host, int32 [cap]); *n = its length. */
pa_status pa_pool_block_table(const pa_pool* pool, int32_t seq_id, int32_t* out,
                              int32_t cap, int32_t* n);

/* Number of tokens of a sequence, or -1 for an unknown id. */
int32_t pa_pool_seq_len(const pa_pool* pool, int32_t seq_id);
int32_t pa_pool_num_free(const pa_pool* pool);
/* Reference count of a block, or -1 when out of range. */
int32_t pa_pool_refcount(const pa_pool* pool, int32_t block);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
