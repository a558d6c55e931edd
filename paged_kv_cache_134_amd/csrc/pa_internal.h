// Internal declarations shared by the library's translation units.
#ifndef PA_INTERNAL_H_
#define PA_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

// Records `msg` as the calling thread's last error and returns `st`.
pa_status pa_fail(pa_status st, const char* msg);

#ifdef __HIPCC__
#include <hip/hip_runtime.h>

namespace pa {

// Compute units of the current device (256 on MI355X), asked once.
int device_cus();

// Geometry of a paged K/V pool, in elements.
struct PoolGeom {
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t num_blocks;
  pa_layout layout;
};

hipError_t launch_reshape_and_cache(const void* key, const void* value, int64_t key_row_stride,
                                    int64_t value_row_stride, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    const PoolGeom& g, int elem_bytes, hipStream_t stream);

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, pa_dtype src_dtype,
                                        int64_t key_row_stride, int64_t value_row_stride,
                                        void* key_cache, void* value_cache,
                                        const int64_t* slot_mapping, int32_t num_tokens,
                                        const PoolGeom& g, float k_scale, float v_scale,
                                        hipStream_t stream);

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                              hipStream_t stream);

struct DecodeArgs {
  void* out;
  pa_dtype out_dtype;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  pa_dtype kv_dtype;        // cache element type
  pa_dtype q_dtype;         // query type (kv_dtype unless the cache is FP8)
  float k_scale = 1.f;      // FP8 caches: stored code value * scale = element
  float v_scale = 1.f;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;
  int32_t num_seqs;
  int32_t num_heads;
  PoolGeom geom;
  float scale;
  int32_t partition_size;  // 0 = single pass, > 0 = split-K
  int32_t max_partitions;  // ceil(max_context_len / partition_size) when split
  float* part_out;         // [num_seqs, max_partitions, num_heads, head_size]
  float* part_ml;          // [num_seqs, max_partitions, num_heads, 2] (max, sum)
  int32_t key_begin = 0;   // cascade: partitions cover [key_begin, L) ...
  int32_t part_base = 0;   // ... and start at this workspace partition
  bool all_partial = false;  // cascade: prefix partials exist, never finish a head early
  // Split-K dispatch list in the workspace (see launch_decode_main): item
  // count, then [items][4] int32 (sequence, kv head, partition, 0).
  int32_t* item_count = nullptr;
  int32_t* items = nullptr;
};

// Single pass (partition_size == 0) or the split-K partition kernel.
// Whether decode takes the grouped (matrix-core) kernel for this element type
// and group size G = num_heads / num_kv_heads.
bool decode_uses_group_kernel(pa_dtype kv_dtype, int G);

hipError_t launch_decode_main(const DecodeArgs& a, hipStream_t stream);
// Split-K reduce over the partials in part_out / part_ml.
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  pa_dtype out_dtype;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  pa_dtype kv_dtype;        // cache element type
  pa_dtype q_dtype;         // query type (kv_dtype unless the cache is FP8)
  float k_scale = 1.f;      // FP8 caches: stored code value * scale = element
  float v_scale = 1.f;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_query_len;
  int32_t num_heads;
  PoolGeom geom;
  float scale;
  // Shared-prefix mode (prefix_keys > 0): the num_tokens query rows attend,
  // without a causal mask, to keys [0, prefix_keys) through block_tables
  // row 0, in key partitions of key_part tokens; each (row, head, partition)
  // writes a (max, sum, unnormalised output) partial at workspace partition
  // index = key partition.
  int32_t prefix_keys = 0;
  int32_t key_part = 0;
  float* part_out = nullptr;
  float* part_ml = nullptr;
  int32_t max_partitions = 0;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
#endif  // __HIPCC__

#endif  // PA_INTERNAL_H_
