// C entry points: argument checks, workspace sizing, dispatch to the kernels.
// Everything here runs on the host; device work is only enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

bool pow2_in(int32_t v, int32_t lo, int32_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pa_dtype t) { return t == PA_F32 ? 4 : t == PA_FP8_E4M3 ? 1 : 2; }

// Types queries, outputs and 16-bit/fp32 caches are computed in.
bool valid_dtype(pa_dtype t) { return t == PA_F32 || t == PA_BF16 || t == PA_F16; }

// Types a cache may hold (bit copies accept every one).
bool valid_storage(pa_dtype t) { return valid_dtype(t) || t == PA_FP8_E4M3; }

bool finite_positive(float x) { return x > 0.f && x <= 3.4028234663852886e38f; }

bool valid_group(int32_t h, int32_t hkv) {
  if (h <= 0 || hkv <= 0 || h % hkv != 0) return false;
  const int32_t g = h / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
}

pa_status hip_fail(hipError_t e, const char* where) {
  std::string msg = std::string(where) + ": " + hipGetErrorString(e);
  return pa_fail(PA_ERR_HIP, msg.c_str());
}

constexpr int32_t kAutoSmallestPartition = 256;

int64_t partitions_for(int32_t max_context_len, int32_t partition_size) {
  return partition_size > 0 ? (max_context_len + (int64_t)partition_size - 1) / partition_size : 0;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Split-K workspace: partial outputs [S, parts, H, D] fp32, partial (max,
// sum) [S, parts, H, 2] fp32 (partition-major), then the dispatch list of the partition
// kernel: a 256-byte header (item count) and one 16-byte item per (sequence,
// kv head, partition), num_heads bounding num_kv_heads.  Each part starts on
// a 256-byte boundary.
size_t workspace_bytes(int64_t num_seqs, int64_t num_heads, int64_t head_size, int64_t parts) {
  const size_t out_b = (size_t)(num_seqs * num_heads * parts * head_size) * sizeof(float);
  const size_t ml_b = (size_t)(num_seqs * num_heads * parts * 2) * sizeof(float);
  const size_t items_b = 256 + (size_t)(num_seqs * num_heads * parts) * 4 * sizeof(int32_t);
  return round256(out_b) + round256(ml_b) + items_b;
}

}  // namespace

pa_status pa_fail(pa_status st, const char* msg) {
  g_last_error = msg ? msg : "";
  return st;
}

extern "C" const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_METADATA: return "PA_ERR_METADATA";
  }
  return "PA_ERR_UNKNOWN";
}

extern "C" const char* pa_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------ write
extern "C" pa_status pa_reshape_and_cache(const void* key, const void* value,
                                          int64_t key_row_stride, int64_t value_row_stride,
                                          void* key_cache, void* value_cache,
                                          const int64_t* slot_mapping, int32_t num_tokens,
                                          int32_t num_kv_heads, int32_t head_size,
                                          int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                                          pa_layout layout, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache: non-positive size");
  if (!valid_storage(dtype)) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache: bad dtype");
  if (layout != PA_LAYOUT_NHD && layout != PA_LAYOUT_HND)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache: bad layout");
  const int eb = elem_bytes(dtype);
  if ((head_size * eb) % 16 != 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: head_size * element size must be a multiple of 16 bytes");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache: null pointer");
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_row_stride < row || value_row_stride < row || (key_row_stride * eb) % 16 ||
      (value_row_stride * eb) % 16)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache: row stride too small or not 16-byte aligned");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache: pointers must be 16-byte aligned");
  pa::PoolGeom g{num_kv_heads, head_size, block_size, num_blocks, layout};
  hipError_t e = pa::launch_reshape_and_cache(key, value, key_row_stride, value_row_stride,
                                              key_cache, value_cache, slot_mapping, num_tokens, g,
                                              eb, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_reshape_and_cache");
}

extern "C" pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, pa_dtype src_dtype,
                                              int64_t key_row_stride, int64_t value_row_stride,
                                              void* key_cache, void* value_cache,
                                              const int64_t* slot_mapping, int32_t num_tokens,
                                              int32_t num_kv_heads, int32_t head_size,
                                              int32_t block_size, int32_t num_blocks,
                                              pa_layout layout, float k_scale, float v_scale,
                                              void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache_fp8: non-positive size");
  if (!valid_dtype(src_dtype))
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache_fp8: source dtype must be f32, bf16 or f16");
  if (layout != PA_LAYOUT_NHD && layout != PA_LAYOUT_HND)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache_fp8: bad layout");
  if (!finite_positive(k_scale) || !finite_positive(v_scale))
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache_fp8: scales must be positive and finite");
  if (head_size % 16 != 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache_fp8: head_size must be a multiple of 16");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache_fp8: null pointer");
  const int eb = elem_bytes(src_dtype);
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_row_stride < row || value_row_stride < row || (key_row_stride * eb) % 16 ||
      (value_row_stride * eb) % 16)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache_fp8: row stride too small or not 16-byte aligned");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_reshape_and_cache_fp8: pointers must be 16-byte aligned");
  pa::PoolGeom g{num_kv_heads, head_size, block_size, num_blocks, layout};
  hipError_t e = pa::launch_reshape_and_cache_fp8(key, value, src_dtype, key_row_stride,
                                                  value_row_stride, key_cache, value_cache,
                                                  slot_mapping, num_tokens, g, k_scale, v_scale,
                                                  (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_reshape_and_cache_fp8");
}

extern "C" pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_pairs,
                                    int32_t num_pairs, int32_t num_kv_heads, int32_t head_size,
                                    int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                                    void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_copy_blocks: non-positive size");
  if (!valid_storage(dtype)) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_copy_blocks: bad dtype");
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_pairs)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_copy_blocks: null pointer");
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_size * elem_bytes(dtype);
  if (block_bytes % 16 || !aligned16(key_cache) || !aligned16(value_cache))
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: blocks must be 16-byte multiples and aligned");
  hipError_t e = pa::launch_copy_blocks(key_cache, value_cache, block_pairs, num_pairs, block_bytes,
                                        num_blocks, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_copy_blocks");
}

extern "C" pa_status pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                                    void* dst_key_cache, void* dst_value_cache,
                                    const int32_t* block_pairs, int32_t num_pairs,
                                    int64_t block_bytes, int32_t src_num_blocks,
                                    int32_t dst_num_blocks, void* stream) {
  if (num_pairs < 0 || block_bytes <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_swap_blocks: non-positive size");
  if (num_pairs == 0) return PA_OK;
  if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !block_pairs)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_swap_blocks: null pointer");
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t sb = block_pairs[2 * i], db = block_pairs[2 * i + 1];
    if (sb < 0 || sb >= src_num_blocks || db < 0 || db >= dst_num_blocks)
      return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_swap_blocks: block id out of range");
  }
  const hipStream_t st = (hipStream_t)stream;
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int64_t so = (int64_t)block_pairs[2 * i] * block_bytes;
    const int64_t dof = (int64_t)block_pairs[2 * i + 1] * block_bytes;
    hipError_t e = hipMemcpyAsync(static_cast<char*>(dst_key_cache) + dof,
                                  static_cast<const char*>(src_key_cache) + so, block_bytes,
                                  hipMemcpyDefault, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(static_cast<char*>(dst_value_cache) + dof,
                         static_cast<const char*>(src_value_cache) + so, block_bytes,
                         hipMemcpyDefault, st);
    if (e != hipSuccess) return hip_fail(e, "pa_swap_blocks");
  }
  return PA_OK;
}

// ----------------------------------------------------------------- decode
namespace pa {

int device_cus() {
  static std::atomic<int> cus{0};
  int c = cus.load(std::memory_order_relaxed);
  if (c == 0) {
    int dev = 0, n = 0;
    c = hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                n > 0
            ? n
            : 256;
    cus.store(c, std::memory_order_relaxed);
  }
  return c;
}

}  // namespace pa

// Per-head kernel: 512-token partitions as soon as a context is longer.
// Grouped kernel (one workgroup reads a kv head for all G query heads, so a
// workgroup has G times the work per token): the largest power-of-two
// partition, at least 512 and shorter than the longest context, that still
// leaves about three workgroups per compute unit (estimated) for balance; a
// workgroup's fixed costs (block-table window, the first tiles' latency, the
// merge, the partial, and its share of deriving the dispatch order) are then
// spread over as many tiles as possible.  The same target serves FP8
// caches, though their kernel holds 3 workgroups per compute unit at head
// size 128 rather than 2.  (Long-context batch, 16-bit: 739 / 700 / 669 /
// 651 / 645 us at 512 / 1024 / 2048 / 4096 / 8192.  70B-like lognormal
// batch, partition span: 168 / 150 / 143 us at 512 / 1024 / 2048 with the
// list kernel; with the order derived in the kernel 141.3-142.3 us at 2048
// and 139.2-139.5 us at 4096, FP8 85.4 / 80.2 / 76.1 us at 1024 / 2048 /
// 4096.  Long context FP8: 336 us at both 4096 and 8192.)
extern "C" int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, pa_dtype kv_dtype,
                                            int32_t max_context_len, int64_t total_context_len) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_heads <= 0 || max_context_len <= 512) return 0;
  if (!pa::decode_uses_group_kernel(kv_dtype, num_heads / num_kv_heads)) return 512;
  const int64_t total = total_context_len > 0 ? total_context_len
                                              : (int64_t)num_seqs * max_context_len;
  const int64_t want = 3 * (int64_t)pa::device_cus();
  for (int32_t ps = 8192; ps > 512; ps /= 2) {
    if (ps >= max_context_len) continue;
    const int64_t wgs = (int64_t)num_kv_heads * (total / ps + num_seqs / 2);
    if (wgs >= want) return ps;
  }
  return 512;
}

extern "C" size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                           int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_size <= 0 || max_context_len <= 0) return 0;
  const int32_t ps = partition_size < 0 ? kAutoSmallestPartition : partition_size;
  if (ps == 0) return 0;
  return workspace_bytes(num_seqs, num_heads, head_size, partitions_for(max_context_len, ps));
}

namespace {

// Checks shared by the decode entry points; fills `a` (workspace pointers
// included when split) and resolves partition_size -1.
pa_status decode_prepare(const char* fn, void* out, pa_dtype out_dtype, const void* query,
                         pa_dtype q_dtype, const void* key_cache, const void* value_cache,
                         pa_dtype kv_dtype, pa_layout layout, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int32_t num_blocks, float scale,
                         int32_t partition_size, void* workspace, size_t workspace_bytes_,
                         bool need_out, bool need_cache, pa::DecodeArgs* a) {
  char msg[200];
  auto fail = [&](pa_status st, const char* what) {
    std::snprintf(msg, sizeof msg, "%s: %s", fn, what);
    return pa_fail(st, msg);
  };
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "negative size or no blocks");
  if (kv_dtype == PA_FP8_E4M3) {
    if ((q_dtype != PA_BF16 && q_dtype != PA_F16) || (out_dtype != PA_F32 && out_dtype != q_dtype))
      return fail(PA_ERR_INVALID_ARGUMENT, "FP8 cache: query must be bf16 or f16, out f32 or the query type");
  } else if (!valid_dtype(kv_dtype) || q_dtype != kv_dtype ||
             (out_dtype != PA_F32 && out_dtype != kv_dtype)) {
    return fail(PA_ERR_INVALID_ARGUMENT, "bad kv/out dtype");
  }
  if (layout != PA_LAYOUT_NHD && layout != PA_LAYOUT_HND)
    return fail(PA_ERR_INVALID_ARGUMENT, "bad layout");
  if (!valid_group(num_heads, num_kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "num_heads / num_kv_heads must be 1, 2, 4, 8 or 16");
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_size must be 64 or 128");
  if (!pow2_in(block_size, 1, 1024))
    return fail(PA_ERR_UNSUPPORTED, "block_size must be a power of two in [1, 1024]");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len exceeds max_blocks_per_seq * block_size");
  if (partition_size < -1 || (partition_size > 0 && partition_size % 16 != 0))
    return fail(PA_ERR_INVALID_ARGUMENT, "partition_size must be -1, 0 or a positive multiple of 16");
  if (!(scale == scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale is NaN");
  if ((int64_t)num_seqs * num_kv_heads > 0x7FFFFFFF || (int64_t)num_seqs * num_heads > 0x7FFFFFFF)
    return fail(PA_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
  int32_t ps = partition_size < 0 ? pa_decode_auto_partition(num_seqs, num_heads, num_kv_heads,
                                                              kv_dtype, max_context_len, 0)
                                  : partition_size;
  const int64_t parts = partitions_for(max_context_len, ps);
  if (ps > 0 && parts == 0) ps = 0;  // empty contexts: nothing to split
  if (ps > 0 && parts > 65535) return fail(PA_ERR_UNSUPPORTED, "more than 65535 partitions");
  *a = pa::DecodeArgs{};
  a->out = out;
  a->out_dtype = out_dtype;
  a->query = query;
  a->key_cache = key_cache;
  a->value_cache = value_cache;
  a->kv_dtype = kv_dtype;
  a->q_dtype = q_dtype;
  a->block_tables = block_tables;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->context_lens = context_lens;
  a->max_context_len = max_context_len;
  a->num_seqs = num_seqs;
  a->num_heads = num_heads;
  a->geom = pa::PoolGeom{num_kv_heads, head_size, block_size, num_blocks, layout};
  a->scale = scale;
  a->partition_size = ps;
  if (num_seqs == 0) return PA_OK;
  if (!context_lens || (need_out && !out))
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer");
  if (need_cache) {
    if (!query || !key_cache || !value_cache || !block_tables)
      return fail(PA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
      return fail(PA_ERR_INVALID_ARGUMENT, "query and caches must be 16-byte aligned");
  }
  if (ps > 0) {
    const size_t need = workspace_bytes(num_seqs, num_heads, head_size, parts);
    if (!workspace || workspace_bytes_ < need) {
      std::snprintf(msg, sizeof msg, "%s: split-K needs %zu workspace bytes, got %zu", fn, need,
                    workspace ? workspace_bytes_ : (size_t)0);
      return pa_fail(PA_ERR_WORKSPACE_TOO_SMALL, msg);
    }
    if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    a->max_partitions = (int32_t)parts;
    const size_t out_b = (size_t)num_seqs * num_heads * parts * head_size * sizeof(float);
    const size_t ml_b = (size_t)num_seqs * num_heads * parts * 2 * sizeof(float);
    char* w = static_cast<char*>(workspace);
    a->part_out = reinterpret_cast<float*>(w);
    a->part_ml = reinterpret_cast<float*>(w + round256(out_b));
    a->item_count = reinterpret_cast<int32_t*>(w + round256(out_b) + round256(ml_b));
    a->items = a->item_count + 64;  // after the 256-byte header
  }
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode(void* out, pa_dtype out_dtype, const void* query,
                               const void* key_cache, const void* value_cache, pa_dtype kv_dtype,
                               pa_layout layout, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                               int32_t num_blocks, float scale, int32_t partition_size,
                               void* workspace, size_t workspace_bytes_, void* stream) {
  if (kv_dtype == PA_FP8_E4M3)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: FP8 caches are read by pa_decode_fp8");
  pa::DecodeArgs a;
  pa_status st = decode_prepare("pa_decode", out, out_dtype, query, kv_dtype, key_cache, value_cache,
                                kv_dtype, layout, block_tables, max_blocks_per_seq, context_lens,
                                max_context_len, num_seqs, num_heads, num_kv_heads, head_size,
                                block_size, num_blocks, scale, partition_size, workspace,
                                workspace_bytes_, true, true, &a);
  if (st != PA_OK || num_seqs == 0) return st;
  hipError_t e = pa::launch_decode_main(a, (hipStream_t)stream);
  if (e == hipSuccess) e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode");
}

namespace {

// pa_decode_fp8 (with_reduce) and pa_decode_partitions_fp8.
pa_status decode_fp8(const char* fn, bool with_reduce, void* out, pa_dtype out_dtype,
                     const void* query, pa_dtype q_dtype, const void* key_cache,
                     const void* value_cache, float k_scale, float v_scale, pa_layout layout,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                     int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                     void* workspace, size_t workspace_bytes_, void* stream) {
  char msg[160];
  if (!finite_positive(k_scale) || !finite_positive(v_scale)) {
    std::snprintf(msg, sizeof msg, "%s: scales must be positive and finite", fn);
    return pa_fail(PA_ERR_INVALID_ARGUMENT, msg);
  }
  pa::DecodeArgs a;
  pa_status st = decode_prepare(fn, out, out_dtype, query, q_dtype, key_cache, value_cache,
                                PA_FP8_E4M3, layout, block_tables, max_blocks_per_seq,
                                context_lens, max_context_len, num_seqs, num_heads, num_kv_heads,
                                head_size, block_size, num_blocks, scale, partition_size,
                                workspace, workspace_bytes_, true, true, &a);
  if (st != PA_OK || num_seqs == 0 || (!with_reduce && a.partition_size == 0)) return st;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  hipError_t e = pa::launch_decode_main(a, (hipStream_t)stream);
  if (e == hipSuccess && with_reduce) e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, fn);
}

}  // namespace

extern "C" pa_status pa_decode_fp8(void* out, pa_dtype out_dtype, const void* query,
                                   pa_dtype q_dtype, const void* key_cache,
                                   const void* value_cache, float k_scale, float v_scale,
                                   pa_layout layout, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                   int32_t num_blocks, float scale, int32_t partition_size,
                                   void* workspace, size_t workspace_bytes_, void* stream) {
  return decode_fp8("pa_decode_fp8", true, out, out_dtype, query, q_dtype, key_cache, value_cache,
                    k_scale, v_scale, layout, block_tables, max_blocks_per_seq, context_lens,
                    max_context_len, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                    num_blocks, scale, partition_size, workspace, workspace_bytes_, stream);
}

extern "C" pa_status pa_decode_partitions_fp8(
    void* out, pa_dtype out_dtype, const void* query, pa_dtype q_dtype, const void* key_cache,
    const void* value_cache, float k_scale, float v_scale, pa_layout layout,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes_, void* stream) {
  if (partition_size <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_partitions_fp8: partition_size must be > 0");
  return decode_fp8("pa_decode_partitions_fp8", false, out, out_dtype, query, q_dtype, key_cache,
                    value_cache, k_scale, v_scale, layout, block_tables, max_blocks_per_seq,
                    context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_size,
                    block_size, num_blocks, scale, partition_size, workspace, workspace_bytes_,
                    stream);
}

extern "C" pa_status pa_decode_partitions(void* out, pa_dtype out_dtype, const void* query,
                                          const void* key_cache,
                                          const void* value_cache, pa_dtype kv_dtype,
                                          pa_layout layout, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t max_context_len, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_size, int32_t block_size, int32_t num_blocks,
                                          float scale, int32_t partition_size, void* workspace,
                                          size_t workspace_bytes_, void* stream) {
  if (partition_size <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_partitions: partition_size must be > 0");
  if (kv_dtype == PA_FP8_E4M3)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_partitions: FP8 caches are read by pa_decode_fp8");
  pa::DecodeArgs a;
  pa_status st = decode_prepare("pa_decode_partitions", out, out_dtype, query, kv_dtype, key_cache,
                                value_cache, kv_dtype, layout, block_tables, max_blocks_per_seq,
                                context_lens, max_context_len, num_seqs, num_heads, num_kv_heads,
                                head_size, block_size, num_blocks, scale, partition_size, workspace,
                                workspace_bytes_, true, true, &a);
  if (st != PA_OK || num_seqs == 0 || a.partition_size == 0) return st;
  hipError_t e = pa::launch_decode_main(a, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode_partitions");
}

extern "C" pa_status pa_decode_reduce(void* out, pa_dtype out_dtype, const int32_t* context_lens,
                                      int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_size,
                                      int32_t partition_size, const void* workspace,
                                      size_t workspace_bytes_, void* stream) {
  if (partition_size <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_reduce: partition_size must be > 0");
  pa::DecodeArgs a;
  // the reduce reads no cache: geometry fields are placeholders that pass the checks
  pa_status st = decode_prepare("pa_decode_reduce", out, out_dtype, nullptr, out_dtype, nullptr,
                                nullptr, out_dtype, PA_LAYOUT_NHD, nullptr,
                                max_context_len, context_lens, max_context_len, num_seqs,
                                num_heads, num_kv_heads, head_size, 1, 1, 1.0f, partition_size,
                                const_cast<void*>(workspace), workspace_bytes_, true, false, &a);
  if (st != PA_OK || num_seqs == 0 || a.partition_size == 0) return st;
  hipError_t e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode_reduce");
}

// ---------------------------------------------------------------- cascade
namespace {

// Shared-prefix pass: key partitions sized so that (heads x query tiles x
// partitions) is about 256 workgroups, in multiples of 64 keys.  (Shared-
// prefix workload, 100 sequences x 32 heads over 2,000 common keys: 149.5 us
// for the whole cascade at 256 workgroups of 256 keys, 152.7-156 us at 512
// of 128 keys, 166 us at 1,024 of 64; FP8 92.7 vs 97 us at 512: fewer,
// longer workgroups write fewer partials and pay their start-up less often.)
int32_t cascade_key_part(int32_t num_seqs, int32_t num_heads, int32_t prefix) {
  const int64_t qt = (num_seqs + 127) / 128;
  const int64_t per = (int64_t)num_heads * qt;
  const int64_t parts = std::max<int64_t>(1, (256 + per - 1) / per);
  const int64_t kp = (prefix + parts - 1) / parts;
  return (int32_t)std::max<int64_t>(64, (kp + 63) / 64 * 64);
}

int64_t cascade_suffix_parts(int32_t max_context_len, int32_t prefix, int32_t ps) {
  return max_context_len > prefix ? (max_context_len - prefix + (int64_t)ps - 1) / ps : 0;
}

}  // namespace

extern "C" size_t pa_decode_cascade_workspace_size(int32_t num_seqs, int32_t num_heads,
                                                   int32_t head_size, int32_t max_context_len,
                                                   int32_t common_prefix_len,
                                                   int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_size <= 0 || common_prefix_len <= 0 ||
      max_context_len < common_prefix_len || partition_size < -1)
    return 0;
  const int32_t kp = cascade_key_part(num_seqs, num_heads, common_prefix_len);
  const int64_t npp = (common_prefix_len + kp - 1) / kp;
  const int32_t suffix = max_context_len - common_prefix_len;
  const int32_t ps = partition_size > 0 ? partition_size
                     : partition_size < 0 ? kAutoSmallestPartition
                                          : std::max(16, (suffix + 15) / 16 * 16);
  return workspace_bytes(num_seqs, num_heads, head_size,
                         npp + cascade_suffix_parts(max_context_len, common_prefix_len, ps));
}

namespace {

// pa_decode_cascade (q_dtype == kv_dtype, 16-bit) and pa_decode_cascade_fp8.
pa_status cascade_impl(const char* fn, void* out, pa_dtype out_dtype, const void* query,
                       pa_dtype q_dtype, const void* key_cache, const void* value_cache,
                       pa_dtype kv_dtype, float k_scale, float v_scale, pa_layout layout,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t max_context_len,
                       int32_t common_prefix_len, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                       int32_t num_blocks, float scale, int32_t partition_size, void* workspace,
                       size_t workspace_bytes_, void* stream) {
  char msg[200];
  auto fail = [&](pa_status st, const char* what) {
    std::snprintf(msg, sizeof msg, "%s: %s", fn, what);
    return pa_fail(st, msg);
  };
  if (!finite_positive(k_scale) || !finite_positive(v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "scales must be positive and finite");
  pa::DecodeArgs a;
  pa_status st = decode_prepare(fn, out, out_dtype, query, q_dtype, key_cache, value_cache,
                                kv_dtype, layout, block_tables, max_blocks_per_seq, context_lens,
                                max_context_len, num_seqs, num_heads, num_kv_heads, head_size,
                                block_size, num_blocks, scale, 0, nullptr, 0, true, true, &a);
  if (st != PA_OK) return st;
  if (q_dtype != PA_BF16 && q_dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "the shared-prefix pass needs bf16 or f16 queries and caches (or FP8 caches)");
  if (common_prefix_len <= 0 || common_prefix_len % block_size != 0 ||
      common_prefix_len > max_context_len)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "common_prefix_len must be a positive multiple of block_size and at most max_context_len");
  if (partition_size < -1 || (partition_size > 0 && partition_size % 16 != 0))
    return fail(PA_ERR_INVALID_ARGUMENT, "partition_size must be -1, 0 or a positive multiple of 16");
  if (num_seqs == 0) return PA_OK;
  const int32_t suffix = max_context_len - common_prefix_len;
  int32_t ps = partition_size > 0 ? partition_size
               : partition_size < 0 ? pa_decode_auto_partition(num_seqs, num_heads, num_kv_heads,
                                                              kv_dtype, suffix, 0)
                                    : 0;
  if (ps <= 0) ps = std::max(16, (suffix + 15) / 16 * 16);  // one partition per suffix
  const int32_t kp = cascade_key_part(num_seqs, num_heads, common_prefix_len);
  const int64_t npp = (common_prefix_len + kp - 1) / kp;
  const int64_t parts = npp + cascade_suffix_parts(max_context_len, common_prefix_len, ps);
  if (parts > 65535) return fail(PA_ERR_UNSUPPORTED, "more than 65535 partitions");
  const size_t need = workspace_bytes(num_seqs, num_heads, head_size, parts);
  if (!workspace || workspace_bytes_ < need) {
    std::snprintf(msg, sizeof msg, "%s: needs %zu workspace bytes, got %zu", fn, need,
                  workspace ? workspace_bytes_ : (size_t)0);
    return pa_fail(PA_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  if (!aligned16(workspace) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARGUMENT, "workspace and out must be 16-byte aligned");
  const size_t out_b = (size_t)num_seqs * num_heads * parts * head_size * sizeof(float);
  a.partition_size = ps;
  a.max_partitions = (int32_t)parts;
  a.part_out = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256(out_b));
  a.key_begin = common_prefix_len;
  a.part_base = (int32_t)npp;
  a.all_partial = true;
  a.k_scale = k_scale;
  a.v_scale = v_scale;

  // 1. shared prefix: every sequence's query against the common blocks
  //    (block_tables row 0), once, on matrix cores
  pa::PrefillArgs pr{};
  pr.query = query;
  pr.key_cache = key_cache;
  pr.value_cache = value_cache;
  pr.kv_dtype = kv_dtype;
  pr.q_dtype = q_dtype;
  pr.k_scale = k_scale;
  pr.v_scale = v_scale;
  pr.out_dtype = PA_F32;
  pr.block_tables = block_tables;
  pr.max_blocks_per_seq = max_blocks_per_seq;
  pr.num_seqs = 1;
  pr.num_tokens = num_seqs;
  pr.max_query_len = 1;
  pr.num_heads = num_heads;
  pr.geom = a.geom;
  pr.scale = scale;
  pr.prefix_keys = common_prefix_len;
  pr.key_part = kp;
  pr.part_out = a.part_out;
  pr.part_ml = a.part_ml;
  pr.max_partitions = (int32_t)parts;
  hipError_t e = pa::launch_prefill(pr, (hipStream_t)stream);
  // 2. each sequence's own keys [common_prefix_len, L), 3. merge of all partials
  if (e == hipSuccess) e = pa::launch_decode_main(a, (hipStream_t)stream);
  if (e == hipSuccess) e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, fn);
}

}  // namespace

extern "C" pa_status pa_decode_cascade(void* out, pa_dtype out_dtype, const void* query,
                                       const void* key_cache, const void* value_cache,
                                       pa_dtype kv_dtype, pa_layout layout,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       int32_t common_prefix_len, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                       int32_t block_size, int32_t num_blocks, float scale,
                                       int32_t partition_size, void* workspace,
                                       size_t workspace_bytes_, void* stream) {
  if (kv_dtype == PA_FP8_E4M3)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_cascade: FP8 caches are read by pa_decode_cascade_fp8");
  return cascade_impl("pa_decode_cascade", out, out_dtype, query, kv_dtype, key_cache, value_cache,
                      kv_dtype, 1.f, 1.f, layout, block_tables, max_blocks_per_seq, context_lens,
                      max_context_len, common_prefix_len, num_seqs, num_heads, num_kv_heads,
                      head_size, block_size, num_blocks, scale, partition_size, workspace,
                      workspace_bytes_, stream);
}

extern "C" pa_status pa_decode_cascade_fp8(
    void* out, pa_dtype out_dtype, const void* query, pa_dtype q_dtype, const void* key_cache,
    const void* value_cache, float k_scale, float v_scale, pa_layout layout,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t max_context_len, int32_t common_prefix_len, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes_, void* stream) {
  return cascade_impl("pa_decode_cascade_fp8", out, out_dtype, query, q_dtype, key_cache,
                      value_cache, PA_FP8_E4M3, k_scale, v_scale, layout, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, common_prefix_len,
                      num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks, scale,
                      partition_size, workspace, workspace_bytes_, stream);
}

// ---------------------------------------------------------------- prefill
namespace {

// pa_prefill (q_dtype == kv_dtype, 16-bit) and pa_prefill_fp8.
pa_status prefill_impl(const char* fn, void* out, pa_dtype out_dtype, const void* query,
                       pa_dtype q_dtype, const void* key_cache, const void* value_cache,
                       pa_dtype kv_dtype, float k_scale, float v_scale, pa_layout layout,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* query_start_loc, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                       int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int32_t num_blocks, float scale,
                       void* stream) {
  char msg[200];
  auto fail = [&](pa_status st, const char* what) {
    std::snprintf(msg, sizeof msg, "%s: %s", fn, what);
    return pa_fail(st, msg);
  };
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || max_context_len < 0 ||
      max_blocks_per_seq < 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "negative size or no blocks");
  if (q_dtype != PA_BF16 && q_dtype != PA_F16)
    return fail(valid_storage(q_dtype) ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARGUMENT,
                "query (and 16-bit cache) dtype must be bf16 or f16");
  if (out_dtype != PA_F32 && out_dtype != q_dtype)
    return fail(PA_ERR_INVALID_ARGUMENT, "out dtype must be f32 or the query dtype");
  if (layout != PA_LAYOUT_NHD && layout != PA_LAYOUT_HND)
    return fail(PA_ERR_INVALID_ARGUMENT, "bad layout");
  if (!valid_group(num_heads, num_kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "num_heads / num_kv_heads must be 1, 2, 4, 8 or 16");
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_size must be 64 or 128");
  if (!pow2_in(block_size, 1, 1024))
    return fail(PA_ERR_UNSUPPORTED, "block_size must be a power of two in [1, 1024]");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len exceeds max_blocks_per_seq * block_size");
  if (max_query_len > max_context_len)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_query_len exceeds max_context_len");
  if (num_heads > 65535 || num_seqs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "at most 65535 heads and 65535 sequences");
  if (!(scale == scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale is NaN");
  if (!finite_positive(k_scale) || !finite_positive(v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "scales must be positive and finite");
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !query_start_loc ||
      !context_lens)
    return fail(PA_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "out, query and caches must be 16-byte aligned");
  pa::PrefillArgs a{};
  a.out = out;
  a.out_dtype = out_dtype;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.kv_dtype = kv_dtype;
  a.q_dtype = q_dtype;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.query_start_loc = query_start_loc;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.num_heads = num_heads;
  a.geom = pa::PoolGeom{num_kv_heads, head_size, block_size, num_blocks, layout};
  a.scale = scale;
  hipError_t e = pa::launch_prefill(a, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, fn);
}

}  // namespace

extern "C" pa_status pa_prefill(void* out, pa_dtype out_dtype, const void* query,
                                const void* key_cache, const void* value_cache, pa_dtype kv_dtype,
                                pa_layout layout, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* query_start_loc,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                                int32_t max_query_len, int32_t max_context_len, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                int32_t num_blocks, float scale, void* stream) {
  if (kv_dtype == PA_FP8_E4M3)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_prefill: FP8 caches are read by pa_prefill_fp8");
  return prefill_impl("pa_prefill", out, out_dtype, query, kv_dtype, key_cache, value_cache,
                      kv_dtype, 1.f, 1.f, layout, block_tables, max_blocks_per_seq,
                      query_start_loc, context_lens, num_seqs, num_tokens, max_query_len,
                      max_context_len, num_heads, num_kv_heads, head_size, block_size,
                      num_blocks, scale, stream);
}

extern "C" pa_status pa_prefill_fp8(void* out, pa_dtype out_dtype, const void* query,
                                    pa_dtype q_dtype, const void* key_cache,
                                    const void* value_cache, float k_scale, float v_scale,
                                    pa_layout layout, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* query_start_loc,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_tokens, int32_t max_query_len,
                                    int32_t max_context_len, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                    int32_t num_blocks, float scale, void* stream) {
  return prefill_impl("pa_prefill_fp8", out, out_dtype, query, q_dtype, key_cache, value_cache,
                      PA_FP8_E4M3, k_scale, v_scale, layout, block_tables, max_blocks_per_seq,
                      query_start_loc, context_lens, num_seqs, num_tokens, max_query_len,
                      max_context_len, num_heads, num_kv_heads, head_size, block_size,
                      num_blocks, scale, stream);
}

// ----------------------------------------------------------- metadata check
extern "C" pa_status pa_check_metadata(const int32_t* block_tables, const int32_t* context_lens,
                                       const int64_t* slot_mapping, int32_t num_seqs,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t num_tokens, int32_t block_size, int32_t num_blocks,
                                       int32_t common_prefix_len, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || num_tokens < 0 ||
      block_size <= 0 || num_blocks <= 0 || common_prefix_len < 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_check_metadata: bad sizes");
  if (common_prefix_len > 0 && (!block_tables || !context_lens))
    return pa_fail(PA_ERR_INVALID_ARGUMENT,
                   "pa_check_metadata: the shared-prefix check needs block_tables and context_lens");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pa_check_metadata: synchronize");
  char msg[200];
  auto bad = [&](const char* fmt, auto... a) {
    std::snprintf(msg, sizeof msg, fmt, a...);
    return pa_fail(PA_ERR_METADATA, msg);
  };
  std::vector<int32_t> lens;
  if (context_lens && num_seqs) {
    lens.resize(num_seqs);
    e = hipMemcpy(lens.data(), context_lens, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "pa_check_metadata: copy context_lens");
    const int64_t cap = block_tables ? (int64_t)max_blocks_per_seq * block_size : INT64_MAX;
    for (int32_t s = 0; s < num_seqs; ++s) {
      if (lens[s] < 0 || lens[s] > max_context_len)
        return bad("context_lens[%d] = %d outside [0, max_context_len = %d]", s, lens[s],
                   max_context_len);
      if (lens[s] > cap)
        return bad("context_lens[%d] = %d exceeds the table's %lld slots", s, lens[s],
                   (long long)cap);
      if (lens[s] < common_prefix_len)
        return bad("context_lens[%d] = %d is shorter than common_prefix_len = %d", s, lens[s],
                   common_prefix_len);
    }
  }
  if (common_prefix_len % block_size != 0)
    return bad("common_prefix_len = %d is not a multiple of block_size = %d", common_prefix_len,
               block_size);
  if (block_tables && num_seqs && max_blocks_per_seq) {
    std::vector<int32_t> bt((size_t)num_seqs * max_blocks_per_seq);
    e = hipMemcpy(bt.data(), block_tables, sizeof(int32_t) * bt.size(), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "pa_check_metadata: copy block_tables");
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int64_t used = lens.empty() ? max_blocks_per_seq
                                        : ((int64_t)lens[s] + block_size - 1) / block_size;
      for (int64_t i = 0; i < used; ++i) {
        const int32_t b = bt[(size_t)s * max_blocks_per_seq + i];
        if (b < 0 || b >= num_blocks)
          return bad("block_tables[%d][%lld] = %d outside [0, %d)", s, (long long)i, b, num_blocks);
      }
    }
    const int32_t nbc = common_prefix_len / block_size;  // <= every row's used entries
    for (int32_t s = 1; s < num_seqs; ++s)
      for (int32_t i = 0; i < nbc; ++i)
        if (bt[(size_t)s * max_blocks_per_seq + i] != bt[i])
          return bad("block_tables[%d][%d] = %d differs from row 0's shared block %d", s, i,
                     bt[(size_t)s * max_blocks_per_seq + i], bt[i]);
  }
  if (slot_mapping && num_tokens) {
    std::vector<int64_t> sl(num_tokens);
    e = hipMemcpy(sl.data(), slot_mapping, sizeof(int64_t) * num_tokens, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "pa_check_metadata: copy slot_mapping");
    const int64_t nslots = (int64_t)num_blocks * block_size;
    std::vector<char> seen((size_t)nslots, 0);
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (sl[i] < 0) continue;
      if (sl[i] >= nslots) return bad("slot_mapping[%d] = %lld out of range [0, %lld)", i,
                                      (long long)sl[i], (long long)nslots);
      if (seen[sl[i]]) return bad("slot_mapping[%d] = %lld repeats an earlier slot", i,
                                  (long long)sl[i]);
      seen[sl[i]] = 1;
    }
  }
  return PA_OK;
}
