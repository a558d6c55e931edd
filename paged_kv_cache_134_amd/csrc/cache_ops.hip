// Cache write (slot_mapping scatter, plain or quantising to FP8) and
// whole-block copies.
//
// The scatter follows the cache-write kernels of "PagedAttention 在 vLLM 中的实现
// 分析" (§6.3, §7.4): every new token carries a global slot
// block * block_size + offset, a negative slot marks padding and is skipped.
// Here one workgroup moves one token row ([num_kv_heads, head_size] of K and
// of V) with 16-byte vector loads and stores; the row is contiguous in the
// source, and in the pool it is contiguous (NHD) or split into num_kv_heads
// head rows of head_size elements (HND).  The copy is a bit copy, so only the
// element width matters.
#include <hip/hip_runtime.h>

#include "kernel_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWriteThreads = 256;

// 16-byte chunk index helpers: a head row has `hc` chunks (head_size * elem / 16).
template <int LAYOUT>
__global__ __launch_bounds__(kWriteThreads) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, int64_t key_stride16,
    int64_t value_stride16, uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int32_t num_kv_heads, int32_t hc, int32_t block_size) {
  const int64_t token = blockIdx.x;
  const int64_t slot = slot_mapping[token];
  if (slot < 0) return;  // padding row
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int32_t row_chunks = num_kv_heads * hc;
  const uint4* k_src = key + token * key_stride16;
  const uint4* v_src = value + token * value_stride16;
  for (int32_t c = threadIdx.x; c < row_chunks; c += kWriteThreads) {
    int64_t dst;
    if (LAYOUT == PA_LAYOUT_NHD) {
      dst = (blk * block_size + off) * row_chunks + c;
    } else {
      const int32_t h = c / hc;
      const int32_t d = c - h * hc;
      dst = ((blk * num_kv_heads + h) * block_size + off) * hc + d;
    }
    const uint4 kv = k_src[c];
    const uint4 vv = v_src[c];
    key_cache[dst] = kv;
    value_cache[dst] = vv;
  }
}

// Quantising write into FP8 (E4M3) pools: one thread per 16-code chunk of a
// row.  Code = nearest E4M3 of x / scale (fp32 quotient, clamped to +-448
// first because the conversion instruction does not saturate); a NaN
// element is stored as 0x7F with the element's sign bit.
template <pa_dtype ST>
__device__ __forceinline__ uint4 quantize16(const char* src, float scale) {
  float x[16];
  if constexpr (ST == PA_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 c = load16(src + 16 * j);
      x[4 * j] = __uint_as_float(c.x);
      x[4 * j + 1] = __uint_as_float(c.y);
      x[4 * j + 2] = __uint_as_float(c.z);
      x[4 * j + 3] = __uint_as_float(c.w);
    }
  } else {
    chunk_to_f32<ST>(load16(src), x);
    chunk_to_f32<ST>(load16(src + 16), x + 8);
  }
  uint32_t nan_mask = 0, neg_mask = 0;  // per element: NaN source, sign bit of the source
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    nan_mask |= (uint32_t)(x[e] != x[e]) << e;
    neg_mask |= (__float_as_uint(x[e]) >> 31) << e;
    x[e] = e4m3_saturate(x[e] / scale);
  }
  uint32_t w[4] = {f32x4_to_fp8x4(x[0], x[1], x[2], x[3]), f32x4_to_fp8x4(x[4], x[5], x[6], x[7]),
                   f32x4_to_fp8x4(x[8], x[9], x[10], x[11]),
                   f32x4_to_fp8x4(x[12], x[13], x[14], x[15])};
  if (nan_mask) {  // rare: a NaN element is stored as 0x7F with its sign bit
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if ((nan_mask >> e) & 1u) {
        const uint32_t code = 0x7Fu | (((neg_mask >> e) & 1u) << 7);
        const int sh = 8 * (e % 4);
        w[e / 4] = (w[e / 4] & ~(0xFFu << sh)) | (code << sh);
      }
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int LAYOUT, pa_dtype ST>
__global__ __launch_bounds__(kWriteThreads) void reshape_and_cache_fp8_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride_b,
    int64_t value_stride_b, uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int32_t num_kv_heads, int32_t hc, int32_t block_size,
    float k_scale, float v_scale) {
  constexpr int kSrcChunk = 16 * Fmt<ST>::kBytes;  // source bytes of 16 elements
  const int64_t token = blockIdx.x;
  const int64_t slot = slot_mapping[token];
  if (slot < 0) return;  // padding row
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int32_t row_chunks = num_kv_heads * hc;
  const char* k_src = key + token * key_stride_b;
  const char* v_src = value + token * value_stride_b;
  for (int32_t c = threadIdx.x; c < row_chunks; c += kWriteThreads) {
    int64_t dst;
    if (LAYOUT == PA_LAYOUT_NHD) {
      dst = (blk * block_size + off) * row_chunks + c;
    } else {
      const int32_t h = c / hc;
      const int32_t d = c - h * hc;
      dst = ((blk * num_kv_heads + h) * block_size + off) * hc + d;
    }
    key_cache[dst] = quantize16<ST>(k_src + (int64_t)c * kSrcChunk, k_scale);
    value_cache[dst] = quantize16<ST>(v_src + (int64_t)c * kSrcChunk, v_scale);
  }
}

template <int LAYOUT>
hipError_t launch_fp8_write(const void* key, const void* value, int64_t ks_b, int64_t vs_b,
                            void* key_cache, void* value_cache, const int64_t* slot_mapping,
                            int32_t num_tokens, const PoolGeom& g, pa_dtype src, float k_scale,
                            float v_scale, hipStream_t stream) {
  const int32_t hc = g.head_size / 16;
  dim3 grid(num_tokens), block(kWriteThreads);
#define PA_FP8_WRITE(ST)                                                                       \
  hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<LAYOUT, ST>), grid, block, 0, stream,       \
                     (const char*)key, (const char*)value, ks_b, vs_b, (uint4*)key_cache,      \
                     (uint4*)value_cache, slot_mapping, g.num_kv_heads, hc, g.block_size,      \
                     k_scale, v_scale)
  switch (src) {
    case PA_F32: PA_FP8_WRITE(PA_F32); break;
    case PA_BF16: PA_FP8_WRITE(PA_BF16); break;
    case PA_F16: PA_FP8_WRITE(PA_F16); break;
    default: return hipErrorInvalidValue;
  }
#undef PA_FP8_WRITE
  return hipGetLastError();
}

// Whole-block copies: one workgroup per (pair, piece of a block, pool).  A
// piece is kCopyUnroll 16-byte chunks per thread (16 KB), all loaded before
// any is stored, so a large block is spread over many workgroups with several
// loads in flight per thread.  The loads are ordinary cached ones: copy-on-
// write copies one shared block to many sequences, and that source then stays
// in L2 (with non-temporal loads the shared-prefix workload's 99 pairs of 2 MB
// blocks took 96 us instead of 64 us; one workgroup per block walking it one
// chunk at a time took about 220 us).
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyPiece = (int64_t)kWriteThreads * kCopyUnroll;  // chunks per workgroup

__global__ __launch_bounds__(kWriteThreads) void copy_blocks_kernel(
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int32_t* __restrict__ pairs, int64_t block_chunks, int32_t pieces, int32_t num_blocks) {
  const int32_t i = blockIdx.x / pieces;
  const int64_t c0 = (int64_t)(blockIdx.x % pieces) * kCopyPiece;
  uint4* pool = blockIdx.y == 0 ? key_cache : value_cache;
  const int32_t bs = pairs[2 * i], bd = pairs[2 * i + 1];
  if (bs < 0 || bs >= num_blocks || bd < 0 || bd >= num_blocks) return;  // not a block of the pool
  const int64_t src = (int64_t)bs * block_chunks + c0;
  const int64_t dst = (int64_t)bd * block_chunks + c0;
  const int64_t n = min(kCopyPiece, block_chunks - c0);
  uint4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = threadIdx.x + (int64_t)u * kWriteThreads;
    if (c < n) v[u] = pool[src + c];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = threadIdx.x + (int64_t)u * kWriteThreads;
    if (c < n) store16(pool + dst + c, v[u]);
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, int64_t key_row_stride,
                                    int64_t value_row_stride, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    const PoolGeom& g, int elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int32_t hc = g.head_size * elem_bytes / 16;
  const int64_t ks = key_row_stride * elem_bytes / 16;
  const int64_t vs = value_row_stride * elem_bytes / 16;
  dim3 grid(num_tokens), block(kWriteThreads);
  if (g.layout == PA_LAYOUT_NHD)
    hipLaunchKernelGGL(reshape_and_cache_kernel<PA_LAYOUT_NHD>, grid, block, 0, stream,
                       (const uint4*)key, (const uint4*)value, ks, vs, (uint4*)key_cache,
                       (uint4*)value_cache, slot_mapping, g.num_kv_heads, hc, g.block_size);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<PA_LAYOUT_HND>, grid, block, 0, stream,
                       (const uint4*)key, (const uint4*)value, ks, vs, (uint4*)key_cache,
                       (uint4*)value_cache, slot_mapping, g.num_kv_heads, hc, g.block_size);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, pa_dtype src_dtype,
                                        int64_t key_row_stride, int64_t value_row_stride,
                                        void* key_cache, void* value_cache,
                                        const int64_t* slot_mapping, int32_t num_tokens,
                                        const PoolGeom& g, float k_scale, float v_scale,
                                        hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int eb = src_dtype == PA_F32 ? 4 : 2;
  const int64_t ks_b = key_row_stride * eb, vs_b = value_row_stride * eb;
  if (g.layout == PA_LAYOUT_NHD)
    return launch_fp8_write<PA_LAYOUT_NHD>(key, value, ks_b, vs_b, key_cache, value_cache,
                                           slot_mapping, num_tokens, g, src_dtype, k_scale,
                                           v_scale, stream);
  return launch_fp8_write<PA_LAYOUT_HND>(key, value, ks_b, vs_b, key_cache, value_cache,
                                         slot_mapping, num_tokens, g, src_dtype, k_scale, v_scale,
                                         stream);
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                              hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  const int64_t pieces = (chunks + kCopyPiece - 1) / kCopyPiece;
  if ((int64_t)num_pairs * pieces > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)(num_pairs * pieces), 2), block(kWriteThreads);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, block, 0, stream, (uint4*)key_cache,
                     (uint4*)value_cache, pairs, chunks, (int32_t)pieces, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
