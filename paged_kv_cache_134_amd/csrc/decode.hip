// Paged decode attention for gfx950: single pass ("V1") or split-K partitions
// plus a reduce ("V2") -- dispatch, launch parameters and the reduce kernel.
//
// What is computed follows "PagedAttention 在 vLLM 中的实现分析" §3.1 (block
// table lookup: block block_table[t / block_size], offset t % block_size),
// §7.2-7.3 (per-block QK, softmax, V accumulation; partitions merged by
// max/sum rescaling) and the block-wise online softmax of the "Paged
// attention" post (k4i.top, attention over non-contiguous blocks).
//
// Three kernels share one contract; the dispatcher picks by GQA group size G
// and element type: the per-head kernel (decode_head.hip) for G <= 2 and
// every fp32 cache, the LDS-staged grouped kernel (decode_group.hip) for
// 16-bit caches otherwise, and the matrix-core grouped kernel
// (decode_group_fp8.hip) for FP8 caches otherwise.  All
// use one workgroup of 4 waves per (sequence, kv head, partition), read each
// kv head's K/V rows once for all G query heads of its group, never load a
// token at or past the context length (so NaN in unused slots cannot reach
// the arithmetic), and order every floating-point operation by logical
// position only, so results are bitwise independent of which physical
// blocks hold the context.  Running maxima are moved lazily: only when a
// batch exceeds the reference by more than 2^8, since the final quotient
// does not depend on where the reference sits.
#include <hip/hip_runtime.h>

#include "decode_common.h"

namespace pa {
namespace dec {
namespace {

// --------------------------------------------------------------------- reduce
// Split-K reduce ("V2" reduce): for one (sequence, head), M = max_p m_p and
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over the partitions
// that hold tokens.  One wave per (sequence, head), D/64 columns per lane,
// 8 partitions' loads in flight together; with at most 8 partitions the
// maximum, sums and outputs come in one round trip.  Heads whose context is a single
// partition were written directly by the partition kernel.
constexpr int kReduceThreads = 256;

template <int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(const DecodeParams p,
                                                                       int64_t num_pairs) {
  constexpr int CPL = D / kWave;  // columns per lane
  const int64_t sh = (int64_t)blockIdx.x * (kReduceThreads / kWave) + threadIdx.x / kWave;
  if (sh >= num_pairs) return;
  const int lane = threadIdx.x % kWave;
  const int s = (int)(sh / p.num_heads);
  const int L = p.context_lens[s];
  if (single_partition(p, L)) return;
  const int np = p.part_base + (L > p.key_begin ? (L - p.key_begin + p.partition_size - 1) / p.partition_size : 0);
  const float* ml = p.part_ml + sh * p.max_partitions * 2;
  const float* po = p.part_out + sh * p.max_partitions * D + lane * CPL;

  float o[CPL], lsum = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = 0.f;
  if (np > 0 && np <= 8) {
    // one round trip: every partial's (max, sum, output) is requested
    // together, the maximum taken from what arrived
    float mv[8], lv[8], ov[8][CPL];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int kk = min(k, np - 1);  // (repeats of the last partial are not used)
      mv[k] = ml[2 * kk];
      lv[k] = ml[2 * kk + 1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ov[k][c] = po[(int64_t)kk * D + c];
    }
    float M = mv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) M = k < np ? fmaxf(M, mv[k]) : M;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < np) {
        const float a = exp2_diff(mv[k], M);
        lsum += a * lv[k];
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] += a * ov[k][c];
      }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) store_out(p.out, sh * D + lane * CPL + c, o[c] * inv, p.out_dtype);
    return;
  }

  float M = -INFINITY;
  for (int i = lane; i < np; i += kWave) M = fmaxf(M, ml[2 * i]);
  M = wave_max(M);
  int i = 0;
  for (; i + 8 <= np; i += 8) {
    float mv[8], lv[8], ov[8][CPL];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mv[k] = ml[2 * (i + k)];
      lv[k] = ml[2 * (i + k) + 1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ov[k][c] = po[(int64_t)(i + k) * D + c];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float a = exp2_diff(mv[k], M);
      lsum += a * lv[k];
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] += a * ov[k][c];
    }
  }
  for (; i < np; ++i) {
    const float a = exp2_diff(ml[2 * i], M);
    lsum += a * ml[2 * i + 1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] += a * po[(int64_t)i * D + c];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) store_out(p.out, sh * D + lane * CPL + c, o[c] * inv, p.out_dtype);
}

DecodeParams make_params(const DecodeArgs& a) {
  const PoolGeom& g = a.geom;
  DecodeParams p{};
  p.out = a.out;
  p.query = a.query;
  p.key_cache = static_cast<const char*>(a.key_cache);
  p.value_cache = static_cast<const char*>(a.value_cache);
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.part_out = a.part_out;
  p.part_ml = a.part_ml;
  const int64_t D = g.head_size, bs = g.block_size, hk = g.num_kv_heads;
  p.blk_stride = bs * hk * D;
  if (g.layout == PA_LAYOUT_NHD) {
    p.tok_stride = hk * D;
    p.head_stride = D;
  } else {
    p.tok_stride = D;
    p.head_stride = bs * D;
  }
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_heads = a.num_heads;
  p.num_kv_heads = g.num_kv_heads;
  p.log2_bs = g.block_size > 0 ? __builtin_ctz((unsigned)g.block_size) : 0;
  p.partition_size = a.partition_size;
  p.max_partitions = a.max_partitions;
  p.key_begin = a.key_begin;
  p.part_base = a.part_base;
  p.all_partial = a.all_partial;
  p.scale_log2e = a.scale * a.k_scale * kLog2e;
  p.v_scale = a.v_scale;
  p.out_dtype = a.out_dtype;
  const int64_t elem = a.kv_dtype == PA_F32 ? 4 : a.kv_dtype == PA_FP8_E4M3 ? 1 : 2;
  p.off32 = (int64_t)g.num_blocks * p.blk_stride * elem <= (int64_t)UINT32_MAX;
  return p;
}

}  // namespace
}  // namespace dec

bool decode_uses_group_kernel(pa_dtype kv_dtype, int G) {
  return kv_dtype != PA_F32 && (G == 4 || G == 8 || G == 16);
}

hipError_t launch_decode_main(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const dec::DecodeParams p = dec::make_params(a);
  const PoolGeom& g = a.geom;
  const int G = a.num_heads / g.num_kv_heads;
  dim3 grid((unsigned)(a.num_seqs * g.num_kv_heads),
            a.partition_size > 0 ? a.max_partitions - a.part_base : 1);
  if (grid.y == 0) return hipSuccess;
  const bool group = decode_uses_group_kernel(a.kv_dtype, G);
  if (a.kv_dtype == PA_FP8_E4M3)
    return group ? dec::launch_group_fp8(p, a.q_dtype, g.head_size, G, grid, stream)
                 : dec::launch_head_fp8(p, a.q_dtype, g.head_size, G, grid, stream);
  if (group) return dec::launch_group(p, a.kv_dtype, g.head_size, G, grid, stream);
  return dec::launch_head(p, a.kv_dtype, g.head_size, G, grid, stream);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.partition_size <= 0) return hipSuccess;
  const dec::DecodeParams p = dec::make_params(a);
  const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
  constexpr int per_block = dec::kReduceThreads / kWave;
  dim3 rgrid((unsigned)((pairs + per_block - 1) / per_block));
  if (a.geom.head_size == 64)
    hipLaunchKernelGGL(dec::decode_reduce_kernel<64>, rgrid, dim3(dec::kReduceThreads), 0, stream, p, pairs);
  else if (a.geom.head_size == 128)
    hipLaunchKernelGGL(dec::decode_reduce_kernel<128>, rgrid, dim3(dec::kReduceThreads), 0, stream, p, pairs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
