// Paged decode attention for gfx950: single pass ("V1") or split-K partitions
// plus a reduce ("V2") -- dispatch, launch parameters and the reduce kernel.
//
// What is computed follows "PagedAttention 在 vLLM 中的实现分析" §3.1 (block
// table lookup: block block_table[t / block_size], offset t % block_size),
// §7.2-7.3 (per-block QK, softmax, V accumulation; partitions merged by
// max/sum rescaling) and the block-wise online softmax of the "Paged
// attention" post (k4i.top, attention over non-contiguous blocks).
//
// Two kernels share one contract; the dispatcher picks by GQA group size G
// and element type: the per-head kernel (decode_head.hip) for G <= 2 and
// every fp32 cache, the matrix-core grouped kernel (decode_group_mfma.hip)
// for 16-bit and FP8 caches otherwise.  Both
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
  // readfirstlane: the row is wave-uniform, so its index arithmetic and the
  // loads of its (max, sum) records are scalar
  const int64_t sh = (int64_t)blockIdx.x * (kReduceThreads / kWave) +
                     __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (sh >= num_pairs) return;
  const int lane = threadIdx.x % kWave;
  const int s = (int)(sh / p.num_heads);
  const int L = p.context_lens[s];
  if (L == 0 && !p.all_partial) {  // empty context: no partition holds a token, the row is zero
#pragma unroll
    for (int c = 0; c < CPL; ++c) store_out(p.out, sh * D + lane * CPL + c, 0.f, p.out_dtype);
    return;
  }
  if (single_partition(p, L)) return;
  const int np = p.part_base + (L > p.key_begin ? (L - p.key_begin + p.partition_size - 1) / p.partition_size : 0);
  // partial k of this row: record (s, k, h), num_heads records after k - 1
  const int64_t r0 = part_record(p, s, 0, (int)(sh - (int64_t)s * p.num_heads));
  const float* ml = p.part_ml + 2 * r0;
  const float* po = p.part_out + r0 * D + lane * CPL;
  const int64_t mls = 2 * (int64_t)p.num_heads, pos = (int64_t)p.num_heads * D;

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
      mv[k] = ml[kk * mls];
      lv[k] = ml[kk * mls + 1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ov[k][c] = po[kk * pos + c];
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
  for (int i = lane; i < np; i += kWave) M = fmaxf(M, ml[i * mls]);
  M = wave_max(M);
  int i = 0;
  for (; i + 8 <= np; i += 8) {
    float mv[8], lv[8], ov[8][CPL];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mv[k] = ml[(i + k) * mls];
      lv[k] = ml[(i + k) * mls + 1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ov[k][c] = po[(i + k) * pos + c];
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
    const float a = exp2_diff(ml[i * mls], M);
    lsum += a * ml[i * mls + 1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] += a * po[i * pos + c];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) store_out(p.out, sh * D + lane * CPL + c, o[c] * inv, p.out_dtype);
}

// Split-K reduce for many partitions per (sequence, head): one workgroup per
// (sequence, head).  Wave w merges partitions w, w + 4, w + 8, ... in one
// pass, kWideBatch partials at a time with the next batch's loads issued
// before the current one is merged: a running maximum of its own (moved when
// a batch exceeds it, the sums rescaled by 2^(m_old - m_new)), so no first
// pass over the maxima is needed.  The waves' (max, sum, output) states then
// meet in LDS by the same rule.  (Two passes -- the maximum first, then the
// weighted sums -- took 23 us on the long-context batch at 512-token
// partitions, 256 partials per row.)  Only the order of the fp32 sums differs
// from the one-wave kernel's, fixed by the launch.
constexpr int kWideBatch = 8;

template <int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_wide_kernel(const DecodeParams p) {
  constexpr int CPL = D / kWave;  // columns per lane
  constexpr int NW = kReduceThreads / kWave;
  constexpr int B = kWideBatch;
  __shared__ float sMax[NW], sSum[NW];
  __shared__ float sO[NW][D];
  const int64_t sh = blockIdx.x;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int s = (int)(sh / p.num_heads);
  const int L = p.context_lens[s];
  if (L == 0 && !p.all_partial) {  // empty context: the row is zero
    for (int d = threadIdx.x; d < D; d += kReduceThreads) store_out(p.out, sh * D + d, 0.f, p.out_dtype);
    return;
  }
  if (single_partition(p, L)) return;
  const int np = p.part_base + (L > p.key_begin ? (L - p.key_begin + p.partition_size - 1) / p.partition_size : 0);
  const int64_t r0 = part_record(p, s, 0, (int)(sh - (int64_t)s * p.num_heads));
  const float* ml = p.part_ml + 2 * r0;
  const float* po = p.part_out + r0 * D + lane * CPL;
  const int64_t mls = 2 * (int64_t)p.num_heads, pos = (int64_t)p.num_heads * D;

  // batch j of this wave: partitions wave + NW (B j + k), k < B (indices past
  // the end repeat the last partition and are not used)
  auto fetch = [&](int j, float (&mv)[B], float (&lv)[B], float (&ov)[B][CPL]) {
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int i = min(wave + NW * (B * j + k), np - 1);
      mv[k] = ml[i * mls];
      lv[k] = ml[i * mls + 1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) ov[k][c] = po[i * pos + c];
    }
  };
  float m = -INFINITY, lsum = 0.f, o[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = 0.f;
  auto merge = [&](int j, const float (&mv)[B], const float (&lv)[B], const float (&ov)[B][CPL]) {
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < B; ++k) mb = wave + NW * (B * j + k) < np ? fmaxf(mb, mv[k]) : mb;
    if (mb > m) {  // wave-uniform (every lane reads the same partials' maxima)
      const float a = exp2_diff(m, mb);
      lsum *= a;
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] *= a;
      m = mb;
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (wave + NW * (B * j + k) < np) {
        const float a = exp2_diff(mv[k], m);
        lsum += a * lv[k];
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] += a * ov[k][c];
      }
    }
  };
  const int nb = (np - wave + NW * B - 1) / (NW * B);  // this wave's batches (wave-uniform)
  float mv0[B], lv0[B], ov0[B][CPL], mv1[B], lv1[B], ov1[B][CPL];
  if (nb > 0) fetch(0, mv0, lv0, ov0);
  for (int j = 0; j < nb; j += 2) {  // every load unconditional: past the end they repeat
    fetch(j + 1, mv1, lv1, ov1);
    merge(j, mv0, lv0, ov0);
    fetch(j + 2, mv0, lv0, ov0);
    if (j + 1 < nb) merge(j + 1, mv1, lv1, ov1);
  }
  if (lane == 0) {
    sMax[wave] = m;
    sSum[wave] = lsum;
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) sO[wave][lane * CPL + c] = o[c];
  __syncthreads();
  float M = sMax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sMax[w]);
  for (int d = threadIdx.x; d < D; d += kReduceThreads) {
    float ot = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = exp2_diff(sMax[w], M);  // a wave without partitions: m = -inf, a = 0
      ot += a * sO[w][d];
      lt += a * sSum[w];
    }
    store_out(p.out, sh * D + d, lt > 0.f ? ot / lt : 0.f, p.out_dtype);
  }
}

// ------------------------------------------------------------ dispatch list
// Split-K dispatch list, one workgroup.  Hardware dispatch starts workgroups
// in id order, so the list orders the partitions largest first: every full
// partition (partition_size tokens), sequence by sequence, then each
// sequence's shorter last partition in kItemClasses classes of decreasing
// size (a class spans partition_size / kItemClasses tokens; the order
// within a class is whatever the LDS atomics give).  Long work then starts
// early and the shortest fills the end (longest-processing-time-first
// scheduling), and no empty workgroup is dispatched before the last item:
// the grid's unused tail is dispatched last and exits at once.  Only an
// order: every partial and the reduce are those of the (pairs, partitions)
// grid, so results do not depend on it.
__global__ __launch_bounds__(kDecodeThreads) void decode_items_kernel(const DecodeParams p) {
  __shared__ int32_t red[kDecodeWaves];
  __shared__ int32_t sCnt[kItemClasses];  // shorter partitions per size class, then the class cursors
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int S = p.num_seqs, hkv = p.num_kv_heads, P = p.partition_size;
  int4* items = reinterpret_cast<int4*>(p.items);
  auto bucket = [&](int r) { return (int)((int64_t)(P - r) * kItemClasses / P); };  // r in [1, P): 0 = longest
  // exclusive prefix of x over the workgroup; total = the sum
  auto scan = [&](int x, int& total) -> int {
    int incl = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) red[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (w < wave) before += red[w];
      total += red[w];
    }
    __syncthreads();  // red is rewritten by the next scan
    return before + incl - x;
  };
  if (tid < kItemClasses) sCnt[tid] = 0;
  __syncthreads();
  // full partitions in sequence order; shorter ones counted per class.  A
  // batch of at most kDecodeThreads sequences is read once (L0 is kept for
  // the second pass).
  int full_base = 0, rem_total = 0;
  const int L0 = tid < S ? p.context_lens[tid] : 0;
  for (int i0 = 0; i0 < S; i0 += kDecodeThreads) {
    const int i = i0 + tid;
    const int L = i0 == 0 ? L0 : i < S ? p.context_lens[i] : 0;
    const int f = L / P, r = L - f * P;
    int nf;
    const int fx = scan(f, nf);
    for (int y = 0; y < f; ++y)
      for (int k = 0; k < hkv; ++k) items[(int64_t)(full_base + fx + y) * hkv + k] = make_int4(i, k, y, 0);
    if (r > 0) atomicAdd(&sCnt[bucket(r)], 1);
    full_base += nf;
  }
  __syncthreads();
  if (wave == 0) {  // class cursors: after the full partitions, longest class first
    const int c = lane < kItemClasses ? sCnt[lane] : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane < kItemClasses) sCnt[lane] = full_base + incl - c;
    rem_total = __shfl(incl, kWave - 1);
  }
  __syncthreads();
  for (int i0 = 0; i0 < S; i0 += kDecodeThreads) {  // shorter partitions at their class cursors
    const int i = i0 + tid;
    const int L = i0 == 0 ? L0 : i < S ? p.context_lens[i] : 0;
    const int f = L / P, r = L - f * P;
    if (r > 0) {
      const int pos = atomicAdd(&sCnt[bucket(r)], 1);
      for (int k = 0; k < hkv; ++k) items[(int64_t)pos * hkv + k] = make_int4(i, k, f, 0);
    }
  }
  if (tid == 0) *p.item_count = (full_base + rem_total) * hkv;
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
  p.item_count = a.item_count;
  p.items = a.items;
  p.num_seqs = a.num_seqs;
  return p;
}

}  // namespace
}  // namespace dec

bool decode_uses_group_kernel(pa_dtype kv_dtype, int G) {
  return kv_dtype != PA_F32 && (G == 4 || G == 8 || G == 16);
}

hipError_t launch_decode_main(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  dec::DecodeParams p = dec::make_params(a);
  const PoolGeom& g = a.geom;
  const int G = a.num_heads / g.num_kv_heads;
  dim3 grid((unsigned)(a.num_seqs * g.num_kv_heads),
            a.partition_size > 0 ? a.max_partitions - a.part_base : 1);
  if (grid.y == 0) return hipSuccess;
  const bool group = decode_uses_group_kernel(a.kv_dtype, G);
  // The grouped kernels' split-K over whole contexts (not a cascade's
  // suffixes) of many (sequence, kv head) pairs takes the largest-first
  // dispatch list: on the lognormal 70B-like batch (1,024 pairs) 169 -> 158
  // us (bf16) and 108 -> 101 us (FP8), the list's one-workgroup launch
  // included.  Few pairs (the long-context batch: 64, every partition full)
  // and the per-head kernel (uniform 7B-like batch) gain no order and would
  // only pay the launch, so they keep the grid.
  const int64_t items = (int64_t)grid.x * grid.y;
  const bool listed = a.items && a.partition_size > 0 && a.key_begin == 0 && a.part_base == 0 &&
                      !a.all_partial && group && grid.x >= 2u * (unsigned)device_cus() &&
                      items <= 0x7FFFFFFF;
  if (listed && a.num_seqs <= dec::kDecodeThreads &&
      (a.partition_size & (a.partition_size - 1)) == 0) {
    // Up to kDecodeThreads sequences and a power-of-two partition size: each
    // workgroup derives its item itself, and the list kernel's launch leaves
    // the step (70B-like batch, same box, alternating builds: step 156.1-156.3
    // -> 153.3-154.0 us; FP8 100.0-100.1 -> 98.6-99.5 us).  Larger batches
    // would read more lengths per workgroup than the list costs.
    p.items = nullptr;
    p.item_count = nullptr;
    p.inline_items = true;
    p.log2_part = __builtin_ctz((unsigned)a.partition_size);
    grid = dim3((unsigned)items);
  } else if (listed) {
    hipLaunchKernelGGL(dec::decode_items_kernel, dim3(1), dim3(dec::kDecodeThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    grid = dim3((unsigned)items);
  } else {
    p.items = nullptr;
    p.item_count = nullptr;
  }
  if (a.kv_dtype == PA_FP8_E4M3)
    return group ? dec::launch_group_fp8(p, a.q_dtype, g.head_size, G, grid, stream)
                 : dec::launch_head_fp8(p, a.q_dtype, g.head_size, G, grid, stream);
  if (group) return dec::launch_group_mfma(p, a.kv_dtype, g.head_size, G, grid, stream);
  return dec::launch_head(p, a.kv_dtype, g.head_size, G, grid, stream);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.partition_size <= 0) return hipSuccess;
  const dec::DecodeParams p = dec::make_params(a);
  const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
  // Many partials per row: a workgroup per (sequence, head).  Up to 64 the
  // one-wave-per-row kernel is faster (shared-prefix cascade, 16 partials:
  // 161 -> 153 us step; long context at 32 partials); at 256 the row's
  // batches in one wave would run one after another.
  if (a.max_partitions > 64) {
    if (pairs > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.geom.head_size == 64)
      hipLaunchKernelGGL(dec::decode_reduce_wide_kernel<64>, dim3((unsigned)pairs),
                         dim3(dec::kReduceThreads), 0, stream, p);
    else if (a.geom.head_size == 128)
      hipLaunchKernelGGL(dec::decode_reduce_wide_kernel<128>, dim3((unsigned)pairs),
                         dim3(dec::kReduceThreads), 0, stream, p);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
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
