// Shared definitions of the paged decode kernels (per-head and grouped
// kernels, split-K reduce): launch parameters, wave reductions and the
// partial/final output rule.  What is computed follows "PagedAttention 在
// vLLM 中的实现分析" §3.1 (block block_table[t / block_size], offset
// t % block_size) and §7.2-7.3 (per-block QK, softmax, V accumulation;
// partitions merged by max/sum rescaling).
#ifndef PA_DECODE_COMMON_H_
#define PA_DECODE_COMMON_H_

#include <hip/hip_runtime.h>

#include "kernel_common.h"
#include "pa_internal.h"

namespace pa {
namespace dec {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * kWave;
constexpr float kLazyRescale = 8.f;  // log2 headroom before a running max moves

typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;

struct DecodeParams {
  void* out;
  const void* query;
  const char* key_cache;
  const char* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_out;
  float* part_ml;
  int64_t blk_stride;   // elements between blocks
  int64_t tok_stride;   // elements between tokens of a block
  int64_t head_stride;  // elements between kv heads
  int32_t max_blocks_per_seq;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t log2_bs;
  int32_t partition_size;  // 0 = single pass
  int32_t max_partitions;  // workspace partitions per (sequence, head)
  int32_t key_begin;       // partitions cover keys [key_begin, L) (0 outside cascades)
  int32_t part_base;       // workspace index of partition 0 (earlier slots hold prefix partials)
  bool all_partial;        // never finish a head here: other partials exist
  float scale_log2e;        // softmax scale * log2(e), times k_scale for FP8 caches
  float v_scale;            // FP8 caches: V scale, applied to the merged output (else 1)
  pa_dtype out_dtype;
  bool off32;  // every byte offset into either cache fits in 32 bits
  // Split-K dispatch list (null: the grid is (pairs, partitions)): workgroup
  // b takes item b -- (sequence, kv head, partition) -- while b < *item_count.
  int32_t* item_count;
  int32_t* items;
  int32_t num_seqs;
  // No list but the same order, derived by each workgroup from the context
  // lengths (decode_item_inline): at most kDecodeThreads sequences and a
  // power-of-two partition_size, 1 << log2_part.
  bool inline_items;
  int32_t log2_part;
};

// The (sequence, kv head, partition) of this workgroup: from the dispatch
// list when there is one, else from the (pairs, partitions) grid, partitions
// taken last-first when last_first (only long contexts have high
// partitions, so their workgroups start early).  False: nothing to do.
__device__ __forceinline__ bool decode_item(const DecodeParams& p, bool last_first, int& s, int& kvh,
                                            int& part) {
  if (p.items) {
    if ((int)blockIdx.x >= *p.item_count) return false;
    const int4 it = reinterpret_cast<const int4*>(p.items)[blockIdx.x];
    s = __builtin_amdgcn_readfirstlane(it.x);
    kvh = __builtin_amdgcn_readfirstlane(it.y);
    part = __builtin_amdgcn_readfirstlane(it.z);
    return true;
  }
  kvh = blockIdx.x % p.num_kv_heads;
  s = blockIdx.x / p.num_kv_heads;
  part = last_first ? gridDim.y - 1 - blockIdx.y : blockIdx.y;
  return true;
}

// Sum over the 64 lanes of a wave, integers (every lane receives it).
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) x += __shfl_xor(x, d);
  return x;
}

// Size classes of the shorter last partitions in the split-K dispatch order
// (the list builder's and decode_item_inline's).
constexpr int kItemClasses = 64;
static_assert(kItemClasses == kWave, "one class per lane");

// Size class of a last partition shorter than 1 << lp by `short_by` tokens
// (1 .. 2^lp - 1): 0 = longest.
__device__ __forceinline__ int item_class(int short_by, int lp) {
  return (int)(((int64_t)short_by * kItemClasses) >> lp);
}

// The dispatch list's order without the list: workgroup b takes item b =
// j * num_kv_heads + kv head, where j numbers every full partition, sequence
// by sequence, then each sequence's shorter last partition by size class
// (partition_size / kItemClasses tokens each), longest class first and by
// sequence within a class.  Every workgroup derives it from the context
// lengths of the (at most kDecodeThreads) sequences: an exclusive scan of
// the full-partition counts for the first part, and for the second one
// lane mask per (wave, class) -- a sequence's place is its class's start
// plus the same-class sequences before it.  False past the last item (the
// grid is an upper bound); L receives the sequence's context length.  Only
// an order: the partials are those of the (pairs, partitions) grid.
__device__ __forceinline__ bool decode_item_inline(const DecodeParams& p, int& s, int& kvh, int& part,
                                                   int& L) {
  static_assert(kDecodeWaves == 4, "one length per thread: kDecodeWaves x kWave sequences");
  __shared__ int32_t sRed[kDecodeWaves];
  __shared__ unsigned long long sMask[kDecodeWaves][kItemClasses];
  __shared__ int32_t sCur[kItemClasses];
  __shared__ int32_t sPick[3];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = p.num_seqs, lp = p.log2_part, P = 1 << lp;
  const int j = blockIdx.x / p.num_kv_heads;
  // Each wave reads every length (sequence lane + 64 k in Ls[k]) and counts
  // the items itself, so a workgroup past the last item leaves before any
  // barrier.
  int Ls[kDecodeWaves];
  int n = 0;
#pragma unroll
  for (int k = 0; k < kDecodeWaves; ++k) {
    const int t = lane + kWave * k;
    Ls[k] = t < S ? p.context_lens[t] : 0;
    n += (Ls[k] >> lp) + ((Ls[k] & (P - 1)) != 0);
  }
  if (j >= wave_sum_int(n)) return false;
  // this thread's sequence is tid
  const int Lt = wave == 0 ? Ls[0] : wave == 1 ? Ls[1] : wave == 2 ? Ls[2] : Ls[3];
  const int f = Lt >> lp, r = Lt & (P - 1);
  const int c = r > 0 ? item_class(P - r, lp) : -1;
  for (int i = tid; i < kDecodeWaves * kItemClasses; i += kDecodeThreads) (&sMask[0][0])[i] = 0ull;
  int incl = f;  // inclusive scan of f within the wave
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) sRed[wave] = incl;
  __syncthreads();
  if (c >= 0) atomicOr(&sMask[wave][c], 1ull << lane);
  int before = 0, F = 0;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) {
    if (w < wave) before += sRed[w];
    F += sRed[w];
  }
  __syncthreads();
  if (j < F) {  // a full partition
    const int fx = before + incl - f;
    if (fx <= j && j < fx + f) {
      sPick[0] = tid;
      sPick[1] = j - fx;
      sPick[2] = Lt;
    }
  } else {  // a shorter last partition (j is the same for the whole workgroup)
    if (wave == 0) {  // lane = class: its start after the full partitions
      int cnt = 0;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) cnt += __popcll(sMask[w][lane]);
      int ci = cnt;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(ci, d);
        if (lane >= d) ci += y;
      }
      sCur[lane] = F + ci - cnt;
    }
    __syncthreads();
    if (c >= 0) {
      int pos = sCur[c] + __popcll(sMask[wave][c] & ((1ull << lane) - 1ull));
      for (int w = 0; w < wave; ++w) pos += __popcll(sMask[w][c]);
      if (pos == j) {
        sPick[0] = tid;
        sPick[1] = f;
        sPick[2] = Lt;
      }
    }
  }
  __syncthreads();
  s = __builtin_amdgcn_readfirstlane(sPick[0]);
  part = __builtin_amdgcn_readfirstlane(sPick[1]);
  L = __builtin_amdgcn_readfirstlane(sPick[2]);
  kvh = blockIdx.x % p.num_kv_heads;
  return true;
}

// Maximum over the 64 lanes of a wave (every lane receives it).
__device__ __forceinline__ float wave_max(float x) {
  x = group_max<16>(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Whether a sequence of context L is finished by its single partition (the
// reduce then skips it).
__device__ __forceinline__ bool single_partition(const DecodeParams& p, int L) {
  return !p.all_partial && L <= p.partition_size;
}

// Split-K partials are partition-major: record (s, k, h) -- sequence s,
// workspace partition k, head h of the sequence -- is row
// (s * max_partitions + k) * num_heads + h of part_out (D floats) and of
// part_ml ((max, sum)).  The workgroups of one (sequence, partition) -- the
// kv heads, dispatched side by side -- thus write one contiguous stretch.
// (Head-major rows, 512-token partitions apart, wrote the same bytes at
// large power-of-two strides; on the long-context batch the partition
// kernel took 807 us with them, 771 us partition-major, 756 us with the
// stores also non-temporal.)
__device__ __forceinline__ int64_t part_record(const DecodeParams& p, int s, int k, int h) {
  return ((int64_t)s * p.max_partitions + k) * p.num_heads + h;
}

// Writes one (max, sum, unnormalised output) partial of sequence s, head h
// of the sequence, or the final output when the whole context is one
// partition (the reduce skips those heads).  The partials are stored
// non-temporally: the reduce reads them once, after this kernel.
__device__ __forceinline__ void emit(const DecodeParams& p, int s, int h, int part, int d, int D,
                                     float M, float lsum, float o, bool single) {
  o *= p.v_scale;
  if (p.partition_size > 0 && !single) {
    const int64_t r = part_record(p, s, p.part_base + part, h);
    __builtin_nontemporal_store(o, p.part_out + r * D + d);
    if (d == 0) {
      p.part_ml[2 * r] = M;
      p.part_ml[2 * r + 1] = lsum;
    }
  } else {
    store_out(p.out, ((int64_t)s * p.num_heads + h) * D + d, lsum > 0.f ? o / lsum : 0.f,
              p.out_dtype);
  }
}

// Single pass over an empty context: the group's output rows are zero.
// Nothing is loaded, so no entry of the (possibly unwritten) block-table row
// is read.
__device__ __forceinline__ void emit_zero_rows(const DecodeParams& p, int64_t head0, int G, int D) {
  for (int i = threadIdx.x; i < G * D; i += kDecodeThreads)
    store_out(p.out, head0 * D + i, 0.f, p.out_dtype);
}

// Kernel launches of one decode pass; grid = (num_seqs * num_kv_heads,
// partitions or 1).
hipError_t launch_head(const DecodeParams& p, pa_dtype dt, int D, int G, dim3 grid, hipStream_t st);
// FP8 (E4M3) caches; qt = query type (bf16 or f16).  Group sizes 1 and 2 take
// the per-head kernel, 4, 8 and 16 the matrix-core grouped kernel.
hipError_t launch_head_fp8(const DecodeParams& p, pa_dtype qt, int D, int G, dim3 grid, hipStream_t st);
hipError_t launch_group_fp8(const DecodeParams& p, pa_dtype qt, int D, int G, dim3 grid, hipStream_t st);
// 16-bit caches on the matrix-core grouped kernel (dt = the cache's and the
// query's type).
hipError_t launch_group_mfma(const DecodeParams& p, pa_dtype dt, int D, int G, dim3 grid, hipStream_t st);

}  // namespace dec
}  // namespace pa

#endif  // PA_DECODE_COMMON_H_
