// Paged decode attention for gfx950: single pass ("V1") or split-K partitions
// plus a reduce ("V2").
//
// What is computed follows "PagedAttention 在 vLLM 中的实现分析" §3.1 (block
// table lookup: block block_table[t / block_size], offset t % block_size),
// §7.2-7.3 (per-block QK, softmax, V accumulation; partitions merged by
// max/sum rescaling) and the block-wise online softmax of the "Paged
// attention" post (k4i.top, attention over non-contiguous blocks).
//
// Work decomposition (this file's own design for wave64 / CDNA4):
//   * one workgroup (4 waves) per (sequence, kv head, partition); a kv head's
//     K/V rows are read once for all G = H / Hkv query heads of its group;
//   * a token row of one kv head (head_size elements) is spread over LPT lanes
//     that each own one 16-byte chunk, so every load is a 16-byte vector load
//     and a wave reads TPW = 64 / LPT whole rows per instruction (coalesced:
//     the LPT lanes of a row cover its contiguous bytes);
//   * each lane group keeps its own running (max, sum, acc) per query head;
//     QK partial dots are summed across the LPT lanes with DPP; the running
//     max is only moved when a batch's max exceeds it by more than 2^8
//     (the final result does not depend on where the reference point sits);
//   * at the end lane groups and waves are merged with the same log-sum-exp
//     rule, then the workgroup writes either the normalised output or its
//     partition's (max, sum, unnormalised output) for the reduce kernel.
// Tokens past the context length are never loaded, so NaN in unused slots or
// blocks cannot reach the arithmetic.  The order of every floating-point
// operation depends only on logical positions, so results are bitwise
// independent of which physical blocks hold the context.
#include <hip/hip_runtime.h>

#include "kernel_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * kWave;
constexpr int kUnroll = 4;          // token rows per lane group per batch
constexpr float kLazyRescale = 8.f; // log2 headroom before the running max moves

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
  int32_t max_partitions;
  float scale_log2e;
  pa_dtype out_dtype;
};

template <pa_dtype DT, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const DecodeParams p) {
  using F = Fmt<DT>;
  constexpr int VEC = F::kVec;         // elements per lane chunk
  constexpr int LPT = D / VEC;         // lanes per token row
  constexpr int TPW = kWave / LPT;     // token rows per wave per step
  constexpr int TPS = TPW * kDecodeWaves;  // token rows per workgroup per step
  static_assert(LPT >= 1 && LPT <= kWave && (kWave % LPT) == 0, "bad head size");

  const int kvh = blockIdx.x % p.num_kv_heads;
  const int s = blockIdx.x / p.num_kv_heads;
  const int part = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int tg = lane / LPT;   // lane group (token row) within the wave
  const int ch = lane % LPT;   // 16-byte chunk of the row owned by this lane

  const int L = p.context_lens[s];
  int t0 = 0, t1 = L;
  if (p.partition_size > 0) {
    t0 = part * p.partition_size;
    if (t0 >= L) return;  // partition past the end: the reduce ignores it
    t1 = min(L, t0 + p.partition_size);
  }

  // query chunks of the G heads of this kv group
  uint4 q[G];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.query) +
                      ((int64_t)s * p.num_heads + (int64_t)kvh * G) * (D / VEC) + ch;
#pragma unroll
    for (int g = 0; g < G; ++g) q[g] = qp[g * (D / VEC)];
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
  }

  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
  const int bs_mask = (1 << p.log2_bs) - 1;
  const int64_t lane_off = (int64_t)kvh * p.head_stride + ch * VEC;

  // wave-uniform trip count: lane groups past the end run with invalid rows
  for (int wbase = t0 + wave * TPW; wbase < t1; wbase += kUnroll * TPS) {
    uint4 kr[kUnroll], vr[kUnroll];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = wbase + u * TPS + tg;
      valid[u] = t < t1;
      if (valid[u]) {
        const int64_t blk = bt[t >> p.log2_bs];
        const int64_t off = blk * p.blk_stride + (int64_t)(t & bs_mask) * p.tok_stride + lane_off;
        kr[u] = *reinterpret_cast<const uint4*>(p.key_cache + off * F::kBytes);
        vr[u] = *reinterpret_cast<const uint4*>(p.value_cache + off * F::kBytes);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    // scores (log2 domain)
    float z[kUnroll][G];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float d = group_sum<LPT>(dot_chunk<DT>(q[g], kr[u], 0.f));
        z[u][g] = valid[u] ? d * p.scale_log2e : -INFINITY;
      }
    }
    // move the running max only when the batch exceeds it by the headroom
    bool need = false;
    float mb[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mb[g] = z[0][g];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mb[g] = fmaxf(mb[g], z[u][g]);
      need |= mb[g] > m[g] + kLazyRescale;
    }
    if (__any(need)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], mb[g]);
        const float a = exp2_diff(m[g], mn);
        m[g] = mn;
        l[g] *= a;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] *= a;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float vf[VEC];
      chunk_to_f32<DT>(vr[u], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pw = valid[u] ? __builtin_amdgcn_exp2f(z[u][g] - m[g]) : 0.f;
        l[g] += pw;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = __builtin_fmaf(pw, vf[e], acc[g][e]);
      }
    }
  }

  // merge the lane groups of the wave (log-sum-exp rule)
#pragma unroll
  for (int x = LPT; x < kWave; x <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], x);
      const float lo = __shfl_xor(l[g], x);
      const float mn = fmaxf(m[g], mo);
      const float a = exp2_diff(m[g], mn);
      const float b = exp2_diff(mo, mn);
      l[g] = a * l[g] + b * lo;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = __shfl_xor(acc[g][e], x);
        acc[g][e] = a * acc[g][e] + b * ao;
      }
      m[g] = mn;
    }
  }

  // merge the waves through LDS
  __shared__ float sm_m[kDecodeWaves][G];
  __shared__ float sm_l[kDecodeWaves][G];
  __shared__ float sm_acc[kDecodeWaves][G][D];
  if (tg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[wave][g][ch * VEC + e] = acc[g][e];
      if (ch == 0) {
        sm_m[wave][g] = m[g];
        sm_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  const int64_t head0 = (int64_t)s * p.num_heads + (int64_t)kvh * G;
  for (int i = threadIdx.x; i < G * D; i += kDecodeThreads) {
    const int g = i / D;
    const int d = i % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float a = exp2_diff(sm_m[w][g], M);
      lsum += a * sm_l[w][g];
      o += a * sm_acc[w][g][d];
    }
    if (p.partition_size > 0) {
      const int64_t pi = (head0 + g) * p.max_partitions + part;
      p.part_out[pi * D + d] = o;
      if (d == 0) {
        p.part_ml[2 * pi] = M;
        p.part_ml[2 * pi + 1] = lsum;
      }
    } else {
      store_out(p.out, (head0 + g) * D + d, lsum > 0.f ? o / lsum : 0.f, p.out_dtype);
    }
  }
}

// Reduce of split-K partials ("V2" reduce): for one (sequence, head),
// M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over the
// partitions that hold tokens.  One thread per output element.
template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const DecodeParams p) {
  const int64_t sh = blockIdx.x;  // s * num_heads + h
  const int s = (int)(sh / p.num_heads);
  const int d = threadIdx.x;
  const int L = p.context_lens[s];
  const int np = (L + p.partition_size - 1) / p.partition_size;
  const float* ml = p.part_ml + sh * p.max_partitions * 2;
  const float* po = p.part_out + sh * p.max_partitions * D + d;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, ml[2 * i]);
  float lsum = 0.f, o = 0.f;
  for (int i = 0; i < np; ++i) {
    const float a = exp2_diff(ml[2 * i], M);
    lsum += a * ml[2 * i + 1];
    o += a * po[(int64_t)i * D];
  }
  store_out(p.out, sh * D + d, lsum > 0.f ? o / lsum : 0.f, p.out_dtype);
}

template <pa_dtype DT, int D>
hipError_t launch_g(const DecodeParams& p, int G, dim3 grid, hipStream_t st) {
  dim3 block(kDecodeThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<DT, D, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<DT, D, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<DT, D, 4>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<DT, D, 8>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((decode_kernel<DT, D, 16>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <pa_dtype DT>
hipError_t launch_d(const DecodeParams& p, int D, int G, dim3 grid, hipStream_t st) {
  if (D == 64) return launch_g<DT, 64>(p, G, grid, st);
  if (D == 128) return launch_g<DT, 128>(p, G, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

namespace {

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
  p.scale_log2e = a.scale * kLog2e;
  p.out_dtype = a.out_dtype;
  return p;
}

}  // namespace

hipError_t launch_decode_main(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const DecodeParams p = make_params(a);
  const PoolGeom& g = a.geom;
  const int G = a.num_heads / g.num_kv_heads;
  dim3 grid((unsigned)(a.num_seqs * g.num_kv_heads), a.partition_size > 0 ? a.max_partitions : 1);
  switch (a.kv_dtype) {
    case PA_F32: return launch_d<PA_F32>(p, g.head_size, G, grid, stream);
    case PA_BF16: return launch_d<PA_BF16>(p, g.head_size, G, grid, stream);
    case PA_F16: return launch_d<PA_F16>(p, g.head_size, G, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.partition_size <= 0) return hipSuccess;
  const DecodeParams p = make_params(a);
  dim3 rgrid((unsigned)(a.num_seqs * a.num_heads));
  if (a.geom.head_size == 64)
    hipLaunchKernelGGL(decode_reduce_kernel<64>, rgrid, dim3(64), 0, stream, p);
  else if (a.geom.head_size == 128)
    hipLaunchKernelGGL(decode_reduce_kernel<128>, rgrid, dim3(128), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
