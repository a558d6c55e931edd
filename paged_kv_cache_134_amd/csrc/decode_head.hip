// Paged decode, per-head kernel (group size 1 or 2, and every fp32 cache;
// FP8 caches with group size 1 or 2).
//
// One workgroup of 4 waves per (sequence, kv head, partition) reads the kv
// head's K/V rows once for its G query heads.  A token row is spread over
// LPT lanes that each own one 16-byte chunk, so a wave reads TPW = 64 / LPT
// whole rows per 16-byte load; QK partial dots are summed across the LPT
// lanes with DPP.  The partition's block-table entries are staged in LDS,
// and the next batch of rows is loaded while the current one is consumed.
// Rows at or past the context length are never loaded, floating-point work
// is ordered by logical position only (results do not depend on which
// physical blocks hold the context), and the running maximum moves only
// when a batch exceeds it by more than 2^8 (the block-wise online softmax of
// the "Paged attention" post, k4i.top, attention over non-contiguous
// blocks).
#include <hip/hip_runtime.h>

#include "decode_common.h"

namespace pa {
namespace dec {
namespace {

constexpr int kUnroll = 4;    // token rows per lane group per batch
constexpr int kWindow = 512;  // tokens per block-table staging window

// FP8: the cache holds E4M3 codes (one byte) and DT is the query's type; a
// lane's 16-byte chunk is then 16 elements, K converts exactly to DT pairs
// for the same dot products and V to fp32.
template <pa_dtype DT, int D, int G, bool FP8 = false>
__global__ __launch_bounds__(kDecodeThreads) void decode_reg_kernel(const DecodeParams p) {
  using F = Fmt<DT>;
  constexpr int CB = FP8 ? 1 : F::kBytes;  // cache bytes per element
  constexpr int VEC = 16 / CB;             // elements per lane chunk
  constexpr int QC = FP8 ? 2 : 1;          // 16-byte query chunks per lane chunk
  constexpr int LPT = D / VEC;             // lanes per token row
  constexpr int TPW = kWave / LPT;         // token rows per wave per step
  constexpr int TPS = TPW * kDecodeWaves;  // token rows per workgroup per step
  static_assert(LPT >= 1 && LPT <= kWave && (kWave % LPT) == 0, "bad head size");
  __shared__ int32_t s_bt[kWindow + 1];

  int s, kvh, part;
  if (!decode_item(p, false, s, kvh, part)) return;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int tg = lane / LPT;  // lane group (token row) within the wave
  const int ch = lane % LPT;  // 16-byte chunk of the row owned by this lane

  const int L = p.context_lens[s];
  int t0 = 0, t1 = L;
  if (p.partition_size > 0) {
    t0 = p.key_begin + part * p.partition_size;
    if (t0 >= L) return;  // partition past the end: the reduce ignores it
    t1 = min(L, t0 + p.partition_size);
  }

  uint4 q[G][QC];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.query) +
                      ((int64_t)s * p.num_heads + (int64_t)kvh * G) * (D / F::kVec) + ch * QC;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < QC; ++c) q[g][c] = qp[g * (D / F::kVec) + c];
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
  const int lbs = p.log2_bs;
  const int bs_mask = (1 << lbs) - 1;
  const int64_t lane_off = (int64_t)kvh * p.head_stride + ch * VEC;

  for (int w0 = t0; w0 < t1; w0 += kWindow) {
    const int w1 = min(t1, w0 + kWindow);
    const int e0 = w0 >> lbs;
    const int ne = ((w1 - 1) >> lbs) - e0 + 1;
    __syncthreads();  // the previous window's readers are done
    for (int i = threadIdx.x; i < ne; i += kDecodeThreads) s_bt[i] = bt[e0 + i];
    __syncthreads();

    // Rows past the window are clamped to its last row (finite data loaded
    // anyway) and masked by `valid`, so the loads are unconditional and none
    // waits for another.
    auto load = [&](int wbase, uint4 (&kr)[kUnroll], uint4 (&vr)[kUnroll], bool (&valid)[kUnroll]) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int t = wbase + u * TPS + tg;
        valid[u] = t < w1;
        const int tc = min(t, w1 - 1);
        const int64_t blk = s_bt[(tc >> lbs) - e0];
        const int64_t off = blk * p.blk_stride + (int64_t)(tc & bs_mask) * p.tok_stride + lane_off;
        kr[u] = load_nt(p.key_cache + off * CB);
        vr[u] = load_nt(p.value_cache + off * CB);
      }
    };

    // consume one batch: scores, lazy rescale, probabilities, V accumulation
    auto consume = [&](int wbase, const uint4 (&kr)[kUnroll], const uint4 (&vr)[kUnroll]) {
      bool valid[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) valid[u] = wbase + u * TPS + tg < w1;
      float z[kUnroll][G];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        uint4 kc[QC];
        if constexpr (FP8)
          fp8x16_to_pairs<DT>(kr[u], kc[0], kc[1]);
        else
          kc[0] = kr[u];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int c = 0; c < QC; ++c) d = dot_chunk<DT>(q[g][c], kc[c], d);
          d = group_sum<LPT>(d);
          z[u][g] = valid[u] ? d * p.scale_log2e : -INFINITY;
        }
      }
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
        if constexpr (FP8)
          fp8x16_to_f32(vr[u], vf);
        else
          chunk_to_f32<DT>(vr[u], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pw = valid[u] ? __builtin_amdgcn_exp2f(z[u][g] - m[g]) : 0.f;
          l[g] += pw;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[g][e] = __builtin_fmaf(pw, vf[e], acc[g][e]);
        }
      }
    };

    // ping-pong buffers: the next batch is always in flight (its rows past
    // the window are clamped, so the load is unconditional and no wait merges
    // across a branch)
    constexpr int kStep = kUnroll * TPS;
    uint4 ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
    bool dummy[kUnroll];
    int wbase = w0 + wave * TPW;  // wave-uniform: groups past the end carry invalid rows
    load(wbase, ka, va, dummy);
    while (wbase < w1) {
      load(wbase + kStep, kb, vb, dummy);
      consume(wbase, ka, va);
      wbase += kStep;
      if (wbase >= w1) break;
      load(wbase + kStep, ka, va, dummy);
      consume(wbase, kb, vb);
      wbase += kStep;
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
    emit(p, s, kvh * G + g, part, d, D, M, lsum, o, single_partition(p, L));
  }
}

template <pa_dtype DT, int D>
hipError_t launch_g(const DecodeParams& p, int G, dim3 grid, hipStream_t st) {
  dim3 block(kDecodeThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_reg_kernel<DT, D, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_reg_kernel<DT, D, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_reg_kernel<DT, D, 4>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_reg_kernel<DT, D, 8>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((decode_reg_kernel<DT, D, 16>), grid, block, 0, st, p); break;
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

// FP8 caches take this kernel for group sizes 1 and 2.
template <pa_dtype QT, int D>
hipError_t launch_fp8_g(const DecodeParams& p, int G, dim3 grid, hipStream_t st) {
  dim3 block(kDecodeThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_reg_kernel<QT, D, 1, true>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_reg_kernel<QT, D, 2, true>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <pa_dtype QT>
hipError_t launch_fp8_d(const DecodeParams& p, int D, int G, dim3 grid, hipStream_t st) {
  if (D == 64) return launch_fp8_g<QT, 64>(p, G, grid, st);
  if (D == 128) return launch_fp8_g<QT, 128>(p, G, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_head(const DecodeParams& p, pa_dtype dt, int D, int G, dim3 grid, hipStream_t st) {
  switch (dt) {
    case PA_F32: return launch_d<PA_F32>(p, D, G, grid, st);
    case PA_BF16: return launch_d<PA_BF16>(p, D, G, grid, st);
    case PA_F16: return launch_d<PA_F16>(p, D, G, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_head_fp8(const DecodeParams& p, pa_dtype qt, int D, int G, dim3 grid, hipStream_t st) {
  switch (qt) {
    case PA_BF16: return launch_fp8_d<PA_BF16>(p, D, G, grid, st);
    case PA_F16: return launch_fp8_d<PA_F16>(p, D, G, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
}  // namespace pa
