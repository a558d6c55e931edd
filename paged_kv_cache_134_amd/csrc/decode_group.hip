// Paged decode, grouped kernel (group size 4, 8 or 16 with bf16/f16 caches).
//
// One workgroup of 4 waves per (sequence, kv head, partition) reads the kv
// head's K/V rows once for all G query heads of its group (contract and
// sources as in the per-head kernel).  Per chunk of 64 tokens the workgroup
// copies K and V rows (coalesced 16-byte loads, prefetched one chunk ahead
// in registers) into LDS.  QK: lane = token, each wave owns G/4 query heads
// whose query vectors are read as scalar (SGPR) operands of v_dot2, and K
// rows sit in LDS with a padded row stride (consecutive rows start in
// consecutive 16-byte bank groups, so a lane-per-row read is conflict-free
// with a constant offset); no cross-lane reduction and one exp per (token,
// head).  PV: lane owns D/32 output columns of all G heads and each wave a
// quarter of the chunk's tokens, as token pairs on f16 v_dot2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "decode_common.h"

namespace pa {
namespace dec {
namespace {

constexpr int kChunk = 64;   // tokens per LDS chunk (one per lane in QK)
constexpr int kBtWin = 128;  // block-table entries staged in LDS at a time

// 4 waves per SIMD (<= 128 VGPRs): with ~35 KB of LDS per workgroup that is
// 4 workgroups, i.e. 128 KB of prefetched K/V in flight, per CU.  (G = 16 at
// head size 128 needs more accumulators and settles for 2.)  OFF32: both
// caches span less than 4 GiB, so row addresses are 32-bit byte offsets from
// the cache base.
//
// Precision: QK products are exact (bf16/f16 pairs on v_dot2, fp32 sums);
// the weights 2^(z - m) stay fp32, the normaliser sums those same fp32
// values, and PV multiplies them with V converted exactly to fp32 (any
// magnitude, infinities and NaN included).
template <int G, int D>
constexpr int kLdsMinWaves = (G >= 16 && D >= 128) ? 2 : 4;

template <pa_dtype DT, int D, int G, bool OFF32>
__global__ __launch_bounds__(kDecodeThreads, (kLdsMinWaves<G, D>)) void decode_lds_kernel(
    const DecodeParams p) {
  static_assert(DT != PA_F32, "LDS kernel takes 16-bit elements");
  static_assert(G % kDecodeWaves == 0, "G must be a multiple of 4");
  constexpr int RC = D / 8;                        // 16-byte pieces per row
  constexpr int PIECES = kChunk * RC;              // pieces per chunk of K (or V)
  constexpr int PPT = PIECES / kDecodeThreads;     // pieces per thread per tensor
  constexpr int RSTEP = kDecodeThreads / RC;       // rows between a thread's pieces
  constexpr int HPW = G / kDecodeWaves;            // query heads per wave in QK
  constexpr int DPL = D / 32;                      // output columns per lane in PV
  constexpr int NPI = kChunk / kDecodeWaves / 4;   // PV token-pair iterations per wave
  static_assert(PPT * kDecodeThreads == PIECES, "chunk must split evenly");
  static_assert(kDecodeWaves * G * D * 4 <= (kChunk * (RC + 1) + PIECES) * 16, "merge fits the tiles");
  constexpr int KSTR = RC + 1;                     // K row stride in pieces (padded)
  __shared__ uint4 sKV[kChunk * KSTR + PIECES];    // K (padded rows) then V; reused by the merges
  __shared__ __align__(16) float sP[kChunk / 2][G][2];  // probabilities, token pairs interleaved
  __shared__ float sAlpha[G];                      // per-head rescale of this chunk
  __shared__ int32_t sResc[kDecodeWaves];          // wave w moved a running max this chunk
  __shared__ float sM[G], sL[G];
  __shared__ int32_t s_bt[kBtWin];                 // block-table window
  uint4* sK = sKV;
  uint4* sV = sKV + kChunk * KSTR;

  int s, kvh, part;
  if (!decode_item(p, true, s, kvh, part)) return;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  // Tokens [t0, t1): the partition (split-K) or the whole context (single
  // pass).
  const int L = p.context_lens[s];
  const int P = p.partition_size;
  int t0 = 0, t1 = L;
  if (P > 0) {
    t0 = p.key_begin + part * P;
    if (t0 >= L) return;
    t1 = min(L, t0 + P);
  }
  const int64_t head0 = (int64_t)s * p.num_heads + (int64_t)kvh * G;
  if (t1 <= t0) {  // single pass over an empty context (split-K returned above)
    emit_zero_rows(p, head0, G, D);
    return;
  }
  const bool single = single_partition(p, L);

  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
  const int lbs = p.log2_bs;
  const int bs_mask = (1 << lbs) - 1;
  const int e_last = (t1 - 1) >> lbs;  // last block-table entry this workgroup reads

  // query vectors of this wave's heads as scalar operands (bf16/f16 pairs)
  const const_u32_ptr qc = (const_u32_ptr)((const char*)p.query + ((head0 + wave * HPW) * D) * 2);

  // Consecutive lanes load consecutive 16-byte chunks of a row, so every
  // load instruction covers whole cache lines (the loads are non-temporal and
  // a partly used line would be fetched again).  Rows at or past the end are
  // clamped to the last row (a valid, finite row the chunk loads anyway) and
  // masked where they are used, so every load is unconditional.  Block ids
  // come from the LDS window, so no load waits on another global load.
  const int prow = tid / RC;
  const int pcol = tid % RC;
  const int64_t lane_off = (int64_t)kvh * p.head_stride + pcol * 8;  // elements
  const uint32_t blk_b = (uint32_t)(p.blk_stride * 2);
  const uint32_t tok_b = (uint32_t)(p.tok_stride * 2);
  const uint32_t lane_b = (uint32_t)(lane_off * 2);

  const int half = lane / 32;  // PV: token parity within a pair
  const int dl = lane % 32;    // PV: output columns dl*DPL .. +DPL-1
  // PV bases: V row 2 (wave * 8 + half) at the lane's columns, and the weight
  // pairs of token pair wave * 8 + half
  const char* pv_base = reinterpret_cast<const char*>(sV) +
                        (2 * (wave * (kChunk / kDecodeWaves / 2) + half) * RC) * 16 + dl * DPL * 2;
  const char* pp_base = reinterpret_cast<const char*>(&sP[wave * (kChunk / kDecodeWaves / 2) + half][0][0]);

  int wb0 = t0 >> lbs;  // the window holds entries wb0 .. wb0 + kBtWin - 1 (clamped to e_last)
  auto stage_bt = [&]() {
    for (int i = tid; i < kBtWin; i += kDecodeThreads) s_bt[i] = bt[min(wb0 + i, e_last)];
  };
  auto fetch = [&](int c0, uint4 (&kr)[PPT], uint4 (&vr)[PPT]) {
    int32_t blk[PPT];
    int tc[PPT];
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      tc[r] = min(c0 + prow + RSTEP * r, t1 - 1);
      blk[r] = s_bt[(tc[r] >> lbs) - wb0];
    }
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      if constexpr (OFF32) {
        const uint32_t off = (uint32_t)blk[r] * blk_b + (uint32_t)(tc[r] & bs_mask) * tok_b + lane_b;
        kr[r] = load_nt(p.key_cache + off);
        vr[r] = load_nt(p.value_cache + off);
      } else {
        const int64_t off = (int64_t)blk[r] * p.blk_stride +
                            (int64_t)(tc[r] & bs_mask) * p.tok_stride + lane_off;
        kr[r] = load_nt(p.key_cache + off * 2);
        vr[r] = load_nt(p.value_cache + off * 2);
      }
    }
  };

  // Softmax state: reference max and lane sums of this wave's QK heads, and
  // the lane's PV accumulators (its tokens, all heads, its columns).
  float m_ref[HPW], l_lane[HPW];
  float acc[G][DPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m_ref[hh] = -INFINITY;
    l_lane[hh] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;

  // One chunk in flight in registers while the previous one is consumed
  // from LDS.
  auto step = [&](int c0, bool more, uint4 (&kr)[PPT], uint4 (&vr)[PPT]) {
    const int cn = c0 + kChunk;
    __syncthreads();  // previous chunk fully consumed, window reads included
#pragma unroll
    for (int r = 0; r < PPT; ++r) {  // piece tid + 256 r: row prow + RSTEP r, column pcol
      sK[(prow + RSTEP * r) * KSTR + pcol] = kr[r];
      sV[tid + kDecodeThreads * r] = vr[r];
    }
    if (more && (min(cn + kChunk - 1, t1 - 1) >> lbs) - wb0 >= kBtWin) {  // uniform
      wb0 = cn >> lbs;
      stage_bt();
    }
    __syncthreads();
    if (more) fetch(cn, kr, vr);  // next chunk in flight

    // ---- QK: lane = token row, this wave's HPW heads
    const int row = lane;
    const bool valid = c0 + row < t1;
    float z[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) z[hh] = 0.f;
#pragma unroll 1
    for (int pc = 0; pc < RC; pc += 4) {
      uint4 kk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) kk[j] = sK[row * KSTR + pc + j];  // padded rows: conflict-free
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const const_u32_ptr qh = qc + hh * (D / 2) + pc * 4;
        float a = z[hh];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 qq = make_uint4(qh[4 * j], qh[4 * j + 1], qh[4 * j + 2], qh[4 * j + 3]);
          a = dot_chunk<DT>(qq, kk[j], a);
        }
        z[hh] = a;
      }
    }
    // ---- online softmax of this wave's heads.  The running max moves only
    // when some token of the chunk exceeds it by more than the headroom, so
    // the wave-wide maximum is taken only then (a ballot decides).
    bool resc = false;
    float alpha[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = wave * HPW + hh;
      const float zz = valid ? z[hh] * p.scale_log2e : -INFINITY;
      alpha[hh] = 1.f;
      if (__any(zz > m_ref[hh] + kLazyRescale)) {
        const float mn = fmaxf(m_ref[hh], wave_max(zz));
        alpha[hh] = exp2_diff(m_ref[hh], mn);
        m_ref[hh] = mn;
        l_lane[hh] *= alpha[hh];
        resc = true;
      }
      // the PV weights and the normaliser use the same fp32 value
      const float pw = valid ? __builtin_amdgcn_exp2f(zz - m_ref[hh]) : 0.f;
      l_lane[hh] += pw;
      sP[row >> 1][h][row & 1] = pw;
    }
    if (lane == 0) {
      sResc[wave] = resc;
      if (resc) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) sAlpha[wave * HPW + hh] = alpha[hh];
      }
    }
    __syncthreads();

    // ---- PV: wave owns rows 16 wave .. +15 as 8 token pairs; a half-wave
    // takes pairs (2j, 2j+1) and a lane D/32 columns of all G heads.  Rows
    // past the end carry p = 0 and finite (clamped) V.
    // Heads of QK wave w are rescaled only when that wave moved a max.
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (__builtin_amdgcn_readfirstlane(sResc[w])) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          const float a = sAlpha[w * HPW + hh];
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[w * HPW + hh][e] *= a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      const char* va = pv_base + i * (4 * RC * 16);  // pair wave * 8 + 2 i + half
      const char* vb = va + RC * 16;
      uint32_t wa[DPL / 2], wb[DPL / 2];
      if constexpr (DPL == 4) {
        const uint2 a2 = *reinterpret_cast<const uint2*>(va);
        const uint2 b2 = *reinterpret_cast<const uint2*>(vb);
        wa[0] = a2.x; wa[1] = a2.y; wb[0] = b2.x; wb[1] = b2.y;
      } else {
        wa[0] = *reinterpret_cast<const uint32_t*>(va);
        wb[0] = *reinterpret_cast<const uint32_t*>(vb);
      }
      float fa[DPL], fb[DPL];
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        fa[c] = chunk_elem<DT>(make_uint4(wa[c / 2], 0, 0, 0), c & 1);
        fb[c] = chunk_elem<DT>(make_uint4(wb[c / 2], 0, 0, 0), c & 1);
      }
      // weights of the pair for all G heads: (token 2j, token 2j+1) per head
      const float4* pq = reinterpret_cast<const float4*>(pp_base + i * (2 * G * 2 * 4));
#pragma unroll
      for (int h2 = 0; h2 < G / 2; ++h2) {
        const float4 w4 = pq[h2];  // heads 2 h2 and 2 h2 + 1
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          acc[2 * h2][c] = __builtin_fmaf(w4.y, fb[c], __builtin_fmaf(w4.x, fa[c], acc[2 * h2][c]));
          acc[2 * h2 + 1][c] =
              __builtin_fmaf(w4.w, fb[c], __builtin_fmaf(w4.z, fa[c], acc[2 * h2 + 1][c]));
        }
      }
    }
  };

  stage_bt();
  __syncthreads();  // window staged
  uint4 kr[PPT], vr[PPT];
  fetch(t0, kr, vr);
  for (int c0 = t0; c0 < t1; c0 += kChunk) step(c0, c0 + kChunk < t1, kr, vr);  // uniform

  // ---- merge of the halves, then of the waves (the statistics come from
  // the QK waves); the chunk tiles' LDS holds the waves' accumulators
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], 32);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float lt = wave_sum(l_lane[hh]);
    if (lane == 0) {
      sM[wave * HPW + hh] = m_ref[hh];
      sL[wave * HPW + hh] = lt;
    }
  }
  __syncthreads();  // the last chunk's PV reads are done: the tiles are free
  float* sAcc = reinterpret_cast<float*>(sKV);  // [waves][G][D]
  if (half == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DPL; ++e) sAcc[(wave * G + h) * D + dl * DPL + e] = acc[h][e];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kDecodeThreads) {
    const int h = i / D, d = i % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) o += sAcc[(w * G + h) * D + d];
    emit(p, s, kvh * G + h, part, d, D, sM[h], sL[h], o, single);
  }
}

template <pa_dtype DT, int D, bool OFF32>
hipError_t launch_lds(const DecodeParams& p, int G, dim3 grid, hipStream_t st) {
  dim3 block(kDecodeThreads);
  switch (G) {
    case 4: hipLaunchKernelGGL((decode_lds_kernel<DT, D, 4, OFF32>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_lds_kernel<DT, D, 8, OFF32>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((decode_lds_kernel<DT, D, 16, OFF32>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <pa_dtype DT>
hipError_t launch_d(const DecodeParams& p, int D, int G, dim3 grid, hipStream_t st) {
  if (D == 64) return p.off32 ? launch_lds<DT, 64, true>(p, G, grid, st) : launch_lds<DT, 64, false>(p, G, grid, st);
  if (D == 128) return p.off32 ? launch_lds<DT, 128, true>(p, G, grid, st) : launch_lds<DT, 128, false>(p, G, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_group(const DecodeParams& p, pa_dtype dt, int D, int G, dim3 grid, hipStream_t st) {
  switch (dt) {
    case PA_BF16: return launch_d<PA_BF16>(p, D, G, grid, st);
    case PA_F16: return launch_d<PA_F16>(p, D, G, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
}  // namespace pa
