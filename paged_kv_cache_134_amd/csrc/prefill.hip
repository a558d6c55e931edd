// Causal packed-sequence prefill over the paged cache, on gfx950 matrix cores.
//
// What is computed follows "PagedAttention 在 vLLM 中的实现分析" §6.2
// (flash_attn_varlen_func with cu_seqlens_q = query_start_loc, seqlen_k =
// seq_lens, block_table, causal=True) and the packed layout of the
// cann-recipes-infer Paged KV Cache + Packed Sequence notes (§2.3: sequences
// packed back to back, located by exclusive-prefix-sum offsets).  Sequence s
// owns rows query_start_loc[s] .. query_start_loc[s+1]-1; with n rows and
// L = context_lens[s], row j sits at position L - n + j and sees keys
// 0 .. L - n + j.  Keys are read through the block table exactly as in decode.
//
// Kernel design (this file's own, for CDNA4 MFMA and wave64):
//   * a workgroup of 4 waves owns BM = 64 * QB query rows of one (sequence,
//     head); wave w owns 16 * QB rows, QB blocks of 16, so every K and V
//     fragment read from LDS feeds QB matrix instructions;
//   * key tiles of 64 keys are gathered through the block table into
//     registers one tile ahead of use, then into LDS: K row-major (bf16/f16
//     as stored) and V transposed to [d][key] in f16; keys past the last
//     visible position are read as the last visible key (finite data) and
//     masked, so no unwritten slot is ever read;
//   * workgroup ids are remapped so the query tiles of one (sequence, head)
//     run on one XCD and share its L2;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_{bf16,f16} (A = 16 keys x 32 d
//     from LDS, B = 32 d x 16 queries held in registers), so each lane holds
//     scores of ONE query (lane % 16) for 4 keys of every 16-key block;
//   * the same lane-to-query map holds for O^T = V^T P^T (A = 16 d x 32 keys
//     from the transposed V tile, B = 32 keys x 16 queries = this lane's own
//     probabilities, converted to f16, with the key order permuted
//     consistently in A and B), so the online-softmax statistics and the
//     output rescaling stay in-lane; the 4 lanes that share a query combine
//     their maxima with two cross-lane exchanges;
//   * probabilities are rounded to f16 before the PV product (relative error
//     at most 2^-11 per weight; V is converted exactly from bf16 and must lie
//     in f16 range); the normaliser sums the unrounded fp32 values; QK^T uses
//     the stored type with fp32 accumulation.
#include <hip/hip_runtime.h>

#include "kernel_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kBN = 64;              // keys per tile
constexpr float kLazyRescaleP = 8.f; // log2 headroom of the running max

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct PrefillParams {
  void* out;
  const char* query;
  const char* key_cache;
  const char* value_cache;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int64_t blk_stride;
  int64_t tok_stride;
  int64_t head_stride;
  int32_t max_blocks_per_seq;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t log2_bs;
  float scale_log2e;
  pa_dtype out_dtype;
  int32_t q_tiles;   // query tiles per sequence (of the longest)
  int32_t num_work;  // q_tiles * num_heads * num_seqs
};

template <pa_dtype DT>
__device__ __forceinline__ f32x4_t mfma_qk(const uint4& a, const uint4& b, f32x4_t c) {
  if constexpr (DT == PA_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_pv(const f16x8_t& a, const f16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D = head size, QB = 16-query blocks per wave.
template <pa_dtype DT, int D, int QB>
__global__ __launch_bounds__(kPrefillThreads, 3) void prefill_kernel(const PrefillParams p) {
  constexpr int BM = kPrefillWaves * 16 * QB;   // query rows per workgroup
  constexpr int KS = D / 32;                    // 32-wide k-steps over the head dim
  constexpr int DB = D / 16;                    // 16-wide output blocks
  constexpr int KROW = D * 2 + 16;              // LDS bytes per K row (padded)
  constexpr int VROW = kBN * 2 + 8;             // LDS bytes per V^T row (padded)
  constexpr int KCH = D / 8;                    // 16-byte chunks per K/V row
  constexpr int KPT = kBN * KCH / kPrefillThreads;        // K chunks per thread per tile
  constexpr int VITEMS = (kBN / 4) * KCH;      // V items of 4 keys x 8 columns per tile
  constexpr int VPT = (VITEMS + kPrefillThreads - 1) / kPrefillThreads;
  static_assert(KPT * kPrefillThreads == kBN * KCH, "K tile must split evenly");
  __shared__ __attribute__((aligned(16))) char sK[kBN * KROW];
  __shared__ __attribute__((aligned(16))) char sV[D * VROW];

  // XCD-aware order: consecutive workgroup ids are spread over the 8 XCDs
  // (each with its own L2), so the ids are remapped to give every XCD a
  // contiguous run of work items, i.e. the query tiles of one (sequence,
  // head), which read the same K/V tiles, share an L2.
  const int nwork = p.num_work;
  const int per_xcd = (nwork + 7) / 8;
  const int b = blockIdx.x;
  const int work = (b % 8) * per_xcd + b / 8;
  if (work >= nwork) return;
  const int qt = work % p.q_tiles;
  const int h = (work / p.q_tiles) % p.num_heads;
  const int s = work / (p.q_tiles * p.num_heads);

  const int q_begin = p.query_start_loc[s];
  const int n = p.query_start_loc[s + 1] - q_begin;
  const int q0 = qt * BM;
  if (q0 >= n) return;
  const int L = p.context_lens[s];
  const int kvh = h / (p.num_heads / p.num_kv_heads);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int lq = lane % 16;     // query (column) owned by this lane within a block
  const int lg = lane / 16;     // lane group: 4 keys / 8 k-elements slice

  // keys visible to the workgroup: 0 .. kend-1
  const int last_row = min(n, q0 + BM) - 1;
  const int kend = L - n + last_row + 1;

  // Q^T fragments (B operand): query row q0 + wave*16*QB + qb*16 + lq,
  // head-dim slice kstep*32 + lg*8 .. +7
  uint4 qf[QB][KS];
  int lim[QB];  // last visible key of this lane's query, per block
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int j = q0 + wave * 16 * QB + qb * 16 + lq;
    lim[qb] = L - n + j;
    const bool ok = j < n;
    const char* qp =
        p.query + (((int64_t)(q_begin + (ok ? j : 0)) * p.num_heads + h) * D) * Fmt<DT>::kBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb][ks] = ok ? load16(qp + (ks * 4 + lg) * 16) : make_uint4(0, 0, 0, 0);
  }

  f32x4_t o[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
  const int lbs = p.log2_bs;
  const int bs_mask = (1 << lbs) - 1;
  const int64_t head_off = (int64_t)kvh * p.head_stride;

  // Global -> registers for one key tile.  Keys past kend are clamped to the
  // last visible key (finite data the tile reads anyway); the causal mask
  // gives them probability 0, so every load is unconditional.  A thread
  // loads KPT consecutive 16-byte chunks of one K row and, for V, 4
  // consecutive keys of one 8-column slice: one block-table lookup each
  // (blocks of >= 4 tokens hold an aligned group of 4 keys).
  constexpr int KTPR = kPrefillThreads / kBN;  // threads per K row
  static_assert(KTPR * KPT == KCH, "K row split");
  const int k_row = tid / KTPR, k_cg = (tid % KTPR) * KPT;
  const int v_item = min(tid, VITEMS - 1);
  const int v_kq = v_item % (kBN / 4), v_dq = v_item / (kBN / 4);
  const bool bs_ge4 = lbs >= 2;
  struct TileRegs {
    uint4 k[KPT];
    uint4 v[4];
  };
  auto fetch = [&](int k0) {
    TileRegs r;
    {
      const int t = min(k0 + k_row, kend - 1);
      const char* src = p.key_cache + ((int64_t)bt[t >> lbs] * p.blk_stride +
                                       (int64_t)(t & bs_mask) * p.tok_stride + head_off + k_cg * 8) * 2;
#pragma unroll
      for (int i = 0; i < KPT; ++i) r.k[i] = load16(src + i * 16);
    }
    {
      const int tb = min(k0 + v_kq * 4, kend - 1);
      const int64_t blk0 = (int64_t)bt[tb >> lbs] * p.blk_stride;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = min(k0 + v_kq * 4 + j, kend - 1);
        const int64_t blk = bs_ge4 ? blk0 : (int64_t)bt[t >> lbs] * p.blk_stride;
        r.v[j] = load16(p.value_cache +
                        (blk + (int64_t)(t & bs_mask) * p.tok_stride + head_off + v_dq * 8) * 2);
      }
    }
    return r;
  };
  // smallest visible-key limit among this wave's query rows
  const int lim_min = L - n + q0 + wave * 16 * QB;

  TileRegs tr = fetch(0);
  for (int k0 = 0; k0 < kend; k0 += kBN) {
    // ---- registers -> LDS: K row-major, V transposed to [d][key] in f16
#pragma unroll
    for (int i = 0; i < KPT; ++i) store16(sK + k_row * KROW + (k_cg + i) * 16, tr.k[i]);
    if (VITEMS % kPrefillThreads == 0 || tid < VITEMS) {  // head size 64: half the threads stage no V
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f16x4_t col;
#pragma unroll
        for (int j = 0; j < 4; ++j) col[j] = (_Float16)chunk_elem<DT>(tr.v[j], e);
        *reinterpret_cast<f16x4_t*>(sV + (v_dq * 8 + e) * VROW + v_kq * 8) = col;
      }
    }
    __syncthreads();
    tr = fetch(k0 + kBN);  // next tile in flight (clamped past the end: never a wait on a branch)

    // ---- S^T = K Q^T for 4 key blocks of 16
    float sc[QB][4][4];  // [query block][key block][key within lane group]
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4_t acc[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) acc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = load16(sK + (kb * 16 + lq) * KROW + ks * 64 + lg * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb] = mfma_qk<DT>(a, qf[qb][ks], acc[qb]);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[qb][kb][i] = acc[qb][i];
    }

    // ---- online softmax, in-lane per query; 4 lanes share a query.  Only
    // tiles that reach past some row's last visible key need the mask.
    const bool need_mask = k0 + kBN - 1 > lim_min;  // wave-uniform
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + kb * 16 + lg * 4 + i;
          float zz = sc[qb][kb][i] * p.scale_log2e;
          if (need_mask && key > lim[qb]) zz = -INFINITY;
          sc[qb][kb][i] = zz;
          mt = fmaxf(mt, zz);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (__any(mt > m[qb] + kLazyRescaleP)) {
        const float mn = fmaxf(m[qb], mt);
        const float a = exp2_diff(m[qb], mn);
        m[qb] = mn;
        l[qb] *= a;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= a;
      }
    }

    // ---- O^T += V^T P^T, 2 k-steps of 32 keys (key blocks 2ks, 2ks+1)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8_t pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // every query sees key 0, so m is finite here and exp2(-inf) = 0
          const float e0 = __builtin_amdgcn_exp2f(sc[qb][2 * ks][i] - m[qb]);
          const float e1 = __builtin_amdgcn_exp2f(sc[qb][2 * ks + 1][i] - m[qb]);
          pb[qb][i] = (_Float16)e0;
          pb[qb][4 + i] = (_Float16)e1;
          l[qb] += e0 + e1;
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* vrow = sV + (db * 16 + lq) * VROW;
        const f16x4_t lo = *reinterpret_cast<const f16x4_t*>(vrow + (ks * 32 + lg * 4) * 2);
        const f16x4_t hi = *reinterpret_cast<const f16x4_t*>(vrow + (ks * 32 + 16 + lg * 4) * 2);
        const f16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma_pv(a, pb[qb], o[qb][db]);
      }
    }
    __syncthreads();
  }

  // ---- normalise and store: lane holds O[query lq][d = db*16 + lg*4 + i]
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float lt = l[qb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int j = q0 + wave * 16 * QB + qb * 16 + lq;
    if (j >= n) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t row = ((int64_t)(q_begin + j) * p.num_heads + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) store_out(p.out, row + db * 16 + lg * 4 + i, o[qb][db][i] * inv, p.out_dtype);
  }
}

template <pa_dtype DT, int D>
hipError_t launch_pd(PrefillParams p, int num_seqs, int max_q, hipStream_t st) {
  constexpr int QB = 1;
  constexpr int BM = kPrefillWaves * 16 * QB;
  p.q_tiles = (max_q + BM - 1) / BM;
  const int64_t nwork = (int64_t)p.q_tiles * p.num_heads * num_seqs;
  if (nwork > 0x7FFFFFFF - 8) return hipErrorInvalidValue;
  p.num_work = (int)nwork;
  dim3 grid((unsigned)(((nwork + 7) / 8) * 8)), block(kPrefillThreads);
  hipLaunchKernelGGL((prefill_kernel<DT, D, QB>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const PoolGeom& g = a.geom;
  if (a.num_seqs == 0 || a.num_tokens == 0 || a.max_query_len == 0) return hipSuccess;
  PrefillParams p{};
  p.out = a.out;
  p.query = static_cast<const char*>(a.query);
  p.key_cache = static_cast<const char*>(a.key_cache);
  p.value_cache = static_cast<const char*>(a.value_cache);
  p.block_tables = a.block_tables;
  p.query_start_loc = a.query_start_loc;
  p.context_lens = a.context_lens;
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
  p.log2_bs = __builtin_ctz((unsigned)g.block_size);
  p.scale_log2e = a.scale * kLog2e;
  p.out_dtype = a.out_dtype;
  if (a.kv_dtype == PA_BF16) {
    if (g.head_size == 64) return launch_pd<PA_BF16, 64>(p, a.num_seqs, a.max_query_len, stream);
    if (g.head_size == 128) return launch_pd<PA_BF16, 128>(p, a.num_seqs, a.max_query_len, stream);
  } else if (a.kv_dtype == PA_F16) {
    if (g.head_size == 64) return launch_pd<PA_F16, 64>(p, a.num_seqs, a.max_query_len, stream);
    if (g.head_size == 128) return launch_pd<PA_F16, 128>(p, a.num_seqs, a.max_query_len, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
