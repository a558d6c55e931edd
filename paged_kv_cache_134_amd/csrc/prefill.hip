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
//   * a workgroup of 4 waves owns 128 query rows of one (sequence, head);
//     wave w owns 32 rows, one 32-wide MFMA column block;
//   * key tiles of 64 keys are gathered through the block table into
//     registers one tile ahead of use, then into LDS: K row-major (bf16/f16
//     as stored) and V transposed to [d][key] in f16, its 4-key groups
//     reordered within each 16-key slice so that a lane's PV operand is one
//     16-byte read (row strides of 4 mod 32 dwords: conflict-free); keys past the last
//     visible position are read as the last visible key (finite data) and
//     masked, so no unwritten slot is ever read;
//   * workgroup ids are remapped so the query tiles of one (sequence, head)
//     run on one XCD and share its L2;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16} (A = 32 keys x 16 d
//     from LDS, B = 16 d x 32 queries held in registers), so each lane holds
//     16 scores of ONE query (lane % 32) and the other half-wave the other 16
//     keys of each 32-key block: one cross-lane exchange per row maximum;
//   * O^T = V^T P^T with the same lane-to-query map (A = 32 d x 16 keys from
//     the transposed V tile, B = 16 keys x 32 queries = this lane's own
//     probabilities, with the key order permuted consistently in A and B),
//     so the online-softmax statistics and the output rescaling stay
//     in-lane;
//   * scores stay unscaled until exp2(fma(z, scale*log2e, 7 - m)); the
//     running max moves only past a 2^8 headroom (a ballot decides), so a
//     weight is at most 2^15; each weight is split into two f16 terms, hi =
//     f16(p) and lo = f16(p - hi), and PV takes both products on the same V
//     operand, so the weights carry about 22 significant bits (relative
//     error below 2^-20, plus 2^-24 absolute in the scaled units for weights
//     below 2^-10 of the reference); the normaliser sums hi + lo with v_dot2,
//     so the weights that multiply V are exactly the ones that are divided
//     out, and the 2^7 cancels (prefix partials are written without it);
//     QK^T uses the stored type with fp32 accumulation;
//   * V is staged as f16: exactly for f16 and FP8 caches, and for bf16
//     values below 2^16 in magnitude.  A bf16 tile holding a finite |v| of
//     2^16 or more (found while it is staged) sends the workgroup back to
//     its first tile with V stored as v * 2^-vsh, vsh chosen from that
//     magnitude so the largest value seen stays below 2^15 (exact but for
//     values under 2^-24 of the scaled range, which become f16 subnormals);
//     the output is multiplied by 2^vsh.  Infinities and NaN pass through
//     as themselves;
//   * a wave whose rows are all padding, or that sees none of a tile's keys,
//     skips that tile's products; the wave index goes through readfirstlane
//     so these tests, and the causal mask (applied only to tiles that reach
//     past some row's last visible key), are scalar branches rather than
//     per-score selects;
//   * FP8 (E4M3) caches: K converts exactly to the query's type and V to f16
//     on their way into LDS, so the products are those of a 16-bit cache;
//     k_scale is folded into the softmax scale and v_scale into the final
//     normalisation.  Every instantiation runs 2 waves per SIMD.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernel_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kQW = 32;                         // query rows per wave
constexpr int kBM = kPrefillWaves * kQW;        // query rows per workgroup
constexpr int kBN = 64;                         // keys per tile
constexpr float kLazyRescaleP = 8.f;            // log2 headroom of the running max
constexpr float kWeightLog2 = 7.f;              // weights carry 2^7 (largest 2^15, within f16)
constexpr int kBtWinP = 256;                    // block-table entries staged in LDS at a time

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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
  float scale_log2e;  // softmax scale * log2(e), times k_scale for FP8 caches
  float v_scale;      // FP8 caches: applied with the normalisation (else 1)
  pa_dtype out_dtype;
  int32_t q_tiles;   // query tiles per sequence (of the longest)
  int32_t num_work;  // (sequence, head) pairs: num_heads * num_seqs (prefix mode: (head, key part))
  // shared-prefix mode: rows 0 .. num_rows-1 attend to keys [0, prefix_keys)
  // of block_tables row 0 in key_parts partitions of key_part keys
  int32_t num_rows;
  int32_t prefix_keys;
  int32_t key_part;
  int32_t key_parts;
  float* part_out;
  float* part_ml;
  int32_t max_partitions;
};


// 32x32x16 products: lane l holds A[m = l%32][k = 8(l/32) .. +7],
// B[k = 8(l/32) .. +7][n = l%32] and D[m = 8(i/4) + 4(l/32) + i%4][n = l%32].
template <pa_dtype DT>
__device__ __forceinline__ f32x16_t mfma_qk(const uint4& a, const uint4& b, f32x16_t c) {
  if constexpr (DT == PA_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// e - (the low / high f16 half of h, widened): one mixed-precision FMA each
// (v_fma_mix_f32 reads an f16 source exactly; the compiler keeps a
// conversion and a subtraction for the same expression).  Register-only.
__device__ __forceinline__ float sub_f16_lo(float e, uint32_t h) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(e));
  return r;
}
__device__ __forceinline__ float sub_f16_hi(float e, uint32_t h) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(e));
  return r;
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes as floats.
__device__ __forceinline__ void fp8x8_to_f32(const uint4& v, float* out) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, false);
  const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, true);
  out[0] = a.x; out[1] = a.y; out[2] = b.x; out[3] = b.y;
  out[4] = c.x; out[5] = c.y; out[6] = d.x; out[7] = d.y;
}

// D = head size; DT = the query's type (and the cache's, unless FP8).
// OFF32: both caches span less than 4 GiB, so rows are addressed by 32-bit
// byte offsets from the cache base.  PREFIX: the shared-prefix pass of a
// cascade -- every query row sees every key of its key partition (no causal
// mask) and writes a (max, sum, unnormalised output) partial instead of a
// normalised row.  FP8: the caches hold E4M3 codes (partials then carry
// v_scale, as the decode kernels' partials do).
// Waves per SIMD the register budget is set for: 2 (218-220 VGPRs at head
// size 128).  The FP8 kernel's staging registers are half as many, but with
// the two-term weights a 3-wave bound spills it (12 VGPRs), and it measured
// slower than at 2 waves (5c over FP8 pools: 2.17-2.22 ms against
// 2.06 ms).
constexpr int kPrefillMinWaves = 2;

template <pa_dtype DT, int D, bool OFF32, bool PREFIX, bool FP8>
__global__ __launch_bounds__(kPrefillThreads, kPrefillMinWaves) void prefill_kernel(
    const PrefillParams p) {
  constexpr int CB = FP8 ? 1 : 2;               // cache bytes per element
  constexpr int KS = D / 16;                    // 16-wide k-steps over the head dim (QK)
  constexpr int DB = D / 32;                    // 32-row blocks of O^T
  constexpr int KROW = D * 2 + 16;              // LDS bytes per K row (padded)
  constexpr int VROW = kBN * 2 + 16;            // LDS bytes per V^T row (padded: 36 dwords)
  constexpr int KCH = D / 8;                    // 16-byte LDS chunks per K row
  constexpr int GCH = D * CB / 16;              // 16-byte cache chunks per K row
  constexpr int KPT = kBN * GCH / kPrefillThreads;        // cache chunks per thread per tile
  constexpr int VITEMS = (kBN / 4) * KCH;      // V items of 4 keys x 8 columns per tile
  static_assert(KPT * kPrefillThreads == kBN * GCH, "K tile must split evenly");
  static_assert(VITEMS <= kPrefillThreads, "one V item per thread");
  __shared__ __attribute__((aligned(16))) char sK[kBN * KROW];
  __shared__ __attribute__((aligned(16))) char sV[D * VROW];
  __shared__ int32_t s_bt[kBtWinP];  // block-table window
  // per tile parity: largest finite |v| (bf16 bits) beyond the current V range, 0 = none
  __shared__ int32_t sVwide[2];
  constexpr bool kWideCheck = !FP8 && DT == PA_BF16;

  // XCD-aware order: consecutive workgroup ids go round-robin to the 8 XCDs
  // (each with its own L2).  Pairs are numbered head-major (pair = head *
  // num_seqs + sequence) and XCD x takes pairs x, x + 8, x + 16, ...: all
  // query tiles of a pair, which read the same K/V tiles, run back to back
  // on one XCD; each XCD works through the heads in order, so a head's
  // shared prefix blocks stay in its L2 while the sequences that share them
  // pass; and interleaving the pairs keeps the XCDs' shares even when
  // sequence lengths vary.
  const int b = blockIdx.x;
  const int local = b / 8;
  const int pair = (local / p.q_tiles) * 8 + b % 8;
  if (pair >= p.num_work) return;  // num_work counts (sequence, head) pairs
  const int qt = local % p.q_tiles;
  int h, s, q_begin, n, L, k_lo;
  if constexpr (PREFIX) {
    // pairs (head, key part); all rows form one batch, keys [k_lo, k_lo + key_part)
    h = pair / p.key_parts;
    const int kp = pair % p.key_parts;
    s = kp;  // block-table row 0 is used; s names the key partition below
    q_begin = 0;
    n = p.num_rows;
    k_lo = kp * p.key_part;
    L = min(p.prefix_keys, k_lo + p.key_part);
  } else {
    const int num_seqs = p.num_work / p.num_heads;
    h = pair / num_seqs;
    s = pair % num_seqs;
    q_begin = p.query_start_loc[s];
    n = p.query_start_loc[s + 1] - q_begin;
    L = p.context_lens[s];
    k_lo = 0;
  }
  const int q0 = qt * kBM;
  if (q0 >= n) return;
  const int kvh = h / (p.num_heads / p.num_kv_heads);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: the mask and skip tests branch on scalars
  const int lq = lane % 32;     // query (column) owned by this lane
  const int hf = lane / 32;     // half: k-slice 8 hf .. +7, rows 4 hf .. +3 of each 8

  // keys visible to the workgroup: k_lo .. kend-1 (prefix mode: all of the
  // partition for every row)
  const int last_row = min(n, q0 + kBM) - 1;
  const int kend = PREFIX ? L : L - n + last_row + 1;

  // Q^T fragments (B operand): query row j, head-dim slice ks*16 + 8 hf .. +7
  const int j = q0 + wave * kQW + lq;
  const int lim = PREFIX ? L - 1 : L - n + j;  // last visible key of this lane's query
  uint4 qf[KS];
  {
    const bool ok = j < n;
    const char* qp =
        p.query + (((int64_t)(q_begin + (ok ? j : 0)) * p.num_heads + h) * D) * Fmt<DT>::kBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = ok ? load16(qp + (ks * 2 + hf) * 16) : make_uint4(0, 0, 0, 0);
  }

  f32x16_t o[DB];
  float m, l;

  const int32_t* bt = p.block_tables + (PREFIX ? 0 : (int64_t)s * p.max_blocks_per_seq);
  const int lbs = p.log2_bs;
  const int bs_mask = (1 << lbs) - 1;
  const int64_t head_off = (int64_t)kvh * p.head_stride;
  const uint32_t blk_b = (uint32_t)(p.blk_stride * CB);
  const uint32_t tok_b = (uint32_t)(p.tok_stride * CB);
  // byte offset of row t (in block blk) at element column col
  auto row_off = [&](int32_t blk, int t, int col) -> int64_t {
    if constexpr (OFF32)
      return (int64_t)((uint32_t)blk * blk_b + (uint32_t)(t & bs_mask) * tok_b +
                       (uint32_t)((head_off + col) * CB));
    else
      return ((int64_t)blk * p.blk_stride + (int64_t)(t & bs_mask) * p.tok_stride + head_off + col) * CB;
  };

  // Block ids come from an LDS window of the table (entries wb0 ..
  // wb0 + kBtWinP - 1, clamped to the last entry the workgroup reads), so no
  // tile load waits on another global load.
  const int e_last = (kend - 1) >> lbs;
  int wb0 = k_lo >> lbs;
  auto stage_bt = [&]() {
    for (int i = tid; i < kBtWinP; i += kPrefillThreads) s_bt[i] = bt[min(wb0 + i, e_last)];
  };

  // Global -> registers for one key tile.  Keys past kend are clamped to the
  // last visible key (finite data the tile reads anyway); the causal mask
  // gives them probability 0, so every load is unconditional.  A thread
  // loads KPT consecutive 16-byte chunks of one K row and, for V, 4
  // consecutive keys of one 8-column slice: one block-table lookup each
  // (blocks of >= 4 tokens hold an aligned group of 4 keys).
  constexpr int KTPR = kPrefillThreads / kBN;  // threads per K row
  static_assert(KTPR * KPT == GCH, "K row split");
  const int k_row = tid / KTPR, k_cg = (tid % KTPR) * KPT;
  // 16-bit caches: chunk i of this thread is 2 q + 8 (i / 2) + i % 2 (q = tid
  // % 4), so the 8 lanes of one LDS write (2 rows) hit 8 different 4-bank
  // groups; FP8 caches take KPT consecutive chunks
  auto k_chunk = [&](int i) { return FP8 ? k_cg + i : 2 * (tid % KTPR) + 8 * (i / 2) + (i % 2); };
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
      const char* src = p.key_cache + row_off(s_bt[(t >> lbs) - wb0], t, 0);
#pragma unroll
      for (int i = 0; i < KPT; ++i) r.k[i] = load16(src + k_chunk(i) * 16);
    }
    {
      const int tb = min(k0 + v_kq * 4, kend - 1);
      const int32_t blk0 = s_bt[(tb >> lbs) - wb0];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = min(k0 + v_kq * 4 + e, kend - 1);
        const char* src = p.value_cache + row_off(bs_ge4 ? blk0 : s_bt[(t >> lbs) - wb0], t, v_dq * 8);
        if constexpr (FP8) {  // 8 codes
          const uint2 c8 = *reinterpret_cast<const uint2*>(src);
          r.v[e] = make_uint4(c8.x, c8.y, 0, 0);
        } else {
          r.v[e] = load16(src);
        }
      }
    }
    return r;
  };
  // smallest and largest visible-key limits among this wave's query rows; a
  // wave whose rows are all padding, or that sees none of a tile's keys,
  // skips that tile's products (it still stages K/V and meets the barriers)
  const int lim_min = PREFIX ? L - 1 : L - n + q0 + wave * kQW;
  const int lim_max = PREFIX ? L - 1 : L - n + min(n - 1, q0 + wave * kQW + kQW - 1);
  const bool wave_rows = q0 + wave * kQW < n;
  const float c = p.scale_log2e;
  const uint32_t ones = pk_f16(1.f, 1.f);

#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  m = -INFINITY;
  l = 0.f;
  stage_bt();
  if (kWideCheck && tid == 0) sVwide[0] = sVwide[1] = 0;
  __syncthreads();
  int vsh = 0;  // V is held in the tile as v * 2^-vsh (grows only for bf16 caches)
  int ti = 0;   // tile count (its parity selects the V-range flag)
  TileRegs tr = fetch(k_lo);
  // V of tile registers -> LDS, transposed to [d][key] in f16 (times
  // 2^-vsh once a shift is in force: a uniform branch, so the common path
  // converts only).  CHECK (bf16 caches): also flag, in sVwide, a finite
  // value too large for the current shift.
  auto stage_v = [&](auto check_tag) {
    constexpr bool CHECK = decltype(check_tag)::value;
    if (VITEMS == kPrefillThreads || tid < VITEMS) {  // head size 64: half the threads stage no V
      // key group v_kq (keys 4 v_kq .. +3) goes to group slot (v_kq & ~3) +
      // 2 (v_kq & 1) + ((v_kq >> 1) & 1) of the row: in every 16-key slice
      // the groups are stored in the order 0, 2, 1, 3, so the 8 keys one
      // half-wave contracts per product (groups hf and hf + 2) are 16
      // contiguous bytes
      const int v_slot = ((v_kq & ~3) + 2 * (v_kq & 1) + ((v_kq >> 1) & 1)) * 8;
      auto put = [&](auto scaled_tag) {
        constexpr bool SCALED = decltype(scaled_tag)::value;
        const float vmul = SCALED ? __builtin_ldexpf(1.f, -vsh) : 1.f;
        float fv[4][8];  // FP8: the 8 columns of each of the 4 keys
        if constexpr (FP8) {
#pragma unroll
          for (int k = 0; k < 4; ++k) fp8x8_to_f32(tr.v[k], fv[k]);
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // columns e, e+1 of keys v_kq*4 .. +3
          float f0[4], f1[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            f0[k] = FP8 ? fv[k][e] : chunk_elem<DT>(tr.v[k], e);
            f1[k] = FP8 ? fv[k][e + 1] : chunk_elem<DT>(tr.v[k], e + 1);
            if constexpr (SCALED) {  // exact power-of-two scaling
              f0[k] *= vmul;
              f1[k] *= vmul;
            }
          }
          const uint2 w0 = make_uint2(pk_f16(f0[0], f0[1]), pk_f16(f0[2], f0[3]));
          const uint2 w1 = make_uint2(pk_f16(f1[0], f1[1]), pk_f16(f1[2], f1[3]));
          *reinterpret_cast<uint2*>(sV + (v_dq * 8 + e) * VROW + v_slot) = w0;
          *reinterpret_cast<uint2*>(sV + (v_dq * 8 + e + 1) * VROW + v_slot) = w1;
        }
      };
      if (kWideCheck && vsh != 0)  // uniform
        put(std::true_type{});
      else
        put(std::false_type{});
      if constexpr (CHECK) {
        // The staged (scaled) values must stay below 2^16 in magnitude
        // (f16's largest finite is 65504; no bf16 value lies in [65504,
        // 65536)), i.e. raw bf16 magnitudes below 2^(16 + vsh).  Magnitudes
        // order as their bf16 bits with the sign cleared (infinities and
        // NaN above every finite value), so packed 16-bit maxima of the raw
        // words find the largest; only past the bound -- or for an infinity
        // or NaN, which pass through as themselves -- are the thread's
        // values looked at one by one for the largest finite one.
        const uint32_t wide_bits = (uint32_t)min(143 + vsh, 255) << 7;  // |v| >= 2^(16 + vsh)
        const uint32_t raw[16] = {tr.v[0].x, tr.v[0].y, tr.v[0].z, tr.v[0].w, tr.v[1].x, tr.v[1].y,
                                  tr.v[1].z, tr.v[1].w, tr.v[2].x, tr.v[2].y, tr.v[2].z, tr.v[2].w,
                                  tr.v[3].x, tr.v[3].y, tr.v[3].z, tr.v[3].w};
        u16x2_t mx = __builtin_bit_cast(u16x2_t, raw[0] & 0x7FFF7FFFu);
#pragma unroll
        for (int q = 1; q < 16; ++q)
          mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, raw[q] & 0x7FFF7FFFu));
        if (max((uint32_t)mx.x, (uint32_t)mx.y) >= wide_bits) {
          uint32_t big = 0;
#pragma unroll
          for (int q = 0; q < 32; ++q) {
            const uint32_t b = (raw[q / 2] >> (16 * (q & 1))) & 0x7FFFu;
            if (b >= wide_bits && b < 0x7F80u) big = max(big, b);
          }
          if (big) atomicMax(&sVwide[ti & 1], (int32_t)big);
        }
      }
    }
  };

  for (int k0 = k_lo; k0 < kend; k0 += kBN, ++ti) {
    // ---- registers -> LDS: K row-major, V transposed to [d][key] in f16
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if constexpr (FP8) {  // 16 codes -> two 16-byte chunks of the query's type
        uint4 lo, hi;
        fp8x16_to_pairs<DT>(tr.k[i], lo, hi);
        store16(sK + k_row * KROW + (k_cg + i) * 32, lo);
        store16(sK + k_row * KROW + (k_cg + i) * 32 + 16, hi);
      } else {
        store16(sK + k_row * KROW + k_chunk(i) * 16, tr.k[i]);
      }
    }
    stage_v(std::integral_constant<bool, kWideCheck>{});
    {
      // the next tile's entries must be in the window; every read of it
      // ended with the previous fetch, which the loop's last barrier orders
      // (the window spans >= 256 keys, so no refill happens before the
      // first tile's fetch has passed a barrier)
      const int kn = k0 + kBN;
      if (kn < kend && (min(kn + kBN - 1, kend - 1) >> lbs) - wb0 >= kBtWinP) {  // uniform
        wb0 = kn >> lbs;
        stage_bt();
      }
    }
    __syncthreads();
    if constexpr (kWideCheck) {
      const int wv = __builtin_amdgcn_readfirstlane(sVwide[ti & 1]);
      if (tid == 0) sVwide[(ti + 1) & 1] = 0;  // its last reader was the previous tile
      if (wv != 0) {  // uniform and rare: a larger shift from this tile on
        // the largest finite |v| seen (2^e <= |v| < 2^(e+1)) lands below 2^15
        const int nv = ((wv >> 7) - 127) - 14;
        const float a = __builtin_ldexpf(1.f, vsh - nv);  // exact rescale of the fp32 sums
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= a;
        vsh = nv;
        if (VITEMS == kPrefillThreads || tid < VITEMS) stage_v(std::false_type{});  // this tile again
        __syncthreads();
      }
    }
    tr = fetch(k0 + kBN);  // next tile in flight (clamped past the end: never a wait on a branch)
    if (wave_rows && k0 <= lim_max) {  // wave-uniform

    // ---- S^T = K Q^T: two blocks of 32 keys; lane holds query lq, keys
    // k0 + 32 kb + 8 (i/4) + 4 hf + i%4
    f32x16_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
    // all K fragments of the tile are requested before the first product
    uint4 ka[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ka[ks][kb] = load16(sK + (kb * 32 + lq) * KROW + ks * 32 + hf * 16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sc[kb] = mfma_qk<DT>(ka[ks][kb], qf[ks], sc[kb]);

    // ---- online softmax in the scaled log2 domain; the two halves of the
    // wave hold the two key sets of each query.  Only tiles that reach past
    // some row's last visible key need the mask.
    if (k0 + kBN - 1 > lim_min) {  // wave-uniform: only such tiles pay for the mask
      // score (kb, i) is key k0 + 4 hf + (32 kb + 8 (i/4) + i%4)
      const int rel = lim - k0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i / 4) + (i % 4) > rel) sc[kb][i] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sc[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * c;  // c > 0: the max commutes with the scale
    if (__any(mt > m + kLazyRescaleP)) {
      const float mn = fmaxf(m, mt);
      const float a = exp2_diff(m, mn);
      m = mn;
      l *= a;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= a;
    }
    // p = 2^(c z - m + 7) (the first key of the range is visible to every
    // query, so m is finite here and masked scores give exp2(-inf) = 0),
    // split into f16 hi = f16(p) and lo = f16(p - hi); the normaliser sums
    // hi + lo
    const float nm = kWeightLog2 - m;
    uint32_t ph[2][8], pl[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i], c, nm));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i + 1], c, nm));
        const uint32_t h2 = pk_f16(e0, e1);
        const f16x2_t hv = __builtin_bit_cast(f16x2_t, h2);
        const uint32_t l2 = pk_f16(sub_f16_lo(e0, h2), sub_f16_hi(e1, h2));
        ph[kb][i / 2] = h2;
        pl[kb][i / 2] = l2;
        l = __builtin_amdgcn_fdot2(hv, __builtin_bit_cast(f16x2_t, ones), l, false);
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, l2), __builtin_bit_cast(f16x2_t, ones),
                                   l, false);
      }

    // ---- O^T += V^T P^T over 4 slices of 16 keys.  Slice t = (kb, jp) uses
    // this lane's registers 8 jp .. 8 jp + 7 of key block kb, i.e. keys
    // 32 kb + 16 jp + 8 (e/4) + 4 hf + e%4 for e = 0..7; the V^T fragment
    // takes its contraction slots in the same order: keys 4 hf .. +3 and
    // 8 + 4 hf .. +3 of the slice, one 16-byte read from the reordered row.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t / 2, jp = t % 2;
      const f16x8_t pbh = __builtin_bit_cast(
          f16x8_t, make_uint4(ph[kb][4 * jp], ph[kb][4 * jp + 1], ph[kb][4 * jp + 2], ph[kb][4 * jp + 3]));
      const f16x8_t pbl = __builtin_bit_cast(
          f16x8_t, make_uint4(pl[kb][4 * jp], pl[kb][4 * jp + 1], pl[kb][4 * jp + 2], pl[kb][4 * jp + 3]));
      const int col = (kb * 32 + jp * 16) * 2 + hf * 16;
      // every block's hi product before the lo products, so no product
      // waits on the one just issued into the same accumulator
      f16x8_t a[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        a[db] = __builtin_bit_cast(f16x8_t, load16(sV + (db * 32 + lq) * VROW + col));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[db], pbh, o[db], 0, 0, 0);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[db], pbl, o[db], 0, 0, 0);
    }
    }  // wave has visible keys in this tile
    __syncthreads();
  }

  // ---- normalise and store: lane holds O[query lq][d = 32 db + 8 g + 4 hf + i]
  const float lt = l + __shfl_xor(l, 32);
  if constexpr (PREFIX) {
    // partial of (row j, head h, key partition s), without the weights'
    // factor 2^7 and with V's 2^vsh
    if (j < n) {
      const int64_t pi = ((int64_t)j * p.max_partitions + s) * p.num_heads + h;  // partition-major
      float* po = p.part_out + pi * D;
      const float vsc = p.v_scale * __builtin_ldexpf(1.f, vsh - (int)kWeightLog2);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store16(po + db * 32 + 8 * g + 4 * hf,
                  make_uint4(__float_as_uint(o[db][4 * g] * vsc), __float_as_uint(o[db][4 * g + 1] * vsc),
                             __float_as_uint(o[db][4 * g + 2] * vsc), __float_as_uint(o[db][4 * g + 3] * vsc)));
      if (hf == 0) {
        p.part_ml[2 * pi] = m;
        p.part_ml[2 * pi + 1] = lt * __builtin_ldexpf(1.f, -(int)kWeightLog2);
      }
    }
    return;
  }
  if (j < n) {
    const float inv = lt > 0.f ? p.v_scale * __builtin_ldexpf(1.f, vsh) / lt : 0.f;
    const int64_t row = ((int64_t)(q_begin + j) * p.num_heads + h) * D;
    // four consecutive columns per group g
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t idx = row + db * 32 + 8 * g + 4 * hf;
        const float v0 = o[db][4 * g] * inv, v1 = o[db][4 * g + 1] * inv;
        const float v2 = o[db][4 * g + 2] * inv, v3 = o[db][4 * g + 3] * inv;
        if (p.out_dtype == PA_F32) {
          store16(reinterpret_cast<float*>(p.out) + idx,
                  make_uint4(__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)));
        } else if (p.out_dtype == PA_BF16) {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + idx) =
              make_uint2(f32_to_bf16(v0) | (uint32_t)f32_to_bf16(v1) << 16,
                         f32_to_bf16(v2) | (uint32_t)f32_to_bf16(v3) << 16);
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + idx) =
              make_uint2(f32_to_f16(v0) | (uint32_t)f32_to_f16(v1) << 16,
                         f32_to_f16(v2) | (uint32_t)f32_to_f16(v3) << 16);
        }
      }
  }
}

template <pa_dtype DT, int D>
hipError_t launch_pd(PrefillParams p, int num_seqs, int max_q, bool off32, bool fp8, hipStream_t st) {
  const bool prefix = p.prefix_keys > 0;
  p.q_tiles = ((prefix ? p.num_rows : max_q) + kBM - 1) / kBM;
  const int64_t pairs = (int64_t)p.num_heads * (prefix ? p.key_parts : num_seqs);
  const int64_t blocks = (pairs + 7) / 8 * 8 * p.q_tiles;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  p.num_work = (int)pairs;
  dim3 grid((unsigned)blocks), block(kPrefillThreads);
  if (prefix && fp8) {
    if (off32)
      hipLaunchKernelGGL((prefill_kernel<DT, D, true, true, true>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((prefill_kernel<DT, D, false, true, true>), grid, block, 0, st, p);
  } else if (prefix) {
    if (off32)
      hipLaunchKernelGGL((prefill_kernel<DT, D, true, true, false>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((prefill_kernel<DT, D, false, true, false>), grid, block, 0, st, p);
  } else if (fp8) {
    if (off32)
      hipLaunchKernelGGL((prefill_kernel<DT, D, true, false, true>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((prefill_kernel<DT, D, false, false, true>), grid, block, 0, st, p);
  } else {
    if (off32)
      hipLaunchKernelGGL((prefill_kernel<DT, D, true, false, false>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((prefill_kernel<DT, D, false, false, false>), grid, block, 0, st, p);
  }
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
  p.scale_log2e = a.scale * a.k_scale * kLog2e;
  p.v_scale = a.v_scale;
  p.out_dtype = a.out_dtype;
  p.num_rows = a.num_tokens;
  p.prefix_keys = a.prefix_keys;
  p.key_part = a.key_part;
  p.key_parts = a.prefix_keys > 0 ? (a.prefix_keys + a.key_part - 1) / a.key_part : 0;
  p.part_out = a.part_out;
  p.part_ml = a.part_ml;
  p.max_partitions = a.max_partitions;
  const bool fp8 = a.kv_dtype == PA_FP8_E4M3;
  const int64_t elem = fp8 ? 1 : 2;
  const bool off32 = (int64_t)g.num_blocks * p.blk_stride * elem <= (int64_t)UINT32_MAX;
  const pa_dtype qt = fp8 ? a.q_dtype : a.kv_dtype;
  if (qt == PA_BF16) {
    if (g.head_size == 64) return launch_pd<PA_BF16, 64>(p, a.num_seqs, a.max_query_len, off32, fp8, stream);
    if (g.head_size == 128) return launch_pd<PA_BF16, 128>(p, a.num_seqs, a.max_query_len, off32, fp8, stream);
  } else if (qt == PA_F16) {
    if (g.head_size == 64) return launch_pd<PA_F16, 64>(p, a.num_seqs, a.max_query_len, off32, fp8, stream);
    if (g.head_size == 128) return launch_pd<PA_F16, 128>(p, a.num_seqs, a.max_query_len, off32, fp8, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
