// Paged decode, grouped kernel on matrix cores (group size 4, 8 or 16;
// bf16 or f16 caches, and FP8 (E4M3) caches with bf16 or f16 queries).
//
// One workgroup of 4 waves per (sequence, kv head, partition), as in the
// per-head kernel (contract and sources in decode.hip).  The partition is
// walked in rounds of 64 tokens; wave w takes tokens 16 w .. 16 w + 15 of
// each round and keeps its own softmax state, so the waves never wait for
// one another until the final merge.  Per 16-token tile:
//   loads    each 16-byte load instruction covers whole cache rows (4 rows
//            of 256 bytes for 16-bit caches at head size 128, 8 of 128
//            bytes for FP8), non-temporally; K rows go to the wave's LDS
//            region as they are, V rows as 16-bit values (FP8 codes as f16,
//            exact for every E4M3 value).  (FP8 lanes loading the quarters
//            their MFMA operands need read half of each 128-byte line per
//            instruction; that measured 3-10% slower, and another 10-15%
//            slower with non-temporal loads, whose lines are gone before
//            the other half is read.)
//   QK       S[16 tokens x 16 heads] = K Q^T on v_mfma_f32_16x16x32 (bf16 or
//            f16 by the query's type).  The A operand is read back from LDS
//            (lane = token l % 16 and quarter l / 16 of the row; FP8 codes
//            convert exactly to the query's type); the B operand is the
//            group's query vectors, held in registers for the whole
//            partition (heads past G are zero).
//   softmax  a lane holds 4 tokens of head l % 16.  The running maximum
//            moves only when some score exceeds it by more than 2^8.
//   PV       O^T[16 d x 16 heads] += V^T P^T on v_mfma_f32_16x16x16, one
//            product per 16 columns and weight term.  The B operand is the
//            lane's own four probabilities: the QK product left tokens
//            4 q4 .. +3 of head l % 16 in exactly the B layout, so P never
//            leaves the registers.  The A operand (16 columns x 16 tokens)
//            is read transposed from the tile's V rows in LDS; a lane then
//            holds O[head l % 16][16 b + 4 q4 .. +3] for every block b.
// Precision: each weight enters PV as terms exact in V's type -- two f16
// terms, hi = f16(p) and lo = f16(p - hi) (about 22 significant bits), for
// f16 and FP8 caches; three bf16 terms (about 24 bits, fp32's precision)
// for bf16 caches, whose V then enters the products exactly at any
// magnitude, infinities and NaN included -- and the normaliser sums the
// same terms.  QK products are exact with fp32 sums.
// Each wave keeps two tiles of K/V in flight (the next two rounds) and reads
// the block ids it needs from the table two rounds ahead of the rows they
// locate; the tiles past the end of the partition are loaded too (clamped
// to its last row, which is cached) so that no load sits on a branch: a
// conditional refill made the compiler copy the just-loaded registers at
// the loop's end, waiting for the loads it meant to keep in flight.  The
// waves' (max, sum, output) states are merged at the end by the log-sum-exp
// rule.  Heads past G are zero in the query operand, so their scores,
// probabilities and outputs are never used.
//
// For 16-bit caches this replaced a kernel doing QK on v_dot2 and PV with
// fp32 weights on fp32 FMAs, which was bound by its vector ALU (70% busy):
// 762 -> 737 us on the long-context batch, 158 -> 151 us on the 70B-like
// one, and at group size 16 228 -> 161 us.
#include <hip/hip_runtime.h>

#include "decode_common.h"

namespace pa {
namespace dec {
namespace {

constexpr int kTile = 16;                     // tokens per wave per round
constexpr int kRound = kTile * kDecodeWaves;  // tokens per workgroup per round

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __fp16 lds_f16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// gfx950 transposing LDS read: in each group of 16 lanes, lane 4 r + c
// addresses 4 consecutive 16-bit values of row r (columns 4 c .. 4 c + 3)
// of a 4 x 16 block, and lane l receives column l of the block (rows 0..3).
__device__ __forceinline__ f16x4_t lds_read_tr16(const _Float16* p) {
  return __builtin_bit_cast(
      f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) lds_f16x4_t*)(p)));
}

template <pa_dtype DT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  if constexpr (DT == PA_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// LDS written by some lanes of a wave and then read by others: keeps the
// compiler from moving the accesses across (a wave's LDS operations run in
// order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Waves per SIMD the register budget is set for (3 = at most 168 VGPRs).
// Group size 16 at head size 128 needs more and settles for 2, and so do
// 16-bit caches at head size 128, whose loads in flight take twice the
// registers: bf16 compiles to 170 registers there (168 under a 3-wave bound,
// which measured 1% slower on the long-context batch and 0.3% faster on the
// 70B-like one); f16 to 161, so it runs 3 waves all the same (its 3-wave
// bound spilled).
template <int G, int D, bool FP8>
constexpr int kMfmaMinWaves = (D >= 128 && (G >= 16 || !FP8)) ? 2 : 3;

// PV on matrix cores, O^T[16 d x 16 heads] += V^T P^T over 16 tokens: a =
// the lane's V^T operand (16-bit rows: f16, or bf16 bits), w = the lane's
// four weights (p = the sum of the terms, each exact in the operand type).
template <bool BF16V>
struct PvWeights;
template <>
struct PvWeights<false> {  // f16 V: p = hi + lo, two f16 terms (~22 bits)
  f16x4_t hi, lo;
  __device__ __forceinline__ float set(int r, float w) {
    hi[r] = (_Float16)w;
    lo[r] = (_Float16)(w - (float)hi[r]);
    return (float)hi[r] + (float)lo[r];
  }
  __device__ __forceinline__ void first(const f16x4_t& a, f32x4_t& o) const {
    o = __builtin_amdgcn_mfma_f32_16x16x16f16(a, hi, o, 0, 0, 0);
  }
  __device__ __forceinline__ void rest(const f16x4_t& a, f32x4_t& o) const {
    o = __builtin_amdgcn_mfma_f32_16x16x16f16(a, lo, o, 0, 0, 0);
  }
};
template <>
struct PvWeights<true> {  // bf16 V: p = t0 + t1 + t2, three bf16 terms (~24 bits)
  __bf16 t[3][4];
  __device__ __forceinline__ float set(int r, float w) {
    t[0][r] = (__bf16)w;
    const float r1 = w - (float)t[0][r];  // exact
    t[1][r] = (__bf16)r1;
    t[2][r] = (__bf16)(r1 - (float)t[1][r]);
    return (float)t[0][r] + (float)t[1][r] + (float)t[2][r];
  }
  __device__ __forceinline__ i16x4_t term(int k) const {
    return i16x4_t{__builtin_bit_cast(short, t[k][0]), __builtin_bit_cast(short, t[k][1]),
                   __builtin_bit_cast(short, t[k][2]), __builtin_bit_cast(short, t[k][3])};
  }
  __device__ __forceinline__ void first(const f16x4_t& a, f32x4_t& o) const {
    o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), term(0), o, 0, 0, 0);
  }
  __device__ __forceinline__ void rest(const f16x4_t& a, f32x4_t& o) const {
    o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), term(1), o, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), term(2), o, 0, 0, 0);
  }
};

// DT = the query's type (and the cache's, unless FP8).
template <pa_dtype DT, int D, int G, bool OFF32, bool FP8>
__global__ __launch_bounds__(kDecodeThreads, (kMfmaMinWaves<G, D, FP8>)) void decode_mfma_kernel(
    const DecodeParams p) {
  static_assert(DT == PA_BF16 || DT == PA_F16, "queries are bf16 or f16");
  static_assert(G == 4 || G == 8 || G == 16, "group size 4, 8 or 16");
  constexpr int CB = FP8 ? 1 : 2;       // cache bytes per element
  constexpr bool kBf16V = !FP8 && DT == PA_BF16;  // V rows in LDS are bf16 (else f16)
  constexpr int KB = D / 32;            // MFMA k-blocks of 32 elements
  constexpr int PPR = D * CB / 16;      // 16-byte pieces per cache row
  constexpr int RPI = kWave / PPR;      // rows one load instruction covers (whole rows)
  constexpr int NLD = kTile / RPI;      // load instructions per tensor per tile
  constexpr int KSTR = PPR + 1;         // padded LDS row stride of the raw K rows, in pieces
  constexpr int RC = D / 8;             // 16-byte LDS pieces per 16-bit V row
  constexpr int VSTR = RC + 1;          // padded LDS row stride in pieces
  constexpr int DB = D / 16;            // PV: 16-column blocks of O^T
  constexpr int kWaveK = kTile * KSTR;                 // pieces of one wave's K region
  constexpr int kWaveV = kTile * VSTR;                 // pieces of one wave's V region
  constexpr int kLdsMain = (kDecodeWaves * (kWaveK + kWaveV)) * 16;
  constexpr int kLdsMerge = kDecodeWaves * G * D * 4;
  constexpr int kLds = kLdsMain > kLdsMerge ? kLdsMain : kLdsMerge;
  __shared__ __align__(16) char smem[kLds];
  __shared__ float sM[kDecodeWaves][G], sL[kDecodeWaves][G];

  int s, kvh, item, L;
  if (p.inline_items) {
    if (!decode_item_inline(p, s, kvh, item, L)) return;
  } else {
    if (!decode_item(p, true, s, kvh, item)) return;
    L = p.context_lens[s];
  }
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  // Tokens [t0, t1): one partition (split-K) or the whole context (single
  // pass).
  const int P = p.partition_size;
  const int part = item;
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

  const int tl = lane % kTile;  // QK: token of the tile, and head of the B operand / scores
  const int q4 = lane / kTile;  // quarter of the K row this lane reads back (its MFMA k-slots)

  // Element d held in slot e of MFMA k-block j by lanes of quarter q4: a
  // lane reads pieces q4, q4 + 4, ... of its K row from LDS -- FP8: 16
  // elements each, piece i feeding blocks 2 i and 2 i + 1; 16-bit: 8
  // elements, piece i = block i.  The query operand uses the same map.
  auto dmap = [&](int j) -> int {
    return FP8 ? 16 * (q4 + 4 * (j >> 1)) + 8 * (j & 1) : 8 * (q4 + 4 * j);
  };

  // B operand: the query vector of head tl (zero past the group).
  uint4 qb[KB];
  {
    const char* qrow = (const char*)p.query +
                       (((int64_t)s * p.num_heads + (int64_t)kvh * G + min(tl, G - 1)) * D) * 2;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint4 v = load16(qrow + dmap(j) * 2);
      qb[j] = tl < G ? v : make_uint4(0, 0, 0, 0);
    }
  }

  const uint32_t blk_b = (uint32_t)(p.blk_stride * CB);
  const uint32_t tok_b = (uint32_t)(p.tok_stride * CB);
  const int64_t head_off = (int64_t)kvh * p.head_stride * CB;  // bytes
  // Loads cover whole rows: in load instruction i the lane reads piece lp of
  // row RPI i + lr of the tile (every 128-byte line is read by one
  // instruction, non-temporally; half-line reads measured slower).  Rows
  // reach LDS as they are, and the MFMA lanes read back their quarters.
  const int lr = lane / PPR, lp = lane % PPR;

  uint4* sK = reinterpret_cast<uint4*>(smem) + wave * (kWaveK + kWaveV);  // K rows as stored
  uint4* sV = sK + kWaveK;                                 // V rows, 16-bit (FP8: as f16)
  // PV A operand: V^T[d = 16 b + tl][token 4 q4 + j], j = 0..3, from the
  // wave's 16-bit V rows (row stride VSTR pieces) by one transposing read per
  // block: lane tl of quarter q4 addresses row 4 q4 + tl / 4, columns
  // 16 b + 4 (tl % 4) .. +3
  const _Float16* vh =
      reinterpret_cast<const _Float16*>(sV) + (4 * q4 + tl / 4) * (VSTR * 8) + 4 * (tl % 4);

  // block id of token ts + tl (lane tl of every quarter holds it)
  auto block_of = [&](int ts) -> int32_t { return bt[min(ts + tl, t1 - 1) >> lbs]; };
  // K and V pieces of tile ts (rows past the end are clamped to the last
  // row: valid, finite, masked where used); blk = block_of(ts), whose value
  // for row r sits in lane r
  auto fetch = [&](int ts, int32_t blk, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = RPI * i + lr;
      const int32_t b = __shfl(blk, r);
      const int t = min(ts + r, t1 - 1);
      if constexpr (OFF32) {
        const uint32_t off =
            (uint32_t)b * blk_b + (uint32_t)(t & bs_mask) * tok_b + (uint32_t)head_off + 16 * lp;
        kr[i] = load_nt(p.key_cache + off);
        vr[i] = load_nt(p.value_cache + off);
      } else {
        const int64_t off = ((int64_t)b * p.blk_stride + (int64_t)(t & bs_mask) * p.tok_stride) * CB +
                            head_off + 16 * lp;
        kr[i] = load_nt(p.key_cache + off);
        vr[i] = load_nt(p.value_cache + off);
      }
    }
  };

  float m_ref, l_lane;  // softmax state of head tl (this wave's tokens of the partition)
  // O^T blocks: lane holds O[head tl][d = 16 b + 4 q4 + j]
  f32x4_t o[DB];
  auto reset = [&]() {
    m_ref = -INFINITY;
    l_lane = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  reset();

  // Consumes tile ts from (kr, vr), then refills them with the tile two
  // rounds ahead (its block ids were read two rounds ago).
  auto tile = [&](int ts, uint4 (&kr)[NLD], uint4 (&vr)[NLD], int32_t& blk_ahead) {
    // ---- K rows into LDS as they are, V rows as 16-bit (FP8: f16)
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = RPI * i + lr;
      sK[r * KSTR + lp] = kr[i];
      if constexpr (FP8) {
        uint4 v0, v1;
        fp8x16_to_pairs<PA_F16>(vr[i], v0, v1);
        sV[r * VSTR + 2 * lp] = v0;
        sV[r * VSTR + 2 * lp + 1] = v1;
      } else {
        sV[r * VSTR + lp] = vr[i];
      }
    }
    fetch(ts + 2 * kRound, blk_ahead, kr, vr);
    blk_ahead = block_of(ts + 4 * kRound);
    wave_lds_sync();  // the tile's K and V rows are visible to the whole wave

    // ---- K as MFMA A operands: pieces q4, q4 + 4, ... of row tl (FP8:
    // exact E4M3 -> query type)
    uint4 ka[KB];
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < KB / 2; ++i) fp8x16_to_pairs<DT>(sK[tl * KSTR + q4 + 4 * i], ka[2 * i], ka[2 * i + 1]);
    } else {
#pragma unroll
      for (int j = 0; j < KB; ++j) ka[j] = sK[tl * KSTR + q4 + 4 * j];
    }

    // ---- QK on matrix cores: the lane holds tokens 4 q4 + r of head tl
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KB; ++j) sc = mfma_16x16x32<DT>(ka[j], qb[j], sc);

    float z[4];
    bool need = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = tl < G && ts + 4 * q4 + r < t1;
      z[r] = valid ? sc[r] * p.scale_log2e : -INFINITY;
      need |= z[r] > m_ref + kLazyRescale;
    }
    if (__any(need)) {  // move the running maximum of every head to the tile's
      float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m_ref, mt);
      const float alpha = exp2_diff(m_ref, mn);
      m_ref = mn;
      l_lane *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;  // the lane's own head
    }
    // weights split into terms exact in V's type; the normaliser sums the
    // terms, so the weights that multiply V are the ones divided out
    PvWeights<kBf16V> pw;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      l_lane += pw.set(r, z[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[r] - m_ref));

    // ---- PV on matrix cores: O^T[16 d x 16 heads] += V^T[16 d x 16 tokens]
    // P^T[16 tokens x 16 heads] per block of 16 columns
    // (v_mfma_f32_16x16x16, f16 or bf16 by V's type).  The B operand is this
    // lane's own four probabilities (tokens 4 q4 .. +3 of head tl, where the
    // QK product put them; zero past the group and the context).  Every
    // block's first product comes before the other terms' products: no
    // product waits on the one just issued into the same accumulator.
    f16x4_t a[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      a[b] = lds_read_tr16(vh + 16 * b);
      pw.first(a[b], o[b]);
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) pw.rest(a[b], o[b]);
    wave_lds_sync();  // this tile's K and V are consumed before the next tile's stores
  };

  // Merge of the waves' states (log-sum-exp rule) -- written as the
  // partition's partial, or as the final rows of a single-partition context.
  // The LDS V rows hold the waves' accumulators meanwhile.
  auto flush = [&]() {
    // this wave's statistics of head tl (summed over the four quarters)
    l_lane += __shfl_xor(l_lane, 16);
    l_lane += __shfl_xor(l_lane, 32);
    if (lane < G) {
      sM[wave][lane] = m_ref;
      sL[wave][lane] = l_lane;
    }
    __syncthreads();  // every wave's tiles of the partition are done: the LDS rows are free
    float* sAcc = reinterpret_cast<float*>(smem);  // [waves][G][D]
    if (tl < G) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
        store16(sAcc + (wave * G + tl) * D + 16 * b + 4 * q4,
                make_uint4(__float_as_uint(o[b][0]), __float_as_uint(o[b][1]), __float_as_uint(o[b][2]),
                           __float_as_uint(o[b][3])));
    }
    __syncthreads();
#pragma unroll 1
    for (int i = tid; i < G * D; i += kDecodeThreads) {
      const int h = i / D, d = i % D;
      float M = sM[0][h];
#pragma unroll
      for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sM[w][h]);
      float lsum = 0.f, ov = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float a = exp2_diff(sM[w][h], M);
        lsum += a * sL[w][h];
        ov += a * sAcc[(w * G + h) * D + d];
      }
      emit(p, s, kvh * G + h, part, d, D, M, lsum, ov, single);
    }
  };

  // Two tile buffers alternate, so two tiles per wave are always in flight.
  // The block ids come first and the two tiles' loads in order (the
  // scheduling barrier keeps them apart), so the first tile can be consumed
  // while the second is still loading.
  const int ts0 = t0 + kTile * wave;
  uint4 ka_[NLD], va_[NLD], kb_[NLD], vb_[NLD];
  const int32_t bid0 = block_of(ts0), bid1 = block_of(ts0 + kRound);
  int32_t bid_a = block_of(ts0 + 2 * kRound), bid_b = block_of(ts0 + 3 * kRound);
  fetch(ts0, bid0, ka_, va_);
  __builtin_amdgcn_sched_barrier(0);
  fetch(ts0 + kRound, bid1, kb_, vb_);
  for (int ts = ts0; ts - kTile * wave < t1; ts += 2 * kRound) {
    tile(ts, ka_, va_, bid_a);
    tile(ts + kRound, kb_, vb_, bid_b);
  }
  flush();
}

template <pa_dtype DT, int D, bool OFF32, bool FP8>
hipError_t launch_g(const DecodeParams& p, int G, dim3 grid, hipStream_t st) {
  dim3 block(kDecodeThreads);
  switch (G) {
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<DT, D, 4, OFF32, FP8>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<DT, D, 8, OFF32, FP8>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<DT, D, 16, OFF32, FP8>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <pa_dtype DT, bool FP8>
hipError_t launch_d(const DecodeParams& p, int D, int G, dim3 grid, hipStream_t st) {
  if (D == 64)
    return p.off32 ? launch_g<DT, 64, true, FP8>(p, G, grid, st) : launch_g<DT, 64, false, FP8>(p, G, grid, st);
  if (D == 128)
    return p.off32 ? launch_g<DT, 128, true, FP8>(p, G, grid, st) : launch_g<DT, 128, false, FP8>(p, G, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_group_fp8(const DecodeParams& p, pa_dtype qt, int D, int G, dim3 grid, hipStream_t st) {
  switch (qt) {
    case PA_BF16: return launch_d<PA_BF16, true>(p, D, G, grid, st);
    case PA_F16: return launch_d<PA_F16, true>(p, D, G, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_group_mfma(const DecodeParams& p, pa_dtype dt, int D, int G, dim3 grid, hipStream_t st) {
  switch (dt) {
    case PA_BF16: return launch_d<PA_BF16, false>(p, D, G, grid, st);
    case PA_F16: return launch_d<PA_F16, false>(p, D, G, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
}  // namespace pa
