// Device helpers shared by the attention kernels: element formats, lane
// reductions and float <-> storage conversions.  gfx950 (wave64) only.
#ifndef PA_KERNEL_COMMON_H_
#define PA_KERNEL_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed once: K/V rows in decode).
__device__ __forceinline__ uint4 load_nt(const void* ptr) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Plain 16-byte load / LDS store through a vector type (a HIP_vector_type
// copy lowers to memcpy and can pin whole arrays in scratch).
__device__ __forceinline__ uint4 load16(const void* ptr) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ptr);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16(void* ptr, const uint4& v) {
  *reinterpret_cast<u32x4_t*>(ptr) = u32x4_t{v.x, v.y, v.z, v.w};
}

// Elements per 16-byte chunk.
template <pa_dtype DT>
struct Fmt {
  static constexpr int kBytes = DT == PA_F32 ? 4 : 2;
  static constexpr int kVec = 16 / kBytes;
};

// acc + dot(q, k) over one 16-byte chunk (fp32 accumulation; bf16/f16
// products are exact in fp32).
template <pa_dtype DT>
__device__ __forceinline__ float dot_chunk(const uint4& q, const uint4& k, float acc) {
  if constexpr (DT == PA_F32) {
    acc = __builtin_fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  } else if constexpr (DT == PA_BF16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x),
                                          __builtin_bit_cast(bf16x2_t, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y),
                                          __builtin_bit_cast(bf16x2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z),
                                          __builtin_bit_cast(bf16x2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w),
                                          __builtin_bit_cast(bf16x2_t, k.w), acc, false);
  } else {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.x), __builtin_bit_cast(f16x2_t, k.x),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.y), __builtin_bit_cast(f16x2_t, k.y),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.z), __builtin_bit_cast(f16x2_t, k.z),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.w), __builtin_bit_cast(f16x2_t, k.w),
                                 acc, false);
  }
  return acc;
}

// Element e of one 16-byte chunk as float (exact).
template <pa_dtype DT>
__device__ __forceinline__ float chunk_elem(const uint4& v, int e) {
  constexpr int kPerWord = 4 / Fmt<DT>::kBytes;
  const int wi = e / kPerWord;
  const uint32_t w = wi == 0 ? v.x : wi == 1 ? v.y : wi == 2 ? v.z : v.w;
  if constexpr (DT == PA_F32) {
    return __uint_as_float(w);
  } else if constexpr (DT == PA_BF16) {
    return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  } else {
    const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu)));
    return (float)h;
  }
}

// Unpack a chunk to kVec floats.
template <pa_dtype DT>
__device__ __forceinline__ void chunk_to_f32(const uint4& v, float* out) {
#pragma unroll
  for (int e = 0; e < Fmt<DT>::kVec; ++e) out[e] = chunk_elem<DT>(v, e);
}

// ---- FP8 (OCP E4M3) cache elements.  gfx950's conversion instructions read
// and write the OCP E4M3 format; reading is exact (every E4M3 value is a
// bf16, f16 and fp32 value), writing rounds to nearest even but does not
// saturate (magnitudes past 464 become NaN), so writers clamp first.
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Codes in bytes 0-1 (HI = false) or 2-3 (HI = true) of w as a packed pair of
// DT (bf16 or f16), element order kept; the scale operand 1.0 leaves the
// values unscaled.
template <pa_dtype DT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_pair(uint32_t w) {
  if constexpr (DT == PA_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// 16 codes (one 16-byte chunk) as 16 elements of DT in two 16-byte chunks.
template <pa_dtype DT>
__device__ __forceinline__ void fp8x16_to_pairs(const uint4& v, uint4& lo, uint4& hi) {
  lo = make_uint4(fp8x2_to_pair<DT, false>(v.x), fp8x2_to_pair<DT, true>(v.x),
                  fp8x2_to_pair<DT, false>(v.y), fp8x2_to_pair<DT, true>(v.y));
  hi = make_uint4(fp8x2_to_pair<DT, false>(v.z), fp8x2_to_pair<DT, true>(v.z),
                  fp8x2_to_pair<DT, false>(v.w), fp8x2_to_pair<DT, true>(v.w));
}

// 16 codes as floats.
__device__ __forceinline__ void fp8x16_to_f32(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);
    out[4 * j] = a.x;
    out[4 * j + 1] = a.y;
    out[4 * j + 2] = b.x;
    out[4 * j + 3] = b.y;
  }
}

// Clamp to the largest finite E4M3 magnitude (NaN passes through).
__device__ __forceinline__ float e4m3_saturate(float y) {
  return y != y ? y : fminf(fmaxf(y, -448.f), 448.f);
}

// Four floats (already in range) as four E4M3 codes, byte i = code of the
// i-th argument.
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 1..64, power of two); every lane of
// the group receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// 2^(a - b) where a = -inf (an empty running state) gives 0 even if b = -inf.
__device__ __forceinline__ float exp2_diff(float a, float b) {
  return a == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(a - b);
}

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Store one float as the output type (PA_F32, PA_BF16 or PA_F16).
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, pa_dtype t) {
  if (t == PA_F32)
    reinterpret_cast<float*>(out)[idx] = v;
  else if (t == PA_BF16)
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  else
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16(v);
}

}  // namespace pa

#endif  // PA_KERNEL_COMMON_H_
