// qsa_device.h — device-side helpers shared by the QSA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kHeadDim = 256;
constexpr int kPage = 64;
constexpr int kRatio = 4;
constexpr int kGroupsPerPage = kPage / kRatio;  // 16
constexpr int kIdxHeads = 8;
constexpr int kIdxDim = 64;
constexpr int kGroupFloats = kIdxHeads * kIdxDim;  // 512 fp32 per k̂ group
constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;

// Order-preserving map of a binary32 value to an unsigned key: a > b as
// floats  <=>  key(a) > key(b) as integers, with -0 mapped like +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (s == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Round a binary32 to bfloat16, nearest-even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_round(float x) {
  return __uint_as_float(bf16_rne_bits(x) << 16);
}

// Two OCP E4M3FN bytes -> two bfloat16 packed in one dword (low half =
// lower byte).  Every E4M3FN value is exactly representable in bfloat16,
// so the conversion is exact.  gfx950's scaled conversion is used with
// scale 1; `hi` picks bytes 2-3 instead of bytes 0-1 of `w`.
template <bool hi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, hi);
  return __builtin_bit_cast(uint32_t, r);
}

// Streaming 16-byte load: data read once per launch is fetched non-temporally
// so it does not displace reused lines (measured ~12% more HBM read
// bandwidth than plain loads on MI355X for multi-GiB streams).
typedef float qsa_f4v __attribute__((ext_vector_type(4)));
typedef unsigned int qsa_u4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 stream_load(const float4* p) {
  const qsa_f4v v = __builtin_nontemporal_load(reinterpret_cast<const qsa_f4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ qsa_u4v stream_load_u4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const qsa_u4v*>(p));
}

// Wave-wide helpers ---------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), result in every
// lane of the row: two quad butterflies, then half-row and row mirrors.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

}  // namespace qsa
