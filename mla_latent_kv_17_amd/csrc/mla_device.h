// Device-side helpers shared by the MLA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Round two floats to bf16 (nearest-even, hardware v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// One output element of the projections: fp32, or rounded to bf16.
__device__ __forceinline__ void store_out(void* out, int64_t i, float v, int bf16) {
  if (bf16)
    ((uint16_t*)out)[i] = f32_to_bf16_bits(v);
  else
    ((float*)out)[i] = v;
}

// Two OCP E4M3FN codes (bytes 0,1 or bytes 2,3 of `w`) -> two bf16; exact
// (a 3-bit mantissa and the E4M3 exponent range fit bf16).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi);
  return __builtin_bit_cast(uint32_t, v);
}

// Four consecutive chunk-partial values as fp32 (fp32 or fp16 storage; the
// pointer is 16- or 8-byte aligned).
__device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load4(const _Float16* p) {
  const f16x4 h = *(const f16x4*)p;
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
// Four fp32 values rounded to nearest-even binary16.
__device__ __forceinline__ f16x4 to_f16x4(f32x4 v) {
  return f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing LDS read: within each 16-lane group, lane i receives element (i % 4)
// of the 8-byte chunk read by lane 4*j + i/4, for j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16_b64(const MLA_LDS void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Lane moves within rows of 16 lanes (every lane has a source in these
// patterns): swap neighbours, swap pairs, mirror within 8, mirror within 16.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp<kCtrl>(__float_as_int(v)));
}

// Every lane of a row of 16 lanes receives the row's maximum / sum (fixed
// order).
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v + dpp<kDppMirror>(v);
}

// The same over the whole wave: the four rows' results combined from lanes
// 0, 16, 32 and 48 (returned to every lane).
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max_rows(float v) {
  v = row_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_rows(float v) {
  v = row_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
}  // namespace mla
