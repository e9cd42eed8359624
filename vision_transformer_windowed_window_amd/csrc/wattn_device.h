// wattn_device.h -- device helpers shared by the attention kernels of libwattn.so (gfx950):
// vector types, bf16/fp16 packing, the 16x16x32 MFMA wrappers, lane-pair reductions, the
// transposed LDS read and the LDS chunk swizzles of 64-byte token rows.
//
// Each kernel source includes it inside its anonymous namespace, after <hip/hip_runtime.h>
// and <stdint.h>.

#pragma once

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 32;          // head dimension of q, k, v
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f32x2 f = {a, b};
  f16x2 h = __builtin_convertvector(f, f16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// The MFMA wrappers below are all the 16x16x32 shape.  Products are chained through srcC (an
// accumulator fed back as the next product's srcC); such chains must keep one shape: the
// compiler inserts no wait states between MFMAs of different shapes whose srcC is exactly
// the previous destination, which the hardware only forwards between identical instructions.

// score product: fp16 operands (k = 32 channels in one instruction), fp32 accumulate
__device__ __forceinline__ f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// value product: bf16 operands (k = 32 keys), fp32 accumulate
__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// Sum / max over the lane pairs (l, l ^ 16) and (l, l ^ 32): the gfx950 swap instructions hand
// every lane the pair {x[l], x[l ^ 16]} (or ^ 32) without a trip through LDS.
__device__ __forceinline__ float xsum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xmax16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposed 8-byte LDS read (gfx950): in each group of 16 lanes, lane j receives element
// j % 4 of the 8-byte reads issued by lanes j/4, j/4 + 4, j/4 + 8 and j/4 + 12.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) void*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// LDS swizzles.  K and V tiles are row-major (64 bytes per key); the 16-byte chunk index
// of a row is XORed with a few bits of the key so that the lanes served in one LDS cycle
// hit distinct banks.  K: the eight keys 8j + 4b + {0..3} (j = 0, 1) read by one group of
// eight lanes.  V: a transposed 8-byte read serves 32 lanes per cycle, lane groups g = 0
// and g = 1 reading keys 8 apart that would otherwise share 32 of the 64 banks; flipping
// bit 1 of the chunk index with bit 3 of the key sends them to the other half.  Bias
// factor tile (32 bytes per key): the 16-byte half index is XORed with bit 3 of the key.
__device__ __forceinline__ int kswz(int key) { return ((key >> 1) & 1) | (((key >> 3) & 1) << 1); }
__device__ __forceinline__ int vswz(int key) { return ((key >> 3) & 1) << 1; }
__device__ __forceinline__ int bswz(int key) { return (key >> 3) & 1; }
