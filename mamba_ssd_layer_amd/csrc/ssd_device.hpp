// ssd_device.hpp -- device-side building blocks shared by the SSD kernels for
// gfx950 (CDNA4): element types, MFMA wrappers, bf16 packing, wave scans and
// the XCD-aware block remap.  No SSD arithmetic lives here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssd_internal.hpp"

namespace ssd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, blocks dispatched round-robin
constexpr float kLog2e = 1.4426950408889634f;

// Element storage type of x, B, C, y: raw bf16 bits or fp32.
struct Bf16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kMfmaK = 16;  // v_mfma_f32_32x32x16_bf16: 8 values per lane
};
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
  static constexpr int kMfmaK = 2;  // v_mfma_f32_32x32x2_f32: 1 value per lane
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = __builtin_convertvector((floatx2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ floatx16_t mfma32x32x16(const uint4& a, const uint4& b, floatx16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx16_t mfma32x32x2(float a, float b, floatx16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16_t zero16() {
  floatx16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Map the hardware block id to a logical id so that each XCD (which receives
// blocks bid % 8) owns one contiguous range of logical ids.  Consecutive
// logical ids then share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / kNumXcd;
  const int r = nblocks % kNumXcd;
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  return xcd * q + (xcd < r ? xcd : r) + slot;
}

// Inclusive prefix sum of one float per lane across a 64-lane wave.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    float o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}


}  // namespace ssd
