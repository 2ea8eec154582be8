// ssd_stage.hpp -- global -> LDS staging of chunk tiles for the SSD kernels.
//
// A chunk tile is `rows` consecutive packed tokens (zero past the chunk length
// L) of `COLS` contiguous elements each, rows `ld` elements apart in global
// memory.  Two forms:
//   stage_rows:       LDS[r][c]  (row pitch DP elements), same orientation;
//   stage_transposed: LDS[c][r]  (row pitch DP elements), optionally scaling
//                     row r by scale[r] (fp32) before rounding to the element
//                     type (round-to-nearest-even for bf16).
// Transposition is what lets a matrix-core product contract over tokens: an
// MFMA operand lane needs consecutive K (token) values in its registers.
#pragma once

#include "ssd_device.hpp"

namespace ssd {

template <class E, int ROWS, int COLS, int DP>
__device__ __forceinline__ void stage_rows(typename E::storage* __restrict__ lds,
                                           const typename E::storage* __restrict__ g,
                                           int64_t ld, int L) {
  using T = typename E::storage;
  constexpr int VEC = 16 / sizeof(T);
  static_assert(COLS % VEC == 0, "row length must be a multiple of 16 bytes");
  constexpr int VPR = COLS / VEC;  // vectors per row
  for (int idx = threadIdx.x; idx < ROWS * VPR; idx += kThreads) {
    const int r = idx / VPR, v = idx % VPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < L) val = *reinterpret_cast<const uint4*>(g + r * ld + v * VEC);
    *reinterpret_cast<uint4*>(lds + r * DP + v * VEC) = val;
  }
}

// bf16: 8x8 element blocks (eight 16-byte row loads -> eight 16-byte column stores).
template <int ROWS, int COLS, int DP, bool SCALE>
__device__ __forceinline__ void stage_transposed_bf16(uint16_t* __restrict__ lds,
                                                      const uint16_t* __restrict__ g, int64_t ld,
                                                      int L, const float* __restrict__ scale) {
  static_assert(ROWS % 8 == 0 && COLS % 8 == 0, "8x8 blocks");
  constexpr int CB = COLS / 8;
  for (int blk = threadIdx.x; blk < (ROWS / 8) * CB; blk += kThreads) {
    const int cb = blk % CB, rb = blk / CB;
    uint4 in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rb * 8 + i;
      in[i] = make_uint4(0, 0, 0, 0);
      if (r < L) in[i] = *reinterpret_cast<const uint4*>(g + r * ld + cb * 8);
    }
    float sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[i] = SCALE ? scale[rb * 8 + i] : 1.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = (c >> 1) == 0 ? in[i].x : (c >> 1) == 1 ? in[i].y : (c >> 1) == 2 ? in[i].z : in[i].w;
        const float f = (c & 1) ? bf16_hi(w) : bf16_lo(w);
        v[i] = SCALE ? f * sc[i] : f;
      }
      uint4 out;
      out.x = pack_bf16x2(v[0], v[1]);
      out.y = pack_bf16x2(v[2], v[3]);
      out.z = pack_bf16x2(v[4], v[5]);
      out.w = pack_bf16x2(v[6], v[7]);
      *reinterpret_cast<uint4*>(lds + (cb * 8 + c) * DP + rb * 8) = out;
    }
  }
}

// fp32: 4x4 element blocks.
template <int ROWS, int COLS, int DP, bool SCALE>
__device__ __forceinline__ void stage_transposed_f32(float* __restrict__ lds,
                                                     const float* __restrict__ g, int64_t ld,
                                                     int L, const float* __restrict__ scale) {
  static_assert(ROWS % 4 == 0 && COLS % 4 == 0, "4x4 blocks");
  constexpr int CB = COLS / 4;
  for (int blk = threadIdx.x; blk < (ROWS / 4) * CB; blk += kThreads) {
    const int cb = blk % CB, rb = blk / CB;
    float4 in[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 4 + i;
      in[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < L) {
        in[i] = *reinterpret_cast<const float4*>(g + r * ld + cb * 4);
        if (SCALE) {
          const float s = scale[r];
          in[i].x *= s; in[i].y *= s; in[i].z *= s; in[i].w *= s;
        }
      }
    }
    *reinterpret_cast<float4*>(lds + (cb * 4 + 0) * DP + rb * 4) = make_float4(in[0].x, in[1].x, in[2].x, in[3].x);
    *reinterpret_cast<float4*>(lds + (cb * 4 + 1) * DP + rb * 4) = make_float4(in[0].y, in[1].y, in[2].y, in[3].y);
    *reinterpret_cast<float4*>(lds + (cb * 4 + 2) * DP + rb * 4) = make_float4(in[0].z, in[1].z, in[2].z, in[3].z);
    *reinterpret_cast<float4*>(lds + (cb * 4 + 3) * DP + rb * 4) = make_float4(in[0].w, in[1].w, in[2].w, in[3].w);
  }
}

template <class E, int ROWS, int COLS, int DP, bool SCALE>
__device__ __forceinline__ void stage_transposed(typename E::storage* __restrict__ lds,
                                                 const typename E::storage* __restrict__ g,
                                                 int64_t ld, int L, const float* __restrict__ scale) {
  if constexpr (E::kBytes == 2)
    stage_transposed_bf16<ROWS, COLS, DP, SCALE>(lds, g, ld, L, scale);
  else
    stage_transposed_f32<ROWS, COLS, DP, SCALE>(lds, g, ld, L, scale);
}

}  // namespace ssd
