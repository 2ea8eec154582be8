// ssd_stage.hpp -- global -> register -> LDS staging of chunk tiles.
//
// A chunk tile is ROWS consecutive packed tokens (zero past the chunk length
// L, L >= 1) of COLS contiguous elements, rows `ld` elements apart in global
// memory.  Every load is issued unconditionally (row index clamped to L-1; the
// rows past L become zeros when the tile is stored, not in the load registers,
// which would force a wait for the loads), so the loads of a tile stay one
// uninterrupted run and later waits can count them exactly.
// Staging is split into load() (every global load of the thread issued back to
// back into registers, so their latencies overlap) and store() (registers ->
// LDS), so that a kernel can issue the loads of its next tile before computing
// on the current one.
//   RowTile:   LDS[r][c]  with row pitch DP elements;
//   TransTile: LDS[c][r]  with row pitch DP elements (tokens contiguous, the
//              layout an MFMA operand needs to contract over tokens), with an
//              optional per-row fp32 scale applied before rounding back to the
//              element type (round-to-nearest-even for bf16).
#pragma once

#include "ssd_device.hpp"

namespace ssd {

// Row permutation of an LDS tile whose rows are MFMA operand rows: row r is
// stored at row r ^ ((r >> 3) & 7), i.e. its low three bits are XORed with the
// next three.  Rows 8 apart (which a transposing store writes in one phase)
// then start in different banks, while 8 consecutive rows (which an operand
// read touches in one phase) stay a permutation of 8 consecutive rows.  The
// map is its own inverse.
__device__ __forceinline__ int lds_row_perm(int r) { return r ^ ((r >> 3) & 7); }

template <class E, int ROWS, int COLS, int NTHR = kThreads>
struct RowTile {
  using T = typename E::storage;
  static constexpr int VEC = 16 / sizeof(T);
  static_assert(COLS % VEC == 0, "row length must be a multiple of 16 bytes");
  static constexpr int VPR = COLS / VEC;
  static constexpr int NV = ROWS * VPR;
  static constexpr int NPT = (NV + NTHR - 1) / NTHR;
  uint4 v[NPT];
  int len;  // rows >= len are stored as zeros

  // t: this thread's index among the NTHR staging threads; NTL: loads with the
  // non-temporal hint (the tile's last read)
  template <bool NTL = false>
  __device__ __forceinline__ void load(const T* __restrict__ g, int64_t ld, int L, int t = threadIdx.x) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = min(t + i * NTHR, NV - 1);
      const int r = idx / VPR, c = idx % VPR;
      const uint4* src = reinterpret_cast<const uint4*>(g + min(r, L - 1) * ld + c * VEC);
      v[i] = NTL ? load_nt(src) : *src;
    }
    len = L;
  }
  // ROWPERM: row r lands at row lds_row_perm(r)
  template <int DP, bool ROWPERM = false>
  __device__ __forceinline__ void store(T* __restrict__ lds, int t = threadIdx.x) const {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = t + i * NTHR;
      const int r = idx / VPR, c = idx % VPR;
      const int rs = ROWPERM ? lds_row_perm(r) : r;
      if (idx < NV) *reinterpret_cast<uint4*>(lds + rs * DP + c * VEC) = r < len ? v[i] : make_uint4(0, 0, 0, 0);
    }
  }
};

// XOR swizzle of the 16-byte blocks of a transposed bf16 tile (rows of ROWS
// tokens, no padding): block b of LDS row r is stored at block b ^ key(r).
// key takes 4 bits of r (3 when a row has only 8 blocks):
//   k0 = r0^r3, k1 = r1^r5^r6, k2 = r2^r4, k3 = r3^r5.
// It makes both access patterns free of bank conflicts: the transposing
// stores, where the lanes of one store phase write the same token block of
// rows 8 apart, and the MFMA operand reads, where they read the same block of
// consecutive rows.
template <int ROWS>
__device__ __forceinline__ int lds_swizzle(int r) {
  constexpr int mask = (ROWS / 8 >= 16 ? 16 : ROWS / 8) - 1;
  const int k = ((r ^ (r >> 3)) & 1) | ((((r >> 1) ^ (r >> 5) ^ (r >> 6)) & 1) << 1) |
                ((((r >> 2) ^ (r >> 4)) & 1) << 2) | ((((r >> 3) ^ (r >> 5)) & 1) << 3);
  return k & mask;
}

// A thread stages blocks of RPB rows x one 16-byte vector (bf16: RPB = 8 or
// 4 rows of 8 elements; fp32: 4 x 4).
template <class E, int ROWS, int COLS, int NTHR = kThreads, int RPB = (E::kBytes == 2 ? 8 : 4)>
struct TransTile {
  using T = typename E::storage;
  static constexpr bool kBf16 = E::kBytes == 2;
  static constexpr int BC = kBf16 ? 8 : 4;  // block width: one 16-byte vector
  static_assert(kBf16 ? (RPB == 8 || RPB == 4) : RPB == 4, "unsupported block height");
  static_assert(ROWS % RPB == 0 && COLS % BC == 0, "tile must be whole blocks");
  static constexpr int CB = COLS / BC;
  static constexpr int NB = (ROWS / RPB) * CB;
  static constexpr int NPT = (NB + NTHR - 1) / NTHR;
  uint4 v[NPT][RPB];
  int len;  // rows >= len are stored as zeros

  // t: this thread's index among the NTHR staging threads
  __device__ __forceinline__ void load(const T* __restrict__ g, int64_t ld, int L, int t = threadIdx.x) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int blk = min(t + i * NTHR, NB - 1);
      const int cb = blk % CB, rb = blk / CB;
#pragma unroll
      for (int rr = 0; rr < RPB; ++rr)
        v[i][rr] = *reinterpret_cast<const uint4*>(g + min(rb * RPB + rr, L - 1) * ld + cb * BC);
    }
    len = L;
  }
  // first tile row of block i of thread t (the rows whose scales store() takes)
  __device__ __forceinline__ static int first_row(int i, int t = threadIdx.x) {
    return (min(t + i * NTHR, NB - 1) / CB) * RPB;
  }
  // row rr of block i as loaded, or zeros past the tile's length
  __device__ __forceinline__ uint4 row(int i, int rb, int rr) const {
    return rb * RPB + rr < len ? v[i][rr] : make_uint4(0, 0, 0, 0);
  }

  // Transposed store.  Row scales: from LDS (scale[r], SCALE == 1), from
  // registers (sreg[i][rr] for row first_row(i) + rr, SCALE == 2), or none.
  // PERM16 (bf16 only): within every 16-token group the tokens are stored in
  // the order 0-3, 8-11, 4-7, 12-15, so that lane group g of a 32x32x16 MFMA
  // finds its tokens {4g..4g+3, 8+4g..8+4g+3} as one contiguous 16-byte run.
  // SWZ (bf16 only, DP == ROWS): 16-byte blocks placed by lds_swizzle<ROWS>.
  // ROWPERM (bf16 only): LDS row c (a column of the global tile) lands at row
  // lds_row_perm(c); with a row pitch of 4 (mod 32) dwords this stores without
  // bank conflicts.
  template <int DP, int SCALE, bool PERM16 = false, bool SWZ = false, bool ROWPERM = false>
  __device__ __forceinline__ void store(T* __restrict__ lds, const float* __restrict__ scale,
                                        const float (*sreg)[RPB] = nullptr, int t = threadIdx.x) const {
    static_assert(!SWZ || (kBf16 && DP == ROWS), "the swizzled layout is unpadded bf16");
    static_assert(!ROWPERM || kBf16, "the row permutation is for bf16 tiles");
    static_assert(!PERM16 || kBf16, "the 16-token permutation is for bf16 tiles");
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int blk = t + i * NTHR;
      if (blk >= NB) continue;
      const int cb = blk % CB, rb = blk / CB;
      float sc[RPB];
#pragma unroll
      for (int rr = 0; rr < RPB; ++rr)
        sc[rr] = SCALE == 1 ? scale[rb * RPB + rr] : SCALE == 2 ? sreg[i][rr] : 1.0f;
      if constexpr (kBf16 && SCALE == 0 && RPB == 8 && !PERM16) {
        // no scale: a pure 16-bit transpose, each output word two halves of
        // input words picked by v_perm_b32 (low halves for even columns,
        // high halves for odd ones), no conversion
        uint32_t w[8][4];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const uint4 q = row(i, rb, rr);
          w[rr][0] = q.x; w[rr][1] = q.y; w[rr][2] = q.z; w[rr][3] = q.w;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          uint4 o;
          o.x = __builtin_amdgcn_perm(w[1][c >> 1], w[0][c >> 1], sel);
          o.y = __builtin_amdgcn_perm(w[3][c >> 1], w[2][c >> 1], sel);
          o.z = __builtin_amdgcn_perm(w[5][c >> 1], w[4][c >> 1], sel);
          o.w = __builtin_amdgcn_perm(w[7][c >> 1], w[6][c >> 1], sel);
          const int r = cb * 8 + c;
          T* lrow = lds + (ROWPERM ? lds_row_perm(r) : r) * DP;
          const int key = SWZ ? lds_swizzle<ROWS>(r) : 0;
          *reinterpret_cast<uint4*>(lrow + (rb ^ key) * 8) = o;
        }
      } else if constexpr (kBf16) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float f[RPB];
#pragma unroll
          for (int rr = 0; rr < RPB; ++rr) {
            const uint4 q = row(i, rb, rr);
            const uint32_t w = (c >> 1) == 0 ? q.x : (c >> 1) == 1 ? q.y : (c >> 1) == 2 ? q.z : q.w;
            const float e = (c & 1) ? bf16_hi(w) : bf16_lo(w);
            f[rr] = SCALE ? e * sc[rr] : e;
          }
          const int r = cb * 8 + c;
          T* lrow = lds + (ROWPERM ? lds_row_perm(r) : r) * DP;
          const int key = SWZ ? lds_swizzle<ROWS>(r) : 0;
          if constexpr (RPB == 8) {
            uint4 o;
            o.x = pack_bf16x2(f[0], f[1]);
            o.y = pack_bf16x2(f[2], f[3]);
            o.z = pack_bf16x2(f[4], f[5]);
            o.w = pack_bf16x2(f[6], f[7]);
            if constexpr (PERM16) {
              // tokens 16g + {0-3, 8-11} -> block 2g, {4-7, 12-15} -> block 2g+1
              const int off = (rb & 1) * 4;
              *reinterpret_cast<uint2*>(lrow + (((rb >> 1) * 2) ^ key) * 8 + off) = make_uint2(o.x, o.y);
              *reinterpret_cast<uint2*>(lrow + (((rb >> 1) * 2 + 1) ^ key) * 8 + off) = make_uint2(o.z, o.w);
            } else {
              *reinterpret_cast<uint4*>(lrow + (rb ^ key) * 8) = o;
            }
          } else {
            const uint2 o = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
            // four tokens 4 rb .. 4 rb + 3: 16-byte block and half within it
            int blk16, half;
            if constexpr (PERM16) {
              const int t0 = (rb & 3) * 4;  // position within the 16-token group
              blk16 = (rb >> 2) * 2 + ((t0 >> 2) & 1);
              half = (t0 >> 3) & 1;
            } else {
              blk16 = rb >> 1;
              half = rb & 1;
            }
            *reinterpret_cast<uint2*>(lrow + (blk16 ^ key) * 8 + half * 4) = o;
          }
        }
      } else {
        float f[4][4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint4 q = row(i, rb, rr);
          f[rr][0] = __uint_as_float(q.x) * sc[rr];
          f[rr][1] = __uint_as_float(q.y) * sc[rr];
          f[rr][2] = __uint_as_float(q.z) * sc[rr];
          f[rr][3] = __uint_as_float(q.w) * sc[rr];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(lds) + (cb * 4 + c) * DP + rb * 4) =
              make_float4(f[0][c], f[1][c], f[2][c], f[3][c]);
      }
    }
  }
};

}  // namespace ssd
