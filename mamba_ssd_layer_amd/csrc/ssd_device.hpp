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

// Stores with the non-temporal hint: for data that the rest of the kernel (or
// the next kernel) does not read back soon, so that it is streamed out instead
// of displacing lines that are reused.  (The hint must be fixed at compile
// time at each site: two otherwise equal stores under a run-time branch are
// merged into one without it.)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(uint4* p, const uint4& v) {
  __builtin_nontemporal_store((u32x4_t){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_nt(uint2* p, const uint2& v) {
  __builtin_nontemporal_store((u32x2_t){v.x, v.y}, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void store_nt(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
// y + d * x on one 16-byte vector of the element type (fp32 arithmetic; bf16
// results rounded to nearest even).
template <class E>
__device__ __forceinline__ uint4 add_scaled(const uint4& y, const uint4& x, float d) {
  if constexpr (E::kBytes == 2) {
    auto f = [&](uint32_t yw, uint32_t xw) {
      return pack_bf16x2(bf16_lo(yw) + d * bf16_lo(xw), bf16_hi(yw) + d * bf16_hi(xw));
    };
    return make_uint4(f(y.x, x.x), f(y.y, x.y), f(y.z, x.z), f(y.w, x.w));
  } else {
    auto f = [&](uint32_t yw, uint32_t xw) { return __float_as_uint(__uint_as_float(yw) + d * __uint_as_float(xw)); };
    return make_uint4(f(y.x, x.x), f(y.y, x.y), f(y.z, x.z), f(y.w, x.w));
  }
}

// The same on one 8-byte vector.
template <class E>
__device__ __forceinline__ uint2 add_scaled(const uint2& y, const uint2& x, float d) {
  const uint4 r = add_scaled<E>(make_uint4(y.x, y.y, 0u, 0u), make_uint4(x.x, x.y, 0u, 0u), d);
  return make_uint2(r.x, r.y);
}

// Load with the non-temporal hint: for the last read of data.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(q.x, q.y, q.z, q.w);
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

// Workgroup barrier that orders LDS only.  __syncthreads() is a workgroup
// fence on every address space, which makes each wave wait for all of its
// outstanding global loads and stores (vmcnt(0)) before the barrier; that would
// serialise the next tile's prefetch and the output stores with every barrier.
// Kernels that share only LDS between waves use this instead.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// Scans over segments of SEG consecutive lanes (SEG a power of two, <= 64).
// They only add: an exclusive sum is the inclusive sum of the shifted values,
// never an inclusive sum minus the lane's own value, so a sum of terms of one
// sign carries a relative rounding error of a few ulps whatever the size of
// the terms around it.
template <int SEG>
__device__ __forceinline__ float seg_inclusive_sum(float v) {
  const int pos = threadIdx.x & (SEG - 1);
#pragma unroll
  for (int off = 1; off < SEG; off <<= 1) {
    const float o = __shfl_up(v, off, kWave);
    if (pos >= off) v += o;
  }
  return v;
}
template <int SEG>
__device__ __forceinline__ float seg_inclusive_suffix_sum(float v) {
  const int pos = threadIdx.x & (SEG - 1);
#pragma unroll
  for (int off = 1; off < SEG; off <<= 1) {
    const float o = __shfl_down(v, off, kWave);
    if (pos + off < SEG) v += o;
  }
  return v;
}
// sum over the lanes before this one in its segment (0 for the first)
template <int SEG>
__device__ __forceinline__ float seg_exclusive_sum(float v) {
  const float e = __shfl_up(v, 1, kWave);
  return seg_inclusive_sum<SEG>((threadIdx.x & (SEG - 1)) == 0 ? 0.0f : e);
}
// sum over the lanes after this one in its segment (0 for the last)
template <int SEG>
__device__ __forceinline__ float seg_exclusive_suffix_sum(float v) {
  const float e = __shfl_down(v, 1, kWave);
  return seg_inclusive_suffix_sum<SEG>((threadIdx.x & (SEG - 1)) == SEG - 1 ? 0.0f : e);
}

// Scans over a whole 64-lane wave on DPP lane moves (VALU latency, no LDS
// round trip per step): Hillis-Steele within each row of 16 lanes, the rows
// then joined by their totals (readlane).  Addition only, as above.
template <int CTRL>
__device__ __forceinline__ float dpp_move0(float v) {  // lanes without a source read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// sum over this lane and the lanes before it
__device__ __forceinline__ float wave_prefix_incl_dpp(float v) {
  v += dpp_move0<0x111>(v);  // row_shr:1
  v += dpp_move0<0x112>(v);  // row_shr:2
  v += dpp_move0<0x114>(v);  // row_shr:4
  v += dpp_move0<0x118>(v);  // row_shr:8
  const float t0 = lane_value(v, 15), t1 = lane_value(v, 31), t2 = lane_value(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  const float o2 = t0 + t1;
  return row == 0 ? v : v + (row == 1 ? t0 : row == 2 ? o2 : o2 + t2);
}
// sum over the lanes before this one (0 for lane 0): the inclusive sum of the
// values shifted up by one lane
__device__ __forceinline__ float wave_prefix_excl_dpp(float v) {
  return wave_prefix_incl_dpp(dpp_move0<0x138>(v));  // wave_shr:1: lane i reads lane i - 1
}
// sum over the lanes after this one; TILE32: only those of its 32-lane half
template <bool TILE32 = false>
__device__ __forceinline__ float wave_suffix_excl_dpp(float v) {
  const int lane = threadIdx.x & 63;
  float u = dpp_move0<0x130>(v);  // wave_shl:1: lane i reads lane i + 1 (lane 63 reads 0)
  if (TILE32 && (lane & 31) == 31) u = 0.0f;
  u += dpp_move0<0x101>(u);  // row_shl:1
  u += dpp_move0<0x102>(u);  // row_shl:2
  u += dpp_move0<0x104>(u);  // row_shl:4
  u += dpp_move0<0x108>(u);  // row_shl:8
  const float t1 = lane_value(u, 16), t2 = lane_value(u, 32), t3 = lane_value(u, 48);
  const int row = lane >> 4;
  if (TILE32) return (row & 1) ? u : u + (row == 0 ? t1 : t3);
  const float o1 = t3 + t2;
  return row == 3 ? u : u + (row == 2 ? t3 : row == 1 ? o1 : o1 + t1);
}

// Mask factorisation of one (chunk, head) of the diagonal block: by the whole
// chunk (x_j staged times exp(-Acs_j), the finished sums times exp(Acs_i)) when
// the chunk's total log-decay lam is at least -limit, else per element from
// addition-only segment sums.  The limit bounds both factors (e^limit) and the
// fp32 rounding of the cumsums they come from (an absolute error of a few
// limit * 2^-24 in the exponent): 64 on the bf16 path, whose operands are
// rounded to 2^-9 anyway, 16 on the fp32 path.  The chunk-state kernel (which
// writes the per-element kernel's tables) and the output kernel decide with
// this one function on the same stored lam.
template <class E>
__device__ __forceinline__ bool mask_by_chunk(float lam) {
  return lam >= (E::kBytes == 2 ? -64.0f : -16.0f);
}

// Chunk descriptor of slot k.  Batched problems (no cu_seqlens) compute it:
// sequence s = k / nc owns slots [s*nc, (s+1)*nc), nc = ceil(T/Q); varlen
// problems read the table the cumsum kernel filled.
__device__ __forceinline__ ChunkDesc chunk_desc(const Problem& p, const Workspace& ws, int64_t k) {
  if (p.cu == nullptr) {
    const int64_t nc = (p.seqlen + p.Q - 1) / p.Q;
    const int64_t s = k / nc, c = k % nc;
    const int64_t rem = p.seqlen - c * p.Q;
    ChunkDesc d;
    d.seq = (int32_t)s;
    d.len = (int32_t)(rem < p.Q ? rem : p.Q);
    d.t0 = s * p.seqlen + c * p.Q;
    return d;
  }
  return ws.chunks[k];
}

// Chunk descriptor of slot k found from the sequence table: the last sequence
// s with seq_off[s] <= k (sequences without chunks share their offset with the
// next one, so the last match is the one that owns slot k).
__device__ __forceinline__ ChunkDesc chunk_desc_search(const Problem& p, const Workspace& ws,
                                                       int64_t k) {
  if (p.cu == nullptr) return chunk_desc(p, ws, k);
  ChunkDesc d;
  d.seq = -1;
  d.len = 0;
  d.t0 = 0;
  const int64_t nch = ws.seq_off[p.nseq];
  if (k >= nch) return d;
  int64_t lo = 0, hi = p.nseq;  // seq_off[lo] <= k < seq_off[hi]
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (ws.seq_off[mid] <= k) lo = mid; else hi = mid;
  }
  const int64_t c = k - ws.seq_off[lo];
  const int64_t rem = ws.seq_len[lo] - c * p.Q;
  d.len = (int32_t)(rem < p.Q ? (rem > 0 ? rem : 0) : p.Q);
  d.seq = d.len > 0 ? (int32_t)lo : -1;
  d.t0 = ws.seq_start[lo] + c * p.Q;
  return d;
}

// First chunk slot of sequence s and one past its last.
__device__ __forceinline__ void seq_chunk_range(const Problem& p, const Workspace& ws, int64_t s,
                                                int64_t* k0, int64_t* k1) {
  if (p.cu == nullptr) {
    const int64_t nc = (p.seqlen + p.Q - 1) / p.Q;
    *k0 = s * nc;
    *k1 = (s + 1) * nc;
  } else {
    *k0 = ws.seq_off[s];
    *k1 = ws.seq_off[s + 1];
  }
}

}  // namespace ssd
