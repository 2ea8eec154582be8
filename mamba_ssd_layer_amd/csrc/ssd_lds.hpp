// ssd_lds.hpp -- load-to-LDS copies and the waits and barriers around them
// (gfx950), and the chunk map, shared by the chunk-local backward kernels.
#pragma once
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {

// One load-to-LDS instruction: each lane's 16 bytes from src to dst + 16 lane
// (dst is the same in every lane of the wave).
__device__ __forceinline__ void lds_copy16(const uint16_t* src, uint4* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (they complete in issue order).  n is a compile-time constant < 64.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) left at their maxima
  __builtin_amdgcn_s_waitcnt((n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier for LDS traffic that leaves the loads in flight alone.
// A fence-based barrier would also wait for the load-to-LDS copies still
// pending (they write LDS); here each wave waits for its own LDS operations,
// and for the copies it needs, explicitly.  The signal fences keep the
// compiler from moving memory operations across the barrier.
__device__ __forceinline__ void dl_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xf | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS slot (16-byte vector index) of vector q of row r in a row-major block
// of rows of V vectors: the vector index is XORed with a function of the row
// so that the same q of 32 consecutive rows spreads over the 16 bank groups.
template <int V>
__device__ __forceinline__ int swz_slot(int r, int q) {
  const int x = V >= 16 ? (r & 15) : ((r / (16 / V)) % V);
  return r * V + (q ^ x);
}

// Chunk k of the chunk-local backward path.  Every sequence there is a whole
// number of chunks (batched: seqlen a multiple of Q; packed: padded so), so
// chunk k covers tokens [kQ, kQ + Q) of one sequence, which starts at token s0,
// has L tokens (CPS chunks) and holds the chunk as its chunk c.  Packed
// sequences are found in cu by binary search (empty ones share their start
// with the next).  A cu that breaks the alignment gives unspecified results,
// never an index outside [0, total): such a chunk is taken as a sequence of
// its own.
struct BwdChunk {
  int64_t t0, s0, L, CPS, c;
};
__device__ __forceinline__ BwdChunk bwd_chunk(const BwdProblem& b, int64_t k, int Q) {
  BwdChunk r;
  r.t0 = k * Q;
  if (b.cu == nullptr) {
    r.L = b.seqlen;
    r.s0 = b.seqlen > 0 ? (r.t0 / b.seqlen) * b.seqlen : r.t0;
  } else {
    int64_t lo = 0, hi = b.nseq;  // last s with cu[s] <= t0
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (b.cu[mid] <= r.t0) lo = mid;
      else hi = mid;
    }
    r.s0 = b.cu[lo];
    r.L = (int64_t)b.cu[lo + 1] - r.s0;
  }
  if (r.s0 < 0 || r.s0 > r.t0 || r.L < Q || r.L % Q != 0 || (r.t0 - r.s0) % Q != 0 || r.s0 + r.L < r.t0 + Q ||
      r.s0 + r.L > b.total) {
    r.s0 = r.t0;
    r.L = Q;
  }
  r.CPS = r.L / Q;
  r.c = (r.t0 - r.s0) / Q;
  return r;
}

}  // namespace ssd
