// k4_state_pass.hip -- inter-chunk state passing of the SSD block
// decomposition (K4).
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba), §3.5.2
// "Center factors" and step 3 of "SSD algorithm: chunking and state passing":
// a scalar SSM (1-SS) recurrence over the chunks of each sequence, run on P*N
// independent channels per head:
//     Hin[first chunk] = 0,   Hin[c+1] = exp(lam_c) * Hin[c] + S_c,
// where lam_c is the chunk's total log-decay; the value after the last chunk is
// the final state.  [M] §3.5.3 prices this scan at T*N*P/Q work, a small part
// of the whole.
//
// Design (gfx950): pure HBM streaming, bound by how many bytes are in flight.
// A thread owns 2 consecutive (p, n) channels of one (sequence, head) and walks
// the sequence's chunks in order; the loads of later chunks' states do not
// depend on the running state, so they are issued a block of 8 chunks ahead
// and only the FMA chain is serial.  Lanes of a wave cover 128 consecutive
// channels: every access is a fully coalesced 4-byte (bf16) or 8-byte (fp32)
// vector.  Chunk states are read and
// Hin is written in the element dtype (the output kernel feeds Hin to the
// matrix cores in that dtype); the running state stays fp32.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kCh = 2;      // channels per thread
constexpr int kDepth = 8;   // chunks per block; one block of loads is in flight ahead of the scan

template <class E>
__device__ __forceinline__ float2 load2(const typename E::storage* ptr) {
  if constexpr (E::kBytes == 2) {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(ptr);
    return make_float2(bf16_lo(q), bf16_hi(q));
  } else {
    return *reinterpret_cast<const float2*>(ptr);
  }
}

// Stores 2 channels in the element dtype; returns the stored values as fp32.
template <class E>
__device__ __forceinline__ float2 store2(typename E::storage* ptr, float2 v) {
  if constexpr (E::kBytes == 2) {
    const uint32_t o = pack_bf16x2(v.x, v.y);
    *reinterpret_cast<uint32_t*>(ptr) = o;
    return make_float2(bf16_lo(o), bf16_hi(o));
  } else {
    *reinterpret_cast<float2*>(ptr) = v;
    return v;
  }
}

template <class E, bool kDebug>
__global__ __launch_bounds__(kThreads) void state_pass_kernel(Problem p, Workspace ws,
                                                              float* __restrict__ hin_f32) {
  using T = typename E::storage;
  const int PN = p.P * p.N;
  const int cblocks = (PN + kCh * kThreads - 1) / (kCh * kThreads);
  const int64_t bid = blockIdx.x;
  const int cb = (int)(bid % cblocks);
  const int h = (int)((bid / cblocks) % p.H);
  const int64_t s = bid / ((int64_t)cblocks * p.H);
  const int ch = (cb * kThreads + threadIdx.x) * kCh;
  if (ch >= PN) return;
  const int H = p.H;
  int64_t k0, k1;
  seq_chunk_range(p, ws, s, &k0, &k1);
  const int nk = (int)(k1 - k0);
  const int stride = H * PN;  // elements between consecutive chunks of one head
  // uniform (per-block) bases; the lane's own offset stays a 32-bit add
  const int64_t blk0 = (k0 * H + h) * PN + (int64_t)cb * kThreads * kCh;
  const int lo = threadIdx.x * kCh;
  const T* st_in = reinterpret_cast<const T*>(ws.states) + blk0;
  T* hin = reinterpret_cast<T*>(ws.hin) + blk0;
  float* hin32 = kDebug ? hin_f32 + blk0 : nullptr;
  const float* lam = ws.lam + k0 * H + h;
  float2 st = make_float2(0.f, 0.f);
  // Software pipeline over blocks of kDepth chunks with two register buffers
  // used in turn (no copies between them): the loads of the next block are in
  // flight while the current block is scanned, so only the FMA chain is serial.
  float2 bufA[kDepth], bufB[kDepth];
  float decA[kDepth], decB[kDepth];
  // Loads are unconditional (indices past the end are clamped to the last
  // chunk and never used) so that the loop body is straight-line code and each
  // wait covers exactly the block it needs.
  auto load_block = [&](int kb, float2 (&sv)[kDepth], float (&dec)[kDepth]) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int kk = min(kb + u, nk - 1);
      sv[u] = load2<E>(st_in + (int64_t)kk * stride + lo);
      dec[u] = lam[(int64_t)kk * H];
    }
  };
  auto step = [&](int kk, float2 sv, float dec) {
    const float2 r = store2<E>(hin + (int64_t)kk * stride + lo, st);
    if constexpr (kDebug) *reinterpret_cast<float2*>(hin32 + (int64_t)kk * stride + lo) = r;
    const float a = __expf(dec);
    st.x = a * st.x + sv.x;
    st.y = a * st.y + sv.y;
  };
  const int nfull = nk / kDepth;
  if (nfull > 0) {
    load_block(0, bufA, decA);
    int b = 0;
    for (; b + 2 <= nfull; b += 2) {
      load_block((b + 1) * kDepth, bufB, decB);
#pragma unroll
      for (int u = 0; u < kDepth; ++u) step(b * kDepth + u, bufA[u], decA[u]);
      load_block((b + 2) * kDepth, bufA, decA);
#pragma unroll
      for (int u = 0; u < kDepth; ++u) step((b + 1) * kDepth + u, bufB[u], decB[u]);
    }
    if (b < nfull) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) step(b * kDepth + u, bufA[u], decA[u]);
    }
  }
  for (int kk = nfull * kDepth; kk < nk; ++kk)
    step(kk, load2<E>(st_in + (int64_t)kk * stride + lo), lam[(int64_t)kk * H]);
  if (p.final_state != nullptr)
    *reinterpret_cast<float2*>(p.final_state + (s * H + h) * (int64_t)PN + ch) = st;
}

hipError_t launch_state_pass(const Problem& p, const Workspace& ws, float* hin_f32,
                             hipStream_t s) {
  const int PN = p.P * p.N;
  const int64_t cblocks = (PN + kCh * kThreads - 1) / (kCh * kThreads);
  const int64_t blocks = p.nseq * p.H * cblocks;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (p.dtype == Dtype::BF16) {
    if (hin_f32) hipLaunchKernelGGL((state_pass_kernel<Bf16, true>), grid, block, 0, s, p, ws, hin_f32);
    else hipLaunchKernelGGL((state_pass_kernel<Bf16, false>), grid, block, 0, s, p, ws, hin_f32);
  } else {
    if (hin_f32) hipLaunchKernelGGL((state_pass_kernel<F32, true>), grid, block, 0, s, p, ws, hin_f32);
    else hipLaunchKernelGGL((state_pass_kernel<F32, false>), grid, block, 0, s, p, ws, hin_f32);
  }
  return hipGetLastError();
}

}  // namespace ssd
