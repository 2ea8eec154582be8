// k4_state_pass.hip -- inter-chunk state passing of the SSD block
// decomposition (K4).
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba), §3.5.2
// "Center factors" and step 3 of "SSD algorithm: chunking and state passing":
// a scalar SSM (1-SS) recurrence over the chunks of each sequence, run on P*N
// independent channels per head:
//     Hin[first chunk] = h0,  Hin[c+1] = exp(lam_c) * Hin[c] + S_c,
// where lam_c is the chunk's total log-decay; the value after the last chunk is
// the final state.  h0 is the sequence's initial state (zero unless the caller
// gives one: [M] §3.7.2 "Sequence Parallelism", where each worker starts from
// the state its predecessor passes on; the §3.5 listing prepends the same
// optional initial state to the chunk states before this scan).  [M] §3.5.3 prices this scan at T*N*P/Q work, a small part
// of the whole.
//
// Design (gfx950): pure HBM streaming, bound by how many bytes are in flight.
// A thread owns kCh (2 or 4) consecutive (p, n) channels of one (sequence, head) and walks
// the sequence's chunks in order; the loads of later chunks' states do not
// depend on the running state, so they are issued a block of kDepth chunks
// ahead (the last block of a sequence may be partial) and only the FMA chain
// is serial.  Lanes of a wave cover 64 kCh consecutive channels: every access
// is a fully coalesced vector of kCh elements.  Chunk states are read and Hin
// is written in the element dtype (the output kernel feeds Hin to the matrix
// cores in that dtype), with the non-temporal hint when the forward's data
// exceeds the last-level cache; the running state stays fp32.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kDepth = 8;   // chunks per block; one block of loads is in flight ahead of the scan

// kCh consecutive channels in the element dtype <-> fp32 registers.
template <class E, int kCh>
__device__ __forceinline__ void load_ch(const typename E::storage* ptr, float (&v)[kCh]) {
  if constexpr (E::kBytes == 2) {
    if constexpr (kCh == 2) {
      const uint32_t q = *reinterpret_cast<const uint32_t*>(ptr);
      v[0] = bf16_lo(q); v[1] = bf16_hi(q);
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(ptr);
      v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    }
  } else {
    if constexpr (kCh == 2) {
      const float2 q = *reinterpret_cast<const float2*>(ptr);
      v[0] = q.x; v[1] = q.y;
    } else {
      const float4 q = *reinterpret_cast<const float4*>(ptr);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
  }
}

// Stores kCh channels in the element dtype (nt: with the non-temporal hint);
// r receives the stored values as fp32.
template <class E, int kCh>
__device__ __forceinline__ void store_ch(typename E::storage* ptr, const float (&v)[kCh], float (&r)[kCh], bool nt) {
  static_assert(kCh == 2 || kCh == 4, "two or four channels per thread");
  if constexpr (E::kBytes == 2) {
    uint32_t o[kCh / 2];
#pragma unroll
    for (int c = 0; c < kCh / 2; ++c) {
      o[c] = pack_bf16x2(v[2 * c], v[2 * c + 1]);
      r[2 * c] = bf16_lo(o[c]);
      r[2 * c + 1] = bf16_hi(o[c]);
    }
    if constexpr (kCh == 2) {
      if (nt) store_nt(reinterpret_cast<uint32_t*>(ptr), o[0]);
      else *reinterpret_cast<uint32_t*>(ptr) = o[0];
    } else {
      if (nt) store_nt(reinterpret_cast<uint2*>(ptr), make_uint2(o[0], o[1]));
      else *reinterpret_cast<uint2*>(ptr) = make_uint2(o[0], o[1]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < kCh; ++c) r[c] = v[c];
    if constexpr (kCh == 2) {
      const uint2 o = make_uint2(__float_as_uint(v[0]), __float_as_uint(v[1]));
      if (nt) store_nt(reinterpret_cast<uint2*>(ptr), o);
      else *reinterpret_cast<uint2*>(ptr) = o;
    } else {
      const uint4 o = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                 __float_as_uint(v[3]));
      if (nt) store_nt(reinterpret_cast<uint4*>(ptr), o);
      else *reinterpret_cast<uint4*>(ptr) = o;
    }
  }
}

// kCh: channels per thread (2 or 4)
template <class E, int kCh, bool kDebug>
__global__ __launch_bounds__(kThreads) void state_pass_kernel(Problem p, Workspace ws,
                                                              float* __restrict__ hin_f32) {
  using T = typename E::storage;
  // channel blocks of the (P, N) states, then (normalised output only) those of
  // the ones column's N-vector states, passed the same way
  const int PNs = p.P * p.N;
  const int cbS = (PNs + kCh * kThreads - 1) / (kCh * kThreads);
  const int cbZ = ws.zs != nullptr ? (p.N + kCh * kThreads - 1) / (kCh * kThreads) : 0;
  const int cblocks = cbS + cbZ;
  const int64_t bid = blockIdx.x;
  const int cbg = (int)(bid % cblocks);
  const bool zc = cbg >= cbS;  // uniform per block
  const int cb = zc ? cbg - cbS : cbg;
  const int PN = zc ? p.N : PNs;
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
  const T* st_in = reinterpret_cast<const T*>(zc ? ws.zs : ws.states) + blk0;
  T* hin = reinterpret_cast<T*>(zc ? ws.zin : ws.hin) + blk0;
  float* hin32 = (kDebug && !zc) ? hin_f32 + blk0 : nullptr;
  const float* lam = ws.lam + k0 * H + h;
  // running state: the sequence's initial state (zero when none is given; the
  // ones column always starts from zero)
  float st[kCh] = {};
  if (p.initial_state != nullptr && !zc) {
#pragma unroll
    for (int c = 0; c < kCh; c += 2) {
      const float2 s0 = *reinterpret_cast<const float2*>(p.initial_state + (s * H + h) * (int64_t)PN + ch + c);
      st[c] = s0.x;
      st[c + 1] = s0.y;
    }
  }
  const bool nt = p.stream_states != 0;
  // Software pipeline over blocks of kDepth chunks with two register buffers
  // used in turn (no copies between them): the loads of the next block are in
  // flight while the current block is scanned, so only the FMA chain is serial.
  float bufA[kDepth][kCh], bufB[kDepth][kCh];
  // the block's log-decays: lane u holds chunk kb + u (a vector load, which
  // completes in order with the state loads; a scalar load would be waited
  // for together with every other scalar load in flight)
  float decA, decB;
  const int lane = threadIdx.x & 63;
  // Loads are unconditional (indices past the end are clamped to the last
  // chunk and never used) so that the loop body is straight-line code and each
  // wait covers exactly the block it needs.
  auto load_block = [&](int kb, float (&sv)[kDepth][kCh], float& dec) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int kk = min(kb + u, nk - 1);
      load_ch<E, kCh>(st_in + (int64_t)kk * stride + lo, sv[u]);
    }
    dec = lam[(int64_t)min(kb + (lane % kDepth), nk - 1) * H];
  };
  auto lane_dec = [&](float dec, int u) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dec), u)); };
  auto step = [&](int kk, const float (&sv)[kCh], float dec) {
    float r[kCh];
    store_ch<E, kCh>(hin + (int64_t)kk * stride + lo, st, r, nt);
    if constexpr (kDebug) {
      if (hin32 != nullptr) {
#pragma unroll
        for (int c = 0; c < kCh; ++c) hin32[(int64_t)kk * stride + lo + c] = r[c];
      }
    }
    const float a = __expf(dec);
#pragma unroll
    for (int c = 0; c < kCh; ++c) st[c] = a * st[c] + sv[c];
  };
  // blocks of kDepth chunks; the last one may be partial (its loads clamped,
  // its steps past the end skipped)
  auto scan_block = [&](int b, const float (&sv)[kDepth][kCh], float dec) {
    if ((b + 1) * kDepth <= nk) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) step(b * kDepth + u, sv[u], lane_dec(dec, u));
    } else {
#pragma unroll
      for (int u = 0; u < kDepth; ++u)
        if (b * kDepth + u < nk) step(b * kDepth + u, sv[u], lane_dec(dec, u));
    }
  };
  const int nb = (nk + kDepth - 1) / kDepth;
  if (nb > 0) {
    load_block(0, bufA, decA);
    int b = 0;
    for (; b + 2 <= nb; b += 2) {
      load_block((b + 1) * kDepth, bufB, decB);
      scan_block(b, bufA, decA);
      load_block((b + 2) * kDepth, bufA, decA);
      scan_block(b + 1, bufB, decB);
    }
    if (b < nb) scan_block(b, bufA, decA);
  }
  if (p.final_state != nullptr && !zc) {
    float* fs = p.final_state + (s * H + h) * (int64_t)PN + ch;
#pragma unroll
    for (int c = 0; c < kCh; c += 2) *reinterpret_cast<float2*>(fs + c) = make_float2(st[c], st[c + 1]);
  }
}

template <class E, int kCh>
static hipError_t launch_sp(const Problem& p, const Workspace& ws, float* hin_f32, hipStream_t s) {
  const int PN = p.P * p.N;
  const int64_t cblocks = (PN + kCh * kThreads - 1) / (kCh * kThreads) +
                          (ws.zs != nullptr ? (p.N + kCh * kThreads - 1) / (kCh * kThreads) : 0);
  const dim3 grid((unsigned)(p.nseq * p.H * cblocks)), block(kThreads);
  if (hin_f32) hipLaunchKernelGGL((state_pass_kernel<E, kCh, true>), grid, block, 0, s, p, ws, hin_f32);
  else hipLaunchKernelGGL((state_pass_kernel<E, kCh, false>), grid, block, 0, s, p, ws, hin_f32);
  return hipGetLastError();
}

hipError_t launch_state_pass(const Problem& p, const Workspace& ws, float* hin_f32,
                             hipStream_t s) {
  const int64_t PN = (int64_t)p.P * p.N;
  if (p.nseq * p.H == 0) return hipSuccess;
  // Four channels per thread (8- or 16-byte accesses) when that still leaves
  // at least two workgroups per CU; else two, for more waves in flight
  // (measured: four channels 6 % faster on 8 x 2048 tokens x 80 heads, 1 %
  // slower on one 16384-token sequence of 32 heads).
  const int64_t blocks4 = p.nseq * p.H * ((PN + 4 * kThreads - 1) / (4 * kThreads));
  const bool ch4 = blocks4 >= 2 * (int64_t)device_cus();
  if (p.dtype == Dtype::BF16)
    return ch4 ? launch_sp<Bf16, 4>(p, ws, hin_f32, s) : launch_sp<Bf16, 2>(p, ws, hin_f32, s);
  return ch4 ? launch_sp<F32, 4>(p, ws, hin_f32, s) : launch_sp<F32, 2>(p, ws, hin_f32, s);
}

}  // namespace ssd
