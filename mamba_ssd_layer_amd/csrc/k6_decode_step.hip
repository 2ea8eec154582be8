// k6_decode_step.hip -- one recurrent step of the SSM for a batch of
// sequences: the decode (autoregressive inference) mode of the layer.
//
// Pages: [T] "Transformers是SSMs…(一)" (nxbn.cn) §2.1: autoregressive
// inference runs the recurrent form one input step at a time, with a state of
// constant size; [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba)
// §3.5.3, cost table: an inference step of SSM and SSD costs N^2 FLOPs (here
// 2PN for the update and 2PN for the output, per head).  For every sequence b
// and head h, with a = exp(dt[b,h] * A_h) and g the head's B/C group:
//     state[b,h] <- a * state[b,h] + x[b,h,:] (outer) B[b,g,:]     (P x N, fp32)
//     y[b,h,p]   <- sum_n state[b,h,p,n] * C[b,g,n]
// the same update as one token of the forward pass, so a state from the
// forward's final_state continues the sequence.  Options as in the forward:
// the input may enter as dt x (B scaled by the step size) and y may get the
// skip term D_h x.
//
// Design (gfx950): pure HBM streaming of the fp32 state, read and written once
// (8PN bytes per head).  One workgroup of 256 threads per (sequence, head);
// thread t owns the 16-byte state vectors t, t + 256, ... of the head's
// (P x N) block.  N/4 divides 64 and 256, so all of a thread's vectors lie in
// one column block of 4 n: it keeps those 4 B and C values in registers, and
// every state access is one fully coalesced 16-byte load or store.  The
// thread issues all its state loads before any arithmetic.  The row sums over
// n are a shuffle reduction across the N/4 consecutive lanes that share a row.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kDecThreads = 256;

template <class E, int N>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(DecodeProblem d) {
  using T = typename E::storage;
  constexpr int P = kHeadDim;
  constexpr int NV = N / 4;                   // 16-byte vectors per state row
  constexpr int VPT = P * NV / kDecThreads;   // vectors per thread
  constexpr int RSTEP = kDecThreads / NV;     // rows between a thread's vectors
  static_assert(64 % NV == 0 && VPT >= 1, "a row's vectors must sit in one wave");
  const int64_t bh = blockIdx.x;
  const int h = (int)(bh % d.H);
  const int64_t b = bh / d.H;
  const int g = h / (d.H / d.G);
  const int t = threadIdx.x;
  const int n4 = t % NV;
  const int row0 = t / NV;

  float4* st = reinterpret_cast<float4*>(d.state) + bh * (P * NV);
  float4 v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) v[i] = st[t + i * kDecThreads];

  const float a = __expf(d.dt[bh] * d.A[h]);
  float bv[4], cv[4];
  const int64_t bc = (b * d.G + g) * N + 4 * n4;
  if constexpr (E::kBytes == 2) {
    const uint2 qb = *reinterpret_cast<const uint2*>(reinterpret_cast<const T*>(d.B) + bc);
    const uint2 qc = *reinterpret_cast<const uint2*>(reinterpret_cast<const T*>(d.C) + bc);
    bv[0] = bf16_lo(qb.x); bv[1] = bf16_hi(qb.x); bv[2] = bf16_lo(qb.y); bv[3] = bf16_hi(qb.y);
    cv[0] = bf16_lo(qc.x); cv[1] = bf16_hi(qc.x); cv[2] = bf16_lo(qc.y); cv[3] = bf16_hi(qc.y);
  } else {
    const float4 qb = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(d.B) + bc);
    const float4 qc = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(d.C) + bc);
    bv[0] = qb.x; bv[1] = qb.y; bv[2] = qb.z; bv[3] = qb.w;
    cv[0] = qc.x; cv[1] = qc.y; cv[2] = qc.z; cv[3] = qc.w;
  }
  const T* xrow = reinterpret_cast<const T*>(d.x) + bh * P;
  T* yrow = reinterpret_cast<T*>(d.y) + bh * P;

  const float xs = d.x_times_dt ? d.dt[bh] : 1.0f;  // the input enters as dt x
  const float dskip = d.D != nullptr ? d.D[h] : 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int p = row0 + i * RSTEP;
    float xraw;
    if constexpr (E::kBytes == 2) xraw = bf16_to_f32(xrow[p]);
    else xraw = xrow[p];
    const float xp = xs * xraw;
    float4 s = v[i];
    s.x = a * s.x + xp * bv[0];
    s.y = a * s.y + xp * bv[1];
    s.z = a * s.z + xp * bv[2];
    s.w = a * s.w + xp * bv[3];
    st[t + i * kDecThreads] = s;
    float part = s.x * cv[0] + s.y * cv[1] + s.z * cv[2] + s.w * cv[3];
#pragma unroll
    for (int off = NV / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if (n4 == 0) {
      part += dskip * xraw;  // skip connection on the raw input
      if constexpr (E::kBytes == 2) yrow[p] = (T)(pack_bf16x2(part, 0.0f) & 0xffffu);
      else yrow[p] = part;
    }
  }
}

template <class E>
static hipError_t launch_dec(const DecodeProblem& d, hipStream_t s) {
  const dim3 grid((unsigned)(d.batch * d.H)), block(kDecThreads);
  switch (d.N) {
    case 16: hipLaunchKernelGGL((decode_step_kernel<E, 16>), grid, block, 0, s, d); break;
    case 32: hipLaunchKernelGGL((decode_step_kernel<E, 32>), grid, block, 0, s, d); break;
    case 64: hipLaunchKernelGGL((decode_step_kernel<E, 64>), grid, block, 0, s, d); break;
    case 128: hipLaunchKernelGGL((decode_step_kernel<E, 128>), grid, block, 0, s, d); break;
    case 256: hipLaunchKernelGGL((decode_step_kernel<E, 256>), grid, block, 0, s, d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeProblem& d, hipStream_t s) {
  if (d.batch == 0) return hipSuccess;
  return d.dtype == Dtype::BF16 ? launch_dec<Bf16>(d, s) : launch_dec<F32>(d, s);
}

}  // namespace ssd
