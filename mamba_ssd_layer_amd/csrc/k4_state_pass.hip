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
// Design (gfx950): pure HBM streaming.  A thread owns 4 consecutive (p, n)
// channels of one (sequence, head) and walks the sequence's chunks in order;
// the loads of the next chunks' states are independent of the running state,
// so they are issued ahead (unroll by 4) and only the FMA chain is serial.
// Lanes of a wave cover 256 consecutive channels: every access is a fully
// coalesced 16-byte (fp32) or 8-byte (bf16) vector.  Hin is written in the
// element dtype: the output kernel feeds it to the matrix cores in that dtype.
#include "ssd_device.hpp"

namespace ssd {

template <class E>
__global__ __launch_bounds__(kThreads) void state_pass_kernel(Problem p, Workspace ws,
                                                              float* __restrict__ hin_f32) {
  const int PN = p.P * p.N;
  const int cblocks = (PN + 4 * kThreads - 1) / (4 * kThreads);
  const int64_t bid = blockIdx.x;
  const int cb = (int)(bid % cblocks);
  const int h = (int)((bid / cblocks) % p.H);
  const int64_t s = bid / ((int64_t)cblocks * p.H);
  const int ch = (cb * kThreads + threadIdx.x) * 4;
  if (ch >= PN) return;
  const int H = p.H;
  const int32_t k0 = ws.seq_off[s], k1 = ws.seq_off[s + 1];
  float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
  using T = typename E::storage;
  T* hin = reinterpret_cast<T*>(ws.hin);
  int32_t k = k0;
  for (; k + 4 <= k1; k += 4) {
    float4 sv[4];
    float dec[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t base = ((int64_t)(k + u) * H + h) * PN + ch;
      sv[u] = *reinterpret_cast<const float4*>(ws.states + base);
      dec[u] = __expf(ws.lam[(int64_t)(k + u) * H + h]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t base = ((int64_t)(k + u) * H + h) * PN + ch;
      if constexpr (E::kBytes == 2) {
        uint2 o;
        o.x = pack_bf16x2(st.x, st.y);
        o.y = pack_bf16x2(st.z, st.w);
        *reinterpret_cast<uint2*>(hin + base) = o;
      } else {
        *reinterpret_cast<float4*>(hin + base) = st;
      }
      if (hin_f32 != nullptr) {
        if constexpr (E::kBytes == 2) {
          float4 r;
          r.x = bf16_lo(pack_bf16x2(st.x, st.y)); r.y = bf16_hi(pack_bf16x2(st.x, st.y));
          r.z = bf16_lo(pack_bf16x2(st.z, st.w)); r.w = bf16_hi(pack_bf16x2(st.z, st.w));
          *reinterpret_cast<float4*>(hin_f32 + base) = r;
        } else {
          *reinterpret_cast<float4*>(hin_f32 + base) = st;
        }
      }
      st.x = dec[u] * st.x + sv[u].x;
      st.y = dec[u] * st.y + sv[u].y;
      st.z = dec[u] * st.z + sv[u].z;
      st.w = dec[u] * st.w + sv[u].w;
    }
  }
  for (; k < k1; ++k) {
    const int64_t base = ((int64_t)k * H + h) * PN + ch;
    const float4 sv = *reinterpret_cast<const float4*>(ws.states + base);
    const float dec = __expf(ws.lam[(int64_t)k * H + h]);
    if constexpr (E::kBytes == 2) {
      uint2 o;
      o.x = pack_bf16x2(st.x, st.y);
      o.y = pack_bf16x2(st.z, st.w);
      *reinterpret_cast<uint2*>(hin + base) = o;
      if (hin_f32 != nullptr) {
        float4 r;
        r.x = bf16_lo(o.x); r.y = bf16_hi(o.x); r.z = bf16_lo(o.y); r.w = bf16_hi(o.y);
        *reinterpret_cast<float4*>(hin_f32 + base) = r;
      }
    } else {
      *reinterpret_cast<float4*>(hin + base) = st;
      if (hin_f32 != nullptr) *reinterpret_cast<float4*>(hin_f32 + base) = st;
    }
    st.x = dec * st.x + sv.x;
    st.y = dec * st.y + sv.y;
    st.z = dec * st.z + sv.z;
    st.w = dec * st.w + sv.w;
  }
  if (p.final_state != nullptr)
    *reinterpret_cast<float4*>(p.final_state + (s * H + h) * (int64_t)PN + ch) = st;
}

hipError_t launch_state_pass_impl(const Problem& p, const Workspace& ws, float* hin_f32,
                                  hipStream_t s) {
  const int PN = p.P * p.N;
  const int64_t cblocks = (PN + 4 * kThreads - 1) / (4 * kThreads);
  const int64_t blocks = p.nseq * p.H * cblocks;
  if (blocks == 0) return hipSuccess;
  if (p.dtype == Dtype::BF16)
    hipLaunchKernelGGL(state_pass_kernel<Bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, ws, hin_f32);
  else
    hipLaunchKernelGGL(state_pass_kernel<F32>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, ws, hin_f32);
  return hipGetLastError();
}

hipError_t launch_state_pass(const Problem& p, const Workspace& ws, hipStream_t s) {
  return launch_state_pass_impl(p, ws, nullptr, s);
}

}  // namespace ssd
