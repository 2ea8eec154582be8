// k10_selective_scan.hip -- the comparator of the SSD layer: a selective scan
// with a diagonal transition (Mamba-1's S6 layer).
//
// Pages: [M] "LLM(十一)——Mamba" §3.1.1 (a structured SSM whose transition is
// diagonal, stored as its N diagonal entries), §3.1.2 (SSD keeps one scalar of
// that diagonal), §2.1.2-2.1.3 (one independent SSM per channel d of D; the
// step size Delta per token and channel; B and C per token, shared by the
// channels).  Per channel d and state entry n, from a zero state:
//     h_t[n] = exp(Delta_t[d] A[d][n]) h_{t-1}[n] + Delta_t[d] x_t[d] B_t[n]
//     y_t[d] = sum_n C_t[n] h_t[n]
// (the input enters as Delta x, the first-order term also used for the SSD
// path's dt-scaled input).  This exists to measure the pages' speed claim for
// SSD against the diagonal selective scan on the same GPU; it is not on the
// SSD path.
//
// Design (gfx950): with a diagonal transition every state entry has its own
// decay, so each (token, channel, entry) costs one exp on the vector ALU and
// nothing maps to the matrix cores.  One wave per (sequence, channel, block of
// 64 entries); lane n carries h[n] through all T tokens (one exp per element,
// the least any scan does; a chunk-parallel scan would need two).  Tokens are
// processed in blocks of 64: the wave loads the block's Delta and x (channel-
// major layout, one 64-token row each) and puts (Delta, Delta x) in LDS, where
// every lane reads token s's pair with one broadcast read;
// B_t and C_t are loaded per token as 64 consecutive entries.  Each lane keeps
// its C_t h_t for the 64 tokens in registers; a butterfly of 63 lane
// exchanges (none through LDS) then sums them over the lanes, leaving token s's
// partial sum in lane s, and the
// waves of one channel (N / 64 of them, in one workgroup) add theirs in LDS.
// Layouts: x, Delta, y (b, D, T) channel-major; A (D, N); B, C (b, T, N);
// final state (b, D, N) fp32.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kScanThreads = 256;
constexpr int kScanBlock = 64;  // tokens per block

template <class E>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
  if constexpr (E::kBytes == 2) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}
// y in the element dtype (bf16: round to nearest even)
template <class E>
__device__ __forceinline__ void st_y(void* p, int64_t i, float v) {
  if constexpr (E::kBytes == 2) reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  else reinterpret_cast<float*>(p)[i] = v;
}

// One butterfly stage: lanes with bit O set keep the upper half of v[0, 2 O)
// and add their partner's copy of it; the partner does the opposite.  No
// stage goes through LDS.  Distances 32 and 16 exchange whole 32- and 16-lane
// rows (v_permlane32_swap / v_permlane16_swap swap the upper row of their
// first operand with the lower row of their second, so after exchanging
// (v[i], v[O + i]) the two results add up to the pair's v[i] in the lower row
// and its v[O + i] in the upper); 8 is a row rotation, 4 two bank-masked row
// shifts, 2 and 1 quad permutations.  Every stage adds the same two values as
// a lane exchange would, so the sums do not depend on how they are moved.
template <int CTRL, int BM>
__device__ __forceinline__ float scan_dpp(float old, float v) {  // lanes of the banks in BM; the others keep old
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xf, BM, false));
}
template <int O>
__device__ __forceinline__ void sum_stage(float (&v)[kScanBlock], int lane) {
  const bool up = lane & O;
#pragma unroll
  for (int i = 0; i < O; ++i) {
    if constexpr (O == 32 || O == 16) {
      const auto sw = O == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[O + i]), false, false)
                              : __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[O + i]), false, false);
      v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    } else {
      const float keep = up ? v[O + i] : v[i];
      const float send = up ? v[i] : v[O + i];
      float recv;
      if constexpr (O == 8) recv = scan_dpp<0x128, 0xf>(0.0f, send);  // row_ror:8
      else if constexpr (O == 4) recv = scan_dpp<0x104, 0x5>(scan_dpp<0x114, 0xA>(0.0f, send), send);  // shr:4 / shl:4
      else if constexpr (O == 2) recv = scan_dpp<0x4E, 0xf>(0.0f, send);  // quad_perm [2, 3, 0, 1]
      else recv = scan_dpp<0xB1, 0xf>(0.0f, send);                         // quad_perm [1, 0, 3, 2]
      v[i] = keep + recv;
    }
  }
}

// v[s] summed over the 64 lanes; lane L returns the sum for s = L.
__device__ __forceinline__ float wave_sum_transpose(float (&v)[kScanBlock], int lane) {
  sum_stage<32>(v, lane);
  sum_stage<16>(v, lane);
  sum_stage<8>(v, lane);
  sum_stage<4>(v, lane);
  sum_stage<2>(v, lane);
  sum_stage<1>(v, lane);
  return v[0];
}

template <class E, int N>
__global__ __launch_bounds__(kScanThreads) void selective_scan_kernel(ScanProblem p) {
  constexpr int NB = N / 64;               // waves per channel
  constexpr int CPB = kScanThreads / N;    // channels per workgroup
  __shared__ float ysum[CPB][NB][kScanBlock];
  // per wave: the block's (Delta_t, Delta_t x_t), read by every lane as one
  // broadcast LDS read per token (the vector ALU then does no lane broadcasts)
  __shared__ float2 du_s[kScanThreads / 64][kScanBlock];
  const int wid = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int cl = wid / NB, nb = wid % NB;  // channel within the workgroup, entry block
  const int64_t chan = (int64_t)blockIdx.x * CPB + cl;  // (sequence, channel)
  const bool active = chan < p.batch * p.D;
  const int64_t b = active ? chan / p.D : 0;
  const int64_t d = active ? chan % p.D : 0;
  const int n = nb * 64 + lane;
  const int64_t T = p.seqlen;
  const float a2 = p.A[d * N + n] * kLog2e;  // exp(Delta A) = 2^(Delta A log2 e)
  const float* drow = p.delta + (b * p.D + d) * T;
  const int64_t xrow = (b * p.D + d) * T;
  const int64_t bc0 = b * T * N + n;
  float h = 0.0f;
  auto lane_val = [](float v, int s) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s)); };
  // y of one block: this wave's partial sums, then the channel's waves added
  auto finish = [&](float (&yp)[kScanBlock], int64_t t0, int nt) {
    const float ys = wave_sum_transpose(yp, lane);  // token t0 + lane, this wave's entries
    if constexpr (NB == 1) {
      if (active && lane < nt) st_y<E>(p.y, xrow + t0 + lane, ys);
    } else {
      ysum[cl][nb][lane] = ys;
      __syncthreads();
      if (nb == 0 && active && lane < nt) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NB; ++k) acc += ysum[cl][k][lane];
        st_y<E>(p.y, xrow + t0 + lane, acc);
      }
      __syncthreads();
    }
  };
  constexpr int SB = 16;  // tokens whose B and C are loaded together
  const int64_t Tfull = T / kScanBlock * kScanBlock;
  for (int64_t t0 = 0; t0 < Tfull; t0 += kScanBlock) {
    // whole block: straight-line code; B and C one sub-block ahead
    {
      const float dl = drow[t0 + lane];
      du_s[wid][lane] = make_float2(dl, dl * ld_elem<E>(p.x, xrow + t0 + lane));
    }
    float yp[kScanBlock];
    float bq[SB], cq[SB];
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      bq[s] = ld_elem<E>(p.B, bc0 + (t0 + s) * N);
      cq[s] = ld_elem<E>(p.C, bc0 + (t0 + s) * N);
    }
#pragma unroll
    for (int sb = 0; sb < kScanBlock / SB; ++sb) {
      float bn[SB], cn[SB];
      if (sb + 1 < kScanBlock / SB) {
#pragma unroll
        for (int s = 0; s < SB; ++s) {
          bn[s] = ld_elem<E>(p.B, bc0 + (t0 + (sb + 1) * SB + s) * N);
          cn[s] = ld_elem<E>(p.C, bc0 + (t0 + (sb + 1) * SB + s) * N);
        }
      }
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int k = sb * SB + s;
        const float2 du = du_s[wid][k];  // (written above by this wave; LDS is in order per wave)
        h = __builtin_amdgcn_exp2f(du.x * a2) * h + du.y * bq[s];
        yp[k] = cq[s] * h;
      }
      if (sb + 1 < kScanBlock / SB) {
#pragma unroll
        for (int s = 0; s < SB; ++s) bq[s] = bn[s], cq[s] = cn[s];
      }
    }
    finish(yp, t0, kScanBlock);
  }
  if (Tfull < T) {
    // ragged last block
    const int64_t t0 = Tfull;
    const int nt = (int)(T - t0);
    const float dl = lane < nt ? drow[t0 + lane] : 0.0f;
    const float ul = lane < nt ? dl * ld_elem<E>(p.x, xrow + t0 + lane) : 0.0f;
    float yp[kScanBlock];
#pragma unroll
    for (int s = 0; s < kScanBlock; ++s) {
      if (s < nt) {
        const int64_t o = bc0 + (t0 + s) * N;
        h = __builtin_amdgcn_exp2f(lane_val(dl, s) * a2) * h + lane_val(ul, s) * ld_elem<E>(p.B, o);
        yp[s] = ld_elem<E>(p.C, o) * h;
      } else {
        yp[s] = 0.0f;
      }
    }
    finish(yp, t0, nt);
  }
  if (active && p.final_state != nullptr) p.final_state[(b * p.D + d) * N + n] = h;
}

template <class E>
static hipError_t launch_scan_e(const ScanProblem& p, hipStream_t s) {
  const int64_t chans = p.batch * p.D;
  const int cpb = kScanThreads / p.N;
  const dim3 grid((unsigned)((chans + cpb - 1) / cpb)), block(kScanThreads);
  switch (p.N) {
    case 64: hipLaunchKernelGGL((selective_scan_kernel<E, 64>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((selective_scan_kernel<E, 128>), grid, block, 0, s, p); break;
    case 256: hipLaunchKernelGGL((selective_scan_kernel<E, 256>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_selective_scan(const ScanProblem& p, hipStream_t s) {
  if (p.batch * p.D == 0) return hipSuccess;
  return p.dtype == Dtype::BF16 ? launch_scan_e<Bf16>(p, s) : launch_scan_e<F32>(p, s);
}

}  // namespace ssd
