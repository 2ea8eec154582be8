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
// nothing maps to the matrix cores.  One wave per (sequence, channel); lane l
// carries the N / 64 entries n = l, l + 64, ... through all T tokens (one exp
// per element, the least any scan does; a chunk-parallel scan would need two)
// and forms its part of C_t h_t over them.  A workgroup of 8 waves holds 8
// channels of one sequence, which share B and C: each sub-block of 4096 / N
// tokens of them is loaded once by the workgroup (16-byte vectors), converted
// to fp32 and stored in LDS as (B_t[n], C_t[n]) pairs, double buffered (the
// next sub-block's loads in flight during this one's products), and each lane
// reads a pair with one 8-byte LDS read: no global load and no conversion per
// element.  Tokens are processed in blocks of 64: the wave loads the block's
// Delta and x (channel-major layout, one 64-token row each) and puts
// (Delta, Delta x) in LDS, where every lane reads token s's pair with one
// broadcast read.  Each lane keeps its part of C_t h_t for the 64 tokens in
// registers; a butterfly of 63 lane exchanges (none through LDS) then sums
// them over the lanes, leaving token s's y in lane s.  Per element that leaves
// Delta A, the exp, the input term, the state update and C h on the vector
// ALU, 2.5 / (N / 64) butterfly operations, and 8 bytes of LDS reads.
// Measured slower and not kept: one wave per 64 entries (16 waves of 8
// channels per workgroup, the waves of a channel adding their parts in LDS),
// a transposed sum through LDS instead of the butterfly (LDS traffic), the
// staged pairs kept as bf16 (two conversions per element).
// Layouts: x, Delta, y (b, D, T) channel-major; A (D, N); B, C (b, T, N);
// final state (b, D, N) fp32.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kScanThreads = 512;   // 8 waves
constexpr int kScanBlock = 64;     // tokens per block
constexpr int kScanStaged = 4096;  // (token, entry) pairs of B and C staged at once

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

// Staged B and C: the workgroup's channels share one batch, so each sub-block of
// SB tokens is loaded once, converted to fp32 and stored as (B_t[n], C_t[n])
// pairs in LDS; every lane then reads its pair with one 8-byte LDS read.  Each
// thread stages RPT runs of VEC consecutive entries of one token (a 16-byte
// vector of B and one of C when kVec, else element loads), each written as two
// pairs per 16-byte LDS store.  The loads keep raw bits (converted at the store, so a
// load in flight is not waited for before the products it overlaps); tokens
// at or past T stage zeros.
__device__ __forceinline__ uint32_t raw_bits(uint16_t v) { return v; }
__device__ __forceinline__ uint32_t raw_bits(float v) { return __float_as_uint(v); }

template <class E, int N, bool kVec>
struct ScanStage {
  static constexpr int VEC = 16 / E::kBytes;     // entries per vector
  static constexpr int SB = kScanStaged / N;     // tokens per sub-block
  static constexpr int POS = kScanStaged / VEC;  // vectors per sub-block
  static constexpr int RPT = (POS + kScanThreads - 1) / kScanThreads;  // per thread
  static_assert(POS % kScanThreads == 0 || POS < kScanThreads, "staging split");
  static_assert(SB * N == kScanStaged && kScanBlock % SB == 0, "staging split");
  static constexpr int W = kVec ? 4 : VEC;       // raw 32-bit words per matrix
  uint32_t rb[RPT][W], rc[RPT][W];
  __device__ __forceinline__ void load(const ScanProblem& p, int64_t b, int64_t t0, int tid) {
    using S = typename E::storage;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int v = tid + r * kScanThreads;
      const int e0 = v * VEC, s = e0 / N, n0 = e0 % N;
      const int64_t t = t0 + s;
      const bool in = v < POS && t < p.seqlen;
      const int64_t o = (b * p.seqlen + (in ? t : 0)) * N + n0;
      if constexpr (kVec) {
        uint4 vb = make_uint4(0, 0, 0, 0), vc = vb;
        if (in) {
          vb = *reinterpret_cast<const uint4*>(reinterpret_cast<const S*>(p.B) + o);
          vc = *reinterpret_cast<const uint4*>(reinterpret_cast<const S*>(p.C) + o);
        }
        rb[r][0] = vb.x; rb[r][1] = vb.y; rb[r][2] = vb.z; rb[r][3] = vb.w;
        rc[r][0] = vc.x; rc[r][1] = vc.y; rc[r][2] = vc.z; rc[r][3] = vc.w;
      } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          rb[r][k] = in ? raw_bits(reinterpret_cast<const S*>(p.B)[o + k]) : 0u;
          rc[r][k] = in ? raw_bits(reinterpret_cast<const S*>(p.C)[o + k]) : 0u;
        }
      }
    }
  }
  __device__ __forceinline__ float val(const uint32_t (&r)[W], int k) const {
    if constexpr (kVec && E::kBytes == 2) return k & 1 ? bf16_hi(r[k / 2]) : bf16_lo(r[k / 2]);
    else if constexpr (E::kBytes == 2) return __uint_as_float(r[k] << 16);
    else return __uint_as_float(r[k]);
  }
  __device__ __forceinline__ void store(float4* buf, int tid) const {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int v = tid + r * kScanThreads;
      if (v >= POS) break;
#pragma unroll
      for (int k = 0; k < VEC; k += 2)
        buf[(v * VEC + k) / 2] = make_float4(val(rb[r], k), val(rc[r], k), val(rb[r], k + 1), val(rc[r], k + 1));
    }
  }
};

template <class E, int N, bool kVec>
__global__ __launch_bounds__(kScanThreads) void selective_scan_kernel(ScanProblem p, int dblocks) {
  using St = ScanStage<E, N, kVec>;
  constexpr int EN = N / 64;                 // state entries per lane
  constexpr int CPB = kScanThreads / 64;     // channels per workgroup, one wave each
  constexpr int SB = St::SB, NSB = kScanBlock / SB;
  // per wave: the block's (Delta_t, Delta_t x_t), read by every lane as one
  // broadcast LDS read per token (the vector ALU then does no lane broadcasts)
  __shared__ float2 du_s[CPB][kScanBlock];
  __shared__ float4 bc_s[2][kScanStaged / 2];  // (B, C) pairs of a sub-block, double buffered
  const int tid = threadIdx.x;
  const int wid = tid / 64, lane = tid % 64;
  const int64_t b = blockIdx.x / dblocks;
  const int64_t d = (int64_t)(blockIdx.x % dblocks) * CPB + wid;
  const bool active = d < p.D;
  const int64_t dc = active ? d : 0;
  const int64_t T = p.seqlen;
  float a2[EN], h[EN];
#pragma unroll
  for (int e = 0; e < EN; ++e) a2[e] = p.A[dc * N + e * 64 + lane] * kLog2e, h[e] = 0.0f;
  const float* drow = p.delta + (b * p.D + dc) * T;
  const int64_t xrow = (b * p.D + dc) * T;
  const float2* bcf = reinterpret_cast<const float2*>(&bc_s[0][0]);
  St st;
  if (T > 0) {
    st.load(p, b, 0, tid);
    st.store(bc_s[0], tid);
  }
  __syncthreads();
  // blocks of 64 tokens; a ragged last block runs whole on zero Delta, B and
  // C past T (decay 1, no input: the state is unchanged) and stores nt outputs
  int64_t sub = 0;  // the sub-block being computed: its pairs are in buffer sub & 1
  for (int64_t t0 = 0; t0 < T; t0 += kScanBlock) {
    const int nt = (int)(T - t0 < kScanBlock ? T - t0 : kScanBlock);
    {
      const bool in = active && lane < nt;
      const float dl = in ? drow[t0 + lane] : 0.0f;
      du_s[wid][lane] = make_float2(dl, in ? dl * ld_elem<E>(p.x, xrow + t0 + lane) : 0.0f);
    }
    float yp[kScanBlock];
#pragma unroll
    for (int j = 0; j < NSB; ++j, ++sub) {
      // the next sub-block: staged within this block always (zeros past T),
      // the next block's first only when it exists
      const int64_t tn = t0 + (j + 1) * SB;
      const bool next = j + 1 < NSB || tn < T;
      if (next) st.load(p, b, tn, tid);
      const float2* cur = bcf + (sub & 1) * kScanStaged;
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int k = j * SB + s;
        const float2 du = du_s[wid][k];  // (written above by this wave; LDS is in order per wave)
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EN; ++e) {
          const float2 bc = cur[s * N + e * 64 + lane];
          h[e] = __builtin_amdgcn_exp2f(du.x * a2[e]) * h[e] + du.y * bc.x;
          acc = e == 0 ? bc.y * h[e] : acc + bc.y * h[e];
        }
        yp[k] = acc;
        // formed here: left to the compiler, the products sink below the
        // barriers to the block's end, every pair read kept live until then
        asm volatile("" : "+v"(yp[k]));
      }
      if (next) st.store(bc_s[(sub + 1) & 1], tid);
      __syncthreads();
    }
    const float ys = wave_sum_transpose(yp, lane);  // token t0 + lane
    if (active && lane < nt) st_y<E>(p.y, xrow + t0 + lane, ys);
  }
  if (active && p.final_state != nullptr)
#pragma unroll
    for (int e = 0; e < EN; ++e) p.final_state[(b * p.D + d) * N + e * 64 + lane] = h[e];
}

template <class E, int N>
static hipError_t launch_scan_n(const ScanProblem& p, hipStream_t s) {
  constexpr int CPB = kScanThreads / 64;
  const int64_t dblocks = (p.D + CPB - 1) / CPB;
  const dim3 grid((unsigned)(p.batch * dblocks)), block(kScanThreads);
  // 16-byte staging loads need 16-byte aligned B and C (every row offset is a
  // multiple of N entries, itself a multiple of the vector)
  if (((reinterpret_cast<uintptr_t>(p.B) | reinterpret_cast<uintptr_t>(p.C)) & 15) == 0)
    hipLaunchKernelGGL((selective_scan_kernel<E, N, true>), grid, block, 0, s, p, (int)dblocks);
  else
    hipLaunchKernelGGL((selective_scan_kernel<E, N, false>), grid, block, 0, s, p, (int)dblocks);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_scan_e(const ScanProblem& p, hipStream_t s) {
  switch (p.N) {
    case 64: return launch_scan_n<E, 64>(p, s);
    case 128: return launch_scan_n<E, 128>(p, s);
    case 256: return launch_scan_n<E, 256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_selective_scan(const ScanProblem& p, hipStream_t s) {
  if (p.batch * p.D == 0) return hipSuccess;
  return p.dtype == Dtype::BF16 ? launch_scan_e<Bf16>(p, s) : launch_scan_e<F32>(p, s);
}

}  // namespace ssd
