// k25_chunk_output.hip -- diagonal blocks fused with the state-to-output
// product of the SSD block decomposition (K2 + K5).
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba):
//   §3.5.1 Diagonal blocks / step 1: within a chunk, from a zero state, the
//     dual (quadratic, attention-like) form Y_diag = (L o C B^T) X with
//     L[i, j] = exp(Acs_i - Acs_j) for j <= i, else 0;
//   §3.5.2 Left factors / step 4: the passed state's contribution
//     Y_off[i] = exp(Acs_i) * (Hin . C_i), a (Q x N) . (N x P) product;
//   y = Y_diag + Y_off.
// [T] "Transformers是SSMs…(一)" (nxbn.cn) §2.4 gives the same dual form for the
// whole sequence.
//
// Design (gfx950), one workgroup of 4 waves per (chunk, head), ordered so that
// the heads of one chunk share an XCD's L2 for the chunk's B and C tiles:
//  * The output is built transposed, Y^T (P x Q), on 32x32 MFMA tiles.  The
//    kernel tile G^T = B_J C_I^T (32 x 32, contraction over N) then leaves each
//    lane holding ONE output token i and 16 input tokens j, which is exactly
//    the register layout of the B operand of the next product
//    Y^T += X^T (L o G)^T: the masked tile never leaves the registers (no LDS
//    round trip), and the K (token) order of that product is chosen to match.
//  * Causality: only tiles J <= I are formed.  Below the diagonal the mask
//    factors as L[i,j] = exp(Acs_i - Acs_e) * exp(Acs_e - Acs_j) with e the last
//    token of tile J: one exp per lane per tile plus a per-token table, both
//    factors in (0, 1] (no overflow); only the 32x32 diagonal tiles take an exp
//    per element and a select for j > i (a true 0, never exp(-inf) arithmetic).
//  * Y_off uses the same lane layout: Hin (P x N, element dtype) is the A
//    operand, the C rows of the lane's token the B operand, and the per-token
//    factor exp(Acs_i) is one scalar per lane.
//  * Operands: B (Q x N) and Hin (P x N) staged row-major in LDS, X staged
//    transposed (P x Q) in LDS, the lane's C row in registers for the whole
//    row tile.  fp32 accumulation; y rounded once to the element dtype.
#include "ssd_stage.hpp"

namespace ssd {

template <class E, int Q, int N>
struct ChunkOutputCfg {
  using T = typename E::storage;
  static constexpr int P = kHeadDim;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int NP = N + PAD;  // LDS pitch of B and Hin rows
  static constexpr int QP = Q + PAD;  // LDS pitch of X^T rows
  static constexpr size_t lds_bytes =
      ((size_t)Q * NP + (size_t)P * QP + (size_t)P * NP) * sizeof(T) + 2 * Q * sizeof(float);
  static constexpr bool fits = lds_bytes <= (size_t)kLdsLimit;
};

template <class E, int Q, int N>
__global__ __launch_bounds__(kThreads) void chunk_output_kernel(Problem p, Workspace ws) {
  using Cfg = ChunkOutputCfg<E, Q, N>;
  using T = typename E::storage;
  constexpr int P = Cfg::P, NP = Cfg::NP, QP = Cfg::QP;
  constexpr bool kBf16 = E::kBytes == 2;
  __shared__ __attribute__((aligned(16))) T Bs[Q * NP];
  __shared__ __attribute__((aligned(16))) T XT[P * QP];
  __shared__ __attribute__((aligned(16))) T Hs[P * NP];
  __shared__ float acs_s[Q];
  __shared__ float w_s[Q];

  const int H = p.H;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t k = lid / H;
  const int h = lid % H;
  const ChunkDesc cd = ws.chunks[k];
  if (cd.seq < 0) return;
  const int L = cd.len;
  const int G = p.G;
  const int g = h / (H / G);
  const int tid = threadIdx.x;

  // per-token tables: Acs and the below-diagonal column factor
  // w_j = exp(Acs_e - Acs_j), e = last token of j's 32-token tile
  const float* acs = ws.acs + (k * H + h) * Q;
  for (int l = tid; l < Q; l += kThreads) {
    const float a = acs[l];
    acs_s[l] = a;
    w_s[l] = __expf(acs[l | 31] - a);
  }
  const T* xg = reinterpret_cast<const T*>(p.x) + (cd.t0 * H + h) * P;
  const T* bg = reinterpret_cast<const T*>(p.B) + (cd.t0 * G + g) * N;
  const T* hg = reinterpret_cast<const T*>(ws.hin) + (k * H + h) * (int64_t)(P * N);
  stage_rows<E, Q, N, NP>(Bs, bg, (int64_t)G * N, L);
  stage_rows<E, P, N, NP>(Hs, hg, N, P);
  stage_transposed<E, Q, P, QP, false>(XT, xg, (int64_t)H * P, L, nullptr);
  __syncthreads();

  const int wid = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lg = lane >> 5;
  const int nI = (L + 31) / 32;
  const T* cg = reinterpret_cast<const T*>(p.C) + (cd.t0 * G + g) * N;
  T* yg = reinterpret_cast<T*>(p.y) + (cd.t0 * H + h) * P;

  // row tiles of 32 output tokens; wave w takes tiles {w, 7-w} of every 8
  // (balanced causal work: tile I costs I+1 kernel tiles)
  for (int tb = 0; tb < nI; tb += 8) {
    for (int half = 0; half < 2; ++half) {
      const int I = tb + (half == 0 ? wid : 7 - wid);
      if (I >= nI) continue;
      const int i_loc = I * 32 + lr;
      const bool row_ok = i_loc < L;
      // C row of this lane's token, as MFMA B-operand slices over N
      constexpr int KS = N / E::kMfmaK;
      using CReg = typename std::conditional<kBf16, uint4, float>::type;
      CReg creg[KS > 0 ? KS : 1];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (kBf16) {
          creg[ks] = row_ok ? *reinterpret_cast<const uint4*>(cg + (int64_t)i_loc * G * N + ks * 16 + lg * 8)
                            : make_uint4(0, 0, 0, 0);
        } else {
          creg[ks] = row_ok ? cg[(int64_t)i_loc * G * N + ks * 2 + lg] : 0.0f;
        }
      }
      floatx16_t acc0 = zero16(), acc1 = zero16();
      // Y_off^T = Hin C^T (contraction over N), then the exp(Acs_i) factor
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (kBf16) {
          const uint4 a0 = *reinterpret_cast<const uint4*>(Hs + lr * NP + ks * 16 + lg * 8);
          const uint4 a1 = *reinterpret_cast<const uint4*>(Hs + (32 + lr) * NP + ks * 16 + lg * 8);
          acc0 = mfma32x32x16(a0, creg[ks], acc0);
          acc1 = mfma32x32x16(a1, creg[ks], acc1);
        } else {
          acc0 = mfma32x32x2(Hs[lr * NP + ks * 2 + lg], creg[ks], acc0);
          acc1 = mfma32x32x2(Hs[(32 + lr) * NP + ks * 2 + lg], creg[ks], acc1);
        }
      }
      const float ai = acs_s[i_loc];
      const float eo = __expf(ai);
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc0[r] *= eo; acc1[r] *= eo; }

      // diagonal block: kernel tiles J <= I
      for (int J = 0; J <= I; ++J) {
        floatx16_t gt = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (kBf16) {
            const uint4 b = *reinterpret_cast<const uint4*>(Bs + (J * 32 + lr) * NP + ks * 16 + lg * 8);
            gt = mfma32x32x16(b, creg[ks], gt);
          } else {
            gt = mfma32x32x2(Bs[(J * 32 + lr) * NP + ks * 2 + lg], creg[ks], gt);
          }
        }
        // gt[r] = G[i_loc][j_r], j_r = 32J + 8(r/4) + 4 lg + r%4
        float v[16];
        if (J < I) {
          const float u = __expf(ai - acs_s[J * 32 + 31]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 w4 = *reinterpret_cast<const float4*>(w_s + J * 32 + q * 8 + lg * 4);
            v[4 * q + 0] = gt[4 * q + 0] * (u * w4.x);
            v[4 * q + 1] = gt[4 * q + 1] * (u * w4.y);
            v[4 * q + 2] = gt[4 * q + 2] * (u * w4.z);
            v[4 * q + 3] = gt[4 * q + 3] * (u * w4.w);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = J * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
            const float m = __expf(ai - acs_s[j]);
            v[r] = (j <= i_loc) ? gt[r] * m : 0.0f;
          }
        }
        // Y^T += X^T (L o G)^T over the 32 tokens of tile J
        if constexpr (kBf16) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            uint4 bop;
            bop.x = pack_bf16x2(v[8 * kk + 0], v[8 * kk + 1]);
            bop.y = pack_bf16x2(v[8 * kk + 2], v[8 * kk + 3]);
            bop.z = pack_bf16x2(v[8 * kk + 4], v[8 * kk + 5]);
            bop.w = pack_bf16x2(v[8 * kk + 6], v[8 * kk + 7]);
            const int col = J * 32 + kk * 16 + lg * 4;
            const uint2 lo0 = *reinterpret_cast<const uint2*>(XT + lr * QP + col);
            const uint2 hi0 = *reinterpret_cast<const uint2*>(XT + lr * QP + col + 8);
            const uint2 lo1 = *reinterpret_cast<const uint2*>(XT + (32 + lr) * QP + col);
            const uint2 hi1 = *reinterpret_cast<const uint2*>(XT + (32 + lr) * QP + col + 8);
            acc0 = mfma32x32x16(make_uint4(lo0.x, lo0.y, hi0.x, hi0.y), bop, acc0);
            acc1 = mfma32x32x16(make_uint4(lo1.x, lo1.y, hi1.x, hi1.y), bop, acc1);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = J * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
            acc0 = mfma32x32x2(XT[lr * QP + j], v[r], acc0);
            acc1 = mfma32x32x2(XT[(32 + lr) * QP + j], v[r], acc1);
          }
        }
      }
      // store: lane holds y[i_loc][p] for p = 32 pt + 8(r/4) + 4 lg + r%4
      if (row_ok) {
        T* yrow = yg + (int64_t)i_loc * H * P;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int pp = q * 8 + lg * 4;
          if constexpr (kBf16) {
            uint2 o0, o1;
            o0.x = pack_bf16x2(acc0[4 * q + 0], acc0[4 * q + 1]);
            o0.y = pack_bf16x2(acc0[4 * q + 2], acc0[4 * q + 3]);
            o1.x = pack_bf16x2(acc1[4 * q + 0], acc1[4 * q + 1]);
            o1.y = pack_bf16x2(acc1[4 * q + 2], acc1[4 * q + 3]);
            *reinterpret_cast<uint2*>(yrow + pp) = o0;
            *reinterpret_cast<uint2*>(yrow + 32 + pp) = o1;
          } else {
            *reinterpret_cast<float4*>(yrow + pp) =
                make_float4(acc0[4 * q + 0], acc0[4 * q + 1], acc0[4 * q + 2], acc0[4 * q + 3]);
            *reinterpret_cast<float4*>(yrow + 32 + pp) =
                make_float4(acc1[4 * q + 0], acc1[4 * q + 1], acc1[4 * q + 2], acc1[4 * q + 3]);
          }
        }
      }
    }
  }
}

template <class E, int Q, int N>
static hipError_t launch_co(const Problem& p, const Workspace& ws, hipStream_t s) {
  if constexpr (ChunkOutputCfg<E, Q, N>::fits) {
    const unsigned blocks = (unsigned)(p.kmax * p.H);
    hipLaunchKernelGGL((chunk_output_kernel<E, Q, N>), dim3(blocks), dim3(kThreads), 0, s, p, ws);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <class E, int Q>
static hipError_t launch_co_n(const Problem& p, const Workspace& ws, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_co<E, Q, 16>(p, ws, s);
    case 32: return launch_co<E, Q, 32>(p, ws, s);
    case 64: return launch_co<E, Q, 64>(p, ws, s);
    case 128: return launch_co<E, Q, 128>(p, ws, s);
    case 256: return launch_co<E, Q, 256>(p, ws, s);
  }
  return hipErrorInvalidValue;
}

template <class E>
static hipError_t launch_co_q(const Problem& p, const Workspace& ws, hipStream_t s) {
  switch (p.Q) {
    case 64: return launch_co_n<E, 64>(p, ws, s);
    case 128: return launch_co_n<E, 128>(p, ws, s);
    case 256: return launch_co_n<E, 256>(p, ws, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_output(const Problem& p, const Workspace& ws, hipStream_t s) {
  return p.dtype == Dtype::BF16 ? launch_co_q<Bf16>(p, ws, s) : launch_co_q<F32>(p, ws, s);
}

bool chunk_output_supported(Dtype dt, int Q, int N) {
#define SSD_CO_CASE(QQ, NN)                                                       \
  if (Q == QQ && N == NN)                                                         \
    return dt == Dtype::BF16 ? ChunkOutputCfg<Bf16, QQ, NN>::fits : ChunkOutputCfg<F32, QQ, NN>::fits;
  SSD_CO_CASE(64, 16) SSD_CO_CASE(64, 32) SSD_CO_CASE(64, 64) SSD_CO_CASE(64, 128) SSD_CO_CASE(64, 256)
  SSD_CO_CASE(128, 16) SSD_CO_CASE(128, 32) SSD_CO_CASE(128, 64) SSD_CO_CASE(128, 128) SSD_CO_CASE(128, 256)
  SSD_CO_CASE(256, 16) SSD_CO_CASE(256, 32) SSD_CO_CASE(256, 64) SSD_CO_CASE(256, 128) SSD_CO_CASE(256, 256)
#undef SSD_CO_CASE
  return false;
}

}  // namespace ssd
