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
// Design (gfx950):
//  * One workgroup of 8 waves (two per SIMD, so one wave's VALU and LDS work
//    overlaps the other's MFMAs) per (chunk, block of HB heads of one B/C
//    group).  Waves w and w+4 own the same two row tiles of 32 output tokens
//    and split the 64 output channels in halves; both form the kernel tile
//    G^T they share (duplicated MFMA work bought for latency hiding).
//    The chunk's B tile is staged in LDS once and each wave's C rows are held
//    in registers once, for all HB heads; the x tile and passed state of the
//    next head are loaded into registers while the current head computes, so
//    their HBM latency is hidden behind MFMA work.  Blocks are ordered so that
//    the head blocks of one chunk land on one XCD and share its L2.
//  * The output is built transposed, Y^T (P x Q), on 32x32 MFMA tiles.  The
//    kernel tile G^T = B_J C_I^T (32 x 32, contraction over N) leaves each lane
//    holding ONE output token i and 16 input tokens j, which is exactly the
//    register layout of the B operand of the next product Y^T += X^T (L o G)^T:
//    the masked tile never leaves the registers, and the K (token) order of
//    that product is chosen to match.
//  * Causality: only tiles J <= I are formed.  The mask factors as
//    L[i,j] = exp(Acs_i - Acs_e) * exp(Acs_e - Acs_j), e the last token of j's
//    32-token tile.  The second factor w_j (in (0, 1]) scales x when it is
//    staged in LDS, once per head; the first is one exp per lane per tile, in
//    (0, 1] below the diagonal.  On a diagonal tile it is >= 1 and bounded by
//    the tile's own decay, so this form is used only while no tile decays by
//    more than e^64; otherwise the head takes the exact path: x staged as is,
//    the first factor times a w_j table below the diagonal and one exp per
//    element on the diagonal.  Entries with j > i are a selected 0 (never
//    exp(-inf) arithmetic).
//  * Y_off uses the same lane layout: Hin (P x N, element dtype) is the A
//    operand, the lane's C row the B operand, exp(Acs_i) one scalar per lane.
//  * fp32 accumulation; y rounded once to the element dtype.
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
  static constexpr int KS = N / E::kMfmaK;                  // MFMA steps over N
  static constexpr int CREG = E::kBytes == 2 ? KS * 4 : KS; // VGPRs of one row tile's C operand
  static constexpr bool kKeepC = 2 * CREG <= 64;            // keep both row tiles' C across heads
};

constexpr int kOutThreads = 512;  // 8 waves: two per SIMD

template <class E, int Q, int N>
__global__ __launch_bounds__(kOutThreads) void chunk_output_kernel(Problem p, Workspace ws, int HB) {
  using Cfg = ChunkOutputCfg<E, Q, N>;
  using T = typename E::storage;
  constexpr int P = Cfg::P, NP = Cfg::NP, QP = Cfg::QP, KS = Cfg::KS;
  constexpr bool kBf16 = E::kBytes == 2;
  constexpr int NI = Q / 32;  // row tiles of the chunk
  constexpr int NTHR = kOutThreads;
  using CReg = typename std::conditional<kBf16, uint4, float>::type;
  __shared__ __attribute__((aligned(16))) T Bs[Q * NP];
  __shared__ __attribute__((aligned(16))) T XT[P * QP];
  __shared__ __attribute__((aligned(16))) T Hs[P * NP];
  __shared__ __attribute__((aligned(16))) float acs_s[Q];
  __shared__ __attribute__((aligned(16))) float w_s[Q];

  const int H = p.H, G = p.G;
  const int nhb = H / HB;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t k = lid / nhb;
  const int h0 = (lid % nhb) * HB;
  const ChunkDesc cd = chunk_desc(p, ws, k);
  if (cd.seq < 0) return;
  const int L = cd.len;
  const int g = h0 / (H / G);
  const int tid = threadIdx.x;
  const int wid = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lg = lane >> 5;
  const int pt = wid >> 2;  // this wave's 32 output channels p: [32 pt, 32 pt + 32)
  const int wq = wid & 3;   // this wave's row tiles: wq and 7 - wq
  const int nI = (L + 31) / 32;

  const T* xbase = reinterpret_cast<const T*>(p.x) + cd.t0 * H * P;
  const T* bg = reinterpret_cast<const T*>(p.B) + (cd.t0 * G + g) * N;
  const T* cg = reinterpret_cast<const T*>(p.C) + (cd.t0 * G + g) * N;
  const T* hbase = reinterpret_cast<const T*>(ws.hin) + k * H * (int64_t)(P * N);
  const float* abase = ws.acs + k * H * Q;
  T* ybase = reinterpret_cast<T*>(p.y) + cd.t0 * H * P;

  // row tiles of this wave: wq and 7-wq (balanced causal work: tile I costs
  // I+1 kernel tiles); chunks of 64 or 128 tokens have 2 or 4 row tiles
  constexpr int NT = NI == 8 ? 2 : 1;
  auto row_tile = [&](int t) { return t == 0 ? wq : 7 - wq; };

  // C rows of this wave's tokens as MFMA B-operand slices over N
  auto load_c = [&](int I, CReg (&c)[KS]) {
    const int i_loc = I * 32 + lr;
    const bool ok = i_loc < L;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (kBf16)
        c[ks] = ok ? *reinterpret_cast<const uint4*>(cg + (int64_t)i_loc * G * N + ks * 16 + lg * 8)
                   : make_uint4(0, 0, 0, 0);
      else
        c[ks] = ok ? cg[(int64_t)i_loc * G * N + ks * 2 + lg] : 0.0f;
    }
  };
  CReg ckeep[NT][KS];

  // ---- prologue: B tile, C rows, first head's x / state / cumsum
  {
    RowTile<E, Q, N, NTHR> bt;
    bt.load(bg, (int64_t)G * N, L);
    bt.template store<NP>(Bs);
  }
  if constexpr (Cfg::kKeepC) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (row_tile(t) < nI) load_c(row_tile(t), ckeep[t]);
  }
  TransTile<E, Q, P, NTHR> xt;
  RowTile<E, P, N, NTHR> ht;
  float a_own = 0.f, a_end = 0.f;
  auto prefetch = [&](int h) {
    xt.load(xbase + h * P, (int64_t)H * P, L);
    ht.load(hbase + h * (int64_t)(P * N), N, P);
    if (tid < Q) {
      a_own = abase[h * Q + tid];
      a_end = abase[h * Q + (tid | 31)];
    }
  };
  prefetch(h0);

  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    lds_barrier();  // every wave is done with the previous head's tiles
    ht.template store<NP>(Hs);
    if (tid < Q) {
      acs_s[tid] = a_own;
      w_s[tid] = __expf(a_end - a_own);  // exp(Acs_e - Acs_j), e = end of j's tile
    }
    lds_barrier();
    // Fast path when no 32-token tile decays by more than e^64: then x is
    // staged pre-scaled by w_j and the mask needs no per-element exp (see the
    // header); otherwise x is staged as is and every mask entry is exact.
    float dmax = 0.0f;
#pragma unroll
    for (int J = 0; J < NI; ++J) dmax = fmaxf(dmax, acs_s[J * 32] - acs_s[J * 32 + 31]);
    const bool fast = dmax <= 64.0f;
    if (fast)
      xt.template store<QP, true, kBf16>(XT, w_s);
    else
      xt.template store<QP, false, kBf16>(XT, nullptr);
    lds_barrier();
    if (hh + 1 < HB) prefetch(h + 1);

#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int I = row_tile(t);
      if (I >= nI) continue;
      const int i_loc = I * 32 + lr;
      CReg cfresh[KS];
      if constexpr (!Cfg::kKeepC) load_c(I, cfresh);
      const CReg (&creg)[KS] = Cfg::kKeepC ? ckeep[t] : cfresh;
      floatx16_t acc = zero16();
      // Y_off^T = Hin C^T (contraction over N), then the exp(Acs_i) factor
      const T* hrow = Hs + (pt * 32 + lr) * NP;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (kBf16)
          acc = mfma32x32x16(*reinterpret_cast<const uint4*>(hrow + ks * 16 + lg * 8), creg[ks], acc);
        else
          acc = mfma32x32x2(hrow[ks * 2 + lg], creg[ks], acc);
      }
      const float ai = acs_s[i_loc];
      const float eo = __expf(ai);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] *= eo;

      // diagonal block: kernel tiles J <= I
      const T* xrow = XT + (pt * 32 + lr) * QP;
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
        if (fast) {
          // x^T already carries w_j = exp(Acs_e - Acs_j); the lane factor is
          // exp(Acs_i - Acs_e) (<= 1 below the diagonal, <= e^64 on it)
          const float u = __expf(ai - acs_s[J * 32 + 31]);
          if (J < I) {
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = gt[r] * u;
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int jr = (r >> 2) * 8 + lg * 4 + (r & 3);  // j - 32J
              v[r] = (jr <= lr) ? gt[r] * u : 0.0f;
            }
          }
        } else if (J < I) {
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
            // tokens are permuted within 16-groups: this lane group's 8 are contiguous
            const uint4 a = *reinterpret_cast<const uint4*>(xrow + J * 32 + kk * 16 + lg * 8);
            acc = mfma32x32x16(a, bop, acc);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = J * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
            acc = mfma32x32x2(xrow[j], v[r], acc);
          }
        }
      }
      // store: lane holds y[i_loc][p] for p = 32 pt + 8(r/4) + 4 lg + r%4
      if (i_loc < L) {
        T* yrow = ybase + (int64_t)i_loc * H * P + h * P + pt * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int pp = q * 8 + lg * 4;
          if constexpr (kBf16) {
            uint2 o;
            o.x = pack_bf16x2(acc[4 * q + 0], acc[4 * q + 1]);
            o.y = pack_bf16x2(acc[4 * q + 2], acc[4 * q + 3]);
            *reinterpret_cast<uint2*>(yrow + pp) = o;
          } else {
            *reinterpret_cast<float4*>(yrow + pp) =
                make_float4(acc[4 * q + 0], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
          }
        }
      }
    }
  }
}

// Heads per workgroup: the largest of 4, 2, 1 that divides the heads of a group.
int chunk_output_heads_per_block(const Problem& p) {
  const int hpg = p.H / p.G;
  return hpg % 4 == 0 ? 4 : (hpg % 2 == 0 ? 2 : 1);
}

template <class E, int Q, int N>
static hipError_t launch_co(const Problem& p, const Workspace& ws, hipStream_t s) {
  if constexpr (ChunkOutputCfg<E, Q, N>::fits) {
    const int HB = chunk_output_heads_per_block(p);
    const unsigned blocks = (unsigned)(p.kmax * (p.H / HB));
    hipLaunchKernelGGL((chunk_output_kernel<E, Q, N>), dim3(blocks), dim3(kOutThreads), 0, s, p, ws, HB);
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
