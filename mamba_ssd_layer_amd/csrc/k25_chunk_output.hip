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
//  * The kernel matrix tiles G = C B^T of the chunk's B/C group come from the
//    chunk kernel-matrix kernel (formed once per chunk and group, not per
//    head), already in the per-lane MFMA register layout: each lane reloads a
//    tile with coalesced 16-byte loads, two tiles in flight (L2-resident).
//  * One workgroup of 4 waves per (chunk, block of HB heads of one group),
//    about 53 KB of LDS, so two or three workgroups share a CU and one's loads
//    and barriers overlap another's MFMA work.  Each wave's C rows stay in
//    registers for all HB heads; the next head's x tile and passed state are
//    loaded into registers while the current head computes.  Blocks are
//    ordered so that the head blocks of one chunk land on one XCD.
//  * The output is built transposed, Y^T (P x Q), on 32x32 MFMA tiles.  A
//    kernel tile as G^T leaves each lane ONE output token i and 16 input
//    tokens j, which is exactly the B-operand layout of Y^T += X^T (L o G)^T;
//    the K (token) order of that product is chosen to match, and x^T is staged
//    with its tokens permuted in 16-groups so the A operand is one 16-byte read.
//  * Causality: only tiles J <= I are used.  The mask factors as
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
//  * C rows come in the same per-lane operand order from the kernel-matrix
//    kernel (contiguous loads); each finished row tile of y is passed through
//    the wave's own LDS rows and written as whole 128-byte rows.
//  * fp32 accumulation; y rounded once to the element dtype.
#include "ssd_stage.hpp"

namespace ssd {

template <class E, int Q, int N>
struct ChunkOutputCfg {
  using T = typename E::storage;
  static constexpr int P = kHeadDim;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int NP = N + PAD;  // LDS pitch of Hin rows
  static constexpr int QP = Q + PAD;  // LDS pitch of X^T rows
  static constexpr int YP = P + PAD;  // LDS pitch of a wave's staged output rows
  static constexpr size_t lds_bytes =
      ((size_t)P * QP + (size_t)P * NP + (size_t)(kThreads / 64) * 32 * YP) * sizeof(T) +
      2 * Q * sizeof(float);
  static constexpr bool fits = lds_bytes <= (size_t)kLdsLimit;
  static constexpr int KS = N / E::kMfmaK;                  // MFMA steps over N
  static constexpr int CREG = E::kBytes == 2 ? KS * 4 : KS; // VGPRs of one row tile's C operand
  static constexpr bool kKeepC = 2 * CREG <= 32;            // keep both row tiles' C across heads
  static constexpr int NI = Q / 32;
  static constexpr int NTILE = NI * (NI + 1) / 2;           // causal 32x32 kernel tiles
  static constexpr int GV = E::kBytes == 2 ? 2 : 4;         // 16-byte vectors per lane per tile
};

template <class E, int Q, int N>
__global__ __launch_bounds__(kThreads, 2) void chunk_output_kernel(Problem p, Workspace ws, int HB) {
  using Cfg = ChunkOutputCfg<E, Q, N>;
  using T = typename E::storage;
  constexpr int P = Cfg::P, NP = Cfg::NP, QP = Cfg::QP, KS = Cfg::KS, GV = Cfg::GV, YP = Cfg::YP;
  constexpr bool kBf16 = E::kBytes == 2;
  constexpr int NI = Cfg::NI;
  using CReg = typename std::conditional<kBf16, uint4, float>::type;
  __shared__ __attribute__((aligned(16))) T XT[P * QP];
  __shared__ __attribute__((aligned(16))) T Hs[P * NP];
  __shared__ __attribute__((aligned(16))) T Ys[(kThreads / 64) * 32 * YP];
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
  const int nI = (L + 31) / 32;

  const T* xbase = reinterpret_cast<const T*>(p.x) + cd.t0 * H * P;
  // C rows as MFMA operand slices, lane after lane (written by the kernel-matrix kernel)
  const CReg* cop = reinterpret_cast<const CReg*>(ws.cop) + (k * G + g) * (int64_t)(NI * KS * 64) + lane;
  const T* hbase = reinterpret_cast<const T*>(ws.hin) + k * H * (int64_t)(P * N);
  const float* abase = ws.acs + k * H * Q;
  // this lane's 16 values of every kernel tile of the chunk's group
  const uint4* gtiles = reinterpret_cast<const uint4*>(
      reinterpret_cast<const T*>(ws.cb) + (k * G + g) * (int64_t)(Cfg::NTILE * 64 * 16) + lane * 16);
  T* ybase = reinterpret_cast<T*>(p.y) + cd.t0 * H * P;

  // row tiles of this wave: w and 7-w (balanced causal work: tile I costs
  // I+1 kernel tiles); chunks of 64 or 128 tokens have 2 or 4 row tiles
  constexpr int NT = NI == 8 ? 2 : 1;
  auto row_tile = [&](int t) { return t == 0 ? wid : 7 - wid; };

  // C row of this lane's token as MFMA B-operand slices over N (coalesced)
  auto load_c = [&](int I, CReg (&c)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) c[ks] = cop[(I * KS + ks) * 64];
  };
  CReg ckeep[NT][KS];
  if constexpr (Cfg::kKeepC) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (row_tile(t) < nI) load_c(row_tile(t), ckeep[t]);
  }

  TransTile<E, Q, P> xt;
  RowTile<E, P, N> ht;
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
    // C rows (when not kept): the first row tile's are loaded before the next
    // head's prefetch so that waiting for them does not also wait for the
    // prefetch; the second row tile's after the first row tile's work
    CReg cfresh[KS];
    if constexpr (!Cfg::kKeepC) {
      if (row_tile(0) < nI) load_c(row_tile(0), cfresh);
    }
    if (hh + 1 < HB) prefetch(h + 1);

#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int I = row_tile(t);
      if (I >= nI) continue;
      const int i_loc = I * 32 + lr;
      if constexpr (!Cfg::kKeepC) {
        if (t > 0) load_c(I, cfresh);
      }
      const CReg (&creg)[KS] = Cfg::kKeepC ? ckeep[t] : cfresh;
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

      // diagonal block: kernel tiles J <= I of row tile I (consecutive tiles)
      const uint4* grow = gtiles + (int64_t)(I * (I + 1) / 2) * (64 * 16 * sizeof(T) / 16);
      auto load_g = [&](int J, uint4 (&gv)[GV]) {
#pragma unroll
        for (int q = 0; q < GV; ++q) gv[q] = grow[(int64_t)J * (64 * 16 * sizeof(T) / 16) + q];
      };
      auto tile = [&](int J, const uint4 (&gv)[GV]) {
        // gt[r] = G[i_loc][j_r], j_r = 32J + 8(r/4) + 4 lg + r%4
        float gt[16];
        if constexpr (kBf16) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            gt[8 * q + 0] = bf16_lo(gv[q].x); gt[8 * q + 1] = bf16_hi(gv[q].x);
            gt[8 * q + 2] = bf16_lo(gv[q].y); gt[8 * q + 3] = bf16_hi(gv[q].y);
            gt[8 * q + 4] = bf16_lo(gv[q].z); gt[8 * q + 5] = bf16_hi(gv[q].z);
            gt[8 * q + 6] = bf16_lo(gv[q].w); gt[8 * q + 7] = bf16_hi(gv[q].w);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gt[4 * q + 0] = __uint_as_float(gv[q].x); gt[4 * q + 1] = __uint_as_float(gv[q].y);
            gt[4 * q + 2] = __uint_as_float(gv[q].z); gt[4 * q + 3] = __uint_as_float(gv[q].w);
          }
        }
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
            const int col = J * 32 + kk * 16 + lg * 8;
            const uint4 a0 = *reinterpret_cast<const uint4*>(XT + lr * QP + col);
            const uint4 a1 = *reinterpret_cast<const uint4*>(XT + (32 + lr) * QP + col);
            acc0 = mfma32x32x16(a0, bop, acc0);
            acc1 = mfma32x32x16(a1, bop, acc1);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = J * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
            acc0 = mfma32x32x2(XT[lr * QP + j], v[r], acc0);
            acc1 = mfma32x32x2(XT[(32 + lr) * QP + j], v[r], acc1);
          }
        }
      };
      // two register buffers used in turn: the next tile's loads are in flight
      // while the current one is masked and multiplied (loads past I are clamped)
      uint4 gA[GV], gB[GV];
      load_g(0, gA);
      for (int J = 0; J <= I; J += 2) {
        load_g(min(J + 1, I), gB);
        tile(J, gA);
        if (J + 1 > I) break;
        load_g(min(J + 2, I), gA);
        tile(J + 1, gB);
      }
      // store: lane holds y[i_loc][p] for p = 32 pt + 8(r/4) + 4 lg + r%4.  The
      // row tile goes through this wave's LDS rows so that global stores are
      // whole 128-byte rows (eight lanes per row) instead of 32 scattered pieces.
      T* ys = Ys + wid * 32 * YP;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pp = q * 8 + lg * 4;
        if constexpr (kBf16) {
          uint2 o0, o1;
          o0.x = pack_bf16x2(acc0[4 * q + 0], acc0[4 * q + 1]);
          o0.y = pack_bf16x2(acc0[4 * q + 2], acc0[4 * q + 3]);
          o1.x = pack_bf16x2(acc1[4 * q + 0], acc1[4 * q + 1]);
          o1.y = pack_bf16x2(acc1[4 * q + 2], acc1[4 * q + 3]);
          *reinterpret_cast<uint2*>(ys + lr * YP + pp) = o0;
          *reinterpret_cast<uint2*>(ys + lr * YP + 32 + pp) = o1;
        } else {
          *reinterpret_cast<float4*>(ys + lr * YP + pp) =
              make_float4(acc0[4 * q + 0], acc0[4 * q + 1], acc0[4 * q + 2], acc0[4 * q + 3]);
          *reinterpret_cast<float4*>(ys + lr * YP + 32 + pp) =
              make_float4(acc1[4 * q + 0], acc1[4 * q + 1], acc1[4 * q + 2], acc1[4 * q + 3]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      constexpr int VPR = P * sizeof(T) / 16;   // 16-byte vectors per output row
      constexpr int RPI = 64 / VPR;             // rows per store instruction
#pragma unroll
      for (int st = 0; st < 32 / RPI; ++st) {
        const int row = st * RPI + lane / VPR;
        const int vec = lane % VPR;
        const int i_row = I * 32 + row;
        const uint4 val = *reinterpret_cast<const uint4*>(ys + row * YP + vec * (16 / sizeof(T)));
        if (i_row < L)
          *reinterpret_cast<uint4*>(ybase + (int64_t)i_row * H * P + h * P + vec * (16 / sizeof(T))) = val;
      }
      __builtin_amdgcn_wave_barrier();
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
    hipLaunchKernelGGL((chunk_output_kernel<E, Q, N>), dim3(blocks), dim3(kThreads), 0, s, p, ws, HB);
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
