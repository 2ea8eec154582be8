// k3_chunk_state.hip -- chunk-local log-decay cumsum (K1, prologue) and chunk
// states (K3) of the SSD block decomposition.
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba).
//  K1, [M] §3.5.4 (segment sums in log space) and §3.5 listing's chunk cumsum:
//    ell_t = dt_t * A_h,  Acs[l] = sum_{k<=l} ell_{t0+k}  (restarting at every
//    chunk; entries past a short chunk's end repeat its last value).  Only
//    chunk-local sums are formed, so |Acs| <= Q * max|ell| and differences of
//    two entries lose little to cancellation ([M] §3.5.4 warns about long
//    cumsums).  exp(Acs_i - Acs_j) is the 1-SS mask of the diagonal block.
//  K3, [M] §3.5.2 "Right factors" and step 2 of "SSD algorithm: chunking and
//    state passing": the final state of each chunk from a zero initial state,
//        S_c[p, n] = sum_{l < L} exp(Acs_{L-1} - Acs_l) * x_l[p] * B_l[n],
//    one (P x Q) . (Q x N) matrix product per (chunk, head).
//
// Design (gfx950): one workgroup of 4 waves per (chunk, block of HB heads of
// one B/C group).  The prologue scans the HB heads' log-decays (one wave per
// head: Q/64 tokens per lane plus a wave-level scan) and writes Acs and the
// chunk total for the later kernels.  The chunk's B tile is staged transposed
// in LDS once (tokens contiguous, as an MFMA operand contracting over tokens
// needs) and serves all HB heads; each head's x tile is loaded into registers
// while the previous head computes, then scaled by its decay-to-chunk-end and
// transposed into LDS.  32x32 output tiles (v_mfma_f32_32x32x16_bf16 /
// _32x32x2_f32) accumulate in fp32; states are stored in the element dtype (the
// state-passing kernel accumulates them in fp32).
#include "ssd_stage.hpp"

namespace ssd {

constexpr int kMaxHB = 4;

template <class E, int Q, int N>
struct ChunkStateCfg {
  using T = typename E::storage;
  static constexpr int P = kHeadDim;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int QP = Q + PAD;          // LDS pitch of the transposed tiles
  static constexpr int NT = N < 32 ? 32 : N;  // B^T rows, padded to an MFMA tile
  static constexpr size_t lds_bytes =
      (size_t)(P + NT) * QP * sizeof(T) + (2 * kMaxHB + 1) * Q * sizeof(float);
  static constexpr bool fits = lds_bytes <= (size_t)kLdsLimit;
};

template <class E, int Q, int N>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(Problem p, Workspace ws, int HB,
                                                               float* __restrict__ states_f32) {
  using Cfg = ChunkStateCfg<E, Q, N>;
  using T = typename E::storage;
  constexpr int P = Cfg::P, QP = Cfg::QP, NT = Cfg::NT;
  constexpr int R = Q / 64;  // tokens per lane in the cumsum
  __shared__ __attribute__((aligned(16))) T xwT[P * QP];
  __shared__ __attribute__((aligned(16))) T bT[NT * QP];
  __shared__ float ell_s[kMaxHB * Q];
  __shared__ float acs_s[kMaxHB * Q];
  __shared__ float w_s[Q];

  const int H = p.H, G = p.G;
  const int nhb = H / HB;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t k = lid / nhb;
  const int h0 = (lid % nhb) * HB;
  const ChunkDesc cd = chunk_desc_search(p, ws, k);
  const int tid = threadIdx.x;
  if (lid % nhb == 0 && tid == 0 && p.cu != nullptr) ws.chunks[k] = cd;  // for the output kernel
  if (cd.seq < 0) return;
  const int L = cd.len;
  const int g = h0 / (H / G);
  const int wid = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lg = lane >> 5;
  const T* xbase = reinterpret_cast<const T*>(p.x) + cd.t0 * H * P;

  // ---- issue the loads: B^T tile, the first head's x tile, the dt tile
  TransTile<E, Q, N> bt;
  bt.load(reinterpret_cast<const T*>(p.B) + (cd.t0 * G + g) * N, (int64_t)G * N, L);
  TransTile<E, Q, P> xt;
  xt.load(xbase + h0 * P, (int64_t)H * P, L);
  if (tid < Q) {
    for (int hh = 0; hh < HB; ++hh) {
      const int h = h0 + hh;
      ell_s[hh * Q + tid] = (tid < L) ? p.dt[(cd.t0 + tid) * H + h] * p.A[h] : 0.0f;
    }
  }
  if (NT > N)
    for (int i = tid; i < (NT - N) * QP; i += kThreads) bT[N * QP + i] = T(0);
  bt.template store<QP, false>(bT, nullptr);
  lds_barrier();

  // ---- K1: chunk-local inclusive cumsum, one wave per head
  if (wid < HB) {
    const int h = h0 + wid;
    float run[R];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      acc += ell_s[wid * Q + lane * R + i];
      run[i] = acc;
    }
    const float incl = wave_inclusive_sum(acc);
    const float excl = incl - acc;
    float* gout = ws.acs + (k * H + h) * Q + lane * R;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float a = excl + run[i];
      acs_s[wid * Q + lane * R + i] = a;
      gout[i] = a;
    }
    if (lane == 63) ws.lam[k * H + h] = incl;
  }

  constexpr int NTN = NT / 32;
  constexpr int NTILES = (P / 32) * NTN;
  for (int hh = 0; hh < HB; ++hh) {
    const int h = h0 + hh;
    lds_barrier();  // Acs ready; previous head's x^T no longer read
    if (tid < Q) {
      const float lam = acs_s[hh * Q + Q - 1];  // entries past L repeat the last one
      w_s[tid] = (tid < L) ? __expf(lam - acs_s[hh * Q + tid]) : 0.0f;
    }
    lds_barrier();
    xt.template store<QP, true>(xwT, w_s);
    lds_barrier();
    if (hh + 1 < HB) xt.load(xbase + (h + 1) * P, (int64_t)H * P, L);

    T* out = reinterpret_cast<T*>(ws.states) + (k * H + h) * (int64_t)(P * N);
    float* out32 = states_f32 ? states_f32 + (k * H + h) * (int64_t)(P * N) : nullptr;
    for (int t = wid; t < NTILES; t += kThreads / 64) {
      const int pt = t / NTN, nt = t % NTN;
      floatx16_t acc = zero16();
      const T* arow = xwT + (pt * 32 + lr) * QP;
      const T* brow = bT + (nt * 32 + lr) * QP;
      if constexpr (E::kBytes == 2) {
#pragma unroll 4
        for (int ks = 0; ks < Q / 16; ++ks) {
          const uint4 a = *reinterpret_cast<const uint4*>(arow + ks * 16 + lg * 8);
          const uint4 b = *reinterpret_cast<const uint4*>(brow + ks * 16 + lg * 8);
          acc = mfma32x32x16(a, b, acc);
        }
      } else {
#pragma unroll 8
        for (int ks = 0; ks < Q / 2; ++ks) acc = mfma32x32x2(arow[ks * 2 + lg], brow[ks * 2 + lg], acc);
      }
      const int n = nt * 32 + lr;
      if (n < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pp = pt * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
          if constexpr (E::kBytes == 2) {
            const uint32_t b2 = pack_bf16x2(acc[r], 0.0f);
            out[pp * N + n] = (uint16_t)(b2 & 0xffffu);
            if (out32) out32[pp * N + n] = bf16_lo(b2);
          } else {
            out[pp * N + n] = acc[r];
            if (out32) out32[pp * N + n] = acc[r];
          }
        }
      }
    }
  }
}

// Heads per workgroup: the largest of 4, 2, 1 that divides the heads of a group.
int chunk_state_heads_per_block(const Problem& p) {
  const int hpg = p.H / p.G;
  return hpg % 4 == 0 ? 4 : (hpg % 2 == 0 ? 2 : 1);
}

template <class E, int Q, int N>
static hipError_t launch_cs(const Problem& p, const Workspace& ws, float* states_f32, hipStream_t s) {
  if constexpr (ChunkStateCfg<E, Q, N>::fits) {
    const int HB = chunk_state_heads_per_block(p);
    const unsigned blocks = (unsigned)(p.kmax * (p.H / HB));
    hipLaunchKernelGGL((chunk_state_kernel<E, Q, N>), dim3(blocks), dim3(kThreads), 0, s, p, ws, HB,
                       states_f32);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <class E, int Q>
static hipError_t launch_cs_n(const Problem& p, const Workspace& ws, float* f, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_cs<E, Q, 16>(p, ws, f, s);
    case 32: return launch_cs<E, Q, 32>(p, ws, f, s);
    case 64: return launch_cs<E, Q, 64>(p, ws, f, s);
    case 128: return launch_cs<E, Q, 128>(p, ws, f, s);
    case 256: return launch_cs<E, Q, 256>(p, ws, f, s);
  }
  return hipErrorInvalidValue;
}

template <class E>
static hipError_t launch_cs_q(const Problem& p, const Workspace& ws, float* f, hipStream_t s) {
  switch (p.Q) {
    case 64: return launch_cs_n<E, 64>(p, ws, f, s);
    case 128: return launch_cs_n<E, 128>(p, ws, f, s);
    case 256: return launch_cs_n<E, 256>(p, ws, f, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state(const Problem& p, const Workspace& ws, float* states_f32,
                              hipStream_t s) {
  return p.dtype == Dtype::BF16 ? launch_cs_q<Bf16>(p, ws, states_f32, s)
                                : launch_cs_q<F32>(p, ws, states_f32, s);
}

bool chunk_state_supported(Dtype dt, int Q, int N) {
#define SSD_CS_CASE(QQ, NN)                                                                   \
  if (Q == QQ && N == NN)                                                                     \
    return dt == Dtype::BF16 ? ChunkStateCfg<Bf16, QQ, NN>::fits : ChunkStateCfg<F32, QQ, NN>::fits;
  SSD_CS_CASE(64, 16) SSD_CS_CASE(64, 32) SSD_CS_CASE(64, 64) SSD_CS_CASE(64, 128) SSD_CS_CASE(64, 256)
  SSD_CS_CASE(128, 16) SSD_CS_CASE(128, 32) SSD_CS_CASE(128, 64) SSD_CS_CASE(128, 128) SSD_CS_CASE(128, 256)
  SSD_CS_CASE(256, 16) SSD_CS_CASE(256, 32) SSD_CS_CASE(256, 64) SSD_CS_CASE(256, 128) SSD_CS_CASE(256, 256)
#undef SSD_CS_CASE
  return false;
}

}  // namespace ssd
