// k3_chunk_state.hip -- chunk states of the SSD block decomposition (K3).
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba), §3.5.2
// "Right factors" and step 2 of "SSD algorithm: chunking and state passing":
// the final state of every chunk assuming a zero initial state,
//     S_c[p, n] = sum_{l < L} exp(Acs_{L-1} - Acs_l) * x_l[p] * B_l[n],
// one (P x Q) . (Q x N) matrix product per (chunk, head).
//
// Design (gfx950): one workgroup of 4 waves per (chunk, head), ordered so that
// the heads of one chunk land on one XCD (their B tile is shared through L2).
// The decay-scaled X tile and the B tile are staged transposed in LDS (tokens
// contiguous) so that each lane's MFMA operand is a run of consecutive tokens;
// output tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16, or _32x32x2_f32 on the
// fp32 path) accumulate in fp32 and go to HBM as fp32.
#include "ssd_stage.hpp"

namespace ssd {

template <class E, int Q, int N>
struct ChunkStateCfg {
  using T = typename E::storage;
  static constexpr int P = kHeadDim;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int QP = Q + PAD;         // LDS pitch (elements) of the transposed tiles
  static constexpr int NT = N < 32 ? 32 : N; // B^T rows, padded to an MFMA tile
  static constexpr size_t lds_bytes = (size_t)(P + NT) * QP * sizeof(T) + Q * sizeof(float);
  static constexpr bool fits = lds_bytes <= (size_t)kLdsLimit;
};

template <class E, int Q, int N>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(Problem p, Workspace ws) {
  using Cfg = ChunkStateCfg<E, Q, N>;
  using T = typename E::storage;
  constexpr int P = Cfg::P, QP = Cfg::QP, NT = Cfg::NT;
  __shared__ __attribute__((aligned(16))) T xwT[P * QP];
  __shared__ __attribute__((aligned(16))) T bT[NT * QP];
  __shared__ float w_s[Q];

  const int H = p.H;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t k = lid / H;
  const int h = lid % H;
  const ChunkDesc cd = ws.chunks[k];
  if (cd.seq < 0) return;
  const int L = cd.len;
  const int g = h / (H / p.G);
  const int tid = threadIdx.x;

  // decay from each token to the chunk end: exp(Acs_{L-1} - Acs_l); 0 past L
  const float* acs = ws.acs + (k * H + h) * Q;
  const float lam = ws.lam[k * H + h];
  for (int l = tid; l < Q; l += kThreads) w_s[l] = (l < L) ? __expf(lam - acs[l]) : 0.0f;
  if (NT > N) {
    for (int i = tid; i < (NT - N) * QP; i += kThreads) bT[N * QP + i] = T(0);
  }
  __syncthreads();
  const T* xg = reinterpret_cast<const T*>(p.x) + (cd.t0 * H + h) * P;
  const T* bg = reinterpret_cast<const T*>(p.B) + (cd.t0 * p.G + g) * N;
  stage_transposed<E, Q, P, QP, true>(xwT, xg, (int64_t)H * P, L, w_s);
  stage_transposed<E, Q, N, QP, false>(bT, bg, (int64_t)p.G * N, L, nullptr);
  __syncthreads();

  const int wid = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lg = lane >> 5;
  constexpr int NTILES_N = NT / 32;
  constexpr int NTILES = (P / 32) * NTILES_N;
  float* out = ws.states + (k * H + h) * (int64_t)(P * N);
  for (int t = wid; t < NTILES; t += kThreads / 64) {
    const int pt = t / NTILES_N, nt = t % NTILES_N;
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
        out[pp * N + n] = acc[r];
      }
    }
  }
}

template <class E, int Q, int N>
static hipError_t launch_cs(const Problem& p, const Workspace& ws, hipStream_t s) {
  if constexpr (ChunkStateCfg<E, Q, N>::fits) {
    const unsigned blocks = (unsigned)(p.kmax * p.H);
    hipLaunchKernelGGL((chunk_state_kernel<E, Q, N>), dim3(blocks), dim3(kThreads), 0, s, p, ws);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <class E, int Q>
static hipError_t launch_cs_n(const Problem& p, const Workspace& ws, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_cs<E, Q, 16>(p, ws, s);
    case 32: return launch_cs<E, Q, 32>(p, ws, s);
    case 64: return launch_cs<E, Q, 64>(p, ws, s);
    case 128: return launch_cs<E, Q, 128>(p, ws, s);
    case 256: return launch_cs<E, Q, 256>(p, ws, s);
  }
  return hipErrorInvalidValue;
}

template <class E>
static hipError_t launch_cs_q(const Problem& p, const Workspace& ws, hipStream_t s) {
  switch (p.Q) {
    case 64: return launch_cs_n<E, 64>(p, ws, s);
    case 128: return launch_cs_n<E, 128>(p, ws, s);
    case 256: return launch_cs_n<E, 256>(p, ws, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state(const Problem& p, const Workspace& ws, hipStream_t s) {
  return p.dtype == Dtype::BF16 ? launch_cs_q<Bf16>(p, ws, s) : launch_cs_q<F32>(p, ws, s);
}

template <class E, int Q, int N>
constexpr bool chunk_state_fits() { return ChunkStateCfg<E, Q, N>::fits; }

bool chunk_state_supported(Dtype dt, int Q, int N) {
#define SSD_CS_CASE(QQ, NN)                                                                   \
  if (Q == QQ && N == NN)                                                                     \
    return dt == Dtype::BF16 ? chunk_state_fits<Bf16, QQ, NN>() : chunk_state_fits<F32, QQ, NN>();
  SSD_CS_CASE(64, 16) SSD_CS_CASE(64, 32) SSD_CS_CASE(64, 64) SSD_CS_CASE(64, 128) SSD_CS_CASE(64, 256)
  SSD_CS_CASE(128, 16) SSD_CS_CASE(128, 32) SSD_CS_CASE(128, 64) SSD_CS_CASE(128, 128) SSD_CS_CASE(128, 256)
  SSD_CS_CASE(256, 16) SSD_CS_CASE(256, 32) SSD_CS_CASE(256, 64) SSD_CS_CASE(256, 128) SSD_CS_CASE(256, 256)
#undef SSD_CS_CASE
  return false;
}

}  // namespace ssd
