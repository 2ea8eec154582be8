// k7_backward.hip -- glue kernels of the SSD backward pass.
//
// The gradients of a loss L, given dL/dy = dy (and optionally dL/dh_last =
// dfinal), follow from the recurrence h_t = a_t h_{t-1} + x'_t B_t^T,
// y_t = h_t C_t (x' = x, or dt x with the dt-scaled input) by the chain rule
// taken in reverse token order.  With G_t = dL/dh_t = dy_t C_t^T + a_{t+1} G_{t+1}
// and L[t, j] = a_{j+1} ... a_t (the 1-SS mask of "Transformers是SSMs…(一)" §3.2.2):
//   dx'_t = G_t B_t      = sum_{i>=t} L[i,t] (B_t . C_i) dy_i     (+ decayed dfinal)
//   dC_t  = sum_h h_t^T dy_t = sum_{j<=t} L[t,j] (dy_t . x'_j) B_j (+ initial state)
//   dB_j  = sum_h G_j^T x'_j = sum_{t>=j} L[t,j] (dy_t . x'_j) C_t (+ decayed dfinal)
//   d(Acs_k) = dy_k . y_k - x'_k . dx'_k (+ <dfinal, h_last> at a sequence's last
//              token), d(ell_t) = sum_{k>=t} d(Acs_k) within the sequence,
//   d(dt_t) = A_h d(ell_t) (+ x_t . dx'_t with the dt-scaled input),
//   dA_h = sum_t dt_t d(ell_t),  dD_h = sum_t x_t . dy_t,  dh0 = a_first G_first.
// The three sums over tokens are SSD forward passes on rearranged inputs
// ("LLM(十一)——Mamba" §3.5: the same block decomposition), run by the forward
// kernels unchanged:
//   dx'  forward over the sequence reversed in time: input dy, B := C, C := B,
//        decays shifted by one token (a~_j = a_{L-j}, a~_0 = 1), initial state
//        dfinal; its output read back reversed is dx', its final state G_first
//        (this pass and the recompute of y run in fp32: d(ell) sums differences
//        of their terms, which bf16 results would not resolve);
//   dC   forward in time with the roles of x and B exchanged: input B (each
//        head's copy, in parts of 64 columns), B := x', C := dy, initial state
//        h0 transposed; the outputs of a group's heads are summed;
//   dB   as dC, reversed in time: input C, B := dy, C := x', initial state
//        dfinal transposed.
// The kernels here build those inputs (reversed, shifted, per-head copies),
// sum the groups, and form d(ell) by a reverse prefix sum per (sequence,
// head).  All of them are HBM-streaming glue; the matrix work is the forward
// kernels'.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kBwThreads = 256;

// sequence of packed token t: index s, first token t0, length L
struct TokSeq {
  int64_t s, t0, L;
};
__device__ __forceinline__ TokSeq token_seq(const BwdProblem& b, int64_t t) {
  TokSeq r;
  if (b.cu == nullptr) {
    r.s = t / b.seqlen;
    r.t0 = r.s * b.seqlen;
    r.L = b.seqlen;
  } else {
    // last s with cu[s] <= t (empty sequences share their start with the next)
    int64_t lo = 0, hi = b.nseq;  // cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (b.cu[mid] <= t) lo = mid;
      else hi = mid;
    }
    r.s = lo;
    r.t0 = b.cu[lo];
    r.L = b.cu[lo + 1] - r.t0;
  }
  // invalid cu_seqlens contents give unspecified results, never an access
  // outside the buffers: keep t inside [t0, t0 + L) within [0, Ttot)
  if (r.t0 > t || r.t0 < 0) r.t0 = t;
  if (r.L < t - r.t0 + 1) r.L = t - r.t0 + 1;
  if (r.t0 + r.L > b.total) r.L = b.total - r.t0;
  return r;
}

template <class E>
__device__ __forceinline__ float ld_e(const void* p, int64_t i) {
  if constexpr (E::kBytes == 2) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}
template <class E>
__device__ __forceinline__ void st_e(void* p, int64_t i, float v) {
  if constexpr (E::kBytes == 2) reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  else reinterpret_cast<float*>(p)[i] = v;
}

// One workgroup per packed token t (f: t's position reversed within its
// sequence).  Writes the rearranged inputs of the three gradient passes.
template <class E>
__global__ __launch_bounds__(kBwThreads) void bwd_prep_kernel(BwdProblem b) {
  using T = typename E::storage;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int H = b.H, P = b.P, N = b.N, G = b.G, NK = b.NK;
  const int hpg = H / G;
  const TokSeq q = token_seq(b, t);
  const int64_t i = t - q.t0;
  const int64_t f = q.t0 + (q.L - 1 - i);
  // 16-byte copies of whole rows: dy -> xr (reversed); B, C -> Cr, Br (reversed)
  constexpr int VEC = 16 / sizeof(T);
  {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.dy) + t * H * P);
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.xr) + f * H * P);
    for (int v = tid; v < H * P / VEC; v += kBwThreads) dst[v] = src[v];
  }
  {
    const uint4* sb = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.B) + t * G * N);
    const uint4* sc = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.C) + t * G * N);
    uint4* db = reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.Br) + f * G * N);
    uint4* dc = reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.Cr) + f * G * N);
    for (int v = tid; v < G * N / VEC; v += kBwThreads) {
      db[v] = sc[v];  // reversed pass: B := C
      dc[v] = sb[v];  //                C := B
    }
  }
  // x' reversed (input scaled by dt with the dt-scaled input), element-wise;
  // on the bf16 path also the fp32 inputs of the recompute and reversed passes
  for (int e = tid; e < H * P; e += kBwThreads) {
    const int h = e / P;
    const float xv = ld_e<E>(b.x, t * H * P + e);
    st_e<E>(b.cb, f * H * P + e, b.x_times_dt ? xv * b.dt[t * H + h] : xv);
    if constexpr (E::kBytes == 2) {
      const_cast<float*>(b.x32)[t * H * P + e] = xv;
      const_cast<float*>(b.xr32)[f * H * P + e] = ld_e<E>(b.dy, t * H * P + e);
    }
  }
  if constexpr (E::kBytes == 2) {
    for (int e = tid; e < G * N; e += kBwThreads) {
      const float bv = ld_e<E>(b.B, t * G * N + e), cv = ld_e<E>(b.C, t * G * N + e);
      const_cast<float*>(b.B32)[t * G * N + e] = bv;
      const_cast<float*>(b.C32)[t * G * N + e] = cv;
      const_cast<float*>(b.Br32)[f * G * N + e] = cv;  // reversed pass: B := C
      const_cast<float*>(b.Cr32)[f * G * N + e] = bv;  //                C := B
    }
  }
  // per-head copies of B (in time) and C (reversed), 64-column parts, zero
  // padded past N
  const int W = 64 * NK;
  for (int e = tid; e < H * W; e += kBwThreads) {
    const int h = e / W, n = e % W;
    const int g = h / hpg;
    const float vb = n < N ? ld_e<E>(b.B, (t * G + g) * N + n) : 0.0f;
    const float vc = n < N ? ld_e<E>(b.C, (t * G + g) * N + n) : 0.0f;
    st_e<E>(b.xc, t * H * W + e, vb);
    st_e<E>(b.xb, f * H * W + e, vc);
  }
  // step sizes: reversed and shifted by one token (the first reversed token
  // has a~ = 1), and per-part copies
  for (int h = tid; h < H; h += kBwThreads) {
    const float dtr = (i == q.L - 1) ? 0.0f : b.dt[(t + 1) * H + h];
    b.dtr[f * H + h] = dtr;
    const float dtt = b.dt[t * H + h];
    for (int k = 0; k < NK; ++k) {
      b.dtc[t * H * NK + h * NK + k] = dtt;
      b.dtb[f * H * NK + h * NK + k] = dtr;
    }
  }
  if (t == 0)
    for (int e = tid; e < H * NK; e += kBwThreads) b.Ac[e] = b.A[e / NK];
}

// The atomically accumulated outputs (dA, dD) start from zero.
__global__ __launch_bounds__(kBwThreads) void bwd_zero_kernel(BwdProblem b) {
  for (int h = threadIdx.x; h < b.H; h += kBwThreads) {
    b.dA[h] = 0.0f;
    if (b.dD != nullptr) b.dD[h] = 0.0f;
  }
}

// Transposed 64 x 64 parts of the initial state (C pass) and of dfinal (B
// pass): out[s, h*NK + k, nl, p] = in[s, h, p, 64k + nl] (0 past N).  One
// workgroup per (sequence, head, part).
__global__ __launch_bounds__(kBwThreads) void bwd_prep_states_kernel(BwdProblem b) {
  const int64_t blk = blockIdx.x;
  const int NK = b.NK, P = b.P, N = b.N;
  const int k = (int)(blk % NK);
  const int64_t sh = blk / NK;  // s * H + h
  for (int e = threadIdx.x; e < 64 * 64; e += kBwThreads) {
    const int nl = e / 64, p = e % 64;
    const int n = 64 * k + nl;
    const int64_t src = sh * P * N + (int64_t)p * N + n;
    const int64_t dst = (sh * NK + k) * 64 * 64 + e;
    if (b.h0c != nullptr) b.h0c[dst] = n < N ? b.h0[src] : 0.0f;
    if (b.dfb != nullptr) b.dfb[dst] = n < N ? b.dfinal[src] : 0.0f;
  }
}

// dC[t, g, n] = sum over the group's heads of the C pass output at t; dB the
// same from the B pass output read at the reversed position.  fp32 sums.
template <class E>
__global__ __launch_bounds__(kBwThreads) void bwd_reduce_kernel(BwdProblem b) {
  const int64_t t = blockIdx.x;
  const int H = b.H, N = b.N, G = b.G, W = 64 * b.NK;
  const int hpg = H / G;
  const TokSeq q = token_seq(b, t);
  const int64_t f = q.t0 + (q.L - 1 - (t - q.t0));
  for (int e = threadIdx.x; e < G * N; e += kBwThreads) {
    const int g = e / N, n = e % N;
    float sc = 0.0f, sb = 0.0f;
    for (int j = 0; j < hpg; ++j) {
      const int h = g * hpg + j;
      sc += ld_e<E>(b.y_c, (t * H + h) * W + n);
      sb += ld_e<E>(b.y_b, (f * H + h) * W + n);
    }
    st_e<E>(b.dC, t * G * N + e, sc);
    st_e<E>(b.dB, t * G * N + e, sb);
  }
}

// Per (token, head): dx = dx' (times dt with the dt-scaled input) + D dy, and
// the per-token terms of d(ell), d(dt), dD, stored head-major (H, Ttot).
// Eight lanes share one head row (8 values each); one workgroup per token.
template <class E>
__global__ __launch_bounds__(kBwThreads) void bwd_token_kernel(BwdProblem b) {
  const int64_t t = blockIdx.x;
  const int H = b.H, P = b.P;
  const TokSeq q = token_seq(b, t);
  const int64_t f = q.t0 + (q.L - 1 - (t - q.t0));
  const int lane8 = threadIdx.x % 8;
  for (int h = threadIdx.x / 8; h < H; h += kBwThreads / 8) {
    const float dth = b.dt[t * H + h];
    const float sx = b.x_times_dt ? dth : 1.0f;
    const float dh = b.D != nullptr ? b.D[h] : 0.0f;
    float s_dyy = 0.0f, s_xdx = 0.0f, s_xdy = 0.0f;
    for (int p = lane8; p < P; p += 8) {
      const int64_t o = (t * H + h) * P + p;
      const float xv = ld_e<E>(b.x, o);
      const float dyv = ld_e<E>(b.dy, o);
      const float yv = b.y_f[o];
      const float dxp = b.y_x[(f * H + h) * P + p];  // dx' = reversed pass output
      s_dyy += dyv * yv;
      s_xdx += xv * dxp;
      s_xdy += xv * dyv;
      st_e<E>(b.dx, o, sx * dxp + dh * dyv);
    }
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
      s_dyy += __shfl_xor(s_dyy, off);
      s_xdx += __shfl_xor(s_xdx, off);
      s_xdy += __shfl_xor(s_xdy, off);
    }
    if (lane8 == 0) {
      b.qd[h * b.total + t] = s_dyy - sx * s_xdx;  // d(Acs_t): dy . y - x' . dx'
      b.rd[h * b.total + t] = s_xdx;               // x . dx' (d(dt) term of the dt-scaled input)
      b.ud[h * b.total + t] = s_xdy;               // x . dy (dD term)
    }
  }
}

// Block-wide sum of v over the 256 threads (result valid in every thread).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x / 64;
  __syncthreads();
  if (threadIdx.x % 64 == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kBwThreads / 64; ++i) s += red[i];
  return s;
}

// Per (sequence, head): <dfinal, h_last>, dh0 = a_first G_first, then
// d(ell_t) = sum_{k>=t} d(Acs_k) (plus <dfinal, h_last> at the last token) by
// a reverse prefix sum, d(dt), and the sequence's shares of dA and dD.
__global__ __launch_bounds__(kBwThreads) void bwd_scan_kernel(BwdProblem b) {
  __shared__ float red[kBwThreads / 64];
  __shared__ double part[kBwThreads];
  const int64_t sh = blockIdx.x;
  const int H = b.H;
  const int h = (int)(sh % H);
  const int64_t s = sh / H;
  const int tid = threadIdx.x;
  int64_t t0, L;
  if (b.cu == nullptr) {
    t0 = s * b.seqlen;
    L = b.seqlen;
  } else {
    // clamped into [0, Ttot] (invalid contents: unspecified results, in bounds)
    t0 = min(max((int64_t)b.cu[s], (int64_t)0), b.total);
    L = max(min((int64_t)b.cu[s + 1], b.total) - t0, (int64_t)0);
  }
  const int64_t PN = (int64_t)b.P * b.N;
  float e = 0.0f;
  if (b.dfinal != nullptr) {
    float acc = 0.0f;
    for (int64_t i = tid; i < PN; i += kBwThreads) acc += b.dfinal[sh * PN + i] * b.hlast[sh * PN + i];
    e = block_sum(acc, red);
  }
  if (b.dinit != nullptr) {
    const float a0 = L > 0 ? __expf(b.dt[t0 * H + h] * b.A[h]) : 1.0f;
    for (int64_t i = tid; i < PN; i += kBwThreads) b.dinit[sh * PN + i] = a0 * b.g0[sh * PN + i];
  }
  if (L == 0) return;
  // thread r owns tokens [r c, (r + 1) c) of the sequence
  const int64_t c = (L + kBwThreads - 1) / kBwThreads;
  const int64_t i0 = min((int64_t)tid * c, L), i1 = min(i0 + c, L);
  // the running sums are fp64: d(ell) is a sum of up to T terms of both signs
  const float* qd = b.qd + h * b.total + t0;
  double local = 0.0;
  for (int64_t i = i0; i < i1; ++i) local += qd[i];
  part[tid] = local;
  __syncthreads();
  // suffix sum of the parts after this thread's range (a plain loop over at
  // most 255 values from LDS: the scan is a small part of the backward)
  double after = e;
  for (int r = tid + 1; r < kBwThreads; ++r) after += part[r];
  const float* rd = b.rd + h * b.total + t0;
  const float* ud = b.ud + h * b.total + t0;
  const float Ah = b.A[h];
  double run = after, sdA = 0.0, sdD = 0.0;
  for (int64_t i = i1 - 1; i >= i0; --i) {
    run += qd[i];
    const float dtv = b.dt[(t0 + i) * H + h];
    b.ddt[(t0 + i) * H + h] = Ah * (float)run + (b.x_times_dt ? rd[i] : 0.0f);
    sdA += dtv * run;
    sdD += ud[i];
  }
  sdA = block_sum((float)sdA, red);
  sdD = block_sum((float)sdD, red);
  if (tid == 0) {
    atomicAdd(b.dA + h, sdA);
    if (b.dD != nullptr) atomicAdd(b.dD + h, sdD);
  }
}

template <class E>
static hipError_t launch_glue(const BwdProblem& b, int stage, hipStream_t s) {
  const dim3 blk(kBwThreads);
  switch (stage) {
    case 0:
      hipLaunchKernelGGL(bwd_zero_kernel, dim3(1), blk, 0, s, b);
      if (b.total > 0) hipLaunchKernelGGL((bwd_prep_kernel<E>), dim3((unsigned)b.total), blk, 0, s, b);
      if ((b.h0c != nullptr || b.dfb != nullptr) && b.nseq > 0)
        hipLaunchKernelGGL(bwd_prep_states_kernel, dim3((unsigned)(b.nseq * b.H * b.NK)), blk, 0, s, b);
      break;
    case 1:
      if (b.total > 0) {
        hipLaunchKernelGGL((bwd_reduce_kernel<E>), dim3((unsigned)b.total), blk, 0, s, b);
        hipLaunchKernelGGL((bwd_token_kernel<E>), dim3((unsigned)b.total), blk, 0, s, b);
      }
      if (b.nseq > 0) hipLaunchKernelGGL(bwd_scan_kernel, dim3((unsigned)(b.nseq * b.H)), blk, 0, s, b);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_backward_glue(const BwdProblem& b, int stage, hipStream_t s) {
  return b.dtype == Dtype::BF16 ? launch_glue<Bf16>(b, stage, s) : launch_glue<F32>(b, stage, s);
}

}  // namespace ssd
