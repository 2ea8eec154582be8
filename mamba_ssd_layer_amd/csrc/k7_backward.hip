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
//        dfinal; its output read back reversed is dx', its final state G_first.
//        This pass and the recompute of y run in fp32 (d(ell) below is a
//        running sum of their terms, which bf16 results would not resolve:
//        errors of several percent in d(dt)) and leave out each token's own term
//        (C_t . B_t) x'_t (resp. dy_t): it appears in both dy . y and x' . dx'
//        and, for fast decays, dominates both, so d(Acs) would be the small
//        difference of two rounded large numbers; without it nothing cancels,
//        and the term is added back to dx exactly;
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

// A 16-byte vector of the element type times d (bf16: rounded to nearest even).
template <class E>
__device__ __forceinline__ uint4 scale_vec(const uint4& v, float d) {
  if constexpr (E::kBytes == 2) {
    auto f = [&](uint32_t w) { return pack_bf16x2(bf16_lo(w) * d, bf16_hi(w) * d); };
    return make_uint4(f(v.x), f(v.y), f(v.z), f(v.w));
  } else {
    auto f = [&](uint32_t w) { return __float_as_uint(__uint_as_float(w) * d); };
    return make_uint4(f(v.x), f(v.y), f(v.z), f(v.w));
  }
}
// Eight bf16 values -> eight fp32 at dst (two 16-byte stores).
__device__ __forceinline__ void store_f32x8(float* dst, const uint4& v) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
  reinterpret_cast<float4*>(dst)[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
}
// 16-byte vector of the element type -> VEC fp32 values.
template <class E>
__device__ __forceinline__ void unpack_vec(const uint4& v, float (&o)[16 / E::kBytes]) {
  if constexpr (E::kBytes == 2) {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  } else {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y); o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
}
template <class E>
__device__ __forceinline__ uint4 pack_vec(const float (&o)[16 / E::kBytes]) {
  if constexpr (E::kBytes == 2)
    return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
  else
    return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
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
  // the head-sum gradients, accumulated by later kernels, start at zero
  if (t == 0)
    for (int h = tid; h < H; h += kBwThreads) {
      b.dA[h] = 0.0f;
      if (b.dD != nullptr) b.dD[h] = 0.0f;
    }
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
  // x' reversed (input scaled by dt with the dt-scaled input), and on the bf16
  // path the fp32 inputs of the recompute and reversed passes, in 16-byte
  // vectors (VEC elements, never straddling a head row)
  const bool x_copies = b.cb != nullptr || (E::kBytes == 2 && !b.chunked_dl);  // else x is not read here
  for (int v = tid; x_copies && v < H * P / VEC; v += kBwThreads) {
    const int h = v * VEC / P;
    const uint4 xv = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.x) + t * H * P)[v];
    if (b.cb != nullptr) {
      uint4* cbv = reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.cb) + f * H * P) + v;
      if (b.x_times_dt) {
        const float d = b.dt[t * H + h];
        *cbv = scale_vec<E>(xv, d);
      } else {
        *cbv = xv;
      }
    }
    if (E::kBytes == 2 && !b.chunked_dl) {  // fp32 inputs of the recompute and reversed passes
      const uint4 dyv = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.dy) + t * H * P)[v];
      store_f32x8(const_cast<float*>(b.x32) + t * H * P + v * 8, xv);
      store_f32x8(const_cast<float*>(b.xr32) + f * H * P + v * 8, dyv);
    }
  }
  if (E::kBytes == 2 && !b.chunked_dl) {
    for (int v = tid; v < G * N / VEC; v += kBwThreads) {
      const uint4 bv = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.B) + t * G * N)[v];
      const uint4 cv = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.C) + t * G * N)[v];
      store_f32x8(const_cast<float*>(b.B32) + t * G * N + v * 8, bv);
      store_f32x8(const_cast<float*>(b.C32) + t * G * N + v * 8, cv);
      store_f32x8(const_cast<float*>(b.Br32) + f * G * N + v * 8, cv);  // reversed pass: B := C
      store_f32x8(const_cast<float*>(b.Cr32) + f * G * N + v * 8, bv);  //                C := B
    }
  }
  // per-head copies of B (in time) and C (reversed), 64-column parts, zero
  // padded past N (absent, like the B pass's x' and the per-part step sizes,
  // when dB and dC are formed per chunk instead)
  const int W = 64 * NK;
  const int WV = W / VEC;
  for (int v = tid; b.xc != nullptr && v < H * WV; v += kBwThreads) {
    const int h = v / WV, n0 = (v % WV) * VEC;
    const int g = h / hpg;
    uint4 vb = make_uint4(0, 0, 0, 0), vc = vb;
    if (n0 < N) {
      vb = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.B) + (t * G + g) * N + n0);
      vc = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.C) + (t * G + g) * N + n0);
    }
    reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.xc) + t * H * W)[v] = vb;
    reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.xb) + f * H * W)[v] = vc;
  }
  // step sizes: reversed and shifted by one token (the first reversed token
  // has a~ = 1), and per-part copies
  for (int h = tid; h < H; h += kBwThreads) {
    const float dtr = (i == q.L - 1) ? 0.0f : b.dt[(t + 1) * H + h];
    b.dtr[f * H + h] = dtr;
    if (b.dtc == nullptr) continue;
    const float dtt = b.dt[t * H + h];
    for (int k = 0; k < NK; ++k) {
      b.dtc[t * H * NK + h * NK + k] = dtt;
      b.dtb[f * H * NK + h * NK + k] = dtr;
    }
  }
  if (t == 0 && b.Ac != nullptr)
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
  using T = typename E::storage;
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float pc[kBwThreads][VEC], pb[kBwThreads][VEC];
  const int64_t t = blockIdx.x;
  const int H = b.H, N = b.N, G = b.G, W = 64 * b.NK;
  const int hpg = H / G;
  const TokSeq q = token_seq(b, t);
  const int64_t f = q.t0 + (q.L - 1 - (t - q.t0));
  const T* yc = reinterpret_cast<const T*>(b.y_c);
  const T* yb = reinterpret_cast<const T*>(b.y_b);
  const int nvec = G * N / VEC;
  // with few output vectors the heads of a group are split into `slices`
  // interleaved subsets summed by different threads, then combined in LDS
  const int slices = nvec < kBwThreads ? kBwThreads / nvec : 1;
  for (int v0 = 0; v0 < nvec; v0 += kBwThreads / slices) {
    const int v = v0 + threadIdx.x % (kBwThreads / slices);
    const int sl = threadIdx.x / (kBwThreads / slices);
    float sc[VEC] = {}, sb[VEC] = {};
    if (v < nvec && sl < slices) {
      const int g = v * VEC / N, n0 = v * VEC % N;
      for (int j = sl; j < hpg; j += slices) {
        const int h = g * hpg + j;
        float a[VEC], c[VEC];
        unpack_vec<E>(*reinterpret_cast<const uint4*>(yc + (t * H + h) * W + n0), a);
        unpack_vec<E>(*reinterpret_cast<const uint4*>(yb + (f * H + h) * W + n0), c);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          sc[k] += a[k];
          sb[k] += c[k];
        }
      }
    }
    if (slices > 1) {
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        pc[threadIdx.x][k] = sc[k];
        pb[threadIdx.x][k] = sb[k];
      }
      __syncthreads();
      if (sl == 0)
        for (int r = 1; r < slices; ++r)
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            sc[k] += pc[threadIdx.x + r * (kBwThreads / slices)][k];
            sb[k] += pb[threadIdx.x + r * (kBwThreads / slices)][k];
          }
      __syncthreads();
    }
    if (v < nvec && sl == 0) {
      reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.dC) + t * G * N)[v] = pack_vec<E>(sc);
      reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.dB) + t * G * N)[v] = pack_vec<E>(sb);
    }
  }
}

// bwd_token_kernel (below; the paths other than the chunk-local d(ell) one,
// whose kernel forms these itself): per (token, head) dx = dx' (with the
// token's own term added back, times dt with the dt-scaled input) + D dy, and
// the per-token terms of d(ell), d(dt), dD, stored head-major (H, Ttot).
// Eight lanes share one head row (8 values each); one workgroup per token.

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

// Token range [t0, t0 + L) of sequence s, clamped into [0, Ttot] (invalid
// cu_seqlens contents: unspecified results, every access in bounds).
__device__ __forceinline__ void seq_range(const BwdProblem& b, int64_t s, int64_t* t0, int64_t* L) {
  if (b.cu == nullptr) {
    *t0 = s * b.seqlen;
    *L = b.seqlen;
  } else {
    *t0 = min(max((int64_t)b.cu[s], (int64_t)0), b.total);
    *L = max(min((int64_t)b.cu[s + 1], b.total) - *t0, (int64_t)0);
  }
}

template <class E>
__global__ __launch_bounds__(kBwThreads) void bwd_token_kernel(BwdProblem b) {
  using T = typename E::storage;
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float cbs[kMaxBwdGroups];
  const int64_t t = blockIdx.x;
  const int H = b.H, P = b.P, N = b.N, G = b.G;
  const int hpg = H / G;
  const TokSeq q = token_seq(b, t);
  const int64_t f = q.t0 + (q.L - 1 - (t - q.t0));
  // c_g = C_t . B_t per group: the weight of each token's own term, which the
  // fp32 passes leave out of y and dx'
  {
    const int wid = threadIdx.x / 64, lane = threadIdx.x % 64;
    for (int g = wid; g < G; g += kBwThreads / 64) {
      float acc = 0.0f;
      for (int n = lane; n < N; n += 64)
        acc += ld_e<E>(b.C, (t * G + g) * N + n) * ld_e<E>(b.B, (t * G + g) * N + n);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      if (lane == 0) cbs[g] = acc;
    }
    __syncthreads();
  }
  const int lane8 = threadIdx.x % 8;  // eight lanes per head row, 8 values each
  for (int h = threadIdx.x / 8; h < H; h += kBwThreads / 8) {
    const float dth = b.dt[t * H + h];
    const float sx = b.x_times_dt ? dth : 1.0f;
    const float dh = b.D != nullptr ? b.D[h] : 0.0f;
    const float cg = cbs[h / hpg];
    const int64_t o = (t * H + h) * P + lane8 * 8;
    const int64_t orev = (f * H + h) * P + lane8 * 8;  // dx' comes reversed
    float xv[8], dyv[8], yv[8] = {}, dxs[8], dx[8];
#pragma unroll
    for (int c = 0; c < 8 / VEC; ++c) {
      unpack_vec<E>(*reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.x) + o + c * VEC),
                    *reinterpret_cast<float(*)[VEC]>(xv + c * VEC));
      unpack_vec<E>(*reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(b.dy) + o + c * VEC),
                    *reinterpret_cast<float(*)[VEC]>(dyv + c * VEC));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float4 a = reinterpret_cast<const float4*>(b.y_f + o)[c];
      const float4 d = reinterpret_cast<const float4*>(b.y_x + orev)[c];
      yv[4 * c] = a.x; yv[4 * c + 1] = a.y; yv[4 * c + 2] = a.z; yv[4 * c + 3] = a.w;
      dxs[4 * c] = d.x; dxs[4 * c + 1] = d.y; dxs[4 * c + 2] = d.z; dxs[4 * c + 3] = d.w;
    }
    // without the own terms in y and dx', d(Acs_t) = dy . y - x' . dx' has
    // nothing that cancels itself; dx' = dx's + c_g dy exactly
    float s_dyy = 0.0f, s_xdx = 0.0f, s_xdy = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      s_dyy += dyv[k] * yv[k];
      s_xdx += xv[k] * dxs[k];
      s_xdy += xv[k] * dyv[k];
      dx[k] = sx * (dxs[k] + cg * dyv[k]) + dh * dyv[k];
    }
#pragma unroll
    for (int c = 0; c < 8 / VEC; ++c)
      *reinterpret_cast<uint4*>(reinterpret_cast<T*>(b.dx) + o + c * VEC) =
          pack_vec<E>(*reinterpret_cast<float(*)[VEC]>(dx + c * VEC));
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
      s_dyy += __shfl_xor(s_dyy, off);
      s_xdx += __shfl_xor(s_xdx, off);
      s_xdy += __shfl_xor(s_xdy, off);
    }
    if (lane8 == 0) {
      b.qd[h * b.total + t] = s_dyy - sx * s_xdx;  // d(Acs_t)
      b.rd[h * b.total + t] = s_xdx + cg * s_xdy;  // x . dx' (full): d(dt) term of the dt-scaled input
      b.ud[h * b.total + t] = s_xdy;               // x . dy (dD term)
    }
  }
}

// dD (chunk-local d(ell) path): per (sequence, head) the sum of x . dy, and
// dh0 = a_first G_first.
__global__ __launch_bounds__(kBwThreads) void bwd_seqsum_kernel(BwdProblem b) {
  __shared__ float red[kBwThreads / 64];
  const int64_t sh = blockIdx.x;
  const int h = (int)(sh % b.H);
  int64_t t0, L;
  seq_range(b, sh / b.H, &t0, &L);
  const int64_t PN = (int64_t)b.P * b.N;
  if (b.dinit != nullptr) {
    const float a0 = L > 0 ? __expf(b.dt[t0 * b.H + h] * b.A[h]) : 1.0f;
    for (int64_t i = threadIdx.x; i < PN; i += kBwThreads) b.dinit[sh * PN + i] = a0 * b.g0[sh * PN + i];
  }
  if (b.dD != nullptr) {
    float acc = 0.0f;
    for (int64_t i = threadIdx.x; i < L; i += kBwThreads) acc += b.ud[h * b.total + t0 + i];
    acc = block_sum(acc, red);
    if (threadIdx.x == 0) atomicAdd(b.dD + h, acc);
  }
}

// d(ell_t) = sum_{k>=t} d(Acs_k) (+ <dfinal, h_last>) is a reverse prefix sum
// over each sequence, split into segments of kSeg tokens so that long
// sequences spread over many workgroups.  Sums are fp64: d(ell) is a sum of up
// to T terms of both signs.
constexpr int kSeg = kBwdScanSeg;

// Pass 1, one workgroup per (sequence, head, segment): the segment's sum; the
// first segment's workgroup also forms <dfinal, h_last> and dh0 = a_first G_first.
__global__ __launch_bounds__(kBwThreads) void bwd_segsum_kernel(BwdProblem b) {
  __shared__ float red[kBwThreads / 64];
  __shared__ double redd[kBwThreads / 64];
  const int64_t blk = blockIdx.x;
  const int64_t sh = blk / b.nseg;
  const int seg = (int)(blk % b.nseg);
  const int h = (int)(sh % b.H);
  const int tid = threadIdx.x;
  int64_t t0, L;
  seq_range(b, sh / b.H, &t0, &L);
  if (seg == 0) {
    const int64_t PN = (int64_t)b.P * b.N;
    if (b.dfinal != nullptr) {
      float acc = 0.0f;
      for (int64_t i = tid; i < PN; i += kBwThreads) acc += b.dfinal[sh * PN + i] * b.hlast[sh * PN + i];
      acc = block_sum(acc, red);
      if (tid == 0) b.edot[sh] = acc;
    }
    if (b.dinit != nullptr) {
      const float a0 = L > 0 ? __expf(b.dt[t0 * b.H + h] * b.A[h]) : 1.0f;
      for (int64_t i = tid; i < PN; i += kBwThreads) b.dinit[sh * PN + i] = a0 * b.g0[sh * PN + i];
    }
  }
  const int64_t i0 = (int64_t)seg * kSeg, i1 = min(i0 + kSeg, L);
  double acc = 0.0;
  for (int64_t i = i0 + tid; i < i1; i += kBwThreads) acc += b.qd[h * b.total + t0 + i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (tid % 64 == 0) redd[tid / 64] = acc;
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int w = 0; w < kBwThreads / 64; ++w) s += redd[w];
    b.segsum[blk] = s;
  }
}

// Pass 2, one workgroup per (sequence, head, segment): offset from the later
// segments, the in-segment reverse prefix sum (kSeg / 256 tokens per thread),
// d(dt), and the segment's shares of dA and dD.
__global__ __launch_bounds__(kBwThreads) void bwd_scan_kernel(BwdProblem b) {
  __shared__ float red[kBwThreads / 64];
  __shared__ double part[kBwThreads];
  constexpr int TPT = kSeg / kBwThreads;
  const int64_t blk = blockIdx.x;
  const int64_t sh = blk / b.nseg;
  const int seg = (int)(blk % b.nseg);
  const int H = b.H;
  const int h = (int)(sh % H);
  const int tid = threadIdx.x;
  int64_t t0, L;
  seq_range(b, sh / H, &t0, &L);
  const int64_t i0 = (int64_t)seg * kSeg;
  if (i0 >= L) return;  // uniform: the whole workgroup leaves
  double after = b.dfinal != nullptr ? (double)b.edot[sh] : 0.0;
  for (int r = seg + 1; r < b.nseg; ++r) after += b.segsum[sh * b.nseg + r];
  const float* qd = b.qd + h * b.total + t0;
  const int64_t j0 = i0 + (int64_t)tid * TPT, j1 = min(j0 + TPT, L);
  double local = 0.0;
  for (int64_t i = j0; i < j1; ++i) local += qd[i];
  // inclusive suffix sums of the threads' parts (Hillis-Steele in LDS)
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kBwThreads; off <<= 1) {
    const double add = tid + off < kBwThreads ? part[tid + off] : 0.0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  double run = after + part[tid] - local;  // everything after this thread's tokens
  const float* rd = b.rd + h * b.total + t0;
  const float* ud = b.ud + h * b.total + t0;
  const float Ah = b.A[h];
  double sdA = 0.0, sdD = 0.0;
  for (int64_t i = j1 - 1; i >= j0; --i) {
    run += qd[i];
    const float dtv = b.dt[(t0 + i) * H + h];
    b.ddt[(t0 + i) * H + h] = Ah * (float)run + (b.x_times_dt ? rd[i] : 0.0f);
    sdA += dtv * run;
    sdD += ud[i];
  }
  const float fa = block_sum((float)sdA, red);
  const float fd = block_sum((float)sdD, red);
  if (tid == 0) {
    atomicAdd(b.dA + h, fa);
    if (b.dD != nullptr) atomicAdd(b.dD + h, fd);
  }
}

// ---- packed sequences padded to whole chunks (chunk-local path) ----
// clamped bounds of packed sequence s (invalid cu: unspecified results, every
// access in bounds)
__device__ __forceinline__ void packed_seq(const PadArgs& a, int64_t s, int64_t* lo, int64_t* L) {
  if (a.cu == nullptr) {  // batched
    *lo = s * a.seqlen;
    *L = a.seqlen;
    return;
  }
  const int64_t c0 = min(max((int64_t)a.cu[s], (int64_t)0), a.T);
  const int64_t c1 = min(max((int64_t)a.cu[s + 1], (int64_t)0), a.T);
  *lo = c0;
  *L = max(c1 - c0, (int64_t)0);
}

// One workgroup: cup[s] = sum over s' < s of ceil(L_s' / Q) Q (runs of
// sequences per thread, then a block-wide scan), cup[S + 1] = Tp.
__global__ __launch_bounds__(kBwThreads) void bwd_pad_offsets_kernel(PadArgs a) {
  __shared__ int64_t part[kBwThreads];
  const int tid = threadIdx.x;
  const int64_t per = (a.S + kBwThreads - 1) / kBwThreads;
  const int64_t s0 = min(a.S, (int64_t)tid * per), s1 = min(a.S, s0 + per);
  auto padded = [&](int64_t s) {
    int64_t lo, L;
    packed_seq(a, s, &lo, &L);
    return (L + a.Q - 1) / a.Q * a.Q;
  };
  int64_t sum = 0;
  for (int64_t s = s0; s < s1; ++s) sum += padded(s);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kBwThreads; off <<= 1) {  // inclusive scan
    const int64_t add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int64_t run = part[tid] - sum;
  for (int64_t s = s0; s < s1; ++s) {
    a.cup[s] = (int32_t)min(run, a.Tp);
    run += padded(s);
  }
  if (tid == kBwThreads - 1) {
    a.cup[a.S] = (int32_t)min(part[tid], a.Tp);
    a.cup[a.S + 1] = (int32_t)a.Tp;
  }
}

// rows of n 16-byte vectors: copy from src (or zeros when src is null)
__device__ __forceinline__ void copy_row(const void* src, void* dst, int n) {
  for (int v = threadIdx.x; v < n; v += kBwThreads)
    reinterpret_cast<uint4*>(dst)[v] = src ? reinterpret_cast<const uint4*>(src)[v] : make_uint4(0, 0, 0, 0);
}

// One workgroup per padded token: its source token, or the padding.
__global__ __launch_bounds__(kBwThreads) void bwd_pad_kernel(PadArgs a) {
  const int64_t tp = blockIdx.x;
  int64_t lo = 0, hi = a.S + 1;  // last s in [0, S] with cup[s] <= tp
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if (a.cup[mid] <= tp) lo = mid;
    else hi = mid;
  }
  int64_t src = -1;
  if (lo < a.S) {
    int64_t c0, L;
    packed_seq(a, lo, &c0, &L);
    const int64_t i = tp - a.cup[lo];
    if (i >= 0 && i < L) src = c0 + i;
  }
  const int eb = a.dtype == Dtype::BF16 ? 2 : 4;
  const int64_t xr = (int64_t)a.H * a.P * eb, br = (int64_t)a.G * a.N * eb;  // row bytes
  auto row = [&](const void* base, int64_t bytes) {
    return src >= 0 ? static_cast<const char*>(base) + src * bytes : nullptr;
  };
  copy_row(row(a.x, xr), static_cast<char*>(a.xp) + tp * xr, (int)(xr / 16));
  copy_row(row(a.dy, xr), static_cast<char*>(a.dyp) + tp * xr, (int)(xr / 16));
  copy_row(row(a.B, br), static_cast<char*>(a.Bp) + tp * br, (int)(br / 16));
  copy_row(row(a.C, br), static_cast<char*>(a.Cp) + tp * br, (int)(br / 16));
  for (int h = threadIdx.x; h < a.H; h += kBwThreads) a.dtp[tp * a.H + h] = src >= 0 ? a.dt[src * a.H + h] : 0.0f;
}

// One workgroup per token: its results from the padded layout.
__global__ __launch_bounds__(kBwThreads) void bwd_unpad_kernel(PadArgs a) {
  const int64_t t = blockIdx.x;
  int64_t lo = 0, hi = a.S;  // last s with cu[s] <= t (clamped)
  if (a.cu == nullptr) {
    lo = min(t / max(a.seqlen, (int64_t)1), a.S - 1);
  } else {
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (min(max((int64_t)a.cu[mid], (int64_t)0), a.T) <= t) lo = mid;
      else hi = mid;
    }
  }
  int64_t c0, L;
  packed_seq(a, lo, &c0, &L);
  const int64_t tp = min(max((int64_t)a.cup[lo] + (t - c0), (int64_t)0), a.Tp - 1);
  const int eb = a.dtype == Dtype::BF16 ? 2 : 4;
  const int64_t xr = (int64_t)a.H * a.P * eb, br = (int64_t)a.G * a.N * eb;
  copy_row(static_cast<const char*>(a.dxp) + tp * xr, static_cast<char*>(a.dx) + t * xr, (int)(xr / 16));
  copy_row(static_cast<const char*>(a.dBp) + tp * br, static_cast<char*>(a.dB) + t * br, (int)(br / 16));
  copy_row(static_cast<const char*>(a.dCp) + tp * br, static_cast<char*>(a.dC) + t * br, (int)(br / 16));
  for (int h = threadIdx.x; h < a.H; h += kBwThreads) a.ddt[t * a.H + h] = a.ddtp[tp * a.H + h];
}

__global__ __launch_bounds__(kBwThreads) void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)kBwThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBwThreads)
    p[i] = 0.0f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + kBwThreads - 1) / kBwThreads, 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kBwThreads), 0, s, p, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(kBwThreads) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)kBwThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBwThreads)
    p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + kBwThreads - 1) / kBwThreads, 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(kBwThreads), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_backward_pad(const PadArgs& a, int stage, hipStream_t s) {
  const dim3 blk(kBwThreads);
  if (stage == 0) {
    hipLaunchKernelGGL(bwd_pad_offsets_kernel, dim3(1), blk, 0, s, a);
    if (a.Tp > 0) hipLaunchKernelGGL(bwd_pad_kernel, dim3((unsigned)a.Tp), blk, 0, s, a);
  } else {
    if (a.T > 0) hipLaunchKernelGGL(bwd_unpad_kernel, dim3((unsigned)a.T), blk, 0, s, a);
  }
  return hipGetLastError();
}

template <class E>
static hipError_t launch_glue(const BwdProblem& b, int stage, hipStream_t s) {
  const dim3 blk(kBwThreads);
  switch (stage) {
    case 0:
      // the prep kernel's first workgroup clears dA and dD; without tokens a
      // kernel of its own does
      if (b.total > 0)
        hipLaunchKernelGGL((bwd_prep_kernel<E>), dim3((unsigned)b.total), blk, 0, s, b);
      else
        hipLaunchKernelGGL(bwd_zero_kernel, dim3(1), blk, 0, s, b);
      if ((b.h0c != nullptr || b.dfb != nullptr) && b.nseq > 0)
        hipLaunchKernelGGL(bwd_prep_states_kernel, dim3((unsigned)(b.nseq * b.H * b.NK)), blk, 0, s, b);
      break;
    case 1:
      if (b.total > 0) {
        if (b.y_c != nullptr) hipLaunchKernelGGL((bwd_reduce_kernel<E>), dim3((unsigned)b.total), blk, 0, s, b);
        // (the chunk-local d(ell) kernel forms the per-token terms itself)
        if (!b.chunked_dl) hipLaunchKernelGGL((bwd_token_kernel<E>), dim3((unsigned)b.total), blk, 0, s, b);
      }
      if (b.chunked_dl) {
        if (b.total > 0) {
          const hipError_t e = launch_backward_dl(b, s);
          if (e != hipSuccess) return e;
        }
        if (b.nseq > 0 && (b.dD != nullptr || b.dinit != nullptr))
          hipLaunchKernelGGL(bwd_seqsum_kernel, dim3((unsigned)(b.nseq * b.H)), blk, 0, s, b);
      } else if (b.nseq > 0) {
        const dim3 grid((unsigned)(b.nseq * b.H * b.nseg));
        hipLaunchKernelGGL(bwd_segsum_kernel, grid, blk, 0, s, b);
        hipLaunchKernelGGL(bwd_scan_kernel, grid, blk, 0, s, b);
      }
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
