// k8_backward_dl.hip -- d(ell) of the SSD backward pass, chunk by chunk.
//
// d(ell_t) (ell = dt A, the log-decay) is the sum of W[i, j] = L[i, j]
// (C_i . B_j)(dy_i . x'_j) over every pair that straddles t (j < t <= i), with
// L[i, j] = a_{j+1} ... a_i the 1-SS mask ("Transformers是SSMs…(一)" §3.2.2)
// and x' the input as the state sees it.  Split by the chunk c = [s, e] of t
// (the block decomposition of "LLM(十一)——Mamba" §3.5):
//   pairs inside the chunk      A_c(t) = sum_{k=t..e} (row_k - col_k), with
//                               row_k = sum_{j<k} W[k, j], col_k = sum_{i>k} W[i, k];
//   i in the chunk, j before it sum_{i=t..e} dy_i . (exp(Acs_i) Hin_c C_i);
//   i after it, j in the chunk  sum_{j=s..t-1} x'_j . (exp(Lam_c - Acs_j) Gout_c B_j);
//   i after it, j before it     <Gout_c, exp(Lam_c) Hin_c>,
// where Hin_c is the state entering the chunk (the forward's passed state,
// with the initial state for the first chunk) and Gout_c = dL/dh_e from the
// tokens after the chunk (a_{e+1} G_{e+1}; dfinal after the last chunk), the
// passed state of the time-reversed pass.  No sum runs past one chunk, so the
// passed states as the passes store them (bf16) are accurate enough, and W is
// formed in fp32 from exact products of the inputs (C B^T and dY X^T on the
// matrix cores), so no rounded output enters.  Used for bf16 inputs when
// every sequence is a whole number of chunks (then the reversed pass's chunks
// coincide with the forward's).
//
// Kernel 1, per (chunk, head, row-tile set): the row and column sums of W,
// the passed-state terms, and the per-token terms of the row tiles' tokens
// (dx = sx dx' + D dy, x . dx', x . dy: sx = dt with the dt-scaled input, else
// 1; dx' from the reversed pass).  Each of the 4 waves owns one row tile I of 32
// tokens and keeps its i-side rows (C_I, dY_I) in registers as MFMA operands
// (lane: one token row, 8 consecutive k).  The j-side tiles (B_J, X_J) and the
// passed states Hin, Gout are copied straight from memory into LDS by the
// load-to-LDS instruction (no registers stage them), each instruction a block
// of whole consecutive rows (8 cache lines); within a row the 16-byte vectors
// are XOR-swizzled by the row so that MFMA operand reads (32 rows, one vector
// each) hit distinct LDS banks.  The j-side tiles pass through a ring of
// kRing buffers with kRing - 1 tiles in flight.  At step J each wave with I >= J forms the
// 32x32 tile W[I, J] once, with the lane holding token i; row sums are sums of
// the lane's values, column sums a butterfly across the 32 lanes.  With 8 row
// tiles (256-token chunks) a chunk's tiles are split over two workgroups,
// {0, 3, 5, 6} and {1, 2, 4, 7}, 18 tile pairs each.  The decay of an
// off-diagonal tile factors as exp(Acs_i - Acs_j) = exp(Acs_i - a) exp(a - Acs_j)
// with a = Acs at the end of tile J; both factors are at most 1.
#include "ssd_device.hpp"
#include "ssd_lds.hpp"

namespace ssd {

constexpr int kDlThreads = 256;

template <int N>
struct RowOps {
  uint4 bc[N / 16];         // B or C
  uint4 xd[kHeadDim / 16];  // x or dy
};

// 32x32 tile D[m][n] = sum_k A_m[k] B_n[k] (lane: m = n = lr); acc[r] holds
// m = 8 (r / 4) + 4 lg + r % 4.
template <int K>
__device__ __forceinline__ floatx16_t prod(const uint4 (&a)[K / 16], const uint4 (&b)[K / 16]) {
  floatx16_t acc = zero16();
#pragma unroll
  for (int s = 0; s < K / 16; ++s) acc = mfma32x32x16(a[s], b[s], acc);
  return acc;
}

// c + a.lo b.lo + a.hi b.hi for two packed bf16 pairs (one instruction)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// DPP move within rows of 16 lanes, written only to the lanes of the banks
// in BM (bank i: lanes 4i .. 4i + 3 of each row); the other lanes keep old.
template <int CTRL, int BM>
__device__ __forceinline__ float dpp_banks(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xf, BM, false));
}

// Sum of v[r] over the 32 lanes of each lane half: returns the sum for
// r = 8 b4 + 4 b3 + 2 b2 + b1 (bits of lr), the same in lanes lr and lr ^ 1.
// Each level halves the values a lane holds: it keeps the half its bit
// selects and adds its partner's copy of that half.  No level goes through
// LDS: lane distance 16 by v_permlane16_swap (it exchanges the odd 16-lane row
// of its first operand with the even row of its second, so after exchanging
// (v[k], v[8 + k]) the two results add up to the pair's v[k] in the lower row
// and its v[8 + k] in the upper), distance 8 by a row rotation, distance 4 by
// two bank-masked row shifts, distances 2 and 1 by quad permutations.
__device__ __forceinline__ float lane_col_sums(const float (&v)[16], int lr) {
  float v8[8], v4[4], v2[2];
  const bool b3 = lr & 8, b2 = lr & 4, b1 = lr & 2;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[8 + k]), false, false);
    v8[k] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b3 ? v8[4 + k] : v8[k], send = b3 ? v8[k] : v8[4 + k];
    v4[k] = keep + dpp_move0<0x128>(send);  // row_ror:8
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b2 ? v4[2 + k] : v4[k], send = b2 ? v4[k] : v4[2 + k];
    // lanes 4..7 of every 8 read lane - 4 (row_shr:4), lanes 0..3 lane + 4 (row_shl:4)
    const float recv = dpp_banks<0x104, 0x5>(dpp_banks<0x114, 0xA>(0.0f, send), send);
    v2[k] = keep + recv;
  }
  const float keep = b1 ? v2[1] : v2[0], send = b1 ? v2[0] : v2[1];
  const float v1 = keep + dpp_move0<0x4E>(send);  // quad_perm [2, 3, 0, 1]
  return v1 + dpp_move0<0xB1>(v1);                // quad_perm [1, 0, 3, 2]
}

template <int Q, int N>
struct DlCfg {
  static constexpr int P = kHeadDim;
  static constexpr int NI = Q / 32;
  static constexpr int NS = NI == 8 ? 2 : 1;      // workgroups per (chunk, head)
  static constexpr int kRing = N <= 128 ? 3 : 2;  // j-side tile buffers
  static constexpr int VB = N / 8, VX = P / 8;    // 16-byte vectors per row of B and of x
  static constexpr int NBB = 32 * VB / 64;        // load-to-LDS instructions (1 KB) of B_J
  static constexpr int NB = NBB + 32 * VX / 64;   // ... of one j-side tile (B_J, then X_J)
  static constexpr int TILE = 32 * (VB + VX);     // vectors of one j-side tile
  static constexpr int DPW = (NB + 3) / 4;        // per wave per tile
  static constexpr int NBS = P * VB / 64;         // instructions of Hin (and of Gout)
  static constexpr int SPW = (NBS + 3) / 4;
  // loads a wave issues after the step sizes of the prologue
  static constexpr int kAfterDt = N / 16 + 2 * (P / 16) + DPW * (kRing < NI ? kRing : NI) + 2 * SPW;
  // loads a wave issues after j-side tile J and before the wait at the top of
  // step J (tiles J+1 .. of the prologue or of earlier steps, and Hin)
  static constexpr int after(int J) {
    const int last_prologue = kRing - 1 < NI - 1 ? kRing - 1 : NI - 1;
    int hi = J + kRing - 2 > last_prologue ? J + kRing - 2 : last_prologue;
    if (hi > NI - 1) hi = NI - 1;
    if (hi < J) hi = J;
    return DPW * (hi - J) + (J <= last_prologue ? SPW : 0);
  }
};

// wait_vm<Cfg::after(J)> for a J that unrolling makes constant
template <class Cfg>
__device__ __forceinline__ void wait_tile(int J) {
  switch (J) {
    case 0: wait_vm<Cfg::after(0)>(); break;
    case 1: wait_vm<Cfg::after(1)>(); break;
    case 2: wait_vm<Cfg::after(2)>(); break;
    case 3: wait_vm<Cfg::after(3)>(); break;
    case 4: wait_vm<Cfg::after(4)>(); break;
    case 5: wait_vm<Cfg::after(5)>(); break;
    case 6: wait_vm<Cfg::after(6)>(); break;
    default: wait_vm<Cfg::after(7)>(); break;
  }
}

// row tile of wave w in workgroup `half` (-1: none)
template <int NI>
__device__ __forceinline__ int dl_tile(int half, int w) {
  if constexpr (NI == 8) {
    const int t0 = half == 0 ? 0x6530 : 0x7421;  // {0,3,5,6} / {1,2,4,7}, 4 bits each
    return (t0 >> (4 * w)) & 0xf;
  } else {
    return w < NI ? w : -1;
  }
}

template <int Q, int N>
__global__ __launch_bounds__(kDlThreads) __attribute__((amdgpu_waves_per_eu(N <= 128 ? 2 : 1)))
void bwd_dl_kernel(BwdProblem b) {
  using Cfg = DlCfg<Q, N>;
  constexpr int P = Cfg::P, NI = Cfg::NI, NS = Cfg::NS, RB = Cfg::kRing, NB = Cfg::NB, NBB = Cfg::NBB;
  // ring buffers as separate arrays: an unrolled step reads one of them while
  // the loads into another are in flight, which the compiler can then tell apart
  __shared__ __align__(16) uint4 ring0[Cfg::TILE];
  __shared__ __align__(16) uint4 ring1[Cfg::TILE];
  __shared__ __align__(16) uint4 ring2[RB > 2 ? Cfg::TILE : 1];
  __shared__ __align__(16) uint4 Hs[P * Cfg::VB];
  __shared__ __align__(16) uint4 Gs[P * Cfg::VB];
  __shared__ __align__(16) float acs[Q];
  __shared__ __align__(16) float fd[Q];  // exp(a_J - Acs_j) (x dt_j): j-factor of the decay
  __shared__ __align__(16) float dts[Q];
  __shared__ float cols[4][Q];  // per wave (filled after the steps)
  __shared__ float dterm[Q];
  __shared__ float red[kDlThreads / 64];
  const int H = b.H, G = b.G;

  // the workgroups of one chunk on one XCD: they share its B and C rows in L2
  const int64_t bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int half = (int)(bid % NS);
  const int64_t kh = bid / NS;
  const int h = (int)(kh % H);
  const int64_t k = kh / H;
  const BwdChunk ch = bwd_chunk(b, k, Q);
  const int64_t CPS = ch.CPS, c = ch.c, t0 = ch.t0;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave choices in scalar registers
  const float Ah = b.A[h];
  const bool xdt = b.x_times_dt != 0;
  const float Dh = b.D != nullptr ? b.D[h] : 0.0f;
  const int I = dl_tile<NI>(half, wid);

  const uint16_t* xb = reinterpret_cast<const uint16_t*>(b.x) + (t0 * H + h) * P;
  const uint16_t* dyb = reinterpret_cast<const uint16_t*>(b.dy) + (t0 * H + h) * P;
  const uint16_t* Bb = reinterpret_cast<const uint16_t*>(b.B) + (t0 * G + g) * N;
  const uint16_t* Cb = reinterpret_cast<const uint16_t*>(b.C) + (t0 * G + g) * N;
  const int64_t xs = (int64_t)H * P, bs = (int64_t)G * N;  // token strides
  // Gout = a_{e+1} G_{e+1}: the reversed pass's passed state of its chunk
  // CPS-1-c; after the last chunk it is dfinal itself (no decay)
  const uint16_t* hin = reinterpret_cast<const uint16_t*>(b.hin_e) + (k * H + h) * (int64_t)(P * N);
  const uint16_t* gout =
      reinterpret_cast<const uint16_t*>(b.gin_e) + ((ch.s0 / Q + (CPS - 1 - c)) * H + h) * (int64_t)(P * N);

  // j-side tile J into ring buffer J % RB.  Instruction q < NBB copies rows
  // 64 q / VB .. of B_J (LDS slots 64 q + lane), the others rows of X_J after
  // them; lane L takes the vector that the swizzle puts in its slot.  Wave w
  // issues instructions w, w + 4, ... (a repeated one, when NB is not a
  // multiple of 4, copies the same bytes again).  A lane's byte offset from the
  // tile's first row is the same for every tile (computed once, 32-bit: the
  // host bounds 32 token rows of x below 2^31 bytes); the tile's own offset is
  // uniform.
  constexpr int VB = Cfg::VB, VX = Cfg::VX;
  auto slot = [&](int r) -> uint4* { return r == 0 ? ring0 : (r == 1 ? ring1 : ring2); };
  uint32_t coff[Cfg::DPW];
#pragma unroll
  for (int u = 0; u < Cfg::DPW; ++u) {
    const int q = (wid + 4 * u) % NB;
    if (q < NBB) {
      const int r = (64 * q + lane) / VB, c = lane % VB;
      coff[u] = 2u * ((uint32_t)r * (uint32_t)bs + 8u * (uint32_t)(c ^ (swz_slot<VB>(r, 0) - r * VB)));
    } else {
      const int r = (64 * (q - NBB) + lane) / VX, c = lane % VX;
      coff[u] = 2u * ((uint32_t)r * (uint32_t)xs + 8u * (uint32_t)(c ^ (swz_slot<VX>(r, 0) - r * VX)));
    }
  }
  auto issue_tile = [&](int J) {
    uint4* dst = slot(J % RB);
#pragma unroll
    for (int u = 0; u < Cfg::DPW; ++u) {
      const int q = (wid + 4 * u) % NB;
      const char* tile = q < NBB ? reinterpret_cast<const char*>(Bb + 32 * J * bs)
                                 : reinterpret_cast<const char*>(xb + 32 * J * xs);
      lds_copy16(reinterpret_cast<const uint16_t*>(tile + coff[u]), dst + q * 64);
    }
  };
  // Hin or Gout (P rows of N, contiguous): instruction q copies slots 64 q ..
  auto issue_state = [&](const uint16_t* src0, uint4* dst) {
#pragma unroll
    for (int u = 0; u < Cfg::SPW; ++u) {
      const int q = (wid + 4 * u) % Cfg::NBS;
      const int r = (64 * q + lane) / VB, c = lane % VB;
      lds_copy16(src0 + r * N + 8 * (c ^ (swz_slot<VB>(r, 0) - r * VB)), dst + q * 64);
    }
  };

  // ---- prologue: the step sizes, the i-side rows of this wave's row tile and
  // their dx' rows (a wave without one loads tile 0 and leaves it unused), then
  // tile 0, Gout, tiles 1 .. RB - 1 and Hin into LDS (in this order: the waits
  // count them).  The chunk-local cumsums of dt A come from the forward's
  // chunk-state kernel (contiguous per (chunk, head)); the step sizes (one
  // cache line per token) only with the dt-scaled input (wave 0)
  constexpr int R = Q / 64;
  float acl[R], dtl[R];
  if (wid == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) acl[i] = b.acs_f[(k * H + h) * Q + lane * R + i];
    if (xdt) {
#pragma unroll
      for (int i = 0; i < R; ++i) dtl[i] = b.dt[(t0 + lane * R + i) * H + h];
    }
  }
  const float dtnext = c + 1 < CPS ? b.dt[(t0 + Q) * H + h] : 0.0f;
  RowOps<N> io;
  uint4 dxr[P / 16];  // dx' rows of the i-side tokens, as io.xd (then dx)
  float sxd = 0.0f, sxy = 0.0f;  // partial x . dx' and x . dy of the lane's token
  {
    const int i = 32 * max(I, 0) + lr;
#pragma unroll
    for (int st = 0; st < N / 16; ++st) io.bc[st] = *reinterpret_cast<const uint4*>(Cb + i * bs + 16 * st + 8 * lg);
#pragma unroll
    for (int st = 0; st < P / 16; ++st) io.xd[st] = *reinterpret_cast<const uint4*>(dyb + i * xs + 16 * st + 8 * lg);
    // dx' of token i comes from the reversed pass at the reversed position
    const int64_t f = ch.s0 + (ch.L - 1 - (c * Q + i));
    const uint16_t* dxp = reinterpret_cast<const uint16_t*>(b.y_x8) + (f * H + h) * P + 8 * lg;
#pragma unroll
    for (int st = 0; st < P / 16; ++st) dxr[st] = *reinterpret_cast<const uint4*>(dxp + 16 * st);
  }
  issue_tile(0);
  issue_state(gout, Gs);
#pragma unroll
  for (int J = 1; J < RB && J < NI; ++J) issue_tile(J);
  issue_state(hin, Hs);
  wait_vm<Cfg::kAfterDt>();  // the cumsums and step sizes (loaded first)
  if (wid == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      acs[lane * R + i] = acl[i];
      if (xdt) dts[lane * R + i] = dtl[i];
    }
  }
  dl_barrier();
  for (int i = tid; i < Q; i += kDlThreads)
    fd[i] = __expf(acs[32 * (i / 32) + 31] - acs[i]) * (xdt ? dts[i] : 1.0f);
  const float lam = acs[Q - 1];
  const float anext = c + 1 < CPS ? __expf(dtnext * Ah) : 1.0f;
  const int i_l = 32 * I + lr;
  const float ai = I >= 0 ? acs[i_l] : 0.0f;

  float rowpart = 0.0f;
  // column sums of step J (lanes with even lr; see lane_col_sums), kept in
  // registers: LDS accesses during the steps would wait for every copy in flight
  float colreg[NI];
#pragma unroll
  for (int J = 0; J < NI; ++J) colreg[J] = 0.0f;
#pragma unroll
  for (int J = 0; J < NI; ++J) {
    // tile J (and, at J = 0, Gout) in LDS for every wave
    wait_tile<Cfg>(J);
    dl_barrier();
    // every wave is past step J - 1: its buffer takes tile J - 1 + RB
    if (J >= 1 && J - 1 + RB < NI) issue_tile(J - 1 + RB);
    const uint4* tb = slot(J % RB);
    // d-term of tile J: by one workgroup of the chunk (J's parity picks it when
    // there are two), in a wave without a tile pair at this step if one exists
    int dw = -1;
    if (NS == 1 || (J & 1) == half) {
      dw = J % 4;
      for (int w = 3; w >= 0; --w)
        if (dl_tile<NI>(half, w) < J) dw = w;
    }
    if (I >= J || wid == dw) {
      RowOps<N> jo;
#pragma unroll
      for (int st = 0; st < N / 16; ++st) jo.bc[st] = tb[swz_slot<VB>(lr, 2 * st + lg)];
      if (I >= J) {
#pragma unroll
        for (int st = 0; st < P / 16; ++st) jo.xd[st] = tb[32 * VB + swz_slot<VX>(lr, 2 * st + lg)];
        // lane holds i: m = j (A = B_J, X_J), n = i (B = C_I, dY_I)
        const floatx16_t gR = prod<N>(jo.bc, io.bc);
        const floatx16_t sR = prod<P>(jo.xd, io.xd);
        float w[16];
        if (I == J) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int m0 = 8 * a + 4 * lg;
            const float4 aJ = *reinterpret_cast<const float4*>(&acs[32 * J + m0]);
            const float4 dJ =
                xdt ? *reinterpret_cast<const float4*>(&dts[32 * J + m0]) : make_float4(1.f, 1.f, 1.f, 1.f);
            const float aJq[4] = {aJ.x, aJ.y, aJ.z, aJ.w}, dJq[4] = {dJ.x, dJ.y, dJ.z, dJ.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 4 * a + q;
              const float e = m0 + q < lr ? __expf(ai - aJq[q]) * dJq[q] : 0.0f;
              w[r] = e * gR[r] * sR[r];
            }
          }
        } else {
          const float ei = __expf(ai - acs[32 * J + 31]);
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float4 fJ = *reinterpret_cast<const float4*>(&fd[32 * J + 8 * a + 4 * lg]);
            const float fJq[4] = {fJ.x, fJ.y, fJ.z, fJ.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) w[4 * a + q] = ei * fJq[q] * gR[4 * a + q] * sR[4 * a + q];
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) rowpart += w[r];
        colreg[J] = lane_col_sums(w, lr);
        if (I == J) {
          // per-token terms of the row tile (its x rows are tile J's here):
          // dx = sx dx' + D dy (sx = dt with the dt-scaled input, else 1),
          // x . dx' (a d(dt) term) and x . dy (the dD term); stored after the
          // steps (a store would hold up the next step's wait for its tile:
          // the wait counts stores too)
#pragma unroll
          for (int st = 0; st < P / 16; ++st) {
            const uint32_t xw[4] = {jo.xd[st].x, jo.xd[st].y, jo.xd[st].z, jo.xd[st].w};
            const uint32_t yw[4] = {io.xd[st].x, io.xd[st].y, io.xd[st].z, io.xd[st].w};
            const uint32_t dw[4] = {dxr[st].x, dxr[st].y, dxr[st].z, dxr[st].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sxd = dot2_bf16(xw[e], dw[e], sxd);
              sxy = dot2_bf16(xw[e], yw[e], sxy);
            }
          }
          if (xdt || Dh != 0.0f) {  // else dx = dx' as it is
            const float sx = xdt ? dts[i_l] : 1.0f;
#pragma unroll
            for (int st = 0; st < P / 16; ++st) {
              const uint32_t yw[4] = {io.xd[st].x, io.xd[st].y, io.xd[st].z, io.xd[st].w};
              const uint32_t dw[4] = {dxr[st].x, dxr[st].y, dxr[st].z, dxr[st].w};
              uint32_t ow[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                ow[e] = pack_bf16x2(sx * bf16_lo(dw[e]) + Dh * bf16_lo(yw[e]), sx * bf16_hi(dw[e]) + Dh * bf16_hi(yw[e]));
              dxr[st] = make_uint4(ow[0], ow[1], ow[2], ow[3]);  // dx' in, dx out
            }
          }
        }
      }
      if (wid == dw) {
        // dterm_j = exp(Lam - Acs_j) x'_j . (Gout B_j): A = Gout rows p, B = B_J
        float dtm = 0.0f;
#pragma unroll
        for (int pt = 0; pt < P / 32; ++pt) {
          uint4 ga[N / 16];
#pragma unroll
          for (int st = 0; st < N / 16; ++st) ga[st] = Gs[swz_slot<VB>(32 * pt + lr, 2 * st + lg)];
          const floatx16_t gx = prod<N>(ga, jo.bc);
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            // x_j at p = 32 pt + 8 a + 4 lg .. + 4: half lg of vector 4 pt + a of row lr
            const uint4 x4 = tb[32 * VB + swz_slot<VX>(lr, 4 * pt + a)];
            const uint2 xv = lg ? make_uint2(x4.z, x4.w) : make_uint2(x4.x, x4.y);
            dtm += gx[4 * a] * bf16_lo(xv.x) + gx[4 * a + 1] * bf16_hi(xv.x) + gx[4 * a + 2] * bf16_lo(xv.y) +
                   gx[4 * a + 3] * bf16_hi(xv.y);
          }
        }
        dtm += __shfl_xor(dtm, 32);
        const int j_l = 32 * J + lr;
        if (lg == 0) dterm[j_l] = __expf(lam - acs[j_l]) * anext * dtm * (xdt ? dts[j_l] : 1.0f);
      }
    }
  }

  // ---- Hin in LDS; row sums and yterm_i = exp(Acs_i) dy_i . (Hin C_i) of the
  // wave's row tile
  wait_vm<0>();
  if ((lr & 1) == 0) {
    const int r = lr >> 1;  // 8 b4 + 4 b3 + 2 b2 + b1
#pragma unroll
    for (int J = 0; J < NI; ++J) cols[wid][32 * J + 8 * (r >> 2) + 4 * lg + (r & 3)] = colreg[J];
  }
  __syncthreads();
  if (I >= 0) {
    const float rp = rowpart + __shfl_xor(rowpart, 32);
    // dy of token i at p = 16 st + 8 h + 4 lg .. + 3 for both halves h, from the
    // dy rows in registers (io.xd[st] of lane half h holds p = 16 st + 8 h ..):
    // v_permlane32_swap exchanges the upper 32 lanes of its first operand with
    // the lower 32 of its second, so after exchanging (words 0 and 2), (words 1
    // and 3) of io.xd[st] the first results hold every lane's words for h = 0
    // and the second for h = 1
    uint2 dyh[P / 16][2];
#pragma unroll
    for (int st = 0; st < P / 16; ++st) {
      const auto s02 = __builtin_amdgcn_permlane32_swap(io.xd[st].x, io.xd[st].z, false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(io.xd[st].y, io.xd[st].w, false, false);
      dyh[st][0] = make_uint2(s02[0], s13[0]);
      dyh[st][1] = make_uint2(s02[1], s13[1]);
    }
    float yt = 0.0f;
#pragma unroll
    for (int pt = 0; pt < P / 32; ++pt) {
      uint4 ha[N / 16];
#pragma unroll
      for (int st = 0; st < N / 16; ++st) ha[st] = Hs[swz_slot<VB>(32 * pt + lr, 2 * st + lg)];
      // lane holds token i (n), value r holds p = 32 pt + 8 (r / 4) + 4 lg + r % 4 (m)
      const floatx16_t hy = prod<N>(ha, io.bc);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint2 dv = dyh[2 * pt + a / 2][a % 2];  // p = 32 pt + 8 a + 4 lg .. + 3
        yt += hy[4 * a] * bf16_lo(dv.x) + hy[4 * a + 1] * bf16_hi(dv.x) + hy[4 * a + 2] * bf16_lo(dv.y) +
              hy[4 * a + 3] * bf16_hi(dv.y);
      }
    }
    yt += __shfl_xor(yt, 32);
    if (lg == 0) b.dl_v[h * b.total + t0 + i_l] = rp + __expf(ai) * yt;
  }
  // ---- column sums of this workgroup, d-terms of its tiles; <Gout, exp(Lam)
  // Hin> (pairs on both sides of the chunk) from the first workgroup
  float* colout = b.dl_cols + ((int64_t)half * H + h) * b.total + t0;
  for (int i = tid; i < Q; i += kDlThreads) {
    colout[i] = cols[0][i] + cols[1][i] + cols[2][i] + cols[3][i];
    if (NS == 1 || ((i / 32) & 1) == half) b.dl_u[h * b.total + t0 + i] = dterm[i];
  }
  if (half == 0) {
    float kpart = 0.0f;
    for (int v = tid; v < P * VB; v += kDlThreads) {  // same swizzle in both: any order
      const uint4 hv = Hs[v], gv = Gs[v];
      kpart += bf16_lo(hv.x) * bf16_lo(gv.x) + bf16_hi(hv.x) * bf16_hi(gv.x) + bf16_lo(hv.y) * bf16_lo(gv.y) +
               bf16_hi(hv.y) * bf16_hi(gv.y) + bf16_lo(hv.z) * bf16_lo(gv.z) + bf16_hi(hv.z) * bf16_hi(gv.z) +
               bf16_lo(hv.w) * bf16_lo(gv.w) + bf16_hi(hv.w) * bf16_hi(gv.w);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kpart += __shfl_xor(kpart, off);
    if (lane == 0) red[wid] = kpart;
    __syncthreads();
    if (tid == 0) b.dl_kc[k * H + h] = anext * __expf(lam) * (red[0] + red[1] + red[2] + red[3]);
  }
  // ---- the row tile's per-token terms, stored last: no later wait or barrier
  // of this workgroup then waits for these stores
  if (I >= 0) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(b.dx) + ((t0 + i_l) * H + h) * P + 8 * lg;
#pragma unroll
    for (int st = 0; st < P / 16; ++st) *reinterpret_cast<uint4*>(dst + 16 * st) = dxr[st];
    const float sd = sxd + __shfl_xor(sxd, 32), sy = sxy + __shfl_xor(sxy, 32);
    if (lg == 0) {
      b.rd[(int64_t)h * b.total + t0 + i_l] = sd;
      b.ud[(int64_t)h * b.total + t0 + i_l] = sy;
    }
  }
}

// Kernel 2, one wave per (chunk, head), the heads of a block of HB in one
// workgroup:
//   d(ell_t) = Vtot + K + sum_{k<t} (u_k - v_k),  v = row - col + yterm, u = dterm
// dt and d(dt) are token-major (Ttot, H): the block's (token, head) values go
// through an LDS tile, loaded and stored with consecutive threads on
// consecutive heads of a token row, instead of one cache line per token and head.
constexpr int kDlScanHeads = 8;
template <int Q>
__global__ __launch_bounds__(64 * kDlScanHeads) void bwd_dl_scan_kernel(BwdProblem b, int HB) {
  constexpr int R = Q / 64;
  constexpr int NS = Q == 256 ? 2 : 1;
  constexpr int TP = kDlScanHeads + 1;  // LDS pitch of a token row (odd: a column read hits distinct banks)
  __shared__ float tile[Q * TP];
  const int H = b.H;
  const int nhb = H / HB;
  const int64_t k = blockIdx.x / nhb;
  const int h0 = (int)(blockIdx.x % nhb) * HB;
  const int64_t t0 = k * Q;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  // step sizes of the block: element e = token e / HB, head e % HB
  for (int e = tid; e < Q * HB; e += 64 * kDlScanHeads)
    tile[(e / HB) * TP + e % HB] = b.dt[(t0 + e / HB) * H + h0 + e % HB];
  __syncthreads();
  const bool active = wid < HB;  // waves past the block's heads only help with the tile
  const int h = h0 + (active ? wid : 0);
  float run = 0.0f, sdA = 0.0f;
  float du[R], dd[R];
  if (active) {
    const float Ah = b.A[h];
    const int64_t base = h * b.total + t0 + lane * R;
    float dtv[R], vsum = 0.0f, wsum = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float v = b.dl_v[base + i];
#pragma unroll
      for (int hf = 0; hf < NS; ++hf) v -= b.dl_cols[(int64_t)hf * H * b.total + base + i];
      vsum += v;
      du[i] = b.dl_u[base + i] - v;
      wsum += du[i];
      dtv[i] = tile[(lane * R + i) * TP + wid];
    }
    float vtot = vsum;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) vtot += __shfl_xor(vtot, off);
    const float incl = wave_inclusive_sum(wsum);
    run = vtot + b.dl_kc[k * H + h] + (incl - wsum);  // everything before this lane's tokens
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t tok = t0 + lane * R + i;
      dd[i] = Ah * run + (b.x_times_dt ? b.rd[h * b.total + tok] : 0.0f);
      sdA += dtv[i] * run;
      run += du[i];
    }
  }
  __syncthreads();  // every wave has read its step sizes
  if (active) {
#pragma unroll
    for (int i = 0; i < R; ++i) tile[(lane * R + i) * TP + wid] = dd[i];
  }
  __syncthreads();
  for (int e = tid; e < Q * HB; e += 64 * kDlScanHeads)
    b.ddt[(t0 + e / HB) * H + h0 + e % HB] = tile[(e / HB) * TP + e % HB];
  if (active) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sdA += __shfl_xor(sdA, off);
    // the chunk's share of dA, in place of the term read above (summed over
    // the chunks by bwd_dA_sum_kernel: one value per (chunk, head), no
    // atomics on the H addresses of dA, which every chunk would contend for)
    if (lane == 0) b.dl_kc[k * H + h] = sdA;
  }
}

// dA_h = the sum of the chunks' shares, in chunk order (fp64 accumulation)
__global__ __launch_bounds__(256) void bwd_dA_sum_kernel(BwdProblem b, int64_t chunks) {
  __shared__ double red[4];
  const int h = blockIdx.x;
  double acc = 0.0;
  for (int64_t k = threadIdx.x; k < chunks; k += 256) acc += b.dl_kc[k * b.H + h];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) b.dA[h] = (float)(red[0] + red[1] + red[2] + red[3]);
}

bool backward_dl_supported(Dtype dt, int Q, int N, int64_t H) {
  return dt == Dtype::BF16 && H > 0 && H <= ((int64_t)1 << 19) && (Q == 64 || Q == 128 || Q == 256) &&
         (N == 16 || N == 32 || N == 64 || N == 128 || N == 256) && !(Q == 256 && N == 256);
}

template <int Q>
static void launch_dl_q(const BwdProblem& b, int64_t chunks, hipStream_t s) {
  const dim3 grid((unsigned)(chunks * b.H * (Q == 256 ? 2 : 1))), block(kDlThreads);
  switch (b.N) {
    case 16: hipLaunchKernelGGL((bwd_dl_kernel<Q, 16>), grid, block, 0, s, b); break;
    case 32: hipLaunchKernelGGL((bwd_dl_kernel<Q, 32>), grid, block, 0, s, b); break;
    case 64: hipLaunchKernelGGL((bwd_dl_kernel<Q, 64>), grid, block, 0, s, b); break;
    case 128: hipLaunchKernelGGL((bwd_dl_kernel<Q, 128>), grid, block, 0, s, b); break;
    default:
      if constexpr (Q <= 128) hipLaunchKernelGGL((bwd_dl_kernel<Q, 256>), grid, block, 0, s, b);
      break;
  }
  // heads per scan workgroup: the largest divisor of H up to kDlScanHeads
  int hb = 1;
  for (int d = kDlScanHeads; d >= 1; --d)
    if (b.H % d == 0) { hb = d; break; }
  hipLaunchKernelGGL((bwd_dl_scan_kernel<Q>), dim3((unsigned)(chunks * (b.H / hb))), dim3(64 * kDlScanHeads), 0, s, b,
                     hb);
  hipLaunchKernelGGL(bwd_dA_sum_kernel, dim3((unsigned)b.H), dim3(256), 0, s, b, chunks);
}

hipError_t launch_backward_dl(const BwdProblem& b, hipStream_t s) {
  if (!backward_dl_supported(b.dtype, b.Q, b.N, b.H) || b.total % b.Q != 0 || (b.cu == nullptr && b.seqlen % b.Q != 0))
    return hipErrorInvalidValue;
  const int64_t chunks = b.total / b.Q;
  if (chunks == 0) return hipSuccess;
  switch (b.Q) {
    case 64: launch_dl_q<64>(b, chunks, s); break;
    case 128: launch_dl_q<128>(b, chunks, s); break;
    default: launch_dl_q<256>(b, chunks, s); break;
  }
  return hipGetLastError();
}

}  // namespace ssd
