// k9_backward_dbdc.hip -- dB and dC of the SSD backward pass, chunk by chunk,
// summed over the heads of a group before the products with B and C.
//
// Within a chunk, with M_h[t, j] = L_h[t, j] (dy_t . x'_j) for j <= t (L_h the
// 1-SS mask of head h, exp(Acs_t - Acs_j): "Transformers是SSMs…(一)" §3.2.2;
// x' the input as the state sees it), the block decomposition of
// "LLM(十一)——Mamba" §3.5 gives for the group's heads h
//   dC_t = sum_h [ sum_{j<=t} M_h[t, j] B_j + exp(Acs_t) Hin_h^T dy_t ]
//   dB_j = sum_h [ sum_{t>=j} M_h[t, j] C_t + a_next exp(Lam - Acs_j) Gout_h^T x'_j ]
// where Hin_h is the state entering the chunk (the forward's passed state,
// the initial state for the first chunk), Gout_h the adjoint after it (a_next
// times the time-reversed pass's passed state; dfinal after the last chunk)
// and Lam = Acs at the chunk's last token.  B and C are shared by a group's
// heads, so the head sum is taken on the Q x Q matrix first: Msum = sum_h M_h,
// then dC = Msum B + ..., dB = Msum^T C + ...  -- one product with B and one
// with C per chunk, where per-head passes would need one per head.
//
// Workgroup: one chunk, one group, 64 columns of N and a subset of the group's
// heads; one wave per 32-token tile of the chunk (Q / 32 waves).  Per head, x
// and dy of the chunk are copied into LDS by the load-to-LDS instruction
// (double buffered: the next head's copies, issued a few at a time between
// this head's tiles, run during its products; rows XOR-swizzled so that
// operand reads hit distinct banks).  Each wave
// forms its share of the 32x32 tiles of M_h on the matrix cores (fp32) and adds
// them, decayed, to Msum in registers; then the state terms of its own tile,
// as products with the 64-column slices of Hin_h and Gout_h, which are loaded
// into registers one head ahead and written transposed into LDS (the matrix
// cores contract over the vector index of an operand row, here p).  After the
// last head, Msum goes to LDS in bf16, row-major beside the transposed slice of
// B, and each wave forms Msum B for its tile; then transposed beside C for
// Msum^T C.  With several head subsets per group the workgroups store fp32
// partial sums that a second kernel adds and rounds.
#include "ssd_device.hpp"
#include "ssd_lds.hpp"

namespace ssd {

template <int Q>
struct DbdcCfg {
  static constexpr int P = kHeadDim;
  static constexpr int NI = Q / 32;              // 32-token tiles, one wave each
  static constexpr int THREADS = 64 * NI;
  static constexpr int NT = NI * (NI + 1) / 2;   // tiles of the lower triangle of Msum
  static constexpr int MT = (NT + NI - 1) / NI;  // Msum tiles per wave, at most
  static constexpr int NW = 64;                  // columns of N per workgroup
  static constexpr int V = P / 8;                // 16-byte vectors per row of x and dy
  static constexpr int ROWV = Q * V;             // vectors of one x (dy) buffer
  static constexpr int NDMA = ROWV / 64;         // load-to-LDS instructions per buffer
  static constexpr int DPW = 2 * NDMA / NI;      // ... per wave per head (x, then dy)
  static constexpr int SV = NW * V;              // vectors of a transposed state slice
  static constexpr int SPT = SV / THREADS;       // state vectors per thread per head
  static constexpr int TPA = ROWV / 128;         // 2 KB Msum tiles per buffer array
  static constexpr int VQ = Q / 8;               // vectors per row of the transposed B, C
  static constexpr int R = Q / 64;               // step sizes per lane (wave 0)
  static_assert(DPW * NI == 2 * NDMA && SPT * THREADS == SV, "copy split");
  static_assert(3 * TPA >= NT, "Msum tiles fit three buffers");
};

// lower-triangle tile k = I (I + 1) / 2 + J, J <= I
__device__ __forceinline__ void tri_tile(int k, int& I, int& J) {
  int i = 0;
  while ((i + 1) * (i + 2) / 2 <= k) ++i;
  I = i;
  J = k - i * (i + 1) / 2;
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu); }

// eight bf16 times d, rounded to nearest even
__device__ __forceinline__ uint4 scale_bf16x8(const uint4& v, float d) {
  return make_uint4(pack_bf16x2(bf16_lo(v.x) * d, bf16_hi(v.x) * d), pack_bf16x2(bf16_lo(v.y) * d, bf16_hi(v.y) * d),
                    pack_bf16x2(bf16_lo(v.z) * d, bf16_hi(v.z) * d), pack_bf16x2(bf16_lo(v.w) * d, bf16_hi(v.w) * d));
}

// v unchanged, but opaque to the compiler: per-lane addresses derived from it
// inside a loop are recomputed there instead of being hoisted out of it (with
// every hoisted address a live register, the loop would spill)
__device__ __forceinline__ int opaque_lane(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int Q>
__global__ __launch_bounds__(DbdcCfg<Q>::THREADS) void bwd_dbdc_kernel(BwdProblem b, float* part, int nsplit,
                                                                        int nsub) {
  using Cfg = DbdcCfg<Q>;
  constexpr int P = Cfg::P, NI = Cfg::NI, NT = Cfg::NT, MT = Cfg::MT, V = Cfg::V, ROWV = Cfg::ROWV;
  constexpr int THREADS = Cfg::THREADS, SPT = Cfg::SPT, VQ = Cfg::VQ, R = Cfg::R;
  // x and dy buffers as separate arrays: reads of one pair while the copies
  // into the other are in flight are then told apart by the compiler.  After
  // the head loop the first three hold Msum's tiles, the fourth B^T or C^T.
  __shared__ __align__(16) uint4 xs0[ROWV];
  __shared__ __align__(16) uint4 xs1[ROWV];
  __shared__ __align__(16) uint4 ys0[ROWV];
  __shared__ __align__(16) uint4 ys1[ROWV];
  __shared__ __align__(16) uint4 hT[Cfg::SV];  // Hin slice transposed: 64 rows n of 64 p
  __shared__ __align__(16) uint4 gT[Cfg::SV];  // Gout slice transposed
  __shared__ __align__(16) float acs[2][Q];    // per head (two in flight): chunk-local cumsum of dt A
  __shared__ __align__(16) float fd[2][Q];     // exp(a_J - Acs_j) (x dt_j): j-factor of a decay
  __shared__ __align__(16) float dts[2][Q];
  __shared__ __align__(16) float ec[2][Q];     // exp(Acs_t): decay of Hin into token t
  __shared__ __align__(16) float eb[2][Q];     // a_next exp(Lam - Acs_j) (x dt_j): of x'_j into Gout

  const int H = b.H, G = b.G, N = b.N;
  const int hpg = H / G;

  // the column slices of one chunk and head subset run on one XCD: they read
  // the same x and dy through its L2
  const int64_t bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int ns = (int)(bid % nsplit);
  int64_t rest = bid / nsplit;
  const int sub = (int)(rest % nsub);
  rest /= nsub;
  const int g = (int)(rest % G);
  const int64_t k = rest / G;
  const BwdChunk ch = bwd_chunk(b, k, Q);
  const int64_t CPS = ch.CPS, c = ch.c, t0 = ch.t0;
  const int n0 = Cfg::NW * ns;
  const int h_lo = g * hpg + (sub * hpg) / nsub;
  const int nh = g * hpg + ((sub + 1) * hpg) / nsub - h_lo;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile indices in scalar registers
  const bool xdt = b.x_times_dt != 0;
  const int64_t xs = (int64_t)H * P;  // token stride of x and dy
  const uint16_t* xg = reinterpret_cast<const uint16_t*>(b.x) + t0 * xs;
  const uint16_t* yg = reinterpret_cast<const uint16_t*>(b.dy) + t0 * xs;
  const int64_t PN = (int64_t)P * N;
  const uint16_t* hin0 = reinterpret_cast<const uint16_t*>(b.hin_e) + k * H * PN + n0;
  const uint16_t* gout0 = reinterpret_cast<const uint16_t*>(b.gin_e) + (ch.s0 / Q + (CPS - 1 - c)) * H * PN + n0;

  // x and dy of head h into (xb, yb): instruction q copies rows 8 q .. 8 q + 7 of
  // the chunk (LDS slots 64 q + lane); lane L takes row 8 q + L / 8 and the
  // vector the swizzle puts in its slot, (L % 8) ^ ((4 q + L / 16) % 8), which
  // depends on q only through its parity: the per-lane offsets of even and odd
  // q are computed once.  Wave w issues q = w, w + NI, ...: x in the first half.
  // copies u0 .. u1 - 1 of this wave's DPW (the step spreads them over its
  // tiles: a burst of them stalls the wave at issue)
  auto issue_xy = [&](int ln, int h, uint4* xb, uint4* yb, int u0 = 0, int u1 = Cfg::DPW) {
    int xoff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
      xoff[par] = (ln / 8) * (int)xs + h * P + 8 * ((ln % 8) ^ ((4 * par + ln / 16) % 8));
#pragma unroll
    for (int u = 0; u < Cfg::DPW; ++u) {
      if (u < u0 || u >= u1) continue;
      const bool isx = u < Cfg::DPW / 2;
      const int q = wid + NI * (isx ? u : u - Cfg::DPW / 2);
      const uint16_t* row = (isx ? xg : yg) + (int64_t)(8 * q) * xs;  // uniform
      lds_copy16(row + xoff[q & 1], (isx ? xb : yb) + q * 64);
    }
  };
  // the 64-column slices of Hin_h and Gout_h (rows p) into registers
  uint4 hreg[SPT], greg[SPT];
  auto load_states = [&](int ln, int h) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int v = 64 * wid + ln + THREADS * i;
      const int p = v / 8, nv = v % 8;
      hreg[i] = *reinterpret_cast<const uint4*>(hin0 + h * PN + p * N + 8 * nv);
      greg[i] = *reinterpret_cast<const uint4*>(gout0 + h * PN + p * N + 8 * nv);
    }
  };
  // ... and from registers into hT, gT transposed (row n holds the 64 p)
  auto store_states = [&](int ln) {
    uint16_t* hd = reinterpret_cast<uint16_t*>(hT);
    uint16_t* gd = reinterpret_cast<uint16_t*>(gT);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int v = 64 * wid + ln + THREADS * i;
      const int p = v / 8, nv = v % 8;
      const uint32_t hw[4] = {hreg[i].x, hreg[i].y, hreg[i].z, hreg[i].w};
      const uint32_t gw[4] = {greg[i].x, greg[i].y, greg[i].z, greg[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int o = swz_slot<V>(8 * nv + e, p / 8) * 8 + (p & 7);
        hd[o] = (uint16_t)((e & 1) ? (hw[e / 2] >> 16) : (hw[e / 2] & 0xffffu));
        gd[o] = (uint16_t)((e & 1) ? (gw[e / 2] >> 16) : (gw[e / 2] & 0xffffu));
      }
    }
  };
  // the cumsums (and step sizes) of head h in wave 0, and the tables built from them
  float acl[R], dtl[R];
  float dtn = 0.0f;
  // head h's chunk-local cumsums of dt A (from the forward's chunk-state
  // kernel, contiguous) and, with the dt-scaled input, its step sizes (one
  // cache line per token): wave 0, R tokens per lane
  auto load_dt = [&](int ln, int h) {
    if (wid == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) acl[i] = b.acs_f[(k * H + h) * Q + ln * R + i];
      if (xdt) {
#pragma unroll
        for (int i = 0; i < R; ++i) dtl[i] = b.dt[(t0 + ln * R + i) * H + h];
      }
      dtn = c + 1 < CPS ? b.dt[(t0 + Q) * H + h] : 0.0f;
    }
  };
  auto make_tables = [&](int ln, int h, int bs) {
    if (wid == 0) {
      const float Ah = b.A[h];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        acs[bs][ln * R + i] = acl[i];
        if (xdt) dts[bs][ln * R + i] = dtl[i];
      }
      const float lam = __shfl(acl[R - 1], 63);
      const float anext = c + 1 < CPS ? __expf(dtn * Ah) : 1.0f;
      // the same wave reads back the tile ends it wrote
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int j = ln * R + i;
        const float aj = acl[i];
        const float dtf = xdt ? dtl[i] : 1.0f;
        fd[bs][j] = __expf(acs[bs][32 * (j / 32) + 31] - aj) * dtf;
        ec[bs][j] = __expf(aj);
        eb[bs][j] = anext * __expf(lam - aj) * dtf;
      }
    }
  };

  floatx16_t msum[MT], accC[2], accB[2];
#pragma unroll
  for (int u = 0; u < MT; ++u) msum[u] = zero16();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) accC[nt] = accB[nt] = zero16();

  // Byte offset, within a block of 32 rows of x or dy (or of hT, gT), of the
  // vector a lane reads for k-step st of an MFMA operand: row lr, vector
  // 2 st + lg, swizzled.  Row 32 B + lr of a buffer is then at 4096 B + this.
  auto operand_offsets = [&](int ln, int (&fo)[4]) {
    const int lr = ln & 31, lg = ln >> 5;
#pragma unroll
    for (int st = 0; st < 4; ++st) fo[st] = 16 * swz_slot<V>(lr, 2 * st + lg);
  };
  auto ldv = [](const uint4* base, int off) { return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off); };

  // this wave's tiles of M_h, decayed, into Msum.  Tile (I, J): A = x_J rows
  // (m = j), B = dy_I rows (n = t): the lane holds token t = 32 I + lr, value r
  // holds j = 32 J + 8 (r / 4) + 4 lg + r % 4.  Off the diagonal the decay
  // exp(Acs_t - Acs_j) (x dt_j) factors into exp(Acs_t - a_J) <= 1, one per lane,
  // and fd_j (a_J = Acs at the end of tile J); a diagonal tile is masked
  // (j <= t) and decayed element by element.
  auto head_tiles = [&](int ln, const int (&fo)[4], const uint4* xb, const uint4* yb, int bs, auto after_tile) {
    const int lr = ln & 31, lg = ln >> 5;
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int kt = wid + NI * u;
      if (kt < NT) {
        int I, J;
        tri_tile(kt, I, J);
        floatx16_t sv = zero16();
#pragma unroll
        for (int st = 0; st < 4; ++st)
          sv = mfma32x32x16(ldv(xb, 4096 * J + fo[st]), ldv(yb, 4096 * I + fo[st]), sv);
        const float at = acs[bs][32 * I + lr];
        if (I == J) {
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const int jl = 8 * a4 + 4 * lg;
            const float4 aj = *reinterpret_cast<const float4*>(&acs[bs][32 * J + jl]);
            const float4 dj = *reinterpret_cast<const float4*>(&dts[bs][32 * J + jl]);
            const float ajq[4] = {aj.x, aj.y, aj.z, aj.w}, djq[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float e = jl + q <= lr ? __expf(at - ajq[q]) * (xdt ? djq[q] : 1.0f) : 0.0f;
              msum[u][4 * a4 + q] += e * sv[4 * a4 + q];
            }
          }
        } else {
          const float ft = __expf(at - acs[bs][32 * J + 31]);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float4 f = *reinterpret_cast<const float4*>(&fd[bs][32 * J + 8 * a4 + 4 * lg]);
            msum[u][4 * a4] += ft * f.x * sv[4 * a4];
            msum[u][4 * a4 + 1] += ft * f.y * sv[4 * a4 + 1];
            msum[u][4 * a4 + 2] += ft * f.z * sv[4 * a4 + 2];
            msum[u][4 * a4 + 3] += ft * f.w * sv[4 * a4 + 3];
          }
        }
      }
      after_tile(u);
      // one tile's operands at a time: hoisting every tile's loads would take
      // the registers that hold Msum
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // state terms of the wave's tile: A = dy rows t scaled by exp(Acs_t) (x rows j
  // scaled by a_next exp(Lam - Acs_j) (x dt_j)), B = Hin^T (Gout^T) rows n; the
  // lane holds column n = 32 nt + lr, value r token 32 wid + 8 (r / 4) + 4 lg + r % 4
  auto head_states = [&](int ln, const int (&fo)[4], const uint4* xb, const uint4* yb, int bs) {
    const int tr = 32 * wid + (ln & 31);  // the lane's operand row
    uint4 a[4];
    const float fc = ec[bs][tr];
#pragma unroll
    for (int st = 0; st < 4; ++st) a[st] = scale_bf16x8(ldv(yb, 4096 * wid + fo[st]), fc);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int st = 0; st < 4; ++st) accC[nt] = mfma32x32x16(a[st], ldv(hT, 4096 * nt + fo[st]), accC[nt]);
    const float fb = eb[bs][tr];
#pragma unroll
    for (int st = 0; st < 4; ++st) a[st] = scale_bf16x8(ldv(xb, 4096 * wid + fo[st]), fb);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int st = 0; st < 4; ++st) accB[nt] = mfma32x32x16(a[st], ldv(gT, 4096 * nt + fo[st]), accB[nt]);
  };
  // one head: its copies were issued one head earlier into (cx, cy); the next
  // head's go into (nx, ny)
  auto step = [&](int u, const uint4* cx, const uint4* cy, int bs, uint4* nx, uint4* ny) {
    wait_vm<0>();  // this wave's copies of head u
    dl_barrier();  // every wave's copies, tables and states of head u; head u - 1 finished
    const int ln = opaque_lane(lane);
    const bool more = u + 1 < nh;
    if (more) {
      load_states(ln, h_lo + u + 1);
      load_dt(ln, h_lo + u + 1);
    }
    int fo[4];
    operand_offsets(ln, fo);
    // the next head's copies, CPT after each tile
    constexpr int CPT = (Cfg::DPW + MT - 1) / MT;
    head_tiles(ln, fo, cx, cy, bs, [&](int t) {
      if (more) issue_xy(ln, h_lo + u + 1, nx, ny, t * CPT, (t + 1) * CPT);
    });
    head_states(ln, fo, cx, cy, bs);
    if (more) {
      make_tables(ln, h_lo + u + 1, bs ^ 1);
      dl_barrier();  // every wave is done with hT, gT of head u
      store_states(ln);
    }
  };

  if (nh > 0) {
    load_states(lane, h_lo);
    load_dt(lane, h_lo);
    issue_xy(lane, h_lo, xs0, ys0);
    make_tables(lane, h_lo, 0);
    store_states(lane);
  }
  for (int u = 0; u < nh; u += 2) {
    step(u, xs0, ys0, 0, xs1, ys1);
    if (u + 1 < nh) step(u + 1, xs1, ys1, 1, xs0, ys0);
  }
  wait_vm<0>();
  __syncthreads();

  // ---- Msum B: Msum tiles row-major (bf16) in xs0, xs1, ys0; B^T in ys1
  auto tile_base = [&](int kt) -> uint4* {
    const int arr = kt / Cfg::TPA;
    uint4* base = arr == 0 ? xs0 : (arr == 1 ? xs1 : ys0);
    return base + (kt % Cfg::TPA) * 128;
  };
  // B or C rows of the chunk, columns n0 .. n0 + 63, into ys1 transposed (row n
  // holds the Q tokens)
  auto store_bc_t = [&](const void* src) {
    const uint16_t* sp = reinterpret_cast<const uint16_t*>(src) + (t0 * G + g) * (int64_t)N + n0;
    uint16_t* d = reinterpret_cast<uint16_t*>(ys1);
    for (int v = tid; v < Q * 8; v += THREADS) {
      const int j = v / 8, nv = v % 8;
      const uint4 val = *reinterpret_cast<const uint4*>(sp + j * (int64_t)G * N + 8 * nv);
      const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        d[swz_slot<VQ>(8 * nv + e, j / 8) * 8 + (j & 7)] =
            (uint16_t)((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu));
    }
  };
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int kt = wid + NI * u;
    if (kt < NT) {
      uint4* tb = tile_base(kt);
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const uint2 w2 = make_uint2(pack_bf16x2(msum[u][4 * a4], msum[u][4 * a4 + 1]),
                                    pack_bf16x2(msum[u][4 * a4 + 2], msum[u][4 * a4 + 3]));
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(tb + swz_slot<4>(lr, a4)) + 8 * lg) = w2;
      }
    }
  }
  store_bc_t(b.B);
  __syncthreads();
  // dC of tile wid: A = Msum rows t (k = j of tile J), B = B^T rows n
  for (int J = 0; J <= wid; ++J) {
    const uint4* tb = tile_base(wid * (wid + 1) / 2 + J);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint4 am = tb[swz_slot<4>(lr, 2 * st + lg)];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        accC[nt] = mfma32x32x16(am, ys1[swz_slot<VQ>(32 * nt + lr, 4 * J + 2 * st + lg)], accC[nt]);
    }
  }
  __syncthreads();
  // ---- Msum^T C: Msum tiles transposed (row j holds the tile's t), C^T in ys1
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int kt = wid + NI * u;
    if (kt < NT) {
      uint16_t* td = reinterpret_cast<uint16_t*>(tile_base(kt));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = 8 * (r / 4) + 4 * lg + r % 4;
        td[swz_slot<4>(jl, lr / 8) * 8 + (lr & 7)] = bf16_bits(msum[u][r]);
      }
    }
  }
  store_bc_t(b.C);
  __syncthreads();
  // dB of tile wid: A = Msum^T rows j (k = t of tile I), B = C^T rows n
  for (int I = wid; I < NI; ++I) {
    const uint4* tb = tile_base(I * (I + 1) / 2 + wid);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint4 am = tb[swz_slot<4>(lr, 2 * st + lg)];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        accB[nt] = mfma32x32x16(am, ys1[swz_slot<VQ>(32 * nt + lr, 4 * I + 2 * st + lg)], accB[nt]);
    }
  }

  // ---- out: lane = column n0 + 32 nt + lr, value r = token 32 wid + 8 (r / 4) + 4 lg + r % 4
  const int64_t GN = (int64_t)G * N;
  if (nsub == 1) {
    uint16_t* dc = reinterpret_cast<uint16_t*>(b.dC) + (t0 + 32 * wid) * GN + (int64_t)g * N + n0 + lr;
    uint16_t* db = reinterpret_cast<uint16_t*>(b.dB) + (t0 + 32 * wid) * GN + (int64_t)g * N + n0 + lr;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t o = (8 * (r / 4) + 4 * lg + r % 4) * GN + 32 * nt;
        dc[o] = bf16_bits(accC[nt][r]);
        db[o] = bf16_bits(accB[nt][r]);
      }
  } else {
    float* pc = part + (2 * (int64_t)sub * b.total + t0 + 32 * wid) * GN + (int64_t)g * N + n0 + lr;
    float* pb = pc + b.total * GN;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t o = (8 * (r / 4) + 4 * lg + r % 4) * GN + 32 * nt;
        pc[o] = accC[nt][r];
        pb[o] = accB[nt][r];
      }
  }
}

// dC and dB = the sums of the head subsets' fp32 partials, rounded once.
__global__ __launch_bounds__(256) void bwd_dbdc_sum_kernel(BwdProblem b, const float* part, int nsub) {
  const int64_t n4 = b.total * (int64_t)b.G * b.N / 4;
  const int64_t stride = b.total * (int64_t)b.G * b.N;
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 sc = make_float4(0.f, 0.f, 0.f, 0.f), sb = sc;
    for (int q = 0; q < nsub; ++q) {
      const float4 a = reinterpret_cast<const float4*>(part + 2 * q * stride)[i];
      const float4 d = reinterpret_cast<const float4*>(part + (2 * q + 1) * stride)[i];
      sc.x += a.x; sc.y += a.y; sc.z += a.z; sc.w += a.w;
      sb.x += d.x; sb.y += d.y; sb.z += d.z; sb.w += d.w;
    }
    reinterpret_cast<uint2*>(b.dC)[i] = make_uint2(pack_bf16x2(sc.x, sc.y), pack_bf16x2(sc.z, sc.w));
    reinterpret_cast<uint2*>(b.dB)[i] = make_uint2(pack_bf16x2(sb.x, sb.y), pack_bf16x2(sb.z, sb.w));
  }
}

bool backward_dbdc_supported(Dtype dt, int Q, int N) {
  return dt == Dtype::BF16 && (Q == 64 || Q == 128 || Q == 256) && (N == 64 || N == 128 || N == 256);
}

// head subsets per group: enough workgroups for one per compute unit, at most
// one subset per head
int backward_dbdc_subsets(int64_t chunks, int G, int H, int N) {
  const int64_t base = chunks * G * (N / 64);
  if (base <= 0) return 1;
  int nsub = (int)std::min<int64_t>((256 + base - 1) / base, H / G);
  return nsub < 1 ? 1 : nsub;
}

template <int Q>
static void launch_dbdc_q(const BwdProblem& b, float* part, int nsub, hipStream_t s) {
  const int64_t chunks = b.total / Q;
  const int nsplit = b.N / 64;
  const dim3 grid((unsigned)(chunks * b.G * nsplit * nsub));
  hipLaunchKernelGGL((bwd_dbdc_kernel<Q>), grid, dim3(DbdcCfg<Q>::THREADS), 0, s, b, part, nsplit, nsub);
}

hipError_t launch_backward_dbdc(const BwdProblem& b, float* part, int nsub, hipStream_t s) {
  if (!backward_dbdc_supported(b.dtype, b.Q, b.N) || b.total % b.Q != 0 || (b.cu == nullptr && b.seqlen % b.Q != 0) ||
      nsub < 1 || (nsub > 1 && !part))
    return hipErrorInvalidValue;
  const int64_t chunks = b.total / b.Q;
  if (chunks == 0) return hipSuccess;
  switch (b.Q) {
    case 64: launch_dbdc_q<64>(b, part, nsub, s); break;
    case 128: launch_dbdc_q<128>(b, part, nsub, s); break;
    default: launch_dbdc_q<256>(b, part, nsub, s); break;
  }
  if (nsub > 1) {
    const int64_t n4 = b.total * (int64_t)b.G * b.N / 4;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(bwd_dbdc_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, b, part, nsub);
  }
  return hipGetLastError();
}

}  // namespace ssd
