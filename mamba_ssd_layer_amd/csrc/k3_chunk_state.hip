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
// Design (gfx950): one workgroup of 8 waves per (chunk, block of HB heads of
// one B/C group), one workgroup per CU.  The prologue loads the log-decays of
// all the block's heads at once (consecutive lanes on consecutive heads) and
// scans them (one wave per head: Q/64 tokens per lane plus a wave-level scan);
// the scan writes Acs, the chunk total and the largest 32-token-tile decay for
// the later kernels and keeps each head's
// decay-to-chunk-end weights w_l = exp(Acs_{L-1} - Acs_l) in LDS.  The chunk's
// B tile is staged transposed in LDS once (tokens contiguous, as an MFMA
// operand contracting over tokens needs); on the bf16 path every wave then
// keeps its 32 rows of B^T as MFMA operands in registers for all HB heads and
// the LDS space is reused for x.  Each head's x tile is loaded into registers
// while the previous head computes, then scaled by w and transposed into LDS
// (bf16 rows unpadded, their 16-byte blocks XOR-swizzled by row so that
// neither the transposing stores nor the MFMA operand reads meet LDS bank
// conflicts).  The product is formed as S^T (N x P) on 32x32 tiles
// (v_mfma_f32_32x32x16_bf16 / _32x32x2_f32, fp32 accumulation), so that each
// lane ends with runs of 4 consecutive n of one p; the tile passes through LDS
// in [p][n] order and leaves as whole 16-byte vectors, the (P x N) state of a
// (chunk, head) being one contiguous block.  States are stored in the element
// dtype (the state-passing kernel accumulates them in fp32), with the
// non-temporal hint when the forward's data exceeds the last-level cache (then
// they would only displace x and B, which are read again).
#include "ssd_stage.hpp"

namespace ssd {

constexpr int kCsThreads = 512;  // 8 waves: two per SIMD

// x^T rows in LDS: the P rows of x, then one MFMA tile of 32 rows whose first
// row carries the decay weights alone (the ones column of the normalised
// output's denominator, [T]/[M] "Incorporating a Normalization (Denominator)
// Term": its chunk state is the weighted sum of B rows).  The tile's other 31
// rows are left as they are: each feeds only its own output column, and those
// columns are not stored.
constexpr int kXRows = kHeadDim + 32;

// fp32 token blocks per chunk: the fewest whose transposed B and x blocks, the
// staged state rows and one head's weights fit in LDS
constexpr int cs_f32_split(int Q, int N) {
  const int NT = N < 32 ? 32 : N;
  for (int s = 1; s < 8; s *= 2) {
    const int kb = Q / s + 4;
    if ((size_t)(NT * kb + kXRows * kb + kHeadDim * (N + 4)) * 4 + (size_t)Q * 4 <= (size_t)kLdsLimit) return s;
  }
  return 8;
}

template <class E, int Q, int N>
struct ChunkStateCfg {
  using T = typename E::storage;
  static constexpr bool kBf16 = E::kBytes == 2;
  static constexpr int P = kHeadDim;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr bool SWZ = kBf16;            // bf16: swizzled, unpadded transposed tiles
  static constexpr bool kRegB = kBf16;          // B^T operands kept in registers, LDS reused
  // fp32: the chunk's tokens go through LDS in KSPL blocks of KB (B^T and x^T
  // staged again for every block and head); bf16: one block
  static constexpr int KSPL = kBf16 ? 1 : cs_f32_split(Q, N);
  static constexpr int KB = Q / KSPL;
  static constexpr int QP = SWZ ? Q : KB + PAD;  // LDS pitch of the transposed tiles
  static constexpr int NT = N < 32 ? 32 : N;    // B^T rows, padded to an MFMA tile
  static constexpr int SP = N + PAD;            // LDS pitch of the staged state rows
  static constexpr int NTN = NT / 32;           // n tiles
  static constexpr int NTILES = NTN * (P / 32);
  // a wave's tiles: one n tile and, with more than 8 tiles, both p tiles
  static constexpr int PPW = NTILES > 8 ? 2 : 1;
  static constexpr int KSTEPS = KB / E::kMfmaK;
  static constexpr size_t bt_bytes = (size_t)NT * QP * sizeof(T);
  static constexpr size_t xs_bytes = ((size_t)kXRows * QP + (size_t)P * SP) * sizeof(T);
  static constexpr size_t tile_bytes = kRegB ? (bt_bytes > xs_bytes ? bt_bytes : xs_bytes) : bt_bytes + xs_bytes;
  // bf16: the step sizes of the block's heads are kept in LDS too (the
  // dt-scaled input's weights need them in the scan)
  static constexpr bool kDtLds = kBf16;
  static constexpr size_t head_bytes = (kDtLds ? 2 : 1) * (size_t)Q * sizeof(float);
  // log-decays, then decay weights (and step sizes), of every head of the
  // block (LDS left over by the tiles bounds the heads per workgroup)
  static constexpr int kMaxHB = (int)(((size_t)kLdsLimit - (tile_bytes < (size_t)kLdsLimit ? tile_bytes : kLdsLimit)) /
                                      head_bytes) < kMaxHeadsPerBlock
                                    ? (int)(((size_t)kLdsLimit - (tile_bytes < (size_t)kLdsLimit ? tile_bytes : kLdsLimit)) /
                                            head_bytes)
                                    : kMaxHeadsPerBlock;
  static constexpr size_t lds_bytes = tile_bytes + (size_t)(kMaxHB > 0 ? kMaxHB : 1) * head_bytes;
  static constexpr bool fits = kMaxHB >= 1 && lds_bytes <= (size_t)kLdsLimit;
  // log-decay loads per thread: Q tokens x kMaxHB heads over the workgroup
  static constexpr int kEllPT = (Q * (kMaxHB > 0 ? kMaxHB : 1) + kCsThreads - 1) / kCsThreads;
};

// kNT: the states are stored with the non-temporal hint (a compile-time choice:
// a run-time one lets the compiler merge the two stores and drop the hint)
template <class E, int Q, int N, bool kDebug, bool kNT>
__global__ __launch_bounds__(kCsThreads, 1) void chunk_state_kernel(Problem p, Workspace ws, int HB,
                                                                    float* __restrict__ states_f32) {
  using Cfg = ChunkStateCfg<E, Q, N>;
  using T = typename E::storage;
  constexpr bool kBf16 = Cfg::kBf16, SWZ = Cfg::SWZ, kRegB = Cfg::kRegB;
  constexpr int P = Cfg::P, QP = Cfg::QP, NT = Cfg::NT, SP = Cfg::SP, NTN = Cfg::NTN;
  constexpr int PPW = Cfg::PPW, KSTEPS = Cfg::KSTEPS, KSPL = Cfg::KSPL, KB = Cfg::KB;
  constexpr int R = Q / 64;    // tokens per lane in the cumsum
  constexpr int SEG = 32 / R;  // lanes per 32-token tile in the cumsum
  __shared__ __attribute__((aligned(16))) char smem[Cfg::tile_bytes];
  __shared__ __attribute__((aligned(16))) float wbuf[(Cfg::kMaxHB > 0 ? Cfg::kMaxHB : 1) * Q];  // log-decays, then w
  // bf16: the step sizes dt (clamped past the chunk's end as the decays are)
  __shared__ __attribute__((aligned(16))) float dtbuf[Cfg::kDtLds ? (Cfg::kMaxHB > 0 ? Cfg::kMaxHB : 1) * Q : 1];
  T* bT = reinterpret_cast<T*>(smem);
  T* xwT = reinterpret_cast<T*>(smem + (kRegB ? 0 : Cfg::bt_bytes));
  T* Ss = xwT + kXRows * QP;
  // normalised output: the chunk state of the ones column (the weighted sum of
  // the chunk's B rows) of every head goes to ws.zs
  const bool zcol = ws.zs != nullptr;

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

  // this wave's output tiles: n tile nt, p tiles pt0 .. pt0 + PPW - 1
  const bool active = Cfg::NTILES > 8 || wid < Cfg::NTILES;
  const int nt = Cfg::NTILES > 8 ? wid : wid % NTN;
  const int pt0 = Cfg::NTILES > 8 ? 0 : wid / NTN;

  // ---- issue the loads: log-decays of all HB heads (consecutive lanes read
  // consecutive heads of a token row; indices clamped so that every load is
  // issued unconditionally), B tile, first x tile
  // element e = tid + i * 512 of the (token, head) table is token e / HB, head
  // e % HB; both advance by a fixed step per i (no division in the loop)
  const int et0 = tid / HB, eh0 = tid % HB;
  const int dt_step = kCsThreads / HB, dh_step = kCsThreads % HB;
  float ell[Cfg::kEllPT], dte[Cfg::kEllPT];
  {
    int t = et0, hh = eh0;
#pragma unroll
    for (int i = 0; i < Cfg::kEllPT; ++i) {
      const bool in = t < Q;  // past the table: clamped to its last element
      const int tc = in ? min(t, L - 1) : L - 1, hc = in ? hh : HB - 1;
      dte[i] = p.dt[(cd.t0 + tc) * H + h0 + hc];
      ell[i] = dte[i] * p.A[h0 + hc];
      t += dt_step;
      hh += dh_step;
      if (hh >= HB) { hh -= HB; ++t; }
    }
  }
  // one token block of B and x (bf16: the whole chunk, loaded here; fp32: per
  // block and head in the head loop)
  using BTile = TransTile<E, KB, N, kCsThreads>;
  using XTile = TransTile<E, KB, P, kCsThreads, 4>;
  // bf16: the x tiles of the next kXDepth heads are in flight at any time (a
  // head's products take far less than a load's latency, so one tile ahead
  // would leave each head waiting out most of it); register set d holds the
  // heads d, d + kXDepth, ...  fp32 uses set 0 alone.
  constexpr int kXDepth = kBf16 ? 2 : 1;
  XTile xr[kXDepth];
  XTile& xt = xr[0];
  {
    BTile bt;
    if constexpr (kBf16) {
      bt.load(reinterpret_cast<const T*>(p.B) + (cd.t0 * G + g) * N, (int64_t)G * N, L);
      // unconditional (a block of fewer heads reloads its last one): a load
      // under a condition would make the B tile's staging below wait for
      // these too
#pragma unroll
      for (int d = 0; d < kXDepth; ++d) xr[d].load(xbase + (h0 + min(d, HB - 1)) * P, (int64_t)H * P, L);
    }
    int t = et0, hh = eh0;
#pragma unroll
    for (int i = 0; i < Cfg::kEllPT; ++i) {
      if (t < Q) {
        wbuf[hh * Q + t] = t < L ? ell[i] : 0.0f;
        if (Cfg::kDtLds && p.x_times_dt) dtbuf[hh * Q + t] = dte[i];
      }
      t += dt_step;
      hh += dh_step;
      if (hh >= HB) { hh -= HB; ++t; }
    }
    if (NT > N)
      for (int i = tid; i < (NT - N) * QP; i += kCsThreads) bT[N * QP + i] = T(0);
    if constexpr (kBf16) bt.template store<QP, 0, false, SWZ>(bT, nullptr);
  }
  lds_barrier();

  // ---- K1: chunk-local inclusive cumsum, one wave per head (waves take heads
  // wid, wid + 8, ...); entries past the chunk end repeat the last value (their
  // log-decay is 0) and get weight 0.  Every sum here only adds terms of one
  // sign (dt*A <= 0): the weight of token l is exp of the sum of dt*A over the
  // chunk's later tokens, summed as such ([M] §3.5.4: segment sums without
  // differences of cumsums), never exp(Acs_end - Acs_l).
  for (int hh = wid; hh < HB; hh += kCsThreads / 64) {
    const int h = h0 + hh;
    float el[R], run[R], sfx[R];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      el[i] = wbuf[hh * Q + lane * R + i];
      acc += el[i];
      run[i] = acc;
    }
    float acc2 = 0.0f;  // the lane's tokens from the last: sfx[i] sums those after i
#pragma unroll
    for (int i = R - 1; i >= 0; --i) {
      sfx[i] = acc2;
      acc2 += el[i];
    }
    const float excl = wave_prefix_excl_dpp(acc);    // the earlier lanes' tokens
    const float sxcl = wave_suffix_excl_dpp(acc2);   // the later lanes' tokens
    const float lam = __shfl(excl + run[R - 1], 63);
    float* gout = ws.acs + (k * H + h) * Q + lane * R;
    if (p.x_times_dt) {
      // the input enters as dt_l x_l: the weights carry dt_l, and the output
      // kernel divides its staged x by exp(Acs_l - ln dt_l) instead of exp(Acs_l)
      const float* dtp = p.dt + cd.t0 * H + h;
      float* xl = ws.xlog + (k * H + h) * Q + lane * R;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float a = excl + run[i];
        // (bf16: from the LDS table, so that the scan waits for no load still
        // in flight, the first heads' x tiles among them)
        const float dtl = Cfg::kDtLds ? dtbuf[hh * Q + lane * R + i] : dtp[(int64_t)min(lane * R + i, L - 1) * H];
        gout[i] = a;
        xl[i] = a - __logf(dtl);
        wbuf[hh * Q + lane * R + i] = (lane * R + i < L) ? __expf(sxcl + sfx[i]) * dtl : 0.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        gout[i] = excl + run[i];
        wbuf[hh * Q + lane * R + i] = (lane * R + i < L) ? __expf(sxcl + sfx[i]) : 0.0f;
      }
    }
    if (lane == 63) ws.lam[k * H + h] = lam;
    if (!mask_by_chunk<E>(lam)) {
      // the output kernel forms this head's mask per element: dt*A, its sum
      // over the later tokens of each 32-token tile, and the tile totals
      const float tsx = seg_exclusive_suffix_sum<SEG>(acc2);
      float* eo = ws.ell + (k * H + h) * Q + lane * R;
      float* ro = ws.rsuf + (k * H + h) * Q + lane * R;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        eo[i] = el[i];
        ro[i] = tsx + sfx[i];
      }
      const bool tile_lane = (lane & (SEG - 1)) == 0;
      if (tile_lane) ws.ttot[(k * H + h) * 8 + lane / SEG] = tsx + acc2;
      // the largest tile decay (-min of the tile sums), which decides whether
      // the output kernel may factor this head's mask by 32-token tile
      float td = tile_lane ? -(tsx + acc2) : 0.0f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) td = fmaxf(td, __shfl_xor(td, off, kWave));
      if (lane == 0) ws.tmax[k * H + h] = td;
    }
  }

  // ---- B^T operands of this wave's n tile, for all heads (bf16)
  uint4 bop[kRegB ? KSTEPS : 1];
  if constexpr (kRegB) {
    const int row = nt * 32 + lr;
    const int key = lds_swizzle<Q>(row);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      bop[ks] = *reinterpret_cast<const uint4*>(bT + row * QP + ((2 * ks + lg) ^ key) * 8);
  }

  // 16-byte vectors of one (P x N) state, and per thread
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int NV = P * N / VEC;
  constexpr int VPT = (NV + kCsThreads - 1) / kCsThreads;

  // the staged state of (chunk, head h) is one contiguous (P x N) block:
  // whole 16-byte vectors
  auto store_state = [&](int h) {
    T* out = reinterpret_cast<T*>(ws.states) + (k * H + h) * (int64_t)(P * N);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * kCsThreads;
      if (NV % kCsThreads == 0 || v < NV) {
        const int row = v / (N / VEC), col = (v % (N / VEC)) * VEC;
        const uint4 val = *reinterpret_cast<const uint4*>(Ss + row * SP + col);
        if constexpr (kNT)
          store_nt(reinterpret_cast<uint4*>(out) + v, val);
        else
          reinterpret_cast<uint4*>(out)[v] = val;
        if constexpr (kDebug) {
          float* o32 = states_f32 + (k * H + h) * (int64_t)(P * N) + (int64_t)v * VEC;
          if constexpr (kBf16) {
            reinterpret_cast<float4*>(o32)[0] =
                make_float4(bf16_lo(val.x), bf16_hi(val.x), bf16_lo(val.y), bf16_hi(val.y));
            reinterpret_cast<float4*>(o32)[1] =
                make_float4(bf16_lo(val.z), bf16_hi(val.z), bf16_lo(val.w), bf16_hi(val.w));
          } else {
            reinterpret_cast<uint4*>(o32)[0] = val;
          }
        }
      }
    }
  };

  // acc[j][4q + e] = S[p = 32 (pt0 + j) + lr][n = 32 nt + 8q + 4lg + e] -> Ss
  auto stage_state = [&](const floatx16_t (&acc)[PPW]) {
#pragma unroll
    for (int j = 0; j < PPW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n0 = nt * 32 + 8 * q + 4 * lg;
        if (NT == N || n0 < N) {
          T* dst = Ss + ((pt0 + j) * 32 + lr) * SP + n0;
          const floatx16_t& c = acc[j];
          if constexpr (kBf16)
            *reinterpret_cast<uint2*>(dst) =
                make_uint2(pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3]));
          else
            *reinterpret_cast<float4*>(dst) = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
        }
      }
  };

  // the ones column's chunk state from its MFMA tile: lanes of row 0 (lr == 0)
  // hold Zs[n = 32 nt + 8q + 4lg + e] at accz[4q + e]
  const bool zwave = zcol && active && pt0 == 0;
  auto store_z = [&](int h, const floatx16_t& accz) {
    if (lr != 0) return;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = nt * 32 + 8 * q + 4 * lg + e;
        if (NT == N || n < N) {
          T* dst = reinterpret_cast<T*>(ws.zs) + (k * H + h) * (int64_t)N + n;
          if constexpr (kBf16)
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(pack_bf16x2(accz[4 * q + e], 0.0f) & 0xffffu);
          else
            *dst = accz[4 * q + e];
        }
      }
  };

  if constexpr (kBf16) {
    // head hh, its x tile in register set xh (head hh + kXDepth is loaded
    // into the same set once it is staged)
    auto head = [&](const int hh, XTile& xh) __attribute__((always_inline)) {
      const int h = h0 + hh;
      lds_barrier();  // w ready; B^T read; the previous head's x^T and state rows no longer read
      xh.template store<QP, 1, false, SWZ>(xwT, wbuf + hh * Q);
      if (zcol && tid < Q / 8) {
        // the weights row of the ones column, 8 tokens per 16-byte block
        const float* wr = wbuf + hh * Q + tid * 8;
        const uint4 v = make_uint4(pack_bf16x2(wr[0], wr[1]), pack_bf16x2(wr[2], wr[3]),
                                   pack_bf16x2(wr[4], wr[5]), pack_bf16x2(wr[6], wr[7]));
        *reinterpret_cast<uint4*>(xwT + P * QP + (tid ^ lds_swizzle<Q>(P)) * 8) = v;
      }
      lds_barrier();
      if (hh + kXDepth < HB) xh.load(xbase + (h + kXDepth) * P, (int64_t)H * P, L);

      // ---- K3: S^T = B^T (w o X) on this wave's tiles
      if (active) {
        floatx16_t acc[PPW];
#pragma unroll
        for (int j = 0; j < PPW; ++j) acc[j] = zero16();
        // x^T operands of step ks + 2 are read while step ks multiplies (LDS
        // latency is several MFMA steps): a ring of three register sets
        int xkey[PPW];
#pragma unroll
        for (int j = 0; j < PPW; ++j) xkey[j] = lds_swizzle<Q>((pt0 + j) * 32 + lr);
        uint4 b[3][PPW];
        auto read_x = [&](int ks, uint4 (&br)[PPW]) {
#pragma unroll
          for (int j = 0; j < PPW; ++j)
            br[j] = *reinterpret_cast<const uint4*>(xwT + ((pt0 + j) * 32 + lr) * QP + ((2 * ks + lg) ^ xkey[j]) * 8);
        };
        read_x(0, b[0]);
        if (KSTEPS > 1) read_x(1, b[1]);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          if (ks + 2 < KSTEPS) read_x(ks + 2, b[(ks + 2) % 3]);
          // keep the reads ahead: the scheduler would otherwise sink each read
          // next to its MFMA and wait for it there
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < PPW; ++j) acc[j] = mfma32x32x16(bop[ks], b[ks % 3][j], acc[j]);
          __builtin_amdgcn_sched_barrier(0);
        }
        stage_state(acc);
      }
      if (zwave) {
        // the ones column: B^T times its weights row (output column P only)
        floatx16_t accz = zero16();
        const int zkey = lds_swizzle<Q>(P + lr);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          accz = mfma32x32x16(bop[ks], *reinterpret_cast<const uint4*>(xwT + (P + lr) * QP + ((2 * ks + lg) ^ zkey) * 8),
                              accz);
        store_z(h, accz);
      }
      lds_barrier();
      store_state(h);
    };
    for (int hb = 0; hb < HB; hb += kXDepth) {
#pragma unroll
      for (int d = 0; d < kXDepth; ++d)
        if (hb + d < HB) head(hb + d, xr[d]);
    }
  } else {
    // fp32: KSPL token blocks per head, B^T and x^T of each staged in turn
    for (int hh = 0; hh < HB; ++hh) {
      const int h = h0 + hh;
      floatx16_t acc[PPW];
#pragma unroll
      for (int j = 0; j < PPW; ++j) acc[j] = zero16();
      floatx16_t accz = zero16();
      for (int kb = 0; kb < KSPL; ++kb) {
        const int Lb = min(KB, L - kb * KB);
        if (Lb <= 0) break;  // past the chunk's end (the same for every thread)
        BTile bt;
        bt.load(reinterpret_cast<const T*>(p.B) + ((cd.t0 + kb * KB) * G + g) * N, (int64_t)G * N, Lb);
        xt.load(xbase + (int64_t)kb * KB * H * P + h * P, (int64_t)H * P, Lb);
        lds_barrier();  // weights ready; the previous block's tiles no longer read
        bt.template store<QP, 0>(bT, nullptr);
        xt.template store<QP, 1>(xwT, wbuf + hh * Q + kb * KB);
        // the weights row of the ones column (zero past the chunk's end)
        if (zcol && tid < KB) xwT[P * QP + tid] = wbuf[hh * Q + kb * KB + tid];
        lds_barrier();
        if (active) {
#pragma unroll 8
          for (int ks = 0; ks < KSTEPS; ++ks) {
            const float a = bT[(nt * 32 + lr) * QP + ks * 2 + lg];
#pragma unroll
            for (int j = 0; j < PPW; ++j)
              acc[j] = mfma32x32x2(a, xwT[((pt0 + j) * 32 + lr) * QP + ks * 2 + lg], acc[j]);
            if (zwave) accz = mfma32x32x2(a, xwT[(P + lr) * QP + ks * 2 + lg], accz);
          }
        }
      }
      if (active) stage_state(acc);
      if (zwave) store_z(h, accz);
      lds_barrier();
      store_state(h);
    }
  }
}

template <class E, int Q, int N>
static hipError_t launch_cs(const Problem& p, const Workspace& ws, float* states_f32, hipStream_t s) {
  if constexpr (ChunkStateCfg<E, Q, N>::fits) {
    const int HB = heads_per_block(p, ChunkStateCfg<E, Q, N>::kMaxHB);
    const unsigned blocks = (unsigned)(p.kmax * (p.H / HB));
    // the fp32 copy for inspection goes with plain stores (the hint changes no value)
    if (states_f32)
      hipLaunchKernelGGL((chunk_state_kernel<E, Q, N, true, false>), dim3(blocks), dim3(kCsThreads), 0, s, p,
                         ws, HB, states_f32);
    else if (p.stream_states)
      hipLaunchKernelGGL((chunk_state_kernel<E, Q, N, false, true>), dim3(blocks), dim3(kCsThreads), 0, s, p,
                         ws, HB, states_f32);
    else
      hipLaunchKernelGGL((chunk_state_kernel<E, Q, N, false, false>), dim3(blocks), dim3(kCsThreads), 0, s, p,
                         ws, HB, states_f32);
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
