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
//  * One workgroup of 8 waves (two per SIMD) per (chunk, block of HB heads of
//    one group) and one workgroup per CU (HB is chosen so that the grid fills
//    the CUs in few rounds).  The chunk's kernel-matrix tiles G = C B^T of the
//    group are formed when the workgroup starts (B rows staged in LDS, each
//    wave's C rows in registers, v_mfma_f32_32x32x16_bf16) and stay in LDS for
//    all HB heads; the C rows stay in registers as well.  The next head's x
//    tile and passed state are loaded into registers while the current head
//    computes, so the compute phase reads only LDS and registers.  Blocks are
//    ordered so that the head blocks of one chunk land on one XCD.  (fp32, and
//    bf16 with N = Q = 256: the tiles do not fit in LDS next to the x tile and
//    come from the kernel-matrix kernel through global memory.)
//  * The output is built transposed, Y^T (P x Q), on 32x32 MFMA tiles.  A
//    kernel tile as G^T leaves each lane ONE output token i and 16 input
//    tokens j, which is exactly the B-operand layout of Y^T += X^T (L o G)^T;
//    the K (token) order of that product is chosen to match, and x^T is staged
//    with its tokens permuted in 16-groups so the A operand is one 16-byte read.
//  * Causality: only tiles J <= I are used; on the diagonal tile the entries
//    with j > i are a selected (or masked-off) 0, never exp(-inf) arithmetic.
//    The mask is exp of the sum of ell = dt*A over the tokens (j, i], formed
//    per head in one of three ways, chosen from the chunk's total log-decay
//    (mask_by_chunk) and, on the plain bf16 path, its largest 32-token-tile
//    decay; each kind runs in a head loop of its own (chunk heads first, then
//    tile, then per element), so that the chunk path's registers, schedule and
//    load waits are not shaped by the other kinds' code:
//    - chunk (total decay within e^64 on the bf16 path, e^16 on fp32): x_j is
//      staged scaled by exp(-Acs_j) and the finished sums by exp(Acs_i), which
//      Y_off needs as well; the kernel tiles go to the matrix cores as stored,
//      with no per-tile work;
//    - tile (plain bf16, no tile decaying by more than e^64): x_j staged times
//      exp(r_j) (r_j: the sum over j's later tokens in its 32-token tile), the
//      kernel tiles as stored, the accumulator scaled by exp(tile total) before
//      each tile's product and each row once by exp(-r_i) (details at
//      diag_blocks_tile); every factor the exp of a one-signed sum;
//    - per element, by additions only ([M] §3.5.4: segment sums formed without
//      subtracting cumsums): below the diagonal the sum over (j, i] is the sum
//      over j's later tokens in its 32-token tile (r_j, a table exp(r_j)), plus
//      the totals of the whole tiles between, plus the sum over i's tile up to
//      i (a lane scan), three terms of one sign, so the exponent carries a few
//      ulps of its own size however large the decays; on the diagonal tile each
//      lane adds up its own sums from its token down.  x is staged as is.  The
//      chunk-state kernel writes ell, r and the tile totals for these heads.
//  * Y_off uses the same lane layout: Hin (P x N, element dtype) is the A
//    operand, the lane's C row the B operand, exp(Acs_i) one scalar per lane.
//  * LDS operand reads are issued ahead of the MFMAs that use them (pinned by
//    scheduling barriers); each finished row tile of y is passed through the
//    wave's own LDS rows and written as whole 128-byte rows.
//  * Options: y may leave out each token's own term (C_i . B_i) x_i (the j == i
//    entries of the diagonal tile are cleared too; the backward pass uses it);
//    with the input entering as dt x, every x staging scale carries
//    dt_j (the chunk-state kernel provides Acs_j - ln dt_j; the per-element
//    mask stages x_j dt_j); the skip term D_h x is one more operand of the
//    diagonal tile's product (entry j == i), added instead to the finished
//    value before its store for the tokens whose dt is too small to divide by.
//  * fp32 accumulation; y rounded once to the element dtype and stored with the
//    non-temporal hint (nothing here reads it again); Hin, read here for the
//    last time, is loaded with that hint too.  (fp32 stores y straight from
//    the accumulators, 16 bytes per lane, so that its tiles fit in LDS at every
//    built chunk length and state size.)
#include "ssd_stage.hpp"

namespace ssd {

constexpr int kCoThreads = 512;  // 8 waves: two per SIMD, one workgroup per CU
// mask factorisation of a head (see the header)
constexpr int kMaskChunk = 0;  // whole chunk: x scaled by exp(-Acs_j), y by exp(Acs_i)
constexpr int kMaskTile = 1;   // per 32-token tile, from the per-element kind's one-signed sums
constexpr int kMaskExact = 2;  // per element, from addition-only segment sums
// |dt| below which the skip term of a token is not carried through the entry
// D_h / dt_i of the diagonal tile (it would overflow or lose x dt_i to
// underflow); D_h x is added to those tokens' finished values instead
constexpr float kSkipTinyDt = 0x1p-64f;
// heads per workgroup of the normalised output (its denominator's passed-state
// term is formed for all of them at once: one MFMA row block)
constexpr int kDenHeads = 8;

template <class E, int Q, int N>
struct ChunkOutputCfg {
  using T = typename E::storage;
  static constexpr bool kBf16 = E::kBytes == 2;
  static constexpr int P = kHeadDim;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int NP = N + PAD;  // LDS pitch of Hin rows
  static constexpr int QP = Q + PAD;  // LDS pitch of X^T rows
  static constexpr int YP = P + PAD;  // LDS pitch of a wave's staged output rows
  static constexpr int NW = kCoThreads / 64;
  static constexpr int NI = Q / 32;
  static constexpr int NTILE = NI * (NI + 1) / 2;            // causal 32x32 kernel tiles
  static constexpr int GV = kBf16 ? 2 : 4;                   // 16-byte vectors per lane per tile
  static constexpr int KS = N / E::kMfmaK;                   // MFMA steps over N
  // work of a wave: one row tile; with 8 row tiles both 32-wide halves of P,
  // with fewer row tiles one half (two waves share a row tile)
  static constexpr int NPH = NI == 8 ? 2 : 1;
  // normalised output with the dt-scaled input: the ones column's dt per token
  static constexpr size_t den_bytes = (size_t)Q * sizeof(float);
  static constexpr size_t ys_bytes = (size_t)NW * 32 * YP * sizeof(T);
  // X^T | Hin | output staging (bf16; with the normalised output and the
  // options, its dt table there instead, after them on fp32), one region (it
  // holds the chunk's B rows while the kernel tiles are formed)
  static constexpr size_t tiles_bytes =
      ((size_t)P * QP + (size_t)P * NP) * sizeof(T) + (kBf16 ? (ys_bytes > den_bytes ? ys_bytes : den_bytes) : den_bytes);
  static constexpr size_t base_bytes = tiles_bytes + 2 * Q * sizeof(float);
  static constexpr size_t g_bytes = (size_t)NTILE * GV * 64 * 16;
  static constexpr bool kGLds = base_bytes + g_bytes <= (size_t)kLdsLimit;  // kernel tiles in LDS
  static constexpr int BP = N + PAD;  // LDS pitch of the staged B rows
  // bf16 with the kernel tiles in LDS: the tiles are formed here, from B and C
  // (no kernel-matrix pass); otherwise they come from it (ws.cb, ws.cop)
  static constexpr bool kGInline = kBf16 && kGLds && (size_t)Q * BP * sizeof(T) <= tiles_bytes;
  static constexpr size_t lds_bytes = base_bytes + (kGLds ? g_bytes : 0);
  static constexpr bool fits = lds_bytes <= (size_t)kLdsLimit;
};

// kOpt: bit 0 the skip term, the dt-scaled input, the strict diagonal; bit 1
// the normalised output (its denominator formed here, y divided by it).
// Separate instantiations, so that the plain forward keeps every register it
// had and the normalised output alone does not carry the other options'
// registers.
template <class E, int Q, int N, int kOpt>
__global__ __launch_bounds__(kCoThreads, 1) void chunk_output_kernel(Problem p, Workspace ws, int HB) {
  using Cfg = ChunkOutputCfg<E, Q, N>;
  using T = typename E::storage;
  constexpr bool kOpts = (kOpt & 1) != 0;  // skip term, dt-scaled input, strict diagonal
  constexpr bool kDen = (kOpt & 2) != 0;   // normalised output
  constexpr int P = Cfg::P, NP = Cfg::NP, QP = Cfg::QP, KS = Cfg::KS, GV = Cfg::GV, YP = Cfg::YP;
  constexpr bool kBf16 = Cfg::kBf16;
  constexpr int NI = Cfg::NI, NTILE = Cfg::NTILE, NPH = Cfg::NPH;
  using CReg = typename std::conditional<kBf16, uint4, float>::type;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::tiles_bytes];
  T* XT = reinterpret_cast<T*>(smem);
  T* Hs = XT + P * QP;
  T* Ys = Hs + P * NP;  // bf16 output staging (all but the normalised output with options)
  // normalised output with options: dt_j of the ones column
  float* const dt_s = reinterpret_cast<float*>(Ys);
  // the normalised output with options finds its denominator in a pass of its
  // own before the products (the skip term's entry needs it); without options
  // the row sums ride along with the products
  constexpr bool kDenPre = kDen && kOpts;
  __shared__ __attribute__((aligned(16))) uint4 Gs[Cfg::kGLds ? NTILE * GV * 64 : 1];
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

  // this wave's row tile I and first half-tile of P.  8 row tiles: waves w and
  // w+4 (one SIMD) take row tiles w and 7-w, so every SIMD does the same
  // causal work; 4 or 2 row tiles: one half of P each.
  int I, ph0;
  if (NI == 8) {
    I = wid < 4 ? wid : 11 - wid;
    ph0 = 0;
  } else if (wid < NI) {
    I = wid;
    ph0 = 0;
  } else {
    I = 2 * NI - 1 - wid;  // negative for waves beyond 2 NI: idle
    ph0 = 1;
  }
  const bool active = I >= 0 && I < nI;

  const T* xbase = reinterpret_cast<const T*>(p.x) + cd.t0 * H * P;
  const T* hbase = reinterpret_cast<const T*>(ws.hin) + k * H * (int64_t)(P * N);
  const float* abase = ws.acs + k * H * Q;
  // log of the divisor x is staged with: Acs, or Acs - ln dt when the input
  // enters as dt x (then every staging scale below carries dt)
  const float* xlbase = (kOpts && p.x_times_dt) ? ws.xlog + k * H * Q : abase;
  // 1: the diagonal tile also clears j == i (y without each token's own term)
  const int sd = kOpts ? p.strict_diag : 0;
  // kernel tiles of the chunk's group: [tile][16-byte vector q][lane]
  const uint4* gsrc = reinterpret_cast<const uint4*>(ws.cb) + (k * G + g) * (int64_t)(NTILE * GV * 64);
  T* ybase = reinterpret_cast<T*>(p.y) + cd.t0 * H * P;

  // ---- issue the loads, in the order they are needed: the heads' chunk
  // decays, B rows (kernel tiles formed here) or the kernel tiles themselves
  // (to LDS), C rows, then the first head's x / Hin / Acs (which the tile
  // formation does not wait for)
  // the chunk's total log-decay of head h0 + (lane % HB), read per head with
  // readlane (a vector load, once: a scalar load in flight would hold up every
  // later wait for LDS reads); it selects each head's mask factorisation
  const float lam_v = ws.lam[k * H + h0 + lane % HB];
  // the plain bf16 forward factors a per-element head's mask by 32-token tile
  // when no tile of its chunk decays by more than the factorisation limit
  // (its largest tile decay, same lanes; written only for such heads)
  constexpr bool kTileMode = kBf16 && kOpt == 0 && Cfg::kGInline;
  const float tmax_v = kTileMode ? ws.tmax[k * H + h0 + lane % HB] : 0.0f;
  constexpr bool kCopyG = Cfg::kGLds && !Cfg::kGInline;
  constexpr int GNV = kCopyG ? NTILE * GV * 64 : 1;
  constexpr int GVPT = (GNV + kCoThreads - 1) / kCoThreads;
  uint4 gtmp[GVPT];
  if constexpr (kCopyG) {
#pragma unroll
    for (int i = 0; i < GVPT; ++i) gtmp[i] = gsrc[min(tid + i * kCoThreads, GNV - 1)];
  }
  RowTile<E, Cfg::kGInline ? Q : 8, N, kCoThreads> brows;
  if constexpr (Cfg::kGInline) brows.load(reinterpret_cast<const T*>(p.B) + (cd.t0 * G + g) * N, (int64_t)G * N, L);

  // every thread stages a 4-token block of x^T (bf16) and part of Hin
  using XTile = TransTile<E, Q, P, kCoThreads, 4>;
  XTile xt;
  RowTile<E, P, N, kCoThreads> ht;
  float a_own = 0.f;
  // bf16 options on the chunk (and tile) kinds: the step sizes come from the
  // coalesced table of Acs - ln dt (|Acs| <= 64 there, so exp(Acs - (Acs - ln dt))
  // gives dt to a few 1e-6), not from gathered loads of dt, one cache line per token
  constexpr bool kXlDt = kBf16;
  float dt_own = 1.0f;  // normalised output with the dt-scaled input: dt of token tid
                        // (kXlDt, chunk kind: Acs - ln dt of token tid instead)
  // chunk mask: log of the staging divisor of this thread's x rows.
  float xa4[XTile::NPT][4];
  // per-element mask: r of token tid (tid < Q); dt*A of this lane's output
  // token (lanes 0-31) or the chunk's tile totals (lane 32 + m: tile m)
  float ex_r = 0.0f, ex_e = 0.0f;
  const int i_tab = max(I, 0) * 32 + lr;  // this lane's token in the tables (idle waves: any)
  float dt_row = 1.0f;  // options: dt of this lane's output token (the skip term's entry)
                        // (kXlDt, chunk kind: Acs - ln dt of that token instead)
  float d_head = 0.0f;  // options: the skip weight D_h of the prefetched head
  // kind: the head's mask factorisation (a constant at every call)
  auto prefetch = [&](int h, int kind) {
    xt.load(xbase + h * P, (int64_t)H * P, L);
    ht.template load<true>(hbase + h * (int64_t)(P * N), N, P);  // Hin's last read
    // token tid's Acs (the tile kind: its r, the LDS table of the row factors)
    if (tid < Q) a_own = (kind == kMaskTile ? ws.rsuf + (k * H + h) * Q : abase + h * Q)[tid];
    // options: dt of token tid (the normalised output's ones column), the
    // skip term's weight D_h, and the dt of this lane's output token its entry
    // divides by, loaded with the head's other values and whatever the
    // run-time options (D_h from dt when there is no D; the options decide at
    // the use).  A load from before the head loop read inside it, or a load
    // under a run-time condition, would make every head wait for all the
    // loads in flight, the next head's among them.
    if constexpr (kOpts) {
      const bool from_xl = kXlDt && kind != kMaskExact;
      if constexpr (kDen)
        dt_own = from_xl ? (xlbase + h * Q)[min(tid, Q - 1)] : p.dt[(cd.t0 + min(tid, L - 1)) * H + h];
      d_head = *(p.D != nullptr ? p.D + h : p.dt);
      dt_row = from_xl ? (xlbase + h * Q)[i_tab] : p.dt[(cd.t0 + min(i_tab, L - 1)) * H + h];
    }
    if (kind != kMaskExact) {
      // the log of x's staging scale: -Acs (chunk) or r (tile) of the thread's rows
      const float* src = kind == kMaskChunk ? xlbase + h * Q : ws.rsuf + (k * H + h) * Q;
#pragma unroll
      for (int i = 0; i < XTile::NPT; ++i) {
        const int r0 = XTile::first_row(i);
        const float4 a4 = *reinterpret_cast<const float4*>(src + r0);
        xa4[i][0] = a4.x; xa4[i][1] = a4.y; xa4[i][2] = a4.z; xa4[i][3] = a4.w;
      }
      // the tile kind's tile totals, threads 0-7
      if (kind == kMaskTile && tid < 8) ex_e = ws.ttot[(k * H + h) * 8 + tid];
    } else {
      const int64_t kh = k * H + h;
      ex_r = ws.rsuf[kh * Q + min(tid, Q - 1)];
      const float* et_src = lane < 32 ? ws.ell + kh * Q + i_tab : ws.ttot + kh * 8 + (lane & 7);
      ex_e = *et_src;
    }
  };
  // C row of this lane's token as MFMA B-operand slices over N, kept in
  // registers for all heads: straight from C (rows past the chunk end clamped;
  // their outputs are never stored), or in lane order from the kernel-matrix
  // pass (coalesced).  fp32 with N > 64: read from that pass's copy at each
  // use instead (the slices would take N/2 registers).
  constexpr bool kCRegs = kBf16 || KS <= 32;
  const CReg* cop_g = reinterpret_cast<const CReg*>(ws.cop) + (k * G + g) * (int64_t)(NI * KS * 64) + lane;
  CReg creg[kCRegs ? KS : 1];
  if (active && kCRegs) {
    if constexpr (Cfg::kGInline) {
      const T* crow = reinterpret_cast<const T*>(p.C) + ((cd.t0 + min(I * 32 + lr, L - 1)) * G + g) * N + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) creg[ks] = *reinterpret_cast<const CReg*>(crow + ks * 16);
    } else {
#pragma unroll
      for (int ks = 0; ks < (kCRegs ? KS : 1); ++ks) creg[ks] = cop_g[(I * KS + ks) * 64];
    }
  }
  // the block's heads by mask factorisation (uniform bit masks over hh):
  // the chunk heads are done first, in a loop built for that factorisation
  // alone, then the per-element heads in a loop of their own, so that the
  // chunk path's registers and schedule are not shaped by the other's code
  const uint64_t hb_bits = HB >= 64 ? ~0ull : ((1ull << HB) - 1);
  const uint64_t exact_bits = __builtin_amdgcn_ballot_w64(!mask_by_chunk<E>(lam_v)) & hb_bits;
  const uint64_t chunk_bits = hb_bits & ~exact_bits;
  const uint64_t tile_bits =
      kTileMode ? (__builtin_amdgcn_ballot_w64(!mask_by_chunk<E>(lam_v) && tmax_v <= 64.0f) & hb_bits) : 0;
  const uint64_t walk_bits = exact_bits & ~tile_bits;
  const int first_exact = exact_bits ? (int)__builtin_ctzll(exact_bits) : -1;
  // normalised output: the Zin rows of the block's heads (rows past HB stored
  // as zeros), issued ahead of the first head's loads so that the
  // denominator's product below does not wait for those
  RowTile<E, 32, N, kCoThreads> zt;
  if constexpr (kDen) zt.load(reinterpret_cast<const T*>(ws.zin) + (k * H + h0) * (int64_t)N, N, HB);
  // the first head's loads, of the chunk kind whatever its factorisation (a
  // conditional prefetch here would make the tile formation below wait for
  // it); a block of per-element heads only issues them again, with its
  // tables, between the two loops below
  prefetch(h0 + (chunk_bits ? (int)__builtin_ctzll(chunk_bits) : first_exact), kMaskChunk);

  if constexpr (kCopyG) {
#pragma unroll
    for (int i = 0; i < GVPT; ++i)
      if (tid + i * kCoThreads < GNV) Gs[tid + i * kCoThreads] = gtmp[i];
  }
  if constexpr (Cfg::kGInline) {
    // kernel tiles G^T = B_J C_I^T of this wave's row tile (one wave per row
    // tile), B rows staged in LDS: acc[r] = G[32I + lr][32J + 8(r/4) + 4lg + r%4]
    constexpr int BP = Cfg::BP;
    T* Bs = reinterpret_cast<T*>(smem);
    brows.template store<BP>(Bs);
    lds_barrier();
    if (active && ph0 == 0) {
      for (int J = 0; J <= I; ++J) {
        uint4 a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          a[ks] = *reinterpret_cast<const uint4*>(Bs + (J * 32 + lr) * BP + ks * 16 + lg * 8);
        floatx16_t acc = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(a[ks], creg[ks], acc);
        uint4 o0, o1;
        o0.x = pack_bf16x2(acc[0], acc[1]);   o0.y = pack_bf16x2(acc[2], acc[3]);
        o0.z = pack_bf16x2(acc[4], acc[5]);   o0.w = pack_bf16x2(acc[6], acc[7]);
        o1.x = pack_bf16x2(acc[8], acc[9]);   o1.y = pack_bf16x2(acc[10], acc[11]);
        o1.z = pack_bf16x2(acc[12], acc[13]); o1.w = pack_bf16x2(acc[14], acc[15]);
        const int tile = I * (I + 1) / 2 + J;
        Gs[(tile * GV + 0) * 64 + lane] = o0;
        Gs[(tile * GV + 1) * 64 + lane] = o1;
      }
    }
    // the head loop's first barrier orders these tiles before their use and
    // the B rows' last read before x^T and Hin overwrite them
  }
  // normalised output: this lane's token's passed-state term of the
  // denominator for heads 4 lg + e (e < 4), in registers for the head loop
  float dofv[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kDen) {
    // ---- normalised output: the passed-state term of the denominator for
    // all the block's heads at once, Doff^T (heads x tokens) = Zin C^T, Zin
    // of each head (its ones column's passed state, N values) an A-operand
    // row and the lane's C row the B operand, as for Y_off
    lds_barrier();  // the tile formation's B rows (same region) are no longer read
    zt.template store<NP>(XT);
    lds_barrier();
    if (active) {  // both waves of a shared row tile keep the term
      floatx16_t accd = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (kBf16) {
          accd = mfma32x32x16(*reinterpret_cast<const uint4*>(XT + lr * NP + ks * 16 + lg * 8), creg[ks], accd);
        } else {
          const float c = kCRegs ? creg[kCRegs ? ks : 0] : cop_g[(I * KS + ks) * 64];
          accd = mfma32x32x2(XT[lr * NP + ks * 2 + lg], c, accd);
        }
      }
      // accd[e] = Doff[head 4 lg + e][token 32 I + lr], kept for the head loop
#pragma unroll
      for (int e = 0; e < 4; ++e) dofv[e] = accd[e];
    }
    // the head loop's first barrier orders the Zin rows' last read before
    // x^T overwrites them
  }

  // one head hh of the block; nxt: the next head of the same factorisation
  // (its loads are issued here, under this head's products), -1 for none.
  // The prefetch's kind is fixed per loop: loads of either kind into shared
  // registers would need copies where the two kinds join, and those wait for
  // every load in flight.
  auto head_iter = [&](const int hh, const int nxt, auto kind_tag) __attribute__((always_inline)) {
    constexpr int kind = decltype(kind_tag)::value;
    constexpr bool by_chunk = kind == kMaskChunk, by_tile = kind == kMaskTile, by_elem = kind == kMaskExact;
    const int h = h0 + hh;
    lds_barrier();  // every wave is done with the previous head's tiles
    ht.template store<NP, kBf16>(Hs);
    // mask factorisation of this head (see the header)
    if (tid < Q) {
      acs_s[tid] = a_own;  // Acs; the tile kind: r (the row factors' exponents)
      // exp of the sum of dt*A over the later tokens of j's tile
      if (by_elem) w_s[tid] = __expf(ex_r);
      // the tile kind's tile totals (its w_s is otherwise unused), written
      // here so that their registers are free for the next head's loads
      if (by_tile && tid < 8) w_s[tid] = ex_e;
      if constexpr (kDen) {
        // the ones column's staging: exp(-Acs_j) dt_j (chunk mask; w_s is
        // free there), dt_j (per-element mask).  bf16 without options: the
        // chunk mask's values as bf16 pairs (j, j + 1) in word j / 2, for the
        // products' row sums on v_dot2_f32_bf16
        if (by_chunk) {
          // (kXlDt: dt_own holds Acs - ln dt, or Acs without the dt-scaled input)
          const float sj = kOpts ? (kXlDt ? __expf(-dt_own) : __expf(-a_own) * (p.x_times_dt ? dt_own : 1.0f))
                                 : __expf(-a_own);
          if constexpr (kBf16 && !kDenPre) {
            const float sn = __shfl_down(sj, 1, kWave);
            if ((tid & 1) == 0) reinterpret_cast<uint32_t*>(w_s)[tid >> 1] = pack_bf16x2(sj, sn);
          } else {
            w_s[tid] = sj;
          }
        } else if (kDenPre) {
          dt_s[tid] = dt_own;
        }
      }
    }
    if (by_chunk || by_tile) {
      // x_j scaled by exp(-Acs_j) (chunk) or exp(r_j) (tile: the sum of dt*A
      // over j's later tokens in its tile, in (0, 1])
      float sreg[XTile::NPT][4];
#pragma unroll
      for (int i = 0; i < XTile::NPT; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sreg[i][rr] = __expf(by_chunk ? -xa4[i][rr] : xa4[i][rr]);
      xt.template store<QP, 2, kBf16, false, kBf16>(XT, nullptr, sreg);
    } else if (kOpts && p.x_times_dt) {
      // per-element mask: x staged times dt_j, read as given (|Acs_j| may be
      // large here, so Acs_j - ln dt_j would not give ln dt_j back to fp32
      // precision)
      float sreg[XTile::NPT][4];
#pragma unroll
      for (int i = 0; i < XTile::NPT; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          sreg[i][rr] = p.dt[(cd.t0 + min(XTile::first_row(i) + rr, L - 1)) * H + h];
      xt.template store<QP, 2, kBf16, false, kBf16>(XT, nullptr, sreg);
    } else {
      xt.template store<QP, 0, kBf16, false, kBf16>(XT, nullptr);
    }
    lds_barrier();
    const float et = ex_e;  // this head's dt*A / tile totals (per-element mask)
    const float dt_cap = dt_row;  // (options) this head's, before the next head's prefetch
    const float dh = d_head;
    if (nxt >= 0) prefetch(h0 + nxt, kind);
    if (!active) return;

    const int i_loc = I * 32 + lr;
    // per-element mask: the sum of dt*A over this lane's tile up to its token
    // (a scan over lanes 0-31, which hold the tile's tokens; lane half 1 takes
    // the value of its row from half 0)
    const float ci = by_elem ? __shfl(seg_inclusive_sum<32>(et), lr) : 0.0f;
    // kernel tile J of row tile I as 16 fp32 values: G[i_loc][32J + 8(r/4) + 4lg + r%4]
    auto g_values = [&](int J, float (&g)[16]) {
      const int tl = I * (I + 1) / 2 + J;
      if constexpr (kBf16) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint4 v = Cfg::kGLds ? Gs[(tl * GV + q) * 64 + lane] : gsrc[(tl * GV + q) * 64 + lane];
          g[8 * q + 0] = bf16_lo(v.x); g[8 * q + 1] = bf16_hi(v.x);
          g[8 * q + 2] = bf16_lo(v.y); g[8 * q + 3] = bf16_hi(v.y);
          g[8 * q + 4] = bf16_lo(v.z); g[8 * q + 5] = bf16_hi(v.z);
          g[8 * q + 6] = bf16_lo(v.w); g[8 * q + 7] = bf16_hi(v.w);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = Cfg::kGLds ? Gs[(tl * GV + q) * 64 + lane] : gsrc[(tl * GV + q) * 64 + lane];
          g[4 * q + 0] = __uint_as_float(v.x); g[4 * q + 1] = __uint_as_float(v.y);
          g[4 * q + 2] = __uint_as_float(v.z); g[4 * q + 3] = __uint_as_float(v.w);
        }
      }
    };
    // normalised output: the token's denominator d_i, the output of the ones
    // column, before the products (the skip term's entry and the division
    // need it):
    //   chunk mask:   d_i = exp(Acs_i) (Doff_i + sum_{j<=i} G_ij s_j),
    //                 s_j = exp(-Acs_j) w_j (w_s), w_j = dt_j or 1
    //   per element:  d_i = exp(Acs_i) Doff_i + sum_{j<=i} L_ij G_ij w_j (w_j in dt_s)
    // with the same mask sums as the products below; the two lane halves
    // hold different columns j of row i and add their partial sums.
    float den = 1.0f;
    // the passed-state term of head hh at this lane's token (held by the lane
    // of the same token in half hh / 4)
    float dof = 0.0f;
    if constexpr (kDen) {
      const int e = hh & 3;
      const float mine = e == 0 ? dofv[0] : e == 1 ? dofv[1] : e == 2 ? dofv[2] : dofv[3];
      dof = __shfl(mine, lr + 32 * (hh >> 2));
    }
    // row sums of the masked tiles against the ones column (both lane halves):
    // in a pass of their own before the products with options (the skip
    // term's entry needs the denominator) and for the per-element mask (the
    // sums ride along the chunk mask's products only)
    float rs = 0.0f;
    if (kDenPre || (kDen && !by_chunk)) {
      if (by_chunk) {
        for (int J = 0; J <= I; ++J) {
          float g[16];
          g_values(J, g);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 s4 = *reinterpret_cast<const float4*>(w_s + J * 32 + q * 8 + lg * 4);
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int jr = q * 8 + lg * 4 + e;
              rs += (J < I || jr + sd <= lr) ? g[4 * q + e] * sv[e] : 0.0f;
            }
          }
        }
        rs += __shfl_xor(rs, 32);
        den = __expf(acs_s[i_loc]) * (dof + rs);
      } else {
        float gs = 0.0f;  // the whole tiles strictly between J and I
        for (int J = I - 1; J >= 0; --J) {
          float g[16];
          g_values(J, g);
          const float u = __expf(ci + gs);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 w4 = *reinterpret_cast<const float4*>(w_s + J * 32 + q * 8 + lg * 4);
            const float4 d4 = (kOpts && p.x_times_dt) ? *reinterpret_cast<const float4*>(dt_s + J * 32 + q * 8 + lg * 4)
                                                      : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            rs += g[4 * q + 0] * (u * w4.x) * d4.x + g[4 * q + 1] * (u * w4.y) * d4.y +
                  g[4 * q + 2] * (u * w4.z) * d4.z + g[4 * q + 3] * (u * w4.w) * d4.w;
          }
          gs += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(et), 32 + J));
        }
        // the diagonal tile: the lane's own sums over (j, i], as in the products
        float g[16];
        g_values(I, g);
        float sq[4];
        float run = 0.0f;
#pragma unroll
        for (int jj = 31; jj >= 0; --jj) {
          if ((jj >> 2) & 1) {
            sq[jj & 3] = run;
          } else {
            const int r = (jj >> 3) * 4 + (jj & 3);
            const int jr = (r >> 2) * 8 + lg * 4 + (r & 3);
            const float sr = lg ? sq[jj & 3] : run;
            rs += (jr + sd <= lr) ? g[r] * __expf(sr) * ((kOpts && p.x_times_dt) ? dt_s[I * 32 + jr] : 1.0f) : 0.0f;
          }
          const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(et), jj));
          run += jj <= lr ? e : 0.0f;
        }
        rs += __shfl_xor(rs, 32);
        den = __expf(acs_s[i_loc]) * dof + rs;
      }
      if (ph0 == 0 && lg == 0 && i_loc < L) p.denom[(cd.t0 + i_loc) * H + h] = den;
    }
    floatx16_t acc[NPH];
#pragma unroll
    for (int j = 0; j < NPH; ++j) acc[j] = zero16();
    // rows of X^T and Hin (p) this wave's halves read
    auto prow = [&](int j) { return (ph0 + j) * 32 + lr; };

    // Y_off^T = Hin C^T (contraction over N), then the exp(Acs_i) factor
    if constexpr (kBf16) {
      // Hin operands of step ks + 2 are read while step ks multiplies
      uint4 ha[3][NPH];
      auto read_h = [&](int ks, uint4 (&r)[NPH]) {
#pragma unroll
        for (int j = 0; j < NPH; ++j)
          r[j] = *reinterpret_cast<const uint4*>(Hs + prow(j) * NP + ks * 16 + lg * 8);
      };
      read_h(0, ha[0]);
      if (KS > 1) read_h(1, ha[1]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) read_h(ks + 2, ha[(ks + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NPH; ++j) acc[j] = mfma32x32x16(ha[ks % 3][j], creg[ks], acc[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll 8
      for (int ks = 0; ks < KS; ++ks) {
        const float c = kCRegs ? creg[kCRegs ? ks : 0] : cop_g[(I * KS + ks) * 64];
#pragma unroll
        for (int j = 0; j < NPH; ++j) acc[j] = mfma32x32x2(Hs[prow(j) * NP + ks * 2 + lg], c, acc[j]);
      }
    }
    const float ai = acs_s[i_loc];
    const float eo = __expf(ai);
    // options: dt of this lane's token (kXlDt, chunk kind: from Acs - ln dt)
    const float dti = (kXlDt && !by_elem) ? __expf(ai - dt_cap) : dt_cap;
    // skip term D_h x_i as an extra diagonal entry of the tile product: x^T_i
    // is x_i times a staging scale that the output factor undoes, so the entry
    // is D_h, over dt_i when the input enters as dt x (x^T_i then carries dt_i),
    // times the denominator when the output is normalised (divided out again).
    // A token with dt_i = 0 has x^T_i = 0 there: its term is added to the
    // finished value before the store.
    float dsk = 0.0f;
    if constexpr (kOpts) {
      if (p.D != nullptr) {
        dsk = dh;
        if constexpr (kDen) dsk *= den;
        if (p.x_times_dt) {
          // x^T_i carries dt_i: a dt too small to divide by (zero included)
          // leaves the term to the store
          dsk = fabsf(dti) < kSkipTinyDt ? 0.0f : dsk / dti;
        }
      }
    }
    float gsum = 0.0f;
    if (by_elem) {
#pragma unroll
      for (int j = 0; j < NPH; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] *= eo;
    }

    // diagonal block: kernel tiles J <= I of row tile I (consecutive tiles)
    const int tile0 = I * (I + 1) / 2;
    auto load_g = [&](int J, uint4 (&gv)[GV]) {
#pragma unroll
      for (int q = 0; q < GV; ++q) {
        if constexpr (Cfg::kGLds)
          gv[q] = Gs[((tile0 + J) * GV + q) * 64 + lane];
        else
          gv[q] = gsrc[((tile0 + J) * GV + q) * 64 + lane];
      }
    };
    // this lane group's x^T operands of tile J
    auto load_x = [&](int J, uint4 (&xa)[2][NPH]) {
      if constexpr (kBf16) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          // tokens are permuted within 16-groups: this lane group's 8 are contiguous
          const int col = J * 32 + kk * 16 + lg * 8;
#pragma unroll
          for (int j = 0; j < NPH; ++j) xa[kk][j] = *reinterpret_cast<const uint4*>(XT + prow(j) * QP + col);
        }
      }
    };
    // operands of one kernel tile: G values, x^T operands
    struct TileOps {
      uint4 g[GV];
      uint4 x[2][NPH];
    };
    auto load_ops = [&](int J, TileOps& o) {
      load_g(J, o.g);
      load_x(J, o.x);
    };
    // kDiag: the diagonal tile J == I (causal mask inside the tile)
    auto tile = [&](int J, const TileOps& o, auto diag_tag, auto mode_tag) {
      constexpr bool kDiag = decltype(diag_tag)::value;
      constexpr int kMode = decltype(mode_tag)::value;
      const uint4 (&gv)[GV] = o.g;
      const uint4 (&xa)[2][NPH] = o.x;
      // value r of this lane: G[i_loc][j_r], j_r = 32J + 8(r/4) + 4 lg + r%4
      if constexpr (kBf16) {
        if constexpr (kMode == kMaskChunk) {
          // the tile is the B operand as stored (bf16 pairs); on the diagonal
          // the entries with j > i are cleared
          uint4 b[2] = {gv[0], gv[1]};
          if constexpr (kDiag) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              uint32_t m[4];
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const int r = 8 * q + 2 * d;
                const int j0 = (r >> 2) * 8 + lg * 4 + (r & 3);  // j - 32J of values r, r+1
                m[d] = (j0 + sd <= lr ? 0x0000ffffu : 0u) | (j0 + 1 + sd <= lr ? 0xffff0000u : 0u);
              }
              b[q].x &= m[0]; b[q].y &= m[1]; b[q].z &= m[2]; b[q].w &= m[3];
            }
            if constexpr (kOpts) {
              if (p.D != nullptr) {
                // the skip weight on the entry j == i, as an operand of its own
                const uint32_t sw = pack_bf16x2(dsk, 0.0f);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                  uint32_t w[4];
#pragma unroll
                  for (int d = 0; d < 4; ++d) {
                    const int j0 = ((8 * q + 2 * d) >> 2) * 8 + lg * 4 + (2 * d & 3);
                    w[d] = (j0 == lr ? sw : 0u) | (j0 + 1 == lr ? sw << 16 : 0u);
                  }
                  const uint4 bd = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
                  for (int j = 0; j < NPH; ++j) acc[j] = mfma32x32x16(xa[q][j], bd, acc[j]);
                }
              }
            }
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < NPH; ++j) acc[j] = mfma32x32x16(xa[kk][j], b[kk], acc[j]);
          if constexpr (kDen && !kDenPre) {
            // the denominator's row sums: the masked tile against s_j (bf16
            // pairs in w_s), two products per v_dot2_f32_bf16
            const uint32_t* sw = reinterpret_cast<const uint32_t*>(w_s) + J * 16 + lg * 2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint2 s2 = *reinterpret_cast<const uint2*>(sw + q * 4);
              const uint4& bq = b[q >> 1];
              const uint32_t w0 = (q & 1) ? bq.z : bq.x, w1 = (q & 1) ? bq.w : bq.y;
              rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0), __builtin_bit_cast(bf16x2_t, s2.x),
                                                   rs, false);
              rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1), __builtin_bit_cast(bf16x2_t, s2.y),
                                                   rs, false);
            }
          }
          return;
        }
      }
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
      if constexpr (kMode == kMaskChunk) {
        // (fp32) x^T carries exp(-Acs_j); exp(Acs_i) is applied to the sum
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jr = (r >> 2) * 8 + lg * 4 + (r & 3);  // j - 32J
          v[r] = (!kDiag || jr + sd <= lr) ? gt[r] : 0.0f;
          if (kOpts && kDiag && jr == lr) v[r] += dsk;
        }
      } else if constexpr (!kDiag) {
        // the sum over (j, i] is r_j (the w table holds exp(r_j)) + the totals
        // of the whole tiles strictly between J and I (gsum) + ci: three sums
        // of one sign, each factor in (0, 1]
        const float u = __expf(ci + gsum);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 w4 = *reinterpret_cast<const float4*>(w_s + J * 32 + q * 8 + lg * 4);
          v[4 * q + 0] = gt[4 * q + 0] * (u * w4.x);
          v[4 * q + 1] = gt[4 * q + 1] * (u * w4.y);
          v[4 * q + 2] = gt[4 * q + 2] * (u * w4.z);
          v[4 * q + 3] = gt[4 * q + 3] * (u * w4.w);
        }
      } else {
        // diagonal tile: the lane adds dt*A from its own token i down, and
        // takes the running sum over (j, i] at each of its 16 columns j
        // (columns 8q + e for lane half 0, 8q + 4 + e for half 1, e < 4: the
        // half-1 column's sum waits in sq[e] for the half-0 column 4 below; a
        // column past i gets an empty sum and is masked)
        float sq[4];
        float run = 0.0f;
#pragma unroll
        for (int jj = 31; jj >= 0; --jj) {
          if ((jj >> 2) & 1) {
            sq[jj & 3] = run;
          } else {
            const int r = (jj >> 3) * 4 + (jj & 3);
            const int jr = (r >> 2) * 8 + lg * 4 + (r & 3);  // j - 32J
            const float sr = lg ? sq[jj & 3] : run;
            v[r] = (jr + sd <= lr) ? gt[r] * __expf(sr) : 0.0f;
            if (kOpts && jr == lr) v[r] += dsk;
          }
          const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(et), jj));
          run += jj <= lr ? e : 0.0f;
        }
      }
      if constexpr (kDen && !kDenPre && kMode == kMaskChunk) {
        // the denominator's row sums (fp32, chunk mask): against s_j (w_s)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 s4 = *reinterpret_cast<const float4*>(w_s + J * 32 + q * 8 + lg * 4);
          rs += v[4 * q] * s4.x + v[4 * q + 1] * s4.y + v[4 * q + 2] * s4.z + v[4 * q + 3] * s4.w;
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
#pragma unroll
          for (int j = 0; j < NPH; ++j) acc[j] = mfma32x32x16(xa[kk][j], bop, acc[j]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = J * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
#pragma unroll
          for (int jj = 0; jj < NPH; ++jj) acc[jj] = mfma32x32x2(XT[prow(jj) * QP + j], v[r], acc[jj]);
        }
      }
    };
    // off-diagonal tiles J < I in pairs, then the diagonal tile J = I; two
    // operand buffers used in turn, the next tile's being read while the
    // current one is masked and multiplied
    using Off = std::integral_constant<bool, false>;
    using Diag = std::integral_constant<bool, true>;
    // one copy of the loop for the chunk factorisation (no per-tile work) and
    // one for the other two
    auto diag_blocks = [&](auto mode_tag) {
      if constexpr (kDen && (kOpts || !Cfg::kGInline)) {
        // normalised output with options, or with the tiles from the
        // kernel-matrix pass: one operand buffer (a second one's registers
        // would push the loop into spills)
        TileOps ob;
        for (int J = 0; J < I; ++J) {
          load_ops(J, ob);
          tile(J, ob, Off(), mode_tag);
        }
        load_ops(I, ob);
        tile(I, ob, Diag(), mode_tag);
        return;
      }
      TileOps ob0, ob1;
      load_ops(0, ob0);
      int J = 0;
      for (; J + 1 < I; J += 2) {
        load_ops(J + 1, ob1);
        tile(J, ob0, Off(), mode_tag);
        load_ops(J + 2, ob0);
        tile(J + 1, ob1, Off(), mode_tag);
      }
      if (J < I) {
        load_ops(I, ob1);
        tile(J, ob0, Off(), mode_tag);
        tile(I, ob1, Diag(), mode_tag);
      } else {
        tile(I, ob0, Diag(), mode_tag);
      }
    };
    // per-element mask: the diagonal tile first, then J = I - 1 down to 0, so
    // that gsum, the sum over the whole tiles strictly between J and I, grows
    // by one tile total per step (additions only).  One operand buffer: the
    // per-element work already hides the LDS reads, and a second buffer's
    // registers would be held through the whole kernel.
    auto diag_blocks_exact = [&]() {
      using M = std::integral_constant<int, kMaskExact>;
      TileOps ob;
      load_ops(I, ob);
      tile(I, ob, Diag(), M());
      for (int J = I - 1; J >= 0; --J) {
        load_ops(J, ob);
        tile(J, ob, Off(), M());
        gsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(et), 32 + J));
      }
    };
    // tile factorisation (plain bf16): with x_j staged times exp(r_j), the
    // sum over (j, i] for j in tile J < I is r_j + the totals of the tiles
    // strictly between + c_i, and c_i = T_I - r_i, so that
    //   y_i = exp(-r_i) [e_0..e_I (C h)_i + sum_J<I e_(J+1)..e_I P_J + P_I]
    // with e_g = exp(T_g) (tile totals, one-signed sums) and P_J the tile
    // products with the kernel tiles as stored: the accumulator is scaled by
    // e_J before each tile J is added (Horner), then by exp(-r_i) once.  Every
    // factor is a one-signed sum's exp: e_g and exp(r_j) in (0, 1], exp(-r_i)
    // within e^64 (the largest tile decay of such a head).
    auto diag_blocks_tile = [&]() {
      using M = std::integral_constant<int, kMaskChunk>;  // tiles to the matrix cores as stored
      auto scale = [&](int g) {
        const float e = __expf(w_s[g]);  // e_g, the same for every lane
#pragma unroll
        for (int j = 0; j < NPH; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][r] *= e;
      };
      TileOps ob0, ob1;
      load_ops(0, ob0);
      int J = 0;
      for (; J + 1 < I; J += 2) {
        load_ops(J + 1, ob1);
        scale(J);
        tile(J, ob0, Off(), M());
        load_ops(J + 2, ob0);
        scale(J + 1);
        tile(J + 1, ob1, Off(), M());
      }
      if (J < I) {
        load_ops(I, ob1);
        scale(J);
        tile(J, ob0, Off(), M());
        scale(I);
        tile(I, ob1, Diag(), M());
      } else {
        scale(I);
        tile(I, ob0, Diag(), M());
      }
      const float er = __expf(-ai);  // ai holds r of this lane's token (the tile kind)
#pragma unroll
      for (int j = 0; j < NPH; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] *= er;
    };
    if constexpr (by_chunk)
      diag_blocks(std::integral_constant<int, kMaskChunk>());
    else if constexpr (by_tile)
      diag_blocks_tile();
    else
      diag_blocks_exact();
    if (kDen && !kDenPre && by_chunk) {
      rs += __shfl_xor(rs, 32);
      den = eo * (dof + rs);
      if (ph0 == 0 && lg == 0 && i_loc < L) p.denom[(cd.t0 + i_loc) * H + h] = den;
    }
    if (by_chunk) {
      // both parts of y carry exp(Acs_i) as one factor
#pragma unroll
      for (int j = 0; j < NPH; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] *= eo;
    }
    if constexpr (kDen) {
      // normalised output: divided by the token's denominator before rounding
      const float inv = 1.0f / den;
#pragma unroll
      for (int j = 0; j < NPH; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] *= inv;
    }
    // store: lane holds Y^T row pr = 32 (ph0 + j) + 8(r/4) + 4 lg + r%4 of token
    // i_loc.
    // options, input entering as dt x, with the skip term: a token whose |dt|
    // is too small to carry the term through the diagonal entry gets D_h x_i
    // added here to its finished value (x read from memory for those only)
    const bool skip_late = kOpts && p.x_times_dt && p.D != nullptr;
    const T* xhead = xbase + h * P;
    if constexpr (!kBf16) {
      // fp32: four consecutive p per 16-byte store, straight from the accumulators
      if (i_loc < L) {
        T* yrow = ybase + (int64_t)i_loc * H * P + h * P;
        const bool late = skip_late && fabsf(dti) < kSkipTinyDt;
#pragma unroll
        for (int j = 0; j < NPH; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float4 v4 = make_float4(acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]);
            if (late) {
              const float4 x4 = *reinterpret_cast<const float4*>(xhead + (int64_t)i_loc * H * P + 32 * (ph0 + j) + 8 * q + 4 * lg);
              v4.x += dh * x4.x; v4.y += dh * x4.y; v4.z += dh * x4.z; v4.w += dh * x4.w;
            }
            store_nt(reinterpret_cast<uint4*>(yrow + 32 * (ph0 + j) + 8 * q + 4 * lg),
                     make_uint4(__float_as_uint(v4.x), __float_as_uint(v4.y), __float_as_uint(v4.z),
                                __float_as_uint(v4.w)));
          }
      }
    } else if constexpr (kDenPre) {
      // bf16, normalised output with options (its dt table occupies the
      // staging rows): the four values of each group straight to y as 8 bytes
      // (p permuted as below)
      if (i_loc < L) {
        T* yrow = ybase + (int64_t)i_loc * H * P + h * P;
        const bool late = skip_late && fabsf(dti) < kSkipTinyDt;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < NPH; ++j) {
            const int pp = q * 8 + 4 * (lg ^ ((ph0 + j) & 1));
            const floatx16_t& a = acc[j];
            uint2 v2 = make_uint2(pack_bf16x2(a[4 * q + (0 ^ q)], a[4 * q + (1 ^ q)]),
                                  pack_bf16x2(a[4 * q + (2 ^ q)], a[4 * q + (3 ^ q)]));
            if (late)
              v2 = add_scaled<E>(v2, *reinterpret_cast<const uint2*>(xhead + (int64_t)i_loc * H * P + 32 * (ph0 + j) + pp), dh);
            *reinterpret_cast<uint2*>(yrow + 32 * (ph0 + j) + pp) = v2;
          }
      }
    } else {
      // bf16 rows are permuted (lds_row_perm), so its p is pr ^ c with
      // c = 4 ((ph0 + j) & 1) + r/4: the four values of a group r/4 = q land in
      // the 4-group 8q + 4 (lg ^ ((ph0 + j) & 1)), value e at position e ^ q.
      // The row tile goes through this wave's LDS rows so that global stores are
      // whole rows (of the wave's part of P) instead of scattered pieces.
      T* ys = Ys + wid * 32 * YP;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int j = 0; j < NPH; ++j) {
          const int pp = q * 8 + 4 * (lg ^ ((ph0 + j) & 1));
          const floatx16_t& a = acc[j];
          *reinterpret_cast<uint2*>(ys + lr * YP + 32 * j + pp) =
              make_uint2(pack_bf16x2(a[4 * q + (0 ^ q)], a[4 * q + (1 ^ q)]),
                         pack_bf16x2(a[4 * q + (2 ^ q)], a[4 * q + (3 ^ q)]));
        }
      }
      __builtin_amdgcn_wave_barrier();
      constexpr int VPR = NPH * 32 * sizeof(T) / 16;  // 16-byte vectors per output row
      constexpr int RPI = 64 / VPR;                   // rows per store instruction
#pragma unroll
      for (int s = 0; s < 32 / RPI; ++s) {
        const int row = s * RPI + lane / VPR;
        const int vec = lane % VPR;
        const int i_row = I * 32 + row;
        uint4 val = *reinterpret_cast<const uint4*>(ys + row * YP + vec * (16 / sizeof(T)));
        if (skip_late) {
          const float dtr = __shfl(dti, row);  // lane `row` holds that token's dt
          if (i_row < L && fabsf(dtr) < kSkipTinyDt)
            val = add_scaled<E>(val, *reinterpret_cast<const uint4*>(xhead + (int64_t)i_row * H * P + ph0 * 32 + vec * (16 / sizeof(T))), dh);
        }
        if (i_row < L)
          store_nt(reinterpret_cast<uint4*>(ybase + (int64_t)i_row * H * P + h * P + ph0 * 32 + vec * (16 / sizeof(T))),
                   val);
      }
      __builtin_amdgcn_wave_barrier();
    }
  };
  using KChunk = std::integral_constant<int, kMaskChunk>;
  using KTile = std::integral_constant<int, kMaskTile>;
  using KElem = std::integral_constant<int, kMaskExact>;
  for (uint64_t m = chunk_bits; m;) {
    const int hh = (int)__builtin_ctzll(m);
    m &= m - 1;
    head_iter(hh, m ? (int)__builtin_ctzll(m) : -1, KChunk());
  }
  if constexpr (kTileMode) {
    if (tile_bits) prefetch(h0 + (int)__builtin_ctzll(tile_bits), kMaskTile);
    for (uint64_t m = tile_bits; m;) {
      const int hh = (int)__builtin_ctzll(m);
      m &= m - 1;
      head_iter(hh, m ? (int)__builtin_ctzll(m) : -1, KTile());
    }
  }
  if (walk_bits) prefetch(h0 + (int)__builtin_ctzll(walk_bits), kMaskExact);
  for (uint64_t m = walk_bits; m;) {
    const int hh = (int)__builtin_ctzll(m);
    m &= m - 1;
    head_iter(hh, m ? (int)__builtin_ctzll(m) : -1, KElem());
  }
}

template <class E, int Q, int N>
static hipError_t launch_co(const Problem& p, const Workspace& ws, hipStream_t s) {
  if constexpr (ChunkOutputCfg<E, Q, N>::fits) {
    const bool den = p.denom != nullptr;
    const bool opts = p.D != nullptr || p.x_times_dt || p.strict_diag;
    // the normalised output forms its denominator's passed-state term for at
    // most kDenHeads heads at once
    const int HB = heads_per_block(p, den ? kDenHeads : kMaxHeadsPerBlock);
    const unsigned blocks = (unsigned)(p.kmax * (p.H / HB));
    const dim3 grid(blocks), blk(kCoThreads);
    if (den && opts)
      hipLaunchKernelGGL((chunk_output_kernel<E, Q, N, 3>), grid, blk, 0, s, p, ws, HB);
    else if (den)
      hipLaunchKernelGGL((chunk_output_kernel<E, Q, N, 2>), grid, blk, 0, s, p, ws, HB);
    else if (opts)
      hipLaunchKernelGGL((chunk_output_kernel<E, Q, N, 1>), grid, blk, 0, s, p, ws, HB);
    else
      hipLaunchKernelGGL((chunk_output_kernel<E, Q, N, 0>), grid, blk, 0, s, p, ws, HB);
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

bool chunk_output_reads_cb(Dtype dt, int Q, int N) {
#define SSD_CO_CB(QQ, NN)                                                           \
  if (Q == QQ && N == NN)                                                           \
    return dt == Dtype::BF16 ? !ChunkOutputCfg<Bf16, QQ, NN>::kGInline : !ChunkOutputCfg<F32, QQ, NN>::kGInline;
  SSD_CO_CB(64, 16) SSD_CO_CB(64, 32) SSD_CO_CB(64, 64) SSD_CO_CB(64, 128) SSD_CO_CB(64, 256)
  SSD_CO_CB(128, 16) SSD_CO_CB(128, 32) SSD_CO_CB(128, 64) SSD_CO_CB(128, 128) SSD_CO_CB(128, 256)
  SSD_CO_CB(256, 16) SSD_CO_CB(256, 32) SSD_CO_CB(256, 64) SSD_CO_CB(256, 128) SSD_CO_CB(256, 256)
#undef SSD_CO_CB
  return true;
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
