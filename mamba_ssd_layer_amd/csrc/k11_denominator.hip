// k11_denominator.hip -- the denominator term of the normalised SSD output.
//
// Pages: [T] / [M] "Incorporating a Normalization (Denominator) Term": the
// denominator of Y = M X is M 1, found by giving X one more column of ones;
// the output is divided by it (with a positive kernel feature map on B and C
// so that it is positive).  That column is an SSM with P = 1 of its own:
//     z_t = a_t z_{t-1} + w_t B_t   (an N-vector per head; w_t = dt_t with the
//                                    dt-scaled input, else 1)
//     d_t = C_t . z_t
// and it takes the same block decomposition ([M] §3.5) as the P columns:
//   chunk states   Zs_c = sum_{l in c} exp(Lam_c - Acs_l) w_l B_l        (zstate_kernel)
//   state passing  Zin_{c+1} = exp(Lam_c) Zin_c + Zs_c
//   output         d_t = sum_{j<=t in c} exp(Acs_t - Acs_j) w_j (C_t . B_j)
//                        + exp(Acs_t) C_t . Zin_c                         (denom_kernel)
// The output kernel then divides y by d before rounding it.
//
// Design (gfx950): both kernels take one workgroup per (chunk, group, block of
// up to 8 (zstate) or 16 (denom) heads of the group).  zstate_kernel is a
// weighted sum of the chunk's B rows on the vector ALU (threads over N, B
// loaded 16 tokens at a time, the heads' weights two 16-byte LDS reads per
// token, partial sums over token ranges added in LDS).  denom_kernel forms each 32x32 tile of C B^T once on the
// matrix cores (lane: token t, registers: 16 tokens j) and applies every head's
// decay weights to it: exp(Acs_t - Acs_j) = exp(Acs_t - a_J) exp(a_J - Acs_j)
// off the diagonal (a_J: Acs at the end of tile J; both factors at most 1, the
// second tabulated per head in LDS), one exp per element on the diagonal.
// The passed-state term is one more MFMA product, Zin (heads as rows) times
// the tile's C rows.  The z states are stored in the element dtype like the
// (P, N) states and the state-passing kernel carries them as N more channels
// per head (1/P more work there, no chain of its own).
#include "ssd_device.hpp"

namespace ssd {

constexpr int kDenThreads = 256;
constexpr int kDenMaxQ = 256;

// workgroup -> (chunk slot k, group g, first head h0, heads nh), HB heads a block
struct DenBlock {
  int64_t k;
  int g, h0, nh;
};
template <int HB>
__device__ __forceinline__ DenBlock den_block(const Problem& p) {
  const int hpg = p.H / p.G;
  const int nhb = (hpg + HB - 1) / HB;
  const int64_t bid = blockIdx.x;
  DenBlock b;
  const int hb = (int)(bid % nhb);
  const int64_t kg = bid / nhb;
  b.g = (int)(kg % p.G);
  b.k = kg / p.G;
  b.h0 = b.g * hpg + hb * HB;
  b.nh = min(HB, hpg - hb * HB);
  return b;
}

template <class E>
__device__ __forceinline__ float ld_el(const void* p, int64_t i) {
  if constexpr (E::kBytes == 2) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}
template <class E>
__device__ __forceinline__ void st_el(void* p, int64_t i, float v) {
  if constexpr (E::kBytes == 2) reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  else reinterpret_cast<float*>(p)[i] = v;
}

constexpr int kZHeads = 8;  // heads per zstate workgroup

template <class E, int N>
__global__ __launch_bounds__(kDenThreads) void zstate_kernel(Problem p, Workspace ws) {
  constexpr int NT = N < kDenThreads ? N : kDenThreads;  // threads per token range
  constexpr int kParts = kDenThreads / NT;                 // token ranges
  constexpr int NPT = N / NT;                              // entries per thread
  constexpr int kB = 16;                                   // tokens loaded together
  __shared__ __align__(16) float w[kDenMaxQ][kZHeads];
  __shared__ float red[kParts > 1 ? kParts : 1][kZHeads][N];
  const int H = p.H, G = p.G, Q = p.Q;
  const DenBlock db = den_block<kZHeads>(p);
  const int64_t k = db.k;
  const ChunkDesc cd = chunk_desc(p, ws, k);
  const int L = cd.len;
  const int tid = threadIdx.x;
  {
    // the weight table: every load first (one round trip), then the exps
    constexpr int kPer = kZHeads * kDenMaxQ / kDenThreads;
    float lamv[kPer], acv[kPer], dtv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kDenThreads;
      const int hh = i % kZHeads, l = i / kZHeads;
      const int h = db.h0 + min(hh, db.nh - 1);
      const int lc = min(l, max(L - 1, 0));
      lamv[u] = ws.lam[k * H + h];
      acv[u] = ws.acs[(k * H + h) * Q + min(l, Q - 1)];
      dtv[u] = p.x_times_dt ? p.dt[(cd.t0 + lc) * H + h] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kDenThreads;
      const int hh = i % kZHeads, l = i / kZHeads;
      w[l][hh] = (hh < db.nh && l < L) ? __expf(lamv[u] - acv[u]) * dtv[u] : 0.0f;
    }
  }
  __syncthreads();
  const int n = tid % NT, part = tid / NT;
  float acc[NPT][kZHeads] = {};
  // token blocks of kB, dealt to the parts in turn; rows past the chunk read
  // its last row and meet weight 0
  auto load_blk = [&](int l0, float (&bv)[kB][NPT]) {
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int64_t row = ((cd.t0 + max(min(l0 + i, L - 1), 0)) * G + db.g) * (int64_t)N;
#pragma unroll
      for (int e = 0; e < NPT; ++e) bv[i][e] = ld_el<E>(p.B, row + n + e * NT);
    }
  };
  float bcur[kB][NPT];
  load_blk(part * kB, bcur);
  for (int l0 = part * kB; l0 < L; l0 += kParts * kB) {
    float bv[kB][NPT];
#pragma unroll
    for (int i = 0; i < kB; ++i)
#pragma unroll
      for (int e = 0; e < NPT; ++e) bv[i][e] = bcur[i][e];
    load_blk(l0 + kParts * kB, bcur);  // the next block, in flight meanwhile
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const float4 w0 = *reinterpret_cast<const float4*>(&w[l0 + i][0]);
      const float4 w1 = *reinterpret_cast<const float4*>(&w[l0 + i][4]);
      const float wq[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < NPT; ++e)
#pragma unroll
        for (int hh = 0; hh < kZHeads; ++hh) acc[e][hh] += wq[hh] * bv[i][e];
    }
  }
  if constexpr (kParts > 1) {
#pragma unroll
    for (int hh = 0; hh < kZHeads; ++hh) red[part][hh][n] = acc[0][hh];
    __syncthreads();
    for (int i = tid; i < kZHeads * N; i += kDenThreads) {
      const int hh = i / N, nn = i % N;
      float sum = 0.0f;
#pragma unroll
      for (int q = 0; q < kParts; ++q) sum += red[q][hh][nn];
      if (hh < db.nh) st_el<E>(ws.zs, (k * H + db.h0 + hh) * (int64_t)N + nn, sum);
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < kZHeads; ++hh)
      if (hh < db.nh)
#pragma unroll
        for (int e = 0; e < NPT; ++e) st_el<E>(ws.zs, (k * H + db.h0 + hh) * (int64_t)N + n + e * NT, acc[e][hh]);
  }
}

// 32x32 tile D[m][n] = sum_k A_m[k] B_n[k] with A's and B's rows read from
// memory (lane: m = n = lr; acc[r] holds m = 8 (r / 4) + 4 lg + r % 4).
template <class E, int K>
__device__ __forceinline__ floatx16_t row_prod(const typename E::storage* arow, const typename E::storage* brow,
                                               int lg) {
  floatx16_t acc = zero16();
  if constexpr (E::kBytes == 2) {
#pragma unroll
    for (int s = 0; s < K / 16; ++s)
      acc = mfma32x32x16(*reinterpret_cast<const uint4*>(arow + 16 * s + 8 * lg),
                         *reinterpret_cast<const uint4*>(brow + 16 * s + 8 * lg), acc);
  } else {
#pragma unroll
    for (int s = 0; s < K / 2; ++s) acc = mfma32x32x2(arow[2 * s + lg], brow[2 * s + lg], acc);
  }
  return acc;
}

constexpr int kDenHeads = 8;  // heads per denom workgroup

// One operand row per lane (bf16: the lane's 8-value slices of the row).
template <int N>
struct RowRegs {
  uint4 v[N / 16];
};
template <int N>
__device__ __forceinline__ void load_row(RowRegs<N>& r, const uint16_t* row, int lg) {
#pragma unroll
  for (int s = 0; s < N / 16; ++s) r.v[s] = *reinterpret_cast<const uint4*>(row + 16 * s + 8 * lg);
}
template <int N>
__device__ __forceinline__ floatx16_t reg_prod(const RowRegs<N>& a, const RowRegs<N>& b) {
  floatx16_t acc = zero16();
#pragma unroll
  for (int s = 0; s < N / 16; ++s) acc = mfma32x32x16(a.v[s], b.v[s], acc);
  return acc;
}

template <class E, int N>
__global__ __launch_bounds__(kDenThreads) void denom_kernel(Problem p, Workspace ws) {
  using T = typename E::storage;
  __shared__ __align__(16) float acsT[kDenHeads][kDenMaxQ];
  __shared__ __align__(16) float fd[kDenHeads][kDenMaxQ];  // exp(a_J - Acs_j) w_j, 0 past the chunk
  __shared__ __align__(16) float wv[kDenHeads][kDenMaxQ];  // w_j, 0 past the chunk
  const int H = p.H, G = p.G, Q = p.Q;
  const DenBlock db = den_block<kDenHeads>(p);
  const int64_t k = db.k;
  const ChunkDesc cd = chunk_desc(p, ws, k);
  const int L = cd.len;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  {
    // the tables: every load first (one round trip), then the exps
    constexpr int kPer = kDenHeads * kDenMaxQ / kDenThreads;
    float av[kPer], aev[kPer], dv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kDenThreads;
      const int hh = i / kDenMaxQ, j = min(i % kDenMaxQ, Q - 1);
      const float* ac = ws.acs + (k * H + db.h0 + min(hh, db.nh - 1)) * Q;
      av[u] = ac[j];
      aev[u] = ac[32 * (j / 32) + 31];
      dv[u] = p.x_times_dt ? p.dt[(cd.t0 + max(min(j, L - 1), 0)) * H + db.h0 + min(hh, db.nh - 1)] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kDenThreads;
      const int hh = i / kDenMaxQ, j = i % kDenMaxQ;
      if (j < Q) {
        const bool in = hh < db.nh && j < L;
        const float wj = in ? dv[u] : 0.0f;
        acsT[hh][j] = hh < db.nh ? av[u] : 0.0f;
        wv[hh][j] = wj;
        fd[hh][j] = in ? __expf(aev[u] - av[u]) * wj : 0.0f;
      }
    }
  }
  __syncthreads();
  const int NI = Q / 32, nI = (L + 31) / 32;
  const T* Bg = reinterpret_cast<const T*>(p.B) + db.g * N;
  const T* Cg = reinterpret_cast<const T*>(p.C) + db.g * N;
  const int64_t ts = (int64_t)G * N;  // token stride of B and C
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // row tiles of this wave: {w, NI-1-w} with 8 of them (equal work), else {w}
    const int I = NI == 8 ? (u == 0 ? wid : NI - 1 - wid) : (u == 0 && wid < NI ? wid : -1);
    if (I < 0 || I >= nI) continue;
    const int t_l = 32 * I + lr;  // this lane's token (chunk-local)
    const T* crow = Cg + (cd.t0 + min(t_l, L - 1)) * ts;
    float rs[kDenHeads] = {};
    // bf16: the tile's C rows in registers and the next tile's B rows loaded
    // while this one is used
    RowRegs<N> cr, bcur;
    if constexpr (E::kBytes == 2) {
      load_row(cr, reinterpret_cast<const uint16_t*>(crow), lg);
      load_row(bcur, reinterpret_cast<const uint16_t*>(Bg + (cd.t0 + min(lr, L - 1)) * ts), lg);
    }
    for (int J = 0; J <= I; ++J) {
      const T* brow = Bg + (cd.t0 + min(32 * J + lr, L - 1)) * ts;
      // lane holds token t (n), value r holds token j = 32 J + m(r) (m)
      floatx16_t gt;
      if constexpr (E::kBytes == 2) {
        RowRegs<N> bnext;
        load_row(bnext, reinterpret_cast<const uint16_t*>(Bg + (cd.t0 + min(32 * min(J + 1, I) + lr, L - 1)) * ts),
                 lg);
        gt = reg_prod(bcur, cr);
        bcur = bnext;
      } else {
        gt = row_prod<E, N>(brow, crow, lg);
      }
      if (J < I) {
#pragma unroll
        for (int hh = 0; hh < kDenHeads; ++hh) {
          const float e = __expf(acsT[hh][t_l] - acsT[hh][32 * J + 31]);
          float sum = 0.0f;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float4 f4 = *reinterpret_cast<const float4*>(&fd[hh][32 * J + 8 * a + 4 * lg]);
            sum += f4.x * gt[4 * a] + f4.y * gt[4 * a + 1] + f4.z * gt[4 * a + 2] + f4.w * gt[4 * a + 3];
          }
          rs[hh] += e * sum;
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < kDenHeads; ++hh) {
          const float at = acsT[hh][t_l];
          float sum = 0.0f;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int m0 = 8 * a + 4 * lg;
            const float4 a4 = *reinterpret_cast<const float4*>(&acsT[hh][32 * J + m0]);
            const float4 w4 = *reinterpret_cast<const float4*>(&wv[hh][32 * J + m0]);
            const float aq[4] = {a4.x, a4.y, a4.z, a4.w}, wq[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (m0 + q <= lr) sum += __expf(at - aq[q]) * wq[q] * gt[4 * a + q];
          }
          rs[hh] += sum;
        }
      }
    }
    // passed-state term: rows = heads (lanes past the block repeat its last
    // head, never stored), columns = this tile's tokens
    const T* zrow = reinterpret_cast<const T*>(ws.zin) + (k * H + db.h0 + min(lr, db.nh - 1)) * (int64_t)N;
    floatx16_t zd;  // lane: token; r: head 8(r/4)+4lg+r%4
    if constexpr (E::kBytes == 2) {
      RowRegs<N> zr;
      load_row(zr, reinterpret_cast<const uint16_t*>(zrow), lg);
      zd = reg_prod(zr, cr);
    } else {
      zd = row_prod<E, N>(zrow, crow, lg);
    }
#pragma unroll
    for (int hh = 0; hh < kDenHeads; ++hh) {
      const float tot = rs[hh] + __shfl_xor(rs[hh], 32);
      const int rr = 4 * (hh >> 3) + (hh & 3);
      const float zv = ((hh >> 2) & 1) == lg ? zd[rr] : 0.0f;
      const float zsum = zv + __shfl_xor(zv, 32);
      if (lg == 0 && t_l < L && hh < db.nh)
        p.denom[(cd.t0 + t_l) * H + db.h0 + hh] = tot + __expf(acsT[hh][t_l]) * zsum;
    }
  }
}

#define SSD_DEN_SWITCH(KERNEL, HB)                                                            \
  const int hpg = p.H / p.G;                                                                   \
  const int64_t blocks = p.kmax * p.G * ((hpg + HB - 1) / HB);                                 \
  if (blocks == 0) return hipSuccess;                                                          \
  const dim3 grid((unsigned)blocks), block(kDenThreads);                                       \
  const bool bf = p.dtype == Dtype::BF16;                                                      \
  switch (p.N) {                                                                               \
    case 16: if (bf) hipLaunchKernelGGL((KERNEL<Bf16, 16>), grid, block, 0, s, p, ws);         \
             else hipLaunchKernelGGL((KERNEL<F32, 16>), grid, block, 0, s, p, ws); break;      \
    case 32: if (bf) hipLaunchKernelGGL((KERNEL<Bf16, 32>), grid, block, 0, s, p, ws);         \
             else hipLaunchKernelGGL((KERNEL<F32, 32>), grid, block, 0, s, p, ws); break;      \
    case 64: if (bf) hipLaunchKernelGGL((KERNEL<Bf16, 64>), grid, block, 0, s, p, ws);         \
             else hipLaunchKernelGGL((KERNEL<F32, 64>), grid, block, 0, s, p, ws); break;      \
    case 128: if (bf) hipLaunchKernelGGL((KERNEL<Bf16, 128>), grid, block, 0, s, p, ws);       \
              else hipLaunchKernelGGL((KERNEL<F32, 128>), grid, block, 0, s, p, ws); break;    \
    case 256: if (bf) hipLaunchKernelGGL((KERNEL<Bf16, 256>), grid, block, 0, s, p, ws);       \
              else hipLaunchKernelGGL((KERNEL<F32, 256>), grid, block, 0, s, p, ws); break;    \
    default: return hipErrorInvalidValue;                                                      \
  }                                                                                            \
  return hipGetLastError();

hipError_t launch_zstate(const Problem& p, const Workspace& ws, hipStream_t s) {
  SSD_DEN_SWITCH(zstate_kernel, kZHeads)
}

hipError_t launch_denominator(const Problem& p, const Workspace& ws, hipStream_t s) {
  SSD_DEN_SWITCH(denom_kernel, kDenHeads)
}

#undef SSD_DEN_SWITCH

}  // namespace ssd
