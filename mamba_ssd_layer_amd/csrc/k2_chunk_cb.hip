// k2_chunk_cb.hip -- the kernel matrix of each chunk's diagonal block, G = C B^T
// (first half of K2).
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba), §3.5.1
// (diagonal blocks in the quadratic form) and §3.5.3 "Center blocks": the
// kernel matrix C^T B of a chunk costs BMM(T/Q, Q, Q, N) and is shared by every
// head that reads the same B and C; only the mask L (and X) differ per head.
// [T] "Transformers是SSMs…(一)" (nxbn.cn) §2.4: (L o Q K^T) V with
// (Q, K, V) = (C, B, X).
//
// Design (gfx950): one wave per causal 32x32 tile (I, J <= I) of each (chunk,
// B/C group): G^T = B_J C_I^T on v_mfma_f32_32x32x16_bf16 (_32x32x2_f32 on the
// fp32 path).  Both operands are loaded straight from global memory into the
// MFMA register layout, all loads of a wave issued at once (no LDS, a single
// memory latency per wave); there are many more waves than CUs.  A tile is
// stored as the accumulator lies in the registers: lane l's 16 values as 16-byte
// vectors, vector-major and lane after lane within a vector, so the output
// kernel copies a tile with fully coalesced loads and reads it back (from LDS)
// straight into the register layout its masked product needs.  The wave of tile
// (I, 0) also stores the C rows of row tile I as MFMA operand slices in the same
// lane-after-lane order (a straight C row load touches 32 rows per
// instruction; this copy is read back 1 KB-contiguous per instruction).  Tiles are in the element dtype (bf16: rounded to
// nearest even), numbered I(I+1)/2 + J per (chunk, group).
#include "ssd_device.hpp"

namespace ssd {

template <class E, int Q, int N>
__global__ __launch_bounds__(kThreads) void chunk_cb_kernel(Problem p, Workspace ws) {
  using T = typename E::storage;
  constexpr bool kBf16 = E::kBytes == 2;
  constexpr int KS = N / E::kMfmaK;
  constexpr int NI = Q / 32;
  constexpr int NTILE = NI * (NI + 1) / 2;
  using CReg = typename std::conditional<kBf16, uint4, float>::type;

  const int G = p.G;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tile_id = (int64_t)blockIdx.x * (kThreads / 64) + wid;
  const int ti = (int)(tile_id % NTILE);
  const int64_t kg = tile_id / NTILE;
  if (kg >= p.kmax * G) return;
  const int64_t k = kg / G;
  const int g = (int)(kg % G);
  int I = 0;
  while ((I + 1) * (I + 2) / 2 <= ti) ++I;
  const int J = ti - I * (I + 1) / 2;
  const ChunkDesc cd = chunk_desc(p, ws, k);
  if (cd.seq < 0) return;
  const int L = cd.len;
  const int nI = (L + 31) / 32;
  if (I >= nI) return;  // rows past the chunk end are never read
  const int lr = lane & 31, lg = lane >> 5;
  const T* bg = reinterpret_cast<const T*>(p.B) + (cd.t0 * G + g) * N;
  const T* cg = reinterpret_cast<const T*>(p.C) + (cd.t0 * G + g) * N;

  auto load_rows = [&](const T* base, int row, CReg (&r)[KS]) {
    const bool ok = row < L;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (kBf16)
        r[ks] = ok ? *reinterpret_cast<const uint4*>(base + (int64_t)row * G * N + ks * 16 + lg * 8)
                   : make_uint4(0, 0, 0, 0);
      else
        r[ks] = ok ? base[(int64_t)row * G * N + ks * 2 + lg] : 0.0f;
    }
  };
  CReg creg[KS], breg[KS];
  load_rows(cg, I * 32 + lr, creg);
  load_rows(bg, J * 32 + lr, breg);
  if (J == 0) {
    // the C rows of row tile I in the same lane layout, for the output kernel
    CReg* cop = reinterpret_cast<CReg*>(ws.cop) + ((kg * NI + I) * KS) * 64 + lane;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cop[ks * 64] = creg[ks];
  }
  floatx16_t acc = zero16();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (kBf16)
      acc = mfma32x32x16(breg[ks], creg[ks], acc);
    else
      acc = mfma32x32x2(breg[ks], creg[ks], acc);
  }
  // acc[r] = G[32I + lr][32J + 8(r/4) + 4 lg + r%4]; the lane's values leave as
  // 16-byte vectors q, stored [tile][q][lane]
  constexpr int GV = kBf16 ? 2 : 4;
  uint4* tile = reinterpret_cast<uint4*>(ws.cb) + (kg * NTILE + ti) * (int64_t)(GV * 64) + lane;
  if constexpr (kBf16) {
    uint4 o0, o1;
    o0.x = pack_bf16x2(acc[0], acc[1]);   o0.y = pack_bf16x2(acc[2], acc[3]);
    o0.z = pack_bf16x2(acc[4], acc[5]);   o0.w = pack_bf16x2(acc[6], acc[7]);
    o1.x = pack_bf16x2(acc[8], acc[9]);   o1.y = pack_bf16x2(acc[10], acc[11]);
    o1.z = pack_bf16x2(acc[12], acc[13]); o1.w = pack_bf16x2(acc[14], acc[15]);
    tile[0] = o0;
    tile[64] = o1;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<float4*>(tile)[q * 64] =
          make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  }
}

template <class E, int Q, int N>
static hipError_t launch_cb(const Problem& p, const Workspace& ws, hipStream_t s) {
  constexpr int NI = Q / 32, NTILE = NI * (NI + 1) / 2, WPB = kThreads / 64;
  const unsigned blocks = (unsigned)((p.kmax * p.G * NTILE + WPB - 1) / WPB);
  hipLaunchKernelGGL((chunk_cb_kernel<E, Q, N>), dim3(blocks), dim3(kThreads), 0, s, p, ws);
  return hipGetLastError();
}

template <class E, int Q>
static hipError_t launch_cb_n(const Problem& p, const Workspace& ws, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_cb<E, Q, 16>(p, ws, s);
    case 32: return launch_cb<E, Q, 32>(p, ws, s);
    case 64: return launch_cb<E, Q, 64>(p, ws, s);
    case 128: return launch_cb<E, Q, 128>(p, ws, s);
    case 256: return launch_cb<E, Q, 256>(p, ws, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_cb(const Problem& p, const Workspace& ws, hipStream_t s) {
  if (p.kmax == 0) return hipSuccess;
  switch (p.Q) {
    case 64: return p.dtype == Dtype::BF16 ? launch_cb_n<Bf16, 64>(p, ws, s) : launch_cb_n<F32, 64>(p, ws, s);
    case 128: return p.dtype == Dtype::BF16 ? launch_cb_n<Bf16, 128>(p, ws, s) : launch_cb_n<F32, 128>(p, ws, s);
    case 256: return p.dtype == Dtype::BF16 ? launch_cb_n<Bf16, 256>(p, ws, s) : launch_cb_n<F32, 256>(p, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
