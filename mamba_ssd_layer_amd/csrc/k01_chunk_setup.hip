// k01_chunk_setup.hip -- sequence/chunk tables (K0) and the chunk-local
// log-decay cumsum (K1) of the SSD forward pass.
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba).
//
// K0: from cu_seqlens (or the batched shape) build, on the device, the first
//     chunk slot of each sequence.  Every sequence is cut into ceil(len/Q)
//     chunks of its own, the last one possibly short: [M] §3.7.3 (variable
//     length: no padding, state reset at every boundary) and [M] §3.5 (the
//     block decomposition stays exact for uneven partitions).
// K1: per chunk and head, ell_t = dt_t * A_h and Acs[l] = sum_{k<=l} ell_{t0+k},
//     the chunk-local inclusive cumsum whose pairwise differences are the
//     segment sums of [M] §3.5.4 (exp of the segment sum is the 1-SS mask L of
//     the diagonal block).  Only chunk-local sums are formed, so magnitudes
//     stay <= Q * max|ell| ([M] §3.5.4 warns about long cumsums).  Entries past
//     a short chunk's end repeat its last value (their ell counts as 0).  K1
//     also fills the chunk descriptor (sequence, first token, length) of its slot.
#include "ssd_device.hpp"

namespace ssd {

// ---------------------------------------------------------------- K0 ----
// One workgroup of 1024 threads walks the sequences in tiles of 1024 with a
// block-wide exclusive scan of the per-sequence chunk counts.
__global__ __launch_bounds__(1024) void seq_table_kernel(Problem p, Workspace ws) {
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  const int64_t S = p.nseq;
  for (int64_t base = 0; base < S; base += 1024) {
    const int64_t s = base + tid;
    int64_t start = 0, len = 0;
    if (s < S) {
      if (p.cu == nullptr) {
        start = s * p.seqlen;
        len = p.seqlen;
      } else {
        int64_t lo = p.cu[s], hi = p.cu[s + 1];
        lo = lo < 0 ? 0 : (lo > p.total ? p.total : lo);
        hi = hi < 0 ? 0 : (hi > p.total ? p.total : hi);
        start = lo;
        len = hi > lo ? hi - lo : 0;
      }
      ws.seq_start[s] = start;
      ws.seq_len[s] = len;
    }
    const int32_t cnt = (int32_t)((len + p.Q - 1) / p.Q);
    // block exclusive scan of cnt
    int32_t v = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int32_t o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) wave_tot[wid] = v;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wid; ++w) before += wave_tot[w];
    int32_t tile_tot = 0;
    for (int w = 0; w < 16; ++w) tile_tot += wave_tot[w];
    const int64_t off = (int64_t)carry_s + before + v - cnt;
    if (s < S) ws.seq_off[s] = (int32_t)(off < p.kmax ? off : p.kmax);
    __syncthreads();
    if (tid == 0) carry_s += tile_tot;
    __syncthreads();
  }
  if (tid == 0) {
    const int64_t tot = carry_s;
    ws.seq_off[S] = (int32_t)(tot < p.kmax ? tot : p.kmax);
  }
}

// ---------------------------------------------------------------- K1 ----
// Grid: (kmax, ceil(H / 16)).  Block: 256 threads.  The dt tile (Q tokens x 16
// heads) is staged through LDS with coalesced 64-byte rows; each wave then
// scans 4 heads, Q/64 tokens per lane plus a wave-level scan.
template <int Q>
__global__ __launch_bounds__(kThreads) void chunk_cumsum_kernel(Problem p, Workspace ws) {
  constexpr int HPB = 16;
  constexpr int R = Q / 64;  // tokens per lane
  __shared__ float ell_s[Q * (HPB + 1)];
  __shared__ ChunkDesc cd_s;
  const int tid = threadIdx.x;
  const int64_t k = blockIdx.x;
  const int hb = blockIdx.y;
  const int H = p.H;

  if (tid == 0) {
    // last sequence s with seq_off[s] <= k (sequences with no chunks share an
    // offset with the next one and are skipped by taking the last match)
    ChunkDesc cd;
    cd.seq = -1; cd.len = 0; cd.t0 = 0;
    const int32_t nch = ws.seq_off[p.nseq];
    if (k < nch) {
      int64_t lo = 0, hi = p.nseq;  // seq_off[lo] <= k < seq_off[hi] (seq_off[S] = nch)
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (ws.seq_off[mid] <= k) lo = mid; else hi = mid;
      }
      const int64_t c = k - ws.seq_off[lo];
      const int64_t rem = ws.seq_len[lo] - c * Q;
      cd.seq = (int32_t)lo;
      cd.t0 = ws.seq_start[lo] + c * Q;
      cd.len = (int32_t)(rem < Q ? (rem > 0 ? rem : 0) : Q);
      if (cd.len == 0) cd.seq = -1;
    }
    cd_s = cd;
    if (hb == 0) ws.chunks[k] = cd;
  }
  __syncthreads();
  const ChunkDesc cd = cd_s;
  if (cd.seq < 0) return;
  const int L = cd.len;
  const int h0 = hb * HPB;
  // stage ell = dt * A for Q tokens x HPB heads (0 past the chunk end / head count)
  for (int idx = tid; idx < Q * HPB; idx += kThreads) {
    const int l = idx / HPB, hh = idx % HPB;
    const int h = h0 + hh;
    float v = 0.0f;
    if (l < L && h < H) v = p.dt[(cd.t0 + l) * H + h] * p.A[h];
    ell_s[l * (HPB + 1) + hh] = v;
  }
  __syncthreads();
  const int wid = tid >> 6, lane = tid & 63;
  for (int hh = wid; hh < HPB; hh += kThreads / 64) {
    const int h = h0 + hh;
    if (h >= H) break;
    float run[R];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      acc += ell_s[(lane * R + i) * (HPB + 1) + hh];
      run[i] = acc;
    }
    const float incl = wave_inclusive_sum(acc);
    const float excl = incl - acc;
    float* out = ws.acs + (k * H + h) * Q + lane * R;
#pragma unroll
    for (int i = 0; i < R; ++i) out[i] = excl + run[i];
    if (lane == 63) ws.lam[k * H + h] = incl;
  }
}

hipError_t launch_seq_table(const Problem& p, const Workspace& ws, hipStream_t s) {
  hipLaunchKernelGGL(seq_table_kernel, dim3(1), dim3(1024), 0, s, p, ws);
  return hipGetLastError();
}

hipError_t launch_chunk_cumsum(const Problem& p, const Workspace& ws, hipStream_t s) {
  const dim3 grid((unsigned)p.kmax, (unsigned)((p.H + 15) / 16));
  switch (p.Q) {
    case 64: hipLaunchKernelGGL(chunk_cumsum_kernel<64>, grid, dim3(kThreads), 0, s, p, ws); break;
    case 128: hipLaunchKernelGGL(chunk_cumsum_kernel<128>, grid, dim3(kThreads), 0, s, p, ws); break;
    case 256: hipLaunchKernelGGL(chunk_cumsum_kernel<256>, grid, dim3(kThreads), 0, s, p, ws); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ssd
