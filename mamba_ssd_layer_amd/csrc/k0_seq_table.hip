// k0_seq_table.hip -- sequence table of a variable-length batch (K0).
//
// Pages: [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba), §3.7.3
// (variable length: the batch is one packed sequence, no padding, the state
// reset at every boundary) and §3.5 (the block decomposition stays exact for
// uneven partitions).  Every sequence is cut into ceil(len/Q) chunks of its
// own, the last one possibly short.  From cu_seqlens, on the device (no host
// copy), this kernel writes each sequence's first token, length and first
// chunk slot; the chunk-state kernel turns a slot into (sequence, first token,
// length) by a binary search over these offsets.  Invalid cu_seqlens are
// clamped so that every later access stays inside the buffers: starts and ends
// to [0, Ttot], negative lengths to 0, chunk offsets to the slot count.
// Batched problems need no table (slots map to chunks arithmetically).
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

hipError_t launch_seq_table(const Problem& p, const Workspace& ws, hipStream_t s) {
  hipLaunchKernelGGL(seq_table_kernel, dim3(1), dim3(1024), 0, s, p, ws);
  return hipGetLastError();
}

}  // namespace ssd
