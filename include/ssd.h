/*
 * ssd.h -- C ABI of libssd.so: the forward pass of the SSD (state space
 * duality) layer of Mamba-2 on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as published):
 *   [T] "Transformers是SSMs：通过结构化状态空间对偶性的广义模型和高效算法(一)"
 *       (nxbn.cn/automobile/1783.html): sections 1-5 of "Transformers are SSMs".
 *   [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba).
 *
 * The operation ([T] §2.4 recurrent form and §5.1; [M] §3.1.2): for every
 * sequence and head h, with a_t = exp(dt_t * A_h),
 *     h_t = a_t * h_{t-1} + x_t (outer) B_t       (state (P, N), zero before
 *                                                   the first token unless
 *                                                   ssd_chunked_fwd_ex is
 *                                                   given an initial state)
 *     y_t = h_t . C_t                              (P values)
 * computed exactly (up to rounding) by the chunked block decomposition of the
 * 1-semiseparable matrix M = L o (C B^T) of [M] §3.5: diagonal blocks in the
 * quadratic (attention-like) form, chunk states, a scan that passes states
 * between chunks, and a state-to-output product.  Head h reads B/C group
 * g = h * G / H (G divides H; [M] §3.6.2 grouped heads).  The first token's
 * a_t of every sequence multiplies the state before it: zero (no effect)
 * unless an initial state is given.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *     and dense.  x, B, C, y and final_state must be 16-byte aligned; dt,
 *     A_head and cu_seqlens 4-byte aligned.  y must not alias an input.
 *   - Element dtype (x, B, C, y): SSD_DTYPE_F32 or SSD_DTYPE_BF16.  dt, A_head
 *     and final_state are always fp32.  Accumulation is fp32; on the bf16 path
 *     the matrix-core operands (masked C B^T tiles, passed states) are rounded
 *     to bf16, y is rounded to bf16 by round-to-nearest-even.
 *   - dt * A_h <= 0 is expected (a_t in (0, 1], [T] §2.4); inputs must be
 *     finite, else results are undefined.
 *   - Supported shapes: headdim P = 64; dstate N in {16, 32, 64, 128, 256};
 *     chunk_len Q in {64, 128, 256}; every (dtype, Q, N) of these is built
 *     (ssd_config_supported tells).  Any sequence length >= 0; a partial last
 *     chunk is handled.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation failure nothing is written and no HIP call is made.
 *   - Execution is asynchronous on `stream` (a hipStream_t, NULL = default
 *     stream) with no host synchronisation.  Errors of kernels that already
 *     ran surface at the caller's next synchronisation, as for any stream work.
 *   - Workspace (every entry point but ssd_chunked_fwd_noalloc): one device
 *     allocation per (device, stream), taken with
 *     hipMallocAsync from the device's default memory pool on first use, grown
 *     (stream-ordered free and allocation) when a larger problem arrives, and
 *     otherwise reused by every later call on that stream; it is kept until
 *     the process ends.  Stream order keeps calls on one stream apart; calls on
 *     different streams use different workspaces.  Do not destroy a stream
 *     while this library's work is pending on it and then reuse its handle
 *     for a new stream before that work has finished.
 *   - Thread-safe: the workspace table, the per-device address of the
 *     no-allocation entry point's scratch and the optional kernel timing
 *     below are the only host-side global state, each guarded by a lock (the
 *     scratch array itself is shared on the device: see
 *     ssd_chunked_fwd_noalloc).
 *   - Return value: SSD_OK or an error code; nothing is thrown or aborted.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, H % G != 0 */
  SSD_ERR_UNSUPPORTED = 2,      /* shape/dtype outside the built set, or not a gfx950 device */
  SSD_ERR_HIP = 3,              /* a HIP runtime call or kernel launch failed */
  SSD_ERR_OUT_OF_MEMORY = 4,    /* workspace allocation failed */
  SSD_ERR_SCRATCH_LIMIT = 5     /* ssd_chunked_fwd_noalloc: the workspace exceeds its static scratch */
} ssd_status;

typedef enum ssd_dtype { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype;

/*
 * Batched forward: `batch` sequences of `seqlen` tokens each.
 *   x           (batch, seqlen, nheads, headdim)  element dtype
 *   dt          (batch, seqlen, nheads)           fp32, step sizes
 *   A_head      (nheads)                          fp32, a_t = exp(dt * A_head)
 *   B, C        (batch, seqlen, ngroups, dstate)  element dtype
 *   chunk_len   Q of the block decomposition ([M] §3.5: Q x Q blocks of M)
 *   y           (batch, seqlen, nheads, headdim)  element dtype, overwritten
 *   final_state (batch, nheads, headdim, dstate)  fp32, state after the last
 *               token ([M] §3.5.2 center factors; listing's bchpn order), or
 *               NULL to skip.  seqlen == 0 gives a zero final state.
 */
ssd_status ssd_chunked_fwd(const void* x, const float* dt, const float* A_head,
                           const void* B, const void* C, int64_t batch, int64_t seqlen,
                           int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                           int32_t chunk_len, ssd_dtype dtype, void* y, float* final_state,
                           void* stream);

/*
 * ssd_chunked_fwd without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Arguments, results and kernels are those of
 * ssd_chunked_fwd (the caller passes every input and output); the workspace
 * (chunk cumsums, chunk states, passed states) lives in a static device array
 * of SSD_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends, in place of the per-stream cached allocation.
 * The call makes no hipMalloc, hipFree or other allocating call.
 *   - A problem whose workspace exceeds the array returns
 *     SSD_ERR_SCRATCH_LIMIT, checked on the host before any HIP call (at
 *     nheads 32, dstate 128, bf16, chunk_len 256 the limit is about 28K
 *     tokens; the workspace grows with tokens x nheads x dstate).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (on different streams, or from several host threads)
 *     race on it and give undefined results; issue them on one stream.  The
 *     array keeps the last call's contents; nothing in it needs clearing.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((int64_t)128 << 20)
ssd_status ssd_chunked_fwd_noalloc(const void* x, const float* dt, const float* A_head,
                                   const void* B, const void* C, int64_t batch, int64_t seqlen,
                                   int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                   int32_t chunk_len, ssd_dtype dtype, void* y, float* final_state,
                                   void* stream);

/*
 * Variable-length forward ([M] §3.7.3: the batch is one packed sequence with
 * the state reset at every boundary, no padding).
 *   x           (total_len, nheads, headdim)
 *   dt          (total_len, nheads)
 *   B, C        (total_len, ngroups, dstate)
 *   cu_seqlens  (nseqs + 1) int32 DEVICE array: cu[0] = 0, non-decreasing,
 *               cu[nseqs] = total_len.  Sequence s is tokens [cu[s], cu[s+1]);
 *               it starts from a zero state.  Read on the device only (no
 *               host copy).  Invalid contents give unspecified y but every
 *               access stays inside the buffers sized above.
 *   y           (total_len, nheads, headdim)
 *   final_state (nseqs, nheads, headdim, dstate) fp32 or NULL; an empty
 *               sequence gets a zero state.
 */
ssd_status ssd_chunked_fwd_varlen(const void* x, const float* dt, const float* A_head,
                                  const void* B, const void* C, const int32_t* cu_seqlens,
                                  int64_t nseqs, int64_t total_len, int32_t nheads,
                                  int32_t headdim, int32_t dstate, int32_t ngroups,
                                  int32_t chunk_len, ssd_dtype dtype, void* y,
                                  float* final_state, void* stream);

/*
 * Forward from given initial states, batched or packed ([M] §3.7.2 "Sequence
 * Parallelism": a worker starts from the state its predecessor hands over and
 * passes its final state on; the §3.5 listing's optional initial state, put
 * in front of the chunk states before they are passed).  Splitting a sequence
 * at any token and running the second part from the first part's final state
 * gives the whole sequence's y and final state (up to rounding).
 *   cu_seqlens     NULL: batched form, nseqs sequences of total_len / nseqs
 *                  tokens each (total_len a multiple of nseqs; x (nseqs, T, H,
 *                  P) ... as for ssd_chunked_fwd).  Otherwise as for
 *                  ssd_chunked_fwd_varlen.
 *   initial_state  (nseqs, nheads, headdim, dstate) fp32 DEVICE array,
 *                  16-byte aligned: h_{-1} of each sequence, the state the
 *                  first token's a_t multiplies; NULL means zero (then the
 *                  call equals ssd_chunked_fwd / ssd_chunked_fwd_varlen).  It
 *                  is read, never written, and may be the final_state buffer
 *                  of an earlier call; it must not alias this call's
 *                  final_state.  An empty sequence's final state is its
 *                  initial state.
 *   D              (nheads) fp32 DEVICE array or NULL: adds the skip term
 *                  y_t += D_h x_t on the raw input ([M] §1.2: D passes the
 *                  input straight to the output, a skip connection; the SSM
 *                  proper is usually written without it).  On the bf16 path
 *                  it is added to the rounded SSM output, then rounded again.
 *   x_times_dt     0 or 1.  1: the input enters the state as dt_t x_t, i.e.
 *                  B_t is scaled by the step size (the first-order
 *                  discretisation that Mamba-2 keeps from Mamba, [M]
 *                  "离散化" after §3.5.4): h_t = a_t h_{t-1} + dt_t x_t B_t^T.
 *                  D still multiplies the raw x.
 * Other arguments, errors and execution as for the entry points above.
 */
ssd_status ssd_chunked_fwd_ex(const void* x, const float* dt, const float* A_head,
                              const void* B, const void* C, const int32_t* cu_seqlens,
                              int64_t nseqs, int64_t total_len, int32_t nheads,
                              int32_t headdim, int32_t dstate, int32_t ngroups,
                              int32_t chunk_len, ssd_dtype dtype, const float* initial_state,
                              const float* D, int32_t x_times_dt, void* y,
                              float* final_state, void* stream);

/*
 * Backward pass of ssd_chunked_fwd_ex: the gradients of a loss L given
 * dy = dL/dy and, optionally, dfinal = dL/d(final state).  The gradients of
 * the recurrence (chain rule in reverse token order; pages: the training
 * direction [M] §3.5.3 prices, the same block decomposition of [M] §3.5):
 *     G_t  = dy_t C_t^T + a_{t+1} G_{t+1}    (dL/dh_t; dfinal past the end)
 *     dx_t = (dt_t if x_times_dt) G_t B_t + D_h dy_t
 *     dB_t = sum over the group's heads of G_t^T x'_t,  dC_t = ... of h_t^T dy_t
 *     d(dt_t), dA_h through a_t = exp(dt_t A_h) (and dt_t x_t with x_times_dt)
 *     dD_h = sum_t x_t . dy_t,  d(initial state) = a_first G_first
 * where x' is the input as the state sees it (dt x with x_times_dt).
 * Inputs as for ssd_chunked_fwd_ex (initial_state, D nullable; x_times_dt 0/1).
 *   dy               (total_len, nheads, headdim) element dtype
 *   dfinal_state     (nseqs, nheads, headdim, dstate) fp32 or NULL (zero)
 * Outputs (caller-owned, overwritten):
 *   dx               like x            dB, dC   like B, C (element dtype)
 *   ddt              like dt (fp32)    dA       (nheads) fp32, required
 *   dD               (nheads) fp32 or NULL (skip)
 *   dinitial_state   (nseqs, nheads, headdim, dstate) fp32 or NULL (skip)
 * dA and dD are sums over all tokens formed with atomic additions: their last
 * bits may differ between runs.  Implementation: passes of the forward
 * kernels on rearranged inputs (the forward's passed states; the sequence
 * reversed in time with the decays shifted by one token, for dx and the
 * adjoint states), then, for bf16 inputs whose sequences are whole numbers
 * of chunks, per-chunk kernels for dB, dC, dx and d(dt) (packed bf16
 * sequences are padded on the device to whole chunks for this, when that at
 * most doubles the tokens: up to total_len + nseqs (chunk_len - 1) padded
 * tokens of workspace); otherwise fp32 passes and role-exchanged passes (the
 * roles of x and B exchanged for dB and dC).  It needs a second per-stream
 * workspace of a few x-sized arrays (about 12 on the fp32 route).  headdim
 * 64; every (dtype, dstate, chunk_len) the forward supports, provided
 * (dtype, 64, Q) is built for some Q.  Alignment, validation, execution and
 * errors as for the forward.
 */
ssd_status ssd_chunked_bwd(const void* x, const float* dt, const float* A_head, const void* B,
                           const void* C, const int32_t* cu_seqlens, int64_t nseqs,
                           int64_t total_len, int32_t nheads, int32_t headdim, int32_t dstate,
                           int32_t ngroups, int32_t chunk_len, ssd_dtype dtype,
                           const float* initial_state, const float* D, int32_t x_times_dt,
                           const void* dy, const float* dfinal_state, void* dx, float* ddt,
                           float* dA, void* dB, void* dC, float* dD, float* dinitial_state,
                           void* stream);

/*
 * One recurrent step for a batch of sequences: the decode (autoregressive
 * inference) mode ([T] §2.1: inference runs the recurrent form one input step
 * at a time with a constant-size state; [M] §3.5.3 cost table: N^2 FLOPs per
 * step).  For every sequence b and head h, a = exp(dt[b,h] * A_head[h]) and g
 * the head's group:
 *     state[b,h] <- a * state[b,h] + x[b,h,:] (outer) B[b,g,:]
 *     y[b,h,p]   <- sum_n state[b,h,p,n] * C[b,g,n]
 * i.e. one more token of the forward pass: the final_state of a forward call
 * continues here, and T steps equal a forward over those T tokens started
 * from the same state (up to rounding).
 *   x      (batch, nheads, headdim)          element dtype (one token each)
 *   dt     (batch, nheads)                   fp32
 *   A_head (nheads)                          fp32
 *   B, C   (batch, ngroups, dstate)          element dtype
 *   state  (batch, nheads, headdim, dstate)  fp32, read and overwritten in
 *          place (the forward's final_state layout)
 *   y      (batch, nheads, headdim)          element dtype, overwritten
 *          (bf16: rounded to nearest even); must not alias an input
 *   D, x_times_dt  as for ssd_chunked_fwd_ex (skip term, input as dt x)
 * headdim 64, dstate in {16, 32, 64, 128, 256}; no workspace.  Alignment,
 * validation, execution and errors as for the forward.  batch == 0 is a
 * no-op.
 */
ssd_status ssd_decode_step(const void* x, const float* dt, const float* A_head, const void* B,
                           const void* C, int64_t batch, int32_t nheads, int32_t headdim,
                           int32_t dstate, int32_t ngroups, ssd_dtype dtype, const float* D,
                           int32_t x_times_dt, float* state, void* y, void* stream);

/*
 * The forward pass with the output normalised by its denominator term ([T] /
 * [M] "Incorporating a Normalization (Denominator) Term": the denominator of
 * Y = M X is M 1, the output of one more input column of ones).  With X~ =
 * [X, 1] run through the layer (the ones column dt-scaled too when
 * x_times_dt is set, from a zero state in every sequence):
 *     denom[t,h] = (M 1)[t,h]        y[t,h,:] = (M X)[t,h,:] / denom[t,h] + D_h x[t,h,:]
 * The pages ask for a positive kernel feature map on B and C so that the
 * denominators are positive; the library does not check it (a zero
 * denominator gives inf or nan in y).  Arguments as ssd_chunked_fwd_ex
 * without an initial state, plus
 *   denom  (total_len, nheads) fp32, written; required when total_len > 0.
 * final_state is the state of the P columns of x, as in the plain forward.
 */
ssd_status ssd_chunked_fwd_normalized(const void* x, const float* dt, const float* A_head, const void* B,
                                      const void* C, const int32_t* cu_seqlens, int64_t nseqs,
                                      int64_t total_len, int32_t nheads, int32_t headdim, int32_t dstate,
                                      int32_t ngroups, int32_t chunk_len, ssd_dtype dtype, const float* D,
                                      int32_t x_times_dt, void* y, float* final_state, float* denom,
                                      void* stream);

/*
 * The comparator of the SSD layer: a selective scan with a diagonal
 * transition (Mamba-1's S6; [M] §3.1.1: a diagonal transition stored as its N
 * entries, of which SSD keeps one scalar, §3.1.2; §2.1.2-2.1.3: one SSM per
 * channel, step size per token and channel, B and C per token).  For every
 * sequence b, channel d and state entry n, from a zero state:
 *     h[n] <- exp(delta[b,d,t] * A[d,n]) h[n] + delta[b,d,t] x[b,d,t] B[b,t,n]
 *     y[b,d,t] = sum_n C[b,t,n] h[n]
 * It is not part of the SSD path: it exists to time the pages' speed claim
 * for SSD against this scan on the same GPU.
 *   x, y   (batch, channels, seqlen)  element dtype, channel-major; y is
 *          overwritten (bf16: rounded to nearest even) and must not alias
 *   delta  (batch, channels, seqlen)  fp32
 *   A      (channels, dstate)         fp32
 *   B, C   (batch, seqlen, dstate)    element dtype
 *   final_state (batch, channels, dstate) fp32, or NULL to skip
 * dstate in {64, 128, 256}, any channels >= 1 and seqlen >= 0; pointers
 * aligned to their element size.  Validation, execution and errors as for the
 * forward; no workspace.  batch == 0 is a no-op.
 */
ssd_status ssd_selective_scan(const void* x, const float* delta, const float* A, const void* B,
                              const void* C, int64_t batch, int64_t seqlen, int32_t channels,
                              int32_t dstate, ssd_dtype dtype, void* y, float* final_state,
                              void* stream);

/*
 * The same pass, also copying the intermediates of the block decomposition
 * ([M] §3.5.2 "SSD algorithm: chunking and state passing") into caller
 * buffers, for checking each kernel on its own.  cu_seqlens == NULL selects
 * the batched form (nseqs sequences of total_len / nseqs tokens).  Chunks are
 * numbered in packed order, ceil(len_s / Q) per sequence; K_slots =
 * ssd_chunk_slots(...).  Each output may be NULL.
 *   acs    (K_slots, nheads, Q)  fp32: chunk-local inclusive cumsum of dt*A
 *          (entries past a partial chunk's end repeat its last value)
 *   states (K_slots, nheads, headdim, dstate) fp32: chunk state from a zero
 *          initial state ([M] §3.5.2 right factors), as stored for the state
 *          passing (bf16 values on the bf16 path)
 *   hin    (K_slots, nheads, headdim, dstate) fp32: state entering the chunk
 *          ([M] §3.5.2 center factors), as the output kernel reads it (bf16
 *          values on the bf16 path)
 * Slots past the real chunk count are left unwritten.
 */
ssd_status ssd_chunked_fwd_intermediates(const void* x, const float* dt, const float* A_head,
                                         const void* B, const void* C,
                                         const int32_t* cu_seqlens, int64_t nseqs,
                                         int64_t total_len, int32_t nheads, int32_t headdim,
                                         int32_t dstate, int32_t ngroups, int32_t chunk_len,
                                         ssd_dtype dtype, void* y, float* final_state,
                                         float* acs, float* states, float* hin, void* stream);

/* Chunk slots the intermediates use: nseqs * ceil(total_len / nseqs / Q) for the
 * batched form (varlen == 0), ceil(total_len / Q) + nseqs for varlen. */
int64_t ssd_chunk_slots(int64_t nseqs, int64_t total_len, int32_t chunk_len, int32_t varlen);

/* 1 if (dtype, dstate, chunk_len) is in the built set for headdim 64, else 0. */
int32_t ssd_config_supported(ssd_dtype dtype, int32_t dstate, int32_t chunk_len);

/* Human-readable name of a status code (static string). */
const char* ssd_status_string(ssd_status status);

/*
 * Host-side check of the workspace layouts (no device needed, nothing is
 * allocated or launched): every entry point that takes a workspace (forward
 * in all its forms, the no-allocation forward, the normalised forward, the
 * backward's routes) is run over a grid of dtypes, chunk lengths, state sizes,
 * lengths, head/group counts and options with fake device pointers, up to the
 * point where its workspace is carved; each carving is checked to put every
 * non-null piece inside the allocation and no two pieces on the same bytes,
 * with absent (zero-byte) pieces null.  The same check runs on every real
 * call before anything is launched (a failure there returns SSD_ERR_HIP and
 * launches nothing).  Returns the number of failed layouts (0: all pass).
 */
int32_t ssd_workspace_selfcheck(void);

/*
 * Optional per-kernel timing (process-wide, off by default).  While enabled,
 * every launch is bracketed by two HIP events recorded on the launch stream.
 * ssd_kernel_timing_read synchronises those events, adds their elapsed times
 * to per-kernel totals and, if reset != 0, clears the totals afterwards.
 * kernel ids: 0 sequence table (varlen calls only), 1 chunk cumsum + chunk
 * states, 2 state passing, 3 chunk output (kernel-matrix tiles, diagonal
 * blocks, state-to-output), 4 separate kernel-matrix pass (only the
 * configurations whose chunk-output kernel cannot hold the tiles in LDS:
 * fp32, and bf16 with dstate 256 at chunk_len 256), 5 decode step, 6 the
 * backward pass's glue kernels (its forward-kernel passes count under 1-4),
 * 7 the diagonal selective scan (ssd_selective_scan).  The normalised
 * output's extra work runs inside kernels 1, 2 and 3.  Ids 0..7; another id
 * is SSD_ERR_INVALID_ARGUMENT.  The events add a few microseconds per launch.
 * Not re-entrant with concurrent forward calls.
 */
ssd_status ssd_kernel_timing_enable(int32_t enable);
ssd_status ssd_kernel_timing_read(int32_t kernel, double* total_ms, int64_t* launches,
                                  int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
