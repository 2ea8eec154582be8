// ssd_internal.hpp -- problem description, workspace layout and kernel
// launchers shared by the C-ABI (ssd_api.cpp) and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

constexpr int kHeadDim = 64;            // P: the head dim built (two MFMA tiles of 32)
constexpr int kLdsLimit = 160 * 1024;   // LDS per workgroup on gfx950
constexpr int kThreads = 256;           // 4 waves per workgroup in every SSD kernel

enum class Dtype : int { F32 = 0, BF16 = 1 };

// Chunk descriptor: sequence index (-1: slot unused), first packed token, length.
struct ChunkDesc {
  int32_t seq;
  int32_t len;
  int64_t t0;
};

// One forward problem.  The token axis is packed: a batched call with b
// sequences of length T is the packed axis of b*T tokens, sequence s at
// [s*T, (s+1)*T).  cu == nullptr selects that batched form.
struct Problem {
  const void* x;          // (Ttot, H, P)  element dtype
  const float* dt;        // (Ttot, H)
  const float* A;         // (H)
  const void* B;          // (Ttot, G, N)  element dtype
  const void* C;          // (Ttot, G, N)  element dtype
  const int32_t* cu;      // (S+1) on the device, or nullptr (batched)
  void* y;                // (Ttot, H, P)  element dtype
  float* final_state;     // (S, H, P, N) or nullptr
  const float* initial_state;  // (S, H, P, N): state before each sequence's first token, or nullptr (zero)
  const float* D;         // (H): y += D_h x (skip connection), or nullptr
  int x_times_dt;         // 1: the input enters as dt_t x_t (B scaled by the step size)
  int strict_diag;        // 1: y leaves out each token's own term (C_t . B_t) x_t (backward's use)
  float* denom;           // (Ttot, H) fp32: normalised output: its denominator, formed by the output
                          // kernel (y is divided by it), or nullptr
  int64_t nseq;           // S
  int64_t seqlen;         // T (batched form only)
  int64_t total;          // Ttot
  int H, P, N, G, Q;
  Dtype dtype;
  int64_t kmax;           // chunk slots: exact when batched, a bound when varlen
  int stream_states;      // 1: chunk states and passed states are stored with the
                          // non-temporal hint (set when a forward's data exceeds the
                          // last-level cache; y always is)
};

// One recurrent (decode) step for a batch of sequences.
// Selective scan with a diagonal transition (the comparator; k10).
struct ScanProblem {
  const void* x;         // (batch, D, T) element dtype, channel-major
  const float* delta;    // (batch, D, T)
  const float* A;        // (D, N)
  const void* B;         // (batch, T, N) element dtype
  const void* C;         // (batch, T, N) element dtype
  void* y;               // (batch, D, T) element dtype
  float* final_state;    // (batch, D, N) or nullptr
  int64_t batch, seqlen;
  int D, N;
  Dtype dtype;
};

struct DecodeProblem {
  const void* x;      // (batch, H, P)  element dtype
  const float* dt;    // (batch, H)
  const float* A;     // (H)
  const void* B;      // (batch, G, N)  element dtype
  const void* C;      // (batch, G, N)  element dtype
  float* state;       // (batch, H, P, N) fp32, updated in place
  void* y;            // (batch, H, P)  element dtype
  const float* D;     // (H) skip weights or nullptr
  int x_times_dt;     // 1: the input enters as dt x
  int64_t batch;
  int H, P, N, G;
  Dtype dtype;
};

// tokens per segment of the backward's reverse prefix sums
constexpr int kBwdScanSeg = 1024;
// B/C groups the backward supports (its per-token kernel keeps one value per group in LDS)
constexpr int kMaxBwdGroups = 256;

// Backward pass: the caller's arrays and the rearranged inputs and outputs of
// the three gradient passes (all in the element dtype unless noted).
struct BwdProblem {
  const void* x; const float* dt; const float* A; const void* B; const void* C;
  const int32_t* cu;      // (S+1) or nullptr (batched)
  const float* h0;        // (S, H, P, N) initial state or nullptr
  const void* dy;         // (Ttot, H, P)
  const float* dfinal;    // (S, H, P, N) gradient of the final state or nullptr
  const float* D;         // (H) or nullptr
  int x_times_dt;
  void* dx; float* ddt; float* dA; void* dB; void* dC; float* dD; float* dinit;
  int64_t nseq, seqlen, total;
  int H, P, N, G;
  int NK;                 // 64-column parts of N (N < 64: one, zero padded)
  Dtype dtype;
  // reversed pass (dx'): input dy reversed, B := C, C := B, shifted decays
  void* xr; void* Br; void* Cr; float* dtr;
  // C pass (in time) and B pass (reversed): per-head copies of B and C in 64-column parts
  void* xc; float* dtc; float* Ac; void* xb; float* dtb;
  void* cb;               // (Ttot, H, P) x' reversed: the B pass's C
  float* h0c; float* dfb; // (S, H*NK, 64, 64) fp32 transposed parts, or nullptr
  // The recompute of y and the reversed pass run in fp32 (on the bf16 path on
  // fp32 copies of their inputs; on the fp32 path these point at the arrays
  // above): d(ell) is a running sum of their terms, which bf16 results would
  // not resolve.  Both leave out each token's own term (strict_diag), which
  // d(ell) would otherwise subtract from itself; the glue adds it back to dx.
  const float* x32; const float* B32; const float* C32;    // (Ttot,H,P), (Ttot,G,N)
  const float* xr32; const float* Br32; const float* Cr32;
  float* y_f; float* hlast;    // recompute: y without D and own term; final state
  float* y_x; float* g0;       // reversed pass: dx' without own term (reversed order); G_first
  void* y_c; void* y_b;        // (Ttot, H*NK, 64) per-head parts of dC and (reversed) dB
  float* qd; float* rd; float* ud;  // (H, Ttot) fp32 per-token terms
  // chunk-local d(ell) (bf16, every sequence a whole number of chunks of Q): the
  // forward's and the reversed pass's passed states as those passes store them
  bool chunked_dl;
  int Q;
  const void* hin_e; const void* gin_e;   // (K, H, P, N) element dtype
  const float* acs_f;          // (K, H, Q) chunk-local cumsums of dt A, as the forward's chunk-state kernel forms them
  const void* y_x8;            // reversed pass in the element dtype: dx' (own terms in), reversed order
  float* dl_v;                 // (H, Ttot) row sums of W + yterm
  float* dl_cols;              // (2, H, Ttot) column sums of W, per workgroup of the chunk
  float* dl_u;                 // (H, Ttot) dterm
  float* dl_kc;                // (K, H) <Gout, exp(Lam) Hin>, then (after the d(ell) scan) each chunk's share of dA
  int nseg;                    // scan segments per (sequence, head): ceil(longest sequence / kBwdScanSeg)
  double* segsum;              // (S, H, nseg) fp64 segment sums of d(Acs)
  float* edot;                 // (S, H) <dfinal, h_last>
};

// Device workspace, carved out of one allocation (256-byte aligned pieces).
struct Workspace {
  int32_t* seq_off = nullptr;    // (S+1) first chunk slot of each sequence; [S] = chunk count
  int64_t* seq_start = nullptr;  // (S)   first token of each sequence (clamped to [0,Ttot])
  int64_t* seq_len = nullptr;    // (S)   tokens of each sequence (clamped, >= 0)
  ChunkDesc* chunks = nullptr;   // (kmax) varlen only: written by the chunk-state kernel
  float* acs = nullptr;          // (kmax, H, Q) chunk-local cumsum of dt*A
  float* lam = nullptr;          // (kmax, H)    its last entry (log of the chunk's decay)
  // Tables of the output kernel's per-element mask, written by the chunk-state
  // kernel only for the (chunk, head) pairs that do not take the whole-chunk
  // factorisation (mask_by_chunk false); elsewhere they are left unwritten.
  float* ell = nullptr;          // (kmax, H, Q) dt*A per token
  float* rsuf = nullptr;         // (kmax, H, Q) sum of dt*A over the later tokens of its 32-token tile
  float* ttot = nullptr;         // (kmax, H, 8) sum of dt*A over each 32-token tile
  float* tmax = nullptr;         // (kmax, H)    the largest decay of a 32-token tile, -min of ttot
  float* xlog = nullptr;         // (kmax, H, Q) Acs - ln dt, the log of x's staging divisor
                                 //              (only with x_times_dt)
  void* states = nullptr;        // (kmax, H, P, N) chunk states, element dtype
  void* hin = nullptr;           // (kmax, H, P, N) state entering each chunk, element dtype
  void* cb = nullptr;            // (kmax, G, NI(NI+1)/2 tiles, 16-byte vector, 64 lanes) kernel
                                 // tiles of C B^T, element dtype, NI = Q/32 (16 values per lane)
  void* zs = nullptr;            // (kmax, H, N) normalised output only: chunk states of the ones
  void* zin = nullptr;           //   column (the chunk-state kernel's extra MFMA tile) and their
                                 //   passed states, element dtype (state passing carries them as
                                 //   N more channels per head)
  void* cop = nullptr;           // (kmax, G, NI, N/K steps, 64 lanes, one MFMA operand slice)
                                 // C rows in MFMA B-operand order, element dtype
};

// Carves 256-byte-aligned pieces out of one workspace allocation (host
// side).  A piece of zero bytes is a null pointer, never an address inside
// (or one past) the allocation: a kernel handed a non-null pointer may write
// through it.  Every piece is logged so that check() can verify, before
// anything is launched, that each non-null piece lies inside the allocation
// and that no two pieces overlap.  No allocation of its own (fixed log).
struct Carver {
  static constexpr int kMaxPieces = 64;
  char* base = nullptr;  // nullptr: only the size is computed
  size_t off = 0;        // bytes carved so far (aligned)
  int n = 0;
  bool overflow = false;
  size_t at[kMaxPieces], bytes[kMaxPieces];
  void reset(char* b) { base = b; off = 0; n = 0; overflow = false; }
  char* take(size_t nbytes) {
    const size_t a = off;
    off = (off + nbytes + 255) & ~(size_t)255;
    if (nbytes == 0) return nullptr;
    if (n < kMaxPieces) { at[n] = a; bytes[n] = nbytes; ++n; } else { overflow = true; }
    return base ? base + a : nullptr;
  }
  // every logged piece inside [0, capacity), no two overlapping
  bool check(size_t capacity) const {
    if (overflow) return false;
    for (int i = 0; i < n; ++i) {
      if (at[i] > capacity || bytes[i] > capacity - at[i]) return false;
      for (int j = 0; j < i; ++j)
        if (at[i] < at[j] + bytes[j] && at[j] < at[i] + bytes[i]) return false;
    }
    return true;
  }
};

// Bytes of workspace for p; fills *ws from base when base != nullptr.  With
// a carver given, the pieces are logged in it (for Carver::check).
size_t workspace_layout(const Problem& p, char* base, Workspace* ws, Carver* carver = nullptr);
// Host self-check of the workspace layouts of the forward and the backward
// over a set of shapes and options (fake base address, nothing launched):
// returns the number of layouts whose pieces fail Carver::check.
int workspace_selfcheck();

// Heads per workgroup of the chunk-state and chunk-output kernels (one
// workgroup per CU): the divisor of the heads of a group, <= kMaxHeadsPerBlock,
// that minimises rounds of workgroups x (heads per workgroup + two heads' worth
// of start-up work).
constexpr int kMaxHeadsPerBlock = 32;
int heads_per_block(const Problem& p, int max_hb = kMaxHeadsPerBlock);
// Compute units of the current device (cached per device).
int device_cus();

// Whether (dtype, Q, N) has an instantiated kernel set that fits in LDS.
bool config_supported(Dtype dt, int Q, int N);

// Kernel launchers; each returns the launch status.  Kernel ids for timing.
enum KernelId { kK0SeqTable = 0, kK13ChunkState = 1, kK4StatePass = 2, kK25ChunkOutput = 3,
                kK2ChunkCB = 4, kK6DecodeStep = 5, kK7BackwardGlue = 6,
                kK10SelectiveScan = 7, kNumKernels = 8 };
// K0 (varlen only): per-sequence first token, length and first chunk slot.
hipError_t launch_seq_table(const Problem& p, const Workspace& ws, hipStream_t s);
// K1 + K3: chunk-local log-decay cumsum (-> acs, lam, dmax), chunk states (-> states);
// states_f32 (nullable) receives an fp32 copy of the stored states.
hipError_t launch_chunk_state(const Problem& p, const Workspace& ws, float* states_f32,
                              hipStream_t s);
// K4: state passing (-> hin, final_state); hin_f32 (nullable) receives an fp32 copy.
hipError_t launch_state_pass(const Problem& p, const Workspace& ws, float* hin_f32, hipStream_t s);
// K2 (first half): kernel matrix tiles C B^T of every chunk and group (-> cb, cop),
// for the configurations whose chunk-output kernel does not form them itself.
hipError_t launch_chunk_cb(const Problem& p, const Workspace& ws, hipStream_t s);
// K2 + K5: diagonal blocks and state-to-output (-> y).
hipError_t launch_chunk_output(const Problem& p, const Workspace& ws, hipStream_t s);
// K6: one recurrent step (decode): state update in place and y.
hipError_t launch_decode_step(const DecodeProblem& d, hipStream_t s);
hipError_t launch_selective_scan(const ScanProblem& p, hipStream_t s);
// K7 backward glue: stage 0 builds the gradient passes' inputs (and zeroes dA,
// dD), stage 1 turns their outputs into dx, dB, dC, d(dt), dA, dD, dh0.
hipError_t launch_backward_glue(const BwdProblem& b, int stage, hipStream_t s);
// K8: chunk-local d(ell) -> d(dt), dA (BwdProblem::chunked_dl).
hipError_t launch_backward_dl(const BwdProblem& b, hipStream_t s);
// H: the kernel's copies take 32-bit offsets within 32 token rows of x (at
// most 2^19 heads of 64 channels).
bool backward_dl_supported(Dtype dt, int Q, int N, int64_t H);
// Sequences padded to whole chunks of Q for the chunk-local backward:
// sequence s starts at cup[s] in the padded layout (cup has S + 2 entries;
// [cup[S], cup[S + 1] = Tp) is one zero sequence up to the host's bound Tp).
// The padding has dt = 0 (decay 1) and zero x, dy, B, C.
struct PadArgs {
  const int32_t* cu; int32_t* cup;  // cu null: batched, S sequences of seqlen tokens
  int64_t S, T, Tp, seqlen;
  int H, P, G, N, Q;
  Dtype dtype;
  const void* x; const float* dt; const void* B; const void* C; const void* dy;  // (T, ...) in
  void* xp; float* dtp; void* Bp; void* Cp; void* dyp;                            // (Tp, ...) padded
  const void* dxp; const float* ddtp; const void* dBp; const void* dCp;          // (Tp, ...) results
  void* dx; float* ddt; void* dB; void* dC;                                        // (T, ...) out
};
// stage 0: cup, then the padded inputs; stage 1: the results back to (T, ...)
hipError_t launch_backward_pad(const PadArgs& a, int stage, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);  // p[0, n) = 0 (a kernel, no memset node)
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);  // p[0, n) = v (a kernel)
// Poisoning of every workspace before use (SSD_POISON_WORKSPACE=1 in the
// environment, read once): each call fills its workspace with quiet NaNs
// before its kernels run, so that a kernel reading a piece it did not write
// first turns its results into NaN.  A checking mode; off by default.
constexpr uint32_t kPoisonNaN = 0x7fc00000u;
bool poison_workspace();

// dB and dC of the chunk-local path summed over heads per chunk (bf16, whole
// chunks of b.Q, N in {64, 128, 256}); with nsub > 1 head subsets, part holds
// (nsub, 2, Ttot, G, N) fp32 partial sums
hipError_t launch_backward_dbdc(const BwdProblem& b, float* part, int nsub, hipStream_t s);
bool backward_dbdc_supported(Dtype dt, int Q, int N);
int backward_dbdc_subsets(int64_t chunks, int G, int H, int N);
bool chunk_state_supported(Dtype dt, int Q, int N);
bool chunk_output_supported(Dtype dt, int Q, int N);
// Whether the chunk-output kernel for (dtype, Q, N) reads the kernel-matrix pass's
// tiles (ws.cb, ws.cop); otherwise it forms them itself and that pass is skipped.
bool chunk_output_reads_cb(Dtype dt, int Q, int N);

}  // namespace ssd
