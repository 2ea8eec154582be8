// ssd_api.cpp -- the C ABI of libssd.so (declared in include/ssd.h).
//
// Host side only: argument validation (before any HIP call), workspace
// layout, the launch sequences on the caller's stream, and the optional
// per-kernel event timing.  The forward follows the four steps of the block
// decomposition in "LLM(十一)——Mamba" (mztchaoqun.com.cn) §3.5.2 "SSD
// algorithm: chunking and state passing", with the chunk tables first:
//   [K0 sequence table, varlen only] -> K1+K3 chunk cumsum and chunk states ->
//   K4 state passing -> K2+K5 diagonal blocks fused with state-to-output.
// The decode step is one kernel (K6); the backward is glue (K7) around four
// runs of the forward sequence on rearranged inputs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <stdlib.h>
#include <string.h>
#include <vector>

#include "ssd.h"
#include "ssd_internal.hpp"

namespace ssd {

bool config_supported(Dtype dt, int Q, int N) {
  return chunk_state_supported(dt, Q, N) && chunk_output_supported(dt, Q, N);
}

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

bool poison_workspace() {
  static const bool on = [] {
    const char* v = getenv("SSD_POISON_WORKSPACE");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}

constexpr double kLastLevelCacheBytes = 256.0 * 1024 * 1024;

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int heads_per_block(const Problem& p, int max_hb) {
  const int hpg = p.H / p.G;
  const int cus = device_cus();
  int best = 1;
  double best_cost = -1.0;
  for (int hb = max_hb < kMaxHeadsPerBlock ? max_hb : kMaxHeadsPerBlock; hb >= 1; --hb) {
    if (hpg % hb) continue;
    const double wgs = (double)p.kmax * (p.H / hb);
    const double rounds = std::ceil(wgs / (double)cus);
    const double cost = rounds * (hb + 2);  // start-up of a workgroup: about two heads' time
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = hb;
    }
  }
  return best;
}

size_t workspace_layout(const Problem& p, char* base, Workspace* ws, Carver* carver) {
  const size_t S = (size_t)p.nseq, K = (size_t)p.kmax, H = (size_t)p.H;
  const size_t PN = (size_t)p.P * p.N;
  const size_t esz = p.dtype == Dtype::BF16 ? 2 : 4;
  Carver local;
  Carver& cv = carver ? *carver : local;
  cv.reset(base);
  auto take = [&](size_t bytes) { return cv.take(bytes); };
  char* seq_off = take((S + 1) * sizeof(int32_t));
  char* seq_start = take(S * sizeof(int64_t));
  char* seq_len = take(S * sizeof(int64_t));
  char* chunks = take(K * sizeof(ChunkDesc));
  char* acs = take(K * H * p.Q * sizeof(float));
  char* lam = take(K * H * sizeof(float));
  char* ell = take(K * H * p.Q * sizeof(float));
  char* rsuf = take(K * H * p.Q * sizeof(float));
  char* ttot = take(K * H * 8 * sizeof(float));
  char* tmax = take(K * H * sizeof(float));
  char* xlog = take(p.x_times_dt ? K * H * p.Q * sizeof(float) : 0);
  char* states = take(K * H * PN * esz);
  char* hin = take(K * H * PN * esz);
  const size_t NI = (size_t)p.Q / 32;
  const bool use_cb = chunk_output_reads_cb(p.dtype, p.Q, p.N);
  char* cb = take(use_cb ? K * (size_t)p.G * (NI * (NI + 1) / 2) * 64 * 16 * esz : 0);
  char* cop = take(use_cb ? K * (size_t)p.G * p.Q * p.N * esz : 0);
  char* zs = take(p.denom ? K * H * p.N * esz : 0);
  char* zin = take(p.denom ? K * H * p.N * esz : 0);
  if (ws && base) {
    ws->seq_off = reinterpret_cast<int32_t*>(seq_off);
    ws->seq_start = reinterpret_cast<int64_t*>(seq_start);
    ws->seq_len = reinterpret_cast<int64_t*>(seq_len);
    ws->chunks = reinterpret_cast<ChunkDesc*>(chunks);
    ws->acs = reinterpret_cast<float*>(acs);
    ws->lam = reinterpret_cast<float*>(lam);
    ws->ell = reinterpret_cast<float*>(ell);
    ws->rsuf = reinterpret_cast<float*>(rsuf);
    ws->ttot = reinterpret_cast<float*>(ttot);
    ws->tmax = reinterpret_cast<float*>(tmax);
    ws->xlog = p.x_times_dt ? reinterpret_cast<float*>(xlog) : nullptr;
    ws->states = states;
    ws->hin = hin;
    ws->cb = cb;
    ws->cop = cop;
    ws->zs = p.denom ? zs : nullptr;
    ws->zin = p.denom ? zin : nullptr;
  }
  return cv.off;
}

// ------------------------------------------------------------ timing ----
namespace {
struct TimedLaunch {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_mu;
bool g_timing = false;
std::vector<TimedLaunch> g_pending;
std::vector<hipEvent_t> g_free_events;
double g_total_ms[kNumKernels] = {0};
int64_t g_launches[kNumKernels] = {0};

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed_launch(int kernel, hipStream_t s, F&& launch) {
  bool timing;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    timing = g_timing;
  }
  if (!timing) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    a = take_event();
    b = take_event();
  }
  if (a == nullptr || b == nullptr) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({kernel, a, b});
  return hipSuccess;
}
}  // namespace

// ------------------------------------------------------------- dry run ----
// Layout check without a device: while g_dry is set on a thread, the entry
// points validate and carve their workspaces from a fake base address, check
// the pieces (Carver::check; a failure counts in g_dry_bad) and return before
// any HIP call.  Used by workspace_selfcheck only.
namespace {
thread_local bool g_dry = false;
thread_local int g_dry_bad = 0;
thread_local int64_t g_dry_checks = 0;
char* const kDryBase = reinterpret_cast<char*>((uintptr_t)1 << 40);
}  // namespace

// In a dry run: count a failed layout check.  Otherwise: whether the carved
// pieces passed (a failure is a layout defect; the caller launches nothing).
static bool layout_ok(const Carver& cv, size_t capacity) {
  const bool ok = cv.check(capacity);
  if (g_dry) {
    ++g_dry_checks;
    if (!ok) ++g_dry_bad;
  }
  return ok;
}

// ----------------------------------------------------------- device check ----
static ssd_status check_device() {
  if (g_dry) return SSD_OK;
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
  if (dev < 0 || dev >= 64) return SSD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SSD_ERR_HIP;
    known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (known[dev] == 1) {
      // keep freed workspace cached in the default pool between calls
      hipMemPool_t pool;
      if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
        uint64_t thr = ~0ull;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
      }
    }
  }
  return known[dev] == 1 ? SSD_OK : SSD_ERR_UNSUPPORTED;
}

static bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// Validates everything that can be checked on the host.  No HIP call.
static ssd_status validate(const Problem& p) {
  if (p.H <= 0 || p.G <= 0 || p.H % p.G != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (p.P <= 0 || p.N <= 0 || p.Q <= 0 || p.nseq < 0 || p.total < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (p.dtype != Dtype::F32 && p.dtype != Dtype::BF16) return SSD_ERR_INVALID_ARGUMENT;
  if (p.P != kHeadDim) return SSD_ERR_UNSUPPORTED;
  if (!(p.N == 16 || p.N == 32 || p.N == 64 || p.N == 128 || p.N == 256)) return SSD_ERR_UNSUPPORTED;
  if (!(p.Q == 64 || p.Q == 128 || p.Q == 256)) return SSD_ERR_UNSUPPORTED;
  if (!config_supported(p.dtype, p.Q, p.N)) return SSD_ERR_UNSUPPORTED;
  if (p.A == nullptr || !aligned(p.A, 4)) return SSD_ERR_INVALID_ARGUMENT;
  if (p.total > 0) {
    if (!p.x || !p.dt || !p.B || !p.C || !p.y) return SSD_ERR_INVALID_ARGUMENT;
    if (!aligned(p.x, 16) || !aligned(p.B, 16) || !aligned(p.C, 16) || !aligned(p.y, 16) ||
        !aligned(p.dt, 4))
      return SSD_ERR_INVALID_ARGUMENT;
  }
  if (p.final_state && !aligned(p.final_state, 16)) return SSD_ERR_INVALID_ARGUMENT;
  if (p.initial_state && !aligned(p.initial_state, 16)) return SSD_ERR_INVALID_ARGUMENT;
  if (p.D && !aligned(p.D, 4)) return SSD_ERR_INVALID_ARGUMENT;
  if (p.x_times_dt != 0 && p.x_times_dt != 1) return SSD_ERR_INVALID_ARGUMENT;
  if (p.cu && !aligned(p.cu, 4)) return SSD_ERR_INVALID_ARGUMENT;
  // sizes must keep every index and grid inside 32/64-bit ranges
  const int64_t lim = (int64_t)1 << 40;
  if (p.total > lim || p.nseq > ((int64_t)1 << 30) || p.kmax > ((int64_t)1 << 30)) return SSD_ERR_INVALID_ARGUMENT;
  if (p.kmax * p.H > 0x7fffffffLL || p.nseq * p.H * 16 > 0x7fffffffLL) return SSD_ERR_INVALID_ARGUMENT;
  if (p.total * p.H * p.P > ((int64_t)1 << 46)) return SSD_ERR_INVALID_ARGUMENT;
  return SSD_OK;
}

static ssd_status map_err(hipError_t e) {
  if (e == hipSuccess) return SSD_OK;
  if (e == hipErrorOutOfMemory) return SSD_ERR_OUT_OF_MEMORY;
  return SSD_ERR_HIP;
}

struct DebugOut {
  float* acs = nullptr;
  float* states = nullptr;
  float* hin = nullptr;
  bool states_only = false;  // stop after the state passing (no y)
  void* hin_buf = nullptr;   // keep the passed states here (element dtype, (kmax, H, P, N))
  float* acs_buf = nullptr;  // keep the chunk-local cumsums here ((kmax, H, Q) fp32)
};

// ------------------------------------------------------------ workspace ----
// The workspace is cached per (device, stream) and reused by the next call on
// the same stream: stream order already keeps two calls on one stream from
// overlapping, so no event or allocation is needed per call (allocating and
// freeing per call made the host wait for the GPU, and an event recorded after
// every call cost the GPU several microseconds).  Calls on different streams
// use different workspaces.  A workspace grows (stream-ordered free and
// allocation) when a larger problem arrives and is otherwise kept until the
// process ends.  A stream destroyed while this library's work is still pending
// on it must not have its handle reused by a new stream before that work
// finishes (synchronise a stream before destroying it).
namespace {
struct WsEntry {
  int device;
  hipStream_t stream;
  int slot;  // 0: forward workspace, 1: backward temporaries
  void* ptr;
  size_t bytes;
};
std::mutex g_ws_mu;
std::vector<WsEntry> g_ws;

// Workspace of >= bytes for (device, stream), or nullptr on allocation failure.
void* ws_acquire(int device, size_t bytes, hipStream_t stream, int slot = 0) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (WsEntry& w : g_ws) {
    if (w.device != device || w.stream != stream || w.slot != slot) continue;
    if (w.bytes >= bytes) return w.ptr;
    // grow in stream order: the previous calls on this stream finish first
    if (hipFreeAsync(w.ptr, stream) != hipSuccess) return nullptr;
    w.ptr = nullptr;
    w.bytes = 0;
    if (hipMallocAsync(&w.ptr, bytes, stream) != hipSuccess || w.ptr == nullptr) {
      w.ptr = nullptr;
      return nullptr;
    }
    w.bytes = bytes;
    return w.ptr;
  }
  void* ptr = nullptr;
  if (hipMallocAsync(&ptr, bytes > 0 ? bytes : 256, stream) != hipSuccess || ptr == nullptr) return nullptr;
  g_ws.push_back({device, stream, slot, ptr, bytes});
  return ptr;
}
}  // namespace

// fixed_base: the workspace to use (at least workspace_layout's bytes, checked
// by the caller), in place of the per-stream cached allocation.
static ssd_status run(const Problem& p, hipStream_t stream, const DebugOut* dbg, char* fixed_base = nullptr) {
  ssd_status st = validate(p);
  if (st != SSD_OK) return st;
  st = check_device();
  if (st != SSD_OK) return st;
  if (p.nseq == 0) return SSD_OK;
  const size_t bytes = workspace_layout(p, nullptr, nullptr);
  char* base = g_dry ? kDryBase : fixed_base;
  if (base == nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    base = static_cast<char*>(ws_acquire(dev, bytes, stream));
    if (base == nullptr) return SSD_ERR_OUT_OF_MEMORY;
  }
  Workspace ws;
  Carver cv;
  workspace_layout(p, base, &ws, &cv);
  if (!layout_ok(cv, bytes)) return g_dry ? SSD_OK : SSD_ERR_HIP;  // a layout defect: launch nothing
  if (g_dry) return SSD_OK;
  if (poison_workspace()) {
    const hipError_t pe = launch_fill_u32(reinterpret_cast<uint32_t*>(base), (int64_t)(bytes / 4), kPoisonNaN, stream);
    if (pe != hipSuccess) return map_err(pe);
  }
  if (dbg && dbg->hin_buf) ws.hin = dbg->hin_buf;
  if (dbg && dbg->acs_buf) ws.acs = dbg->acs_buf;
  hipError_t e = hipSuccess;
  const size_t KH = (size_t)p.kmax * p.H;
  do {
    if (p.cu != nullptr) {
      e = timed_launch(kK0SeqTable, stream, [&] { return launch_seq_table(p, ws, stream); });
      if (e != hipSuccess) break;
    }
    if (p.kmax > 0) {
      e = timed_launch(kK13ChunkState, stream, [&] {
        return launch_chunk_state(p, ws, dbg ? dbg->states : nullptr, stream);
      });
      if (e != hipSuccess) break;
      if (dbg && dbg->acs) {
        e = hipMemcpyAsync(dbg->acs, ws.acs, KH * p.Q * sizeof(float), hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) break;
      }
    }
    const bool states_only = dbg != nullptr && dbg->states_only;
    if (p.kmax > 0 && !states_only && chunk_output_reads_cb(p.dtype, p.Q, p.N)) {
      e = timed_launch(kK2ChunkCB, stream, [&] { return launch_chunk_cb(p, ws, stream); });
      if (e != hipSuccess) break;
    }
    e = timed_launch(kK4StatePass, stream, [&] {
      return launch_state_pass(p, ws, dbg ? dbg->hin : nullptr, stream);
    });
    if (e != hipSuccess) break;
    if (p.kmax > 0 && !states_only) {
      e = timed_launch(kK25ChunkOutput, stream, [&] { return launch_chunk_output(p, ws, stream); });
      if (e != hipSuccess) break;
    }
  } while (false);
  return map_err(e);
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------ static scratch ----
// The workspace of ssd_chunked_fwd_noalloc: a file-scope device array, one
// copy on every GPU the library runs on, held until the process ends.  In
// host code `scratch` is a host-side stand-in for the symbol, not a device
// address: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// passed to kernels.
constexpr size_t kScratchBytes = (size_t)SSD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
char* g_scratch_ptr[64] = {nullptr};
}  // namespace

// Device address of the current device's scratch array (looked up on the
// device's first call).
static ssd_status scratch_base(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
  if (dev < 0 || dev >= 64) return SSD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SSD_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return SSD_OK;
}

}  // namespace ssd

using namespace ssd;

extern "C" {

int64_t ssd_chunk_slots(int64_t nseqs, int64_t total_len, int32_t chunk_len, int32_t varlen) {
  if (nseqs <= 0 || total_len < 0 || chunk_len <= 0) return 0;
  if (varlen) return ceil_div(total_len, chunk_len) + nseqs;
  return nseqs * ceil_div(total_len / nseqs, chunk_len);
}

int32_t ssd_config_supported(ssd_dtype dtype, int32_t dstate, int32_t chunk_len) {
  if (dtype != SSD_DTYPE_F32 && dtype != SSD_DTYPE_BF16) return 0;
  return config_supported(static_cast<Dtype>(dtype), chunk_len, dstate) ? 1 : 0;
}

static Problem make_problem(const void* x, const float* dt, const float* A_head, const void* B,
                            const void* C, const int32_t* cu, int64_t nseq, int64_t seqlen,
                            int64_t total, int32_t nheads, int32_t headdim, int32_t dstate,
                            int32_t ngroups, int32_t chunk_len, ssd_dtype dtype, void* y,
                            float* final_state, const float* initial_state = nullptr,
                            const float* D = nullptr, int32_t x_times_dt = 0, int strict_diag = 0) {
  Problem p;
  p.x = x; p.dt = dt; p.A = A_head; p.B = B; p.C = C; p.cu = cu; p.y = y;
  p.final_state = final_state;
  p.initial_state = initial_state;
  p.D = D;
  p.x_times_dt = x_times_dt;
  p.strict_diag = strict_diag;
  p.denom = nullptr;
  p.nseq = nseq; p.seqlen = seqlen; p.total = total;
  p.H = nheads; p.P = headdim; p.N = dstate; p.G = ngroups; p.Q = chunk_len;
  p.dtype = static_cast<Dtype>(dtype);
  p.kmax = 0;
  if (chunk_len > 0 && nseq >= 0 && total >= 0)
    p.kmax = cu ? ceil_div(total, chunk_len) + nseq : nseq * ceil_div(seqlen, chunk_len);
  // A forward touches x and y, the chunk states and the passed states (each
  // (chunks, H, P, N)), B and C.  While that fits in the memory-side last-level
  // cache (MI355X: 256 MiB of Infinity Cache) the states written by one kernel
  // are still there when the next one reads them, and are stored normally;
  // beyond it they are streamed out with the non-temporal hint so that they do
  // not displace the inputs.
  const double esz = p.dtype == Dtype::BF16 ? 2.0 : 4.0;
  const double footprint = esz * ((double)p.total * p.H * p.P * 2.0 + (double)p.kmax * p.H * p.P * p.N * 2.0 +
                                  (double)p.total * p.G * p.N * 2.0);
  p.stream_states = footprint > kLastLevelCacheBytes ? 1 : 0;
  return p;
}

ssd_status ssd_chunked_fwd(const void* x, const float* dt, const float* A_head, const void* B,
                           const void* C, int64_t batch, int64_t seqlen, int32_t nheads,
                           int32_t headdim, int32_t dstate, int32_t ngroups, int32_t chunk_len,
                           ssd_dtype dtype, void* y, float* final_state, void* stream) {
  if (batch < 0 || seqlen < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return SSD_ERR_INVALID_ARGUMENT;
  const Problem p = make_problem(x, dt, A_head, B, C, nullptr, batch, seqlen, batch * seqlen,
                                 nheads, headdim, dstate, ngroups, chunk_len, dtype, y, final_state);
  return run(p, static_cast<hipStream_t>(stream), nullptr);
}

ssd_status ssd_chunked_fwd_noalloc(const void* x, const float* dt, const float* A_head,
                                   const void* B, const void* C, int64_t batch, int64_t seqlen,
                                   int32_t nheads, int32_t headdim, int32_t dstate, int32_t ngroups,
                                   int32_t chunk_len, ssd_dtype dtype, void* y, float* final_state,
                                   void* stream) {
  if (batch < 0 || seqlen < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (batch > 0 && seqlen > ((int64_t)1 << 40) / batch) return SSD_ERR_INVALID_ARGUMENT;
  const Problem p = make_problem(x, dt, A_head, B, C, nullptr, batch, seqlen, batch * seqlen,
                                 nheads, headdim, dstate, ngroups, chunk_len, dtype, y, final_state);
  // host-side checks first: nothing is looked up or launched for a problem
  // that is invalid or does not fit
  ssd_status st = validate(p);
  if (st != SSD_OK) return st;
  if (workspace_layout(p, nullptr, nullptr) > kScratchBytes) return SSD_ERR_SCRATCH_LIMIT;
  st = check_device();
  if (st != SSD_OK) return st;
  char* base = nullptr;
  if (!g_dry) {
    st = scratch_base(&base);
    if (st != SSD_OK) return st;
  }
  return run(p, static_cast<hipStream_t>(stream), nullptr, base);
}

ssd_status ssd_chunked_fwd_varlen(const void* x, const float* dt, const float* A_head,
                                  const void* B, const void* C, const int32_t* cu_seqlens,
                                  int64_t nseqs, int64_t total_len, int32_t nheads,
                                  int32_t headdim, int32_t dstate, int32_t ngroups,
                                  int32_t chunk_len, ssd_dtype dtype, void* y,
                                  float* final_state, void* stream) {
  if (nseqs < 0 || total_len < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (nseqs > 0 && cu_seqlens == nullptr) return SSD_ERR_INVALID_ARGUMENT;
  const Problem p = make_problem(x, dt, A_head, B, C, cu_seqlens, nseqs, 0, total_len, nheads,
                                 headdim, dstate, ngroups, chunk_len, dtype, y, final_state);
  return run(p, static_cast<hipStream_t>(stream), nullptr);
}

ssd_status ssd_chunked_fwd_ex(const void* x, const float* dt, const float* A_head, const void* B,
                              const void* C, const int32_t* cu_seqlens, int64_t nseqs,
                              int64_t total_len, int32_t nheads, int32_t headdim, int32_t dstate,
                              int32_t ngroups, int32_t chunk_len, ssd_dtype dtype,
                              const float* initial_state, const float* D, int32_t x_times_dt,
                              void* y, float* final_state, void* stream) {
  if (nseqs < 0 || total_len < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs > 0 && total_len % nseqs != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs == 0 && total_len != 0) return SSD_ERR_INVALID_ARGUMENT;
  const int64_t seqlen = (cu_seqlens == nullptr && nseqs > 0) ? total_len / nseqs : 0;
  const Problem p = make_problem(x, dt, A_head, B, C, cu_seqlens, nseqs, seqlen, total_len, nheads,
                                 headdim, dstate, ngroups, chunk_len, dtype, y, final_state,
                                 initial_state, D, x_times_dt);
  return run(p, static_cast<hipStream_t>(stream), nullptr);
}

ssd_status ssd_chunked_fwd_normalized(const void* x, const float* dt, const float* A_head, const void* B,
                                      const void* C, const int32_t* cu_seqlens, int64_t nseqs,
                                      int64_t total_len, int32_t nheads, int32_t headdim, int32_t dstate,
                                      int32_t ngroups, int32_t chunk_len, ssd_dtype dtype, const float* D,
                                      int32_t x_times_dt, void* y, float* final_state, float* denom,
                                      void* stream) {
  if (nseqs < 0 || total_len < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs > 0 && total_len % nseqs != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs == 0 && total_len != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (total_len > 0 && (denom == nullptr || !aligned(denom, 4))) return SSD_ERR_INVALID_ARGUMENT;
  const int64_t seqlen = (cu_seqlens == nullptr && nseqs > 0) ? total_len / nseqs : 0;
  Problem p = make_problem(x, dt, A_head, B, C, cu_seqlens, nseqs, seqlen, total_len, nheads, headdim, dstate,
                           ngroups, chunk_len, dtype, y, final_state, nullptr, D, x_times_dt);
  p.denom = total_len > 0 ? denom : nullptr;
  return run(p, static_cast<hipStream_t>(stream), nullptr);
}

ssd_status ssd_chunked_fwd_intermediates(const void* x, const float* dt, const float* A_head,
                                         const void* B, const void* C,
                                         const int32_t* cu_seqlens, int64_t nseqs,
                                         int64_t total_len, int32_t nheads, int32_t headdim,
                                         int32_t dstate, int32_t ngroups, int32_t chunk_len,
                                         ssd_dtype dtype, void* y, float* final_state,
                                         float* acs, float* states, float* hin, void* stream) {
  if (nseqs < 0 || total_len < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs > 0 && total_len % nseqs != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs == 0 && total_len != 0) return SSD_ERR_INVALID_ARGUMENT;
  if ((acs && !aligned(acs, 16)) || (states && !aligned(states, 16)) || (hin && !aligned(hin, 16)))
    return SSD_ERR_INVALID_ARGUMENT;
  const int64_t seqlen = (cu_seqlens == nullptr && nseqs > 0) ? total_len / nseqs : 0;
  const Problem p = make_problem(x, dt, A_head, B, C, cu_seqlens, nseqs, seqlen, total_len, nheads,
                                 headdim, dstate, ngroups, chunk_len, dtype, y, final_state);
  DebugOut dbg;
  dbg.acs = acs; dbg.states = states; dbg.hin = hin;
  return run(p, static_cast<hipStream_t>(stream), &dbg);
}

ssd_status ssd_decode_step(const void* x, const float* dt, const float* A_head, const void* B,
                           const void* C, int64_t batch, int32_t nheads, int32_t headdim,
                           int32_t dstate, int32_t ngroups, ssd_dtype dtype, const float* D,
                           int32_t x_times_dt, float* state, void* y, void* stream) {
  if (batch < 0 || nheads <= 0 || ngroups <= 0 || nheads % ngroups != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (dtype != SSD_DTYPE_F32 && dtype != SSD_DTYPE_BF16) return SSD_ERR_INVALID_ARGUMENT;
  if (headdim <= 0 || dstate <= 0) return SSD_ERR_INVALID_ARGUMENT;
  if ((x_times_dt != 0 && x_times_dt != 1) || (D && !aligned(D, 4))) return SSD_ERR_INVALID_ARGUMENT;
  if (headdim != kHeadDim) return SSD_ERR_UNSUPPORTED;
  if (!(dstate == 16 || dstate == 32 || dstate == 64 || dstate == 128 || dstate == 256)) return SSD_ERR_UNSUPPORTED;
  if (batch > ((int64_t)1 << 40) / nheads || batch * nheads > 0x7fffffffLL) return SSD_ERR_INVALID_ARGUMENT;
  if (batch > 0) {
    if (!x || !dt || !A_head || !B || !C || !state || !y) return SSD_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(state, 16) ||
        !aligned(dt, 4) || !aligned(A_head, 4))
      return SSD_ERR_INVALID_ARGUMENT;
  }
  ssd_status st = check_device();
  if (st != SSD_OK) return st;
  DecodeProblem d;
  d.x = x; d.dt = dt; d.A = A_head; d.B = B; d.C = C; d.state = state; d.y = y;
  d.batch = batch; d.H = nheads; d.P = headdim; d.N = dstate; d.G = ngroups;
  d.D = D; d.x_times_dt = x_times_dt;
  d.dtype = static_cast<Dtype>(dtype);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return map_err(timed_launch(kK6DecodeStep, s, [&] { return launch_decode_step(d, s); }));
}

ssd_status ssd_selective_scan(const void* x, const float* delta, const float* A, const void* B,
                              const void* C, int64_t batch, int64_t seqlen, int32_t channels,
                              int32_t dstate, ssd_dtype dtype, void* y, float* final_state,
                              void* stream) {
  if (batch < 0 || seqlen < 0 || channels <= 0 || dstate <= 0) return SSD_ERR_INVALID_ARGUMENT;
  if (dtype != SSD_DTYPE_F32 && dtype != SSD_DTYPE_BF16) return SSD_ERR_INVALID_ARGUMENT;
  if (!(dstate == 64 || dstate == 128 || dstate == 256)) return SSD_ERR_UNSUPPORTED;
  // every index (b, d, t) and (b, t, n) stays below 2^40; the grid below 2^31
  if (batch > 0 && (batch > ((int64_t)1 << 40) / channels || seqlen > ((int64_t)1 << 40) / (batch * channels) ||
                    seqlen > ((int64_t)1 << 40) / (batch * dstate) || batch * channels > 0x7fffffffLL))
    return SSD_ERR_INVALID_ARGUMENT;
  const size_t e = dtype == SSD_DTYPE_BF16 ? 2 : 4;
  if (batch > 0) {
    if (!A || !aligned(A, 4) || (final_state && !aligned(final_state, 4))) return SSD_ERR_INVALID_ARGUMENT;
    if (seqlen > 0) {
      if (!x || !delta || !B || !C || !y) return SSD_ERR_INVALID_ARGUMENT;
      if (!aligned(x, e) || !aligned(B, e) || !aligned(C, e) || !aligned(y, e) || !aligned(delta, 4))
        return SSD_ERR_INVALID_ARGUMENT;
    }
  }
  ssd_status st = check_device();
  if (st != SSD_OK) return st;
  ScanProblem p;
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.y = y; p.final_state = final_state;
  p.batch = batch; p.seqlen = seqlen; p.D = channels; p.N = dstate;
  p.dtype = static_cast<Dtype>(dtype);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return map_err(timed_launch(kK10SelectiveScan, s, [&] { return launch_selective_scan(p, s); }));
}

// The backward, arguments as ssd_chunked_bwd.  aligned_q > 0: the caller
// guarantees that every packed sequence is a whole number of chunks of
// aligned_q = chunk_len (the padded layout below), so the chunk-local path
// takes cu_seqlens too.
static ssd_status bwd_impl(const void* x, const float* dt, const float* A_head, const void* B,
                           const void* C, const int32_t* cu_seqlens, int64_t nseqs,
                           int64_t total_len, int32_t nheads, int32_t headdim, int32_t dstate,
                           int32_t ngroups, int32_t chunk_len, ssd_dtype dtype,
                           const float* initial_state, const float* D, int32_t x_times_dt,
                           const void* dy, const float* dfinal_state, void* dx, float* ddt,
                           float* dA, void* dB, void* dC, float* dD, float* dinitial_state,
                           void* stream, int aligned_q) {
  if (nseqs < 0 || total_len < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs > 0 && total_len % nseqs != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr && nseqs == 0 && total_len != 0) return SSD_ERR_INVALID_ARGUMENT;
  const int64_t seqlen = (cu_seqlens == nullptr && nseqs > 0) ? total_len / nseqs : 0;
  // the forward problem, with dx standing in for y (same shape and dtype)
  Problem p = make_problem(x, dt, A_head, B, C, cu_seqlens, nseqs, seqlen, total_len, nheads, headdim,
                           dstate, ngroups, chunk_len, dtype, dx, nullptr, initial_state, D, x_times_dt);
  ssd_status st = validate(p);
  if (st != SSD_OK) return st;
  if (dA == nullptr || !aligned(dA, 4) || (dD && !aligned(dD, 4))) return SSD_ERR_INVALID_ARGUMENT;
  if ((dfinal_state && !aligned(dfinal_state, 16)) || (dinitial_state && !aligned(dinitial_state, 16)))
    return SSD_ERR_INVALID_ARGUMENT;
  if (total_len > 0) {
    if (!dy || !ddt || !dB || !dC) return SSD_ERR_INVALID_ARGUMENT;
    if (!aligned(dy, 16) || !aligned(dB, 16) || !aligned(dC, 16) || !aligned(ddt, 4))
      return SSD_ERR_INVALID_ARGUMENT;
  }
  // chunk length of the two passes whose state is (64 x 64): the caller's if
  // that configuration is built, else the longest that is (any partition gives
  // the same sums)
  int Q2 = 0;
  for (int q : {chunk_len, 256, 128, 64})
    if (config_supported(p.dtype, q, kHeadDim)) {
      Q2 = q;
      break;
    }
  // the fp32 passes (recompute of y, reversed pass for dx')
  int Qf = 0;
  for (int q : {chunk_len, 256, 128, 64})
    if (config_supported(Dtype::F32, q, dstate)) {
      Qf = q;
      break;
    }
  if (Q2 == 0 || Qf == 0 || ngroups > kMaxBwdGroups) return SSD_ERR_UNSUPPORTED;
  // Chunk-local d(ell) for bf16 inputs when every sequence is a whole number
  // of chunks of a built length Qd (then the reversed pass's chunks coincide
  // with the forward's): its passes run in bf16, and no fp32 recompute or
  // reversed pass is needed.
  int Qd = 0;
  if (aligned_q > 0 && aligned_q == chunk_len && backward_dl_supported(p.dtype, aligned_q, dstate, nheads) &&
      config_supported(p.dtype, aligned_q, dstate))
    Qd = aligned_q;
  else if (cu_seqlens == nullptr && seqlen > 0)
    for (int q : {chunk_len, 256, 128, 64})
      if (seqlen % q == 0 && backward_dl_supported(p.dtype, q, dstate, nheads) && config_supported(p.dtype, q, dstate)) {
        Qd = q;
        break;
      }
  const bool cdl = Qd > 0;
  // dB and dC per chunk, summed over heads before the products with B and C
  // (then no role-exchanged passes and none of their per-head copies)
  const bool dbdc = cdl && backward_dbdc_supported(p.dtype, Qd, dstate);
  const bool bf16 = dtype == SSD_DTYPE_BF16;
  st = check_device();
  if (st != SSD_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);

  const int H = nheads, P = headdim, N = dstate, G = ngroups;
  const int NK = (N + 63) / 64, W = 64 * NK;
  const size_t T = (size_t)total_len, S = (size_t)nseqs, e = dtype == SSD_DTYPE_BF16 ? 2 : 4;
  // chunk slots of the d(ell) path's passed states (packed: the forward's bound)
  const size_t Kd = cdl ? (cu_seqlens ? T / Qd + S : T / Qd) : 0;
  const int nsub = dbdc ? backward_dbdc_subsets((int64_t)(T / Qd), G, H, N) : 0;
  const bool rx = !dbdc;                                // role-exchanged dB, dC passes
  const bool f32c = bf16 && !cdl;                       // fp32 copies of the inputs
  const bool fpass = !cdl;                              // fp32 recompute and reversed passes
  Carver cv;
  char* base = nullptr;
  auto take = [&](size_t bytes) { return cv.take(bytes); };
  // longest possible sequence: seqlen (batched), total_len (packed)
  const int64_t maxlen = cu_seqlens == nullptr ? seqlen : total_len;
  const int64_t nseg64 = std::max<int64_t>(1, (maxlen + kBwdScanSeg - 1) / kBwdScanSeg);
  if (nseqs * (int64_t)nheads * nseg64 > 0x7fffffffLL) return SSD_ERR_INVALID_ARGUMENT;
  const int nseg = (int)nseg64;
  BwdProblem b;
  b.nseg = nseg;
  float* part = nullptr;  // fp32 partial dC, dB of the head subsets
  auto layout = [&]() {
    cv.reset(base);
    b.xr = take(T * H * P * e);
    b.Br = take(T * G * N * e);
    b.Cr = take(T * G * N * e);
    b.dtr = reinterpret_cast<float*>(take(T * H * 4));
    b.xc = take(rx ? T * H * W * e : 0);
    b.xb = take(rx ? T * H * W * e : 0);
    b.dtc = reinterpret_cast<float*>(take(rx ? T * H * NK * 4 : 0));
    b.dtb = reinterpret_cast<float*>(take(rx ? T * H * NK * 4 : 0));
    b.Ac = reinterpret_cast<float*>(take(rx ? (size_t)H * NK * 4 : 0));
    b.cb = take(rx ? T * H * P * e : 0);
    b.h0c = reinterpret_cast<float*>(take(rx && initial_state ? S * H * NK * 4096 * 4 : 0));
    b.dfb = reinterpret_cast<float*>(take(rx && dfinal_state ? S * H * NK * 4096 * 4 : 0));
    b.x32 = reinterpret_cast<float*>(take(f32c ? T * H * P * 4 : 0));
    b.xr32 = reinterpret_cast<float*>(take(f32c ? T * H * P * 4 : 0));
    b.B32 = reinterpret_cast<float*>(take(f32c ? T * G * N * 4 : 0));
    b.C32 = reinterpret_cast<float*>(take(f32c ? T * G * N * 4 : 0));
    b.Br32 = reinterpret_cast<float*>(take(f32c ? T * G * N * 4 : 0));
    b.Cr32 = reinterpret_cast<float*>(take(f32c ? T * G * N * 4 : 0));
    b.y_f = reinterpret_cast<float*>(take(fpass ? T * H * P * 4 : 0));
    b.hlast = reinterpret_cast<float*>(take(fpass && dfinal_state ? S * H * P * N * 4 : 0));
    b.y_x = reinterpret_cast<float*>(take(fpass ? T * H * P * 4 : 0));
    b.y_x8 = take(cdl ? T * H * P * e : 0);
    b.hin_e = take(Kd * H * P * N * e);
    b.gin_e = take(Kd * H * P * N * e);
    b.acs_f = reinterpret_cast<float*>(take(Kd * H * (size_t)Qd * 4));
    b.dl_v = reinterpret_cast<float*>(take(cdl ? T * H * 4 : 0));
    b.dl_cols = reinterpret_cast<float*>(take(cdl ? 2 * T * H * 4 : 0));
    b.dl_u = reinterpret_cast<float*>(take(cdl ? T * H * 4 : 0));
    b.dl_kc = reinterpret_cast<float*>(take(Kd * H * 4));
    b.g0 = reinterpret_cast<float*>(take(dinitial_state ? S * H * P * N * 4 : 0));
    b.y_c = take(rx ? T * H * W * e : 0);
    b.y_b = take(rx ? T * H * W * e : 0);
    part = reinterpret_cast<float*>(take(nsub > 1 ? 2 * (size_t)nsub * T * G * N * 4 : 0));
    b.qd = reinterpret_cast<float*>(take(fpass ? T * H * 4 : 0));
    b.rd = reinterpret_cast<float*>(take(T * H * 4));
    b.ud = reinterpret_cast<float*>(take(T * H * 4));
    b.segsum = reinterpret_cast<double*>(take(fpass ? S * H * (size_t)nseg * 8 : 0));
    b.edot = reinterpret_cast<float*>(take(fpass ? S * H * 4 : 0));
  };
  layout();
  const size_t off = cv.off;
  if (g_dry) {
    base = kDryBase;
  } else {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    base = static_cast<char*>(ws_acquire(dev, off > 0 ? off : 256, s, 1));
    if (base == nullptr) return SSD_ERR_OUT_OF_MEMORY;
  }
  layout();
  if (!layout_ok(cv, off)) return g_dry ? SSD_OK : SSD_ERR_HIP;  // a layout defect: launch nothing
  if (g_dry) return SSD_OK;
  if (poison_workspace()) {
    const hipError_t pe = launch_fill_u32(reinterpret_cast<uint32_t*>(base), (int64_t)(off / 4), kPoisonNaN, s);
    if (pe != hipSuccess) return map_err(pe);
  }
  if (!initial_state) b.h0c = nullptr;
  if (!dfinal_state) b.dfb = nullptr, b.hlast = nullptr;
  if (!rx) b.xc = b.xb = b.cb = b.y_c = b.y_b = nullptr, b.dtc = b.dtb = b.Ac = b.h0c = b.dfb = nullptr;
  if (nsub <= 1) part = nullptr;
  if (!dinitial_state) b.g0 = nullptr;
  b.x = x; b.dt = dt; b.A = A_head; b.B = B; b.C = C; b.cu = cu_seqlens; b.h0 = initial_state;
  b.dy = dy; b.dfinal = dfinal_state; b.D = D; b.x_times_dt = x_times_dt;
  b.dx = dx; b.ddt = ddt; b.dA = dA; b.dB = dB; b.dC = dC; b.dD = dD; b.dinit = dinitial_state;
  b.nseq = nseqs; b.seqlen = seqlen; b.total = total_len;
  b.H = H; b.P = P; b.N = N; b.G = G; b.NK = NK; b.dtype = p.dtype;
  b.chunked_dl = cdl; b.Q = Qd;
  if (!bf16) {
    b.x32 = static_cast<const float*>(x);
    b.B32 = static_cast<const float*>(B);
    b.C32 = static_cast<const float*>(C);
    b.xr32 = static_cast<const float*>(b.xr);
    b.Br32 = static_cast<const float*>(b.Br);
    b.Cr32 = static_cast<const float*>(b.Cr);
  }

  hipError_t err = timed_launch(kK7BackwardGlue, s, [&] { return launch_backward_glue(b, 0, s); });
  if (err != hipSuccess) return map_err(err);
  if (nseqs == 0) return SSD_OK;
  if (cdl) {
    // passed states of the forward (fp32 copies of the stored values)
    Problem pf = make_problem(x, dt, A_head, B, C, cu_seqlens, nseqs, seqlen, total_len, H, P, N, G, Qd, dtype,
                              dx, nullptr, initial_state, nullptr, x_times_dt);
    // reversed pass in the element dtype: dx' (own terms in), its passed states
    // (the adjoint after each chunk) and G_first
    Problem px = make_problem(b.xr, b.dtr, A_head, b.Br, b.Cr, cu_seqlens, nseqs, seqlen, total_len, H, P, N, G,
                              Qd, dtype, const_cast<void*>(b.y_x8), b.g0, dfinal_state, nullptr, 0);
    Problem pc = make_problem(b.xc, b.dtc, b.Ac, x, dy, nullptr, nseqs, seqlen, total_len, H * NK, kHeadDim, P,
                              H, Q2, dtype, b.y_c, nullptr, b.h0c, nullptr, x_times_dt);
    Problem pb = make_problem(b.xb, b.dtb, b.Ac, b.xr, b.cb, nullptr, nseqs, seqlen, total_len, H * NK,
                              kHeadDim, P, H, Q2, dtype, b.y_b, nullptr, b.dfb, nullptr, 0);
    DebugOut df, dxo;
    df.hin_buf = const_cast<void*>(b.hin_e);
    df.acs_buf = const_cast<float*>(b.acs_f);  // read by the d(ell) and dB/dC kernels
    df.states_only = true;
    dxo.hin_buf = const_cast<void*>(b.gin_e);
    for (auto [q, d] : {std::pair<const Problem*, const DebugOut*>{&pf, &df}, {&px, &dxo}, {&pc, nullptr},
                        {&pb, nullptr}}) {
      if (!rx && (q == &pc || q == &pb)) continue;
      st = run(*q, s, d);
      if (st != SSD_OK) return st;
    }
    if (dbdc) {
      err = timed_launch(kK7BackwardGlue, s, [&] { return launch_backward_dbdc(b, part, nsub, s); });
      if (err != hipSuccess) return map_err(err);
    }
    return map_err(timed_launch(kK7BackwardGlue, s, [&] { return launch_backward_glue(b, 1, s); }));
  }
  // forward recompute (fp32): y without the skip term and the own terms, final state
  Problem pf = make_problem(b.x32, dt, A_head, b.B32, b.C32, cu_seqlens, nseqs, seqlen, total_len, H, P, N,
                            G, Qf, SSD_DTYPE_F32, b.y_f, b.hlast, initial_state, nullptr, x_times_dt, 1);
  // dx' (fp32) without the own terms: reversed in time, decays shifted, from dfinal
  Problem px = make_problem(b.xr32, b.dtr, A_head, b.Br32, b.Cr32, cu_seqlens, nseqs, seqlen, total_len, H,
                            P, N, G, Qf, SSD_DTYPE_F32, b.y_x, b.g0, dfinal_state, nullptr, 0, 1);
  // dC: x and B exchanged (per-head copies of B as the input), from h0^T
  Problem pc = make_problem(b.xc, b.dtc, b.Ac, x, dy, cu_seqlens, nseqs, seqlen, total_len, H * NK,
                            kHeadDim, P, H, Q2, dtype, b.y_c, nullptr, b.h0c, nullptr, x_times_dt);
  // dB: as dC, reversed in time, from dfinal^T
  Problem pb = make_problem(b.xb, b.dtb, b.Ac, b.xr, b.cb, cu_seqlens, nseqs, seqlen, total_len, H * NK,
                            kHeadDim, P, H, Q2, dtype, b.y_b, nullptr, b.dfb, nullptr, 0);
  for (const Problem* q : {&pf, &px, &pc, &pb}) {
    st = run(*q, s, nullptr);
    if (st != SSD_OK) return st;
  }
  return map_err(timed_launch(kK7BackwardGlue, s, [&] { return launch_backward_glue(b, 1, s); }));
}

// bf16 sequences that are not whole numbers of chunks (packed, or batched
// with a length no built chunk length divides) take the chunk-local path
// through a padded copy: each sequence is padded on the device to a whole number of chunks (dt = 0, zero
// x, dy, B, C: decay 1, no input, no output, so every gradient and the final
// state are unchanged), one zero sequence fills the rest of the host's bound
// on the padded length, and the results are copied back.  The bound needs no
// host read of cu_seqlens: T + S (Q - 1).  Used when that at most doubles the
// tokens and the configuration is built.
static int padded_bwd_chunk(const int32_t* cu_seqlens, int64_t nseqs, int64_t total_len, int32_t nheads,
                            int32_t dstate, int32_t ngroups, int32_t chunk_len, ssd_dtype dtype) {
  if (total_len <= 0 || nseqs <= 0 || dtype != SSD_DTYPE_BF16 || ngroups > kMaxBwdGroups) return 0;
  if (cu_seqlens == nullptr) {
    // batched: only when no built chunk length divides the sequence length
    if (total_len % nseqs != 0) return 0;
    const int64_t seqlen = total_len / nseqs;
    for (int q : {chunk_len, 256, 128, 64})
      if (seqlen % q == 0 && backward_dl_supported(Dtype::BF16, q, dstate, nheads) && config_supported(Dtype::BF16, q, dstate))
        return 0;
  }
  for (int q : {chunk_len, 256, 128, 64}) {
    if (q != 64 && q != 128 && q != 256) continue;
    const int64_t tp = (total_len + nseqs * (int64_t)(q - 1) + q - 1) / q * q;
    if (nseqs * (int64_t)(q - 1) <= total_len && tp < 0x7fffffffLL && backward_dl_supported(Dtype::BF16, q, dstate, nheads) &&
        backward_dbdc_supported(Dtype::BF16, q, dstate) && config_supported(Dtype::BF16, q, dstate))
      return q;
  }
  return 0;
}

ssd_status ssd_chunked_bwd(const void* x, const float* dt, const float* A_head, const void* B,
                           const void* C, const int32_t* cu_seqlens, int64_t nseqs,
                           int64_t total_len, int32_t nheads, int32_t headdim, int32_t dstate,
                           int32_t ngroups, int32_t chunk_len, ssd_dtype dtype,
                           const float* initial_state, const float* D, int32_t x_times_dt,
                           const void* dy, const float* dfinal_state, void* dx, float* ddt,
                           float* dA, void* dB, void* dC, float* dD, float* dinitial_state,
                           void* stream) {
  const int Qp = padded_bwd_chunk(cu_seqlens, nseqs, total_len, nheads, dstate, ngroups, chunk_len, dtype);
  if (Qp == 0)
    return bwd_impl(x, dt, A_head, B, C, cu_seqlens, nseqs, total_len, nheads, headdim, dstate, ngroups, chunk_len,
                    dtype, initial_state, D, x_times_dt, dy, dfinal_state, dx, ddt, dA, dB, dC, dD, dinitial_state,
                    stream, 0);
  // the caller's arguments are checked as for the unpadded call
  {
    Problem p = make_problem(x, dt, A_head, B, C, cu_seqlens, nseqs, cu_seqlens ? 0 : total_len / nseqs, total_len,
                             nheads, headdim, dstate, ngroups, chunk_len, dtype, dx, nullptr, initial_state, D,
                             x_times_dt);
    ssd_status st = validate(p);
    if (st != SSD_OK) return st;
    if (dA == nullptr || !aligned(dA, 4) || (dD && !aligned(dD, 4))) return SSD_ERR_INVALID_ARGUMENT;
    if ((dfinal_state && !aligned(dfinal_state, 16)) || (dinitial_state && !aligned(dinitial_state, 16)))
      return SSD_ERR_INVALID_ARGUMENT;
    if (!dy || !ddt || !dB || !dC || !aligned(dy, 16) || !aligned(dB, 16) || !aligned(dC, 16) || !aligned(ddt, 4))
      return SSD_ERR_INVALID_ARGUMENT;
    st = check_device();
    if (st != SSD_OK) return st;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t S = nseqs, T = total_len, S1 = nseqs + 1;
  const int64_t Tp = (T + S * (Qp - 1) + Qp - 1) / Qp * Qp;
  const size_t H = nheads, P = headdim, N = dstate, G = ngroups, PN = P * N;
  Carver cv;
  char* base = nullptr;
  auto take = [&](size_t bytes) { return cv.take(bytes); };
  PadArgs a;
  float *h0p = nullptr, *dfp = nullptr, *dinitp = nullptr;
  auto layout = [&]() {
    cv.reset(base);
    a.cup = reinterpret_cast<int32_t*>(take((size_t)(S + 2) * 4));
    a.xp = take(Tp * H * P * 2);
    a.dyp = take(Tp * H * P * 2);
    a.Bp = take(Tp * G * N * 2);
    a.Cp = take(Tp * G * N * 2);
    a.dtp = reinterpret_cast<float*>(take(Tp * H * 4));
    a.dxp = take(Tp * H * P * 2);
    a.dBp = take(Tp * G * N * 2);
    a.dCp = take(Tp * G * N * 2);
    a.ddtp = reinterpret_cast<float*>(take(Tp * H * 4));
    h0p = reinterpret_cast<float*>(take(initial_state ? S1 * H * PN * 4 : 0));
    dfp = reinterpret_cast<float*>(take(dfinal_state ? S1 * H * PN * 4 : 0));
    dinitp = reinterpret_cast<float*>(take(dinitial_state ? S1 * H * PN * 4 : 0));
  };
  layout();
  const size_t off = cv.off;
  if (g_dry) {
    base = kDryBase;
  } else {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    base = static_cast<char*>(ws_acquire(dev, off, s, 2));
    if (base == nullptr) return SSD_ERR_OUT_OF_MEMORY;
  }
  layout();  // absent optional arrays are zero-byte pieces: null pointers
  if (!layout_ok(cv, off)) return g_dry ? SSD_OK : SSD_ERR_HIP;  // a layout defect: launch nothing
  a.cu = cu_seqlens;
  a.S = S; a.T = T; a.Tp = Tp; a.seqlen = cu_seqlens ? 0 : T / S;
  a.H = nheads; a.P = headdim; a.G = ngroups; a.N = dstate; a.Q = Qp;
  a.dtype = Dtype::BF16;
  a.x = x; a.dt = dt; a.B = B; a.C = C; a.dy = dy;
  a.dx = dx; a.ddt = ddt; a.dB = dB; a.dC = dC;
  if (!g_dry && poison_workspace()) {
    const hipError_t pe = launch_fill_u32(reinterpret_cast<uint32_t*>(base), (int64_t)(off / 4), kPoisonNaN, s);
    if (pe != hipSuccess) return map_err(pe);
  }
  if (g_dry)  // the padded pass's own layout only: its inputs are fakes too
    return bwd_impl(a.xp, a.dtp, A_head, a.Bp, a.Cp, a.cup, S1, Tp, nheads, headdim, dstate, ngroups, Qp, dtype, h0p,
                    D, x_times_dt, a.dyp, dfp, const_cast<void*>(a.dxp), const_cast<float*>(a.ddtp), dA,
                    const_cast<void*>(a.dBp), const_cast<void*>(a.dCp), dD, dinitp, stream, Qp);
  hipError_t err = timed_launch(kK7BackwardGlue, s, [&] { return launch_backward_pad(a, 0, s); });
  if (err != hipSuccess) return map_err(err);
  // per-sequence states with a zero entry for the filling sequence
  for (auto [src, dst] : {std::pair<const float*, float*>{initial_state, h0p}, {dfinal_state, dfp}}) {
    if (src == nullptr) continue;
    if (hipMemcpyAsync(dst, src, S * H * PN * 4, hipMemcpyDeviceToDevice, s) != hipSuccess) return SSD_ERR_HIP;
    err = launch_fill_zero(dst + S * H * PN, H * PN, s);
    if (err != hipSuccess) return map_err(err);
  }
  ssd_status st = bwd_impl(a.xp, a.dtp, A_head, a.Bp, a.Cp, a.cup, S1, Tp, nheads, headdim, dstate, ngroups, Qp,
                           dtype, h0p, D, x_times_dt, a.dyp, dfp, const_cast<void*>(a.dxp),
                           const_cast<float*>(a.ddtp), dA, const_cast<void*>(a.dBp), const_cast<void*>(a.dCp), dD,
                           dinitp, stream, Qp);
  if (st != SSD_OK) return st;
  err = timed_launch(kK7BackwardGlue, s, [&] { return launch_backward_pad(a, 1, s); });
  if (err != hipSuccess) return map_err(err);
  if (dinitial_state &&
      hipMemcpyAsync(dinitial_state, dinitp, S * H * PN * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return SSD_ERR_HIP;
  return SSD_OK;
}

const char* ssd_status_string(ssd_status status) {
  switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_INVALID_ARGUMENT: return "SSD_ERR_INVALID_ARGUMENT";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
    case SSD_ERR_OUT_OF_MEMORY: return "SSD_ERR_OUT_OF_MEMORY";
    case SSD_ERR_SCRATCH_LIMIT: return "SSD_ERR_SCRATCH_LIMIT";
  }
  return "SSD_ERR_UNKNOWN";
}

int32_t ssd_workspace_selfcheck(void) { return workspace_selfcheck(); }

ssd_status ssd_kernel_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_timing = enable != 0;
  return SSD_OK;
}

ssd_status ssd_kernel_timing_read(int32_t kernel, double* total_ms, int64_t* launches,
                                  int32_t reset) {
  if (kernel < 0 || kernel >= kNumKernels) return SSD_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(g_mu);
  ssd_status st = SSD_OK;
  for (auto& t : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess)
      st = SSD_ERR_HIP;
    g_total_ms[t.kernel] += ms;
    g_launches[t.kernel] += 1;
    g_free_events.push_back(t.start);
    g_free_events.push_back(t.stop);
  }
  g_pending.clear();
  if (total_ms) *total_ms = g_total_ms[kernel];
  if (launches) *launches = g_launches[kernel];
  if (reset) {
    g_total_ms[kernel] = 0.0;
    g_launches[kernel] = 0;
  }
  return st;
}

}  // extern "C"

namespace ssd {

int workspace_selfcheck() {
  g_dry = true;
  g_dry_bad = 0;
  int bad = 0;
  // fake, aligned, never dereferenced: the dry run launches nothing
  void* const F = reinterpret_cast<void*>((uintptr_t)1 << 32);
  float* const Ff = static_cast<float*>(F);
  const int32_t* const Fi = static_cast<const int32_t*>(F);
  // every call must return SSD_OK after carving (and checking) at least one workspace
  auto expect_ok = [&](ssd_status st) {
    static thread_local int64_t seen = 0;
    if (st != SSD_OK || g_dry_checks <= seen) ++bad;
    seen = g_dry_checks;
  };
  for (ssd_dtype dt : {SSD_DTYPE_F32, SSD_DTYPE_BF16})
    for (int Q : {64, 128, 256})
      for (int N : {16, 32, 64, 128, 256})
        for (int64_t T : {(int64_t)1, (int64_t)300, (int64_t)1024})
          for (auto hg : {std::pair<int, int>{4, 1}, {8, 2}}) {
            const int H = hg.first, G = hg.second;
            const int64_t b = 3;
            expect_ok(ssd_chunked_fwd(F, Ff, Ff, F, F, b, T, H, 64, N, G, Q, dt, F, Ff, nullptr));
            expect_ok(ssd_chunked_fwd_noalloc(F, Ff, Ff, F, F, b, T, H, 64, N, G, Q, dt, F, nullptr, nullptr));
            expect_ok(ssd_chunked_fwd_varlen(F, Ff, Ff, F, F, Fi, 5, b * T, H, 64, N, G, Q, dt, F, Ff, nullptr));
            for (int opt = 0; opt < 4; ++opt) {
              const float* Dp = (opt & 1) ? Ff : nullptr;
              const int xdt = (opt >> 1) & 1;
              expect_ok(ssd_chunked_fwd_ex(F, Ff, Ff, F, F, nullptr, b, b * T, H, 64, N, G, Q, dt, Ff, Dp, xdt, F,
                                           Ff, nullptr));
              expect_ok(ssd_chunked_fwd_ex(F, Ff, Ff, F, F, Fi, 5, b * T, H, 64, N, G, Q, dt, nullptr, Dp, xdt, F,
                                           Ff, nullptr));
              expect_ok(ssd_chunked_fwd_normalized(F, Ff, Ff, F, F, (opt & 2) ? Fi : nullptr, (opt & 2) ? 5 : b,
                                                   b * T, H, 64, N, G, Q, dt, Dp, xdt, F, Ff, Ff, nullptr));
              for (int opt2 = 0; opt2 < 4; ++opt2) {
                const float* h0 = (opt2 & 1) ? Ff : nullptr;
                const float* dfin = (opt2 & 2) ? Ff : nullptr;
                float* dD = (opt & 1) ? Ff : nullptr;
                float* dinit = (opt2 & 1) ? Ff : nullptr;
                // batched (whole chunks when T % Q == 0, else ragged) and packed
                expect_ok(ssd_chunked_bwd(F, Ff, Ff, F, F, nullptr, b, b * T, H, 64, N, G, Q, dt, h0, Dp, xdt, F,
                                          dfin, F, Ff, Ff, F, F, dD, dinit, nullptr));
                expect_ok(ssd_chunked_bwd(F, Ff, Ff, F, F, Fi, 5, b * T, H, 64, N, G, Q, dt, h0, Dp, xdt, F, dfin,
                                          F, Ff, Ff, F, F, dD, dinit, nullptr));
              }
            }
          }
  g_dry = false;
  return bad + g_dry_bad;
}

}  // namespace ssd
