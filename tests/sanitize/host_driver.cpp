// host_driver.cpp -- the host logic of libssd.so (csrc/ssd_api.cpp: argument
// validation, workspace carving and its check) built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side (tests/test_host_sanitizers.py
// builds it; the kernels are linked unchanged and never launched).  Checks the
// carver on hand-made logs, runs the workspace layout self-check (every entry
// point that takes a workspace, dry, over a grid of shapes and options) and
// calls every entry point with invalid arguments, which must be refused on the
// host.  No GPU is used.  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>

#include "ssd.h"
#include "ssd_internal.hpp"

int main() {
  int bad = 0;
  auto expect = [&](bool ok, const char* what) {
    if (!ok) {
      ++bad;
      printf("FAILED: %s\n", what);
    }
  };
  // ---- the carver
  {
    ssd::Carver c;
    c.reset(reinterpret_cast<char*>(4096));
    expect(c.take(0) == nullptr, "a zero-byte piece is null");
    char* a = c.take(100);
    expect(a == reinterpret_cast<char*>(4096), "first piece at the base");
    expect(c.take(0) == nullptr, "a zero-byte piece between others is null");
    char* b = c.take(300);
    expect(b == reinterpret_cast<char*>(4096 + 256), "pieces 256-byte aligned");
    expect(c.off == 768, "carved size");
    expect(c.check(556), "pieces inside their allocation pass");
    expect(!c.check(555), "a piece past the allocation fails");
    ssd::Carver o;
    o.reset(nullptr);
    o.take(512);
    o.take(512);
    o.at[1] = 256;  // a hand-made overlap
    expect(!o.check(1 << 20), "overlapping pieces fail");
    ssd::Carver f;
    f.reset(nullptr);
    for (int i = 0; i < ssd::Carver::kMaxPieces + 1; ++i) f.take(16);
    expect(!f.check((size_t)1 << 30), "a log overflow fails");
  }
  // ---- every workspace layout of every entry point, dry
  expect(ssd_workspace_selfcheck() == 0, "workspace layout self-check");
  // ---- invalid arguments are refused before any HIP call
  void* const F = reinterpret_cast<void*>((uintptr_t)1 << 20);
  float* const Ff = static_cast<float*>(F);
  const int32_t* const Fi = static_cast<const int32_t*>(F);
  char* const mis = static_cast<char*>(F) + 4;
  expect(ssd_chunked_fwd(F, Ff, Ff, F, F, 1, 256, 3, 64, 128, 2, 256, SSD_DTYPE_BF16, F, nullptr, nullptr) ==
             SSD_ERR_INVALID_ARGUMENT, "fwd: H % G");
  expect(ssd_chunked_fwd(mis, Ff, Ff, F, F, 1, 256, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, F, nullptr, nullptr) ==
             SSD_ERR_INVALID_ARGUMENT, "fwd: misaligned x");
  expect(ssd_chunked_fwd(F, Ff, Ff, F, F, 1, 256, 4, 64, 48, 1, 256, SSD_DTYPE_BF16, F, nullptr, nullptr) ==
             SSD_ERR_UNSUPPORTED, "fwd: dstate 48");
  expect(ssd_chunked_fwd(F, Ff, Ff, F, F, (int64_t)1 << 31, 2, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, F, nullptr,
                         nullptr) == SSD_ERR_INVALID_ARGUMENT, "fwd: too many sequences");
  expect(ssd_chunked_fwd_noalloc(F, Ff, Ff, F, F, 1, 1 << 16, 32, 64, 128, 1, 256, SSD_DTYPE_BF16, F, nullptr,
                                 nullptr) == SSD_ERR_SCRATCH_LIMIT, "noalloc: past its scratch");
  expect(ssd_chunked_fwd_varlen(F, Ff, Ff, F, F, nullptr, 2, 100, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, F, nullptr,
                                nullptr) == SSD_ERR_INVALID_ARGUMENT, "varlen: null cu_seqlens");
  expect(ssd_chunked_fwd_ex(F, Ff, Ff, F, F, nullptr, 3, 512, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, nullptr, nullptr,
                            0, F, Ff, nullptr) == SSD_ERR_INVALID_ARGUMENT, "ex: total_len % nseqs");
  expect(ssd_chunked_fwd_ex(F, Ff, Ff, F, F, nullptr, 2, 512, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, nullptr, nullptr,
                            2, F, Ff, nullptr) == SSD_ERR_INVALID_ARGUMENT, "ex: x_times_dt flag");
  expect(ssd_chunked_fwd_normalized(F, Ff, Ff, F, F, nullptr, 2, 512, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, nullptr,
                                    0, F, nullptr, nullptr, nullptr) == SSD_ERR_INVALID_ARGUMENT,
         "normalized: no denominator buffer");
  expect(ssd_chunked_bwd(F, Ff, Ff, F, F, nullptr, 2, 512, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, nullptr, nullptr, 0,
                         F, nullptr, F, Ff, nullptr, F, F, nullptr, nullptr, nullptr) == SSD_ERR_INVALID_ARGUMENT,
         "bwd: no dA");
  expect(ssd_chunked_bwd(F, Ff, Ff, F, F, Fi, 2, 512, 4, 64, 128, 1, 256, SSD_DTYPE_BF16, nullptr, nullptr, 0, F,
                         nullptr, F, Ff, Ff, F, mis, nullptr, nullptr, nullptr) == SSD_ERR_INVALID_ARGUMENT,
         "bwd: misaligned dC");
  expect(ssd_decode_step(F, Ff, Ff, F, F, 4, 6, 64, 128, 4, SSD_DTYPE_BF16, nullptr, 0, Ff, F, nullptr) ==
             SSD_ERR_INVALID_ARGUMENT, "decode: H % G");
  expect(ssd_selective_scan(F, Ff, Ff, F, F, 2, 512, 256, 100, SSD_DTYPE_BF16, F, nullptr, nullptr) ==
             SSD_ERR_UNSUPPORTED, "scan: dstate 100");
  expect(ssd_kernel_timing_read(99, nullptr, nullptr, 0) == SSD_ERR_INVALID_ARGUMENT, "timing: kernel id");
  printf("host driver: %d failed checks\n", bad);
  return bad ? 1 : 0;
}
