"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The fp64 oracle (oracle/ssd_oracle.c) with gcc, driven by
  tests/sanitize/oracle_driver.c on small packed inputs and invalid arguments.
- The library's host logic (csrc/ssd_api.cpp: validation, workspace carving and
  its check) with hipcc, sanitizers on the host side only (each -fsanitize= put
  after -Xarch_host), linked with the unchanged kernel objects, driven by
  tests/sanitize/host_driver.cpp; no kernel is launched.
Each driver exits 0 when its checks hold; a sanitizer report fails it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "mamba_ssd_layer_amd")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert "0 failed checks" in r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_host_logic_under_asan_ubsan(tmp_path):
    from mamba_ssd_layer_amd import build as b

    def kernel_objects():
        # the objects build.py makes, one per kernel source (not any other file
        # a build with --asm leaves in the folder)
        names = [os.path.basename(src) + ".o" for src in b.sources() if not os.path.basename(src).startswith("ssd_api")]
        return [os.path.join(b.BUILD, n) for n in names if os.path.exists(os.path.join(b.BUILD, n))]

    objs = kernel_objects()
    if len(objs) < len(b.sources()) - 1:
        b.build()
        objs = kernel_objects()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={b.ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    api = str(tmp_path / "ssd_api_san.o")
    drv = str(tmp_path / "host_driver.o")
    exe = str(tmp_path / "host_driver")
    _run([b.HIPCC, "-x", "hip", *flags, *san, "-c", os.path.join(PKG, "csrc", "ssd_api.cpp"), "-o", api])
    _run([b.HIPCC, "-x", "hip", *flags, *san, "-c", os.path.join(SAN, "host_driver.cpp"), "-o", drv])
    _run([b.HIPCC, f"--offload-arch={b.ARCH}", *san, drv, api, *objs, "-o", exe])
    r = _run([exe], env=ENV)
    assert "0 failed checks" in r.stdout
