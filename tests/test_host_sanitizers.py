"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

`fa_api.cpp` is compiled with both sanitizers on its host side only (the
kernel objects are the ordinary ones) and linked into a small driver that
calls every entry point with arguments each check must reject, including
sizes at INT_MAX where 32-bit arithmetic would overflow, plus the size and
split-policy helpers over their whole input range. Nothing reaches a kernel
launch or a device query, so this runs without a GPU. Any out-of-bounds
access, signed overflow or other undefined behaviour aborts the driver, and
a status that differs from the expected one fails it.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_online_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
KERNELS = ["fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fp8.hip"]
COMMON = ["-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

DRIVER = r"""
#include <climits>
#include <cmath>
#include <cstdio>
#include "fa.h"

static int fails = 0;
#define EXPECT(expr, want)                                                                      \
  do {                                                                                          \
    const long long got_ = (long long)(expr);                                                   \
    if (got_ != (long long)(want)) {                                                            \
      std::fprintf(stderr, "line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_, (long long)(want)); \
      ++fails;                                                                                  \
    }                                                                                           \
  } while (0)

int main() {
  // never dereferenced: every call below is rejected, or is a no-op, before any launch
  void* P = (void*)64;
  float* F = (float*)64;
  const int32_t* I = (const int32_t*)64;
  uint8_t* U = (uint8_t*)64;
  const int M = INT_MAX;
  const float nan = std::nanf("");
  const int OK = FA_OK, INV = FA_ERR_INVALID_ARG, UNS = FA_ERR_UNSUPPORTED, WS = FA_ERR_WORKSPACE;

  EXPECT(fa_abi_version(), 2);
  for (int s = -3; s < 8; ++s) EXPECT(fa_status_string(s) != nullptr, 1);

  // fa_fwd
  EXPECT(fa_fwd(P, P, P, P, F, 1, 6, 4, 8, 8, 128, 0, 0.1f, FA_DTYPE_BF16, nullptr), INV);
  EXPECT(fa_fwd(P, P, P, P, F, -1, 4, 2, 8, 8, 128, 0, 0.1f, 0, nullptr), INV);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 2, 8, 8, 128, 2, 0.1f, 0, nullptr), INV);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 2, 8, 8, 128, 0, nan, 0, nullptr), INV);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 2, 8, 8, 128, 0, INFINITY, 0, nullptr), INV);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 2, 8, 8, 96, 0, 0.1f, 0, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 2, 8, 8, 128, 0, 0.1f, 7, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, M, M, M, M, M, M, 1, 0.1f, 0, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 1, 1, M, M, 128, 1, 0.1f, 0, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 1, 1, 8, M - 100, 128, 1, 0.1f, 0, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, 65535, 65535, 1, M, M, 128, 1, 0.1f, 0, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, M, M, 1, M - 2048, 8, 128, 1, 0.1f, 0, nullptr), UNS);
  EXPECT(fa_fwd_window(P, P, P, P, F, M, M, 1, M - 2048, 8, 128, -1, 0, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd_varlen(P, P, P, P, F, I, I, M, M, 1, M - 2048, 8, 8, 128, -1, 0, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, 2, 1, 1, (1 << 30) + 64, 8, 128, 1, 0.1f, 0, nullptr), UNS);
  EXPECT(fa_fwd(P, P, P, P, F, 0, 4, 2, 8, 8, 128, 0, 0.1f, 0, nullptr), OK);
  EXPECT(fa_fwd(nullptr, P, P, P, F, 1, 4, 2, 8, 8, 128, 0, 0.1f, 0, nullptr), INV);

  // windows and packed batches
  EXPECT(fa_fwd_window(P, P, P, P, F, 1, 1, 1, M, M, 128, -1, 0, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd_window(P, P, P, P, F, 1, 3, 2, 8, 8, 128, -1, 0, 0.1f, nullptr), INV);
  EXPECT(fa_fwd_varlen(P, P, P, P, F, I, I, 1, 1, 1, M, M, M, 128, -1, 0, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd_varlen(P, P, P, P, F, I, I, 1, 1, 1, 8, M, 8, 128, -1, 0, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd_varlen(P, P, P, P, F, nullptr, I, 1, 1, 1, 8, 8, 8, 128, -1, 0, 0.1f, nullptr), INV);

  // decode
  EXPECT(fa_fwd_kvcache(P, P, P, I, P, F, 2, 2, 8, 2, M, 128, 0.1f, P, (size_t)1 << 30, nullptr), UNS);
  EXPECT(fa_fwd_kvcache(P, P, P, I, P, F, 0, 2, 8, 2, 256, 128, 0.1f, P, (size_t)1 << 30, nullptr), INV);
  EXPECT(fa_fwd_kvcache(P, P, P, I, P, F, 4, 2, 8, 2, 256, 128, 0.1f, P, 100, nullptr), WS);
  EXPECT(fa_fwd_kvcache(P, P, P, I, P, F, 4, 2, 64, 2, 256, 128, 0.1f, P, (size_t)1 << 30, nullptr), UNS);
  EXPECT(fa_fwd_kvcache(P, P, P, I, P, F, M, M, M, M, M, 128, 0.1f, P, (size_t)-1, nullptr), UNS);
  EXPECT(fa_fwd_kvcache(P, P, P, I, P, F, 4, 0, 8, 2, 256, 128, 0.1f, nullptr, 0, nullptr), OK);
  EXPECT(fa_fwd_kvcache_noalloc(P, P, P, I, P, F, 4, 2, 8, 2, M, 128, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd_kvcache_noalloc(P, P, P, I, P, F, 0, 2, 8, 2, 256, 128, 0.1f, nullptr), INV);
  EXPECT(fa_fwd_kvcache_noalloc(P, P, P, I, P, F, 64, 4096, 64, 8, 256, 256, 0.1f, nullptr), WS);
  EXPECT(fa_fwd_kvcache_paged(P, P, P, I, I, P, F, 2, 2, 8, 2, 1 << 16, 1 << 16, 4, 128, 0.1f, P,
                              (size_t)1 << 30, nullptr), UNS);
  EXPECT(fa_fwd_kvcache_paged(P, P, P, I, I, P, F, 2, 2, 8, 2, 1 << 30, 2, M, 128, 0.1f, P, (size_t)1 << 30, nullptr),
         UNS);
  EXPECT(fa_fwd_kvcache_paged(P, P, P, I, I, P, F, 2, 2, 8, 2, M, M, M, 128, 0.1f, P, (size_t)1 << 30, nullptr),
         INV);  // pages must be whole 64-key tiles
  EXPECT(fa_fwd_kvcache_append(P, P, P, P, P, I, P, F, 1, 2, 2, M, 8, 2, 256, 128, 0.1f, P, (size_t)1 << 30, nullptr),
         UNS);
  EXPECT(fa_fwd_kvcache_append(P, P, P, P, P, I, P, F, 1, 2, 2, 4, 8, 2, M - 10, 128, 0.1f, P, (size_t)1 << 30,
                               nullptr), UNS);
  EXPECT(fa_fwd_kvcache_paged_append(P, P, P, P, P, I, I, P, F, 1, 2, 2, 4, 8, 2, 1 << 30, 2, M, 128, 0.1f, P,
                                     (size_t)1 << 30, nullptr), UNS);

  // size and split helpers over their whole range: defined results, no overflow
  EXPECT(fa_fwd_kvcache_workspace_size(2, 8, 128, 4), (long long)2 * 8 * 4 * 129 * 4);
  EXPECT(fa_fwd_kvcache_workspace_size(0, 8, 128, 4), 0);
  EXPECT(fa_fwd_kvcache_workspace_size(M, M, 256, 1), 0);
  (void)fa_fwd_kvcache_workspace_size(65535, 65535, 256, 65535);
  EXPECT(fa_kvcache_default_splits(64, 8, 8192, 128, 256, 2), 2);
  EXPECT(fa_kvcache_default_splits(M, M, M, 128, 256, 2), 1);
  const int big[] = {1, 2, 63, 64, 65, 1 << 20, M - 1024, M - 1, M};
  for (int a : big)
    for (int c : big) {
      EXPECT(fa_kvcache_default_splits(a, 1, c, 128, M, M) >= 1, 1);
      EXPECT(fa_kvcache_default_splits(1, a, c, 64, 1, 1) >= 1, 1);
      EXPECT(fa_kvcache_default_splits(a, a, c, 256, c, a) >= 1, 1);
      EXPECT(fa_kvcache_append_default_splits(a, a, 1, 16, c, 128, M, M) >= 1, 1);
      EXPECT(fa_kvcache_append_default_splits(1, a, a, a, c, 128, 1, 1) >= 1, 1);
      EXPECT(fa_kvcache_append_default_splits(a, 1, a, a, c, 64, c, a) >= 1, 1);
    }
  EXPECT(fa_bwd_workspace_size(2, 3, 33), 2 * 2 * 3 * 64 * 4);
  (void)fa_bwd_workspace_size(M, M, M);
  EXPECT(fa_fp8_padded_rows(65), 128);
  EXPECT(fa_fp8_padded_rows(0), 0);
  EXPECT(fa_fp8_padded_rows(M), 0);
  EXPECT(fa_fp8_padded_rows(M - 1024), (long long)(M - 1024 + 63) / 64 * 64);

  // backward
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, 1, 1, 1, M, M, 128, 1, 0.1f, P, (size_t)1 << 30, nullptr), UNS);
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, 2, 1, 1, 64, (1 << 30) + 64, 128, 1, 0.1f, P, (size_t)1 << 30, nullptr),
         UNS);
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, M, M, M, M, M, M, 1, 0.1f, P, (size_t)-1, nullptr), UNS);
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, M, M, 1, M - 2048, M - 2048, 128, 1, 0.1f, P, (size_t)-1, nullptr), UNS);
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, 1, 4, 2, 64, 64, 128, 1, 0.1f, P, 8, nullptr), WS);
  EXPECT(fa_bwd_window(P, P, P, P, F, P, P, P, P, 1, 1, 1, M - 512, 64, 128, -1, 0, 0.1f, P, (size_t)1 << 30, nullptr),
         UNS);
  EXPECT(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, I, I, 1, 1, 1, 64, 64, M, 64, 128, -1, 0, 0.1f, P, (size_t)1 << 30,
                       nullptr), UNS);
  EXPECT(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, nullptr, I, 1, 1, 1, 64, 64, 64, 64, 128, -1, 0, 0.1f, P,
                       (size_t)1 << 30, nullptr), INV);

  // FP8
  EXPECT(fa_quantize_fp8(P, nullptr, P, U, 0, 1, M, 1, 128, nullptr), UNS);
  EXPECT(fa_quantize_fp8(P, nullptr, P, U, 2, 1, 10, 1, 128, nullptr), INV);
  EXPECT(fa_quantize_fp8(P, nullptr, P, U, 0, M, 10, M, 128, nullptr), UNS);
  EXPECT(fa_fwd_fp8(P, U, P, U, P, U, P, F, 1, 1, 1, M, 64, 128, 1, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd_fp8(P, U, P, U, P, U, P, F, 1, 1, 1, 64, M, 128, 1, 0.1f, nullptr), UNS);
  EXPECT(fa_fwd_fp8(P, U, P, U, P, U, P, F, M, M, M, M - 200, 64, 128, 1, 0.1f, nullptr), UNS);

  if (fails) return 1;
  std::puts("ok");
  return 0;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd[:6]), r.stdout[-2000:], r.stderr[-4000:])
    return r


@pytest.mark.timeout(900)
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    drv = tmp_path / "driver.cpp"
    drv.write_text(DRIVER)
    objs = []
    jobs = [("fa_api.cpp", True)] + [(k, False) for k in KERNELS]
    procs = []
    for src, san in jobs:
        out = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, "-O1" if san else "-O3", "-g" if san else "-g0", "-fPIC", *COMMON, *(SAN if san else []),
               "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), cmd))
        objs.append(out)
    drv_o = str(tmp_path / "driver.o")
    procs.append((subprocess.Popen([HIPCC, "-O1", "-g", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}",
                                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                                    "-c", str(drv), "-o", drv_o],
                                   stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), ["driver"]))
    for p, cmd in procs:
        _, err = p.communicate()
        assert p.returncode == 0, (cmd[-1], err[-3000:])
    exe = str(tmp_path / "driver")
    _run([HIPCC, "--offload-arch=gfx950", *SAN, drv_o, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = _run([exe], env=env, timeout=300)
    assert r.stdout.strip() == "ok", (r.stdout, r.stderr[-3000:])
