"""Division by invariants (csrc/internal.h), checked on the host.

Every kernel maps a key's index in its box to a token with two divisions by
invariants (Granlund and Montgomery, PLDI 1994): q = (umulhi(n, m) + n) >> s.
``make_fastdiv`` computes (m, s) with a 64-bit division; ``make_fastdiv_fp64``
(what the 128-query kernel uses on the device) computes the same constants
from a double-precision quotient and an integer correction.  This compiles a
small host program against the header and checks, for divisors up to 2^31,
that both give the same constants and that the quotient equals n / d for
dividends at and around the multiples of d and up to 2^31 - 1."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "video_dit_sparse_amd", "csrc")

PROGRAM = r"""
#include <cstdint>
#include <cstdio>
#define __host__
#define __device__
#include "internal.h"

static uint32_t quot(uint32_t n, const vdsa::FastDiv& f) {
  return (uint32_t)((((uint64_t)n * f.m) >> 32) + n) >> f.s;
}

int main() {
  long bad = 0, n_div = 0, n_q = 0;
  auto check = [&](uint32_t d) {
    const vdsa::FastDiv a = vdsa::make_fastdiv(d), b = vdsa::make_fastdiv_fp64(d);
    ++n_div;
    if (a.d != b.d || a.m != b.m || a.s != b.s) {
      if (bad++ < 5) printf("constants differ at d = %u\n", d);
      return;
    }
    const uint32_t lim = 0x7FFFFFFFu;   // dividends below 2^31
    const uint32_t probes[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, lim, lim - 1, lim / d * d, lim / d * d - 1};
    for (uint32_t n : probes) {
      if (n > lim) continue;
      ++n_q;
      if (quot(n, b) != n / d) {
        if (bad++ < 5) printf("quotient differs at n = %u, d = %u\n", n, d);
      }
    }
  };
  for (uint32_t d = 1; d < (1u << 16); ++d) check(d);
  for (uint64_t d = 1u << 16; d <= (1ull << 31); d += 9973) check((uint32_t)d);
  for (uint32_t k = 1; k <= 31; ++k) {
    check(1u << k);
    check((1u << k) - 1);
    if (k < 31) check((1u << k) + 1);
  }
  printf("%ld divisors, %ld quotients, %ld mismatches\n", n_div, n_q, bad);
  return bad != 0;
}
"""


def test_fastdiv_constants_and_quotients():
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "fastdiv.cpp")
        exe = os.path.join(tmp, "fastdiv")
        with open(src, "w") as f:
            f.write(PROGRAM)
        cmd = [cxx, "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", CSRC, "-I", "/opt/rocm/include", src,
               "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "0 mismatches" in r.stdout
