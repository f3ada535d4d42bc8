"""The multiply-high division helper the kernels use for index math, checked
exhaustively against integer division on the host (built with g++)."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_ring_ulysses_amd", "csrc")

PROG = r"""
#include <cstdio>
#include <cstdint>
#include "fastdiv.h"
int main() {
  const uint32_t divisors[] = {1, 2, 3, 5, 6, 7, 12, 15, 24, 30, 48, 64, 100, 127, 128, 576,
                               581, 1536, 4276, 4608, 4645, 65535, 65536, 1000003, 2147483647u,
                               2147483648u, 4294967295u};
  uint64_t checked = 0;
  for (uint32_t d : divisors) {
    cru::FastDiv f = cru::make_fastdiv(d);
    for (uint64_t n = 0; n < 300000; ++n) {
      if (cru::fdiv((uint32_t)n, f) != (uint32_t)n / d) { printf("FAIL d=%u n=%llu\n", d, (unsigned long long)n); return 1; }
      ++checked;
    }
    for (uint64_t n = 4294967295ull; n > 4294967295ull - 300000; --n) {
      if (cru::fdiv((uint32_t)n, f) != (uint32_t)n / d) { printf("FAIL d=%u n=%llu\n", d, (unsigned long long)n); return 1; }
      ++checked;
    }
    uint64_t x = 88172645463325252ull;   // xorshift64 sample of the whole range
    for (int i = 0; i < 1000000; ++i) {
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      const uint32_t n = (uint32_t)x;
      if (cru::fdiv(n, f) != n / d) { printf("FAIL d=%u n=%u\n", d, n); return 1; }
      ++checked;
    }
  }
  printf("OK %llu\n", (unsigned long long)checked);
  return 0;
}
"""


def test_fastdiv_matches_integer_division():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "fd.cpp")
        exe = os.path.join(tmp, "fd")
        open(src, "w").write(PROG)
        r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
