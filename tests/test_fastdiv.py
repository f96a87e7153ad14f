"""The kernels divide wave ids and columns by constants with a multiply and a shift
(Granlund and Montgomery's round-up method; the host computes the constants).  Check
the host's constants against exact division over every divisor the launcher can use
and numerators across the whole 31-bit range, compiled on the CPU with g++."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "rotate_then_bit_amd", "csrc", "kvq_internal.h")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include "%s"
static uint32_t fdiv(uint32_t n, kvq::FastDiv f) { return (uint32_t)(((uint64_t)n * f.mul) >> f.shift); }
int main() {
  uint64_t bad = 0, checked = 0;
  uint32_t ds[200000]; int nd = 0;
  for (uint32_t d = 1; d <= 70000; ++d) ds[nd++] = d;
  for (int k = 17; k < 31; ++k) { ds[nd++] = (1u << k) - 1; ds[nd++] = 1u << k; ds[nd++] = (1u << k) + 1; ds[nd++] = 3u << (k - 1); }
  ds[nd++] = 0x7fffffffu;
  uint64_t x = 88172645463325252ull;
  for (int i = 0; i < nd; ++i) {
    const uint32_t d = ds[i];
    const kvq::FastDiv f = kvq::make_fastdiv(d);
    if (f.mul == 0) { ++bad; continue; }
    const uint32_t edge[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7fffffffu, 0x7fffffffu - (0x7fffffffu %% d),
                             0x7fffffffu - (0x7fffffffu %% d) - 1};
    for (uint32_t n : edge) {
      if (n > 0x7fffffffu) continue;
      ++checked; if (fdiv(n, f) != n / d) ++bad;
    }
    for (int j = 0; j < 64; ++j) {
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      const uint32_t n = (uint32_t)(x & 0x7fffffffu);
      ++checked; if (fdiv(n, f) != n / d) ++bad;
    }
  }
  printf("%%llu %%llu\n", (unsigned long long)checked, (unsigned long long)bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_fastdiv_matches_exact_division():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "fastdiv.cpp")
        exe = os.path.join(d, "fastdiv")
        with open(src, "w") as f:
            f.write(PROGRAM % HEADER)
        subprocess.run(["g++", "-O2", "-std=c++17", src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True)
        checked, bad = (int(v) for v in out.stdout.split())
        assert checked > 5_000_000
        assert bad == 0 and out.returncode == 0
