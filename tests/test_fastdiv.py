"""The invariant-divisor constants the host computes for the generic kernel's
index arithmetic (multiply-high and shift, Granlund and Montgomery 1994)
against plain integer division: every divisor up to 4096 on a grid of
numerators, and the extremes of the stated range (n < 2^31)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduction_attention_gqa_amd", "csrc")

SRC = r"""
#include <stdio.h>
#include "fastdiv.hpp"
int main() {
  long bad = 0, n_checked = 0;
  for (int d = 1; d <= 4096; ++d) {
    const attn::FastDiv f = attn::make_fastdiv(d);
    for (uint32_t n = 0; n < 70000; ++n, ++n_checked)
      if (attn::fastdiv_apply(n, f) != n / (uint32_t)d) ++bad;
    for (uint32_t n = 0x7fffffffu - 5000; n <= 0x7fffffffu - 1; n += 7, ++n_checked)
      if (attn::fastdiv_apply(n, f) != n / (uint32_t)d) ++bad;
    const uint32_t top = 0x7fffffffu;
    if (attn::fastdiv_apply(top, f) != top / (uint32_t)d) ++bad;
  }
  const int big[] = {65535, 65536, 1 << 20, (1 << 30) + 3, 0x7fffffff};
  for (int d : big) {
    const attn::FastDiv f = attn::make_fastdiv(d);
    for (uint32_t n = 0; n < 0x80000000u; n += 65521, ++n_checked)
      if (attn::fastdiv_apply(n, f) != n / (uint32_t)d) ++bad;
  }
  printf("%ld %ld\n", bad, n_checked);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fd.cpp"
    exe = tmp_path / "fd"
    src.write_text(SRC)
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    bad, n = map(int, r.stdout.split())
    assert r.returncode == 0 and bad == 0 and n > 280_000_000
