"""The XCD-aware workgroup numbering of the prefill kernels
(grouped_query_kv_amd/csrc/xcd_order.h, xcd_block_id), compiled from the
header itself for the host and checked on the CPU: for every launch size
it is a permutation of the workgroup ids, and each XCD (ids x + 8 m, dealt
round-robin) receives one contiguous block of the new order."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "grouped_query_kv_amd" / "csrc"

PROGRAM = r"""
#include "xcd_order.h"
#include <cstdio>
#include <vector>
int main() {
  for (int n = 1; n <= 3000; n += (n < 200 ? 1 : 37)) {
    std::vector<int> seen(n, 0);
    for (int w = 0; w < n; ++w) {
      const int l = gqa::xcd_block_id(w, n);
      if (l < 0 || l >= n || seen[l]++) { std::printf("not a permutation: n=%d w=%d l=%d\n", n, w, l); return 1; }
    }
    for (int x = 0; x < gqa::kXcds; ++x) {   // XCD x's ids map onto one contiguous run
      int lo = n, hi = -1, cnt = 0;
      for (int w = x; w < n; w += gqa::kXcds) {
        const int l = gqa::xcd_block_id(w, n);
        lo = l < lo ? l : lo; hi = l > hi ? l : hi; ++cnt;
        if (w >= gqa::kXcds && l != gqa::xcd_block_id(w - gqa::kXcds, n) + 1) { std::printf("not in order: n=%d w=%d\n", n, w); return 1; }
      }
      if (cnt && hi - lo + 1 != cnt) { std::printf("not contiguous: n=%d x=%d\n", n, x); return 1; }
    }
  }
  std::printf("ok\n");
  return 0;
}
"""


def test_xcd_block_id_is_a_contiguous_permutation(tmp_path):
    hipcc = Path("/opt/rocm/bin/hipcc")
    if not hipcc.exists():
        pytest.skip("hipcc not available")
    src = tmp_path / "xcd.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "xcd"
    r = subprocess.run([str(hipcc), "--offload-arch=gfx950", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
