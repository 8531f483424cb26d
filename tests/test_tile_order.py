"""The workgroup -> (head, tile) mapping of the attention kernels (tile_of in
fa_device.hpp), compiled for the host and checked on the CPU.

Every launch must compute each (batch*head, tile) exactly once whatever the
dealing order, so the mapping is checked to be a bijection over a sweep of
grid shapes (heads that do and do not split evenly over the 8 XCDs, tile
counts on both sides of the rank-major limit of 64, resident-pass counts 0-4).
The balance it is for is checked on the GPT-2-shaped causal forward (8 x 12
heads, 8 query tiles of 2, 4, ..., 16 key tiles, three workgroups per CU): the
per-CU totals of the first three passes stay within 24-30 key tiles, where
dealing the longest-first list in order gives 20-34.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_33_amd", "csrc")

PROGRAM = r"""
#include "fa_device.hpp"
#include <cstdio>
#include <vector>
int main() {
  int bad = 0, cases = 0;
  const int nbhs[] = {1, 7, 8, 12, 16, 24, 96, 100, 128, 256};
  const int ntiles[] = {1, 2, 3, 5, 8, 12, 16, 33, 64, 65, 128};
  for (int nbh : nbhs)
    for (int nt : ntiles)
      for (int rm = 0; rm < 2; ++rm)
        for (int fill = 0; fill <= 4; ++fill) {
          const int total = nbh * nt;
          std::vector<int> seen(total, 0);
          for (int id = 0; id < total; ++id) {
            int bh = -1, r = -1;
            fa::tile_of(id, total, nt, rm != 0, fill, bh, r);
            if (bh < 0 || bh >= nbh || r < 0 || r >= nt) { ++bad; continue; }
            seen[bh * nt + r]++;
          }
          for (int v : seen) bad += (v != 1);
          ++cases;
        }
  printf("%d %d\n", cases, bad);
  // GPT-2-shaped causal forward: 96 heads x 8 query tiles, the tile of rank
  // r (longest first) visits 16 - 2 r key tiles; CU c of an XCD holds its
  // slots c, c + 32, c + 64 (ids 8 slot + xcd).
  for (int fill : {1, 3}) {
    int lo = 1 << 30, hi = 0;
    for (int xcd = 0; xcd < 8; ++xcd)
      for (int c = 0; c < 32; ++c) {
        int sum = 0;
        for (int k = 0; k < 3; ++k) {
          int bh, r;
          fa::tile_of(8 * (c + 32 * k) + xcd, 768, 8, true, fill, bh, r);
          sum += 16 - 2 * r;
        }
        lo = sum < lo ? sum : lo;
        hi = sum > hi ? sum : hi;
      }
    printf("%d %d\n", lo, hi);
  }
  return 0;
}
"""


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_tile_mapping_is_a_bijection_and_balances_cus(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "tile_order.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "tile_order"
    subprocess.run([hipcc, "--offload-arch=gfx950", "--offload-host-only", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    cases, bad = map(int, out[0].split())
    assert cases == 10 * 11 * 2 * 5 and bad == 0
    in_order = tuple(map(int, out[1].split()))      # fill 1: only the first pass dealt
    alternating = tuple(map(int, out[2].split()))   # fill 3: the three resident passes
    assert in_order == (20, 34)
    assert alternating == (24, 30)
