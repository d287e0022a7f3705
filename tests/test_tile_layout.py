"""The unit-tiled operand layout on the host (no GPU): `tile_off` of the
kernels' shared header, compiled into a small host program, must place a
[rows, K] matrix (rows a multiple of 16, K of 32) one-to-one onto
[0, rows * K), each 16-row x 32-k block in its own 1 KB tile (tiles of a row
block consecutive along k), and inside a tile in the lane order of the
16x16x32 MFMA operand: lane i + 16 g holds row i, k 8 g .. 8 g + 7, as 8
consecutive values at 8 * lane."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decoder_only_transformer_qwen2_amd", "csrc")

PROGRAM = r"""
#include "qw_internal.h"
#include <cstdio>
#include <vector>

// every (row, k) of each shape: 0 = pass; a positive code names the failure
static int check(int rows, int K) {
  std::vector<int> seen((size_t)rows * K, 0);
  for (int r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) {
      const int64_t o = qw::tile_off(r, k, K);
      if (o < 0 || o >= (int64_t)rows * K) return 1;           // outside the matrix
      if (seen[o]++) return 2;                                   // two elements, one place
      const int64_t tile = ((int64_t)(r / 16) * (K / 32) + k / 32);
      if (o / 512 != tile) return 3;                             // wrong 1 KB tile
      const int lane = r % 16 + 16 * ((k % 32) / 8);
      if (o % 512 != 8 * lane + k % 8) return 4;                 // not the MFMA lane order
    }
  return 0;
}

int main() {
  const int shapes[][2] = {{16, 32}, {16, 96}, {48, 64}, {64, 1536}, {32, 896}};
  for (auto &s : shapes) {
    const int e = check(s[0], s[1]);
    if (e) {
      std::printf("FAIL %d x %d: code %d\n", s[0], s[1], e);
      return 1;
    }
  }
  std::printf("ok\n");
  return 0;
}
"""


def hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def test_tile_off_is_a_bijection_in_mfma_lane_order(tmp_path):
    cc = hipcc()
    if cc is None:
        pytest.skip("hipcc not found")
    src = tmp_path / "tile_layout.hip"
    exe = tmp_path / "tile_layout"
    src.write_text(PROGRAM)
    subprocess.run([cc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
