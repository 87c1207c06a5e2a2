"""The GEMM launch's workgroup -> (problem, tile) map is a bijection onto the
tiles of all its problems (a long group of up to two problems and a short
one), for launches of any size, gives every XCD a contiguous share of the
long group and of the short problem, and runs each XCD's tiles of one kind
before the other's (the long group's first, or the short problem's with
short_first).  The map is the
host- and device-callable code of csrc/tile_map.h, compiled here for the host
(no GPU involved)."""

import os
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "megatron_tensor_transformer_amd", "csrc")

PROGRAM = r"""
#include "tile_map.h"
#include <cstdio>
#include <vector>
int main() {
  const int sizes[] = {0, 1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 72, 100, 144, 192, 255, 256, 257,
                       384, 576, 1000, 1536, 3072};
  int bad = 0, cases = 0;
  const int shapes[][2] = {{1, 0}, {1, 1}, {2, 3}, {72, 72}, {576, 576}, {0, 0}};
  for (int sf = 0; sf < 2; ++sf)
  for (auto sh : shapes)
    for (int mult : {1, 3})
      for (int t2 : sizes) {
        const int t0 = sh[0] * mult, t1 = sh[1] * mult, total = t0 + t1 + t2;
        if (total == 0) continue;
        ++cases;
        const int t[3] = {t0, t1, t2};
        const tpmlp::XcdSplit split = tpmlp::make_split(t0, t1, t2, sf == 1);
        std::vector<std::vector<int>> seen(3);
        for (int p = 0; p < 3; ++p) seen[p].assign(t[p], 0);
        std::vector<int> lo(8, 1 << 30), hi(8, -1), n(8, 0), lo2(8, 1 << 30), hi2(8, -1), n2(8, 0);
        std::vector<int> phase(8, 0);  // each XCD: first-kind tiles, then the other kind, never back
        for (int wg = 0; wg < total; ++wg) {
          int prob, tile;
          tpmlp::map_workgroup(split, t0, wg, prob, tile);
          const int x = wg & 7;
          if (prob < 0 || prob > 2 || tile < 0 || tile >= t[prob]) {
            ++bad;
            std::printf("out of range: %d %d %d wg=%d -> (%d, %d)\n", t0, t1, t2, wg, prob, tile);
            continue;
          }
          ++seen[prob][tile];
          const bool first_kind = sf ? prob == 2 : prob < 2;
          if (first_kind && phase[x]) ++bad;
          if (!first_kind) phase[x] = 1;
          if (prob < 2) {  // index in the long group
            const int k = prob == 0 ? tile : t0 + tile;
            lo[x] = k < lo[x] ? k : lo[x]; hi[x] = k > hi[x] ? k : hi[x]; ++n[x];
          } else {
            lo2[x] = tile < lo2[x] ? tile : lo2[x]; hi2[x] = tile > hi2[x] ? tile : hi2[x]; ++n2[x];
          }
        }
        for (int p = 0; p < 3; ++p)
          for (int v : seen[p]) bad += v != 1;
        for (int x = 0; x < 8; ++x) {  // each XCD's shares are contiguous
          if (n[x] && hi[x] - lo[x] + 1 != n[x]) ++bad;
          if (n2[x] && hi2[x] - lo2[x] + 1 != n2[x]) ++bad;
        }
      }
  std::printf("cases %d bad %d\n", cases, bad);
  return bad != 0;
}
"""


def test_map_is_a_bijection(tmp_path):
    src = tmp_path / "map_check.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "map_check"
    cc = subprocess.run(["hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17", f"-I{CSRC}", str(src), "-o",
                         str(exe)], capture_output=True, text=True)
    if cc.returncode != 0:
        pytest.fail(cc.stderr[-2000:])
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout[-2000:]
    assert "bad 0" in run.stdout


HEAVY_FIRST = r"""
#include "tile_map.h"
#include <cstdio>
#include <vector>
int main() {
  int bad = 0, cases = 0;
  for (int heads : {1, 2, 3, 7, 8, 9, 24, 100, 192, 193})
    for (int nblk : {1, 2, 3, 5, 8, 9, 16}) {
      const int total = heads * nblk;
      ++cases;
      std::vector<int> seen(total, 0);
      std::vector<int> prev_p(8, -1);
      for (int wg = 0; wg < total; ++wg) {
        int h, p;
        tpmlp::heavy_first_block(heads, nblk, wg, h, p);
        if (h < 0 || h >= heads || p < 0 || p >= nblk) { ++bad; continue; }
        const int logical = h * nblk + p;
        ++seen[logical];
        // the block lies in the XCD's own contiguous range ...
        int begin, count;
        tpmlp::xcd_range(total, wg & 7, begin, count);
        if (logical < begin || logical >= begin + count) ++bad;
        // ... and each XCD sees its positions in non-decreasing order
        if (p < prev_p[wg & 7]) ++bad;
        prev_p[wg & 7] = p;
      }
      for (int v : seen) bad += v != 1;
    }
  std::printf("%d %d\n", cases, bad);
  return 0;
}
"""


def test_heavy_first_block_order(tmp_path):
    """Attention block order: a bijection onto (head, position); every block
    stays in its XCD's contiguous range of the head-major order; within an XCD
    the positions (0 = most work) come in non-decreasing order."""
    src = tmp_path / "hf.cpp"
    src.write_text(HEAVY_FIRST)
    exe = tmp_path / "hf"
    r = subprocess.run(["hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17", f"-I{CSRC}", str(src), "-o",
                        str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True, timeout=60).stdout.split()
    cases, bad = int(out[0]), int(out[1])
    assert cases == 70 and bad == 0
