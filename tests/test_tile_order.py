"""The tiled GEMM's tile order (grid_tile, grid_bands in gemm.hip) visits every
tile of every grid exactly once.  The two functions are compiled for the host from
the kernel source itself (device qualifiers defined away) and run over all grids up
to 140 x 90 tiles, which covers every launch the library makes at the 1024px and
2048px shapes.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM = os.path.join(ROOT, "image_generation_amd", "csrc", "gemm.hip")


def _function(src: str, signature: str) -> str:
    i = src.index(signature)
    j = src.index("\n}\n", i) + 3
    return src[i:j]


def test_every_tile_visited_once(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = open(GEMM).read()
    body = (_function(src, "__device__ __forceinline__ void grid_tile(") +
            _function(src, "static int grid_bands(int gm, int gn) {"))
    prog = tmp_path / "tile_order.cpp"
    prog.write_text(
        "#include <cstdio>\n#include <algorithm>\n#include <vector>\nusing std::min;\n"
        "#define __device__\n#define __forceinline__ inline\n" + body + r'''
int main() {
  int bad = 0;
  for (int gm = 1; gm <= 140; ++gm)
    for (int gn = 1; gn <= 90; ++gn) {
      const int P = grid_bands(gm, gn);
      if (P < 1 || P > 8 || P > gm || (P & (P - 1))) { ++bad; continue; }
      std::vector<int> seen((size_t)gm * gn, 0);
      for (int lid = 0; lid < gm * gn; ++lid) {
        int tm = -1, tn = -1;
        grid_tile(lid, gm, gn, P, tm, tn);
        if (tm < 0 || tm >= gm || tn < 0 || tn >= gn) { ++bad; break; }
        seen[(size_t)tm * gn + tn]++;
      }
      for (int v : seen)
        if (v != 1) { ++bad; break; }
    }
  // the 1024px block grids (18 row tiles) split into 2 row bands of 9
  const int want[4][2] = {{12, 2}, {36, 2}, {48, 2}, {84, 2}};
  for (auto& w : want)
    if (grid_bands(18, w[0]) != w[1]) ++bad;
  printf("%d\n", bad);
  return bad != 0;
}
''')
    exe = tmp_path / "tile_order"
    r = subprocess.run([cxx, "-O2", "-std=c++17", str(prog), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout + r.stderr
