"""The physical layouts (csrc/layout.h) are bijections and their forward and
inverse maps agree.  Host logic only: the header is compiled with g++ into a
small checker and run on the CPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHECK = r"""
#include <cstdio>
#include <vector>
#include "layout.h"
using namespace kvtier::layout;
int main() {
  int bad = 0;
  for (int D : {64, 128}) {
    // bf16 tile: K and V offsets cover 0..64*D-1 exactly once
    std::vector<int> seen(64 * D, 0);
    for (int t = 0; t < 32; ++t)
      for (int d = 0; d < D; ++d) { seen[bf16_k_offset(t, d, D)]++; seen[bf16_v_offset(t, d, D)]++; }
    for (int x : seen) bad += x != 1;
    // chunk inverse maps agree with the forward offsets
    for (int cmb = 0; cmb < D / 16; ++cmb)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          int t, d;
          k_chunk_elem(cmb, lane, e, D, &t, &d);
          bad += bf16_k_offset(t, d, D) != (cmb * 64 + lane) * 8 + e;
          v_chunk_elem(cmb, lane, e, &t, &d);
          bad += bf16_v_offset(t, d, D) != 32 * D + (cmb * 64 + lane) * 8 + e;
        }
    for (int bits : {2, 4, 8}) {
      // code positions: every (token, dim) gets its own b-bit field in Kc / Vc
      const LedgerTile LT(D, bits);
      bad += LT.vc != 32 * D * bits / 8 || LT.bytes != 2 * LT.vc + 8 * D;
      const int fields = 32 / bits;
      std::vector<int> kb(LT.vc / 4 * fields, 0), vb(LT.vc / 4 * fields, 0);
      for (int t = 0; t < 32; ++t)
        for (int d = 0; d < D; ++d) {
          int wb, bit;
          k_code_pos(t, d, D, bits, &wb, &bit);
          bad += wb % 4 != 0 || bit % bits != 0 || bit + bits > 32 || wb >= LT.vc;
          kb[wb / 4 * fields + bit / bits]++;
          v_code_pos(t, d, D, bits, &wb, &bit);
          vb[wb / 4 * fields + bit / bits]++;
        }
      for (int x : kb) bad += x != 1;
      for (int x : vb) bad += x != 1;
      // field_elem_b inverts code_pos; a lane's words are its own
      const int lane_bytes = bits * D / 16;
      for (int cmb = 0; cmb < D / 16; ++cmb)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            int wb, bit, c2, e2;
            code_pos(cmb, lane, e, D, bits, &wb, &bit);
            field_elem_b(bits, (wb - lane * lane_bytes) / 4, bit / bits, &c2, &e2);
            bad += (c2 != cmb) || (e2 != e) || wb / lane_bytes != lane;
            // elements 2r and 2r + 1 of a chunk sit 16 bits apart in one word
            // (b = 2, 4) or in the same word's bytes 2(r%2), 2(r%2)+1 (b = 8)
            if (e & 1) {
              int wb0, bit0;
              code_pos(cmb, lane, e - 1, D, bits, &wb0, &bit0);
              bad += wb0 != wb || bit != bit0 + (bits == 8 ? 8 : 16);
            }
          }
    }
    // token permutation of the QK rows is a bijection on 0..31
    std::vector<int> tk(32, 0);
    for (int blk = 0; blk < 2; ++blk)
      for (int m = 0; m < 16; ++m) tk[qk_token(blk, m)]++;
    for (int x : tk) bad += x != 1;
  }
  std::printf("%d\n", bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_layout_maps_are_consistent_bijections():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "check.cpp")
        exe = os.path.join(tmp, "check")
        open(src, "w").write(CHECK)
        subprocess.run(["g++", "-std=c++17", "-O1", "-I",
                        os.path.join(ROOT, "tiered_int2_fp16_amd", "csrc"), src, "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True)
        assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout + r.stderr
