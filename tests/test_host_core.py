"""The library's host-side geometry (csrc/host_core.cpp) under AddressSanitizer
and UndefinedBehaviorSanitizer.  Host logic only: the C++ file and a small
driver are compiled with g++ and run on the CPU.

The driver checks, for every ledger width (0 = 2, 2, 4, 8):
  * arena regions are 256-byte aligned, in order, disjoint, and sized by the
    layout formulas (bf16 block 4*W*D bytes, ledger entry (b+1)*W*D/4);
  * every out-of-range configuration is rejected with a message;
  * tier counts spend the byte budget (16 bits per bf16 value, b + 1 per
    ledger value) without exceeding it;
  * attention workspace regions are aligned and hold the documented arrays.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiered_int2_fp16_amd", "csrc")

DRIVER = r"""
#include <cmath>
#include <cstdio>
#include <random>
#include <string>
#include "host_core.h"
using namespace kvtier;
static int bad = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL line %d: %s\n", __LINE__, #c); ++bad; } } while (0)

static kv_pool_config base() {
  kv_pool_config c{};
  c.batch = 2; c.layers = 3; c.q_heads = 32; c.kv_heads = 8; c.head_dim = 128; c.window = 128;
  c.max_windows = 300; c.n_recent = 4; c.bf16_slots = 40; c.ledger_slots = 200; c.ledger_bits = 2;
  return c;
}

int main() {
  // ---- valid geometries at every width
  for (int bits : {0, 2, 4, 8}) {
    kv_pool_config c = base();
    c.ledger_bits = bits;
    Geometry g;
    std::string err;
    CHECK(geometry_init(c, &g, &err));
    const int b = bits == 0 ? 2 : bits;
    CHECK(g.cfg.ledger_bits == b);
    const size_t wd = size_t(c.window) * c.head_dim;
    CHECK(g.bf16_block == 4 * wd);
    CHECK(g.entry == size_t(b + 1) * wd / 4);
    const size_t segs = size_t(c.batch) * c.layers;
    CHECK(g.size[KV_REGION_BF16] == segs * c.bf16_slots * c.kv_heads * g.bf16_block);
    CHECK(g.size[KV_REGION_LEDGER] == segs * c.ledger_slots * c.kv_heads * g.entry);
    CHECK(g.size[KV_REGION_PAGES] == segs * c.max_windows * 4);
    size_t end = 0;
    for (int r = 0; r < KV_REGION_COUNT; ++r) {
      CHECK(g.off[r] % 256 == 0);
      CHECK(g.off[r] >= end);
      end = g.off[r] + g.size[r];
    }
    CHECK(g.total >= end && g.total % 256 == 0);
    for (int cus : {1, 80, 256, 304}) {
      const int s = attn_splits(g, cus);
      CHECK(s >= 1 && s <= 64);
      const AttnWorkspace w = attn_workspace(g, s);
      const size_t pairs = size_t(c.batch) * c.kv_heads, rows = size_t(c.batch) * c.q_heads;
      CHECK(w.partials % 256 == 0 && w.ml % 256 == 0 && w.tile_mass % 256 == 0);
      CHECK(w.app_mass % 256 == 0 && w.app_info % 256 == 0 && w.total % 256 == 0);
      CHECK(w.ml >= w.partials + pairs * s * g.group * c.head_dim * 4);
      CHECK(w.tile_mass >= w.ml + rows * s * 8);
      CHECK(w.app_mass >= w.tile_mass + rows * size_t(c.max_windows) * (c.window / 32) * 8);
      CHECK(w.total >= w.app_info + size_t(c.batch) * 8 * 4);
    }
  }
  // ---- every out-of-range field is rejected with a message
  struct Bad { const char* what; void (*edit)(kv_pool_config&); };
  const Bad cases[] = {
    {"batch", [](kv_pool_config& c) { c.batch = 0; }},
    {"layers", [](kv_pool_config& c) { c.layers = 0; }},
    {"kv_heads", [](kv_pool_config& c) { c.kv_heads = 0; }},
    {"q_heads multiple", [](kv_pool_config& c) { c.q_heads = 30; }},
    {"group 3", [](kv_pool_config& c) { c.q_heads = 24; }},
    {"head_dim", [](kv_pool_config& c) { c.head_dim = 96; }},
    {"window 48", [](kv_pool_config& c) { c.window = 48; }},
    {"window 288", [](kv_pool_config& c) { c.window = 288; }},
    {"max_windows 0", [](kv_pool_config& c) { c.max_windows = 0; }},
    {"max_windows 4097", [](kv_pool_config& c) { c.max_windows = 4097; }},
    {"tiles", [](kv_pool_config& c) { c.window = 256; c.max_windows = 1025; }},
    {"n_recent", [](kv_pool_config& c) { c.n_recent = -1; }},
    {"n_recent 0", [](kv_pool_config& c) { c.n_recent = 0; }},
    {"bf16_slots 0", [](kv_pool_config& c) { c.bf16_slots = 0; }},
    {"bf16_slots", [](kv_pool_config& c) { c.bf16_slots = 16384; }},
    {"ledger_slots", [](kv_pool_config& c) { c.ledger_slots = 32768; }},
    {"ledger_bits 3", [](kv_pool_config& c) { c.ledger_bits = 3; }},
    {"ledger_bits 16", [](kv_pool_config& c) { c.ledger_bits = 16; }},
    {"ledger_bits -2", [](kv_pool_config& c) { c.ledger_bits = -2; }},
  };
  for (const Bad& x : cases) {
    kv_pool_config c = base();
    x.edit(c);
    Geometry g;
    std::string err;
    const bool ok = geometry_init(c, &g, &err);
    if (ok || err.empty()) { std::printf("FAIL: %s accepted\n", x.what); ++bad; }
  }
  // ---- tier counts spend the budget at b + 1 bits per ledger value
  std::mt19937_64 rng(7);
  std::uniform_real_distribution<double> u01(0.0, 1.0);
  const int widths[3] = {2, 4, 8};
  for (int it = 0; it < 20000; ++it) {
    const int n = int(rng() % 5000), R = int(rng() % 8);
    const int bits = widths[rng() % 3];
    const double beta = u01(rng) * 0.7, phi = u01(rng) * beta;
    int hi = -1, lo = -1;
    tier_counts(n, R, beta, phi, bits, &hi, &lo);
    CHECK(hi == std::min(n, std::max(R, int(std::floor(phi * n)))));
    CHECK(lo >= 0 && hi + lo <= n);
    const double budget = 16.0 * beta * n;
    if (lo > 0) CHECK(16.0 * hi + (bits + 1.0) * lo <= budget * (1 + 1e-12));
    if (hi + lo < n && 16.0 * hi <= budget)
      CHECK(16.0 * hi + (bits + 1.0) * (lo + 1) > budget * (1 - 1e-12));
  }
  std::printf("%d\n", bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_core_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "driver.cpp")
        exe = os.path.join(tmp, "driver")
        open(src, "w").write(DRIVER)
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               src, os.path.join(CSRC, "host_core.cpp"), "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env)
        assert r.returncode == 0 and r.stdout.strip().endswith("0"), r.stdout + r.stderr
